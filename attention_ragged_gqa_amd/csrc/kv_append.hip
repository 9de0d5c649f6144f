// Append K/V tokens into the paged cache, rotating K on the way (the "normal"
// RoPE mode of the KV cache on the "_kernel_common.py" page, RopeMode: k is
// rotated before it is added to the cache). Page addressing follows the page
// gather of the paged tree kernel on the "tree_attn.py" page.
//
// A workgroup of 256 threads handles a group of T = 256 / (h_kv * D/16)
// consecutive tokens at a time (one when a token has more chunk pairs than
// threads; its pairs are then looped over). A thread holds one 16-byte
// chunk of a head row's first half and its RoPE partner in the second half
// (dims +- D/2), for K and for V, so the rotation needs no cross-lane
// exchange; the pairs of a token sit on consecutive threads, and each
// wave-wide load or store covers 128-byte runs of the head rows.
//
// The grid holds at most eight workgroups per compute unit of the MI355X
// (2048); each loads the batch's append_indptr, page_indptr and
// append_start into LDS once (batches too large for that search
// append_indptr in global memory instead) and then walks token groups
// blockIdx.x, + gridDim.x, ...: a group's sequences come from a binary
// search in LDS, so its page numbers, K/V pairs and positions go out in one
// round trip; cos/sin are evaluated once per (token, frequency) into an LDS
// table that the pairs of every head read.

#include "device_common.h"
#include "ra_internal.h"

namespace ra {

namespace {

constexpr int kAppendThreads = 256;

// Tokens per group (the host sizes the grid with the same rule).
__host__ __device__ inline int append_tokens_per_group(int h_kv, int head_dim) {
  const int per_tok = h_kv * (head_dim / 16);
  return per_tok >= kAppendThreads ? 1 : kAppendThreads / per_tok;
}

// Workgroups in the grid at most: eight resident on each of 256 CUs.
constexpr long kAppendMaxGroups = 2048;

// Index arrays in LDS while 3 (batch + 1) int32 fit in this many bytes.
constexpr int kAppendIdxLdsBytes = 16 * 1024;

template <bool BF, int D, bool IDX_LDS>
__global__ __launch_bounds__(kAppendThreads) void kv_append_kernel(AppendParams p) {
  constexpr int CP = D / 16;                   // chunk pairs per head row
  constexpr int HALF = D / 2;
  constexpr int kMaxT = kAppendThreads / CP;   // tokens per group at most (h_kv = 1)
  constexpr int TABN = (kMaxT * HALF + kAppendThreads - 1) / kAppendThreads;
  extern __shared__ int idx_s[];               // [append_indptr | page_indptr | append_start]
  __shared__ double inv_freq_s[HALF];
  __shared__ float2 tab_s[kMaxT * HALF];       // (cos, sin) per (token slot, frequency)

  const int tid = threadIdx.x;
  const int nb = p.batch;
  const int per_tok = p.h_kv * CP;
  const int T = append_tokens_per_group(p.h_kv, D);
  const int n_groups = (p.n_tokens + T - 1) / T;
  const bool rope = p.rope_position != nullptr;
  const int ti = per_tok >= kAppendThreads ? 0 : tid / per_tok;
  const int u_first = per_tok >= kAppendThreads ? tid : tid - ti * per_tok;

  if constexpr (IDX_LDS) {
    for (int i = tid; i <= nb; i += kAppendThreads) {
      idx_s[i] = p.append_indptr[i];
      idx_s[nb + 1 + i] = p.page_indptr[i];
      if (i < nb) idx_s[2 * (nb + 1) + i] = p.append_start[i];
    }
  }
  if (rope && tid < HALF) inv_freq_s[tid] = p.inv_freq[tid];
  __syncthreads();   // index arrays and frequencies visible

  for (int grp = blockIdx.x; grp < n_groups; grp += gridDim.x) {
    const int tok0 = grp * T;
    const int tok = tok0 + ti;
    const bool tok_ok = ti < T && tok < p.n_tokens;
    int off = 0, pi = 0;
    bool ok = false;
    if (tok_ok) {
      int lo = 0, hi = nb - 1;
      while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        const int a = IDX_LDS ? idx_s[mid] : p.append_indptr[mid];
        if (a <= tok) lo = mid; else hi = mid - 1;
      }
      const int b = lo;
      const int a0 = IDX_LDS ? idx_s[b] : p.append_indptr[b];
      const int a1 = IDX_LDS ? idx_s[b + 1] : p.append_indptr[b + 1];
      const int p0 = IDX_LDS ? idx_s[nb + 1 + b] : p.page_indptr[b];
      const int p1 = IDX_LDS ? idx_s[nb + 1 + b + 1] : p.page_indptr[b + 1];
      const int st = IDX_LDS ? idx_s[2 * (nb + 1) + b] : p.append_start[b];
      off = st + (tok - a0);
      pi = p0 + (off >> 4);
      ok = tok >= a0 && tok < a1 && off >= 0 && pi >= 0 && pi < p1 && pi < p.nnz_pages;
    }
    // one round trip: page number, K/V pairs, positions
    // (pair c of head h: dims 8c + [0, 8) and HALF + 8c + [0, 8))
    int page = ok ? p.page_values[pi] : 0;
    u32x4 k1{0, 0, 0, 0}, k2{0, 0, 0, 0}, v1{0, 0, 0, 0}, v2{0, 0, 0, 0};
    auto load_pair = [&](int u) __attribute__((always_inline)) {
      const int h = u / CP, c = u - (u / CP) * CP;
      const size_t src = (static_cast<size_t>(tok) * p.h_kv + h) * D + 8 * c;
      k1 = *reinterpret_cast<const u32x4*>(p.k + src);
      k2 = *reinterpret_cast<const u32x4*>(p.k + src + HALF);
      v1 = *reinterpret_cast<const u32x4*>(p.v + src);
      v2 = *reinterpret_cast<const u32x4*>(p.v + src + HALF);
    };
    if (tok_ok && u_first < per_tok) load_pair(u_first);
    int tpos[TABN];
#pragma unroll
    for (int j = 0; j < TABN; ++j) {
      const int e = tid + j * kAppendThreads;
      const int t = tok0 + e / HALF;
      tpos[j] = (rope && e < T * HALF && t < p.n_tokens) ? p.rope_position[t] : 0;
    }
    const int slot = off & 15;
    __syncthreads();   // the previous group's table reads are done
    if (rope) {
#pragma unroll
      for (int j = 0; j < TABN; ++j) {
        const int e = tid + j * kAppendThreads;
        if (e < T * HALF) {
          float cs, sn;
          rope_cos_sin(tpos[j], p.rope_scale, inv_freq_s[e % HALF], cs, sn);
          tab_s[e] = make_float2(cs, sn);
        }
      }
    }
    __syncthreads();   // table visible
    ok = ok && static_cast<unsigned>(page) < static_cast<unsigned>(p.num_pages);
    for (int u = u_first; u < per_tok; u += kAppendThreads) {
      const int h = u / CP;
      const int c = u - h * CP;
      if (u != u_first) {   // further pairs of a token wider than the workgroup
        k1 = k2 = v1 = v2 = u32x4{0, 0, 0, 0};
        if (tok_ok) load_pair(u);
      }
      if (rope) {
        const float2* trow = tab_s + ti * HALF + 8 * c;
        u32x4 r1, r2;
#pragma unroll
        for (int e = 0; e < 8; e += 2) {
          float y1[2], y2[2];
#pragma unroll
          for (int v = 0; v < 2; ++v) {
            const float2 t = trow[e + v];
            rope_pair(t.x, t.y, to_f32<BF>(half_of(k1, e + v)), to_f32<BF>(half_of(k2, e + v)), y1[v], y2[v]);
          }
          r1[e >> 1] = pack2<BF>(y1[0], y1[1]);
          r2[e >> 1] = pack2<BF>(y2[0], y2[1]);
        }
        k1 = r1;
        k2 = r2;
      }
      if (ok) {
        const size_t dk = (((static_cast<size_t>(page) * 2 + 0) * p.h_kv + h) * 16 + slot) * D + 8 * c;
        const size_t dv = (((static_cast<size_t>(page) * 2 + 1) * p.h_kv + h) * 16 + slot) * D + 8 * c;
        *reinterpret_cast<u32x4*>(p.pages + dk) = k1;
        *reinterpret_cast<u32x4*>(p.pages + dk + HALF) = k2;
        *reinterpret_cast<u32x4*>(p.pages + dv) = v1;
        *reinterpret_cast<u32x4*>(p.pages + dv + HALF) = v2;
      }
    }
  }
}

template <bool BF, int D>
void launch_append_d(const AppendParams& p, hipStream_t stream) {
  const int t = append_tokens_per_group(p.h_kv, D);
  const long groups = (p.n_tokens + t - 1) / t;
  const dim3 grid(static_cast<unsigned>(groups < kAppendMaxGroups ? groups : kAppendMaxGroups));
  const long idx_bytes = 4L * (3L * p.batch + 2);
  if (idx_bytes <= kAppendIdxLdsBytes)
    hipLaunchKernelGGL((kv_append_kernel<BF, D, true>), grid, dim3(kAppendThreads),
                       static_cast<unsigned>(idx_bytes), stream, p);
  else
    hipLaunchKernelGGL((kv_append_kernel<BF, D, false>), grid, dim3(kAppendThreads), 0, stream, p);
}

}  // namespace

hipError_t launch_append(const AppendParams& p, int is_bf16, int head_dim, hipStream_t stream) {
  if (is_bf16) {
    if (head_dim == 128) launch_append_d<true, 128>(p, stream);
    else launch_append_d<true, 64>(p, stream);
  } else {
    if (head_dim == 128) launch_append_d<false, 128>(p, stream);
    else launch_append_d<false, 64>(p, stream);
  }
  return hipGetLastError();
}

}  // namespace ra
