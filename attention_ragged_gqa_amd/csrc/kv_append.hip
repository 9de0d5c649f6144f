// Append K/V tokens into the paged cache, rotating K on the way (the "normal"
// RoPE mode of the KV cache on the "_kernel_common.py" page, RopeMode: k is
// rotated before it is added to the cache). Page addressing follows the page
// gather of the paged tree kernel on the "tree_attn.py" page.
//
// One workgroup per token; its h_kv * D/8 16-byte chunks of K and of V are
// spread over the threads, so each head row is read and written with
// contiguous 16-byte accesses. A chunk's RoPE partner (dims +- D/2) is in
// lane ^ (D/16) of the same head row.

#include "device_common.h"
#include "ra_internal.h"

namespace ra {

namespace {

template <bool BF, int D>
__global__ __launch_bounds__(256) void kv_append_kernel(AppendParams p) {
  constexpr int CH = D / 8;
  __shared__ double inv_freq_s[D / 2];
  const int tok = blockIdx.x;
  const int tid = threadIdx.x;
  if (p.rope_position != nullptr) {
    if (tid < D / 2) inv_freq_s[tid] = p.inv_freq[tid];
    __syncthreads();
  }
  // sequence of this token: last b with append_indptr[b] <= tok
  int lo = 0, hi = p.batch - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (p.append_indptr[mid] <= tok) lo = mid; else hi = mid - 1;
  }
  const int b = lo;
  const bool in_seq = tok >= p.append_indptr[b] && tok < p.append_indptr[b + 1];
  const int off = p.append_start[b] + (tok - p.append_indptr[b]);
  const int pi = p.page_indptr[b] + (off >> 4);
  bool ok = in_seq && off >= 0 && pi >= 0 && pi < p.page_indptr[b + 1] && pi < p.nnz_pages;
  int page = 0;
  if (ok) {
    page = p.page_values[pi];
    ok = static_cast<unsigned>(page) < static_cast<unsigned>(p.num_pages);
  }
  const int slot = off & 15;
  const int pos = (ok && p.rope_position != nullptr) ? p.rope_position[tok] : 0;

  for (int u0 = 0; u0 < p.h_kv * CH; u0 += 256) {
    const int u = u0 + tid;
    const bool act = u < p.h_kv * CH;
    const int h = u / CH;
    const int c = u - h * CH;
    u32x4 kx{0, 0, 0, 0}, vx{0, 0, 0, 0};
    if (act) {
      const size_t src = (static_cast<size_t>(tok) * p.h_kv + h) * D + 8 * c;
      kx = *reinterpret_cast<const u32x4*>(p.k + src);
      vx = *reinterpret_cast<const u32x4*>(p.v + src);
    }
    if (p.rope_position != nullptr) {
      u32x4 other;
#pragma unroll
      for (int i = 0; i < 4; ++i) other[i] = __shfl_xor(kx[i], CH / 2, 64);
      const bool first = c < CH / 2;
      u32x4 res;
#pragma unroll
      for (int e = 0; e < 8; e += 2) {
        float y[2];
#pragma unroll
        for (int v = 0; v < 2; ++v) {
          const int dim = 8 * c + e + v;
          float cs, sn, y1, y2;
          rope_cos_sin(pos, p.rope_scale, inv_freq_s[dim & (D / 2 - 1)], cs, sn);
          const float x = to_f32<BF>(half_of(kx, e + v));
          const float xp = to_f32<BF>(half_of(other, e + v));
          if (first) { rope_pair(cs, sn, x, xp, y1, y2); y[v] = y1; }
          else { rope_pair(cs, sn, xp, x, y1, y2); y[v] = y2; }
        }
        res[e >> 1] = pack2<BF>(y[0], y[1]);
      }
      kx = res;
    }
    if (act && ok) {
      const size_t dk = (((static_cast<size_t>(page) * 2 + 0) * p.h_kv + h) * 16 + slot) * D + 8 * c;
      const size_t dv = (((static_cast<size_t>(page) * 2 + 1) * p.h_kv + h) * 16 + slot) * D + 8 * c;
      *reinterpret_cast<u32x4*>(p.pages + dk) = kx;
      *reinterpret_cast<u32x4*>(p.pages + dv) = vx;
    }
  }
}

}  // namespace

hipError_t launch_append(const AppendParams& p, int is_bf16, int head_dim, hipStream_t stream) {
  const dim3 grid(static_cast<unsigned>(p.n_tokens));
  if (is_bf16) {
    if (head_dim == 128) hipLaunchKernelGGL((kv_append_kernel<true, 128>), grid, dim3(256), 0, stream, p);
    else hipLaunchKernelGGL((kv_append_kernel<true, 64>), grid, dim3(256), 0, stream, p);
  } else {
    if (head_dim == 128) hipLaunchKernelGGL((kv_append_kernel<false, 128>), grid, dim3(256), 0, stream, p);
    else hipLaunchKernelGGL((kv_append_kernel<false, 64>), grid, dim3(256), 0, stream, p);
  }
  return hipGetLastError();
}

}  // namespace ra
