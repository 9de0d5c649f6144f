// Ragged, batched, masked GQA attention forward for gfx950 (MI355X).
//
// What is computed follows the TVM pages: scores and online softmax from the
// prefill macros of the "_kernel_common.py" page (compute_s_gemm,
// softmax_update_causal, compute_o_gemm, paged_store_output_lse), the causal
// test (_causal_mask), paged chunk lengths and the sliding-window remap
// (_get_kv_chunk_len, _get_seq_offset), the tree test (_check_tree_order on the
// "tree_attn.py" page) and the page gather of that page's paged tree kernel.
// How it is computed is designed for CDNA4:
//
//  * Work item = (sequence, KV head, tile of 128 packed query rows). Packed
//    row R of a sequence is token R / g, query head kvh*g + R % g (g = h_q/h_kv),
//    so one K/V tile feeds all g heads that share it. Items are enumerated
//    sequence-major with the heaviest tile of each (sequence, KV head) first,
//    and split into 8 contiguous chunks, one per XCD (workgroups are handed
//    to XCDs round-robin), so the tiles that share K/V run on one XCD's L2.
//  * A workgroup is 4 waves of 64; each wave owns 32 packed rows. Scores are
//    computed transposed, S^T = K Q^T, with v_mfma_f32_32x32x16_{bf16,f16}:
//    each lane then holds one query row and 16 keys per 32-key block, so row
//    max and row sum are in-lane plus one exchange with lane ^ 32, and the
//    fp32 accumulators convert in place into the B operand of O^T += V^T P^T.
//  * Q stays in registers (RoPE applied on load). K tiles are staged in LDS
//    row-major; V tiles are transposed in registers and staged as V^T with
//    keys permuted so each lane's 8 keys of a PV step are one 16-byte read.
//    Global loads for tile i+1 are issued before tile i is computed (LDS is
//    double buffered, one barrier per tile).
//  * Masks are classified per (wave, tile): skipped, full (no test) or
//    partial (per-element test); causal work stops at the last visible tile.
//  * The softmax runs in the log2 domain (v_exp_f32 is exp2): scores are
//    scaled by sm_scale*log2(e), lse = m + log2(l) as on the pages.

#include <climits>
#include <cmath>

#include "device_common.h"
#include "ra_internal.h"

namespace ra {

namespace {

// Locate this workgroup's work item. Returns false when the block has none.
// Item list: for each sequence b (in order), for each KV head, ranks
// 0..tiles_b-1 with rank 0 = the last (heaviest under a causal mask) q-tile.
__device__ bool locate_item(const AttnParams& p, int& b, int& kvh, int& tile) {
  const int lane = threadIdx.x & 63;
  int total = 0;
  for (int c0 = 0; c0 < p.batch; c0 += 64) {
    const int i = c0 + lane;
    int cnt = 0;
    if (i < p.batch) {
      const int len = max(p.q_indptr[i + 1] - p.q_indptr[i], 0);
      cnt = ((len * p.group + kBM - 1) / kBM) * p.h_kv;
    }
    total += wave_sum(cnt);
  }
  // XCD-contiguous mapping: block L runs on XCD L % 8; give XCD x the items
  // [x*chunk, (x+1)*chunk) in order.
  const int chunk = (total + 7) / 8;
  const int L = blockIdx.x;
  const int slot = L >> 3;
  if (slot >= chunk) return false;
  const int item = (L & 7) * chunk + slot;
  if (item >= total) return false;
  int base = 0;
  for (int c0 = 0; c0 < p.batch; c0 += 64) {
    const int i = c0 + lane;
    int cnt = 0;
    if (i < p.batch) {
      const int len = max(p.q_indptr[i + 1] - p.q_indptr[i], 0);
      cnt = ((len * p.group + kBM - 1) / kBM) * p.h_kv;
    }
    const int incl = wave_inclusive_scan(cnt) + base;
    const unsigned long long hit = __ballot(i < p.batch && item < incl);
    if (hit) {
      const int l = __ffsll(static_cast<long long>(hit)) - 1;
      b = c0 + l;
      const int excl = __shfl(incl - cnt, l, 64);
      const int tiles_b = __shfl(cnt, l, 64) / p.h_kv;
      const int local = item - excl;
      kvh = local / tiles_b;
      tile = tiles_b - 1 - (local - kvh * tiles_b);
      return true;
    }
    base = __shfl(incl, 63, 64);
  }
  return false;
}

template <bool BF, int D, int LAYOUT, int MASK>
__global__ __launch_bounds__(kThreads, 2) void attn_fwd_kernel(AttnParams p) {
  constexpr int CH = D / 8;               // 16-byte chunks per head row
  constexpr int HC = CH / 2;              // chunk pairs (dims k and k + D/2)
  constexpr int KSTEP = kThreads / HC;    // K rows staged per pass
  constexpr int KP = kBN / KSTEP;         // K passes per tile
  constexpr int KS = D * 2 + 16;          // LDS K row stride (bytes)
  constexpr int VS = kBN * 2 + 16;        // LDS V^T row stride (bytes)
  constexpr int K_OFF = 0;
  constexpr int V_OFF = kBN * KS;
  constexpr int T_OFF = V_OFF + D * VS;   // tree intervals (int2 per key)
  constexpr int BUF = T_OFF + kBN * 8;
  constexpr int VUNITS = 16 * CH;         // (4-key group, chunk) pairs
  static_assert(KP >= 1 && VUNITS <= kThreads, "tile shape");
  static_assert((kBM / 1 + 1) * (D / 2) * 8 <= 2 * BUF, "RoPE table fits in the tile buffers");

  __shared__ __attribute__((aligned(16))) char smem[2 * BUF];
  __shared__ double inv_freq_s[D / 2];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = tid >> 6;
  const int r32 = lane & 31;
  const int hh = lane >> 5;

  int b = 0, kvh = 0, tile = 0;
  if (!locate_item(p, b, kvh, tile)) return;   // uniform over the workgroup

  const int g = p.group;
  const int q0 = p.q_indptr[b];
  const int qo_len = p.q_indptr[b + 1] - q0;
  const int row0 = tile * kBM;

  // ---- KV chunk of this sequence ----
  int kv_len = 0, kv_base = 0, page_base = 0, page_end = 0, sink = 0, win_off = 0;
  if constexpr (LAYOUT == kContiguous) {
    kv_base = p.kv_indptr[b];
    kv_len = p.kv_indptr[b + 1] - kv_base;
  } else {
    page_base = p.page_indptr[b];
    page_end = min(p.page_indptr[b + 1], p.nnz_pages);
    const int np = p.page_indptr[b + 1] - page_base;
    if (np > 0) {
      if (!p.sliding) {
        kv_len = (np - 1) * 16 + p.length_info[b];
      } else {
        win_off = p.length_info[p.batch + b];
        sink = p.length_info[2 * p.batch + b];
        kv_len = (np - 1) * 16 + p.length_info[b] - win_off + sink;
      }
    }
  }
  kv_len = max(kv_len, 0);

  int tree_base = 0, tree_len = 0;
  if constexpr (MASK == kMaskTree) {
    tree_base = p.tree_indptr[b];
    tree_len = max(p.tree_indptr[b + 1] - tree_base, 0);
  }
  const int tree_start = kv_len - tree_len;

  // ---- this lane's query row ----
  const int R = row0 + w * 32 + r32;
  const int t = R / g;
  const int head = kvh * g + (R - t * g);
  const bool row_ok = t < qo_len && q0 + t >= 0 && q0 + t < p.total_q;
  const int t_lo = (row0 + w * 32) / g;
  const int t_hi = min((row0 + w * 32 + 31) / g, qo_len - 1);
  const bool wave_active = t_lo < qo_len;

  const bool causal = (MASK == kMaskCausal) && p.causal;
  const int lim = causal ? min(kv_len, kv_len - qo_len + t + 1) : kv_len;
  const int lim_lo = causal ? min(kv_len, kv_len - qo_len + t_lo + 1) : kv_len;
  const int lim_hi = causal ? min(kv_len, kv_len - qo_len + t_hi + 1) : kv_len;
  int kv_hi = kv_len;
  if (causal) {
    const int t_last = min((row0 + kBM - 1) / g, qo_len - 1);
    kv_hi = min(kv_len, kv_len - qo_len + t_last + 1);
  }
  const int n_tiles = kv_hi > 0 ? (kv_hi + kBN - 1) / kBN : 0;

  int enter_c = INT_MIN;   // sentinel: sees the prefix only
  if constexpr (MASK == kMaskTree) {
    const int c = t + tree_len - qo_len;
    if (row_ok && c >= 0 && c < tree_len && tree_base + c >= 0 && tree_base + c < p.tree_size)
      enter_c = p.tree_order[2 * (tree_base + c)];
  }

  // ---- rotary frequency table ----
  const bool any_rope = p.rope_q | p.rope_k;
  if (any_rope) {
    if (tid < D / 2) inv_freq_s[tid] = exp2(-(2.0 * tid / D) * p.log2_theta);
    __syncthreads();
  }

  // ---- Q fragments: lane holds row R, dims 16*s + 8*hh + [0, 8) ----
  u32x4 qf[D / 16];
#pragma unroll
  for (int s = 0; s < D / 16; ++s) qf[s] = u32x4{0, 0, 0, 0};
  if (row_ok) {
    const uint16_t* qrow = p.q + (static_cast<size_t>(q0 + t) * p.h_q + head) * D + 8 * hh;
#pragma unroll
    for (int s = 0; s < D / 16; ++s) qf[s] = *reinterpret_cast<const u32x4*>(qrow + 16 * s);
  }

  // ---- K/V tile staging ----
  const int kpc = tid % HC;          // K: chunk pair (chunks kpc and kpc + HC)
  const int kkey = tid / HC;         // K: first row, then + KSTEP
  const bool v_active = tid < VUNITS;
  const int vg = tid & 15;           // V: 4-key group
  const int vc = tid >> 4;           // V: chunk

  // storage offset of chunk position kidx (sliding window: sink, then window)
  auto seq_off = [&](int kidx) -> int {
    return (p.sliding && kidx >= sink) ? kidx - sink + win_off : kidx;
  };
  // page holding chunk position kidx, or -1 (paged layout only)
  auto page_of = [&](int kidx) -> int {
    if (kidx >= kv_len) return -1;
    const int off = seq_off(kidx);
    if (off < 0) return -1;
    const int pi = page_base + (off >> 4);
    if (pi < 0 || pi >= page_end) return -1;
    const int page = p.page_values[pi];
    return static_cast<unsigned>(page) < static_cast<unsigned>(p.num_pages) ? page : -1;
  };
  // Page numbers of this thread's K and V rows in the next tile to load,
  // fetched one tile ahead of the K/V loads that use them.
  int kpage[KP], vpage[4];
  auto fetch_pages = [&](int j0) {
    if constexpr (LAYOUT == kPaged) {
#pragma unroll
      for (int i = 0; i < KP; ++i) kpage[i] = page_of(j0 + kkey + i * KSTEP);
#pragma unroll
      for (int k = 0; k < 4; ++k) vpage[k] = v_active ? page_of(j0 + 4 * vg + k) : -1;
    }
  };
  auto kv_row = [&](int kidx, int which, int page) -> const uint16_t* {
    if (kidx >= kv_len) return nullptr;
    if constexpr (LAYOUT == kContiguous) {
      const int r = kv_base + kidx;
      if (r < 0 || r >= p.total_kv) return nullptr;
      return (which ? p.v : p.k) + (static_cast<size_t>(r) * p.h_kv + kvh) * D;
    } else {
      if (page < 0) return nullptr;
      return p.pages + (((static_cast<size_t>(page) * 2 + which) * p.h_kv + kvh) * 16 + (seq_off(kidx) & 15)) * D;
    }
  };

  u32x4 klo[KP], khi[KP];
  u32x4 vreg[4];
  int tree_e = 0, tree_x = 0;

  // global loads of one K/V tile into registers (pages from fetch_pages)
  auto load_tile = [&](int j0) {
#pragma unroll
    for (int i = 0; i < KP; ++i) {
      const uint16_t* src = kv_row(j0 + kkey + i * KSTEP, 0, kpage[i]);
      if (src) {
        klo[i] = *reinterpret_cast<const u32x4*>(src + 8 * kpc);
        khi[i] = *reinterpret_cast<const u32x4*>(src + 8 * (kpc + HC));
      } else {
        klo[i] = u32x4{0, 0, 0, 0};
        khi[i] = u32x4{0, 0, 0, 0};
      }
    }
    if (v_active) {
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const uint16_t* src = kv_row(j0 + 4 * vg + k, 1, vpage[k]);
        vreg[k] = src ? *reinterpret_cast<const u32x4*>(src + 8 * vc) : u32x4{0, 0, 0, 0};
      }
    }
    if constexpr (MASK == kMaskTree) {
      if (tid < kBN) {
        const int kidx = j0 + tid;
        if (kidx >= kv_len) {
          tree_e = INT_MAX; tree_x = INT_MIN;
        } else if (kidx < tree_start) {
          tree_e = INT_MIN; tree_x = INT_MAX;
        } else {
          const int idx = tree_base + (kidx - tree_start);
          if (idx >= 0 && idx < p.tree_size) {
            tree_e = p.tree_order[2 * idx];
            tree_x = p.tree_order[2 * idx + 1];
          } else {
            tree_e = INT_MAX; tree_x = INT_MIN;
          }
        }
      }
    }
  };

  // rotate the staged K rows in registers (this thread holds both halves)
  auto rope_k_tile = [&](int j0) {
#pragma unroll
    for (int i = 0; i < KP; ++i) {
      const int kidx = j0 + kkey + i * KSTEP;
      if (kidx < kv_len) {
        int pos;
        if constexpr (LAYOUT == kContiguous) {
          const int pi = kv_base + kidx;   // K positions share the query position array
          pos = (pi >= 0 && pi < p.total_q) ? p.q_rope_position[pi] : 0;
        } else {
          pos = p.k_rope_pos_offset[b] + kidx;
        }
        u32x4 lo, hi;
#pragma unroll
        for (int e = 0; e < 8; e += 2) {
          float y1[2], y2[2];
#pragma unroll
          for (int u = 0; u < 2; ++u) {
            float cs, sn;
            rope_cos_sin(pos, p.rope_scale, inv_freq_s[8 * kpc + e + u], cs, sn);
            rope_pair(cs, sn, to_f32<BF>(half_of(klo[i], e + u)), to_f32<BF>(half_of(khi[i], e + u)),
                      y1[u], y2[u]);
          }
          lo[e >> 1] = pack2<BF>(y1[0], y1[1]);
          hi[e >> 1] = pack2<BF>(y2[0], y2[1]);
        }
        klo[i] = lo;
        khi[i] = hi;
      }
    }
  };

  auto store_tile = [&](int bufi) {
    char* buf = smem + bufi * BUF;
#pragma unroll
    for (int i = 0; i < KP; ++i) {
      char* row = buf + K_OFF + (kkey + i * KSTEP) * KS;
      *reinterpret_cast<u32x4*>(row + kpc * 16) = klo[i];
      *reinterpret_cast<u32x4*>(row + (kpc + HC) * 16) = khi[i];
    }
    if (v_active) {
      // keys 4*vg..4*vg+3 -> V^T positions: within each group of 16 keys the
      // 4-key quarters are stored in the order 0, 2, 1, 3
      const int q4 = vg & 3;
      const int pos = 16 * (vg >> 2) + 4 * (((q4 & 1) << 1) | (q4 >> 1));
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        u32x2 val;
        val[0] = half_of(vreg[0], e) | (half_of(vreg[1], e) << 16);
        val[1] = half_of(vreg[2], e) | (half_of(vreg[3], e) << 16);
        *reinterpret_cast<u32x2*>(buf + V_OFF + (8 * vc + e) * VS + pos * 2) = val;
      }
    }
    if constexpr (MASK == kMaskTree) {
      if (tid < kBN) *reinterpret_cast<int2*>(buf + T_OFF + tid * 8) = make_int2(tree_e, tree_x);
    }
  };

  // first K/V tile in flight before the Q rotation
  if (n_tiles > 0) {
    fetch_pages(0);
    load_tile(0);
    if (n_tiles > 1) fetch_pages(kBN);
  }

  // ---- RoPE on Q: a cos/sin table per (token of this tile, frequency) in
  // the tile buffers, shared by the g heads of each token ----
  if (p.rope_q) {
    const int t_first = row0 / g;
    const int t_end = min((row0 + kBM - 1) / g + 1, qo_len);
    const int n_entries = max(t_end - t_first, 0) * (D / 2);
    float2* tab = reinterpret_cast<float2*>(smem);
    for (int e = tid; e < n_entries; e += kThreads) {
      const int tl = e / (D / 2);
      const int kf = e - tl * (D / 2);
      const int qi = q0 + t_first + tl;
      const int pos = (qi >= 0 && qi < p.total_q) ? p.q_rope_position[qi] : 0;
      float cs, sn;
      rope_cos_sin(pos, p.rope_scale, inv_freq_s[kf], cs, sn);
      tab[e] = make_float2(cs, sn);
    }
    __syncthreads();
    if (row_ok) {
      const float2* trow = tab + (t - t_first) * (D / 2);
#pragma unroll
      for (int s = 0; s < D / 32; ++s) {
        const u32x4 a = qf[s], c2 = qf[s + D / 32];
#pragma unroll
        for (int e = 0; e < 8; e += 2) {
          float y1[2], y2[2];
#pragma unroll
          for (int u = 0; u < 2; ++u) {
            const float2 cs = trow[16 * s + 8 * hh + e + u];
            rope_pair(cs.x, cs.y, to_f32<BF>(half_of(a, e + u)), to_f32<BF>(half_of(c2, e + u)),
                      y1[u], y2[u]);
          }
          qf[s][e >> 1] = pack2<BF>(y1[0], y1[1]);
          qf[s + D / 32][e >> 1] = pack2<BF>(y2[0], y2[1]);
        }
      }
    }
    __syncthreads();   // the tile buffers are reused for K/V below
  }

  // ---- online softmax state (row R; both half-waves carry it) ----
  float m_run = -INFINITY;   // reference max (log2 domain), shared by both halves
  float l_run = 0.f;
  f32x16 o[D / 32];
#pragma unroll
  for (int i = 0; i < D / 32; ++i) o[i] = f32x16{};
  const float sc = p.sm_scale_log2;

  if (n_tiles > 0) {
    if (p.rope_k) rope_k_tile(0);
    store_tile(0);
  }
  __syncthreads();

  for (int it = 0; it < n_tiles; ++it) {
    const int j0 = it * kBN;
    if (it + 1 < n_tiles) {
      load_tile(j0 + kBN);
      if (it + 2 < n_tiles) fetch_pages(j0 + 2 * kBN);
    }
    const char* buf = smem + (it & 1) * BUF;

    // tile class for this wave: 0 skip, 1 full, 2 partial
    int cls;
    if constexpr (MASK == kMaskTree) {
      cls = (j0 + kBN <= min(tree_start, kv_len)) ? 1 : 2;
    } else {
      cls = (j0 >= lim_hi) ? 0 : ((j0 + kBN <= lim_lo) ? 1 : 2);
    }

    if (wave_active && cls != 0) {
      f32x16 sacc[2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        sacc[kb] = f32x16{};
        const char* kp = buf + K_OFF + (32 * kb + r32) * KS + 16 * hh;
#pragma unroll
        for (int s = 0; s < D / 16; ++s)
          sacc[kb] = mma32<BF>(*reinterpret_cast<const u32x4*>(kp + 32 * s), qf[s], sacc[kb]);
      }
      if (cls == 2) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int kl = 32 * kb + 8 * (r >> 2) + 4 * hh + (r & 3);
            bool vis;
            if constexpr (MASK == kMaskTree) {
              const int2 iv = *reinterpret_cast<const int2*>(buf + T_OFF + kl * 8);
              vis = enter_c >= iv.x && enter_c < iv.y;
            } else {
              vis = j0 + kl < lim;
            }
            if (!vis) sacc[kb][r] = -INFINITY;
          }
        }
      }
      float mx = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sacc[kb][r]);
      mx = pair_max(mx) * sc;
      // The O / l rescale is skipped when no row of the wave has a new max.
      const bool grow = mx > m_run;
      if (__any(grow)) {
        const float m_new = grow ? mx : m_run;
        // rows still without a visible key keep O = l = 0 (alpha 0, never NaN)
        const float alpha = __builtin_amdgcn_exp2f(m_run - (m_new == -INFINITY ? 0.f : m_new));
        m_run = m_new;
        l_run *= alpha;
#pragma unroll
        for (int i = 0; i < D / 32; ++i) o[i] *= alpha;
      }
      const float m_use = (m_run == -INFINITY) ? 0.f : m_run;
      float lsum = 0.f;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float pv = __builtin_amdgcn_exp2f(fmaf(sacc[kb][r], sc, -m_use));
          sacc[kb][r] = pv;
          lsum += pv;
        }
      l_run += lsum;
#pragma unroll
      for (int sp = 0; sp < kBN / 16; ++sp) {
        const f32x16& sa = sacc[sp >> 1];
        const int e0 = 8 * (sp & 1);
        u32x4 pf;
#pragma unroll
        for (int u = 0; u < 4; ++u) pf[u] = pack2<BF>(sa[e0 + 2 * u], sa[e0 + 2 * u + 1]);
        const char* vp = buf + V_OFF + r32 * VS + 32 * sp + 16 * hh;
#pragma unroll
        for (int db = 0; db < D / 32; ++db)
          o[db] = mma32<BF>(*reinterpret_cast<const u32x4*>(vp + 32 * db * VS), pf, o[db]);
      }
    }
    if (it + 1 < n_tiles) {
      if (p.rope_k) rope_k_tile(j0 + kBN);
      store_tile((it + 1) & 1);
    }
    __syncthreads();
  }

  // ---- epilogue: out = O / l (dtype), lse = m + log2(l) ----
  const float l_tot = pair_sum(l_run);
  if (row_ok) {
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
    uint16_t* orow = static_cast<uint16_t*>(p.out) + (static_cast<size_t>(q0 + t) * p.h_q + head) * D;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int jb = 0; jb < 4; ++jb) {
        u32x2 val;
        val[0] = pack2<BF>(o[db][4 * jb + 0] * inv, o[db][4 * jb + 1] * inv);
        val[1] = pack2<BF>(o[db][4 * jb + 2] * inv, o[db][4 * jb + 3] * inv);
        *reinterpret_cast<u32x2*>(orow + 32 * db + 8 * jb + 4 * hh) = val;
      }
    if (hh == 0)
      p.lse[static_cast<size_t>(q0 + t) * p.h_q + head] = l_tot > 0.f ? m_run + log2f(l_tot) : -INFINITY;
  }
}

template <bool BF, int D>
hipError_t launch_d(const AttnParams& p, KvLayout layout, MaskKind mask, dim3 grid,
                    hipStream_t stream) {
  if (layout == kContiguous) {
    if (mask == kMaskTree)
      hipLaunchKernelGGL((attn_fwd_kernel<BF, D, kContiguous, kMaskTree>), grid, dim3(kThreads), 0, stream, p);
    else
      hipLaunchKernelGGL((attn_fwd_kernel<BF, D, kContiguous, kMaskCausal>), grid, dim3(kThreads), 0, stream, p);
  } else {
    if (mask == kMaskTree)
      hipLaunchKernelGGL((attn_fwd_kernel<BF, D, kPaged, kMaskTree>), grid, dim3(kThreads), 0, stream, p);
    else
      hipLaunchKernelGGL((attn_fwd_kernel<BF, D, kPaged, kMaskCausal>), grid, dim3(kThreads), 0, stream, p);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attn(const AttnParams& p, int is_bf16, int head_dim, KvLayout layout,
                       MaskKind mask, hipStream_t stream) {
  // Upper bound on the number of work items, plus slack so that the
  // XCD-contiguous mapping (8 * ceil(items / 8) blocks) always fits.
  const long tiles = (static_cast<long>(p.total_q) * p.group + kBM - 1) / kBM + p.batch;
  long blocks = tiles * p.h_kv + 7;
  blocks = (blocks + 7) / 8 * 8;
  if (blocks > INT_MAX) return hipErrorInvalidValue;
  const dim3 grid(static_cast<unsigned>(blocks));
  if (is_bf16) {
    return head_dim == 128 ? launch_d<true, 128>(p, layout, mask, grid, stream)
                           : launch_d<true, 64>(p, layout, mask, grid, stream);
  }
  return head_dim == 128 ? launch_d<false, 128>(p, layout, mask, grid, stream)
                         : launch_d<false, 64>(p, layout, mask, grid, stream);
}

}  // namespace ra
