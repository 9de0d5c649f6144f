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
//    max and row sum are in-lane plus one v_permlane32_swap, and the fp32
//    accumulators convert in place into the B operand of O^T += V^T P^T.
//  * Q stays in registers (RoPE applied on load, from a per-tile cos/sin
//    table shared by the g heads of a token).
//  * K and V tiles (64 keys) go from HBM straight into LDS with
//    global_load_lds_dwordx4 (no staging registers), two stages deep, as
//    row-major tiles whose 16-byte chunks are XOR-swizzled per row. The LDS
//    serves 256 bytes (64 banks) per clock; with rr = the row's index in
//    256-byte units, K chunk c sits at c ^ (rr mod 16 chunks) so the b128
//    K-operand reads of 16 consecutive rows hit distinct banks, and V chunk
//    c sits at c ^ 4(rr mod 4) so ds_read_b64_tr_b16 (which returns 4
//    consecutive keys of one dim per lane) reads 4 rows x 32 bytes per
//    16-lane group without conflicts (both measured). With in-kernel K RoPE
//    the K tile is rotated in registers and written instead.
//  * Masks are classified per (wave, tile): skipped, full (no test) or
//    partial (per-element test); causal work stops at the last visible tile.
//    Tree intervals of the sequence are staged in LDS once.
//  * The softmax runs in the log2 domain (v_exp_f32 is exp2): scores are
//    scaled by sm_scale*log2(e), lse = m + log2(l) as on the pages; the O
//    rescale is skipped when no row of the wave has a new max.

#include <climits>
#include <cmath>
#include <type_traits>

#include "device_common.h"
#include "ra_internal.h"

namespace ra {

namespace {

typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4i16 lds_v4i16;

constexpr int kStages = 2;
constexpr int kTreeLds = 1024;   // tree nodes whose (enter, exit) are staged in LDS

// 16 bytes per lane from global memory straight into LDS: lane l's bytes land
// at lds_base + 16*l (lds_base wave-uniform, passed in M0). Issued through
// inline asm so the compiler does not treat these asynchronous LDS writes as
// aliasing every later LDS read (it would wait for them before each read and
// undo the prefetch); wait_all_and_barrier() orders them explicitly.
__device__ __forceinline__ void dma16(const void* gptr, const void* lds_base) {
  const unsigned lds = static_cast<unsigned>(
      reinterpret_cast<size_t>((__attribute__((address_space(3))) const char*)lds_base));
  asm volatile("global_load_lds_dwordx4 %0, off" ::"v"(gptr), "{m0}"(lds) : "memory");
}

// Wait for this wave's outstanding global loads (including loads into LDS)
// and LDS accesses, then the workgroup barrier. Written out because the
// compiler neither tracks loads into LDS nor should it fence in between.
__device__ __forceinline__ void wait_all_and_barrier() {
  asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
  // Free (everything has retired), but visible to the compiler: loads it
  // tracks need no further waits before the next DMA is issued.
  __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0)
}

// Locate this workgroup's work item. Returns false when the block has none.
// Item list: for each sequence b (in order), for each KV head, ranks
// 0..tiles_b-1 with rank 0 = the last (heaviest under a causal mask) q-tile.
__device__ bool locate_item(const int32_t* q_indptr, int batch, int group, int h_kv, int& b,
                            int& kvh, int& tile) {
  const int lane = threadIdx.x & 63;
  int total = 0;
  for (int c0 = 0; c0 < batch; c0 += 64) {
    const int i = c0 + lane;
    int cnt = 0;
    if (i < batch) {
      const int len = max(q_indptr[i + 1] - q_indptr[i], 0);
      cnt = ((len * group + kBM - 1) / kBM) * h_kv;
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
  for (int c0 = 0; c0 < batch; c0 += 64) {
    const int i = c0 + lane;
    int cnt = 0;
    if (i < batch) {
      const int len = max(q_indptr[i + 1] - q_indptr[i], 0);
      cnt = ((len * group + kBM - 1) / kBM) * h_kv;
    }
    const int incl = wave_inclusive_scan(cnt) + base;
    const unsigned long long hit = __ballot(i < batch && item < incl);
    if (hit) {
      const int l = __ffsll(static_cast<long long>(hit)) - 1;
      b = c0 + l;
      const int excl = __shfl(incl - cnt, l, 64);
      const int tiles_b = __shfl(cnt, l, 64) / h_kv;
      const int local = item - excl;
      kvh = local / tiles_b;
      tile = tiles_b - 1 - (local - kvh * tiles_b);
      return true;
    }
    base = __shfl(incl, 63, 64);
  }
  return false;
}

template <bool BF, int D, int LAYOUT, int MASK, bool ROPE_K>
__global__ __launch_bounds__(kThreads, 2) void attn_fwd_kernel(AttnParams p) {
  constexpr int RB = D * 2;                  // bytes per head row
  constexpr int CH = D / 8;                  // 16-byte chunks per row
  constexpr int TILE = kBN * RB;             // bytes of one K or V tile
  constexpr int STAGE = 2 * TILE;            // K tile, then V tile
  constexpr int RPL = 1024 / RB;             // rows one wave-wide 16-byte load covers
  constexpr int LOADS = kBN / (4 * RPL);     // per wave and tile, for K and for V each
  constexpr int TREE_OFF = kStages * STAGE;
  constexpr int SMEM = TREE_OFF + (MASK == kMaskTree ? kTreeLds * 8 : 0);
  static_assert(LOADS >= 1 && 4 * RPL * LOADS == kBN, "tile shape");
  static_assert((STAGE & (STAGE - 1)) == 0, "stage size is a power of two");
  // LDS chunk swizzles (see the header comment): K chunk c of row r sits at
  // c ^ KSWZ(r), V chunk c at c ^ VSWZ(r); RSH = log2(rows per 256 bytes).
  constexpr int RSH = (D == 64) ? 1 : 0;
#define KSWZ(r) ((((r) >> RSH)) & (CH - 1))
#define VSWZ(r) (4 * ((((r) >> RSH)) & (CH / 4 - 1)))
  // the Q RoPE table holds at most 128 tokens x D/2 frequencies of float2
  static_assert(128 * (D / 2) * 8 <= kStages * STAGE, "RoPE table fits in the stages");

  __shared__ __attribute__((aligned(1024))) char smem[SMEM];
  __shared__ double inv_freq_s[D / 2];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  // wave index as a scalar, so per-wave bounds and tile classes are uniform
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int r32 = lane & 31;
  const int hh = lane >> 5;

  // kernel arguments as scalars (nothing below takes the address of p)
  const auto q_ = p.q;
  const auto q_indptr_ = p.q_indptr;
  const auto out_ = p.out;
  const auto lse_ = p.lse;
  const auto k_ = p.k;
  const auto v_ = p.v;
  const auto kv_indptr_ = p.kv_indptr;
  const auto pages_ = p.pages;
  const auto page_indptr_ = p.page_indptr;
  const auto page_values_ = p.page_values;
  const auto length_info_ = p.length_info;
  const auto k_rope_pos_offset_ = p.k_rope_pos_offset;
  const auto tree_indptr_ = p.tree_indptr;
  const auto tree_order_ = p.tree_order;
  const auto q_rope_position_ = p.q_rope_position;
  const auto batch_ = p.batch;
  const auto total_q_ = p.total_q;
  const auto total_kv_ = p.total_kv;
  const auto tree_size_ = p.tree_size;
  const auto h_q_ = p.h_q;
  const auto h_kv_ = p.h_kv;
  const auto group_ = p.group;
  const auto num_pages_ = p.num_pages;
  const auto nnz_pages_ = p.nnz_pages;
  const auto sliding_ = p.sliding;
  const auto causal_ = p.causal;
  const auto rope_q_ = p.rope_q;
  const auto rope_k_ = p.rope_k;
  const auto rope_scale_ = p.rope_scale;
  const auto sm_scale_log2_ = p.sm_scale_log2;
  const auto log2_theta_ = p.log2_theta;

  int b = 0, kvh = 0, tile = 0;
  if (!locate_item(q_indptr_, batch_, group_, h_kv_, b, kvh, tile)) return;   // uniform over the workgroup
  b = __builtin_amdgcn_readfirstlane(b);
  kvh = __builtin_amdgcn_readfirstlane(kvh);
  tile = __builtin_amdgcn_readfirstlane(tile);

  const int g = group_;
  const int q0 = q_indptr_[b];
  const int qo_len = q_indptr_[b + 1] - q0;
  const int row0 = tile * kBM;

  // ---- KV chunk of this sequence ----
  int kv_len_m = 0, kv_base_m = 0, page_base_m = 0, page_end_m = 0, sink_m = 0, win_off_m = 0;
  if constexpr (LAYOUT == kContiguous) {
    kv_base_m = kv_indptr_[b];
    kv_len_m = kv_indptr_[b + 1] - kv_base_m;
  } else {
    page_base_m = page_indptr_[b];
    page_end_m = min(page_indptr_[b + 1], nnz_pages_);
    const int np = page_indptr_[b + 1] - page_base_m;
    if (np > 0) {
      if (!sliding_) {
        kv_len_m = (np - 1) * 16 + length_info_[b];
      } else {
        win_off_m = length_info_[batch_ + b];
        sink_m = length_info_[2 * batch_ + b];
        kv_len_m = (np - 1) * 16 + length_info_[b] - win_off_m + sink_m;
      }
    }
  }
  const int kv_len = max(kv_len_m, 0);
  const int kv_base = kv_base_m, page_base = page_base_m, page_end = page_end_m;
  const int sink = sink_m, win_off = win_off_m;

  int tree_base_m = 0, tree_len_m = 0;
  if constexpr (MASK == kMaskTree) {
    tree_base_m = tree_indptr_[b];
    tree_len_m = max(tree_indptr_[b + 1] - tree_base_m, 0);
  }
  const int tree_base = tree_base_m, tree_len = tree_len_m;
  const int tree_start = kv_len - tree_len;
  const bool tree_in_lds = tree_len <= kTreeLds;   // uniform

  // ---- this lane's query row ----
  const int R = row0 + w * 32 + r32;
  const int t = R / g;
  const int head = kvh * g + (R - t * g);
  const bool row_ok = t < qo_len && q0 + t >= 0 && q0 + t < total_q_;
  const int t_lo = (row0 + w * 32) / g;
  const int t_hi = min((row0 + w * 32 + 31) / g, qo_len - 1);
  const bool wave_active = t_lo < qo_len;

  const bool causal = (MASK == kMaskCausal) && causal_;
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
    if (row_ok && c >= 0 && c < tree_len && tree_base + c >= 0 && tree_base + c < tree_size_)
      enter_c = tree_order_[2 * (tree_base + c)];
  }

  // ---- rotary frequency table ----
  if (rope_q_ | rope_k_) {
    if (tid < D / 2) inv_freq_s[tid] = exp2(-(2.0 * tid / D) * log2_theta_);
    __syncthreads();
  }

  // ---- Q fragments: lane holds row R, dims 16*s + 8*hh + [0, 8) ----
  u32x4 qf[D / 16];
#pragma unroll
  for (int s = 0; s < D / 16; ++s) qf[s] = u32x4{0, 0, 0, 0};
  if (row_ok) {
    const uint16_t* qrow = q_ + (static_cast<size_t>(q0 + t) * h_q_ + head) * D + 8 * hh;
#pragma unroll
    for (int s = 0; s < D / 16; ++s) qf[s] = *reinterpret_cast<const u32x4*>(qrow + 16 * s);
  }

  // ---- K/V tile loads: wave w fills tile rows [16w, 16w + 16); lane covers
  // rows 16w + RPL*i + lane/CH (i < LOADS) at physical chunk lane % CH ----
  const int pc = lane % CH;
  const int lrow = lane / CH;
  auto tile_row = [&](int i) __attribute__((always_inline)) { return 16 * w + RPL * i + lrow; };
  const int delta = sliding_ ? win_off - sink : 0;   // window: storage offset - position
  // Page numbers are wave-uniform scalars: the 16 rows [B, B + 16) a wave
  // loads (B = j0 + 16w, 16-aligned) touch at most three pages: the page of
  // sink positions (storage offset = position) and the two pages that the
  // window offsets starting at max(B, sink) + delta can straddle.
  // The loaded page numbers are only inspected when the next tile is issued
  // (after the barrier): validating them right after the load would make the
  // compiler wait for all outstanding loads, including the K/V prefetch.
  struct PageSet {
    int ia, ib, ic;   // page_values indices (wave-uniform)
    int va, vb, vc;   // raw page numbers loaded from them
    int offb;         // first window storage offset of the block
  };
  auto load_page = [&](int pidx) __attribute__((always_inline)) -> int {
    return page_values_[min(max(pidx, 0), nnz_pages_ - 1)];   // in bounds; checked at use
  };
  auto fetch_pages = [&](int j0) __attribute__((always_inline)) -> PageSet {
    PageSet ps{-1, -1, -1, 0, 0, 0, 0};
    if constexpr (LAYOUT == kPaged) {
      const int B = j0 + 16 * w;
      ps.offb = (sliding_ ? max(B, sink) : B) + delta;
      ps.ia = (sliding_ && B < sink) ? page_base + (B >> 4) : -1;
      ps.ib = page_base + (ps.offb >> 4);
      ps.ic = (ps.offb & 15) ? ps.ib + 1 : -1;
      ps.va = load_page(ps.ia);
      ps.vb = load_page(ps.ib);
      ps.vc = load_page(ps.ic);
    }
    return ps;
  };
  auto page_ok = [&](int idx, int val) __attribute__((always_inline)) -> bool {
    return idx >= page_base && idx < page_end &&
           static_cast<unsigned>(val) < static_cast<unsigned>(num_pages_);
  };
  PageSet pages_next{-1, -1, -1, 0, 0, 0, 0};   // pages of the next tile to load
  // byte address of the head row of chunk position kidx (K: which = 0, V: 1)
  const size_t kv_stride = static_cast<size_t>(h_kv_) * RB;              // contiguous: per token
  const size_t page_stride = static_cast<size_t>(2) * h_kv_ * 16 * RB;   // paged: per page
  const char* kv_head_k;
  const char* kv_head_v;
  if constexpr (LAYOUT == kContiguous) {
    kv_head_k = reinterpret_cast<const char*>(k_) + (static_cast<size_t>(kv_base) * h_kv_ + kvh) * RB;
    kv_head_v = reinterpret_cast<const char*>(v_) + (static_cast<size_t>(kv_base) * h_kv_ + kvh) * RB;
  } else {
    kv_head_k = reinterpret_cast<const char*>(pages_) + static_cast<size_t>(kvh) * 16 * RB;
    kv_head_v = kv_head_k + static_cast<size_t>(h_kv_) * 16 * RB;
  }
  auto row_addr = [&](int kidx, int which, PageSet ps) __attribute__((always_inline)) -> const char* {
    const char* base = which ? kv_head_v : kv_head_k;
    if (kidx >= kv_len) return nullptr;
    if constexpr (LAYOUT == kContiguous) {
      const int r = kv_base + kidx;
      if (r < 0 || r >= total_kv_) return nullptr;
      return base + static_cast<size_t>(kidx) * kv_stride;
    } else {
      const bool in_sink = sliding_ && kidx < sink;
      const int off = in_sink ? kidx : kidx + delta;
      // values, not an indexed struct (which the compiler would put in memory)
      const int ia = ps.ia, ib = ps.ib, ic = ps.ic, va = ps.va, vb = ps.vb, vc = ps.vc;
      const bool second = (off >> 4) != (ps.offb >> 4);
      const int idx = in_sink ? ia : (second ? ic : ib);
      const int page = in_sink ? va : (second ? vc : vb);
      if (!page_ok(idx, page)) return nullptr;
      return base + static_cast<size_t>(page) * page_stride + (off & 15) * RB;
    }
  };

  // One address and one exec region per row for both K and V.
  const size_t v_minus_k = static_cast<size_t>(kv_head_v - kv_head_k);
  auto issue_tile = [&](int j0, char* stage) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < LOADS; ++i) {
      const int r = tile_row(i);
      char* dst_k = stage + (16 * w + RPL * i) * RB;          // wave-uniform
      const char* src = row_addr(j0 + r, 0, pages_next);
      if (src) {
        if constexpr (!ROPE_K)
          dma16(src + 16 * (pc ^ KSWZ(r)), dst_k);
        dma16(src + v_minus_k + 16 * (pc ^ VSWZ(r)), dst_k + TILE);
      }
    }
  };

  // In-kernel K RoPE: K goes through registers (same lanes and rows as the
  // direct loads); the partner chunk (dims +- D/2) is in lane ^ (CH/2).
  u32x4 kreg[ROPE_K ? LOADS : 1];
  auto load_k_regs = [&](int j0) __attribute__((always_inline)) {
    if constexpr (ROPE_K) {
#pragma unroll
      for (int i = 0; i < LOADS; ++i) {
        const int r = tile_row(i);
        const char* src = row_addr(j0 + r, 0, pages_next);
        kreg[i] = src ? *reinterpret_cast<const u32x4*>(src + 16 * (pc ^ KSWZ(r))) : u32x4{0, 0, 0, 0};
      }
    }
  };
  auto rope_store_k = [&](int j0, char* stage) __attribute__((always_inline)) {
    if constexpr (ROPE_K) {
#pragma unroll
      for (int i = 0; i < LOADS; ++i) {
        const int r = tile_row(i);
        const int kidx = j0 + r;
        const int lc = pc ^ KSWZ(r);               // logical chunk held
        u32x4 other;
#pragma unroll
        for (int u = 0; u < 4; ++u) other[u] = __shfl_xor(kreg[i][u], CH / 2, 64);
        u32x4 res = kreg[i];
        if (kidx < kv_len) {
          int pos;
          if constexpr (LAYOUT == kContiguous) {
            const int pi = kv_base + kidx;   // K positions share the query position array
            pos = (pi >= 0 && pi < total_q_) ? q_rope_position_[pi] : 0;
          } else {
            pos = k_rope_pos_offset_[b] + kidx;
          }
          const bool first = lc < CH / 2;
#pragma unroll
          for (int e = 0; e < 8; e += 2) {
            float y[2];
#pragma unroll
            for (int u = 0; u < 2; ++u) {
              float cs, sn, y1, y2;
              rope_cos_sin(pos, rope_scale_, inv_freq_s[(8 * lc + e + u) & (D / 2 - 1)], cs, sn);
              const float x = to_f32<BF>(half_of(kreg[i], e + u));
              const float xp = to_f32<BF>(half_of(other, e + u));
              if (first) { rope_pair(cs, sn, x, xp, y1, y2); y[u] = y1; }
              else { rope_pair(cs, sn, xp, x, y1, y2); y[u] = y2; }
            }
            res[e >> 1] = pack2<BF>(y[0], y[1]);
          }
        }
        *reinterpret_cast<u32x4*>(stage + r * RB + 16 * pc) = res;
      }
    }
  };

  // ---- RoPE on Q: a cos/sin table per (token of this tile, frequency) in
  // the stage buffers, shared by the g heads of each token ----
  if (rope_q_) {
    const int t_first = row0 / g;
    const int t_end = min((row0 + kBM - 1) / g + 1, qo_len);
    const int n_entries = max(t_end - t_first, 0) * (D / 2);
    float2* tab = reinterpret_cast<float2*>(smem);
    for (int e = tid; e < n_entries; e += kThreads) {
      const int tl = e / (D / 2);
      const int kf = e - tl * (D / 2);
      const int qi = q0 + t_first + tl;
      const int pos = (qi >= 0 && qi < total_q_) ? q_rope_position_[qi] : 0;
      float cs, sn;
      rope_cos_sin(pos, rope_scale_, inv_freq_s[kf], cs, sn);
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
    __syncthreads();   // the stage buffers are reused below
  }

  // ---- clear the stages (rows a load skips must hold finite values), stage
  // the tree intervals ----
  for (int off = tid * 16; off < kStages * STAGE; off += kThreads * 16)
    *reinterpret_cast<u32x4*>(smem + off) = u32x4{0, 0, 0, 0};
  if constexpr (MASK == kMaskTree) {
    int2* tl = reinterpret_cast<int2*>(smem + TREE_OFF);
    const int n_st = min(tree_len, kTreeLds);
    for (int n = tid; n < n_st; n += kThreads) {
      const int idx = tree_base + n;
      tl[n] = (idx >= 0 && idx < tree_size_)
                  ? make_int2(tree_order_[2 * idx], tree_order_[2 * idx + 1])
                  : make_int2(INT_MAX, INT_MIN);
    }
  }
  __syncthreads();

  // per-lane LDS byte offsets of the MFMA operands
  int koff[D / 16];   // K rows 32*kb + r32: logical chunk 2s + hh
#pragma unroll
  for (int s = 0; s < D / 16; ++s) koff[s] = r32 * RB + 16 * ((2 * s + hh) ^ KSWZ(r32));
  int voff[D / 32];   // V pieces for ds_read_b64_tr_b16 (16-lane groups)
  {
    const int gi = lane & 15, grp = lane >> 4;
    const int vrow = 4 * hh + (gi >> 2);           // + 16*sp (+ 8 for the second read)
#pragma unroll
    for (int db = 0; db < D / 32; ++db) {
      const int dim = 32 * db + 16 * (grp & 1) + 4 * (gi & 3);
      const int lc = dim >> 3;
      voff[db] = TILE + vrow * RB + 16 * (lc ^ VSWZ(vrow)) + 2 * (dim & 7);
    }
  }

  // ---- online softmax state (row R; both half-waves carry it) ----
  float m_run = -INFINITY;
  float l_run = 0.f;
  f32x16 o[D / 32];
#pragma unroll
  for (int i = 0; i < D / 32; ++i) o[i] = f32x16{};
  const float sc = sm_scale_log2_;

  // Retire every load the compiler tracks (Q rows, tree intervals) before the
  // first LDS DMA: a wait the compiler placed for them inside the loop would
  // also count the untracked DMAs and stall on the prefetch.
  __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0)
  if (n_tiles > 0) {
    pages_next = fetch_pages(0);
    issue_tile(0, smem);
    load_k_regs(0);
    if (n_tiles > 1) pages_next = fetch_pages(kBN);   // pages of tile 1
    rope_store_k(0, smem);
  }

  // One KV tile: S^T = K Q^T, mask, online softmax, O^T += V^T P^T.
  auto compute = [&](int j0, bool masked) __attribute__((always_inline)) {
    f32x16 sacc[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      sacc[kb] = f32x16{};
#pragma unroll
      for (int s = 0; s < D / 16; ++s)
        sacc[kb] = mma32<BF>(*reinterpret_cast<const u32x4*>(smem + kb * 32 * RB + koff[s]), qf[s], sacc[kb]);
    }
    if (masked) {   // uniform: only partial tiles test each element
      asm volatile("");   // keeps this a branch (the compiler would otherwise select)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int kidx = j0 + 32 * kb + 8 * (r >> 2) + 4 * hh + (r & 3);
          bool vis;
          if constexpr (MASK == kMaskTree) {
            vis = kidx < kv_len;
            if (vis && kidx >= tree_start) {
              const int n = kidx - tree_start;
              int2 iv;
              if (tree_in_lds) {
                iv = reinterpret_cast<const int2*>(smem + TREE_OFF)[n];
              } else {   // trees larger than the LDS copy: read the intervals directly
                const int idx = tree_base + n;
                iv = (idx < tree_size_) ? make_int2(tree_order_[2 * idx], tree_order_[2 * idx + 1])
                                         : make_int2(INT_MAX, INT_MIN);
              }
              vis = enter_c >= iv.x && enter_c < iv.y;
            }
          } else {
            vis = kidx < lim;
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
#pragma unroll
      for (int db = 0; db < D / 32; ++db) {
        const char* vp = smem + voff[db] + 16 * sp * RB;
        const v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(vp));
        const v4i16 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(vp + 8 * RB));
        u32x4 a;
        a[0] = __builtin_bit_cast(u32x2, lo)[0];
        a[1] = __builtin_bit_cast(u32x2, lo)[1];
        a[2] = __builtin_bit_cast(u32x2, hi)[0];
        a[3] = __builtin_bit_cast(u32x2, hi)[1];
        o[db] = mma32<BF>(a, pf, o[db]);
      }
    }
  };

  // Main loop. koff / voff hold the offsets of the stage being computed and
  // flip to the other stage (XOR STAGE, a power of two) after every tile.
  int cur = 0;   // byte offset of the stage being computed
  for (int it = 0; it < n_tiles; ++it) {
    const int j0 = it * kBN;
    char* next = smem + (cur ^ STAGE);
    wait_all_and_barrier();   // tile it is in LDS; everyone is done with tile it-1
    if (it + 1 < n_tiles) {
      issue_tile(j0 + kBN, next);
      load_k_regs(j0 + kBN);
      if (it + 2 < n_tiles) pages_next = fetch_pages(j0 + 2 * kBN);
    }
    // tile class for this wave: 0 skip, 1 full, 2 partial
    int cls;
    if constexpr (MASK == kMaskTree) {
      cls = (j0 + kBN <= min(tree_start, kv_len)) ? 1 : 2;
    } else {
      cls = (j0 >= lim_hi) ? 0 : ((j0 + kBN <= lim_lo) ? 1 : 2);
    }
    cls = __builtin_amdgcn_readfirstlane(cls);
    if (wave_active && cls != 0) compute(j0, cls == 2);
    if (it + 1 < n_tiles) rope_store_k(j0 + kBN, next);
    cur ^= STAGE;
#pragma unroll
    for (int s = 0; s < D / 16; ++s) koff[s] ^= STAGE;
#pragma unroll
    for (int db = 0; db < D / 32; ++db) voff[db] ^= STAGE;
  }

  // ---- epilogue: out = O / l (dtype), lse = m + log2(l) ----
  const float l_tot = pair_sum(l_run);
  if (row_ok) {
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
    uint16_t* orow = static_cast<uint16_t*>(out_) + (static_cast<size_t>(q0 + t) * h_q_ + head) * D;
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
      lse_[static_cast<size_t>(q0 + t) * h_q_ + head] = l_tot > 0.f ? m_run + log2f(l_tot) : -INFINITY;
  }
}

#undef KSWZ
#undef VSWZ

template <bool BF, int D, int LAYOUT, int MASK>
void launch_r(const AttnParams& p, dim3 grid, hipStream_t stream) {
  if (p.rope_k)
    hipLaunchKernelGGL((attn_fwd_kernel<BF, D, LAYOUT, MASK, true>), grid, dim3(kThreads), 0, stream, p);
  else
    hipLaunchKernelGGL((attn_fwd_kernel<BF, D, LAYOUT, MASK, false>), grid, dim3(kThreads), 0, stream, p);
}

template <bool BF, int D>
hipError_t launch_d(const AttnParams& p, KvLayout layout, MaskKind mask, dim3 grid,
                    hipStream_t stream) {
  if (layout == kContiguous) {
    if (mask == kMaskTree) launch_r<BF, D, kContiguous, kMaskTree>(p, grid, stream);
    else launch_r<BF, D, kContiguous, kMaskCausal>(p, grid, stream);
  } else {
    if (mask == kMaskTree) launch_r<BF, D, kPaged, kMaskTree>(p, grid, stream);
    else launch_r<BF, D, kPaged, kMaskCausal>(p, grid, stream);
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
