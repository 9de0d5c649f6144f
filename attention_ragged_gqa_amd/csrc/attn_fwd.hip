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
//  * Work item = (sequence, KV head, tile of 32 NW packed query rows, NW = 4
//    or 8 waves per workgroup). Packed
//    row R of a sequence is token R / g, query head kvh*g + R % g (g = h_q/h_kv),
//    so one K/V tile feeds all g heads that share it. Items are enumerated
//    KV-head-major, then by sequence, with the heaviest tile of each
//    (sequence, KV head) first, and split into 8 contiguous chunks, one per
//    XCD (workgroups are handed to XCDs round-robin): the tiles that share
//    K/V run on one XCD's L2 and every XCD gets the same mix of sequences.
//  * A workgroup is NW waves of 64; each wave owns 32 packed rows and loads
//    64 / NW rows of every K/V tile (eight waves share a tile between twice
//    the rows, at one workgroup per CU; four run two per CU). Scores are
//    computed transposed, S^T = K Q^T, with v_mfma_f32_32x32x16_{bf16,f16}:
//    each lane then holds one query row and 16 keys per 32-key block, so row
//    max and row sum are in-lane plus one v_permlane32_swap, and the fp32
//    accumulators convert in place into the B operand of O^T += V^T P^T.
//  * Q stays in registers (RoPE applied on load from a cos/sin table in
//    LDS: one row per position value when the item's positions span at most
//    64 values, so tree nodes at equal depth share it, else one row per
//    token, shared by its g heads). Rows that see no key load no Q.
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
//  * Paged KV: each wave loads a 16-row block per tile, which with page size
//    16 is one page; sliding windows shift the tile grid so that this holds
//    past the sink. Other blocks (sink rows, ragged ends, bad pages) are
//    loaded row by row.
//  * Masks are classified per (wave, tile): skipped, full (no test) or
//    partial (per-element test); causal work stops at the last visible tile
//    (and, with left padding, starts at the first). Tree masks use a
//    per-stage LDS window of (enter, length) per key of the tile.
//  * The softmax runs in the log2 domain (v_exp_f32 is exp2): scores are
//    scaled by sm_scale*log2(e), lse = m + log2(l) as on the pages; the
//    running max only moves (and O is rescaled) when a tile raises it by
//    more than kRescaleSlack.

#include <atomic>
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
// The O rescale is skipped while a row's running maximum grows by at most
// this much (log2 units): probabilities then stay below 2^8, and the output
// is normalised by the sum of the same rounded P that fed the PV MFMAs.
constexpr float kRescaleSlack = 8.0f;

// First token of the work item starting at packed row row0.
__device__ __forceinline__ int t_first_of(int row0, int g) { return row0 / g; }

// NW waves per workgroup (4 or 8; two or one workgroups per CU): the work
// item is BM = 32 NW packed query rows, and each wave loads kBN / NW rows of
// every K/V tile, so eight waves issue half the K/V loads per query row.
template <int NW, bool BF, int D, int LAYOUT, int MASK, bool ROPE_K>
__global__ __launch_bounds__(64 * NW, 8 / NW) void attn_fwd_kernel(AttnParams p) {
  constexpr int NT = 64 * NW;                // threads
  constexpr int BM = 32 * NW;                // packed query rows per work item
  constexpr int RW = kBN / NW;               // rows of a K/V tile each wave loads
  constexpr int RB = D * 2;                  // bytes per head row
  constexpr int CH = D / 8;                  // 16-byte chunks per row
  constexpr int TILE = kBN * RB;             // bytes of one K or V tile
  constexpr int STAGE = 2 * TILE;            // K tile, then V tile
  constexpr int RPL = 1024 / RB;             // rows one wave-wide 16-byte load covers
  constexpr int LOADS = kBN / (NW * RPL);    // per wave and tile, for K and for V each
  // tree masks: an (enter, length) entry per key of a tile (win_entry),
  // one window per stage, filled alongside the K/V tile
  constexpr int WIN = kBN * 8;
  constexpr int TREE_OFF = kStages * STAGE;
  constexpr int SMEM = TREE_OFF + (MASK == kMaskTree ? kStages * WIN : 0);
  static_assert(LOADS >= 1 && NW * RPL * LOADS == kBN, "tile shape");
  static_assert(16 % RW == 0, "a wave's block of a tile lies within one page");
  static_assert((STAGE & (STAGE - 1)) == 0, "stage size is a power of two");
  // LDS chunk swizzles (see the header comment): K chunk c of row r sits at
  // c ^ KSWZ(r), V chunk c at c ^ VSWZ(r); RSH = log2(rows per 256 bytes).
  constexpr int RSH = (D == 64) ? 1 : 0;
#define KSWZ(r) ((((r) >> RSH)) & (CH - 1))
#define VSWZ(r) (4 * ((((r) >> RSH)) & (CH / 4 - 1)))

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

  // RoPE frequency of this thread (the table is written to LDS later); loaded
  // first so that no later wait includes it
  double ifreq = p.inv_freq[tid & 63];

  const int splits = max(p.num_splits, 1);
  int b = 0, kvh = 0, tile = 0, split_m = 0, q0_m = 0, qo_len_m = 0;
  if (!locate_item(q_indptr_, batch_, group_, h_kv_, splits, BM, b, kvh, tile, split_m, q0_m, qo_len_m))
    return;   // uniform over the workgroup
  b = __builtin_amdgcn_readfirstlane(b);
  kvh = __builtin_amdgcn_readfirstlane(kvh);
  tile = __builtin_amdgcn_readfirstlane(tile);
  const int split = __builtin_amdgcn_readfirstlane(split_m);
  pin(ifreq);   // arrived with the sequence table (no wait of its own later)

  const int g = group_;
  const int q0 = __builtin_amdgcn_readfirstlane(q0_m);
  const int qo_len = __builtin_amdgcn_readfirstlane(qo_len_m);
  const int row0 = tile * BM;

  // ---- KV chunk of this sequence ----
  // The per-sequence scalars come in one vector load (lane i fetches value i)
  // and are read back with v_readlane: one round trip instead of a chain.
  int kv_len_m = 0, kv_base_m = 0, page_base_m = 0, page_end_m = 0, sink_m = 0, win_off_m = 0;
  int li0 = 0, li1 = 0, li2 = 0, pi1 = 0, ti0 = 0, ti1 = 0, kp0 = 0, valid_m = 0;
  {
    const int32_t* src = q_indptr_ + b;   // any valid address for unused lanes
    if constexpr (LAYOUT == kContiguous) {
      if (lane == 0) src = kv_indptr_ + b;
      if (lane == 1) src = kv_indptr_ + b + 1;
    } else {
      if (lane == 0) src = page_indptr_ + b;
      if (lane == 1) src = page_indptr_ + b + 1;
      if (lane == 2) src = length_info_ + b;
      if (lane == 3 && sliding_) src = length_info_ + batch_ + b;
      if (lane == 4 && sliding_) src = length_info_ + 2 * batch_ + b;
      if (lane == 7 && ROPE_K) src = k_rope_pos_offset_ + b;
    }
    if constexpr (MASK == kMaskTree) {
      if (lane == 5) src = tree_indptr_ + b;
      if (lane == 6) src = tree_indptr_ + b + 1;
    }
    if constexpr (MASK == kMaskCausal) {
      if (p.pad_mode != 0) valid_m = p.valid_len[b];   // uniform
    }
    const int v = *src;
    if constexpr (LAYOUT == kContiguous) {
      kv_base_m = __builtin_amdgcn_readlane(v, 0);
      kv_len_m = __builtin_amdgcn_readlane(v, 1);
    } else {
      page_base_m = __builtin_amdgcn_readlane(v, 0);
      pi1 = __builtin_amdgcn_readlane(v, 1);
      li0 = __builtin_amdgcn_readlane(v, 2);
      li1 = __builtin_amdgcn_readlane(v, 3);
      li2 = __builtin_amdgcn_readlane(v, 4);
      kp0 = __builtin_amdgcn_readlane(v, 7);
    }
    if constexpr (MASK == kMaskTree) {
      ti0 = __builtin_amdgcn_readlane(v, 5);
      ti1 = __builtin_amdgcn_readlane(v, 6);
    }
  }
  if constexpr (LAYOUT == kContiguous) {
    kv_len_m -= kv_base_m;
  } else {
    page_end_m = min(pi1, nnz_pages_);
    const int np = pi1 - page_base_m;
    if (np > 0) {
      if (sliding_) {
        win_off_m = li1;
        sink_m = li2;
        kv_len_m = (np - 1) * 16 + li0 - win_off_m + sink_m;
      } else {
        kv_len_m = (np - 1) * 16 + li0;
      }
    }
  }
  const int kv_len = max(kv_len_m, 0);
  const int kv_base = kv_base_m, page_base = page_base_m, page_end = page_end_m;
  const int sink = sink_m, win_off = win_off_m;
  const int tree_base = ti0, tree_len = max(ti1 - ti0, 0);
  const int tree_start = kv_len - tree_len;
  const __amdgpu_buffer_rsrc_t pos_rsrc = make_rsrc(q_rope_position_, 4L * total_q_);
  const __amdgpu_buffer_rsrc_t tree_rsrc = make_rsrc(tree_order_, 8L * tree_size_);
  const int k_pos0 = kp0;   // paged: RoPE position of chunk key 0

  // ---- this lane's query row ----
  const int R = row0 + w * 32 + r32;
  const int t = R / g;
  const int head = kvh * g + (R - t * g);
  const bool row_ok = t < qo_len && q0 + t >= 0 && q0 + t < total_q_;
  const int t_lo = (row0 + w * 32) / g;
  const int t_hi = min((row0 + w * 32 + 31) / g, qo_len - 1);
  const bool wave_active = t_lo < qo_len;

  // Causal-or-none masks: row t sees keys [lo, lim) of the chunk (lo > 0
  // only with left padding). lim_lo / lim_hi (and lo_min / lo_max) bound
  // them over the wave's rows for the per-tile classification.
  const bool causal = (MASK == kMaskCausal) && causal_;
  const int pad_mode = MASK == kMaskCausal ? p.pad_mode : 0;
  int lim_m = causal ? min(kv_len, kv_len - qo_len + t + 1) : kv_len;
  int lo_m = 0;
  int kv_hi = kv_len;
  int kv_lo = 0;   // first key any row of the tile can see
  const int t_last = min((row0 + BM - 1) / g, qo_len - 1);
  if (causal) kv_hi = min(kv_len, kv_len - qo_len + t_last + 1);
  if (pad_mode == 1) {          // right padding: rows and keys below valid_len
    const int vl = min(max(valid_m, 0), kv_len);
    lim_m = (t < valid_m) ? min(lim_m, vl) : 0;
    kv_hi = (t_first_of(row0, g) < valid_m) ? min(kv_hi, vl) : 0;
  } else if (pad_mode == 2) {   // left padding, causal: valid suffixes
    const int vq = min(max(valid_m, 0), qo_len), vk = min(max(valid_m, 0), kv_len);
    lo_m = kv_len - vk;
    if (t < qo_len - vq) lim_m = 0;
    kv_lo = kv_len - vk;
    if (t_last < qo_len - vq) kv_hi = 0;   // the whole tile is padding
  }
  const int lim = lim_m, lo = lo_m;
  int lim_lo = causal ? min(kv_len, kv_len - qo_len + t_lo + 1) : kv_len;
  int lim_hi = causal ? min(kv_len, kv_len - qo_len + t_hi + 1) : kv_len;
  int lo_min = 0, lo_max = 0;
  if (pad_mode != 0) {
    // per-wave bounds by reduction over the wave's valid rows (uniform)
    const bool in_seq = t < qo_len;
    int hmin = in_seq ? lim : INT_MAX, hmax = in_seq ? lim : INT_MIN;
    int lmin = in_seq ? lo : INT_MAX, lmax = in_seq ? lo : INT_MIN;
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) {
      hmin = min(hmin, __shfl_xor(hmin, m, 64));
      hmax = max(hmax, __shfl_xor(hmax, m, 64));
      lmin = min(lmin, __shfl_xor(lmin, m, 64));
      lmax = max(lmax, __shfl_xor(lmax, m, 64));
    }
    lim_lo = __builtin_amdgcn_readfirstlane(hmin);
    lim_hi = __builtin_amdgcn_readfirstlane(hmax);
    lo_min = __builtin_amdgcn_readfirstlane(lmin);
    lo_max = __builtin_amdgcn_readfirstlane(lmax);
  }
  // Paged sliding window: keys past the sink sit at storage offset j + delta.
  // The tile grid is shifted back by kshift = delta mod 16 keys, so that every
  // 16-row block past the sink is exactly one page (the keys j < 0 this adds
  // to the first tile are masked).
  const int delta = (LAYOUT == kPaged && sliding_) ? win_off - sink : 0;
  const int kshift = delta & 15;
  // KV tiles the item needs: [kv_lo, kv_hi) on that grid
  const int tile0 = (kv_lo + kshift) / kBN;
  const int n_tiles_all = kv_hi > kv_lo ? (kv_hi + kshift + kBN - 1) / kBN - tile0 : 0;
  // split-KV: this item's contiguous range of those tiles
  const int tile_lo = (splits > 1) ? split * n_tiles_all / splits : 0;
  const int tile_hi = (splits > 1) ? (split + 1) * n_tiles_all / splits : n_tiles_all;
  const int n_tiles = tile_hi - tile_lo;   // tiles this workgroup processes
  const int jbase = (tile0 + tile_lo) * kBN - kshift;   // first key of the range

  // enter index of this row's tree node (selected after the prologue)
  const int c_node = t + tree_len - qo_len;
  int enter_raw = 0;
  if constexpr (MASK == kMaskTree) enter_raw = load_i32x2(tree_rsrc, tree_base + c_node).x;

  // ---- K/V tile loads: wave w fills tile rows [RW w, RW w + RW); lane covers
  // rows RW w + RPL*i + lane/CH (i < LOADS) at physical chunk lane % CH ----
  const int pc = lane % CH;
  const int lrow = lane / CH;
  auto tile_row = [&](int i) __attribute__((always_inline)) { return RW * w + RPL * i + lrow; };
  // Page of the wave's RW-row block [B, B + RW) of a tile, B = j0 + RW w.
  // Past the sink such a block lies within one page (storage offsets from
  // B + delta; j0 + delta is a multiple of 16 on the shifted grid and RW
  // divides 16). The page number is
  // loaded a tile ahead and only read (v_readfirstlane) when the block is
  // issued; out-of-range indices read 0 and are rejected there.
  const __amdgpu_buffer_rsrc_t page_rsrc = make_rsrc(page_values_, 4L * nnz_pages_);
  auto fetch_page = [&](int j0) __attribute__((always_inline)) -> int {
    if constexpr (LAYOUT == kPaged) return load_i32(page_rsrc, page_base + ((j0 + RW * w + delta) >> 4));
    else return 0;
  };
  int page_next = 0;   // page of this wave's block of the next tile to issue
  const size_t kv_stride = static_cast<size_t>(h_kv_) * RB;           // contiguous: per token
  const uint32_t page_stride = static_cast<uint32_t>(2 * h_kv_ * 16 * RB);   // paged: per page
  const char* kv_head_k;
  const char* kv_head_v;
  if constexpr (LAYOUT == kContiguous) {
    kv_head_k = reinterpret_cast<const char*>(k_) + (static_cast<size_t>(kv_base) * h_kv_ + kvh) * RB;
    kv_head_v = reinterpret_cast<const char*>(v_) + (static_cast<size_t>(kv_base) * h_kv_ + kvh) * RB;
  } else {
    kv_head_k = reinterpret_cast<const char*>(pages_) + static_cast<size_t>(kvh) * 16 * RB;
    kv_head_v = kv_head_k + static_cast<size_t>(h_kv_) * 16 * RB;
  }
  const size_t v_minus_k = static_cast<size_t>(kv_head_v - kv_head_k);
  // Blocks that take the whole-block path: B in [fast_lo, fast_hi - RW] and,
  // when paged, a page number below num_pages. Everything else (sink rows,
  // keys j < 0, the chunk's ragged end, rows of pages outside the sequence's
  // range or past the cache) goes row by row.
  int fast_lo = 0, fast_hi;
  if constexpr (LAYOUT == kContiguous) {
    fast_hi = min(kv_len, total_kv_ - kv_base);
  } else {
    if (sliding_) fast_lo = max(sink, 0);
    fast_hi = min(kv_len, (page_end - page_base) * 16 - delta);
  }
  auto block_fast = [&](int B, int pg) __attribute__((always_inline)) -> bool {
    const bool rows = B >= fast_lo && B + RW <= fast_hi;
    if constexpr (LAYOUT == kPaged) return rows && static_cast<unsigned>(pg) < static_cast<unsigned>(num_pages_);
    else return rows;
  };
  auto block_base = [&](int B, int pg) __attribute__((always_inline)) -> const char* {
    if constexpr (LAYOUT == kContiguous) return kv_head_k + static_cast<size_t>(B) * kv_stride;
    else
      return kv_head_k + static_cast<size_t>(static_cast<uint32_t>(pg)) * page_stride + ((B + delta) & 15) * RB;
  };
  // Per-row K source of chunk position kidx (V: + v_minus_k), or null for a
  // row outside the chunk or with an invalid page. page: the page number
  // loaded for the row (row_page_index below).
  auto row_page_index = [&](int kidx) __attribute__((always_inline)) -> int {
    const int off = (sliding_ && kidx < sink) ? kidx : kidx + delta;
    return page_base + (off >> 4);
  };
  auto row_src = [&](int kidx, int page) __attribute__((always_inline)) -> const char* {
    if (kidx < 0 || kidx >= kv_len) return nullptr;
    if constexpr (LAYOUT == kContiguous) {
      const int r = kv_base + kidx;
      if (r < 0 || r >= total_kv_) return nullptr;
      return kv_head_k + static_cast<size_t>(kidx) * kv_stride;
    } else {
      const int off = (sliding_ && kidx < sink) ? kidx : kidx + delta;
      const int idx = page_base + (off >> 4);
      if (off < 0 || idx >= page_end || static_cast<unsigned>(page) >= static_cast<unsigned>(num_pages_))
        return nullptr;
      return kv_head_k + static_cast<size_t>(static_cast<uint32_t>(page)) * page_stride + (off & 15) * RB;
    }
  };

  // Tile-invariant part of each lane's source address: row RPL*i + lrow of
  // the wave's 16-row block (one token apart when contiguous, one page slot
  // apart when paged) and the lane's swizzled chunk. Per tile only the
  // wave-uniform base (SGPRs) changes.
  const uint32_t mem_rs = LAYOUT == kContiguous ? static_cast<uint32_t>(kv_stride) : RB;
  auto lane_off = [&](int i, bool v) __attribute__((always_inline)) -> uint32_t {
    const int r = tile_row(i);
    return static_cast<uint32_t>(RPL * i + lrow) * mem_rs + 16 * (pc ^ (v ? VSWZ(r) : KSWZ(r)));
  };
  auto zero_row = [&](char* dst) __attribute__((always_inline)) {
    *reinterpret_cast<u32x4*>(dst + 16 * lane) = u32x4{0, 0, 0, 0};
  };
  // Row pages of the slow path: all loads first, then one wait, here. (A
  // load left pending past the slow path would make the tile loop wait for
  // it, and with it for the next tile's loads, before every tile.)
  auto row_pages = [&](int j0, int (&pg)[LOADS]) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < LOADS; ++i)
      pg[i] = LAYOUT == kPaged ? load_i32(page_rsrc, row_page_index(j0 + tile_row(i))) : 0;
#pragma unroll
    for (int i = 0; i < LOADS; ++i) pin(pg[i]);
  };

  auto issue_tile = [&](int j0, char* stage) __attribute__((always_inline)) {
    const int B = j0 + RW * w;
    const int pg = __builtin_amdgcn_readfirstlane(page_next);
    if (block_fast(B, pg)) {
      const char* base = block_base(B, pg);
#pragma unroll
      for (int i = 0; i < LOADS; ++i) {
        char* dst_k = stage + (RW * w + RPL * i) * RB;          // wave-uniform
        if constexpr (!ROPE_K) dma16s(base, lane_off(i, false), dst_k);
        dma16s(base + v_minus_k, lane_off(i, true), dst_k + TILE);
      }
    } else {
      int rp[LOADS];
      row_pages(j0, rp);
#pragma unroll
      for (int i = 0; i < LOADS; ++i) {
        const int r = tile_row(i);
        char* dst_k = stage + (RW * w + RPL * i) * RB;
        const char* src = row_src(j0 + r, rp[i]);
        if (src) {
          if constexpr (!ROPE_K) dma16(src + 16 * (pc ^ KSWZ(r)), dst_k);
          dma16(src + v_minus_k + 16 * (pc ^ VSWZ(r)), dst_k + TILE);
        } else {
          // rows outside the chunk: zeros, so masked products stay finite
          if constexpr (!ROPE_K) zero_row(dst_k);
          zero_row(dst_k + TILE);
        }
      }
    }
  };

  // In-kernel K RoPE: K goes through registers (same lanes and rows as the
  // direct loads); the partner chunk (dims +- D/2) is in lane ^ (CH/2).
  u32x4 kreg[ROPE_K ? LOADS : 1];
  int kpos[ROPE_K ? LOADS : 1];   // RoPE positions of those rows
  // positions first: the angles need only them and are computed while the
  // K rows are still in flight
  auto load_k_pos = [&](int j0) __attribute__((always_inline)) {
    if constexpr (ROPE_K) {
#pragma unroll
      for (int i = 0; i < LOADS; ++i) {
        if constexpr (LAYOUT == kContiguous)
          kpos[i] = load_i32(pos_rsrc, kv_base + j0 + tile_row(i));   // K shares the query positions
        else
          kpos[i] = k_pos0 + j0 + tile_row(i);
      }
    }
  };
  auto load_k_regs = [&](int j0) __attribute__((always_inline)) {
    if constexpr (ROPE_K) {
      const int B = j0 + RW * w;
      const int pg = __builtin_amdgcn_readfirstlane(page_next);
      if (block_fast(B, pg)) {
        const char* base = block_base(B, pg);
#pragma unroll
        for (int i = 0; i < LOADS; ++i) kreg[i] = *reinterpret_cast<const u32x4*>(base + lane_off(i, false));
      } else {
        int rp[LOADS];
        row_pages(j0, rp);
#pragma unroll
        for (int i = 0; i < LOADS; ++i) {
          const int r = tile_row(i);
          const char* src = row_src(j0 + r, rp[i]);
          kreg[i] = src ? *reinterpret_cast<const u32x4*>(src + 16 * (pc ^ KSWZ(r))) : u32x4{0, 0, 0, 0};
        }
      }
    }
  };
  // The partner lanes (chunks c and c ^ CH/2 of one row) need the same 8
  // frequencies: each evaluates 4 of them and they swap the results, or,
  // with from_tab, both read them from the (cos, sin) table in the other
  // stage (built in the prologue): row r for tile row r, or with by_pos the
  // row of the key's position, kpos - pos_base.
  auto rope_store_k = [&](int j0, char* stage, bool from_tab, bool by_pos, int pos_base)
                          __attribute__((always_inline)) {
    if constexpr (ROPE_K) {
#pragma unroll
      for (int i = 0; i < LOADS; ++i) {
        const int r = tile_row(i);
        const int kidx = j0 + r;
        const int lc = pc ^ KSWZ(r);               // logical chunk held
        const bool first = lc < CH / 2;
        float cs[8], sn[8];
        if (from_tab) {
          // frequencies 8*(lc mod CH/2) + [0, 8): one 8-entry chunk of table
          // row tr (keys outside the chunk, which are zero or left as they
          // are, read a clamped row)
          int tr = r;
          if (by_pos) {
            int kp = kpos[i];
            pin(kp);
            tr = min(max(kp - pos_base, 0), kBN - 1);
          }
          const float4* tc = reinterpret_cast<const float4*>(smem + STAGE) + tr * (D / 4) +
                             4 * (((lc & (CH / 2 - 1)) + tr) & (D / 16 - 1));
#pragma unroll
          for (int v = 0; v < 4; ++v) {
            const float4 x = tc[v];
            cs[2 * v] = x.x;
            sn[2 * v] = x.y;
            cs[2 * v + 1] = x.z;
            sn[2 * v + 1] = x.w;
          }
        } else {
          int kp = kpos[i];
          pin(kp);
          const int pos = kidx < kv_len ? kp : 0;
          // frequencies 8*(lc mod CH/2) + e; this lane evaluates e in [emine, emine + 4)
          const int kbase = 8 * (lc & (CH / 2 - 1));
          const int emine = first ? 0 : 4;
          float cmine[4], smine[4];
#pragma unroll
          for (int u = 0; u < 4; ++u)
            rope_cos_sin(pos, rope_scale_, inv_freq_s[kbase + emine + u], cmine[u], smine[u]);
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            const float co = __shfl_xor(cmine[u], CH / 2, 64);
            const float so = __shfl_xor(smine[u], CH / 2, 64);
            cs[u] = first ? cmine[u] : co;
            sn[u] = first ? smine[u] : so;
            cs[u + 4] = first ? co : cmine[u];
            sn[u + 4] = first ? so : smine[u];
          }
        }
        u32x4 other;
#pragma unroll
        for (int u = 0; u < 4; ++u) other[u] = __shfl_xor(kreg[i][u], CH / 2, 64);
        u32x4 res = kreg[i];
        if (kidx < kv_len) {
#pragma unroll
          for (int e = 0; e < 8; e += 2) {
            float y[2];
#pragma unroll
            for (int u = 0; u < 2; ++u) {
              float y1, y2;
              const float x = to_f32<BF>(half_of(kreg[i], e + u));
              const float xp = to_f32<BF>(half_of(other, e + u));
              if (first) { rope_pair(cs[e + u], sn[e + u], x, xp, y1, y2); y[u] = y1; }
              else { rope_pair(cs[e + u], sn[e + u], xp, x, y1, y2); y[u] = y2; }
            }
            res[e >> 1] = pack2<BF>(y[0], y[1]);
          }
        }
        *reinterpret_cast<u32x4*>(stage + r * RB + 16 * pc) = res;
      }
    }
  };

  // ---- prologue: every load that depends only on the sequence goes out
  // together; tile 0 is in flight while RoPE tables are computed ----
  const int t_first = row0 / g;
  const int t_end = min((row0 + BM - 1) / g + 1, qo_len);
  const int n_tok = max(t_end - t_first, 0);
  // RoPE table (cos, sin) per (row, frequency) in stage 1. Q table: one row
  // per token of this tile, shared by the g heads of a token (with g = 1
  // each lane computes its own). With in-kernel K RoPE on contiguous KV, K
  // row j of the chunk rotates at position entry kv_base + j; when the
  // tile's query tokens index entries of the first K tile's range, one
  // table over that tile's 64 rows serves K and Q alike (KQ table): query
  // token t reads row kq0 + t - t_first.
  const int kq0 = q0 + t_first - (kv_base + jbase);
  const bool kq_table = ROPE_K && LAYOUT == kContiguous && rope_q_ && n_tiles > 0 && kq0 >= 0 &&
                        kq0 + n_tok <= kBN;
  const bool q_table = rope_q_ && !kq_table && n_tok * (D / 2) * 8 <= STAGE;
  const int tab_pos0 = kq_table ? kv_base + jbase : q0 + t_first;   // position entry of table row 0
  // Order of the prologue loads. Positions first (the RoPE tables need only
  // them). Paged: the tile-0 addresses need the page numbers, so the pages
  // go next and tile 0 is issued when they arrive, then Q. Contiguous: with
  // in-kernel K RoPE the K rows (rotated, then stored, before the first
  // tile), then Q, then V; otherwise Q, then tile 0. (Loads complete in
  // issue order, so whatever a wait needs should have gone out early.)
  constexpr int TPOS = STAGE / 8 / NT;         // table entries per thread at most
  static_assert(TPOS * NT * 8 == STAGE, "table entries per thread");
  static_assert(kBN * (D / 2) == TPOS * NT, "KQ table rows");
  int tpos[TPOS];                                // token positions of those entries
  if (q_table || kq_table) {
#pragma unroll
    for (int u = 0; u < TPOS; ++u) tpos[u] = load_i32(pos_rsrc, tab_pos0 + (tid + u * NT) / (D / 2));
  }
  int my_pos = 0;
  if (rope_q_) my_pos = load_i32(pos_rsrc, q0 + t);
  if (n_tiles > 0) load_k_pos(jbase);
  // tree intervals of tile 0 (raw; turned into window entries when stored)
  int2 win_iv = make_int2(0, 0);
  // Window entry of chunk key kidx from its raw (enter, exit) interval:
  // (enter, exit - enter) for tree keys, (INT_MIN, 2^32 - 1) for prefix keys
  // (every row passes the compare), length 0 past the chunk (none does).
  auto win_entry = [&](int kidx, int2 iv) __attribute__((always_inline)) -> int2 {
    if (kidx >= kv_len) return make_int2(INT_MAX, 0);
    if (kidx < tree_start) return make_int2(INT_MIN, -1);
    const unsigned len = iv.y > iv.x ? static_cast<unsigned>(iv.y) - static_cast<unsigned>(iv.x) : 0u;
    return make_int2(iv.x, static_cast<int>(len));
  };
  if constexpr (MASK == kMaskTree)
    win_iv = load_i32x2(tree_rsrc, tree_base + jbase + (tid & (kBN - 1)) - tree_start);

  auto issue_first_tile = [&]() __attribute__((always_inline)) {
    if (n_tiles > 0) {
      issue_tile(jbase, smem);                             // V (and K) straight into stage 0
      if (LAYOUT == kPaged || !ROPE_K) load_k_regs(jbase);
      if (n_tiles > 1) page_next = fetch_page(jbase + kBN);   // page of the second tile
    }
  };
  if constexpr (LAYOUT == kPaged) {
    if (n_tiles > 0) page_next = fetch_page(jbase);
    // one wait for the page number here, before the tile-0 loads go out
    pin(page_next);
    issue_first_tile();
  } else if constexpr (ROPE_K) {
    if (n_tiles > 0) load_k_regs(jbase);
  }

  // ---- Q fragments: lane holds row R, dims 16*s + 8*hh + [0, 8) ----
  u32x4 qf[D / 16];
#pragma unroll
  for (int s = 0; s < D / 16; ++s) qf[s] = u32x4{0, 0, 0, 0};
  // Rows that see no key (padding, or more queries than keys under the
  // causal mask) are masked everywhere: their Q is never read.
  if (row_ok && lim > lo) {
    // (token, head) row index fits in 32 bits; only the byte offset needs 64
    const unsigned qr = static_cast<unsigned>((q0 + t) * h_q_ + head);
    const uint16_t* qrow = q_ + static_cast<size_t>(qr) * D + 8 * hh;
#pragma unroll
    for (int s = 0; s < D / 16; ++s) qf[s] = *reinterpret_cast<const u32x4*>(qrow + 16 * s);
  }
  if constexpr (LAYOUT == kContiguous) issue_first_tile();
  if (rope_q_ | rope_k_) {
    if (tid < D / 2) inv_freq_s[tid] = ifreq;
  }
  // Position table: when every position the prologue rotates (this item's
  // query rows and, with in-kernel K RoPE, the keys of the first tile) lies
  // in kBN consecutive values, the table holds one row per position value
  // from the smallest on, and rows at the same position (tree nodes at equal
  // depth) share it. Each wave's smallest and largest position go through
  // LDS across the barrier below.
  __shared__ int pos_mm[2 * NW];
  if (rope_q_) {
    int pmin = INT_MAX, pmax = INT_MIN;
    if (row_ok) {
      pin(my_pos);
      pmin = my_pos;
      pmax = my_pos;
    }
    if constexpr (ROPE_K) {
      if (n_tiles > 0) {
#pragma unroll
        for (int i = 0; i < LOADS; ++i) {
          const int kidx = jbase + tile_row(i);
          int kp = kpos[i];
          pin(kp);
          if (kidx >= 0 && kidx < kv_len) {
            pmin = min(pmin, kp);
            pmax = max(pmax, kp);
          }
        }
      }
    }
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) {
      pmin = min(pmin, __shfl_xor(pmin, m, 64));
      pmax = max(pmax, __shfl_xor(pmax, m, 64));
    }
    if (lane == 0) {
      pos_mm[2 * w] = pmin;
      pos_mm[2 * w + 1] = pmax;
    }
  }
  __syncthreads();   // inv_freq and pos_mm are visible (the loads above are still in flight)
  int pos_base = 0, pos_rows = 0;
  bool pos_table = false;
  if (rope_q_) {
    int pmin = INT_MAX, pmax = INT_MIN;
#pragma unroll
    for (int v = 0; v < NW; ++v) {
      pmin = min(pmin, pos_mm[2 * v]);
      pmax = max(pmax, pos_mm[2 * v + 1]);
    }
    pos_base = __builtin_amdgcn_readfirstlane(pmin);
    // span - 1 as an unsigned difference (no overflow for any int32 pair)
    const unsigned span1 = static_cast<unsigned>(pmax) - static_cast<unsigned>(pmin);
    pos_table = __builtin_amdgcn_readfirstlane((pmax >= pmin && span1 < static_cast<unsigned>(kBN)) ? 1 : 0) != 0;
    if (pos_table) pos_rows = static_cast<int>(span1) + 1;
  }
  const bool row_table = !pos_table && (q_table || kq_table);   // one row per token or key
  const bool any_table = pos_table || row_table;

  if (any_table) {
    float2* tab = reinterpret_cast<float2*>(smem + STAGE);
    const int n_ent = (pos_table ? pos_rows : (kq_table ? kBN : n_tok)) * (D / 2);
    if (row_table) {
#pragma unroll
      for (int u = 0; u < TPOS; ++u) pin(tpos[u]);
    }
#pragma unroll
    for (int u = 0; u < TPOS; ++u) {
      const int e = tid + u * NT;
      if (e < n_ent) {
        float cs, sn;
        const int pos = pos_table ? pos_base + e / (D / 2) : tpos[u];
        rope_cos_sin(pos, rope_scale_, inv_freq_s[e % (D / 2)], cs, sn);
        // 8-entry chunks of a token's row rotated by the token index, so
        // that lanes reading different tokens' chunks hit different banks
        const int te = e / (D / 2), kk = e % (D / 2);
        tab[te * (D / 2) + 8 * (((kk >> 3) + te) & (D / 16 - 1)) + (kk & 7)] = make_float2(cs, sn);
      }
    }
  }
  if constexpr (MASK == kMaskTree) {
    pin(win_iv.x);
    pin(win_iv.y);
    if (tid < kBN) reinterpret_cast<int2*>(smem + TREE_OFF)[tid] = win_entry(jbase + tid, win_iv);
  }
  int enter_c = INT_MIN;   // sentinel: sees the prefix only
  if constexpr (MASK == kMaskTree) {
    pin(enter_raw);
    if (row_ok && c_node >= 0 && c_node < tree_len) enter_c = enter_raw;
  }
  if (any_table) __syncthreads();   // the table is visible to every wave
  if (n_tiles > 0) rope_store_k(jbase, smem, pos_table || kq_table, pos_table, pos_base);
  if (rope_q_) {
    pin(my_pos);
    if (row_ok) {
      const int tr = pos_table ? my_pos - pos_base : t - t_first + (kq_table ? kq0 : 0);
      const float4* trow = reinterpret_cast<const float4*>(smem + STAGE) + tr * (D / 4);
#pragma unroll
      for (int s = 0; s < D / 32; ++s) {
        const u32x4 a = qf[s], c2 = qf[s + D / 32];
        // frequencies 16s + 8hh + [0, 8): one 8-entry chunk of the table row
        float cs[8], sn[8];
        if (any_table) {
          const float4* tc = trow + 4 * (((2 * s + hh) + tr) & (D / 16 - 1));
#pragma unroll
          for (int v = 0; v < 4; ++v) {
            const float4 x = tc[v];
            cs[2 * v] = x.x;
            sn[2 * v] = x.y;
            cs[2 * v + 1] = x.z;
            sn[2 * v + 1] = x.w;
          }
        } else {
#pragma unroll
          for (int e = 0; e < 8; ++e)
            rope_cos_sin(my_pos, rope_scale_, inv_freq_s[16 * s + 8 * hh + e], cs[e], sn[e]);
        }
#pragma unroll
        for (int e = 0; e < 8; e += 2) {
          float y1[2], y2[2];
#pragma unroll
          for (int u = 0; u < 2; ++u)
            rope_pair(cs[e + u], sn[e + u], to_f32<BF>(half_of(a, e + u)), to_f32<BF>(half_of(c2, e + u)),
                      y1[u], y2[u]);
          qf[s][e >> 1] = pack2<BF>(y1[0], y1[1]);
          qf[s + D / 32][e >> 1] = pack2<BF>(y2[0], y2[1]);
        }
      }
    }
  }
  // (the loop's first barrier publishes the K rows, tree intervals and tile 0)

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
  float l_run = 0.f;    // sum of p (float32): the log-sum-exp
  float l_mma = 0.f;    // sum of p as rounded for the PV MFMA: the normaliser of O
  f32x16 o[D / 32];
#pragma unroll
  for (int i = 0; i < D / 32; ++i) o[i] = f32x16{};
  const float sc = sm_scale_log2_;

  // One KV tile: S^T = K Q^T, mask, online softmax, O^T += V^T P^T.
  // SO: byte offset of the stage holding the tile (a compile-time constant,
  // so that it lands in the offset field of the LDS reads)
  auto compute = [&](int j0, bool masked, auto so_c) __attribute__((always_inline)) {
    constexpr int SO = decltype(so_c)::value;
    char* const sm = smem + SO;
    constexpr int twin = TREE_OFF + (SO ? WIN : 0);   // the tile's tree window
    // The two 32-key blocks alternate, so consecutive MFMAs are independent,
    // and every K fragment is read kAhead MFMAs before its use: the LDS
    // latency hides behind the MFMAs instead of stalling each one.
    constexpr int NF = 2 * (D / 16);
    constexpr int kAhead = 4;
    f32x16 sacc[2] = {f32x16{}, f32x16{}};
    u32x4 kf[NF];
#pragma unroll
    for (int t = 0; t < NF; ++t)
      kf[t] = *reinterpret_cast<const u32x4*>(sm + (t & 1) * 32 * RB + koff[t >> 1]);
#pragma unroll
    for (int t = 0; t < NF; ++t) sacc[t & 1] = mma32<BF>(kf[t], qf[t >> 1], sacc[t & 1]);
    // V pieces of the first 16 keys, read behind the last MFMAs so that they
    // have arrived when the softmax of this tile reaches its first PV MFMA
    // (not with in-kernel K RoPE, whose registers are needed elsewhere)
    constexpr bool kVEarly = !ROPE_K;
    v4i16 v0[D / 32][2];
    if constexpr (kVEarly) {
#pragma unroll
      for (int db = 0; db < D / 32; ++db) {
        v0[db][0] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(sm + voff[db]));
        v0[db][1] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(sm + voff[db] + 8 * RB));
      }
    }
    __builtin_amdgcn_sched_group_barrier(0x100, kAhead, 0);   // DS reads
#pragma unroll
    for (int t = 0; t < NF - kAhead; ++t) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);      // MFMA
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);      // DS read
    }
    __builtin_amdgcn_sched_group_barrier(0x008, kAhead, 0);
    if constexpr (kVEarly) __builtin_amdgcn_sched_group_barrier(0x100, D / 16, 0);   // the V reads
    if (masked) {
      if constexpr (MASK == kMaskTree) {
        // element r of block kb is key j0 + 32kb + 8(r/4) + 4hh + r%4; its
        // window entry (enter, length) makes the ancestor test one unsigned
        // compare: visible iff enter_c - enter < length
        const unsigned ec = static_cast<unsigned>(enter_c);
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
          for (int q4 = 0; q4 < 4; ++q4) {
            const u32x4* wp = reinterpret_cast<const u32x4*>(smem + twin + 8 * (32 * kb + 8 * q4 + 4 * hh));
            const u32x4 a = wp[0], c = wp[1];
            const unsigned ex[4] = {a[0], a[2], c[0], c[2]};
            const unsigned ln[4] = {a[1], a[3], c[1], c[3]};
#pragma unroll
            for (int u = 0; u < 4; ++u)
              if (!(ec - ex[u] < ln[u])) sacc[kb][4 * q4 + u] = -INFINITY;
          }
        }
      } else {
        // key j0 + 4hh + c(kb, r) is visible iff lo - j0 - 4hh <= c < lim - j0 - 4hh
        const int rel = lim - j0 - 4 * hh;
        if (lo_max == 0 && j0 >= 0) {   // uniform: no lower bound (no left padding, no keys j < 0)
#pragma unroll
          for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int r = 0; r < 16; ++r)
              if (32 * kb + 8 * (r >> 2) + (r & 3) >= rel) sacc[kb][r] = -INFINITY;
        } else {
          const int rel_lo = lo - j0 - 4 * hh;
#pragma unroll
          for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              const int c = 32 * kb + 8 * (r >> 2) + (r & 3);
              if ((c >= rel) | (c < rel_lo)) sacc[kb][r] = -INFINITY;
            }
        }
      }
    }
    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sacc[kb][r]);
    mx = pair_max(mx) * sc;
    const bool grow = mx > m_run + kRescaleSlack;   // always true while m_run = -inf
    if (__any(grow)) {
      // O is exactly zero while no row of the wave has seen a visible key
      // (every P so far was 2^-inf): then it needs no rescale
      const bool o_zero = !__any(m_run != -INFINITY);
      const float m_new = grow ? mx : m_run;
      // rows still without a visible key keep O = l = 0 (alpha 0, never NaN)
      const float alpha = __builtin_amdgcn_exp2f(m_run - (m_new == -INFINITY ? 0.f : m_new));
      m_run = m_new;
      l_run *= alpha;
      l_mma *= alpha;
      if (!o_zero) {
#pragma unroll
        for (int i = 0; i < D / 32; ++i) o[i] *= alpha;
      }
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
      for (int u = 0; u < 4; ++u) {
        pf[u] = pack2<BF>(sa[e0 + 2 * u], sa[e0 + 2 * u + 1]);
        l_mma = add_pair<BF>(pf[u], l_mma);
      }
#pragma unroll
      for (int db = 0; db < D / 32; ++db) {
        const char* vp = sm + voff[db] + 16 * sp * RB;
        const bool early = kVEarly && sp == 0;
        const v4i16 lo = early ? v0[db][0] : __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(vp));
        const v4i16 hi = early ? v0[db][1] : __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(vp + 8 * RB));
        u32x4 a;
        a[0] = __builtin_bit_cast(u32x2, lo)[0];
        a[1] = __builtin_bit_cast(u32x2, lo)[1];
        a[2] = __builtin_bit_cast(u32x2, hi)[0];
        a[3] = __builtin_bit_cast(u32x2, hi)[1];
        o[db] = mma32<BF>(a, pf, o[db]);
      }
    }
  };

  // Main loop, two tiles per trip: the stage of tile it is it % 2 (a
  // compile-time offset), the loads for tile it + 1 go to the other one.
  auto tile_step = [&](int it, auto so_c) __attribute__((always_inline)) {
    constexpr int SO = decltype(so_c)::value;
    constexpr int NSO = SO ^ STAGE;
    const int j0 = jbase + it * kBN;
    char* next = smem + NSO;
    wait_all_and_barrier();   // tile it is in LDS; everyone is done with tile it-1
    if (it + 1 < n_tiles) {
      issue_tile(j0 + kBN, next);
      load_k_pos(j0 + kBN);
      load_k_regs(j0 + kBN);
      if constexpr (MASK == kMaskTree)
        win_iv = load_i32x2(tree_rsrc, tree_base + j0 + kBN + (tid & (kBN - 1)) - tree_start);
      if (it + 2 < n_tiles) page_next = fetch_page(j0 + 2 * kBN);
    }
    // tile class for this wave: 0 skip, 1 full, 2 partial
    int cls;
    if constexpr (MASK == kMaskTree) {
      cls = (j0 + kBN <= min(tree_start, kv_len)) ? 1 : 2;
    } else {
      cls = (j0 >= lim_hi || j0 + kBN <= lo_min) ? 0
                                                : ((j0 + kBN <= lim_lo && j0 >= lo_max) ? 1 : 2);
    }
    cls = __builtin_amdgcn_readfirstlane(cls);
    if (wave_active && cls != 0) compute(j0, cls == 2, so_c);
    if (it + 1 < n_tiles) {
      rope_store_k(j0 + kBN, next, false, false, 0);
      if constexpr (MASK == kMaskTree)
        if (tid < kBN)
          reinterpret_cast<int2*>(smem + TREE_OFF + (NSO ? WIN : 0))[tid] = win_entry(j0 + kBN + tid, win_iv);
    }
  };
  for (int it = 0; it < n_tiles; it += 2) {
    tile_step(it, std::integral_constant<int, 0>{});
    if (it + 1 < n_tiles) tile_step(it + 1, std::integral_constant<int, STAGE>{});
  }
  const int cur = (n_tiles & 1) ? STAGE : 0;   // stage after the last tile

  // ---- epilogue: out = O / l (dtype), lse = m + log2(l) ----
  // O^T fragments go through LDS so that each row is stored as whole 16-byte
  // chunks by consecutive lanes. The stage at `cur` is free: its last reads
  // finished before the previous barrier and no load targets it.
  const float l_tot = pair_sum(l_run);
  const float l_o = pair_sum(l_mma);
  const float inv = l_o > 0.f ? 1.f / l_o : 0.f;
  if (splits > 1) {
    // split-KV partial state: O / l in fp32 and the range's lse, row-major at
    // [split][row]; the merge kernel combines the ranges
    if (row_ok) {
      int re = row0 + 32 * w + r32;
      pin(re);
      const int te = re / g;
      const size_t li = static_cast<size_t>(split) * total_q_ * h_q_ +
                        static_cast<unsigned>((q0 + te) * h_q_ + kvh * g + (re - te * g));
      float* prow = p.part_out + li * D;
#pragma unroll
      for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int jb = 0; jb < 4; ++jb) {
          const float4 v = make_float4(o[db][4 * jb + 0] * inv, o[db][4 * jb + 1] * inv,
                                       o[db][4 * jb + 2] * inv, o[db][4 * jb + 3] * inv);
          *reinterpret_cast<float4*>(prow + 32 * db + 8 * jb + 4 * hh) = v;
        }
      if (hh == 0) p.part_lse[li] = l_tot > 0.f ? m_run + log2f(l_tot) : -INFINITY;
    }
    return;
  }
  // This wave's 32 rows, same swizzle as K. Four waves fit in the stage at
  // `cur`; eight need both stages, once every wave is done with the last tile.
  char* obuf = smem + cur + (32 * w) * RB;
  if constexpr (NW == 8) {
    static_assert(NW * 32 * RB == kStages * STAGE, "eight waves' rows fill both stages");
    __syncthreads();
    obuf = smem + (32 * w) * RB;
  }
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int jb = 0; jb < 4; ++jb) {
      // dims 32db + 8jb + 4hh + [0, 4): half hh of logical chunk 4db + jb
      u32x2 val;
      val[0] = pack2<BF>(o[db][4 * jb + 0] * inv, o[db][4 * jb + 1] * inv);
      val[1] = pack2<BF>(o[db][4 * jb + 2] * inv, o[db][4 * jb + 3] * inv);
      *reinterpret_cast<u32x2*>(obuf + r32 * RB + 16 * ((4 * db + jb) ^ KSWZ(r32)) + 8 * hh) = val;
    }
  if (row_ok && hh == 0) {
    // the row's (token, head) index, recomputed here rather than kept live
    // across the loop
    int re = row0 + 32 * w + r32;
    pin(re);
    const int te = re / g;
    const unsigned li = static_cast<unsigned>((q0 + te) * h_q_ + kvh * g + (re - te * g));
    lse_[li] = l_tot > 0.f ? m_run + log2f(l_tot) : -INFINITY;
  }
  // lane: chunk pc of rows lrow + RPL*i (i < 32 / RPL) of the wave's block
#pragma unroll
  for (int i = 0; i < 32 / RPL; ++i) {
    const int rr = RPL * i + lrow;                 // row within the wave's 32
    const int Rg = row0 + 32 * w + rr;
    const int tg = Rg / g;
    const u32x4 val = *reinterpret_cast<const u32x4*>(obuf + rr * RB + 16 * (pc ^ KSWZ(rr)));
    if (tg < qo_len && q0 + tg < total_q_) {
      const unsigned orr = static_cast<unsigned>((q0 + tg) * h_q_ + kvh * g + (Rg - tg * g));
      *reinterpret_cast<u32x4*>(static_cast<uint16_t*>(out_) + static_cast<size_t>(orr) * D + 8 * pc) = val;
    }
  }
}

#undef KSWZ
#undef VSWZ

template <int NW, bool BF, int D, int LAYOUT, int MASK>
void launch_r(const AttnParams& p, dim3 grid, hipStream_t stream) {
  if (p.rope_k)
    hipLaunchKernelGGL((attn_fwd_kernel<NW, BF, D, LAYOUT, MASK, true>), grid, dim3(64 * NW), 0, stream, p);
  else
    hipLaunchKernelGGL((attn_fwd_kernel<NW, BF, D, LAYOUT, MASK, false>), grid, dim3(64 * NW), 0, stream, p);
}

template <int NW, bool BF, int D>
void launch_d(const AttnParams& p, KvLayout layout, MaskKind mask, dim3 grid, hipStream_t stream) {
  if (layout == kContiguous) {
    if (mask == kMaskTree) launch_r<NW, BF, D, kContiguous, kMaskTree>(p, grid, stream);
    else launch_r<NW, BF, D, kContiguous, kMaskCausal>(p, grid, stream);
  } else {
    if (mask == kMaskTree) launch_r<NW, BF, D, kPaged, kMaskTree>(p, grid, stream);
    else launch_r<NW, BF, D, kPaged, kMaskCausal>(p, grid, stream);
  }
}

template <int NW>
hipError_t launch_nw(const AttnParams& p, int is_bf16, int head_dim, KvLayout layout, MaskKind mask,
                     hipStream_t stream) {
  // Upper bound on the number of work items, plus slack so that the
  // XCD-contiguous mapping (8 * ceil(items / 8) blocks) always fits.
  constexpr long bm = 32 * NW;
  const long tiles = (static_cast<long>(p.total_q) * p.group + bm - 1) / bm + p.batch;
  long blocks = tiles * p.h_kv * (p.num_splits > 1 ? p.num_splits : 1) + 7;
  blocks = (blocks + 7) / 8 * 8;
  if (blocks > INT_MAX) return hipErrorInvalidValue;
  const dim3 grid(static_cast<unsigned>(blocks));
  if (is_bf16) {
    if (head_dim == 128) launch_d<NW, true, 128>(p, layout, mask, grid, stream);
    else launch_d<NW, true, 64>(p, layout, mask, grid, stream);
  } else {
    if (head_dim == 128) launch_d<NW, false, 128>(p, layout, mask, grid, stream);
    else launch_d<NW, false, 64>(p, layout, mask, grid, stream);
  }
  return hipGetLastError();
}

}  // namespace

// Eight-wave workgroups load each K/V tile once for 256 query rows (half the
// loads per row) but are one per CU, so they pay off only when the 256-row
// items cover the device's CUs at least twice; split-KV ranges are short and
// use four waves. (The item count here ignores ragged tails: a lower bound.)
namespace {
std::atomic<int> g_waves_override{0};

// Compute units of the current device (256 on a whole MI355X, fewer on a
// partition of one), queried once per device; 256 when none is visible.
constexpr int kMaxDevices = 64;
std::atomic<int> g_cu_count[kMaxDevices];

long current_cu_count() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    (void)hipGetLastError();   // clear the sticky error state of a failed query
    return 256;
  }
  int n = g_cu_count[dev].load(std::memory_order_relaxed);
  if (n <= 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) {
      (void)hipGetLastError();
      n = 256;
    }
    g_cu_count[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}
}  // namespace

void set_waves_override(int waves) { g_waves_override.store(waves, std::memory_order_relaxed); }

int waves_per_item(const AttnParams& p) {
  if (p.num_splits > 1) return 4;
  const int forced = g_waves_override.load(std::memory_order_relaxed);
  if (forced != 0) return forced;
  const long items8 = (static_cast<long>(p.total_q) * p.group + 255) / 256 * p.h_kv;
  return items8 >= 2 * current_cu_count() ? 8 : 4;
}

hipError_t launch_attn(const AttnParams& p, int is_bf16, int head_dim, KvLayout layout,
                       MaskKind mask, hipStream_t stream) {
  if (waves_per_item(p) == 8) return launch_nw<8>(p, is_bf16, head_dim, layout, mask, stream);
  return launch_nw<4>(p, is_bf16, head_dim, layout, mask, stream);
}

}  // namespace ra
