// Multi-head latent attention prefill over a paged latent cache, for gfx950.
//
// What is computed follows the "_kernel_common.py" page: AttnKind MLA, the
// buffers of _alloc_mla_qkvo_buffers (one combined KV tile of d_qk columns
// per key, read as K over all d_qk columns and as V over the first d_latent,
// and an O accumulator of d_latent columns), the prefill macros
// (compute_s_gemm, softmax_update_causal, compute_o_gemm) and the epilogue
// paged_store_output_lse with every query head in one group, plus
// _causal_mask. Here d_latent = 512 and d_qk = 512 + 64.
//
// How it is computed on CDNA4:
//  * Work item = (sequence, tile of 128 packed query rows); packed row R is
//    token R / h_q, head R % h_q, since every head reads the same latent
//    rows. A workgroup is four waves of 32 rows each, one wave per SIMD:
//    a wave keeps its 32 Q rows (576 values each) in 144 VGPRs and the O^T
//    accumulators (512 dims x 32 rows in fp32, 256 registers) in the
//    accumulation registers, which only one wave per SIMD can hold.
//  * Scores are computed transposed, S^T = KV Q^T, on
//    v_mfma_f32_32x32x16_{bf16,f16} (36 steps over d_qk per 32-key block),
//    so each lane holds one query row: row max and sum are in-lane plus one
//    v_permlane32_swap, and P converts in place into the B operand of
//    O^T += V^T P^T (16 MFMAs of 32 dims per 16-key piece).
//  * The score MFMAs are inline assembly with ordinary-register operands:
//    O takes all 256 accumulation registers, and with the compiler's own
//    MFMAs the score accumulator landed there too, so one O block moved out
//    and back around every tile (80 register moves per tile). The compiler
//    does not see these MFMAs, so the wait states before vector instructions
//    read their results are written out (20, more than an MFMA of this shape
//    needs); consecutive MFMAs accumulating in place, and LDS reads reusing
//    an operand register right after its MFMA issued, need none (the
//    compiler schedules its own MFMAs the same way).
//  * With one wave per SIMD nothing hides a wave's own LDS latency, so the
//    operands are read ahead explicitly: K and Q fragments four MFMAs before
//    their use, V pieces four PV steps ahead (the first four behind the score
//    MFMAs, so they arrive during the softmax), the order pinned with
//    scheduling barriers (left to itself the compiler reads each operand
//    right before its MFMA and waits for it).
//  * KV tiles of 32 keys go from HBM straight into LDS with
//    global_load_lds_dwordx4, two stages of 36 KiB: the latent part as
//    32 rows of 1024 bytes (one wave-wide load per row) and the rope part as
//    32 rows of 128 bytes. With 16-byte chunks and 64 four-byte banks, a
//    chunk's bank group is its index mod 16 in the latent rows; logical
//    chunk c of latent row r sits at c ^ lswz(r), lswz(r) = 4(r mod 4) +
//    (r / 4 mod 4), which keeps both the b128 K-operand reads (16 rows, one
//    chunk) and the ds_read_b64_tr_b16 V-operand reads (4 rows x 4 chunks)
//    conflict-free. In the rope rows (two per 256 bytes) chunk c of row r
//    sits at c ^ (r / 2 mod 8).
//  * Each wave loads an 8-key block per tile: with page size 16 and a
//    tile grid aligned to 32 keys that block is half a page, so one page
//    number per wave and tile (loaded a tile ahead). Blocks past the chunk's end or on
//    an invalid page are loaded row by row and zero-filled.
//  * Causal tiles are classified per wave as skipped, full or partial; the
//    softmax runs in the log2 domain with the running maximum moved (and O
//    rescaled) only when a tile raises it by more than 8.

#include <climits>
#include <type_traits>

#include "device_common.h"
#include "ra_internal.h"

namespace ra {

namespace {

typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4i16 lds_v4i16;

constexpr int kDL = 512;                    // latent width (V and O)
constexpr int kDR = 64;                     // rope width
constexpr int kDQK = kDL + kDR;             // score reduction width
constexpr int kTN = 32;                     // keys per tile
constexpr int kNW = 4;                      // waves per workgroup
constexpr int kMBM = 32 * kNW;              // packed rows per work item
constexpr int kLatRB = kDL * 2;             // LDS bytes per latent row
constexpr int kRopeRB = kDR * 2;            // LDS bytes per rope row
constexpr int kRowB = kDQK * 2;             // bytes per cached token
constexpr int kLatTile = kTN * kLatRB;      // 32 KiB
constexpr int kStage = kLatTile + kTN * kRopeRB;   // 36 KiB
constexpr int kMlaStages = 2;
constexpr int kQS = 16;                     // Q steps (16 dims each) kept in LDS
constexpr int kQRB = kQS * 32;              // LDS bytes per Q row (512)
constexpr int kQOff = kMlaStages * kStage;  // Q rows after the KV stages
constexpr int kMlaSmem = kQOff + kMBM * kQRB;   // 72 KiB + 64 KiB
// P = 2^(s - m_ref) is fed to the MFMA in the input type: at most 2^15 in
// fp16 (largest value 65504); bf16 has fp32's exponent range, where 2^64
// leaves room for the fp32 sums of O and l.
template <bool BF>
constexpr float kMlaHeadroom = BF ? 64.0f : 15.0f;

// LDS chunk swizzles (16-byte chunks; in rows of 512 or 1024 bytes a chunk's
// bank group is its index mod 16, in 128-byte rows it is 8 (row mod 2) +
// index)
__device__ __forceinline__ int lswz(int r) { return 4 * (r & 3) + ((r >> 2) & 3); }
__device__ __forceinline__ int rswz(int r) { return (r >> 1) & 7; }
__device__ __forceinline__ int qswz(int r) { return r & 15; }

template <bool BF>
__global__ __launch_bounds__(64 * kNW, 1) void mla_fwd_kernel(MlaParams p) {
  static_assert(kMlaSmem <= 160 * 1024, "LDS");
  static_assert(kNW * 32 * kLatRB <= kMlaSmem, "output staging fits");
  __shared__ __attribute__((aligned(1024))) char smem[kMlaSmem];
  __shared__ int votes[kNW];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int r32 = lane & 31;
  const int hh = lane >> 5;

  const auto q_ = p.q;
  const auto out_ = p.out;
  const auto lse_ = p.lse;
  const auto h_q_ = p.h_q;
  const auto total_q_ = p.total_q;
  const auto num_pages_ = p.num_pages;
  const auto nnz_pages_ = p.nnz_pages;
  const float sc = p.sm_scale_log2;

  int b = 0, kvh = 0, tile = 0, split = 0, q0_m = 0, qo_len_m = 0;
  if (!locate_item(p.q_indptr, p.batch, h_q_, 1, 1, kMBM, b, kvh, tile, split, q0_m, qo_len_m))
    return;   // uniform over the workgroup
  b = __builtin_amdgcn_readfirstlane(b);
  tile = __builtin_amdgcn_readfirstlane(tile);
  const int g = h_q_;
  const int q0 = __builtin_amdgcn_readfirstlane(q0_m);
  const int qo_len = __builtin_amdgcn_readfirstlane(qo_len_m);
  const int row0 = tile * kMBM;

  // ---- this sequence's chunk: pages [page_base, page_end), kv_len keys ----
  int pv = 0;
  {
    const int32_t* src = p.page_indptr + b;
    if (lane == 1) src = p.page_indptr + b + 1;
    if (lane == 2) src = p.last_page_len + b;
    pv = *src;
  }
  const int page_base = __builtin_amdgcn_readlane(pv, 0);
  const int page_hi = __builtin_amdgcn_readlane(pv, 1);
  const int last_len = __builtin_amdgcn_readlane(pv, 2);
  const int np = page_hi - page_base;
  const int kv_len = np > 0 ? max((np - 1) * 16 + last_len, 0) : 0;
  const int page_end = min(page_hi, nnz_pages_);

  // ---- this lane's query row and its visible keys [0, lim) ----
  const int R = row0 + w * 32 + r32;
  const int t = R / g;
  const int head = R - t * g;
  const bool row_ok = t < qo_len && q0 + t < total_q_;
  const bool causal = p.causal != 0;
  const int lim = causal ? min(kv_len, kv_len - qo_len + t + 1) : kv_len;
  const int t_lo = (row0 + w * 32) / g;
  const int t_hi = min((row0 + w * 32 + 31) / g, qo_len - 1);
  const bool wave_active = t_lo < qo_len;
  const int lim_lo = causal ? min(kv_len, kv_len - qo_len + t_lo + 1) : kv_len;
  const int lim_hi = causal ? min(kv_len, kv_len - qo_len + t_hi + 1) : kv_len;
  const int t_last = min((row0 + kMBM - 1) / g, qo_len - 1);
  const int kv_hi = causal ? min(kv_len, kv_len - qo_len + t_last + 1) : kv_len;
  const int n_tiles = kv_hi > 0 ? (kv_hi + kTN - 1) / kTN : 0;

  // ---- KV tile loads: wave w fills keys [8w, 8w + 8) of each tile, half a
  // page (tiles start at multiples of 32) ----
  const __amdgpu_buffer_rsrc_t page_rsrc = make_rsrc(p.page_values, 4L * nnz_pages_);
  auto fetch_page = [&](int j0) __attribute__((always_inline)) -> int {
    return load_i32(page_rsrc, page_base + ((j0 + 8 * w) >> 4));
  };
  const char* pages_ = reinterpret_cast<const char*>(p.pages);
  constexpr uint32_t kPageB = 16 * kRowB;
  const int rl = lane >> 3, rc = lane & 7;   // rope rows: one wave-wide load covers 8 rows
  auto issue_tile = [&](int j0, char* stage, int pg) __attribute__((always_inline)) {
    const int B = j0 + 8 * w;
    const int pidx = page_base + (B >> 4);
    const int slot0 = B & 15;
    char* lat = stage + (8 * w) * kLatRB;
    char* rope = stage + kLatTile + (8 * w) * kRopeRB;
    const bool page_ok = pidx < page_end && static_cast<unsigned>(pg) < static_cast<unsigned>(num_pages_);
    const char* base = pages_ + static_cast<size_t>(static_cast<uint32_t>(pg)) * kPageB +
                       static_cast<uint32_t>(slot0) * kRowB;
    if (page_ok && B + 8 <= kv_len) {
#pragma unroll
      for (int r = 0; r < 8; ++r)
        dma16s(base, static_cast<uint32_t>(r * kRowB + 16 * (lane ^ lswz(8 * w + r))), lat + r * kLatRB);
      dma16s(base, static_cast<uint32_t>(rl * kRowB + kLatRB + 16 * (rc ^ rswz(8 * w + rl))), rope);
    } else {
      // row by row: rows past the chunk or on an invalid page read as zero
#pragma unroll
      for (int r = 0; r < 8; ++r) {
        if (page_ok && B + r < kv_len)
          dma16(base + r * kRowB + 16 * (lane ^ lswz(8 * w + r)), lat + r * kLatRB);
        else
          *reinterpret_cast<u32x4*>(lat + r * kLatRB + 16 * lane) = u32x4{0, 0, 0, 0};
      }
      if (page_ok && B + rl < kv_len)
        dma16(base + rl * kRowB + kLatRB + 16 * (rc ^ rswz(8 * w + rl)), rope);
      else
        *reinterpret_cast<u32x4*>(rope + 16 * lane) = u32x4{0, 0, 0, 0};
    }
  };

  // ---- Q: lane holds row R, dims 16 s + 8 hh + [0, 8). Steps s < kQS go to
  // this wave's rows of the LDS Q block (chunk c of row r at c ^ qswz(r)),
  // the others stay in registers ----
  u32x4 qf[kDQK / 16 - kQS];
  char* const qrows = smem + kQOff + (32 * w) * kQRB;
  {
    u32x4 ql[kQS];
#pragma unroll
    for (int s = 0; s < kQS; ++s) ql[s] = u32x4{0, 0, 0, 0};
#pragma unroll
    for (int s = 0; s < kDQK / 16 - kQS; ++s) qf[s] = u32x4{0, 0, 0, 0};
    if (row_ok) {
      const unsigned qr = static_cast<unsigned>((q0 + t) * h_q_ + head);
      const uint16_t* qrow = q_ + static_cast<size_t>(qr) * kDQK + 8 * hh;
#pragma unroll
      for (int s = 0; s < kQS; ++s) ql[s] = *reinterpret_cast<const u32x4*>(qrow + 16 * s);
#pragma unroll
      for (int s = kQS; s < kDQK / 16; ++s) qf[s - kQS] = *reinterpret_cast<const u32x4*>(qrow + 16 * s);
    }
#pragma unroll
    for (int s = 0; s < kQS; ++s)
      *reinterpret_cast<u32x4*>(qrows + r32 * kQRB + 16 * ((2 * s + hh) ^ qswz(r32))) = ql[s];
  }

  // per-lane LDS offsets of the MFMA operands (swizzles depend on the row
  // mod 16 only). K: row r32 of the tile, logical chunk 2 s + hh ->
  // physical (2 s) ^ y, y = hh ^ swizzle(r32); Q likewise in the Q block.
  const int ylat = hh ^ lswz(r32);
  const int yrope = hh ^ rswz(r32);
  const int yq = hh ^ qswz(r32);
  int koff[8], qoff[8];
#pragma unroll
  for (int u = 0; u < 8; ++u) {
    koff[u] = r32 * kLatRB + 16 * ((2 * u) ^ ylat);
    qoff[u] = kQOff + (32 * w + r32) * kQRB + 16 * ((2 * u) ^ yq);
  }
  int kroff[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) kroff[u] = kLatTile + r32 * kRopeRB + 16 * ((2 * u) ^ yrope);
  // V pieces (ds_read_b64_tr_b16): 16-lane groups read rows
  // 4 hh + (gi >> 2) (+ 8 for the second read) of a 16-key piece, dims
  // 32 db + 16 (grp & 1) + 4 (gi & 3); by db mod 4 (higher bits of db move
  // the chunk by 256-byte multiples).
  int voff[2][4];
  {
    const int gi = lane & 15, grp = lane >> 4;
    const int vrow = 4 * hh + (gi >> 2);
    const int clo = 2 * (grp & 1) + ((gi & 3) >> 1);
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const int vr = vrow + 8 * e;
#pragma unroll
      for (int dq = 0; dq < 4; ++dq)
        voff[e][dq] = vr * kLatRB + 16 * ((4 * dq + clo) ^ lswz(vr)) + 8 * (gi & 1);
    }
  }

  // ---- online softmax against a fixed reference per row ----
  // A row's reference m_ref is the maximum of its first tile with a visible
  // key (O and l are still zero then). Later tiles are accumulated with
  // P = 2^(s - m_ref) without rescaling O: P may exceed 1 by up to
  // kMlaHeadroom (log2 units). If any row of the workgroup outgrows that,
  // the item is computed once more with m_ref = that row's final maximum,
  // which no score exceeds. (The accumulators are never touched by vector
  // instructions inside the loop, so they stay in the accumulation registers.)
  constexpr float kHead = kMlaHeadroom<BF>;
  float m_ref = -INFINITY;   // second attempt: the row maximum of the first
  float m_seen = -INFINITY;
  float l_run = 0.f;
  float l_mma = 0.f;
  f32x16 o[kDL / 32];
  bool over = false;

  auto compute = [&](int j0, bool masked, auto so_c) __attribute__((always_inline)) {
    constexpr int SO = decltype(so_c)::value;
    const char* const sm = smem + SO;
    constexpr int NS = kDQK / 16;   // 36 steps
    constexpr int kAhead = 4;
    // operands of step s (compile-time s): K fragment, and the Q fragment
    // for the steps whose Q lives in LDS
    auto kfrag = [&](int s) __attribute__((always_inline)) -> u32x4 {
      if (s < 32) return *reinterpret_cast<const u32x4*>(sm + koff[s & 7] + 256 * (s >> 3));
      return *reinterpret_cast<const u32x4*>(sm + kroff[(s - 32) & 3]);
    };
    auto qfrag = [&](int s) __attribute__((always_inline)) -> u32x4 {
      return *reinterpret_cast<const u32x4*>(smem + qoff[s & 7] + 256 * (s >> 3));
    };
    f32x16 sacc;
    u32x4 kf[kAhead], qa[kAhead];
#pragma unroll
    for (int x = 0; x < kAhead; ++x) {
      kf[x] = kfrag(x);
      if (x < kQS) qa[x] = qfrag(x);
    }
#pragma unroll
    for (int x = 0; x < NS; ++x) {
      const u32x4 ck = kf[x % kAhead];
      const u32x4 cq = x < kQS ? qa[x % kAhead] : qf[x - kQS];
      if (x + kAhead < NS) {
        kf[x % kAhead] = kfrag(x + kAhead);
        if (x + kAhead < kQS) qa[x % kAhead] = qfrag(x + kAhead);
      }
      // score MFMAs in ordinary registers (O fills the accumulation
      // registers); the first starts from zero, the rest accumulate in place
      if (x == 0) {
        if constexpr (BF)
          asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=&v"(sacc) : "v"(ck), "v"(cq));
        else
          asm volatile("v_mfma_f32_32x32x16_f16 %0, %1, %2, 0" : "=&v"(sacc) : "v"(ck), "v"(cq));
      } else {
        if constexpr (BF)
          asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(sacc) : "v"(ck), "v"(cq));
        else
          asm volatile("v_mfma_f32_32x32x16_f16 %0, %1, %2, %0" : "+v"(sacc) : "v"(ck), "v"(cq));
      }
    }

    // V pieces of the first kVA PV steps, read behind the score MFMAs so that
    // they have arrived when the softmax is done
    constexpr int NV = (kTN / 16) * (kDL / 32);   // PV steps: 16-key piece sp, 32 dims db
    constexpr int kVA = 4;
    auto vpiece = [&](int x) __attribute__((always_inline)) -> u32x4 {
      const int sp = x / (kDL / 32), db = x % (kDL / 32);
      const int add = 16 * sp * kLatRB + 256 * (db >> 2);
      const v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(sm + voff[0][db & 3] + add));
      const v4i16 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(sm + voff[1][db & 3] + add));
      u32x4 a;
      a[0] = __builtin_bit_cast(u32x2, lo)[0];
      a[1] = __builtin_bit_cast(u32x2, lo)[1];
      a[2] = __builtin_bit_cast(u32x2, hi)[0];
      a[3] = __builtin_bit_cast(u32x2, hi)[1];
      return a;
    };
    u32x4 vr[kVA];
#pragma unroll
    for (int x = 0; x < kVA; ++x) vr[x] = vpiece(x);
    // Wait states before vector instructions read the score MFMAs' results:
    // the compiler does not see the inline MFMAs above, so it inserts none.
    // 20 is more than an MFMA of this shape needs (and more than the
    // compiler inserts after its own ones); stalls only add to it.
    asm volatile("s_nop 15\n\ts_nop 3" : "+v"(sacc)::"memory");
    // issue order: the first kAhead steps' reads, then each MFMA followed by
    // the reads it made room for, then the first V reads
    __builtin_amdgcn_sched_group_barrier(0x100, kAhead + (kAhead < kQS ? kAhead : kQS), 0);
    static_assert(kAhead <= kQS && kQS <= NS, "read-ahead ranges");
#pragma unroll
    for (int x = 0; x < kQS - kAhead; ++x) {   // K and Q fragments
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
    }
#pragma unroll
    for (int x = kQS - kAhead; x < NS - kAhead; ++x) {   // K only
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, kAhead, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, 2 * kVA, 0);
    if (masked) {
      // key j0 + 8 (r / 4) + 4 hh + r % 4 is visible iff below lim
      const int rel = lim - j0 - 4 * hh;
#pragma unroll
      for (int r = 0; r < 16; ++r)
        if (8 * (r >> 2) + (r & 3) >= rel) sacc[r] = -INFINITY;
    }
    float mx = -INFINITY;
#pragma unroll
    for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sacc[r]);
    mx = pair_max(mx) * sc;
    m_seen = fmaxf(m_seen, mx);
    if (m_ref == -INFINITY) m_ref = mx;    // first visible keys of the row (or still none)
    over |= mx > m_ref + kHead;
    const float m_use = (m_ref == -INFINITY) ? 0.f : m_ref;
    float lsum = 0.f;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      // (a row whose scores outgrow the reference may overflow P here; the
      // item is then computed again and this attempt's results are dropped)
      const float pv = __builtin_amdgcn_exp2f(fmaf(sacc[r], sc, -m_use));
      sacc[r] = pv;
      lsum += pv;
    }
    l_run += lsum;
    u32x4 pf[kTN / 16];
#pragma unroll
    for (int sp = 0; sp < kTN / 16; ++sp) {
      const int e0 = 8 * sp;
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        pf[sp][u] = pack2<BF>(sacc[e0 + 2 * u], sacc[e0 + 2 * u + 1]);
        l_mma = add_pair<BF>(pf[sp][u], l_mma);
      }
    }
    // O^T += V^T P^T, V pieces read kVA steps ahead
#pragma unroll
    for (int x = 0; x < NV; ++x) {
      const u32x4 cv = vr[x % kVA];
      if (x + kVA < NV) vr[x % kVA] = vpiece(x + kVA);
      o[x % (kDL / 32)] = mma32<BF>(cv, pf[x / (kDL / 32)], o[x % (kDL / 32)]);
    }
#pragma unroll
    for (int x = 0; x < NV; ++x) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      if (x + kVA < NV) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
    }
  };

  int page_next = 0;
  auto tile_step = [&](int it, auto so_c) __attribute__((always_inline)) {
    constexpr int SO = decltype(so_c)::value;
    const int j0 = it * kTN;
    wait_all_and_barrier();   // tile it is in LDS; everyone is done with tile it-1
    if (it + 1 < n_tiles) {
      issue_tile(j0 + kTN, smem + (SO == 0 ? kStage : 0), __builtin_amdgcn_readfirstlane(page_next));
      if (it + 2 < n_tiles) page_next = fetch_page(j0 + 2 * kTN);
    }
    int cls = (j0 >= lim_hi) ? 0 : (j0 + kTN <= lim_lo ? 1 : 2);
    cls = __builtin_amdgcn_readfirstlane(cls);
    if (wave_active && cls != 0) compute(j0, cls == 2, so_c);
  };
#pragma unroll 1
  for (int attempt = 0; attempt < 2; ++attempt) {
#pragma unroll
    for (int i = 0; i < kDL / 32; ++i) o[i] = f32x16{};
    l_run = 0.f;
    l_mma = 0.f;
    over = false;
    if (n_tiles > 0) page_next = fetch_page(0);
    pin(page_next);
    if (n_tiles > 0) issue_tile(0, smem, __builtin_amdgcn_readfirstlane(page_next));
    if (n_tiles > 1) page_next = fetch_page(kTN);
    for (int it = 0; it < n_tiles; it += 2) {
      tile_step(it, std::integral_constant<int, 0>{});
      if (it + 1 < n_tiles) tile_step(it + 1, std::integral_constant<int, kStage>{});
    }
    if (attempt == 1) break;
    // did any row of the workgroup outgrow its reference? (one word per
    // wave, read after a barrier)
    __syncthreads();   // all waves are done with the last tile
    const int vote = __any(over && row_ok) ? 1 : 0;   // over the whole wave
    if (lane == 0) votes[w] = vote;
    __syncthreads();
    int any = 0;
#pragma unroll
    for (int v = 0; v < kNW; ++v) any |= votes[v];
    if (__builtin_amdgcn_readfirstlane(any) == 0) break;
    __syncthreads();   // everyone has read the votes before tile 0 is reissued
    m_ref = m_seen;    // the row's maximum: no score exceeds it now
  }

  // ---- epilogue: out = O / l (dtype), lse = m + log2(l) ----
  const float l_tot = pair_sum(l_run);
  const float l_o = pair_sum(l_mma);
  const float inv = l_o > 0.f ? 1.f / l_o : 0.f;
  __syncthreads();   // every wave is done with the stages and its Q rows
  char* obuf = smem + (32 * w) * kLatRB;
#pragma unroll
  for (int db = 0; db < kDL / 32; ++db)
#pragma unroll
    for (int jb = 0; jb < 4; ++jb) {
      // dims 32 db + 8 jb + 4 hh + [0, 4): half hh of logical chunk 4 db + jb
      u32x2 val;
      val[0] = pack2<BF>(o[db][4 * jb + 0] * inv, o[db][4 * jb + 1] * inv);
      val[1] = pack2<BF>(o[db][4 * jb + 2] * inv, o[db][4 * jb + 3] * inv);
      *reinterpret_cast<u32x2*>(obuf + r32 * kLatRB + 16 * ((4 * db + jb) ^ lswz(r32)) + 8 * hh) = val;
    }
  if (row_ok && hh == 0) {
    const unsigned li = static_cast<unsigned>((q0 + t) * h_q_ + head);
    lse_[li] = l_tot > 0.f ? m_ref + log2f(l_tot) : -INFINITY;
  }
  // one row of 1024 bytes per wave-wide store (rows this wave wrote)
#pragma unroll 4
  for (int rr = 0; rr < 32; ++rr) {
    const int Rg = row0 + 32 * w + rr;
    const int tg = Rg / g;
    const u32x4 val = *reinterpret_cast<const u32x4*>(obuf + rr * kLatRB + 16 * (lane ^ lswz(rr)));
    if (tg < qo_len && q0 + tg < total_q_) {
      const unsigned orr = static_cast<unsigned>((q0 + tg) * h_q_ + (Rg - tg * g));
      *reinterpret_cast<u32x4*>(static_cast<uint16_t*>(out_) + static_cast<size_t>(orr) * kDL + 8 * lane) = val;
    }
  }
}

}  // namespace

hipError_t launch_mla(const MlaParams& p, int is_bf16, hipStream_t stream) {
  // one item per (sequence, 128 packed rows), at most ceil(total_q h_q / 128)
  // + batch of them; XCD-contiguous mapping needs 8 * ceil(items / 8) blocks
  const long items = (static_cast<long>(p.total_q) * p.h_q + kMBM - 1) / kMBM + p.batch;
  long blocks = (items + 7) / 8 * 8 + 8;
  if (blocks > INT_MAX) return hipErrorInvalidValue;
  const dim3 grid(static_cast<unsigned>(blocks));
  if (is_bf16)
    hipLaunchKernelGGL(mla_fwd_kernel<true>, grid, dim3(64 * kNW), 0, stream, p);
  else
    hipLaunchKernelGGL(mla_fwd_kernel<false>, grid, dim3(64 * kNW), 0, stream, p);
  return hipGetLastError();
}

}  // namespace ra
