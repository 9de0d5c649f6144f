// Device helpers for the gfx950 kernels: vector types, fp16/bf16 conversion,
// the 32x32x16 MFMA wrapper, wave reductions and the rotary embedding.
#pragma once

#include <hip/hip_runtime.h>
#include <climits>
#include <stdint.h>

namespace ra {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));

// ---- storage-type conversion (round to nearest even) ----------------------
template <bool BF>
__device__ __forceinline__ float to_f32(uint32_t bits16) {
  if constexpr (BF) {
    return __uint_as_float(bits16 << 16);
  } else {
    return static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(bits16)));
  }
}

template <bool BF>
__device__ __forceinline__ uint32_t from_f32(float x) {
  if constexpr (BF) {
    return __builtin_bit_cast(uint16_t, static_cast<__bf16>(x));
  } else {
    return __builtin_bit_cast(uint16_t, static_cast<_Float16>(x));
  }
}

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

// Two floats -> one dword of two 16-bit values (one v_cvt_pk_{bf16,f16}_f32).
template <bool BF>
__device__ __forceinline__ uint32_t pack2(float lo, float hi) {
  const f32x2 v = {lo, hi};
  if constexpr (BF) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
  } else {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, f16x2));
  }
}

// c + lo + hi of a dword holding two 16-bit values (v_dot2c_f32_{f16,bf16}
// with the constant pair (1, 1)): sums exactly the rounded values that feed
// an MFMA.
template <bool BF>
__device__ __forceinline__ float add_pair(uint32_t packed, float c) {
  if constexpr (BF) {
    const bf16x2 one = {static_cast<__bf16>(1.0f), static_cast<__bf16>(1.0f)};
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, packed), one, c, false);
  } else {
    const f16x2 one = {static_cast<_Float16>(1.0f), static_cast<_Float16>(1.0f)};
    return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, packed), one, c, false);
  }
}

// Element e (0..7) of a 16-byte chunk of 16-bit values.
__device__ __forceinline__ uint32_t half_of(const u32x4& x, int e) {
  return (x[e >> 1] >> ((e & 1) * 16)) & 0xffffu;
}

// ---- MFMA: D(32x32, f32) += A(32x16) * B(16x32) ---------------------------
// A: lane l supplies row l%32, 8 K-values; B: lane l supplies column l%32,
// 8 K-values, with the same K-slot assignment as A. Result: lane l holds
// column l%32, rows 8*(r/4) + 4*(l/32) + r%4 in element r.
template <bool BF>
__device__ __forceinline__ f32x16 mma32(const u32x4& a, const u32x4& b, const f32x16& c) {
  if constexpr (BF) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
  } else {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                  __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
  }
}

// ---- memory helpers ----------------------------------------------------------
// Bounds-checked loads through a buffer resource: offsets at or past the end
// of the range (negative offsets wrap past it) read as zero, with no branch.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, long bytes) {
  const int n = static_cast<int>(min(max(bytes, 0L), static_cast<long>(INT_MAX)));
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), static_cast<short>(0), n,
                                           0x00020000);
}
__device__ __forceinline__ int load_i32(__amdgpu_buffer_rsrc_t r, int index) {
  return __builtin_amdgcn_raw_buffer_load_b32(r, index * 4, 0, 0);
}
__device__ __forceinline__ int2 load_i32x2(__amdgpu_buffer_rsrc_t r, int index) {
  const auto v = __builtin_amdgcn_raw_buffer_load_b64(r, index * 8, 0, 0);
  return make_int2(static_cast<int>(v[0]), static_cast<int>(v[1]));
}
// An opaque use of a loaded value at the point where it is needed: without it
// the compiler moves dependent arithmetic up to the load and waits there,
// before the remaining loads of the prologue have been issued.
__device__ __forceinline__ void pin(int& x) { asm volatile("" : "+v"(x)); }
__device__ __forceinline__ void pin(double& x) { asm volatile("" : "+v"(x)); }

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

// Same, with a wave-uniform 64-bit base in SGPRs and a 32-bit per-lane
// offset (the saddr form: no 64-bit address arithmetic per lane).
__device__ __forceinline__ void dma16s(const char* sbase, uint32_t voff, const void* lds_base) {
  const unsigned lds = static_cast<unsigned>(
      reinterpret_cast<size_t>((__attribute__((address_space(3))) const char*)lds_base));
  asm volatile("global_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(sbase), "{m0}"(lds) : "memory");
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

// ---- wave reductions (wave64) ---------------------------------------------
__device__ __forceinline__ int wave_sum(int x) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) x += __shfl_xor(x, m, 64);
  return x;
}

__device__ __forceinline__ int wave_inclusive_scan(int x) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    int y = __shfl_up(x, d, 64);
    if (lane >= d) x += y;
  }
  return x;
}

// Locate this workgroup's work item. Returns false when the block has none.
// Item list: for each KV head, for each sequence b (in order), ranks
// 0..tiles_b-1 with rank 0 = the last (heaviest under a causal mask) q-tile.
// KV-head-major order: with the list cut into 8 equal chunks (one per XCD),
// every XCD gets the same mix of long and short sequences (exactly one KV
// head each when h_kv = 8), while all tiles of one (sequence, KV head) still
// share an XCD's L2.
// With split-KV (splits > 1) each q-tile is `splits` items, one per KV range.
// Also returns the sequence's query offset q0 and length qo_len.
__device__ inline bool locate_item(const int32_t* q_indptr, int batch, int group, int h_kv, int splits, int bm,
                            int& b, int& kvh, int& tile, int& split, int& q0, int& qo_len) {
  const int lane = threadIdx.x & 63;
  // q-tiles of sequence i, and its query range
  auto count = [&](int i, int& lo, int& len) __attribute__((always_inline)) -> int {
    lo = 0;
    len = 0;
    if (i >= batch) return 0;
    lo = q_indptr[i];
    len = max(q_indptr[i + 1] - lo, 0);
    return (len * group + bm - 1) / bm * splits;
  };
  int lo0, len0;
  const int cnt0 = count(lane, lo0, len0);   // first 64 sequences, kept for the search
  int per_head = wave_sum(cnt0);
  for (int c0 = 64; c0 < batch; c0 += 64) {
    int lo, len;
    per_head += wave_sum(count(c0 + lane, lo, len));
  }
  const int total = per_head * h_kv;
  // XCD-contiguous mapping: block L runs on XCD L % 8; give XCD x the items
  // [x*chunk, (x+1)*chunk) in order.
  const int chunk = (total + 7) / 8;
  const int L = blockIdx.x;
  const int slot = L >> 3;
  if (slot >= chunk) return false;
  const int item = (L & 7) * chunk + slot;
  if (item >= total) return false;
  kvh = item / per_head;
  const int rem = item - kvh * per_head;
  int base = 0;
  for (int c0 = 0; c0 < batch; c0 += 64) {
    int lo = lo0, len = len0, cnt = cnt0;
    if (c0 > 0) cnt = count(c0 + lane, lo, len);
    const int incl = wave_inclusive_scan(cnt) + base;
    const unsigned long long hit = __ballot(c0 + lane < batch && rem < incl);
    if (hit) {
      const int l = __ffsll(static_cast<long long>(hit)) - 1;
      b = c0 + l;
      const int excl = __shfl(incl - cnt, l, 64);
      const int tiles_b = __shfl(cnt, l, 64) / splits;
      q0 = __shfl(lo, l, 64);
      qo_len = __shfl(len, l, 64);
      const int local = rem - excl;
      const int rank = local / splits;
      split = local - rank * splits;
      tile = tiles_b - 1 - rank;
      return true;
    }
    base = __shfl(incl, 63, 64);
  }
  return false;
}

// ---- lane l and lane l ^ 32 (v_permlane32_swap, no LDS traffic) ----------
// permlane32_swap(x, x) returns {x[l % 32], x[l % 32 + 32]} at lane l, i.e.
// both values of the pair in a lane-independent order.
__device__ __forceinline__ float pair_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

__device__ __forceinline__ float pair_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// ---- rotary embedding ------------------------------------------------------
// Rotate-half RoPE of the "_kernel_common.py" page (_rope): for dims k and
// k + D/2 the angle is float32(pos * scale) * inv_freq[k] with
// inv_freq[k] = theta^(-2k/D), and cos/sin are float32 values.
//   angle = pos_f * inv_freq (float64), n = nearest integer to angle/(pi/2),
//   r = angle - n*pi/2 with pi/2 split in two parts (|r| <= pi/4 + tiny),
//   all in float64, so r is accurate to ~1e-16 relative even for large
//   positions; sin r and cos r come from their Taylor series in float64
//   (sin through r^15, cos through r^16: the first omitted terms are below
//   5e-17 and 3e-18 on |r| <= pi/4; summed in Estrin's scheme, which rounds
//   differently from Horner's rule by a few float64 ulps at most), the
//   quadrant n mod 4 swaps and negates them, and each is rounded once to
//   float32. That is the correctly rounded float32 value
//   unless the exact one lies within a few float64 ulps of a float32
//   rounding boundary (about 4e-9 of arguments), so rotated values match a
//   reference that rounds float64 cos/sin the same way.
// n is taken as an int32, which holds it while |angle| < 3e9 (any int32
// position with scale <= 1).
// The rotated value is evaluated in float32 as cos*x + sin*partner (two
// rounded products and a rounded sum, no fused multiply-add) and rounded to
// the storage type.
__device__ __forceinline__ void rope_cos_sin(int pos, float scale, double inv_freq, float& c,
                                             float& s) {
  const float pos_f = static_cast<float>(pos) * scale;
  const double ang = static_cast<double>(pos_f) * inv_freq;
  const double kPio2Hi = 1.5707963267948966;       // float64(pi/2)
  const double kPio2Lo = 6.123233995736766e-17;    // pi/2 - kPio2Hi
  const double n = rint(ang * 0.6366197723675814);  // 2/pi
  double r = fma(-n, kPio2Hi, ang);
  r = fma(-n, kPio2Lo, r);
  const double r2 = r * r;
  // sin r = r + r^3 (-1/3! + r^2/5! - ... - r^12/15!) and
  // cos r = 1 + r^2 (-1/2! + r^2/4! - ... + r^14/16!); the two inner
  // polynomials in x = r^2 are evaluated in Estrin's scheme (pairs of
  // coefficients, then x^2 and x^4), which halves the dependent chain of
  // Horner's rule
  const double x2 = r2 * r2, x4 = x2 * x2;
  const double sa = fma(1.0 / 120.0, r2, -1.0 / 6.0);                  //  1/5!,  -1/3!
  const double sb = fma(1.0 / 362880.0, r2, -1.0 / 5040.0);            //  1/9!,  -1/7!
  const double sc = fma(1.0 / 6227020800.0, r2, -1.0 / 39916800.0);    //  1/13!, -1/11!
  const double sd = -1.0 / 1307674368000.0;                            // -1/15!
  const double sp = fma(fma(sd, x2, sc), x4, fma(sb, x2, sa));
  const double sr = fma(sp * r2, r, r);
  const double ca = fma(1.0 / 24.0, r2, -0.5);                         //  1/4!,  -1/2!
  const double cb = fma(1.0 / 40320.0, r2, -1.0 / 720.0);              //  1/8!,  -1/6!
  const double cc = fma(1.0 / 479001600.0, r2, -1.0 / 3628800.0);      //  1/12!, -1/10!
  const double cd = fma(1.0 / 20922789888000.0, r2, -1.0 / 87178291200.0);   // 1/16!, -1/14!
  const double cp = fma(fma(cd, x2, cc), x4, fma(cb, x2, ca));
  const double cr = fma(cp, r2, 1.0);
  const int q = static_cast<int>(n) & 3;
  const double sv = (q & 1) ? cr : sr;
  const double cv = (q & 1) ? sr : cr;
  s = static_cast<float>((q & 2) ? -sv : sv);
  c = static_cast<float>(((q + 1) & 2) ? -cv : cv);
}

// y1 = cos*x1 - sin*x2 (first half), y2 = cos*x2 + sin*x1 (second half),
// each product rounded to float32 and then the sum: contraction into a fused
// multiply-add is switched off here (the compiler would otherwise fuse them,
// and the result would differ from the twice-rounded one near ties of the
// storage-type rounding).
__device__ __forceinline__ void rope_pair(float c, float s, float x1, float x2, float& y1,
                                          float& y2) {
#pragma clang fp contract(off)
  y1 = c * x1 - s * x2;
  y2 = c * x2 + s * x1;
}

}  // namespace ra
