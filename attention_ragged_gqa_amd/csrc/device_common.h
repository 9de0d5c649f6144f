// Device helpers for the gfx950 kernels: vector types, fp16/bf16 conversion,
// the 32x32x16 MFMA wrapper, wave reductions and the rotary embedding.
#pragma once

#include <hip/hip_runtime.h>
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
// inv_freq[k] = theta^(-2k/D).
//   angle = pos_f * inv_freq (float64), n = nearest integer to angle/(pi/2),
//   r = angle - n*pi/2 with pi/2 split in two parts (|r| <= pi/4 + tiny),
//   all in float64, so r is accurate to ~1e-16 relative even for large
//   positions; then r is rounded to float32 and sin r, cos r come from their
//   Taylor series in float32 (sin through r^9, cos through r^10: truncation
//   below 2e-9 on |r| <= pi/4), and the quadrant n mod 4 swaps and negates
//   them. Against the correctly rounded float32 cos and sin the error is
//   below 1e-7 absolute (at most one float32 ulp away from zero crossings).
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
  double rd = fma(-n, kPio2Hi, ang);
  rd = fma(-n, kPio2Lo, rd);
  const float r = static_cast<float>(rd);
  const float r2 = r * r;
  // sin r = r - r^3/3! + r^5/5! - r^7/7! + r^9/9!
  float sp = 2.7557319e-06f;                        //  1/9!
  sp = fmaf(sp, r2, -1.9841270e-04f);               // -1/7!
  sp = fmaf(sp, r2, 8.3333333e-03f);                //  1/5!
  sp = fmaf(sp, r2, -1.6666667e-01f);               // -1/3!
  const float sr = fmaf(sp * r2, r, r);
  // cos r = 1 - r^2/2! + r^4/4! - r^6/6! + r^8/8! - r^10/10!
  float cp = -2.7557319e-07f;                       // -1/10!
  cp = fmaf(cp, r2, 2.4801587e-05f);                //  1/8!
  cp = fmaf(cp, r2, -1.3888889e-03f);               // -1/6!
  cp = fmaf(cp, r2, 4.1666668e-02f);                //  1/4!
  cp = fmaf(cp, r2, -0.5f);                         // -1/2!
  const float cr = fmaf(cp, r2, 1.0f);
  const int q = static_cast<int>(n) & 3;
  const float sv = (q & 1) ? cr : sr;
  const float cv = (q & 1) ? sr : cr;
  s = (q & 2) ? -sv : sv;
  c = ((q + 1) & 2) ? -cv : cv;
}

// y1 = cos*x1 - sin*x2 (first half), y2 = cos*x2 + sin*x1 (second half).
__device__ __forceinline__ void rope_pair(float c, float s, float x1, float x2, float& y1,
                                          float& y2) {
  y1 = __fsub_rn(__fmul_rn(c, x1), __fmul_rn(s, x2));
  y2 = __fadd_rn(__fmul_rn(c, x2), __fmul_rn(s, x1));
}

}  // namespace ra
