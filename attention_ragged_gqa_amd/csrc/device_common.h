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

template <bool BF>
__device__ __forceinline__ uint32_t pack2(float lo, float hi) {
  return from_f32<BF>(lo) | (from_f32<BF>(hi) << 16);
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

// ---- rotary embedding ------------------------------------------------------
// Rotate-half RoPE of the "_kernel_common.py" page (_rope): for dims k and
// k + D/2 the angle is float32(pos * scale) * inv_freq[k] with
// inv_freq[k] = theta^(-2k/D). The angle is formed and reduced mod 2*pi in
// float64 (so positions in the thousands keep full float32 accuracy), then
// cos/sin are taken in float32. The rotated value is evaluated in float32 as
// cos*x + sin*partner (two rounded products and a rounded sum, no fused
// multiply-add) and then rounded to the storage type.
__device__ __forceinline__ void rope_cos_sin(int pos, float scale, double inv_freq, float& c,
                                             float& s) {
  const float pos_f = static_cast<float>(pos) * scale;
  const double ang = static_cast<double>(pos_f) * inv_freq;
  const double kTwoPiHi = 6.283185307179586;
  const double kTwoPiLo = 2.4492935982947064e-16;
  const double n = rint(ang * 0.15915494309189535);
  double r = fma(-n, kTwoPiHi, ang);
  r = fma(-n, kTwoPiLo, r);
  sincosf(static_cast<float>(r), &s, &c);
}

// y1 = cos*x1 - sin*x2 (first half), y2 = cos*x2 + sin*x1 (second half).
__device__ __forceinline__ void rope_pair(float c, float s, float x1, float x2, float& y1,
                                          float& y2) {
  y1 = __fsub_rn(__fmul_rn(c, x1), __fmul_rn(s, x2));
  y2 = __fadd_rn(__fmul_rn(c, x2), __fmul_rn(s, x1));
}

}  // namespace ra
