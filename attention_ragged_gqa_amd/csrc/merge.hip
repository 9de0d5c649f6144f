// Merge of split-KV partial attention states for gfx950.
//
// Each split s of a row holds the softmax-normalised output o_s over its KV
// range and that range's base-2 log-sum-exp lse_s (the state the epilogue of
// the "_kernel_common.py" page stores as m + log2(d)). Over the union of the
// ranges
//   lse = log2 sum_s 2^lse_s,   out = sum_s 2^(lse_s - lse) * o_s,
// which is the online-softmax update applied to whole ranges instead of
// tiles. Ranges without a visible key have lse_s = -inf and weight 0; a row
// with none at all gets out = 0, lse = -inf.
//
// One wave per row: lane s < num_splits reads lse_s, the weights are formed
// with wave reductions, then every lane accumulates its head_dim / 64 columns
// over the splits (each split's row is one coalesced 4*head_dim-byte read).

#include <cmath>

#include "device_common.h"
#include "ra_internal.h"

namespace ra {

namespace {

constexpr int kMergeRows = 4;   // rows (waves) per workgroup

__device__ __forceinline__ float wave_max_f(float x) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) x = fmaxf(x, __shfl_xor(x, m, 64));
  return x;
}

__device__ __forceinline__ float wave_sum_f(float x) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) x += __shfl_xor(x, m, 64);
  return x;
}

template <bool BF, int D>
__global__ __launch_bounds__(64 * kMergeRows) void merge_kernel(MergeParams p) {
  constexpr int C = D / 64;   // columns per lane
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * kMergeRows + static_cast<int>(threadIdx.x >> 6);
  if (row >= p.rows) return;   // whole wave
  const int S = p.num_splits;  // 1..64 (checked by the caller)
  const size_t rows = static_cast<size_t>(p.rows);

  const float l_s = lane < S ? p.part_lse[static_cast<size_t>(lane) * rows + row] : -INFINITY;
  const float m = wave_max_f(l_s);
  const float w_s = (m == -INFINITY) ? 0.f : exp2f(l_s - m);
  const float sum_w = wave_sum_f(w_s);
  const float inv = sum_w > 0.f ? 1.f / sum_w : 0.f;

  float acc[C];
#pragma unroll
  for (int c = 0; c < C; ++c) acc[c] = 0.f;
  for (int s = 0; s < S; ++s) {
    const float ws = __shfl(w_s, s, 64) * inv;
    if (ws == 0.f) continue;   // uniform: an empty range
    const float* src = p.part_out + (static_cast<size_t>(s) * rows + row) * D + C * lane;
    if constexpr (C == 2) {
      const float2 v = *reinterpret_cast<const float2*>(src);
      acc[0] = fmaf(ws, v.x, acc[0]);
      acc[1] = fmaf(ws, v.y, acc[1]);
    } else {
      acc[0] = fmaf(ws, src[0], acc[0]);
    }
  }
  uint16_t* dst = static_cast<uint16_t*>(p.out) + static_cast<size_t>(row) * D + C * lane;
  if constexpr (C == 2) {
    *reinterpret_cast<uint32_t*>(dst) = pack2<BF>(acc[0], acc[1]);
  } else {
    dst[0] = static_cast<uint16_t>(from_f32<BF>(acc[0]));
  }
  if (lane == 0) p.lse[row] = sum_w > 0.f ? m + log2f(sum_w) : -INFINITY;
}

}  // namespace

hipError_t launch_merge(const MergeParams& p, int is_bf16, int head_dim, hipStream_t stream) {
  if (p.rows <= 0) return hipSuccess;
  const dim3 grid(static_cast<unsigned>((p.rows + kMergeRows - 1) / kMergeRows));
  const dim3 block(64 * kMergeRows);
  if (is_bf16) {
    if (head_dim == 128) hipLaunchKernelGGL((merge_kernel<true, 128>), grid, block, 0, stream, p);
    else hipLaunchKernelGGL((merge_kernel<true, 64>), grid, block, 0, stream, p);
  } else {
    if (head_dim == 128) hipLaunchKernelGGL((merge_kernel<false, 128>), grid, block, 0, stream, p);
    else hipLaunchKernelGGL((merge_kernel<false, 64>), grid, block, 0, stream, p);
  }
  return hipGetLastError();
}

}  // namespace ra
