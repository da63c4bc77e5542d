// Combine: y[t] = sum over kept slots j of w[t][j] * y_perm[row_of[t][j]] + shared[t].
//
// Transformers & Math 17.2 equation: the shared expert's output plus the
// gate-weighted outputs of the chosen experts.  ML Interview Notes, MoELayer:
// out[tok] += weights * expert(x), then the always-on experts added unweighted.
// Transformers & Math 17.5: a dropped slot contributes nothing.
//
// One wave per token; each lane owns 16-byte column chunks.  Rows are gathered
// (no atomics), summed in slot order in fp32 and rounded once, so the result is
// deterministic.
#include "common.h"
#include "kernels.h"

namespace moe {
namespace {

template <bool BF16>
__global__ __launch_bounds__(256) void combine_kernel(const void* __restrict__ y_perm,
                                                       const int32_t* __restrict__ row_of,
                                                       const float* __restrict__ topk_w,
                                                       const void* __restrict__ shared_y, int T, int k, int d,
                                                       void* __restrict__ y) {
  constexpr int EPC = BF16 ? 8 : 4;  // elements per 16-byte chunk
  const int t = __builtin_amdgcn_readfirstlane(blockIdx.x * 4 + (threadIdx.x >> 6));
  if (t >= T) return;
  const int lane = threadIdx.x & 63;
  const int chunks = d / EPC;
  const int64_t rows = (int64_t)T * k;
  const size_t row_bytes = (size_t)d * (BF16 ? 2 : 4);
  const char* yp = static_cast<const char*>(y_perm);
  for (int c = lane; c < chunks; c += 64) {
    float acc[EPC];
#pragma unroll
    for (int e = 0; e < EPC; ++e) acc[e] = 0.f;
    for (int j = 0; j < k; ++j) {
      const int r = row_of[(size_t)t * k + j];
      if (r < 0 || r >= rows) continue;
      const float w = topk_w[(size_t)t * k + j];
      const u32x4 v = ld16(yp + (size_t)r * row_bytes + (size_t)c * 16);
      if (BF16) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          acc[2 * q] = fmaf(w, __uint_as_float(v[q] << 16), acc[2 * q]);
          acc[2 * q + 1] = fmaf(w, __uint_as_float(v[q] & 0xffff0000u), acc[2 * q + 1]);
        }
      } else {
#pragma unroll
        for (int q = 0; q < 4; ++q) acc[q] = fmaf(w, __uint_as_float(v[q]), acc[q]);
      }
    }
    if (shared_y != nullptr) {
      const u32x4 v = ld16(static_cast<const char*>(shared_y) + (size_t)t * row_bytes + (size_t)c * 16);
      if (BF16) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          acc[2 * q] += __uint_as_float(v[q] << 16);
          acc[2 * q + 1] += __uint_as_float(v[q] & 0xffff0000u);
        }
      } else {
#pragma unroll
        for (int q = 0; q < 4; ++q) acc[q] += __uint_as_float(v[q]);
      }
    }
    u32x4 o;
    if (BF16) {
#pragma unroll
      for (int q = 0; q < 4; ++q)
        o[q] = (uint32_t)f32_to_bf16(acc[2 * q]) | ((uint32_t)f32_to_bf16(acc[2 * q + 1]) << 16);
    } else {
#pragma unroll
      for (int q = 0; q < 4; ++q) o[q] = __float_as_uint(acc[q]);
    }
    st16(static_cast<char*>(y) + (size_t)t * row_bytes + (size_t)c * 16, o);
  }
}

}  // namespace

hipError_t launch_combine(const CombineArgs& a, hipStream_t stream) {
  const dim3 grid((a.T + 3) / 4), block(256);
  if (a.dtype == MOE_BF16)
    hipLaunchKernelGGL(combine_kernel<true>, grid, block, 0, stream, a.y_perm, a.row_of, a.topk_w, a.shared_y,
                       a.T, a.k, a.d, a.y);
  else
    hipLaunchKernelGGL(combine_kernel<false>, grid, block, 0, stream, a.y_perm, a.row_of, a.topk_w,
                       a.shared_y, a.T, a.k, a.d, a.y);
  return hipGetLastError();
}

}  // namespace moe
