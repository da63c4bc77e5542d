// Combine: y[t] = sum over kept slots j of w[t][j] * y_perm[row_of[t][j]] + shared[t].
//
// Transformers & Math 17.2 equation: the shared expert's output plus the
// gate-weighted outputs of the chosen experts.  ML Interview Notes, MoELayer:
// out[tok] += weights * expert(x), then the always-on experts added unweighted.
// Transformers & Math 17.5: a dropped slot contributes nothing.
//
// One wave per token; each lane owns 16-byte column chunks.  Rows are gathered
// (no atomics) and summed in slot order in fp32, then rounded once: the result is
// deterministic.  The loads of all k slots (and the shared row) for up to 4 chunks
// are issued before any arithmetic, so a lane keeps up to 4 (k + 1) loads in
// flight; k is a template parameter for the common values.  Every byte is read
// or written once, so the loads and stores are non-temporal: with the default
// policy the read-once rows took cache space to no use, and the combine ran at
// 4.97 TB/s instead of 5.86 (qwen3 prefill shape, 121.6 vs 103.4 us).
#include "common.h"
#include "kernels.h"

namespace moe {
namespace {

__device__ __forceinline__ u32x4 ld16_nt(const void* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}
__device__ __forceinline__ void st16_nt(void* p, u32x4 v) {
  __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(p));
}

template <bool BF16>
__device__ __forceinline__ void accumulate(float* acc, const u32x4 v, float w) {
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

// KT > 0: k known at compile time; KT == 0: runtime k (any value).  With KT > 0
// the token's slot rows and weights are read once, and the slot loads of up to
// kChunksPerLane 16-byte chunks per lane are all issued before any is summed.
constexpr int kChunksPerLane = 4;

template <bool BF16, int KT, bool SHARED>
__global__ __launch_bounds__(256) void combine_kernel(const void* __restrict__ y_perm,
                                                       const int32_t* __restrict__ row_of,
                                                       const float* __restrict__ topk_w,
                                                       const void* __restrict__ shared_y, int T, int k_rt, int d,
                                                       int y_rows, void* __restrict__ y) {
  constexpr int EPC = BF16 ? 8 : 4;  // elements per 16-byte chunk
  const int k = KT > 0 ? KT : k_rt;
  const int t = __builtin_amdgcn_readfirstlane(blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6));
  if (t >= T) return;
  const int lane = threadIdx.x & 63;
  const int chunks = d / EPC;
  const int64_t rows = y_rows;
  const size_t row_bytes = (size_t)d * (BF16 ? 2 : 4);
  const char* yp = static_cast<const char*>(y_perm);
  const char* sh = static_cast<const char*>(shared_y);
  char* yt = static_cast<char*>(y) + (size_t)t * row_bytes;
  const u32x4 zero = {0u, 0u, 0u, 0u};
  if constexpr (KT > 0) {
    // A dropped slot reads row 0 (this form runs only with y_rows >= 1) and its
    // values are replaced by zeros after the load: no load sits under a branch.
    const char* src[KT];
    float w[KT];
    bool kept[KT];
#pragma unroll
    for (int j = 0; j < KT; ++j) {
      const int r = __builtin_amdgcn_readfirstlane(row_of[(size_t)t * KT + j]);
      kept[j] = r >= 0 && r < rows;
      w[j] = kept[j] ? topk_w[(size_t)t * KT + j] : 0.f;
      src[j] = yp + (size_t)(kept[j] ? r : 0) * row_bytes;
    }
    const char* shrow = SHARED ? sh + (size_t)t * row_bytes : nullptr;
    for (int c0 = lane; c0 < chunks; c0 += 64 * kChunksPerLane) {
      u32x4 v[kChunksPerLane][KT], vs[kChunksPerLane];
#pragma unroll
      for (int u = 0; u < kChunksPerLane; ++u) {
        const size_t off = (size_t)min(c0 + 64 * u, chunks - 1) * 16;  // past the end: re-read, not stored
#pragma unroll
        for (int j = 0; j < KT; ++j) v[u][j] = ld16_nt(src[j] + off);
        if (SHARED) vs[u] = ld16_nt(shrow + off);
      }
#pragma unroll
      for (int u = 0; u < kChunksPerLane; ++u) {
        const int c = c0 + 64 * u;
        float acc[EPC];
#pragma unroll
        for (int e = 0; e < EPC; ++e) acc[e] = 0.f;
#pragma unroll
        for (int j = 0; j < KT; ++j) accumulate<BF16>(acc, kept[j] ? v[u][j] : zero, w[j]);
        if (SHARED) accumulate<BF16>(acc, vs[u], 1.f);
        u32x4 o;
        if (BF16) {
#pragma unroll
          for (int q = 0; q < 4; ++q) o[q] = pack_bf16x2(acc[2 * q], acc[2 * q + 1]);
        } else {
#pragma unroll
          for (int q = 0; q < 4; ++q) o[q] = __float_as_uint(acc[q]);
        }
        if (c < chunks) st16_nt(yt + (size_t)c * 16, o);
      }
    }
  } else {
    for (int c = lane; c < chunks; c += 64) {
      float acc[EPC];
#pragma unroll
      for (int e = 0; e < EPC; ++e) acc[e] = 0.f;
      for (int j = 0; j < k; ++j) {
        const int r = row_of[(size_t)t * k + j];
        if (r < 0 || r >= rows) continue;
        accumulate<BF16>(acc, ld16_nt(yp + (size_t)r * row_bytes + (size_t)c * 16), topk_w[(size_t)t * k + j]);
      }
      if (SHARED) accumulate<BF16>(acc, ld16_nt(sh + (size_t)t * row_bytes + (size_t)c * 16), 1.f);
      u32x4 o;
      if (BF16) {
#pragma unroll
        for (int q = 0; q < 4; ++q) o[q] = pack_bf16x2(acc[2 * q], acc[2 * q + 1]);
      } else {
#pragma unroll
        for (int q = 0; q < 4; ++q) o[q] = __float_as_uint(acc[q]);
      }
      st16_nt(yt + (size_t)c * 16, o);
    }
  }
}

constexpr int kCombineOneWaveBelowT = 1024;

template <bool BF16>
hipError_t launch_dtype(const CombineArgs& a, hipStream_t stream) {
  // One wave per token; four per block, or one when there are few tokens (decode),
  // so that the tokens spread over as many CUs as there are.
  const int waves = a.T < kCombineOneWaveBelowT ? 1 : 4;
  const dim3 grid((a.T + waves - 1) / waves), block(64 * waves);
#define MOE_COMBINE(KT)                                                                                       \
  do {                                                                                                        \
    if (a.shared_y != nullptr)                                                                                \
      hipLaunchKernelGGL((combine_kernel<BF16, KT, true>), grid, block, 0, stream, a.y_perm, a.row_of,      \
                         a.topk_w, a.shared_y, a.T, a.k, a.d, a.y_rows, a.y);                                 \
    else                                                                                                      \
      hipLaunchKernelGGL((combine_kernel<BF16, KT, false>), grid, block, 0, stream, a.y_perm, a.row_of,     \
                         a.topk_w, nullptr, a.T, a.k, a.d, a.y_rows, a.y);                                    \
  } while (0)
  // The fixed-k forms read row 0 for a dropped slot; with an empty y_perm
  // (y_rows = 0: every slot dropped) the runtime-k form runs, which reads no row.
  switch (a.y_rows > 0 ? a.k : 0) {
    case 1: MOE_COMBINE(1); break;
    case 2: MOE_COMBINE(2); break;
    case 4: MOE_COMBINE(4); break;
    case 8: MOE_COMBINE(8); break;
    default: MOE_COMBINE(0); break;
  }
#undef MOE_COMBINE
  return hipGetLastError();
}

// Scatter combine (the weighted sum done by the down GEMM's epilogue, as the
// weighted scatter-add of ML Interview Notes, MoELayer and The Residual Stream,
// "An MoE tiny GPT"): before the GEMM, zero the fp32 accumulator and give each
// kept row its slot's gate weight; after it, add the shared expert and round once.
__global__ __launch_bounds__(256) void scatter_prologue_kernel(float* __restrict__ y_acc, float* __restrict__ row_w,
                                                                const int32_t* __restrict__ row_of,
                                                                const float* __restrict__ topk_w, int64_t n4,
                                                                int64_t pairs, int max_rows) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i < n4) reinterpret_cast<float4*>(y_acc)[i] = make_float4(0.f, 0.f, 0.f, 0.f);
  if (i < pairs) {
    const int r = row_of[i];
    if (r >= 0 && r < max_rows) row_w[r] = topk_w[i];
  }
}

// One 16-byte output chunk per thread: y = y_acc + shared_y, one rounding.
template <bool BF16, bool SHARED>
__global__ __launch_bounds__(256) void scatter_finish_kernel(const float* __restrict__ y_acc,
                                                              const void* __restrict__ shared_y, int64_t chunks,
                                                              void* __restrict__ y) {
  constexpr int EPC = BF16 ? 8 : 4;
  const int64_t c = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (c >= chunks) return;
  float acc[EPC];
  const u32x4 a0 = ld16_nt(y_acc + c * EPC);
#pragma unroll
  for (int q = 0; q < 4; ++q) acc[q] = __uint_as_float(a0[q]);
  if (BF16) {
    const u32x4 a1 = ld16_nt(y_acc + c * EPC + 4);
#pragma unroll
    for (int q = 0; q < 4; ++q) acc[4 + q] = __uint_as_float(a1[q]);
  }
  if (SHARED) {
    const u32x4 v = ld16_nt(static_cast<const char*>(shared_y) + c * 16);
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
    for (int q = 0; q < 4; ++q) o[q] = pack_bf16x2(acc[2 * q], acc[2 * q + 1]);
  } else {
#pragma unroll
    for (int q = 0; q < 4; ++q) o[q] = __float_as_uint(acc[q]);
  }
  st16_nt(static_cast<char*>(y) + c * 16, o);
}

}  // namespace

hipError_t launch_combine(const CombineArgs& a, hipStream_t stream) {
  return a.dtype == MOE_BF16 ? launch_dtype<true>(a, stream) : launch_dtype<false>(a, stream);
}

hipError_t launch_scatter_prologue(float* y_acc, float* row_w, const int32_t* row_of, const float* topk_w, int T,
                                   int k, int d, int max_rows, hipStream_t stream) {
  const int64_t n4 = (int64_t)T * d / 4, pairs = (int64_t)T * k;
  const int64_t n = n4 > pairs ? n4 : pairs;
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(scatter_prologue_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream, y_acc, row_w,
                     row_of, topk_w, n4, pairs, max_rows);
  return hipGetLastError();
}

hipError_t launch_scatter_finish(const float* y_acc, const void* shared_y, int dtype, int T, int d, void* y,
                                 hipStream_t stream) {
  const bool bf16 = dtype == MOE_BF16;
  const int64_t chunks = (int64_t)T * d / (bf16 ? 8 : 4);
  if (chunks <= 0) return hipSuccess;
  const dim3 grid((unsigned)((chunks + 255) / 256)), block(256);
  if (bf16) {
    if (shared_y != nullptr)
      hipLaunchKernelGGL((scatter_finish_kernel<true, true>), grid, block, 0, stream, y_acc, shared_y, chunks, y);
    else
      hipLaunchKernelGGL((scatter_finish_kernel<true, false>), grid, block, 0, stream, y_acc, nullptr, chunks, y);
  } else {
    if (shared_y != nullptr)
      hipLaunchKernelGGL((scatter_finish_kernel<false, true>), grid, block, 0, stream, y_acc, shared_y, chunks, y);
    else
      hipLaunchKernelGGL((scatter_finish_kernel<false, false>), grid, block, 0, stream, y_acc, nullptr, chunks, y);
  }
  return hipGetLastError();
}

}  // namespace moe
