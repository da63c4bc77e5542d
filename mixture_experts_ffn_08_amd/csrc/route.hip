// Router: scores s = x W_r^T (+ bias), top-k selection and gate weights.
//
// Latent "Mixture of experts", "Where the experts live": one score per expert,
// s = W_r x, and the gate equation (softmax over the chosen scores).
// The Residual Stream "Mixture of Experts: More Parameters, Same FLOPs", "The
// router": softmax over all experts, keep the k most probable, renormalize over
// them.  Transformers & Math 17.2: the two softmax orders.
//
// One block of 4 waves takes 64 tokens and every expert (E <= 256, padded to
// EP = 16*NB).  bf16: the score tile is a 64 x EP MFMA GEMM (16x16x32 bf16, fp32
// accumulate); router weight chunks of 64 k-values are staged in LDS and shared
// by the 4 waves, x rows stream straight from HBM into MFMA operands.  The fp32
// tile goes to LDS, then each wave selects top-k for its 16 tokens with
// ds_swizzle butterflies and writes scores, indices, weights and near-tie flags.
#include "common.h"
#include "kernels.h"

namespace moe {
namespace {

constexpr int kTokens = 64;   // tokens per block
constexpr int kWsStride = 72; // bf16 elements per staged router row: 64 + 8 pad

template <int NB>
struct RouteLds {
  static constexpr int EP = NB * 16;
  static constexpr int kTileStride = EP + 4;  // floats; breaks 4-row bank aliasing
  static constexpr int kTileBytes = kTokens * kTileStride * 4;
  static constexpr int kWsBytes = EP * kWsStride * 2;
  static constexpr int kBytes = kTileBytes > kWsBytes ? kTileBytes : kWsBytes;
};

// a beats b: larger key, or equal key and lower expert index.
__device__ __forceinline__ bool beats(uint32_t ao, uint32_t ai, uint32_t bo, uint32_t bi) {
  return ao > bo || (ao == bo && ai < bi);
}

template <int X>
__device__ __forceinline__ void argmax_step(uint32_t& bo, uint32_t& bi) {
  uint32_t oo = swz_xor<X>(bo), oi = swz_xor<X>(bi);
  if (beats(oo, oi, bo, bi)) { bo = oo; bi = oi; }
}

// Top-k for rows [lr0, lr0 + nrows) of the score tile; executed by one wave.
__device__ void select_rows(const float* tile, int stride, int t0, int lr0, int nrows, int T, int E,
                            int k, int mode, int renorm, float* __restrict__ logits,
                            int32_t* __restrict__ topk_idx, float* __restrict__ topk_w,
                            int32_t* __restrict__ near_tie) {
  const int lane = threadIdx.x & 63;
  for (int lr = lr0; lr < lr0 + nrows; ++lr) {
    const int t = t0 + lr;
    if (t >= T) break;
    const float* s = tile + lr * stride;
    float kf[4];
    uint32_t ko[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int e = lane + 64 * i;
      const bool present = e < E;
      const float v = present ? s[e] : 0.f;
      kf[i] = v;
      ko[i] = present ? max(order_key(v), 1u) : 0u;  // 0 marks "absent or taken"
      if (present) logits[(size_t)t * E + e] = v;
    }
    const int rounds = k < E ? k + 1 : k;
    uint32_t my_idx[4] = {0, 0, 0, 0};
    float my_key[4] = {0.f, 0.f, 0.f, 0.f};
    float top = 0.f, kth = 0.f, next = 0.f;
    for (int r = 0; r < rounds; ++r) {
      uint32_t bo = 0u, bi = 0xffffffffu;
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (ko[i] > bo) { bo = ko[i]; bi = lane + 64 * i; }  // strict: lower index keeps ties
      argmax_step<1>(bo, bi);
      argmax_step<2>(bo, bi);
      argmax_step<4>(bo, bi);
      argmax_step<8>(bo, bi);
      argmax_step<16>(bo, bi);
      const uint32_t o0 = __builtin_amdgcn_readlane(bo, 0), i0 = __builtin_amdgcn_readlane(bi, 0);
      const uint32_t o1 = __builtin_amdgcn_readlane(bo, 32), i1 = __builtin_amdgcn_readlane(bi, 32);
      const uint32_t wi = beats(o1, i1, o0, i0) ? i1 : i0;
      const float wkey = s[wi];
      if (r == 0) top = wkey;
      if (r < k) {
        if (r == k - 1) kth = wkey;
#pragma unroll
        for (int q = 0; q < 4; ++q)
          if (r == lane + 64 * q) { my_idx[q] = wi; my_key[q] = wkey; }
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (wi == (uint32_t)(lane + 64 * i)) ko[i] = 0u;
      } else {
        next = wkey;
      }
    }
    // Softmax pieces, relative to the best score.
    float z = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (lane + 64 * i < E) z += expf(kf[i] - top);
    float ej[4], esum = 0.f;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      ej[q] = (lane + 64 * q < k) ? expf(my_key[q] - top) : 0.f;
      esum += ej[q];
    }
    const float Z = wave_sum(z);
    const float S = wave_sum(esum);
    const float denom = (mode == MOE_TOPK_THEN_SOFTMAX || renorm) ? S : Z;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int j = lane + 64 * q;
      if (j < k) {
        topk_idx[(size_t)t * k + j] = (int32_t)my_idx[q];
        topk_w[(size_t)t * k + j] = ej[q] / denom;
      }
    }
    if (lane == 0)
      near_tie[t] = (k < E && ((double)kth - (double)next) < MOE_NEAR_TIE_GAP) ? 1 : 0;
  }
}

template <int NB>
__global__ __launch_bounds__(256) void route_bf16_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ wr, const float* __restrict__ bias,
    int T, int d, int E, int k, int mode, int renorm, float* __restrict__ logits,
    int32_t* __restrict__ topk_idx, float* __restrict__ topk_w, int32_t* __restrict__ near_tie) {
  using L = RouteLds<NB>;
  __shared__ __attribute__((aligned(16))) char smem[L::kBytes];
  uint16_t* ws = reinterpret_cast<uint16_t*>(smem);
  float* tile = reinterpret_cast<float*>(smem);

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int t0 = blockIdx.x * kTokens;
  const int kg = lane >> 4;
  const int arow = min(t0 + wave * 16 + (lane & 15), T - 1);
  const uint16_t* xrow = x + (size_t)arow * d;

  f32x4 acc[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) acc[nb] = f32x4{0.f, 0.f, 0.f, 0.f};

  for (int k0 = 0; k0 < d; k0 += 64) {
    const int ka = k0 + 8 * kg, kb = k0 + 32 + 8 * kg;
    const u32x4 zero = {0u, 0u, 0u, 0u};
    const u32x4 a0 = ka < d ? ld16(xrow + ka) : zero;
    const u32x4 a1 = kb < d ? ld16(xrow + kb) : zero;
    __syncthreads();
    for (int c = tid; c < L::EP * 8; c += 256) {
      const int n = c >> 3, kc = k0 + 8 * (c & 7);
      u32x4 v = zero;
      if (n < E && kc < d) v = ld16(wr + (size_t)n * d + kc);
      st16(ws + n * kWsStride + 8 * (c & 7), v);
    }
    __syncthreads();
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const uint16_t* brow = ws + (nb * 16 + (lane & 15)) * kWsStride + 8 * kg;
      acc[nb] = mfma16x16x32(as_bf16x8(a0), as_bf16x8(ld16(brow)), acc[nb]);
      acc[nb] = mfma16x16x32(as_bf16x8(a1), as_bf16x8(ld16(brow + 32)), acc[nb]);
    }
  }
  __syncthreads();
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    const int n = nb * 16 + (lane & 15);
    const float b = (bias != nullptr && n < E) ? bias[n] : 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) tile[(wave * 16 + 4 * kg + i) * L::kTileStride + n] = acc[nb][i] + b;
  }
  __syncthreads();
  select_rows(tile, L::kTileStride, t0, wave * 16, 16, T, E, k, mode, renorm, logits, topk_idx, topk_w,
              near_tie);
}

template <int NB>
__global__ __launch_bounds__(256) void route_f32_kernel(
    const float* __restrict__ x, const float* __restrict__ wr, const float* __restrict__ bias, int T,
    int d, int E, int k, int mode, int renorm, float* __restrict__ logits, int32_t* __restrict__ topk_idx,
    float* __restrict__ topk_w, int32_t* __restrict__ near_tie) {
  using L = RouteLds<NB>;
  __shared__ __attribute__((aligned(16))) float tile[kTokens * L::kTileStride];
  const int tid = threadIdx.x;
  const int t0 = blockIdx.x * kTokens;
  for (int p = tid; p < kTokens * L::EP; p += 256) {
    const int lr = p / L::EP, n = p % L::EP;
    const int t = min(t0 + lr, T - 1);
    float acc = 0.f;
    if (n < E) {
      const float* xr = x + (size_t)t * d;
      const float* wrow = wr + (size_t)n * d;
      for (int i = 0; i < d; ++i) acc = fmaf(xr[i], wrow[i], acc);
      if (bias != nullptr) acc += bias[n];
    }
    tile[lr * L::kTileStride + n] = acc;
  }
  __syncthreads();
  const int wave = tid >> 6;
  select_rows(tile, L::kTileStride, t0, wave * 16, 16, T, E, k, mode, renorm, logits, topk_idx, topk_w,
              near_tie);
}

template <int NB>
hipError_t launch_nb(const RouteArgs& a, hipStream_t stream) {
  const dim3 grid((a.T + kTokens - 1) / kTokens), block(256);
  if (a.dtype == MOE_BF16)
    hipLaunchKernelGGL(route_bf16_kernel<NB>, grid, block, 0, stream, (const uint16_t*)a.x,
                       (const uint16_t*)a.w_router, a.bias, a.T, a.d, a.E, a.k, a.mode, a.renorm,
                       a.logits, a.topk_idx, a.topk_w, a.near_tie);
  else
    hipLaunchKernelGGL(route_f32_kernel<NB>, grid, block, 0, stream, (const float*)a.x,
                       (const float*)a.w_router, a.bias, a.T, a.d, a.E, a.k, a.mode, a.renorm, a.logits,
                       a.topk_idx, a.topk_w, a.near_tie);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_route(const RouteArgs& a, hipStream_t stream) {
  if (a.E <= 16) return launch_nb<1>(a, stream);
  if (a.E <= 32) return launch_nb<2>(a, stream);
  if (a.E <= 64) return launch_nb<4>(a, stream);
  if (a.E <= 128) return launch_nb<8>(a, stream);
  return launch_nb<16>(a, stream);
}

}  // namespace moe
