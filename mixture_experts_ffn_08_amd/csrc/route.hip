// Router: scores s = x W_r^T (+ bias), top-k selection and gate weights, with an
// optional selection-only bias (bias balancing) and sigmoid scoring.
//
// Latent "Mixture of experts", "Where the experts live": one score per expert,
// s = W_r x, and the gate equation (softmax over the chosen scores).
// The Residual Stream "Mixture of Experts: More Parameters, Same FLOPs", "The
// router": softmax over all experts, keep the k most probable, renormalize over
// them; DeepSeek-V3's sigmoid scores normalized over the chosen experts.  Same
// page, "Keeping the load even": a per-expert bias that only chooses.
// Transformers & Math 17.2: the two softmax orders.
//
// Launch shapes, chosen by T and E (bf16):
//  * many tokens: one block of 4 waves takes 64 tokens and every expert (E <= 256,
//    padded to EP = 16*NB); scores and selection in one kernel (below).
//  * few tokens (T <= MOE_ROUTE_SPLIT_MAX_T): a grid over (16 tokens, 16 experts)
//    tiles whose 8 waves each take every 8th 128-wide slice of d, summed in wave
//    order through LDS, writes the scores; a second kernel selects from them.  At
//    decode sizes this spreads the router matrix over many CUs instead of one.
//  * many tokens and E > 64 (while T ceil(E / 64) <= 32768): the fused kernel's
//    loop on 64-expert blocks (two fit on a CU) writes the scores, and the select
//    kernel above selects.
// The fused shape:
//  * Scores (bf16): a 64 x EP MFMA GEMM (16x16x32 bf16, fp32 accumulate).  Each
//    wave owns 16 tokens; router-weight chunks of 256 k-values (128 for E > 128)
//    are staged in a double-buffered LDS ring shared by the 4 waves, and the next
//    chunk (and the next x operands) are fetched into registers while the current
//    one is multiplied.  fp32 inputs take a plain FMA loop.
//  * Selection: the fp32 score tile goes to LDS; each 16-lane row of a wave takes
//    one token (4 tokens per wave at once), lane r holding experts r + 16 i.
//    k+1 rounds of arg-max over (score, -index) with DPP butterflies inside the
//    row; the owner lane retires each winner.
#include "common.h"
#include "kernels.h"

namespace moe {
namespace {

constexpr int kTokens = 64;   // tokens per block of the fused kernel

#ifndef MOE_ROUTE_SPLIT_MAX_T
#define MOE_ROUTE_SPLIT_MAX_T 2048
#endif
constexpr int kSplitWaves = 8;    // waves per block of the split score kernel
constexpr int kSplitTile = 16;    // tokens and experts per block of the split score kernel
constexpr int kSelectTokens = 16; // tokens per block of the select kernel
constexpr int kScoreSplitExperts = 64;  // experts per score block when T is large and E > 64
// Measured (router alone, MI355X): E = 128, T = 16384: 44 us split vs 50 fused; E = 256:
// T = 2048 64 vs 166, T = 16384 212 vs 183 (x, d = 7168, read four times).
constexpr int64_t kScoreSplitMaxRowReads = 32768;

// K chunk per pipeline stage: large enough that each stage keeps many bytes in
// flight (a stage round trip is latency-bound), small enough for two stages of
// router weights in LDS.
template <int NB>
struct RouteLds {
  static constexpr int EP = NB * 16;
  static constexpr int BK = EP <= 128 ? 256 : 128;
  static constexpr int kWsStride = BK + 8;               // bf16 per staged router row (16-byte pad)
  static constexpr int kTileStride = EP + 4;             // floats; breaks 4-row bank aliasing
  static constexpr int kTileBytes = kTokens * kTileStride * 4;
  static constexpr int kWsBytes = 2 * EP * kWsStride * 2;  // two stages
  static constexpr int kBytes = kTileBytes > kWsBytes ? kTileBytes : kWsBytes;
  static constexpr int kRowChunks = BK / 8;              // 16-byte chunks per router row per stage
  static constexpr int kChunks = EP * kRowChunks;
  static constexpr int kChunksPerThread = (kChunks + 255) / 256;
  static constexpr int kSteps = BK / 32;                 // MFMA k-steps per stage
};

// a beats b: larger key, or equal key and lower expert index.
__device__ __forceinline__ bool beats(uint32_t ao, uint32_t ai, uint32_t bo, uint32_t bi) {
  return ao > bo || (ao == bo && ai < bi);
}

// One butterfly step of the row arg-max; the winner's value bv travels with it.
template <int CTRL>
__device__ __forceinline__ void argmax_step(uint32_t& bo, uint32_t& bi, float& bv) {
  const uint32_t oo = dpp<CTRL>(bo), oi = dpp<CTRL>(bi);
  const float ov = __uint_as_float(dpp<CTRL>(__float_as_uint(bv)));
  if (beats(oo, oi, bo, bi)) { bo = oo; bi = oi; bv = ov; }
}

// Top-k for 16 * PASSES tokens of a score tile (LDS, or the score rows in global
// memory).  Each pass gives every 16-lane row of the 4 waves one token: tile row
// 16 pass + 4 wave + row.  NB keys per lane; SPL result slots per lane (slot j
// lives in lane j % 16, register j / 16).  WRITE_SCORES copies the tile rows to
// the score output.
//
// Each expert has a base value, which its weight is built from, and a selection
// key (the base plus the selection bias when there is one):
//   softmax then top-k:  base e = exp(s - max s); key s, or e / z + b
//   top-k then softmax:  base s;                  key s, or s + b
//   sigmoid then top-k:  base g = 1 / (1 + exp(-s)); key g, or g + b
// The arg-max carries the winner's base; the weights are then e / z (e / sum of
// the chosen e with renorm), the softmax of the chosen s (an online maximum: with
// a bias the first winner need not have the largest score), or g / sum of the
// chosen g.
template <int NB, int SPL, int PASSES, bool WRITE_SCORES>
__device__ void select_tile(const float* tile, int stride, int t0, int T, int E, int k, int mode, int renorm,
                            const float* __restrict__ sel_bias, float* __restrict__ logits,
                            int32_t* __restrict__ topk_idx, float* __restrict__ topk_w,
                            int32_t* __restrict__ near_tie) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int r = lane & 15, row = lane >> 4;
  const bool biased = sel_bias != nullptr;
  float sb[NB];
#pragma unroll
  for (int i = 0; i < NB; ++i) {
    const int e = r + 16 * i;
    sb[i] = biased ? sel_bias[min(e, E - 1)] : 0.f;
  }
#pragma unroll 1
  for (int pass = 0; pass < PASSES; ++pass) {
    const int lr = pass * 16 + wave * 4 + row;
    const int t = t0 + lr;
    const bool live = t < T;
    const float* s = tile + lr * stride;
    float kf[NB];
#pragma unroll
    for (int i = 0; i < NB; ++i) {
      const int e = r + 16 * i;
      const bool present = e < E;
      const float v = (present && live) ? s[e] : 0.f;
      kf[i] = v;
      if (WRITE_SCORES && present && live) logits[(size_t)t * E + e] = v;
    }
    // softmax maximum and denominator over all E
    float m = 0.f, z = 0.f;
    float ev[NB];
    if (mode == MOE_SOFTMAX_THEN_TOPK) {
      m = -INFINITY;
#pragma unroll
      for (int i = 0; i < NB; ++i)
        if (r + 16 * i < E) m = fmaxf(m, kf[i]);
      m = row16_max(m);
#pragma unroll
      for (int i = 0; i < NB; ++i) {
        ev[i] = r + 16 * i < E ? expf(kf[i] - m) : 0.f;
        z += ev[i];
      }
      z = row16_sum(z);
    }
    float bv[NB];
    uint32_t ko[NB];
#pragma unroll
    for (int i = 0; i < NB; ++i) {
      float base, key;
      if (mode == MOE_SOFTMAX_THEN_TOPK) {
        base = ev[i];
        key = biased ? ev[i] / z + sb[i] : kf[i];
      } else if (mode == MOE_TOPK_THEN_SOFTMAX) {
        base = kf[i];
        key = biased ? kf[i] + sb[i] : kf[i];
      } else {
        base = 1.f / (1.f + expf(-kf[i]));
        key = biased ? base + sb[i] : base;
      }
      bv[i] = base;
      ko[i] = r + 16 * i < E ? max(order_key(key), 1u) : 0u;  // 0 marks "absent or taken"
    }
    const int rounds = k < E ? k + 1 : k;
    uint32_t my_idx[SPL];
    float my_val[SPL];
#pragma unroll
    for (int q = 0; q < SPL; ++q) { my_idx[q] = 0u; my_val[q] = 0.f; }
    float kth = 0.f, next = 0.f, vsum = 0.f, vmax = 0.f;
    for (int j = 0; j < rounds; ++j) {
      uint32_t bo = 0u, bi = 0xffffffffu;
      float bval = 0.f;
#pragma unroll
      for (int i = 0; i < NB; ++i)
        if (ko[i] > bo) { bo = ko[i]; bi = r + 16 * i; bval = bv[i]; }  // strict: the lower index keeps a tie
      argmax_step<kDppXor1>(bo, bi, bval);
      argmax_step<kDppXor2>(bo, bi, bval);
      argmax_step<kDppHalfMirror>(bo, bi, bval);
      argmax_step<kDppMirror>(bo, bi, bval);
      const float wkey = key_value(bo);
      if (j < k) {
        if (j == k - 1) kth = wkey;
        if (mode == MOE_TOPK_THEN_SOFTMAX) {  // running softmax over the chosen scores
          if (j == 0) {
            vmax = bval;
            vsum = 1.f;
          } else if (bval > vmax) {
            vsum = vsum * expf(vmax - bval) + 1.f;
            vmax = bval;
          } else {
            vsum += expf(bval - vmax);
          }
        } else {
          vsum += bval;
        }
#pragma unroll
        for (int q = 0; q < SPL; ++q)
          if (j == r + 16 * q) { my_idx[q] = bi; my_val[q] = bval; }
#pragma unroll
        for (int i = 0; i < NB; ++i)
          if (bi == (uint32_t)(r + 16 * i)) ko[i] = 0u;
      } else {
        next = wkey;
      }
    }
    if (live) {
#pragma unroll
      for (int q = 0; q < SPL; ++q) {
        const int j = r + 16 * q;
        if (j < k) {
          float w;
          if (mode == MOE_SOFTMAX_THEN_TOPK) w = my_val[q] / (renorm ? vsum : z);
          else if (mode == MOE_TOPK_THEN_SOFTMAX) w = expf(my_val[q] - vmax) / vsum;
          else w = my_val[q] / vsum;
          topk_idx[(size_t)t * k + j] = (int32_t)my_idx[q];
          topk_w[(size_t)t * k + j] = w;
        }
      }
      if (r == 0) near_tie[t] = (k < E && ((double)kth - (double)next) < MOE_NEAR_TIE_GAP) ? 1 : 0;
    }
  }
}

// SELECT = false: block (i, j) scores tokens 64 i .. against experts EP j .. EP j +
// EP - 1 and writes them; route_select_kernel selects afterwards (more, smaller
// blocks: two fit on a CU).
template <int NB, int SPL, bool SELECT>
__global__ __launch_bounds__(256) void route_bf16_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ wr_all, const float* __restrict__ bias,
    const float* __restrict__ sel_bias, int T, int d, int E_all, int k, int mode, int renorm,
    float* __restrict__ logits, int32_t* __restrict__ topk_idx, float* __restrict__ topk_w,
    int32_t* __restrict__ near_tie) {
  using L = RouteLds<NB>;
  __shared__ __attribute__((aligned(16))) char smem[L::kBytes];
  uint16_t* ws = reinterpret_cast<uint16_t*>(smem);
  float* tile = reinterpret_cast<float*>(smem);

  const int e0 = SELECT ? 0 : blockIdx.y * L::EP;  // first expert of the block
  const int E = SELECT ? E_all : min(L::EP, E_all - e0);
  const uint16_t* wr = wr_all + (size_t)e0 * d;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int t0 = blockIdx.x * kTokens;
  const int kg = lane >> 4;
  const int arow = min(t0 + wave * 16 + (lane & 15), T - 1);
  const uint16_t* xrow = x + (size_t)arow * d;
  const u32x4 zero = {0u, 0u, 0u, 0u};

  // Router-weight chunk c of a stage: row n = c / kRowChunks, k offset 8 * (c % kRowChunks).
  u32x4 wreg[L::kChunksPerThread];
  auto load_w = [&](int k0) {
#pragma unroll
    for (int i = 0; i < L::kChunksPerThread; ++i) {
      const int c = tid + 256 * i;
      const int n = c / L::kRowChunks, kc = k0 + 8 * (c % L::kRowChunks);
      wreg[i] = (c < L::kChunks && n < E && kc < d) ? ld16(wr + (size_t)n * d + kc) : zero;
    }
  };
  auto store_w = [&](int stage) {
    uint16_t* dst = ws + stage * (L::EP * L::kWsStride);
#pragma unroll
    for (int i = 0; i < L::kChunksPerThread; ++i) {
      const int c = tid + 256 * i;
      if (c < L::kChunks) st16(dst + (c / L::kRowChunks) * L::kWsStride + 8 * (c % L::kRowChunks), wreg[i]);
    }
  };
  // x operand of k-step s of the stage: 8 values at k0 + 32 s + 8 kg of this lane's token.
  u32x4 areg[L::kSteps], anext[L::kSteps];
  auto load_a = [&](int k0, u32x4* dst) {
#pragma unroll
    for (int s = 0; s < L::kSteps; ++s) {
      const int ka = k0 + 32 * s + 8 * kg;
      dst[s] = ka < d ? ld16(xrow + ka) : zero;
    }
  };

  f32x4 acc[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) acc[nb] = f32x4{0.f, 0.f, 0.f, 0.f};

  load_a(0, areg);
  load_w(0);
  store_w(0);
  __syncthreads();
  int stage = 0;
  for (int k0 = 0; k0 < d; k0 += L::BK) {
    const bool more = k0 + L::BK < d;
    if (more) {
      load_a(k0 + L::BK, anext);
      load_w(k0 + L::BK);
    }
    const uint16_t* cur = ws + stage * (L::EP * L::kWsStride);
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const uint16_t* brow = cur + (nb * 16 + (lane & 15)) * L::kWsStride + 8 * kg;
#pragma unroll
      for (int s = 0; s < L::kSteps; ++s)
        acc[nb] = mfma16x16x32(as_bf16x8(areg[s]), as_bf16x8(ld16(brow + 32 * s)), acc[nb]);
    }
    if (more) {
      store_w(stage ^ 1);
#pragma unroll
      for (int s = 0; s < L::kSteps; ++s) areg[s] = anext[s];
    }
    __syncthreads();
    stage ^= 1;
  }
  if (!SELECT) {
    // accumulator element i of lane l: token 16 wave + 4 (l / 16) + i, expert nb 16 + l % 16
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const int n = nb * 16 + (lane & 15);
      if (n < E) {
        const float b = bias != nullptr ? bias[e0 + n] : 0.f;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int t = t0 + wave * 16 + 4 * kg + i;
          if (t < T) logits[(size_t)t * E_all + e0 + n] = acc[nb][i] + b;
        }
      }
    }
    return;
  }
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    const int n = nb * 16 + (lane & 15);
    const float b = (bias != nullptr && n < E) ? bias[n] : 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) tile[(wave * 16 + 4 * kg + i) * L::kTileStride + n] = acc[nb][i] + b;
  }
  __syncthreads();
  select_tile<NB, SPL, 4, true>(tile, L::kTileStride, t0, T, E, k, mode, renorm, sel_bias, logits, topk_idx,
                                topk_w, near_tie);
}

// Scores for few tokens: block (i, j) computes tokens 16 i .. 16 i + 15 against
// experts 16 j .. 16 j + 15.  MFMA 16x16x32 with operands loaded straight from
// global memory: in k-step s of a 128-wide slice of d, lane group q (lanes
// 16q .. 16q+15) holds k values 32s + 8q .. 32s + 8q + 7 of its row (the
// instruction's own order), so each load instruction reads 64 contiguous bytes of
// 16 rows.  Wave w takes slices w, w + 8, ...;
// the 8 partial tiles are added in wave order, then the bias.
__global__ __launch_bounds__(kSplitWaves * 64) void route_scores_split_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ wr, const float* __restrict__ bias, int T,
    int d, int E, float* __restrict__ logits) {
  __shared__ f32x4 red[kSplitWaves][64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int q = lane >> 4, r = lane & 15;
  const int t0 = blockIdx.x * kSplitTile, e0 = blockIdx.y * kSplitTile;
  const uint16_t* xrow = x + (size_t)min(t0 + r, T - 1) * d + 8 * q;
  const uint16_t* wrow = wr + (size_t)min(e0 + r, E - 1) * d + 8 * q;
  const int nslices = d / 128;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  for (int c0 = wave; c0 < nslices; c0 += 2 * kSplitWaves) {
    const int c1 = c0 + kSplitWaves;
    const bool two = c1 < nslices;  // uniform over the wave
    const int c1c = two ? c1 : c0;
    u32x4 a0[4], b0[4], a1[4], b1[4];
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      a0[s] = ld16(xrow + c0 * 128 + 32 * s);
      b0[s] = ld16(wrow + c0 * 128 + 32 * s);
      a1[s] = ld16(xrow + c1c * 128 + 32 * s);
      b1[s] = ld16(wrow + c1c * 128 + 32 * s);
    }
#pragma unroll
    for (int s = 0; s < 4; ++s) acc = mfma16x16x32(as_bf16x8(a0[s]), as_bf16x8(b0[s]), acc);
    if (two) {
#pragma unroll
      for (int s = 0; s < 4; ++s) acc = mfma16x16x32(as_bf16x8(a1[s]), as_bf16x8(b1[s]), acc);
    }
  }
  red[wave][lane] = acc;
  __syncthreads();
  if (wave == 0) {
    f32x4 sum = red[0][lane];
#pragma unroll
    for (int w = 1; w < kSplitWaves; ++w) sum += red[w][lane];
    // accumulator element i: token 4q + i of the tile, expert r
    const int e = e0 + r;
    if (e < E) {
      const float b = bias != nullptr ? bias[e] : 0.f;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int t = t0 + 4 * q + i;
        if (t < T) logits[(size_t)t * E + e] = sum[i] + b;
      }
    }
  }
}

// Selection from the score rows written by route_scores_split_kernel.
template <int NB, int SPL>
__global__ __launch_bounds__(256) void route_select_kernel(int T, int E, int k, int mode, int renorm,
                                                           const float* __restrict__ sel_bias,
                                                           const float* __restrict__ scores,
                                                           int32_t* __restrict__ topk_idx,
                                                           float* __restrict__ topk_w,
                                                           int32_t* __restrict__ near_tie) {
  const int t0 = blockIdx.x * kSelectTokens;
  select_tile<NB, SPL, kSelectTokens / 16, false>(scores + (size_t)t0 * E, E, t0, T, E, k, mode, renorm, sel_bias,
                                                  nullptr, topk_idx, topk_w, near_tie);
}

template <int NB, int SPL>
__global__ __launch_bounds__(256) void route_f32_kernel(
    const float* __restrict__ x, const float* __restrict__ wr, const float* __restrict__ bias,
    const float* __restrict__ sel_bias, int T, int d, int E, int k, int mode, int renorm,
    float* __restrict__ logits, int32_t* __restrict__ topk_idx,
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
  select_tile<NB, SPL, 4, true>(tile, L::kTileStride, t0, T, E, k, mode, renorm, sel_bias, logits, topk_idx,
                                topk_w, near_tie);
}

template <int NB, int SPL>
hipError_t launch_variant(const RouteArgs& a, hipStream_t stream) {
  const dim3 grid((a.T + kTokens - 1) / kTokens), block(256);
  if (a.dtype == MOE_BF16 && a.T <= MOE_ROUTE_SPLIT_MAX_T) {
    const dim3 sgrid((a.T + kSplitTile - 1) / kSplitTile, (a.E + kSplitTile - 1) / kSplitTile);
    hipLaunchKernelGGL(route_scores_split_kernel, sgrid, dim3(kSplitWaves * 64), 0, stream,
                       (const uint16_t*)a.x, (const uint16_t*)a.w_router, a.bias, a.T, a.d, a.E, a.logits);
    hipLaunchKernelGGL((route_select_kernel<NB, SPL>), dim3((a.T + kSelectTokens - 1) / kSelectTokens), block, 0,
                       stream, a.T, a.E, a.k, a.mode, a.renorm, a.select_bias, a.logits, a.topk_idx, a.topk_w,
                       a.near_tie);
  } else if (a.dtype == MOE_BF16 && a.E > kScoreSplitExperts &&
             (int64_t)a.T * ((a.E + kScoreSplitExperts - 1) / kScoreSplitExperts) <= kScoreSplitMaxRowReads) {
    // many experts: 64-expert score blocks (two per CU), then selection; each block
    // group re-reads x, so this stops paying once T x (E / 64) grows large
    const dim3 sgrid((a.T + kTokens - 1) / kTokens, (a.E + kScoreSplitExperts - 1) / kScoreSplitExperts);
    hipLaunchKernelGGL((route_bf16_kernel<kScoreSplitExperts / 16, 1, false>), sgrid, block, 0, stream,
                       (const uint16_t*)a.x, (const uint16_t*)a.w_router, a.bias, nullptr, a.T, a.d, a.E, a.k,
                       a.mode, a.renorm, a.logits, nullptr, nullptr, nullptr);
    hipLaunchKernelGGL((route_select_kernel<NB, SPL>), dim3((a.T + kSelectTokens - 1) / kSelectTokens), block, 0,
                       stream, a.T, a.E, a.k, a.mode, a.renorm, a.select_bias, a.logits, a.topk_idx, a.topk_w,
                       a.near_tie);
  } else if (a.dtype == MOE_BF16)
    hipLaunchKernelGGL((route_bf16_kernel<NB, SPL, true>), grid, block, 0, stream, (const uint16_t*)a.x,
                       (const uint16_t*)a.w_router, a.bias, a.select_bias, a.T, a.d, a.E, a.k, a.mode, a.renorm,
                       a.logits, a.topk_idx, a.topk_w, a.near_tie);
  else
    hipLaunchKernelGGL((route_f32_kernel<NB, SPL>), grid, block, 0, stream, (const float*)a.x,
                       (const float*)a.w_router, a.bias, a.select_bias, a.T, a.d, a.E, a.k, a.mode, a.renorm,
                       a.logits, a.topk_idx, a.topk_w, a.near_tie);
  return hipGetLastError();
}

template <int NB>
hipError_t launch_nb(const RouteArgs& a, hipStream_t stream) {
  // slots per lane: one when k <= 16, else NB (k <= E <= 16 NB)
  if (a.k <= 16) return launch_variant<NB, 1>(a, stream);
  return launch_variant<NB, NB>(a, stream);
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
