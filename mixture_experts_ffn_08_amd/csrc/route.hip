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
//    loop on 64-expert blocks (three fit on a CU) writes the scores, and the select
//    kernel above selects.
// The fused shape:
//  * Scores (bf16): a 64 x EP MFMA GEMM (16x16x32 bf16, fp32 accumulate).  Each
//    wave owns 16 tokens, whose x operands it loads straight into registers; the
//    router rows of each 64-wide k stage go through LDS (two stages), shared by
//    the 4 waves.  Loads run in a register ring 4 or 6 stages deep with no
//    branch and no drain in the loop: the kernel does little arithmetic per byte,
//    so it needs many bytes in flight (one round trip per stage cost 40% more).
//    fp32 inputs take a plain FMA loop.
//  * Selection: the fp32 score tile goes to LDS; each 16-lane row of a wave takes
//    one token (4 tokens per wave at once), lane r holding experts r + 16 i.
//    k+1 rounds of arg-max over (score, -index) with DPP butterflies inside the
//    row; the owner lane retires each winner.
#include <type_traits>

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
// Measured (router with selection, MI355X, split vs fused): E = 128, d = 2048: T = 4096 21.5
// vs 37.6 us, T = 16384 39.5 vs 41.3; E = 256, d = 7168: T = 4096 48 vs 134, T = 16384 180
// vs 146 (x read four times).
constexpr int64_t kScoreSplitMaxRowReads = 32768;

// Router-weight staging: 64 k per stage, rows padded to 72 bf16 (conflict-free
// 16-byte fragment reads); at least 32 rows so that every thread stores one
// 16-byte chunk per stage (rows past E hold zeros).  The score kernel keeps kRing
// stages of loads in flight in registers: its arithmetic per byte is low, so
// only many bytes in flight per CU hide the memory latency.
template <int NB>
struct RouteLds {
  static constexpr int EP = NB * 16;
  static constexpr int BK = 64;
  static constexpr int kRows = EP > 32 ? EP : 32;
  static constexpr int kWsStride = BK + 8;
  static constexpr int kChunksPerThread = kRows * (BK / 8) / 256;
  static constexpr int kRing = NB <= 8 ? 6 : 4;
  static constexpr int kTileStride = EP + 4;             // floats; breaks 4-row bank aliasing
  static constexpr int kTileBytes = kTokens * kTileStride * 4;
  static constexpr int kWsBytes = 2 * kRows * kWsStride * 2;  // two stages
  static constexpr int kBytes = kTileBytes > kWsBytes ? kTileBytes : kWsBytes;
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
  constexpr int R = L::kRing, CPT = L::kChunksPerThread;
  __shared__ __attribute__((aligned(16))) char smem[L::kBytes];
  uint16_t* ws = reinterpret_cast<uint16_t*>(smem);
  float* tile = reinterpret_cast<float*>(smem);

  // Blocks in XCD-contiguous order (the hardware deals them round-robin in x-major
  // order), with a token block's expert blocks next to each other: each XCD reads
  // its own run of x, each row twice through its L2 rather than from two XCDs.
  const int lb = xcd_contiguous((int)(blockIdx.x + blockIdx.y * gridDim.x), (int)(gridDim.x * gridDim.y));
  const int tb = lb / (int)gridDim.y, eb = lb % (int)gridDim.y;
  const int e0 = SELECT ? 0 : eb * L::EP;  // first expert of the block
  const int E = SELECT ? E_all : min(L::EP, E_all - e0);
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int kg = lane >> 4;
  const int t0 = tb * kTokens;
  const int rows = min(kTokens, T - t0);
  const int nst = d / L::BK;  // d % 128 == 0
  // Buffer resources over the block's token rows and its experts' router rows;
  // 32-bit lane offsets, the stage's k offset as the uniform offset.
  const __amdgpu_buffer_rsrc_t rx = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(x + (size_t)t0 * d), (short)0, (int)((uint32_t)rows * (uint32_t)d * 2u), kBufferFlags);
  const __amdgpu_buffer_rsrc_t rw = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(wr_all + (size_t)e0 * d), (short)0, (int)((uint32_t)E * (uint32_t)d * 2u), kBufferFlags);
  constexpr uint32_t kOut = 0x80000000u;  // an offset past every resource: reads zeros
  // x operand (16x16x32 MFMA "A"): token row wave 16 + lane % 16, k = 8 (lane / 16) + 32 q.
  const uint32_t xoff = ((uint32_t)min(wave * 16 + (lane & 15), rows - 1) * (uint32_t)d + 8u * kg) * 2u;
  // Router chunk i of this thread: c = tid + 256 i, row c / 8, k 8 (c % 8).
  uint32_t woff[CPT];
#pragma unroll
  for (int i = 0; i < CPT; ++i) {
    const int c = tid + 256 * i, n = c >> 3;
    woff[i] = n < E ? ((uint32_t)n * (uint32_t)d + 8u * (c & 7)) * 2u : kOut;
  }

  // Stage s into register set P.  Stages past the end (the loop runs in whole
  // rings) read x as zeros and keep the last stage's k offset (inside both buffers).
  u32x4 xr[R][2], wreg[R][CPT];
  auto load = [&](auto set, int s) {
    constexpr int P = decltype(set)::value;
    const int kb = 2 * L::BK * min(s, nst - 1);
    const uint32_t pad = s < nst ? 0u : kOut;
#pragma unroll
    for (int q = 0; q < 2; ++q)
      xr[P][q] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rx, (int)((xoff + 64u * q) | pad),
                                                                                  kb, 0));
#pragma unroll
    for (int i = 0; i < CPT; ++i)
      wreg[P][i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rw, (int)woff[i], kb, 0));
  };
  auto store_w = [&](auto set, int stage) {
    constexpr int P = decltype(set)::value;
    uint16_t* dst = ws + stage * (L::kRows * L::kWsStride);
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
      const int c = tid + 256 * i;
      st16(dst + (c >> 3) * L::kWsStride + 8 * (c & 7), wreg[P][i]);
    }
  };
  f32x4 acc[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) acc[nb] = f32x4{0.f, 0.f, 0.f, 0.f};
  auto mma = [&](auto set, int stage) {
    constexpr int P = decltype(set)::value;
    const uint16_t* cur = ws + stage * (L::kRows * L::kWsStride);
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const uint16_t* brow = cur + (nb * 16 + (lane & 15)) * L::kWsStride + 8 * kg;
#pragma unroll
      for (int q = 0; q < 2; ++q) acc[nb] = mfma16x16x32(as_bf16x8(xr[P][q]), as_bf16x8(ld16(brow + 32 * q)), acc[nb]);
    }
  };
  // Step s (register set J, LDS stage s & 1): multiply; refill set J with stage
  // s + R; store the router rows of stage s + 1 (set J + 1, loaded R - 1 steps
  // ago) to the other LDS stage; one fence-free barrier.  No branch anywhere in
  // the loop: the compiler's wait counts then leave R - 1 stages in flight.
  auto step = [&](auto set, int s) {
    constexpr int J = decltype(set)::value;
    using Next = std::integral_constant<int, (J + 1) % R>;
    mma(set, s & 1);
    load(set, s + R);
    __builtin_amdgcn_sched_barrier(0);
    store_w(Next{}, (s + 1) & 1);
    lds_barrier();
  };
  using C0 = std::integral_constant<int, 0>;
  using C1 = std::integral_constant<int, 1>;
  using C2 = std::integral_constant<int, 2>;
  using C3 = std::integral_constant<int, 3>;
  using C4 = std::integral_constant<int, 4 % R>;
  using C5 = std::integral_constant<int, 5 % R>;
  // Prologue in ring order (the loop head's wait counts merge with it).
  load(C0{}, 0);
  __builtin_amdgcn_sched_barrier(0);
  load(C1{}, 1);
  __builtin_amdgcn_sched_barrier(0);
  load(C2{}, 2);
  __builtin_amdgcn_sched_barrier(0);
  load(C3{}, 3);
  __builtin_amdgcn_sched_barrier(0);
  if constexpr (R > 4) {
    load(C4{}, 4);
    __builtin_amdgcn_sched_barrier(0);
    load(C5{}, 5);
    __builtin_amdgcn_sched_barrier(0);
  }
  store_w(C0{}, 0);
  lds_barrier();
  // nst >= 2: a do-while leaves no guard branch for the compiler to sink the
  // prologue's loads behind (which would break their ring order).
  int s0 = 0;
  do {
    step(C0{}, s0);
    step(C1{}, s0 + 1);
    step(C2{}, s0 + 2);
    step(C3{}, s0 + 3);
    if constexpr (R > 4) {
      step(C4{}, s0 + 4);
      step(C5{}, s0 + 5);
    }
    s0 += R;
  } while (s0 < nst);
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // the last ring's loads (past the end) land before exit
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
