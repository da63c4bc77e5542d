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
#include "dispatch_single.h"
#include "kernels.h"
#include "stats_partial.h"
#include "stats_single.h"

namespace moe {
namespace {

constexpr int kTokens = 64;   // tokens per block of the fused kernel

#ifndef MOE_ROUTE_SPLIT_MAX_T
#define MOE_ROUTE_SPLIT_MAX_T 2048
#endif
#ifndef MOE_ROUTE_GEMM
#define MOE_ROUTE_GEMM 1
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

// Row arg-max step over packed candidates: the order key in the upper 32 bits and
// the complemented expert index in the lower, so that one unsigned compare puts
// the larger key first and, between equal keys, the lower index.
template <int CTRL>
__device__ __forceinline__ void pmax_step(uint64_t& best) {
  const uint64_t o = ((uint64_t)dpp<CTRL>((uint32_t)(best >> 32)) << 32) | dpp<CTRL>((uint32_t)best);
  best = o > best ? o : best;
}

// Top-k for 4 NW PASSES tokens of a score tile (LDS, or the score rows in global
// memory).  Each pass gives every 16-lane row of the NW waves one token: tile row
// 4 NW pass + 4 wave + row.  NB keys per lane (lane r of a row holds experts
// r + 16 i); SPL result slots per lane (slot j lives in lane j % 16, register
// j / 16).  WRITE_SCORES copies the tile rows to the score output.
//
// Selection keys: the score s, or with a selection bias b, softmax(s) + b
// (softmax then top-k), s + b (top-k then softmax); sigmoid(s), or sigmoid(s) + b
// (sigmoid scoring).  k + 1 rounds of a row arg-max over (key, -index) (the
// (k+1)-th best only for the near-tie flag); a winner's key is cleared, which
// ranks it below every present key (present keys are at least 1).  The weights
// are then built once from the chosen experts' scores, read back from the tile:
//   softmax then top-k:  e = exp(s - max s), w = e / z (z: all experts), or
//                        e / (sum of the chosen e) with renorm
//   top-k then softmax:  softmax over the chosen s
//   sigmoid then top-k:  g / (sum of the chosen g), g = sigmoid(s)
// exp is the hardware exponential (v_exp_f32, about 1 ulp) and the divisions use
// the hardware reciprocal: the weights are compared to 1e-4 relative.
template <int NB, int SPL, int PASSES, bool WRITE_SCORES, int NW = 4>
__device__ void select_tile(const float* tile, int stride, int t0, int T, int E, int k, int mode, int renorm,
                            const float* __restrict__ sel_bias, float* __restrict__ logits,
                            int32_t* __restrict__ topk_idx, float* __restrict__ topk_w,
                            int32_t* __restrict__ near_tie, int32_t* __restrict__ idx_copy = nullptr) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int r = lane & 15, row = lane >> 4;
  const bool biased = sel_bias != nullptr;
  float sb[NB];
#pragma unroll
  for (int i = 0; i < NB; ++i) {
    const int e = r + 16 * i;
    sb[i] = biased ? sel_bias[min(e, E - 1)] : 0.f;
  }
  // the score output: rows t0 .. t0 + 16 PASSES - 1 that exist; a buffer store
  // past the range (dead rows, experts >= E) is dropped, so no store sits under
  // a branch
  const int live_rows = max(0, min(4 * NW * PASSES, T - t0));
  const __amdgpu_buffer_rsrc_t rl = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(WRITE_SCORES ? logits + (size_t)t0 * E : logits), (short)0,
      WRITE_SCORES ? (int)((uint32_t)live_rows * (uint32_t)E * 4u) : 0, kBufferFlags);
#pragma unroll 1
  for (int pass = 0; pass < PASSES; ++pass) {
    const int lr = pass * 4 * NW + wave * 4 + row;
    const int t = t0 + lr;
    const bool live = t < T;
    const float* s = tile + lr * stride;
    float kf[NB];
#pragma unroll
    for (int i = 0; i < NB; ++i) {
      const int e = r + 16 * i;
      const bool present = e < E;
      kf[i] = (present && live) ? s[e] : 0.f;
      if (WRITE_SCORES)
        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(kf[i]), rl,
                                              present ? (int)(((uint32_t)lr * (uint32_t)E + e) * 4u) : (int)0x80000000,
                                              0, 0);
    }
    // softmax maximum and denominator over all E (softmax scoring)
    float m = -INFINITY, z = 0.f;
    if (mode == MOE_SOFTMAX_THEN_TOPK) {
#pragma unroll
      for (int i = 0; i < NB; ++i)
        if (r + 16 * i < E) m = fmaxf(m, kf[i]);
      m = row16_max(m);
#pragma unroll
      for (int i = 0; i < NB; ++i) z += r + 16 * i < E ? __expf(kf[i] - m) : 0.f;
      z = row16_sum(z);
    }
    const float rz = __builtin_amdgcn_rcpf(z);
    uint64_t cand[NB];
#pragma unroll
    for (int i = 0; i < NB; ++i) {
      float key;
      if (mode == MOE_SOFTMAX_THEN_TOPK) key = biased ? __expf(kf[i] - m) * rz + sb[i] : kf[i];
      else if (mode == MOE_TOPK_THEN_SOFTMAX) key = biased ? kf[i] + sb[i] : kf[i];
      else {
        const float g = __builtin_amdgcn_rcpf(1.f + __expf(-kf[i]));
        key = biased ? g + sb[i] : g;
      }
      const uint32_t ko = r + 16 * i < E ? max(order_key(key), 1u) : 0u;  // 0: absent or taken
      cand[i] = ((uint64_t)ko << 32) | (uint32_t)~(uint32_t)(r + 16 * i);
    }
    const int rounds = k < E ? k + 1 : k;
    uint32_t my_idx[SPL];
#pragma unroll
    for (int q = 0; q < SPL; ++q) my_idx[q] = 0u;
    uint32_t kth = 0u, next = 0u;
    for (int j = 0; j < rounds; ++j) {
      uint64_t best = cand[0];
#pragma unroll
      for (int i = 1; i < NB; ++i) best = cand[i] > best ? cand[i] : best;
      pmax_step<kDppXor1>(best);
      pmax_step<kDppXor2>(best);
      pmax_step<kDppHalfMirror>(best);
      pmax_step<kDppMirror>(best);
      const uint32_t widx = ~(uint32_t)best, wkey = (uint32_t)(best >> 32);
      if (j < k) {
        if (j == k - 1) kth = wkey;
#pragma unroll
        for (int q = 0; q < SPL; ++q)
          if (j == r + 16 * q) my_idx[q] = widx;
#pragma unroll
        for (int i = 0; i < NB; ++i)
          if (widx == (uint32_t)(r + 16 * i)) cand[i] &= 0xffffffffull;  // taken
      } else {
        next = wkey;
      }
    }
    // weights from the chosen scores; slot j = r + 16 q
    float sv[SPL], part = 0.f, vmax = -INFINITY;
#pragma unroll
    for (int q = 0; q < SPL; ++q) {
      const bool slot = r + 16 * q < k;
      sv[q] = slot && live ? s[my_idx[q]] : 0.f;
      if (slot) vmax = fmaxf(vmax, sv[q]);
    }
    if (mode == MOE_TOPK_THEN_SOFTMAX) vmax = row16_max(vmax);
    float base[SPL];
#pragma unroll
    for (int q = 0; q < SPL; ++q) {
      const bool slot = r + 16 * q < k;
      if (mode == MOE_SOFTMAX_THEN_TOPK) base[q] = __expf(sv[q] - m);
      else if (mode == MOE_TOPK_THEN_SOFTMAX) base[q] = __expf(sv[q] - vmax);
      else base[q] = __builtin_amdgcn_rcpf(1.f + __expf(-sv[q]));
      part += slot ? base[q] : 0.f;
    }
    const bool own_sum = mode != MOE_SOFTMAX_THEN_TOPK || renorm;
    const float rden = __builtin_amdgcn_rcpf(own_sum ? row16_sum(part) : z);
    if (live) {
#pragma unroll
      for (int q = 0; q < SPL; ++q) {
        const int j = r + 16 * q;
        if (j < k) {
          topk_idx[(size_t)t * k + j] = (int32_t)my_idx[q];
          topk_w[(size_t)t * k + j] = base[q] * rden;
          if (idx_copy != nullptr) idx_copy[(t - t0) * k + j] = (int32_t)my_idx[q];
        }
      }
      if (r == 0)
        near_tie[t] = (k < E && ((double)key_value(kth) - (double)key_value(next)) < MOE_NEAR_TIE_GAP) ? 1 : 0;
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

// Scores as a GEMM with DMA-fed LDS stages, then selection, for many tokens and
// 64 < E <= 128.  Block: 8 NW tokens and every expert on NW waves (NW = 4 or 8):
// wave w multiplies experts 32 (w % 4) .. 32 (w % 4) + 31 against tokens
// 32 (w / 4) .. 32 (w / 4) + 31 (32x32x16 MFMA, router rows as the "A" operand),
// so an x byte is read from HBM once and a router row once per block.  The
// selection then runs on the same waves.
//  * NW = 8 (64 tokens, one block per CU) halves the router reads from L2, which
//    bound the loop once every CU is busy; NW = 4 (32 tokens, two blocks per CU)
//    keeps more CUs busy when T is small.
//  * Each K step of 64 loads the block's x rows and E router rows (128 bytes
//    each: whole lines) straight into LDS (buffer_load_dwordx4 ... lds writes
//    lane l's 16 bytes at M0 + 16 l), four stages deep with 64 tokens (three with
//    32); each stage is its own
//    __shared__ array, so the compiler waits only for the DMA a read needs.
//    16-byte chunk c of LDS row r sits at position c ^ ((r & 7) ^ ((r >> 3) & 1)):
//    conflict-free fragment reads.
//  * Measured (qwen3 shape, router alone, x in cache): T = 16384 24.3 us with 64
//    tokens, 26.8 with 32, 35.9 for the register-operand scores and the separate
//    selection; T = 4096 18.9 / 20.2; T = 2304 18.4 / 16.8 (36 against 72 busy CUs).
//    Four stages against three with 64 tokens: 24.9 -> 23.6 us with x in cache,
//    47.2 -> 44.7 us with x and W_r evicted first (a 512 MB write before each call);
//    five: no further gain.  A six-deep x ring beside a three-deep router ring
//    ran slower (31.4 us).
constexpr int kGemmWideMinT = 4096;  // 64-token blocks from this T on
// Loads per thread that warm the L2 with W_r before the loop (a block's share of
// the router matrix, up to kWarmLoads x 16 bytes per thread).
#ifndef MOE_ROUTE_WARM_L2
#define MOE_ROUTE_WARM_L2 1
#endif
constexpr int kWarmLoads = 2;
// ... from this grid size on, where every block's share is at most kWarmLoads loads
// per thread (at 256 blocks of 512 threads and E d = 128 x 2048 the shares cover W_r);
// smaller grids would warm only part of it, for a net loss (T = 4096: +0.5 us).
constexpr unsigned kWarmMinBlocks = 256;
// DMA stages of the 64-token form (the 32-token form, two blocks per CU, has three).
#ifndef MOE_ROUTE_GEMM_WIDE_STAGES
#define MOE_ROUTE_GEMM_WIDE_STAGES 4
#endif
__device__ __forceinline__ int route_swz(int r) { return (r & 7) ^ ((r >> 3) & 1); }
typedef __attribute__((address_space(3))) void* route_lds_t;

template <int SPL, int NW, int STG>
__global__ __launch_bounds__(64 * NW, NW == 4 ? 2 : 1) void route_gemm_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ wr, const float* __restrict__ bias,
    const float* __restrict__ sel_bias, int T, int d, int E, int k, int mode, int renorm,
    float* __restrict__ logits, int32_t* __restrict__ topk_idx, float* __restrict__ topk_w,
    int32_t* __restrict__ near_tie, int32_t* __restrict__ block_hist, float* __restrict__ stats_part) {
  static_assert(NW == 4 || NW == 8, "32 or 64 tokens a block");
  static_assert(STG == 3 || STG == 4, "DMA stages");
  constexpr int EP = 128, BK = 64, TT = 8 * NW;
  constexpr int RPW = 16 / NW;           // router DMA instructions per wave and step
  constexpr int STAGE = (TT + EP) * BK;  // bf16: TT x rows, then 128 router rows
  constexpr int TSTR = EP + 4;           // score tile stride (floats)
  __shared__ __attribute__((aligned(1024))) uint16_t s0[STAGE];
  __shared__ __attribute__((aligned(1024))) uint16_t s1[STAGE];
  __shared__ __attribute__((aligned(1024))) uint16_t s2[STAGE];
  __shared__ __attribute__((aligned(1024))) uint16_t s3[STG > 3 ? STAGE : 8];
  __shared__ __attribute__((aligned(16))) float tile[TT * TSTR];

  const int tid = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int eg = wave & 3, th = wave >> 2;
  const int t0 = blockIdx.x * TT;
  const int rows = min(TT, T - t0);
  const int nst = d / BK;
  const int nsteps = (nst + STG - 1) / STG * STG;  // padded with zero steps
  // over the block's token rows only (32-bit offsets whatever T is)
  const __amdgpu_buffer_rsrc_t rx = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(x + (size_t)t0 * d), (short)0, (int)((uint32_t)rows * (uint32_t)d * 2u), kBufferFlags);
  const __amdgpu_buffer_rsrc_t rw = __builtin_amdgcn_make_buffer_rsrc(
      (void*)wr, (short)0, (int)((uint32_t)E * (uint32_t)d * 2u), kBufferFlags);
  constexpr uint32_t kOut = 0x80000000u;  // past every resource: reads zeros

  // DMA: a step is NW x instructions (8 rows each) and 16 router instructions;
  // wave w issues x instruction w and router instructions RPW w .. RPW w + RPW - 1.
  // Lane l: row 8 j + l / 8 of instruction j, position l % 8, global chunk
  // (l % 8) ^ (l / 8) ^ (j & 1).
  const int c0 = (lane & 7) ^ (lane >> 3);
  const uint32_t xo =
      ((uint32_t)min(8 * wave + (lane >> 3), rows - 1) * (uint32_t)d + 8u * (c0 ^ (wave & 1))) * 2u;
  uint32_t wo[RPW];
#pragma unroll
  for (int u = 0; u < RPW; ++u) {
    const int j = RPW * wave + u;
    const int n = 8 * j + (lane >> 3);
    wo[u] = n < E ? ((uint32_t)n * (uint32_t)d + 8u * (c0 ^ (j & 1))) * 2u : kOut;
  }
  // step s loads K offset 64 min(s, nst - 1); the padding steps past nst read zeros
  auto dma = [&](uint16_t* st, int s) __attribute__((always_inline)) {
    const int kb = 2 * BK * min(s, nst - 1);
    const uint32_t pad = s < nst ? 0u : kOut;
    const route_lds_t xdst = (route_lds_t)(st + 8 * wave * BK);
    const uint32_t xoff = xo | pad;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rx, xdst, 16, xoff, kb, 0, 0);
#pragma unroll
    for (int u = 0; u < RPW; ++u) {
      const route_lds_t wdst = (route_lds_t)(st + (TT + 8 * (RPW * wave + u)) * BK);
      const uint32_t woff = wo[u] | pad;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rw, wdst, 16, woff, kb, 0, 0);
    }
  };
  // Fragments: lane l reads row l % 32 of a 32-row block, chunk 2 ks + l / 32.
  const int frow = lane & 31, fsw = route_swz(frow);
  f32x16 acc = f32x16{};
  auto compute = [&](const uint16_t* st) __attribute__((always_inline)) {
    bf16x8 wf[4], xf[4];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const int pos = 8 * ((2 * ks + (lane >> 5)) ^ fsw);
      wf[ks] = as_bf16x8(ld16(st + (TT + 32 * eg + frow) * BK + pos));
      xf[ks] = as_bf16x8(ld16(st + (32 * th + frow) * BK + pos));
    }
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) acc = mfma32x32x16(wf[ks], xf[ks], acc);
  };
  // Step s in stage `cur`: this wave's DMA of the stage has landed (the compiler
  // waits for it before the read below), then every wave's has and every wave
  // has finished the previous stage, which takes the DMA of step s + STG - 1.
  auto step = [&](uint16_t* cur, uint16_t* prev, int s) __attribute__((always_inline)) {
    const uint32_t probe = *reinterpret_cast<const uint32_t*>(cur + lane * 2);
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::"v"(probe) : "memory");
    dma(prev, s + STG - 1);
    compute(cur);
  };
  // Warm the L2 with W_r: the blocks of an XCD (dealt to the 8 XCDs in turn) each
  // touch their share of the router rows before the first DMA, so that the DMAs of
  // later steps hit the XCD's L2 instead of all missing at the same step (qwen3
  // prefill, in the layer: 31.8 -> 29.8 us).  The values only feed a store that
  // d > 0 rules out, which keeps the loads.
  // No branch: with a small grid the loads go past the resource (dropped, read
  // zeros), and the values are read only after the loop, so nothing waits for them.
  const bool warm = MOE_ROUTE_WARM_L2 && gridDim.x >= kWarmMinBlocks;
  const uint32_t per_xcd = (gridDim.x + 7u) / 8u;
  const uint32_t share = ((uint32_t)E * (uint32_t)d * 2u + per_xcd - 1u) / per_xcd;
  u32x4 wv[kWarmLoads];
#pragma unroll
  for (int j = 0; j < kWarmLoads; ++j) {
    const uint32_t off = (uint32_t)(j * 64 * NW + tid) * 16u;
    wv[j] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                          rw, (int)(warm && off < share ? (blockIdx.x / 8u) * share + off : kOut),
                                          0, 0));
  }
  dma(s0, 0);
  dma(s1, 1);
  if constexpr (STG == 3) {
    for (int s = 0; s < nsteps; s += 3) {
      step(s0, s2, s);
      step(s1, s0, s + 1);
      step(s2, s1, s + 2);
    }
  } else {
    dma(s2, 2);
    for (int s = 0; s < nsteps; s += 4) {
      step(s0, s3, s);
      step(s1, s0, s + 1);
      step(s2, s1, s + 2);
      step(s3, s2, s + 3);
    }
  }
  // the padding DMAs (zeros, past the last step) land before the block ends
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  uint32_t touch = 0u;
#pragma unroll
  for (int j = 0; j < kWarmLoads; ++j) touch ^= wv[j][0] ^ wv[j][1] ^ wv[j][2] ^ wv[j][3];
  if (d <= 0 && touch == 0x5a5a5a5au) logits[0] = 0.f;  // never: d > 0
  // accumulator element e of lane l: expert 32 eg + 8 (e / 4) + 4 (l / 32) + e % 4,
  // token 32 th + l % 32
#pragma unroll
  for (int e = 0; e < 16; ++e) {
    const int n = 32 * eg + 8 * (e / 4) + 4 * (lane >> 5) + (e & 3);
    const float b = (bias != nullptr && n < E) ? bias[n] : 0.f;
    tile[(32 * th + frow) * TSTR + n] = acc[e] + b;
  }
  __syncthreads();
  // With block_hist (k = 8, so the block's TT k = 512 assignments are one dispatch
  // block), the chosen experts also go to LDS and the block writes their histogram.
  // With stats_part (TT = 64 tokens, the statistics' block), the block also writes
  // its partial sums of P from the score tile, with the statistics' own code.
  __shared__ int32_t s_idx[TT * 8];
  __shared__ int32_t s_cnt[EP];
  __shared__ float s_smax[64], s_sinv[64], s_red[256];
  if (block_hist != nullptr && tid < EP) s_cnt[tid] = 0;
  select_tile<8, SPL, TT / (4 * NW), true, NW>(tile, TSTR, t0, T, E, k, mode, renorm, sel_bias, logits, topk_idx,
                                                topk_w, near_tie, block_hist != nullptr ? s_idx : nullptr);
  if (block_hist == nullptr && stats_part == nullptr) return;  // uniform
  __syncthreads();
  if (block_hist != nullptr)
    for (int i = tid; i < rows * 8; i += 64 * NW) atomicAdd(&s_cnt[s_idx[i]], 1);
  if (TT == 64 && stats_part != nullptr)  // uniform; the call holds barriers
    block_softmax_sums<64 * NW>(tile, TSTR, rows, E, s_smax, s_sinv, s_red, stats_part + (size_t)blockIdx.x * E);
  __syncthreads();
  if (block_hist != nullptr && tid < E) block_hist[(size_t)blockIdx.x * E + tid] = s_cnt[tid];
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

// Few tokens: after route_scores_split_kernel, one block of 16 waves selects for
// all T <= 64 tokens (one token per 16-lane row, one pass), then dispatches the
// T k <= 512 assignments and computes the balance statistics: three dependent
// steps without a launch between them.  The chosen experts and the counts pass
// from step to step through LDS, and the statistics' score loads are issued
// before the selection.
template <int NB, int SPL>
__global__ __launch_bounds__(1024) void route_dispatch_small_kernel(
    int T, int E, int k, int mode, int renorm, const float* __restrict__ sel_bias, const float* __restrict__ scores,
    int32_t* __restrict__ topk_idx, float* __restrict__ topk_w, int32_t* __restrict__ near_tie, int64_t cap,
    int32_t* __restrict__ counts, int32_t* __restrict__ offsets, int32_t* __restrict__ row_of,
    int32_t* __restrict__ perm_token, float alpha, float* __restrict__ f, float* __restrict__ P,
    float* __restrict__ l_aux, float* __restrict__ max_over_mean) {
  __shared__ int32_t s_idx[kSingleMaxPairs];
  __shared__ int32_t s_counts[MOE_MAX_EXPERTS];
  float sv[kSingleStatsRegs];
  stats_single_load(scores, T, E, sv);  // in flight through the selection
  select_tile<NB, SPL, 1, false, 16>(scores, E, 0, T, E, k, mode, renorm, sel_bias, nullptr, topk_idx, topk_w,
                                     near_tie, s_idx);
  lds_barrier();
  dispatch_single(s_idx, (int64_t)T * k, k, E, cap, 0, counts, offsets, row_of, perm_token, s_counts);
  lds_barrier();
  stats_single_finish(sv, T, E, s_counts, k, alpha, f, P, l_aux, max_over_mean);
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
  } else if (a.dtype == MOE_BF16 && NB == 8 && MOE_ROUTE_GEMM) {
    // 64 < E <= 128: scores as a DMA-fed GEMM, selection in the same block
    if (a.T >= kGemmWideMinT)
      hipLaunchKernelGGL((route_gemm_kernel<SPL, 8, MOE_ROUTE_GEMM_WIDE_STAGES>), dim3((a.T + 63) / 64), dim3(512), 0, stream,
                         (const uint16_t*)a.x, (const uint16_t*)a.w_router, a.bias, a.select_bias, a.T, a.d, a.E,
                         a.k, a.mode, a.renorm, a.logits, a.topk_idx, a.topk_w, a.near_tie,
                         route_writes_block_hist(a.dtype, a.T, a.E, a.k) ? a.block_hist : nullptr,
                         route_writes_block_hist(a.dtype, a.T, a.E, a.k) ? a.stats_partial : nullptr);
    else
      hipLaunchKernelGGL((route_gemm_kernel<SPL, 4, 3>), dim3((a.T + 31) / 32), dim3(256), 0, stream,
                         (const uint16_t*)a.x, (const uint16_t*)a.w_router, a.bias, a.select_bias, a.T, a.d, a.E,
                         a.k, a.mode, a.renorm, a.logits, a.topk_idx, a.topk_w, a.near_tie, nullptr, nullptr);
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

template <int NB, int SPL>
hipError_t launch_dispatch_small(const RouteDispatchArgs& d, hipStream_t stream) {
  const RouteArgs& a = d.route;
  const dim3 sgrid((a.T + kSplitTile - 1) / kSplitTile, (a.E + kSplitTile - 1) / kSplitTile);
  hipLaunchKernelGGL(route_scores_split_kernel, sgrid, dim3(kSplitWaves * 64), 0, stream, (const uint16_t*)a.x,
                     (const uint16_t*)a.w_router, a.bias, a.T, a.d, a.E, a.logits);
  hipLaunchKernelGGL((route_dispatch_small_kernel<NB, SPL>), dim3(1), dim3(1024), 0, stream, a.T, a.E, a.k, a.mode,
                     a.renorm, a.select_bias, a.logits, a.topk_idx, a.topk_w, a.near_tie, d.capacity, d.counts,
                     d.offsets, d.row_of, d.perm_token, d.alpha, d.f, d.P, d.l_aux, d.max_over_mean);
  return hipGetLastError();
}

template <int NB>
hipError_t launch_dispatch_small_nb(const RouteDispatchArgs& d, hipStream_t stream) {
  if (d.route.k <= 16) return launch_dispatch_small<NB, 1>(d, stream);
  return launch_dispatch_small<NB, NB>(d, stream);
}

template <int NB>
hipError_t launch_nb(const RouteArgs& a, hipStream_t stream) {
  // slots per lane: one when k <= 16, else NB (k <= E <= 16 NB)
  if (a.k <= 16) return launch_variant<NB, 1>(a, stream);
  return launch_variant<NB, NB>(a, stream);
}

}  // namespace

bool route_writes_block_hist(int dtype, int T, int E, int k) {
  return dtype == MOE_BF16 && MOE_ROUTE_GEMM && T > MOE_ROUTE_SPLIT_MAX_T && T >= kGemmWideMinT && E > 64 &&
         E <= 128 && k == 8 && 64 * k == kPairsPerBlock;
}

bool route_dispatch_small_fits(int dtype, int T, int k, int E) {
  return dtype == MOE_BF16 && T >= 1 && T <= kSingleStatsTokens && (int64_t)T * k <= kSingleMaxPairs &&
         T <= MOE_ROUTE_SPLIT_MAX_T && E >= 1 && E <= MOE_MAX_EXPERTS;
}

hipError_t launch_route_dispatch_small(const RouteDispatchArgs& d, hipStream_t stream) {
  const int E = d.route.E;
  if (E <= 16) return launch_dispatch_small_nb<1>(d, stream);
  if (E <= 32) return launch_dispatch_small_nb<2>(d, stream);
  if (E <= 64) return launch_dispatch_small_nb<4>(d, stream);
  if (E <= 128) return launch_dispatch_small_nb<8>(d, stream);
  return launch_dispatch_small_nb<16>(d, stream);
}

hipError_t launch_route(const RouteArgs& a, hipStream_t stream) {
  if (a.E <= 16) return launch_nb<1>(a, stream);
  if (a.E <= 32) return launch_nb<2>(a, stream);
  if (a.E <= 64) return launch_nb<4>(a, stream);
  if (a.E <= 128) return launch_nb<8>(a, stream);
  return launch_nb<16>(a, stream);
}

}  // namespace moe
