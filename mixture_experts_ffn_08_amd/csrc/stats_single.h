// Balance statistics of at most 64 tokens in one block of 16 waves: f, P, L_aux
// and max/mean, as the multi-block kernels compute them (no atomics).
//
// Transformers & Math 17.4 equation; The Residual Stream "Keeping the load even"
// and its MoE listing (f = counts / counts.sum(), P = mean softmax probability);
// Understanding Data "Load imbalance".
#pragma once

#include "../../include/moe.h"
#include "common.h"

namespace moe {

constexpr int kSingleStatsTokens = 64;

constexpr int kSingleStatsRegs = MOE_MAX_EXPERTS / 16;  // score registers per lane

// Each 16-lane row takes one token (lane r holds experts r + 16 i): the loads of
// its scores, issued on their own so that a caller can have them in flight while
// it does other work.  Called by every thread of a block of exactly 1024 threads.
__device__ inline void stats_single_load(const float* __restrict__ logits, int T, int E,
                                         float (&v)[kSingleStatsRegs]) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int r = lane & 15, t = wave * 4 + (lane >> 4);
  const float* row = logits + (size_t)min(t, T - 1) * E;
#pragma unroll
  for (int i = 0; i < kSingleStatsRegs; ++i) v[i] = row[min(r + 16 * i, E - 1)];  // clamped, no branch
}

// The token's softmax goes to LDS, and thread e sums column e over the tokens in
// token order.  f, P, L_aux and max/mean follow, with the two block-wide
// reductions done by wave shuffles (fixed tree) and one LDS step.  The block's
// threads exchange data through LDS only, so the barriers wait for LDS
// operations, not for the block's global stores.  counts may be in LDS.
// T <= 64.
__device__ inline void stats_single_finish(float (&v)[kSingleStatsRegs], int T, int E,
                                           const int32_t* __restrict__ counts, int k, float alpha,
                                           float* __restrict__ f, float* __restrict__ P, float* __restrict__ l_aux,
                                           float* __restrict__ max_over_mean) {
  constexpr int NB = kSingleStatsRegs;
  constexpr int S = MOE_MAX_EXPERTS + 1;  // LDS row stride (floats)
  __shared__ float prob[kSingleStatsTokens * S];
  __shared__ double w_fp[16];
  __shared__ int w_max[16];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int r = lane & 15, t = wave * 4 + (lane >> 4);
  const bool live = t < T;
  float m = -INFINITY;
#pragma unroll
  for (int i = 0; i < NB; ++i)
    if (r + 16 * i < E) m = fmaxf(m, v[i]);
  m = row16_max(m);
  float z = 0.f;
#pragma unroll
  for (int i = 0; i < NB; ++i) {
    v[i] = r + 16 * i < E ? __expf(v[i] - m) : 0.f;
    z += v[i];
  }
  const float inv = 1.f / row16_sum(z);
#pragma unroll
  for (int i = 0; i < NB; ++i)
    if (r + 16 * i < E) prob[t * S + r + 16 * i] = live ? v[i] * inv : 0.f;
  lds_barrier();
  const float tk = (float)((int64_t)T * k);
  double fp = 0.0;
  int c = 0;
  if (tid < E) {
    float acc = 0.f;
    // in token order; unrolled so that the LDS reads go out ahead of the adds
#pragma unroll 16
    for (int u = 0; u < T; ++u) acc += prob[u * S + tid];
    const float p = (float)((double)acc / (double)T);
    c = counts[tid];
    const float fi = (float)c / tk;
    f[tid] = fi;
    P[tid] = p;
    fp = (double)fi * (double)p;
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    fp += __shfl_xor(fp, o, 64);
    c = max(c, __shfl_xor(c, o, 64));
  }
  if (lane == 0) {
    w_fp[wave] = fp;
    w_max[wave] = c;
  }
  lds_barrier();
  if (tid == 0) {
    double sum = 0.0;
    int cmax = 0;
    for (int w = 0; w < 16; ++w) {
      sum += w_fp[w];
      cmax = max(cmax, w_max[w]);
    }
    *l_aux = (float)((double)alpha * (double)E * sum);
    *max_over_mean = (float)((int64_t)E * cmax) / tk;
  }
}

// Both parts in a row.
__device__ inline void stats_single(const float* __restrict__ logits, int T, int E, const int32_t* __restrict__ counts,
                                    int k, float alpha, float* __restrict__ f, float* __restrict__ P,
                                    float* __restrict__ l_aux, float* __restrict__ max_over_mean) {
  float v[kSingleStatsRegs];
  stats_single_load(logits, T, E, v);
  stats_single_finish(v, T, E, counts, k, alpha, f, P, l_aux, max_over_mean);
}

}  // namespace moe
