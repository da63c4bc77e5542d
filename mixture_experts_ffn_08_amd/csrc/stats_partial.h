// The balance statistics in blocks (Transformers & Math 17.4; The Residual Stream,
// "Keeping the load even"): per-block partial sums of P for a block of nt <= 64
// tokens whose scores sit in LDS (sum over the block's tokens of softmax(scores)[e],
// for every expert e), and the final reduction of those rows into f, P, L_aux and
// max/mean.  One definition for every kernel that runs them, so that the results
// are the same bits whichever kernel did.
#pragma once

#include "../../include/moe.h"
#include "common.h"

namespace moe {

// Thread groups for the per-expert sums: G = 256 / E groups of E threads (one group
// when E > 128); group g takes every G-th token, and the G partial sums are added in
// group order.
__device__ __forceinline__ int expert_groups(int E) { return E > 128 ? 1 : 256 / E; }

// Called by every thread of a block of NTHREADS >= 256 threads (a multiple of 64).
// tile: the block's scores, row lt (token) at tile + lt * stride, experts 0..E-1.
// s_max, s_inv: LDS [64]; red: LDS [256]; out: E floats (global).  The
// exponentials use the hardware exp2 (relative error about 1e-6, far inside what
// P is compared to).
template <int NTHREADS>
__device__ inline void block_softmax_sums(const float* tile, int stride, int nt, int E, float* s_max, float* s_inv,
                                          float* red, float* __restrict__ out) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int r = lane & 15;
  // softmax normalizers, one token per 16-lane row
  for (int lt = wave * 4 + (lane >> 4); lt < 64; lt += NTHREADS / 16) {
    float m = -INFINITY;
    if (lt < nt)
      for (int e = r; e < E; e += 16) m = fmaxf(m, tile[lt * stride + e]);
    m = row16_max(m);
    float z = 0.f;
    if (lt < nt)
      for (int e = r; e < E; e += 16) z += __expf(tile[lt * stride + e] - m);
    z = row16_sum(z);
    if (r == 0 && lt < nt) {
      s_max[lt] = m;
      s_inv[lt] = 1.f / z;
    }
  }
  __syncthreads();
  const int G = expert_groups(E);
  const int g = tid / E, e = tid % E;
  if (tid < 256 && g < G) {
    float part = 0.f;
#pragma unroll 4
    for (int lt = g; lt < nt; lt += G) part += __expf(tile[lt * stride + e] - s_max[lt]) * s_inv[lt];
    red[tid] = part;
  }
  __syncthreads();
  if (tid < E) {
    float acc = red[tid];
    for (int q = 1; q < G; ++q) acc += red[q * E + tid];
    out[tid] = acc;
  }
}

// Block-wide finish: thread e < E holds sum_t softmax(s_t)_e in fp64.  Writes f, P,
// L_aux = alpha E sum_e f_e P_e and max/mean = E max_e counts_e / (T k).  Called by
// every thread of a block of at least 256 threads.
__device__ inline void finish_stats(double sum, const int32_t* __restrict__ counts, int T, int k, int E, float alpha,
                             float* __restrict__ f, float* __restrict__ P, float* __restrict__ l_aux,
                             float* __restrict__ max_over_mean) {
  __shared__ double s_fp[256];
  __shared__ int s_max[256];
  const int e = threadIdx.x;
  const float tk = (float)((int64_t)T * k);
  double fp = 0.0;
  int c = 0;
  if (e < E) {
    const float p = (float)(sum / (double)T);
    c = counts[e];
    const float fi = (float)c / tk;
    f[e] = fi;
    P[e] = p;
    fp = (double)fi * (double)p;
  }
  if (e < 256) {  // every thread of the block reaches the barriers below
    s_fp[e] = fp;
    s_max[e] = c;
  }
  __syncthreads();
  for (int h = 128; h > 0; h >>= 1) {
    if (e < h) {
      s_fp[e] += s_fp[e + h];
      s_max[e] = max(s_max[e], s_max[e + h]);
    }
    __syncthreads();
  }
  if (e == 0) {
    *l_aux = (float)((double)alpha * (double)E * s_fp[0]);
    *max_over_mean = (float)((int64_t)E * s_max[0]) / tk;
  }
}

constexpr int kStatsFinalThreads = 512;
constexpr int kFinalBatch = 32;  // partial rows in flight per thread

// The final reduction, by every thread of a block of NTHREADS >= 256 threads:
// thread (g, e) sums partial[b][e] over blocks b = g, g + G, ... (G = NTHREADS / E)
// in fp64, kFinalBatch loads in flight (indices clamped, out-of-range terms zeroed, no
// branch around a load); the group sums are added in group order.  Then f, P,
// L_aux and max/mean (counts may be in LDS).  No atomics: deterministic.
template <int NTHREADS>
__device__ inline void stats_final_block(const int32_t* __restrict__ counts, const float* __restrict__ partial,
                                         int nblk, int T, int k, int E, float alpha, float* __restrict__ f,
                                         float* __restrict__ P, float* __restrict__ l_aux,
                                         float* __restrict__ max_over_mean) {
  __shared__ double s_part[NTHREADS];
  const int tid = threadIdx.x;
  const int G = NTHREADS / E;
  const int g = tid / E, ge = tid % E;
  if (g < G) {
    double part[kFinalBatch];
#pragma unroll
    for (int q = 0; q < kFinalBatch; ++q) part[q] = 0.0;
    for (int b0 = g; b0 < nblk; b0 += kFinalBatch * G) {
      float pv[kFinalBatch];
#pragma unroll
      for (int q = 0; q < kFinalBatch; ++q) pv[q] = partial[(size_t)min(b0 + q * G, nblk - 1) * E + ge];
#pragma unroll
      for (int q = 0; q < kFinalBatch; ++q) part[q] += b0 + q * G < nblk ? (double)pv[q] : 0.0;
    }
    double sum = 0.0;
#pragma unroll
    for (int q = 0; q < kFinalBatch; ++q) sum += part[q];
    s_part[tid] = sum;
  }
  __syncthreads();
  double sum = 0.0;
  if (tid < E) {
    sum = s_part[tid];
    for (int q = 1; q < G; ++q) sum += s_part[q * E + tid];
  }
  finish_stats(sum, counts, T, k, E, alpha, f, P, l_aux, max_over_mean);
}

}  // namespace moe
