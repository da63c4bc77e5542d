// Per-block partial sums of the balance statistic P (Transformers & Math 17.4;
// The Residual Stream, "Keeping the load even"): for a block of nt <= 64 tokens
// whose scores sit in LDS, sum over the block's tokens of softmax(scores)[e], for
// every expert e.  One definition for every kernel that produces them, so that the
// partials are the same bits whichever kernel wrote them.
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

}  // namespace moe
