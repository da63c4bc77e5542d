// Dispatch of at most 512 assignments in one block: histogram, capacity, scan over
// experts and ranks, with the results of the multi-block kernels (per-expert
// bitmaps of the assignments, ranks by popcount of the earlier bits: fixed by the
// data, not by the order of the atomics).
//
// ML Interview Notes, MoELayer listing (each expert collects the pairs that chose
// it); "Capacity factor" and Transformers & Math 17.5 (an expert keeps at most C,
// later arrivals are dropped).
#pragma once

#include "../../include/moe.h"
#include "common.h"

namespace moe {

constexpr int kSingleMaxPairs = 512;             // assignments one block dispatches
constexpr int kSingleWords = kSingleMaxPairs / 32;  // bitmap words per expert

// Kept counts and their inclusive scan over E <= MOE_MAX_EXPERTS experts, by the
// block's first wave alone (lane l takes experts 4 l .. 4 l + 3, a shuffle prefix
// adds the earlier lanes' sums): one barrier afterwards instead of one per step of a
// block-wide scan.  cnt in LDS; kept and incl (LDS) receive min(cnt, cap) (cnt when
// dropless) and the inclusive prefix of kept.  Every thread calls it.
__device__ inline void wave0_kept_scan(const int* __restrict__ cnt, int E, int64_t cap, int* __restrict__ kept,
                                       int* __restrict__ incl) {
  static_assert(MOE_MAX_EXPERTS <= 4 * 64, "four experts a lane");
  if (threadIdx.x >= 64) return;
  const int lane = threadIdx.x;
  int v[4], sum = 0;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int i = 4 * lane + j;
    const int c = i < E ? cnt[i] : 0;
    v[j] = cap < 0 ? c : (int)min((int64_t)c, cap);
    sum += v[j];
  }
  int run = sum;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int u = __shfl_up(run, o, 64);
    if (lane >= o) run += u;
  }
  run -= sum;  // exclusive prefix of this lane's first expert
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int i = 4 * lane + j;
    run += v[j];
    if (i < E) {
      kept[i] = v[j];
      incl[i] = run;
    }
  }
}

// Called by every thread of a block of at least kSingleMaxPairs threads; P <= 512.
// idx may be in LDS.  The block's threads exchange data through LDS only, so the
// barriers wait for LDS operations, not for global stores.  counts_copy (LDS or
// global, may be NULL) receives the counts as well.
__device__ inline void dispatch_single(const int32_t* __restrict__ idx, int64_t P, int k, int E, int64_t cap,
                                       int padded, int32_t* __restrict__ counts, int32_t* __restrict__ offsets,
                                       int32_t* __restrict__ row_of, int32_t* __restrict__ perm_token,
                                       int32_t* __restrict__ counts_copy = nullptr) {
  __shared__ uint32_t mask[MOE_MAX_EXPERTS * kSingleWords];
  __shared__ int cnt[MOE_MAX_EXPERTS];
  __shared__ int kept[MOE_MAX_EXPERTS];
  __shared__ int incl[MOE_MAX_EXPERTS];
  const int tid = threadIdx.x, nthr = blockDim.x;
  for (int i = tid; i < E * kSingleWords; i += nthr) mask[i] = 0u;
  for (int i = tid; i < E; i += nthr) cnt[i] = 0;
  lds_barrier();
  const int e = tid < P ? idx[tid] : -1;
  const bool valid = (unsigned)e < (unsigned)E;
  const int w = tid >> 5;
  const uint32_t bit = 1u << (tid & 31);
  if (valid) {
    atomicOr(&mask[e * kSingleWords + w], bit);
    atomicAdd(&cnt[e], 1);
  }
  lds_barrier();
  for (int i = tid; i < E; i += nthr) {
    counts[i] = cnt[i];
    if (counts_copy != nullptr) counts_copy[i] = cnt[i];
  }
  wave0_kept_scan(cnt, E, cap, kept, incl);
  lds_barrier();
  if (!padded) {
    for (int i = tid; i < E; i += nthr) offsets[i + 1] = incl[i];
    if (tid == 0) offsets[0] = 0;
  }
  if (tid >= P) return;
  int32_t row = -1;
  if (valid) {
    const uint32_t* m = mask + e * kSingleWords;
    int rank = __popc(m[w] & (bit - 1u));
    for (int q = 0; q < w; ++q) rank += __popc(m[q]);
    if (cap < 0 || rank < cap) {
      row = padded ? (int)(e * cap) + rank : incl[e] - kept[e] + rank;
      perm_token[row] = tid / k;
    }
  }
  row_of[tid] = row;
}

}  // namespace moe
