// Dispatch: per-expert histogram, capacity, stable permutation and row gather.
//
// ML Interview Notes, MoELayer listing: each expert collects the (token, slot)
// pairs that chose it.  "Capacity factor" and Transformers & Math 17.5: an
// expert holds at most C tokens, later arrivals are dropped by that expert.
//
// Assignments p = t*k + j arrive in ascending p.  The rank of p in its expert
// is fixed by the data, not by atomics: block b (512 assignments) records which
// of its assignments chose each expert in an LDS bitmap (atomicOr commutes, so
// the bitmap is the same in any order); rank = (assignments of earlier blocks,
// from a scan of per-block histograms) + popcount of the earlier bits.
//
//   hist_kernel   per-block expert histograms (LDS atomics)
//   scan_kernel   one block: per-expert scan over blocks, demand counts,
//                 capacity, exclusive scan over experts -> offsets
//   rank_kernel   bitmap ranks -> row_of, perm_token
//   rank_scan_kernel        scan + rank in one launch, up to 256 blocks: each block
//                           sums the histograms it needs itself
//   permute_single_kernel   the three above in one block when T k <= 512
//   gather_kernel x_perm[r] = x[perm_token[r]], one wave per row, 16-byte lanes
#include <algorithm>

#include "common.h"
#include "dispatch_single.h"
#include "kernels.h"
#include "stats_partial.h"

namespace moe {
namespace {

#ifndef MOE_RANK_SCAN
#define MOE_RANK_SCAN 1
#endif
constexpr int kBP = kPairsPerBlock;  // 512 threads, one assignment each
constexpr int kWords = kBP / 32;     // bitmap words per expert

__global__ __launch_bounds__(kBP) void hist_kernel(const int32_t* __restrict__ idx, int64_t P, int E,
                                                    int32_t* __restrict__ block_counts) {
  __shared__ int cnt[MOE_MAX_EXPERTS];
  const int tid = threadIdx.x;
  for (int e = tid; e < E; e += kBP) cnt[e] = 0;
  __syncthreads();
  const int64_t p = (int64_t)blockIdx.x * kBP + tid;
  if (p < P) {
    const int e = idx[p];
    if ((unsigned)e < (unsigned)E) atomicAdd(&cnt[e], 1);
  }
  __syncthreads();
  for (int e = tid; e < E; e += kBP) block_counts[(size_t)blockIdx.x * E + e] = cnt[e];
}

// One block of 1024 threads.  tpe threads per expert (thread c * ep + e) split the
// block list into contiguous chunks; chunk sums are scanned in LDS, then each thread writes the
// running base of its blocks; the kept counts are then scanned over experts in
// LDS for the offsets.
__global__ __launch_bounds__(1024) void scan_kernel(const int32_t* __restrict__ block_counts, int nblk,
                                                     int E, int ep, int tpe, int64_t cap, int padded,
                                                     int32_t* __restrict__ block_base,
                                                     int32_t* __restrict__ counts,
                                                     int32_t* __restrict__ offsets) {
  __shared__ int part[1024];
  __shared__ int tot_s[MOE_MAX_EXPERTS], kept_s[MOE_MAX_EXPERTS], incl_s[MOE_MAX_EXPERTS];
  constexpr int kBatch = 16;  // loads in flight per thread
  const int tid = threadIdx.x;
  // expert fastest (ep >= E, a power of two): a wave reads 64 consecutive experts'
  // counts of one block, one contiguous run, instead of 64 scattered words
  const int e = tid % ep, c = tid / ep;
  const bool active = e < E && c < tpe;
  const int chunk = (nblk + tpe - 1) / tpe;
  const int b0 = min(c * chunk, nblk), b1 = active ? min(b0 + chunk, nblk) : b0;
  const int ec = active ? e : 0;
  // Batches of clamped loads with the out-of-range terms zeroed: no branch
  // around a load, so a batch waits once.
  int sum = 0;
  for (int b = b0; b < b1; b += kBatch) {
    int v[kBatch];
#pragma unroll
    for (int q = 0; q < kBatch; ++q) v[q] = block_counts[(size_t)min(b + q, b1 - 1) * E + ec];
#pragma unroll
    for (int q = 0; q < kBatch; ++q) sum += b + q < b1 ? v[q] : 0;
  }
  part[tid] = sum;
  __syncthreads();
  int base = 0;
  if (active)
    for (int q = 0; q < c; ++q) base += part[q * ep + e];
  for (int b = b0; b < b1; b += kBatch) {
    int v[kBatch];
#pragma unroll
    for (int q = 0; q < kBatch; ++q) v[q] = block_counts[(size_t)min(b + q, b1 - 1) * E + ec];
#pragma unroll
    for (int q = 0; q < kBatch; ++q) {
      if (b + q < b1) {
        block_base[(size_t)(b + q) * E + ec] = base;
        base += v[q];
      }
    }
  }
  if (active && c == tpe - 1) {
    counts[e] = base;
    tot_s[e] = base;
  }
  __syncthreads();
  // kept counts and their inclusive scan over experts (the first wave)
  wave0_kept_scan(tot_s, E, cap, kept_s, incl_s);
  __syncthreads();
  if (!padded) {
    if (tid < E) offsets[tid + 1] = incl_s[tid];
    if (tid == 0) offsets[0] = 0;
  }
}

// Padded layout: offsets[e] = e C, and every slot past its expert's kept count
// marked -1 (the rank kernels fill the kept slots; the two write disjoint slots).
__global__ __launch_bounds__(256) void pad_kernel(const int32_t* __restrict__ counts, int E, int cap,
                                                   int32_t* __restrict__ offsets, int32_t* __restrict__ slot_token) {
  const int64_t s = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (s <= E) offsets[s] = (int32_t)(s * cap);
  if (s >= (int64_t)E * cap) return;
  const int e = (int)(s / cap), r = (int)(s % cap);
  if (r >= min(counts[e], cap)) slot_token[s] = -1;
}

__global__ __launch_bounds__(kBP) void rank_kernel(const int32_t* __restrict__ idx, int64_t P, int k, int E,
                                                    int64_t cap, const int32_t* __restrict__ block_base,
                                                    const int32_t* __restrict__ offsets, int padded,
                                                    int32_t* __restrict__ row_of,
                                                    int32_t* __restrict__ perm_token) {
  __shared__ uint32_t mask[MOE_MAX_EXPERTS * kWords];
  const int tid = threadIdx.x;
  for (int i = tid; i < E * kWords; i += kBP) mask[i] = 0u;
  __syncthreads();
  const int64_t p = (int64_t)blockIdx.x * kBP + tid;
  const int e = p < P ? idx[p] : -1;
  const bool valid = (unsigned)e < (unsigned)E;
  const int w = tid >> 5;
  const uint32_t bit = 1u << (tid & 31);
  if (valid) atomicOr(&mask[e * kWords + w], bit);
  __syncthreads();
  if (p >= P) return;
  int32_t row = -1;
  if (valid) {
    const uint32_t* m = mask + e * kWords;
    int r = __popc(m[w] & (bit - 1u));
    for (int q = 0; q < w; ++q) r += __popc(m[q]);
    const int rank = block_base[(size_t)blockIdx.x * E + e] + r;
    if (cap < 0 || rank < cap) {
      row = padded ? (int)(e * cap) + rank : offsets[e] + rank;
      perm_token[row] = (int32_t)(p / k);
    }
  }
  row_of[p] = row;
}

// rank_kernel with the scan folded in, for up to kRankScanMaxBlocks blocks: each
// block sums the per-block histograms itself (its base, the assignments of earlier
// blocks, and the totals), scans the kept totals over experts for the offsets, then
// ranks as rank_kernel does; block 0 writes counts and offsets.  Integer sums, so
// the results are those of scan_kernel + rank_kernel whatever the order.  Every
// block reads all nblk x E counts (L2), which is why the block count is bounded.
constexpr int kRankScanMaxBlocks = 256;

__global__ __launch_bounds__(kBP) void rank_scan_kernel(const int32_t* __restrict__ idx, int64_t P, int k, int E,
                                                         int64_t cap, int padded,
                                                         const int32_t* __restrict__ block_counts, int nblk, int ep,
                                                         int32_t* __restrict__ counts, int32_t* __restrict__ offsets,
                                                         int32_t* __restrict__ row_of,
                                                         int32_t* __restrict__ perm_token, StatsArgs st) {
  __shared__ uint32_t mask[MOE_MAX_EXPERTS * kWords];
  __shared__ int part_base[kBP], part_total[kBP];
  __shared__ int32_t s_tot[MOE_MAX_EXPERTS];
  __shared__ int base_s[MOE_MAX_EXPERTS], kept_s[MOE_MAX_EXPERTS], incl[MOE_MAX_EXPERTS];
  constexpr int kBatch = 16;  // loads in flight per thread
  const int tid = threadIdx.x;
  for (int i = tid; i < E * kWords; i += kBP) mask[i] = 0u;
  // Sums over the blocks: thread (c, e) = (tid / ep, tid % ep) (ep >= E a power of
  // two) takes chunk c of the block list; expert fastest, so a wave reads runs of
  // consecutive experts' counts.  Clamped loads, out-of-range terms zeroed.
  const int e2 = tid % ep, c = tid / ep, nch = kBP / ep;
  const int chunk = (nblk + nch - 1) / nch;
  const int b0 = min(c * chunk, nblk), b1 = e2 < E ? min(b0 + chunk, nblk) : b0;
  const int ec = e2 < E ? e2 : 0;
  const int me = blockIdx.x;
  int sb = 0, stot = 0;
  for (int b = b0; b < b1; b += kBatch) {
    int v[kBatch];
#pragma unroll
    for (int q = 0; q < kBatch; ++q) v[q] = block_counts[(size_t)min(b + q, b1 - 1) * E + ec];
#pragma unroll
    for (int q = 0; q < kBatch; ++q) {
      const int x = b + q < b1 ? v[q] : 0;
      stot += x;
      sb += b + q < me ? x : 0;
    }
  }
  part_base[tid] = sb;
  part_total[tid] = stot;
  __syncthreads();
  if (me == nblk) {
    // the extra block (uniform): the totals are the counts; then the statistics'
    // final reduction over the partial rows the router wrote
    if (tid < E) {
      int total = 0;
      for (int q = 0; q < nch; ++q) total += part_total[q * ep + tid];
      s_tot[tid] = total;
    }
    __syncthreads();
    stats_final_block<kBP>(s_tot, st.partial, stats_blocks(st.T), st.T, k, E, st.alpha, st.f, st.P, st.l_aux,
                           st.max_over_mean);
    return;
  }
  const int64_t p = (int64_t)blockIdx.x * kBP + tid;
  const int e = p < P ? idx[p] : -1;
  const bool valid = (unsigned)e < (unsigned)E;
  const int w = tid >> 5;
  const uint32_t bit = 1u << (tid & 31);
  if (valid) atomicOr(&mask[e * kWords + w], bit);
  if (tid < E) {
    int base = 0, total = 0;
    for (int q = 0; q < nch; ++q) {
      base += part_base[q * ep + tid];
      total += part_total[q * ep + tid];
    }
    base_s[tid] = base;
    s_tot[tid] = total;
    if (me == 0) counts[tid] = total;
  }
  __syncthreads();
  // kept totals and their inclusive scan over experts (the first wave)
  wave0_kept_scan(s_tot, E, cap, kept_s, incl);
  __syncthreads();
  if (me == 0 && !padded) {
    if (tid < E) offsets[tid + 1] = incl[tid];
    if (tid == 0) offsets[0] = 0;
  }
  if (p >= P) return;
  int32_t row = -1;
  if (valid) {
    const uint32_t* m = mask + e * kWords;
    int r = __popc(m[w] & (bit - 1u));
    for (int q = 0; q < w; ++q) r += __popc(m[q]);
    const int rank = base_s[e] + r;
    if (cap < 0 || rank < cap) {
      row = padded ? (int)(e * cap) + rank : incl[e] - kept_s[e] + rank;
      perm_token[row] = (int32_t)(p / k);
    }
  }
  row_of[p] = row;
}

__global__ __launch_bounds__(256) void gather_kernel(const char* __restrict__ x,
                                                      const int32_t* __restrict__ perm_token,
                                                      const int32_t* __restrict__ offsets_end, int T,
                                                      int max_rows, int row_bytes, int zero_padding,
                                                      char* __restrict__ x_perm) {
  const int R = min(*offsets_end, max_rows);
  const int lane = threadIdx.x & 63;
  const int wave = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int nwaves = gridDim.x * 4;
  for (int r = wave; r < R; r += nwaves) {
    const int t = perm_token[r];
    if ((unsigned)t >= (unsigned)T) {  // a padding slot
      if (zero_padding) {
        const u32x4 zero = {0u, 0u, 0u, 0u};
        for (int off = lane * 16; off < row_bytes; off += 1024) st16(x_perm + (size_t)r * row_bytes + off, zero);
      }
      continue;
    }
    const char* src = x + (size_t)t * row_bytes;
    char* dst = x_perm + (size_t)r * row_bytes;
    int off = lane * 16;
    // four 16-byte loads in flight per lane, then their stores
    for (; off + 3 * 1024 < row_bytes; off += 4 * 1024) {
      const u32x4 v0 = ld16(src + off), v1 = ld16(src + off + 1024);
      const u32x4 v2 = ld16(src + off + 2048), v3 = ld16(src + off + 3072);
      st16(dst + off, v0);
      st16(dst + off + 1024, v1);
      st16(dst + off + 2048, v2);
      st16(dst + off + 3072, v3);
    }
    for (; off < row_bytes; off += 1024) st16(dst + off, ld16(src + off));
  }
}

// All of histogram, scan and rank in one block, for T k <= 512 assignments (the
// decode shapes): the same results as the three kernels above with one block.
static_assert(kBP == kSingleMaxPairs, "one thread per assignment");
__global__ __launch_bounds__(kBP) void permute_single_kernel(const int32_t* __restrict__ idx, int64_t P, int k,
                                                              int E, int64_t cap, int padded,
                                                              int32_t* __restrict__ counts,
                                                              int32_t* __restrict__ offsets,
                                                              int32_t* __restrict__ row_of,
                                                              int32_t* __restrict__ perm_token) {
  dispatch_single(idx, P, k, E, cap, padded, counts, offsets, row_of, perm_token);
}

}  // namespace

bool permute_fuses_stats(int T, int k) {
  const int nblk = permute_blocks(T, k);
  return MOE_RANK_SCAN && nblk > 1 && nblk <= kRankScanMaxBlocks;
}

hipError_t launch_permute(const PermuteArgs& a, hipStream_t stream) {
  const int64_t P = (int64_t)a.T * a.k;
  const int nblk = permute_blocks(a.T, a.k);
  int ep = 1;
  while (ep < a.E) ep <<= 1;
  const int tpe = min(64, 1024 / ep);
  if (nblk == 1) {
    hipLaunchKernelGGL(permute_single_kernel, dim3(1), dim3(kBP), 0, stream, a.topk_idx, P, a.k, a.E, a.capacity,
                       a.padded, a.counts, a.offsets, a.row_of, a.perm_token);
  } else if (nblk <= kRankScanMaxBlocks && MOE_RANK_SCAN) {
    if (!a.hist_given)
      hipLaunchKernelGGL(hist_kernel, dim3(nblk), dim3(kBP), 0, stream, a.topk_idx, P, a.E, a.block_counts);
    // with a final statistics reduction, one more block (index nblk) runs it
    const StatsArgs st = a.stats != nullptr ? *a.stats : StatsArgs{};
    hipLaunchKernelGGL(rank_scan_kernel, dim3(nblk + (a.stats != nullptr ? 1 : 0)), dim3(kBP), 0, stream,
                       a.topk_idx, P, a.k, a.E, a.capacity, a.padded, a.block_counts, nblk, ep, a.counts, a.offsets,
                       a.row_of, a.perm_token, st);
  } else {
    if (!a.hist_given)
      hipLaunchKernelGGL(hist_kernel, dim3(nblk), dim3(kBP), 0, stream, a.topk_idx, P, a.E, a.block_counts);
    hipLaunchKernelGGL(scan_kernel, dim3(1), dim3(1024), 0, stream, a.block_counts, nblk, a.E, ep, tpe,
                       a.capacity, a.padded, a.block_base, a.counts, a.offsets);
    hipLaunchKernelGGL(rank_kernel, dim3(nblk), dim3(kBP), 0, stream, a.topk_idx, P, a.k, a.E, a.capacity,
                       a.block_base, a.offsets, a.padded, a.row_of, a.perm_token);
  }
  if (a.padded) {
    const int64_t slots = (int64_t)a.E * a.capacity;
    const int64_t n = std::max<int64_t>(slots, a.E + 1);
    hipLaunchKernelGGL(pad_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream, a.counts, a.E,
                       (int)a.capacity, a.offsets, a.perm_token);
  }
  if (a.x_perm == nullptr) return hipGetLastError();
  const int max_rows = a.padded ? (int)((int64_t)a.E * a.capacity) : (int)P;
  const int blocks = (int)std::min<int64_t>((max_rows + 3) / 4, 8192);
  hipLaunchKernelGGL(gather_kernel, dim3(blocks > 0 ? blocks : 1), dim3(256), 0, stream,
                     (const char*)a.x, a.perm_token, a.offsets + a.E, a.T, max_rows, a.row_bytes, a.padded,
                     (char*)a.x_perm);
  return hipGetLastError();
}

}  // namespace moe
