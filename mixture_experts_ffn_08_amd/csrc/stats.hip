// Balance statistics: f_i, P_i, L_aux = alpha * E * sum_i f_i P_i, demand max/mean.
//
// Transformers & Math 17.4 equation; The Residual Stream "Keeping the load even"
// and its MoE listing (f = counts / counts.sum(), P = mean softmax probability);
// Latent "Keeping the load balanced"; Understanding Data "Load imbalance"
// (measured on demand, before any capacity cut).
//
// stats_partial_kernel: 64 tokens per block; per-token softmax normalizers, then
// per-expert sums over the block's tokens in token order -> partial[block][E].
// stats_final_kernel: one block; sums the partials (fp64) in a fixed order, then
// f, P, L_aux and max/mean.  When T fits one block (T <= 64), stats_small_kernel
// does everything in one launch.  No atomics: results are deterministic.
#include "common.h"
#include "kernels.h"
#include "stats_partial.h"
#include "stats_single.h"

namespace moe {
namespace {

// One block per 64 tokens.  The block's 64 x E score tile is copied to LDS with
// all loads in flight; each 16-lane row of a wave then takes one token (max and
// sum of exponentials with DPP butterflies); finally thread (g, e) sums
// exp(s[t][e] - max_t) / sum_t over the tokens t = g, g + G, ... of the block.
__global__ __launch_bounds__(256) void stats_partial_kernel(const float* __restrict__ logits, int T, int E,
                                                             float* __restrict__ partial) {
  __shared__ float tile[kStatsTokens * MOE_MAX_EXPERTS];
  __shared__ float s_max[kStatsTokens], s_inv[kStatsTokens];
  __shared__ float red[256];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int t0 = blockIdx.x * kStatsTokens;
  const int nt = min(kStatsTokens, T - t0);
  const float* src = logits + (size_t)t0 * E;
  // The block's rows are copied to LDS as they lie (row stride E), all loads
  // issued before any is stored (at most 64 per thread).
  constexpr int kMaxPerThread = kStatsTokens * MOE_MAX_EXPERTS / 256;
  const int n = nt * E;
  float v[kMaxPerThread];
#pragma unroll
  for (int j = 0; j < kMaxPerThread; ++j) v[j] = src[min(tid + 256 * j, n - 1)];  // n >= 1
#pragma unroll
  for (int j = 0; j < kMaxPerThread; ++j)
    if (tid + 256 * j < n) tile[tid + 256 * j] = v[j];
  __syncthreads();
  block_softmax_sums<256>(tile, E, nt, E, s_max, s_inv, red, partial + (size_t)blockIdx.x * E);
}

// All T <= 64 tokens in one block of 16 waves (stats_single).
static_assert(kStatsTokens == kSingleStatsTokens, "one block takes T <= kStatsTokens");
__global__ __launch_bounds__(1024) void stats_small_kernel(const float* __restrict__ logits, int T, int E,
                                                            const int32_t* __restrict__ counts, int k, float alpha,
                                                            float* __restrict__ f, float* __restrict__ P,
                                                            float* __restrict__ l_aux,
                                                            float* __restrict__ max_over_mean) {
  stats_single(logits, T, E, counts, k, alpha, f, P, l_aux, max_over_mean);
}

// One block: stats_final_block.
__global__ __launch_bounds__(kStatsFinalThreads) void stats_final_kernel(
    const int32_t* __restrict__ counts, const float* __restrict__ partial, int nblk, int T, int k, int E,
    float alpha, float* __restrict__ f, float* __restrict__ P, float* __restrict__ l_aux,
    float* __restrict__ max_over_mean) {
  stats_final_block<kStatsFinalThreads>(counts, partial, nblk, T, k, E, alpha, f, P, l_aux, max_over_mean);
}

// Bias balancing (The Residual Stream, "Keeping the load even", and the MoE
// listing's step after each batch): raise b_e by `rate` when expert e got fewer
// than its share of the T k assignments, lower it when it got more.  The share is
// compared exactly, as integers: T k against E counts_e.
__global__ __launch_bounds__(256) void bias_update_kernel(const int32_t* __restrict__ counts, int64_t tk, int E,
                                                           float rate, float* __restrict__ bias) {
  const int e = blockIdx.x * 256 + threadIdx.x;
  if (e >= E) return;
  const int64_t diff = tk - (int64_t)E * counts[e];
  const float sign = diff > 0 ? 1.f : (diff < 0 ? -1.f : 0.f);
  bias[e] = bias[e] + rate * sign;  // rate * sign is exact: one rounding, as in float32 arithmetic
}

}  // namespace

hipError_t launch_bias_update(const int32_t* counts, int T, int k, int E, float rate, float* bias,
                              hipStream_t stream) {
  hipLaunchKernelGGL(bias_update_kernel, dim3((E + 255) / 256), dim3(256), 0, stream, counts, (int64_t)T * k, E,
                     rate, bias);
  return hipGetLastError();
}

hipError_t launch_stats(const StatsArgs& a, hipStream_t stream) {
  const int nblk = stats_blocks(a.T);
  if (nblk == 1) {
    hipLaunchKernelGGL(stats_small_kernel, dim3(1), dim3(1024), 0, stream, a.logits, a.T, a.E, a.counts, a.k,
                       a.alpha, a.f, a.P, a.l_aux, a.max_over_mean);
    return hipGetLastError();
  }
  hipLaunchKernelGGL(stats_partial_kernel, dim3(nblk), dim3(256), 0, stream, a.logits, a.T, a.E, a.partial);
  return launch_stats_final(a, stream);
}

hipError_t launch_stats_final(const StatsArgs& a, hipStream_t stream) {
  hipLaunchKernelGGL(stats_final_kernel, dim3(1), dim3(kStatsFinalThreads), 0, stream, a.counts, a.partial,
                     stats_blocks(a.T),
                     a.T, a.k, a.E, a.alpha, a.f, a.P, a.l_aux, a.max_over_mean);
  return hipGetLastError();
}

}  // namespace moe
