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

// Block-wide finish: thread e < E holds sum_t softmax(s_t)_e in fp64.  Writes f, P,
// L_aux = alpha E sum_e f_e P_e and max/mean = E max_e counts_e / (T k).  Called by
// every thread of a block of at least 256 threads.
__device__ void finish_stats(double sum, const int32_t* __restrict__ counts, int T, int k, int E, float alpha,
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

// One block.  Thread (g, e) sums partial[b][e] over blocks b = g, g + G, ... in
// fp64, 16 loads in flight (indices clamped, out-of-range terms zeroed, no
// branch around a load); the group sums are added in group order.  Then f, P,
// L_aux and max/mean.  No atomics: results are deterministic.
__global__ __launch_bounds__(1024) void stats_final_kernel(const int32_t* __restrict__ counts,
                                                            const float* __restrict__ partial, int nblk, int T,
                                                            int k, int E, float alpha, float* __restrict__ f,
                                                            float* __restrict__ P, float* __restrict__ l_aux,
                                                            float* __restrict__ max_over_mean) {
  __shared__ double s_part[1024];
  const int tid = threadIdx.x;
  const int G = 1024 / E;  // groups of E threads (4 at E = 256, 8 at E = 128)
  const int g = tid / E, ge = tid % E;
  if (g < G) {
    double part[16];
#pragma unroll
    for (int q = 0; q < 16; ++q) part[q] = 0.0;
    for (int b0 = g; b0 < nblk; b0 += 16 * G) {
      float pv[16];
#pragma unroll
      for (int q = 0; q < 16; ++q) pv[q] = partial[(size_t)min(b0 + q * G, nblk - 1) * E + ge];
#pragma unroll
      for (int q = 0; q < 16; ++q) part[q] += b0 + q * G < nblk ? (double)pv[q] : 0.0;
    }
    double sum = 0.0;
#pragma unroll
    for (int q = 0; q < 16; ++q) sum += part[q];
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
  hipLaunchKernelGGL(stats_final_kernel, dim3(1), dim3(1024), 0, stream, a.counts, a.partial, stats_blocks(a.T),
                     a.T, a.k, a.E, a.alpha, a.f, a.P, a.l_aux, a.max_over_mean);
  return hipGetLastError();
}

}  // namespace moe
