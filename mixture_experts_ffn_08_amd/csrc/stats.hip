// Balance statistics: f_i, P_i, L_aux = alpha * E * sum_i f_i P_i, demand max/mean.
//
// Transformers & Math 17.4 equation; The Residual Stream "Keeping the load even"
// and its MoE listing (f = counts / counts.sum(), P = mean softmax probability);
// Latent "Keeping the load balanced"; Understanding Data "Load imbalance"
// (measured on demand, before any capacity cut).
//
// stats_partial_kernel: 64 tokens per block, one wave per token at a time,
// softmax over all E (lane holds experts lane + 64 i), per-lane fp32 sums, then
// the four waves' sums added in fixed order -> partial[block][E].
// stats_final_kernel: one block; sums the partials in block order (fp64), then
// f, P, L_aux and max/mean.  No atomics: results are deterministic.
#include "common.h"
#include "kernels.h"

namespace moe {
namespace {

__global__ __launch_bounds__(256) void stats_partial_kernel(const float* __restrict__ logits, int T, int E,
                                                             float* __restrict__ partial) {
  __shared__ float s_part[4][MOE_MAX_EXPERTS];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int t0 = blockIdx.x * kStatsTokens;
  float acc[4] = {0.f, 0.f, 0.f, 0.f};
  for (int lt = wave; lt < kStatsTokens; lt += 4) {
    const int t = t0 + lt;
    if (t >= T) break;
    const float* s = logits + (size_t)t * E;
    float v[4];
    float m = -INFINITY;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int e = lane + 64 * i;
      v[i] = e < E ? s[e] : -INFINITY;
      m = fmaxf(m, v[i]);
    }
    m = wave_max(m);
    float z = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[i] = (lane + 64 * i < E) ? expf(v[i] - m) : 0.f;
      z += v[i];
    }
    z = wave_sum(z);
    const float inv = 1.f / z;
#pragma unroll
    for (int i = 0; i < 4; ++i) acc[i] += v[i] * inv;
  }
#pragma unroll
  for (int i = 0; i < 4; ++i)
    if (lane + 64 * i < E) s_part[wave][lane + 64 * i] = acc[i];
  __syncthreads();
  for (int e = tid; e < E; e += 256)
    partial[(size_t)blockIdx.x * E + e] = ((s_part[0][e] + s_part[1][e]) + s_part[2][e]) + s_part[3][e];
}

__global__ __launch_bounds__(256) void stats_final_kernel(const int32_t* __restrict__ counts,
                                                           const float* __restrict__ partial, int nblk, int T,
                                                           int k, int E, float alpha, float* __restrict__ f,
                                                           float* __restrict__ P, float* __restrict__ l_aux,
                                                           float* __restrict__ max_over_mean) {
  __shared__ double s_fp[256];
  __shared__ int s_max[256];
  const int e = threadIdx.x;
  const float tk = (float)((int64_t)T * k);
  double fp = 0.0;
  int c = 0;
  if (e < E) {
    double sum = 0.0;
    for (int b = 0; b < nblk; ++b) sum += (double)partial[(size_t)b * E + e];
    const float p = (float)(sum / (double)T);
    c = counts[e];
    const float fi = (float)c / tk;
    f[e] = fi;
    P[e] = p;
    fp = (double)fi * (double)p;
  }
  s_fp[e] = fp;
  s_max[e] = c;
  __syncthreads();
  for (int s = 128; s > 0; s >>= 1) {
    if (e < s) {
      s_fp[e] += s_fp[e + s];
      s_max[e] = max(s_max[e], s_max[e + s]);
    }
    __syncthreads();
  }
  if (e == 0) {
    *l_aux = (float)((double)alpha * (double)E * s_fp[0]);
    *max_over_mean = (float)((int64_t)E * s_max[0]) / tk;
  }
}

}  // namespace

hipError_t launch_stats(const StatsArgs& a, hipStream_t stream) {
  const int nblk = stats_blocks(a.T);
  hipLaunchKernelGGL(stats_partial_kernel, dim3(nblk), dim3(256), 0, stream, a.logits, a.T, a.E, a.partial);
  hipLaunchKernelGGL(stats_final_kernel, dim3(1), dim3(256), 0, stream, a.counts, a.partial, nblk, a.T, a.k,
                     a.E, a.alpha, a.f, a.P, a.l_aux, a.max_over_mean);
  return hipGetLastError();
}

}  // namespace moe
