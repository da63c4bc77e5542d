// Balance statistics: f_i, P_i, L_aux = alpha * E * sum_i f_i P_i, demand max/mean.
//
// Transformers & Math 17.4 equation; The Residual Stream "Keeping the load even"
// and its MoE listing (f = counts / counts.sum(), P = mean softmax probability);
// Latent "Keeping the load balanced"; Understanding Data "Load imbalance"
// (measured on demand, before any capacity cut).
//
// stats_partial_kernel: 64 tokens per block; per-token softmax normalizers, then
// per-expert sums over the block's tokens in token order -> partial[block][E].
// stats_final_kernel: one block; sums the partials in block order (fp64), then
// f, P, L_aux and max/mean.  No atomics: results are deterministic.
#include "common.h"
#include "kernels.h"

namespace moe {
namespace {

// One block per 64 tokens.  The block's 64 x E score tile is copied to LDS with
// all loads in flight; each 16-lane row of a wave then takes one token (max and
// sum of exponentials with DPP butterflies), and finally thread e sums
// exp(s[t][e] - max_t) / sum_t over the 64 tokens in token order.
__global__ __launch_bounds__(256) void stats_partial_kernel(const float* __restrict__ logits, int T, int E,
                                                             float* __restrict__ partial) {
  __shared__ float tile[kStatsTokens * (MOE_MAX_EXPERTS + 1)];
  __shared__ float s_max[kStatsTokens], s_inv[kStatsTokens];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int t0 = blockIdx.x * kStatsTokens;
  const int nt = min(kStatsTokens, T - t0);
  const int stride = E + 1;
  const float* src = logits + (size_t)t0 * E;
  for (int i = tid; i < nt * E; i += 256) tile[(i / E) * stride + i % E] = src[i];
  __syncthreads();
  const int r = lane & 15;
  for (int lt = wave * 4 + (lane >> 4); lt < kStatsTokens; lt += 16) {  // 16 tokens per pass
    float m = -INFINITY;
    if (lt < nt)
      for (int e = r; e < E; e += 16) m = fmaxf(m, tile[lt * stride + e]);
    m = row16_max(m);
    float z = 0.f;
    if (lt < nt)
      for (int e = r; e < E; e += 16) z += expf(tile[lt * stride + e] - m);
    z = row16_sum(z);
    if (r == 0 && lt < nt) {
      s_max[lt] = m;
      s_inv[lt] = 1.f / z;
    }
  }
  __syncthreads();
  for (int e = tid; e < E; e += 256) {
    float acc = 0.f;
    for (int lt = 0; lt < nt; ++lt) acc += expf(tile[lt * stride + e] - s_max[lt]) * s_inv[lt];
    partial[(size_t)blockIdx.x * E + e] = acc;
  }
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
