// Internal launchers of the MoE kernels.  Arguments are validated by the C ABI
// layer (api.cpp) before any of these is called.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/moe.h"

namespace moe {

struct RouteArgs {
  const void* x;
  const void* w_router;
  const float* bias;
  const float* select_bias;
  int dtype, T, d, E, k, mode, renorm;
  float* logits;
  int32_t* topk_idx;
  float* topk_w;
  int32_t* near_tie;
  // [nblk][E] or null: with route_writes_block_hist, the histogram of each block of
  // kPairsPerBlock assignments (the dispatch's hist_kernel output) is written too
  int32_t* block_hist = nullptr;
  // [stats_blocks(T)][E] or null: with route_writes_block_hist, the per-block partial
  // sums of the balance statistic P (stats_partial_kernel's output) as well
  float* stats_partial = nullptr;
};
hipError_t launch_route(const RouteArgs& a, hipStream_t stream);

// Few tokens (bf16, T <= 64, T k <= 512): the scores, then selection, the compact
// dispatch and the balance statistics in one block (the results of launch_route,
// launch_permute with capacity and no x_perm, and launch_stats).
struct RouteDispatchArgs {
  RouteArgs route;
  int64_t capacity;  // < 0: dropless
  int32_t *counts, *offsets, *row_of, *perm_token;
  float alpha;
  float *f, *P, *l_aux, *max_over_mean;
};
bool route_dispatch_small_fits(int dtype, int T, int k, int E);
hipError_t launch_route_dispatch_small(const RouteDispatchArgs& a, hipStream_t stream);

// b_e += rate * sign(T k - E counts_e) for e < E.
hipError_t launch_bias_update(const int32_t* counts, int T, int k, int E, float rate, float* bias,
                              hipStream_t stream);

constexpr int kStatsTokens = 64;  // tokens per partial-sum block
__host__ __device__ inline int stats_blocks(int T) { return (T + kStatsTokens - 1) / kStatsTokens; }

struct StatsArgs {
  const int32_t* counts;
  const float* logits;
  int T, k, E;
  float alpha;
  float *f, *P, *l_aux, *max_over_mean;
  float* partial;  // workspace [nblk][E]
};
hipError_t launch_stats(const StatsArgs& a, hipStream_t stream);
// The final reduction alone, over stats_blocks(T) partial rows another kernel wrote.
hipError_t launch_stats_final(const StatsArgs& a, hipStream_t stream);

// Dispatch works on the flattened assignment index p = t*k + j in blocks of
// kPairsPerBlock assignments.
constexpr int kPairsPerBlock = 512;
inline int permute_blocks(int T, int k) { return (int)(((int64_t)T * k + kPairsPerBlock - 1) / kPairsPerBlock); }

struct PermuteArgs {
  const int32_t* topk_idx;
  int T, k, E;
  int64_t capacity;  // < 0: dropless
  const void* x;
  int row_bytes;     // d * element size, a multiple of 16
  int32_t* counts;
  int32_t* offsets;
  int32_t* row_of;
  int32_t* perm_token;
  void* x_perm;
  int32_t* block_counts;  // workspace [nblk][E]
  int32_t* block_base;    // workspace [nblk][E]
  int padded;             // 1: slot e * capacity + rank, offsets e * capacity, padding -1 / zero rows
  int hist_given = 0;     // 1: block_counts already hold the per-block histograms (the router wrote them)
  // With permute_fuses_stats: the statistics' final reduction over stats->partial
  // (rows another kernel wrote) runs as one more block of the rank launch.
  const StatsArgs* stats = nullptr;
};
hipError_t launch_permute(const PermuteArgs& a, hipStream_t stream);
// Whether launch_permute runs a given final statistics reduction inside its rank launch.
bool permute_fuses_stats(int T, int k);
// Whether launch_route with a block_hist writes the dispatch's per-block histograms
// for these sizes (its blocks of 64 tokens then hold exactly kPairsPerBlock assignments).
bool route_writes_block_hist(int dtype, int T, int E, int k);

struct GroupedGemmArgs {
  const void* A;        // [max_rows][K], or [a_nrows][K] read through a_rows
  const int32_t* a_rows;  // null, or row r of the product reads A[a_rows[r]]
  int a_nrows;
  const int32_t* offsets;
  int G, max_rows, N, K;
  const void* B0;       // [G][N][K]
  const void* B1;       // [G][N][K] (gate/up: the up projection) or null
  void* C;              // [max_rows][N]
  int dtype;
  // Scatter form (single only): instead of writing C, row r of the product, rounded
  // to dtype, times out_w[r] is added (fp32 atomics) to y_acc[out_tok[r]] ([T][N]
  // fp32); rows with out_tok[r] outside [0, T) are skipped.
  const int32_t* out_tok = nullptr;
  const float* out_w = nullptr;
  float* y_acc = nullptr;
  int T = 0;
};
// dual = true: C = SiLU(A B0^T) * (A B1^T); dual = false: C = A B0^T.
// bf16 launches with max_rows <= kSkinnyRowsPerGroup * G use the skinny kernel for
// the groups of up to 16 rows and the tiled kernel for the others.
constexpr int kSkinnyRowsPerGroup = 8;
hipError_t launch_grouped_gemm(const GroupedGemmArgs& a, bool dual, hipStream_t stream);

// Around the scatter form of the down GEMM: zero y_acc [T][d] and write
// row_w[row_of[t][j]] = topk_w[t][j] for kept slots (before); y = y_acc +
// shared_y, rounded to dtype (after).
hipError_t launch_scatter_prologue(float* y_acc, float* row_w, const int32_t* row_of, const float* topk_w, int T,
                                   int k, int d, int max_rows, hipStream_t stream);
hipError_t launch_scatter_finish(const float* y_acc, const void* shared_y, int dtype, int T, int d, void* y,
                                 hipStream_t stream);

struct CombineArgs {
  const void* y_perm;
  const int32_t* row_of;
  const float* topk_w;
  const void* shared_y;
  int dtype, T, k, d;
  int y_rows;  // rows of y_perm; row_of values outside [0, y_rows) count as dropped
  void* y;
};
hipError_t launch_combine(const CombineArgs& a, hipStream_t stream);



}  // namespace moe
