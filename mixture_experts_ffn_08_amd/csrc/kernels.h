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
};
hipError_t launch_route(const RouteArgs& a, hipStream_t stream);

// b_e += rate * sign(T k - E counts_e) for e < E.
hipError_t launch_bias_update(const int32_t* counts, int T, int k, int E, float rate, float* bias,
                              hipStream_t stream);

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
};
hipError_t launch_permute(const PermuteArgs& a, hipStream_t stream);

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
};
// dual = true: C = SiLU(A B0^T) * (A B1^T); dual = false: C = A B0^T.
// bf16 launches with max_rows <= kSkinnyRowsPerGroup * G use the skinny kernel.
constexpr int kSkinnyRowsPerGroup = 16;
hipError_t launch_grouped_gemm(const GroupedGemmArgs& a, bool dual, hipStream_t stream);

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

constexpr int kStatsTokens = 64;  // tokens per partial-sum block
inline int stats_blocks(int T) { return (T + kStatsTokens - 1) / kStatsTokens; }

struct StatsArgs {
  const int32_t* counts;
  const float* logits;
  int T, k, E;
  float alpha;
  float *f, *P, *l_aux, *max_over_mean;
  float* partial;  // workspace [nblk][E]
};
hipError_t launch_stats(const StatsArgs& a, hipStream_t stream);

}  // namespace moe
