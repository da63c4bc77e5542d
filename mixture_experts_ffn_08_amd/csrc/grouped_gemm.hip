// Variable-size grouped GEMM for the SwiGLU experts.
//
// The Residual Stream, "An MoE tiny GPT" listing: expert e runs on its rows h as
// (SiLU(h @ gate[e]) * (h @ up[e])) @ down[e].  ML Interview Notes "Capacity
// factor": dropless routing runs the experts as one variable-size grouped GEMM.
//
// C[r] = A[r] B_g^T for rows r of group g (dual: C = SiLU(A B0_g^T) * (A B1_g^T)).
// A is [rows][K] and B is [N][K], both K-contiguous, so both MFMA operands load
// as 16-byte K-vectors with no transpose.
//
// bf16 kernel: 256 threads (2 x 2 waves), block tile 128 rows x 128 columns (of
// each B in the dual form), K step 64.  Global -> registers -> LDS with the next
// K step prefetched into registers while the current one is multiplied; MFMA
// 32x32x16 bf16 with fp32 accumulation; SiLU * up fused into the epilogue.
// Tiles of all groups are enumerated on the device: each block scans the
// per-group tile counts (from offsets) to find its group and first row, so the
// host never reads the routing back.
#include <algorithm>

#include "common.h"
#include "kernels.h"

namespace moe {
namespace {

constexpr int BM = 128, BN = 128, BK = 64;
constexpr int LDS_STRIDE = BK + 8;  // bf16 elements per LDS row (16-byte pad)

__device__ __forceinline__ int clamp_off(int v, int max_rows) { return min(max(v, 0), max_rows); }

// Block-wide: locate m-tile `mt` among the groups.  Returns false (uniformly) when
// mt is past the last tile.
__device__ bool find_tile(const int32_t* __restrict__ offsets, int G, int max_rows, int mt, int& g,
                          int& row0, int& row_end) {
  __shared__ int s_incl[256];
  __shared__ int s_wave_tot[4];
  __shared__ int s_info[3];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  int lo = 0, hi = 0, cnt = 0;
  if (tid < G) {
    lo = clamp_off(offsets[tid], max_rows);
    hi = clamp_off(offsets[tid + 1], max_rows);
    cnt = hi > lo ? (hi - lo + BM - 1) / BM : 0;
  }
  // inclusive scan of cnt over the 256 threads
  int v = cnt;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int u = __shfl_up(v, o, 64);
    if (lane >= o) v += u;
  }
  if (lane == 63) s_wave_tot[wave] = v;
  if (tid == 0) s_info[0] = -1;
  __syncthreads();
  for (int w = 0; w < wave; ++w) v += s_wave_tot[w];
  s_incl[tid] = v;
  __syncthreads();
  const int total = s_incl[255];
  if (mt >= total) return false;
  const int excl = v - cnt;
  if (tid < G && cnt > 0 && mt >= excl && mt < v) {
    s_info[0] = tid;
    s_info[1] = lo + (mt - excl) * BM;
    s_info[2] = hi;
  }
  __syncthreads();
  g = s_info[0];
  row0 = s_info[1];
  row_end = s_info[2];
  return g >= 0;
}

template <bool DUAL>
__global__ __launch_bounds__(256, 2) void grouped_gemm_bf16_kernel(
    const uint16_t* __restrict__ A, const int32_t* __restrict__ offsets, int G, int max_rows, int N, int K,
    const uint16_t* __restrict__ B0, const uint16_t* __restrict__ B1, uint16_t* __restrict__ C,
    int n_tiles) {
  constexpr int NMAT = DUAL ? 2 : 1;
  __shared__ __attribute__((aligned(16))) uint16_t sA[BM * LDS_STRIDE];
  __shared__ __attribute__((aligned(16))) uint16_t sB[NMAT][BN * LDS_STRIDE];

  const int mt = blockIdx.x / n_tiles, nt = blockIdx.x % n_tiles;
  int g, row0, row_end;
  if (!find_tile(offsets, G, max_rows, mt, g, row0, row_end)) return;

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int wm = wave >> 1, wn = wave & 1;
  const int n0 = nt * BN;

  // Copy mapping: a 128 x 64 tile is 1024 16-byte chunks; thread tid moves chunks
  // tid + 256*i: row (tid >> 3) + 32*i, column 8*(tid & 7).
  const int crow = tid >> 3, ccol = 8 * (tid & 7);
  const uint16_t* a_src[4];
  const uint16_t* b_src[NMAT][4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = min(row0 + crow + 32 * i, row_end - 1);
    a_src[i] = A + (size_t)r * K + ccol;
    const size_t brow = (size_t)g * N + n0 + crow + 32 * i;
    b_src[0][i] = B0 + brow * K + ccol;
    if (DUAL) b_src[NMAT - 1][i] = B1 + brow * K + ccol;
  }

  u32x4 ra[4], rb[NMAT][4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    ra[i] = ld16(a_src[i]);
#pragma unroll
    for (int m = 0; m < NMAT; ++m) rb[m][i] = ld16(b_src[m][i]);
  }

  f32x16 acc[NMAT][2][2];
#pragma unroll
  for (int m = 0; m < NMAT; ++m)
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[m][i][j][r] = 0.f;

  const int frow = lane & 31, fk = 8 * (lane >> 5);
  for (int k0 = 0; k0 < K; k0 += BK) {
    __syncthreads();
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      st16(&sA[(crow + 32 * i) * LDS_STRIDE + ccol], ra[i]);
#pragma unroll
      for (int m = 0; m < NMAT; ++m) st16(&sB[m][(crow + 32 * i) * LDS_STRIDE + ccol], rb[m][i]);
    }
    __syncthreads();
    if (k0 + BK < K) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        ra[i] = ld16(a_src[i] + k0 + BK);
#pragma unroll
        for (int m = 0; m < NMAT; ++m) rb[m][i] = ld16(b_src[m][i] + k0 + BK);
      }
    }
#pragma unroll
    for (int ks = 0; ks < BK; ks += 16) {
      bf16x8 af[2], bfr[NMAT][2];
#pragma unroll
      for (int i = 0; i < 2; ++i) af[i] = as_bf16x8(ld16(&sA[(wm * 64 + i * 32 + frow) * LDS_STRIDE + ks + fk]));
#pragma unroll
      for (int m = 0; m < NMAT; ++m)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          bfr[m][j] = as_bf16x8(ld16(&sB[m][(wn * 64 + j * 32 + frow) * LDS_STRIDE + ks + fk]));
#pragma unroll
      for (int m = 0; m < NMAT; ++m)
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
          for (int j = 0; j < 2; ++j) acc[m][i][j] = mfma32x32x16(af[i], bfr[m][j], acc[m][i][j]);
    }
  }

  // Epilogue: accumulator element r of lane l is row 8*(r/4) + 4*(l/32) + r%4,
  // column l%32 of its 32 x 32 fragment.
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int col = n0 + wn * 64 + j * 32 + (lane & 31);
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = row0 + wm * 64 + i * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
        if (row < row_end) {
          float v = acc[0][i][j][r];
          if (DUAL) {
            const float u = acc[NMAT - 1][i][j][r];
            v = v / (1.f + expf(-v)) * u;
          }
          C[(size_t)row * N + col] = f32_to_bf16(v);
        }
      }
    }
}

// fp32 path: one thread per output element, plain K loop.
template <bool DUAL>
__global__ __launch_bounds__(256) void grouped_gemm_f32_kernel(const float* __restrict__ A,
                                                                const int32_t* __restrict__ offsets, int G,
                                                                int max_rows, int N, int K,
                                                                const float* __restrict__ B0,
                                                                const float* __restrict__ B1,
                                                                float* __restrict__ C) {
  const int64_t id = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (id >= (int64_t)max_rows * N) return;
  const int row = (int)(id / N), n = (int)(id % N);
  int g = -1;
  for (int q = 0; q < G; ++q) {
    const int lo = clamp_off(offsets[q], max_rows), hi = clamp_off(offsets[q + 1], max_rows);
    if (row >= lo && row < hi) { g = q; break; }
  }
  if (g < 0) return;
  const float* a = A + (size_t)row * K;
  const float* b0 = B0 + ((size_t)g * N + n) * K;
  float s0 = 0.f, s1 = 0.f;
  if (DUAL) {
    const float* b1 = B1 + ((size_t)g * N + n) * K;
    for (int i = 0; i < K; ++i) {
      s0 = fmaf(a[i], b0[i], s0);
      s1 = fmaf(a[i], b1[i], s1);
    }
    s0 = s0 / (1.f + expf(-s0)) * s1;
  } else {
    for (int i = 0; i < K; ++i) s0 = fmaf(a[i], b0[i], s0);
  }
  C[(size_t)row * N + n] = s0;
}

}  // namespace

hipError_t launch_grouped_gemm(const GroupedGemmArgs& a, bool dual, hipStream_t stream) {
  if (a.dtype == MOE_BF16) {
    const int n_tiles = a.N / BN;
    const int64_t m_tiles = (a.max_rows + BM - 1) / BM + std::min(a.G, a.max_rows);
    const int64_t blocks = m_tiles * n_tiles;
    if (blocks <= 0) return hipSuccess;
    if (dual)
      hipLaunchKernelGGL(grouped_gemm_bf16_kernel<true>, dim3((unsigned)blocks), dim3(256), 0, stream,
                         (const uint16_t*)a.A, a.offsets, a.G, a.max_rows, a.N, a.K, (const uint16_t*)a.B0,
                         (const uint16_t*)a.B1, (uint16_t*)a.C, n_tiles);
    else
      hipLaunchKernelGGL(grouped_gemm_bf16_kernel<false>, dim3((unsigned)blocks), dim3(256), 0, stream,
                         (const uint16_t*)a.A, a.offsets, a.G, a.max_rows, a.N, a.K, (const uint16_t*)a.B0,
                         nullptr, (uint16_t*)a.C, n_tiles);
  } else {
    const int64_t blocks = ((int64_t)a.max_rows * a.N + 255) / 256;
    if (blocks <= 0) return hipSuccess;
    if (dual)
      hipLaunchKernelGGL(grouped_gemm_f32_kernel<true>, dim3((unsigned)blocks), dim3(256), 0, stream,
                         (const float*)a.A, a.offsets, a.G, a.max_rows, a.N, a.K, (const float*)a.B0,
                         (const float*)a.B1, (float*)a.C);
    else
      hipLaunchKernelGGL(grouped_gemm_f32_kernel<false>, dim3((unsigned)blocks), dim3(256), 0, stream,
                         (const float*)a.A, a.offsets, a.G, a.max_rows, a.N, a.K, (const float*)a.B0,
                         nullptr, (float*)a.C);
  }
  return hipGetLastError();
}

}  // namespace moe
