// Variable-size grouped GEMM for the SwiGLU experts.
//
// The Residual Stream, "An MoE tiny GPT" listing: expert e runs on its rows h as
// (SiLU(h @ gate[e]) * (h @ up[e])) @ down[e].  ML Interview Notes "Capacity
// factor": dropless routing runs the experts as one variable-size grouped GEMM.
//
// C[r] = A[r] B_g^T for rows r of group g (dual: C = SiLU(A B0_g^T) * (A B1_g^T)).
// A is [rows][K] and B is [N][K], both K-contiguous, so both MFMA operands load
// as 16-byte K-vectors with no transpose.  With a row index, row r of A is read
// from A[a_rows[r]]: the gate/up GEMM then gathers token rows straight from x
// (the dispatch permutation) instead of reading a materialized copy.
//
// bf16 kernel (gfx950):
//  * 256 threads = 4 waves; block tile 256 rows x 256 B-rows (dual: 128 gate rows
//    and the same 128 up rows, so one block produces 256 x 128 of SiLU*up);
//    each wave owns 128 x 128 as 4 x 4 MFMA 32x32x16 tiles (256 fp32 accumulators,
//    so one wave per SIMD).  The largest tile 4 waves can hold, it moves the fewest
//    L2 and LDS bytes per MFMA: with one wave per SIMD the LDS serves about 126
//    B/clk per CU (latency-bound; far more with more waves), and a K step's LDS
//    reads and writes must fit in its MFMA time.
//  * K step 64; global -> registers -> LDS, two LDS stages (147 KB) and two
//    register sets: the 16-byte loads of step kt+2 are issued while step kt is
//    multiplied, because under full load a global round trip takes longer than one
//    step of MFMA work.  One barrier per step, a plain s_barrier (a __syncthreads
//    fence would also wait for the loads in flight), placed before the step's last
//    16-wide k slice so that the next stage's first fragments are read while that
//    slice is multiplied.  LDS rows padded to 144 bytes:
//    conflict-free ds_read_b128.  Within a step, the fragments of the next 16-wide
//    k slice are read while the current one is multiplied, and the step's global
//    loads and LDS writes are spread between the MFMAs (one wave per SIMD: a wave
//    stalled on issuing a burst of loads leaves its MFMA unit idle).  The LDS
//    writes go evenly over the four slices, two chunk pairs each: a stage's first
//    two pairs right after the barrier of the step that finished reading it, the
//    other six in the next step's first three slices.  The LDS pipe then never
//    has more queued than it serves in one slice's MFMA time, and waves stall
//    less on issuing LDS instructions.
//  * MFMA operands swapped (weights as the "A" input), so each lane's accumulators
//    hold 4 consecutive output columns.  The epilogue applies SiLU(gate) * up in
//    fp32, rounds to bf16 (v_cvt_pk_bf16_f32), stages the tile in LDS and stores
//    whole rows.  With K >= 256 the tile is staged in stage 1's memory (single: in
//    two passes of 128 rows) while the next tile's step 0 goes to stage 0, so the
//    loads of its step 2 can be issued before the output stores: gfx950 retires
//    loads and stores through one in-order counter, and a load queued behind
//    128 KB of stores cannot be waited for until they have been written.
//  * Persistent: one block per CU.  Tiles of all groups are enumerated on the
//    device from offsets (no host round trip); each XCD (blocks are dealt
//    round-robin to the 8 XCDs) owns a contiguous run of tiles that its blocks take
//    in turn, and inside an expert the tiles run in bands of up to 8 m-tiles (down
//    the band, then across n), so the tiles an XCD holds at once share their
//    weight slices and their rows through that XCD's L2.
//    The last two K steps of a tile load the first two of the block's next tile,
//    spread over their MFMAs like every other step's loads (issued as a burst in
//    the epilogue they held the waves for a memory round trip), and the gather's
//    row indices are fetched a tile ahead.
//  * Global loads are buffer loads (scalar resource, 32-bit lane offset, the K
//    offset as the scalar offset), which keeps 64-bit per-lane addresses out of the
//    register budget.
#include <algorithm>
#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace moe {
namespace {

// y += v at device scope, result unused: one global_atomic_add_f32 (no return).
__device__ __forceinline__ void atomic_add_f32(float* y, float v) {
  __hip_atomic_fetch_add(y, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

constexpr int BN = 256, BK = 64;
constexpr int LDS_STRIDE = BK + 8;  // bf16 elements per LDS row (16-byte pad)
// Block tile rows by the average rows per group: 128 up to kSmallTileRowsPerGroup,
// 192 up to kMidTileRowsPerGroup, else 256.  A tile's time follows the bytes it
// streams (A rows + weight rows), not its MFMAs, so a tile mostly of padding rows
// costs nearly what a full one does.  Thresholds measured on the Qwen3-30B-A3B
// shape (E = 128, T = 1024..4096, each tile size forced in turn): 128-row tiles
// win up to 100 rows per group and lose from 104, 192-row tiles win up to 156
// and lose from 160 (groups of a few rows over the mean then need two tiles).
constexpr int kSmallTileRowsPerGroup = 100;
constexpr int kMidTileRowsPerGroup = 156;
constexpr int kXcds = 8;
// A chunks among the chunk pairs [lo, hi) of a K step's copy, with NAC A chunks per
// thread (pair i holds A chunk i when i < NAC, and B chunk i).
template <int NAC>
constexpr int a_chunks(int lo, int hi) {
  return (NAC < hi ? NAC : hi) > lo ? (NAC < hi ? NAC : hi) - lo : 0;
}

__device__ __forceinline__ int clamp_off(int v, int max_rows) { return min(max(v, 0), max_rows); }

struct TileScan {
  int incl[256];   // inclusive prefix of per-group m-tile counts
  int start[257];  // clamped group bounds: group g holds rows [start[g], start[g + 1])
  int wave_tot[4];
};


// The rest of a round of a k slice's pattern: its other MPR - 1 MFMAs, each
// after its share of the round's N LDS operations (spread one or two at a time
// between MFMAs rather than bunched after the first).
template <int MASK, int N, int MPR, int S>
__device__ __forceinline__ void lds_slots() {
  if constexpr (S < MPR) {
    constexpr int c = N / (MPR - 1) + (S <= N % (MPR - 1) ? 1 : 0);
    if constexpr (c > 0) __builtin_amdgcn_sched_group_barrier(MASK, c, 0);  // LDS
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                       // MFMA
    lds_slots<MASK, N, MPR, S + 1>();
  }
}

// Block-wide: per-group m-tile counts, their inclusive prefix and the clamped group
// bounds; returns the total.  Groups of at most min_rows rows hold no tiles (the
// weight-streaming kernel takes them).
template <int BM>
__device__ int scan_tiles(const int32_t* __restrict__ offsets, int G, int max_rows, int min_rows, TileScan& s) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  int cnt = 0;
  if (tid < G) {
    const int lo = clamp_off(offsets[tid], max_rows), hi = clamp_off(offsets[tid + 1], max_rows);
    cnt = hi - lo > min_rows ? (hi - lo + BM - 1) / BM : 0;
    s.start[tid] = lo;
    if (tid == G - 1) s.start[G] = hi;
  }
  int v = cnt;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int u = __shfl_up(v, o, 64);
    if (lane >= o) v += u;
  }
  if (lane == 63) s.wave_tot[wave] = v;
  __syncthreads();
  for (int w = 0; w < wave; ++w) v += s.wave_tot[w];
  s.incl[tid] = v;
  __syncthreads();
  return s.incl[255];
}

// Tile t -> group g, first row, end row and n-tile.  Group g owns the tiles
// [excl n_tiles, incl n_tiles) (excl, incl: its m-tile prefix), so a binary search
// for m-tile t / n_tiles on the inclusive prefix finds it.  Inside a group the
// tiles run in bands of kBandRows m-tiles: down the band's m-tiles first, then
// across the n-tiles, then the next band.  The tiles that the CUs of one XCD hold
// at the same time then form a block of a few m-tiles x a few n-tiles, whose A
// rows and weight rows each sit once in that XCD's L2 and are read by several
// tiles (m-tile-major order would stream a fresh weight slice for every tile).
// With 8 rows to a band, an expert of up to 2048 rows is one band, and its weights
// are streamed once: with bands of 4, a fifth m-tile (an expert a little over
// 1024 rows) ran as a band of its own and streamed every weight slice again
// (Mixtral-shaped gate/up 1.695 -> 1.660 ms, qwen3 down 0.484 -> 0.472 ms).
constexpr int kBandRows = 8;
template <int BM>
__device__ void locate(int G, const TileScan& s, int n_tiles, int t, int& g, int& row0, int& row_end, int& nt) {
  const int mt = t / n_tiles;
  int lo = 0, hi = G - 1;
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    if (s.incl[mid] > mt) hi = mid; else lo = mid + 1;
  }
  g = lo;
  const int excl = g > 0 ? s.incl[g - 1] : 0;
  const int u = t - excl * n_tiles;                   // tile index inside the group
  const int band = u / (kBandRows * n_tiles), v = u - band * (kBandRows * n_tiles);
  const int h = min(kBandRows, s.incl[g] - excl - band * kBandRows);  // m-tiles in this band
  nt = v / h;
  row0 = s.start[g] + (band * kBandRows + v % h) * BM;
  row_end = s.start[g + 1];
}


template <bool DUAL, int BM, bool EARLY, bool SCATTER>
__global__ __launch_bounds__(256, 1) void grouped_gemm_bf16_kernel(
    const uint16_t* __restrict__ A, const int32_t* __restrict__ a_rows, int a_nrows,
    const int32_t* __restrict__ offsets, int G, int max_rows, int N, int K, const uint16_t* __restrict__ B0,
    const uint16_t* __restrict__ B1, uint16_t* __restrict__ C, int n_tiles, const int32_t* __restrict__ out_tok,
    const float* __restrict__ out_w, float* __restrict__ y_acc, int T_out, int min_rows) {
  static_assert(!(SCATTER && DUAL), "the scatter form is single");
  constexpr int STAGE = (BM + BN) * LDS_STRIDE;  // bf16 elements per LDS stage (A rows, then B rows)
  constexpr int NAC = BM / 32;                   // A chunks per thread per K step
  // Wave layout.  BM = 256: the 4 waves as 2 x 2, each 128 rows x 128 B rows (dual:
  // 64 gate rows and the same 64 up rows), 4 x 4 fragments of 32.  BM = 128 or 192:
  // the 4 waves split the B rows four ways, each all BM rows x 64 B rows (dual: 32
  // gate and the same 32 up rows), BM / 32 x 2 fragments.
  static_assert(BM == 128 || BM == 192 || BM == 256, "block tile rows");
  constexpr int NAF = BM == 256 ? 4 : BM / 32;  // A fragments per wave
  constexpr int NBF = BM == 256 ? 4 : 2;        // B fragments per wave
  __shared__ __attribute__((aligned(16))) uint16_t lds[2 * STAGE];
  __shared__ TileScan scan;
  __shared__ int tile_rows[256];  // gather: row indices of the tile being set up

  const int total = scan_tiles<BM>(offsets, G, max_rows, min_rows, scan) * n_tiles;
  // Persistent schedule.  Hardware block b runs on XCD b % 8 (blocks are dealt
  // round-robin); XCD x owns the contiguous tile run [x per, (x + 1) per) and its
  // blocks take the run's tiles in turn, so the CUs of an XCD work on neighbouring
  // tiles (the same expert's weights, the same rows) at the same time and share
  // them through that XCD's L2.
  const int xcd = blockIdx.x % kXcds, slot = blockIdx.x / kXcds, nslots = gridDim.x / kXcds;
  const int per = (total + kXcds - 1) / kXcds;
  const int run_end = min((xcd + 1) * per, total);
  int tile = xcd * per + slot;
  if (tile >= run_end) return;

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int wm = wave >> 1, wn = wave & 1;
  const int nk = K / BK;  // even: K % 128 == 0

  // Copy mapping: an operand tile is BM (A) or 256 (B) rows x 8 chunks of 16 bytes;
  // thread tid moves chunks tid + 256 i: row (tid >> 3) + 32 i, k offset 8 (tid & 7).
  // Addresses: block-uniform bases (scalar registers) plus 32-bit byte offsets per
  // thread (the host checks that every operand fits in 4 GiB).
  const int crow = tid >> 3, ccol = 8 * (tid & 7);
  // Loads go through buffer resources (a scalar base and size) with a 32-bit lane
  // offset and the block-uniform K offset as the scalar offset: no 64-bit address
  // per lane is ever formed (the compiler would otherwise keep 16 of them live).
  const __amdgpu_buffer_rsrc_t rsrc_a =
      __builtin_amdgcn_make_buffer_rsrc((void*)A, (short)0, (int)((uint32_t)a_nrows * (uint32_t)K * 2u), kBufferFlags);
  __amdgpu_buffer_rsrc_t rsrc_b0, rsrc_b1;
  uint32_t a_off8[NAC];
  // B chunk i of this thread: row (first row of the tile) + crow + 32 (i & b_mask),
  // i.e. the lane offset b_lane plus the block-uniform step (i & b_mask) * b_step.
  const uint32_t b_lane = ((uint32_t)crow * (uint32_t)K + ccol) * 2u;
  const uint32_t b_step = 32u * (uint32_t)K * 2u;
  int b_mask;
  int row0, row_end, n0;
  int pre_row = 0;
  // B rows of a tile: dual -> gate rows [n0, n0+128) then up rows [n0, n0+128);
  // single -> rows [n0, n0+256), or [n0, n0+128) twice for a last tile of 128
  // columns (the columns past N are not stored).
  auto setup = [&](int t) {
    int g, nt;
    locate<BM>(G, scan, n_tiles, t, g, row0, row_end, nt);
    g = __builtin_amdgcn_readfirstlane(g);  // block-uniform: keep the bases in scalar registers
    row0 = __builtin_amdgcn_readfirstlane(row0);
    row_end = __builtin_amdgcn_readfirstlane(row_end);
    n0 = DUAL ? nt * (BN / 2) : nt * BN;
    const int b_bytes = (int)((uint32_t)(N - n0) * (uint32_t)K * 2u);  // rows [n0, N) of the expert
    rsrc_b0 = __builtin_amdgcn_make_buffer_rsrc((void*)(B0 + ((size_t)g * N + n0) * K), (short)0, b_bytes,
                                                kBufferFlags);
    rsrc_b1 = DUAL ? __builtin_amdgcn_make_buffer_rsrc((void*)(B1 + ((size_t)g * N + n0) * K), (short)0, b_bytes,
                                                       kBufferFlags)
                   : rsrc_b0;
    b_mask = (DUAL || n0 + BN > N) ? 3 : 7;
    int arow[NAC];
    if (a_rows != nullptr) {
      // thread tid fetched the index of the tile's row tid; each thread needs those
      // of its rows crow + 32 i
      tile_rows[tid] = pre_row;
      lds_barrier();
#pragma unroll
      for (int i = 0; i < NAC; ++i) arow[i] = min(max(tile_rows[crow + 32 * i], 0), a_nrows - 1);
    } else {
#pragma unroll
      for (int i = 0; i < NAC; ++i) arow[i] = min(row0 + crow + 32 * i, row_end - 1);
    }
#pragma unroll
    for (int i = 0; i < NAC; ++i) a_off8[i] = ((uint32_t)arow[i] * (uint32_t)K + ccol) * 2u;
  };
  // Gather: thread tid loads the row index of tile t's row tid, a tile ahead of
  // setup(t), so that setup issues no load of its own (one register across the K
  // loop; setup shares the indices through LDS).
  auto fetch_rows = [&](int t) {
    if (a_rows == nullptr) return;
    int g, nt, r0, re;
    locate<BM>(G, scan, n_tiles, t, g, r0, re, nt);
    pre_row = a_rows[min(r0 + tid, re - 1)];
  };

  // Two register sets: the loads of K step kt+2 are issued while step kt is
  // multiplied and step kt+1 is still in flight.
  u32x4 ra[2][NAC], rb[2][8];
  // Quarter q of a K step's loads: A and B chunks 2q and 2q + 1.
  auto load_part = [&](auto set, int k0, int q) {
    constexpr int S = decltype(set)::value;
    const int kb = k0 * 2;
#pragma unroll
    for (int i = 2 * q; i < 2 * q + 2; ++i) {
      if (i < NAC)
        ra[S][i % NAC] =
            __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rsrc_a, (int)a_off8[i % NAC], kb, 0));
      rb[S][i] = __builtin_bit_cast(
          u32x4, __builtin_amdgcn_raw_buffer_load_b128(DUAL && i >= 4 ? rsrc_b1 : rsrc_b0, (int)b_lane,
                                                       kb + (int)((i & b_mask) * b_step), 0));
    }
  };
  auto load = [&](auto set, int k0) {
#pragma unroll
    for (int q = 0; q < 4; ++q) load_part(set, k0, q);
  };
  // LDS writes of chunks i in [lo, hi) (A chunk i if i < NAC, and B chunk i), in
  // the order load_part issued them.
  auto store_range = [&](auto set, int stage, int lo, int hi) {
    constexpr int S = decltype(set)::value;
    uint16_t* sa = lds + stage * STAGE;
    uint16_t* sb = sa + BM * LDS_STRIDE;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      if (i < lo || i >= hi) continue;
      if (i < NAC) st16(sa + (crow + 32 * i) * LDS_STRIDE + ccol, ra[S][i % NAC]);
      st16(sb + (crow + 32 * i) * LDS_STRIDE + ccol, rb[S][i]);
    }
  };
  auto store = [&](auto set, int stage) { store_range(set, stage, 0, 8); };

  f32x16 acc[NAF][NBF];
  // Fragment offsets inside a stage: A rows wm*128 + 32 i; B rows per the layout above.
  const int frow = lane & 31, half = lane >> 5, fk = 8 * half;
  int a_off[NAF], b_off[NBF];
#pragma unroll
  for (int i = 0; i < NAF; ++i) a_off[i] = ((BM == 256 ? wm * 128 : 0) + i * 32 + frow) * LDS_STRIDE + fk;
#pragma unroll
  for (int j = 0; j < NBF; ++j) {
    // BM = 256, dual: fragments 0,1 = gate rows wn*64 + {0,32}; 2,3 = the same rows of up.
    // BM = 128, dual: fragment 0 = gate rows 32 wave .., 1 = the same rows of up.
    const int brow = BM == 256 ? (DUAL ? (j >> 1) * (BN / 2) + wn * 64 + (j & 1) * 32 : wn * 128 + j * 32)
                               : (DUAL ? j * (BN / 2) + wave * 32 : wave * 64 + j * 32);
    b_off[j] = (BM + brow + frow) * LDS_STRIDE + fk;
  }
  bf16x8 fa[2][NAF], fb[2][NBF];
  auto read_frags = [&](const uint16_t* st, int ks, int buf) {
#pragma unroll
    for (int i = 0; i < NAF; ++i) fa[buf][i] = as_bf16x8(ld16(st + a_off[i] + ks));
#pragma unroll
    for (int j = 0; j < NBF; ++j) fb[buf][j] = as_bf16x8(ld16(st + b_off[j] + ks));
  };
  auto mma = [&](int buf) {
#pragma unroll
    for (int i = 0; i < NAF; ++i)
#pragma unroll
      for (int j = 0; j < NBF; ++j) acc[i][j] = mfma32x32x16(fb[buf][j], fa[buf][i], acc[i][j]);
  };

  using R0 = std::integral_constant<int, 0>;
  using R1 = std::integral_constant<int, 1>;
  // Step kt: stage kt & 1 is in LDS, register set kt & 1 is free again, set
  // (kt + 1) & 1 holds step kt+1 in flight.  Every step loads K offset kn into its
  // own set: step kt+2 of this tile, or in the last two steps, steps 0 and 1 of
  // the block's next tile (whose first stage is then in flight through this
  // tile's epilogue, not issued as a burst in it).  Modes: kFull also stores step
  // kt+1 to the other stage; kPre (step nk-2) stores but writes no pair of the
  // next tile; kPreLast (step nk-1) stores nothing and leaves the final barrier to
  // the epilogue.  No step has a branch (a join would make the compiler's wait
  // counts drain the loads just issued).
  constexpr int kFull = 0, kPre = 1, kPreLast = 2, kFirst = 3;
  auto step = [&](auto set, int kn, auto mode) {
    constexpr int S = decltype(set)::value;
    constexpr int MODE = decltype(mode)::value;
    using Other = std::integral_constant<int, S ^ 1>;
    const uint16_t* st = lds + S * STAGE;
    // The global loads and LDS traffic are spread over the MFMAs: a wave that
    // issued its 16 loads back to back would stall on the vector memory queue
    // with its MFMA unit idle.  Per k slice (fenced, so that fragment lifetimes
    // stay one slice long): 4 loads, the 8 fragment reads of the next slice and
    // 4 LDS writes, in 4 rounds of a load and the round's MFMAs with its LDS
    // operations one or two between each pair of MFMAs (bunched three at a time
    // they ran about 1% slower).  The step's barrier sits before the last slice.
    auto slice_pattern = [&](auto lds_mask, auto lds_n) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        if constexpr (MODE != kFirst) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);  // global load
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
        lds_slots<decltype(lds_mask)::value, decltype(lds_n)::value, NAF * NBF / 4, 1>();
      }
    };
    using DsRead = std::integral_constant<int, 0x100>;
    using AnyDs = std::integral_constant<int, 0x080>;
    using Two = std::integral_constant<int, 2>;
    // LDS writes, two chunk pairs per slice: step kt+1's pairs 2..7 (register set
    // Other, loaded in step kt-1) in the first three slices, and step kt+2's pairs
    // 0 and 1 (this step's own set, loaded in the first slice) after the barrier,
    // into this step's stage, which every wave has then finished reading.  Each
    // load thus has three slices to land, and no slice asks more of the LDS than
    // it serves in that slice's MFMA time.
    constexpr int kW[4] = {2 + a_chunks<NAC>(2, 4), 2 + a_chunks<NAC>(4, 6), 2 + a_chunks<NAC>(6, 8),
                           2 + a_chunks<NAC>(0, 2)};
    using Ops0 = std::integral_constant<int, (NAF + NBF + kW[0] + 3) / 4>;  // LDS reads + writes per MFMA group
    using Ops1 = std::integral_constant<int, (NAF + NBF + kW[1] + 3) / 4>;
    using Ops2 = std::integral_constant<int, (NAF + NBF + kW[2] + 3) / 4>;
    using Ops3 = std::integral_constant<int, (NAF + NBF + kW[3] + 3) / 4>;
    read_frags(st, 16, 1);
    if constexpr (MODE != kFirst) load_part(set, kn, 0);
    if constexpr (MODE != kPreLast) store_range(Other{}, S ^ 1, 2, 4);
    mma(0);
    if constexpr (MODE != kPreLast) slice_pattern(AnyDs{}, Ops0{}); else slice_pattern(DsRead{}, Two{});
    __builtin_amdgcn_sched_barrier(0);
    read_frags(st, 32, 0);
    if constexpr (MODE != kFirst) load_part(set, kn, 1);
    if constexpr (MODE != kPreLast) store_range(Other{}, S ^ 1, 4, 6);
    mma(1);
    if constexpr (MODE != kPreLast) slice_pattern(AnyDs{}, Ops1{}); else slice_pattern(DsRead{}, Two{});
    __builtin_amdgcn_sched_barrier(0);
    read_frags(st, 48, 1);
    if constexpr (MODE != kFirst) load_part(set, kn, 2);
    if constexpr (MODE != kPreLast) store_range(Other{}, S ^ 1, 6, 8);
    mma(0);
    if constexpr (MODE != kPreLast) slice_pattern(AnyDs{}, Ops2{}); else slice_pattern(DsRead{}, Two{});
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (MODE != kPreLast) {
      // Every wave has read its last fragments of this stage and written the next
      // one: after the barrier the next stage's first fragments are read while the
      // last slice is multiplied, so no wave waits on LDS at the step boundary.
      lds_barrier();
      read_frags(lds + (S ^ 1) * STAGE, 0, 0);
    }
    if constexpr (MODE != kFirst) load_part(set, kn, 3);
    if constexpr (MODE == kFull || MODE == kFirst) store_range(set, S, 0, 2);
    mma(1);
    if constexpr (MODE == kFull || MODE == kFirst) slice_pattern(AnyDs{}, Ops3{});
    else slice_pattern(DsRead{}, std::integral_constant<int, MODE != kPreLast ? 2 : 0>{});
  };

  using Full = std::integral_constant<int, kFull>;
  using Pre = std::integral_constant<int, kPre>;
  using PreLast = std::integral_constant<int, kPreLast>;
  using First = std::integral_constant<int, kFirst>;
  constexpr int TN = DUAL ? BN / 2 : BN;  // output columns of a block tile
  constexpr int OST = TN + 8;             // bf16 per LDS output row
  // Output staging.  EARLY: the tile goes through stage 1's memory, in one pass
  // (dual) or two passes of half the rows (single), while stage 0 takes the next
  // tile's step 0; otherwise it takes both stages in one pass.
  constexpr int PASSES = EARLY && !DUAL ? 2 : 1;
  constexpr int PROWS = BM / PASSES;      // output rows per pass
  static_assert(PROWS * OST <= (EARLY ? 1 : 2) * STAGE, "output tile must fit in the stage memory");

  // The row indices of the block's next tile are fetched before the operand
  // loads of the steps that follow, so that the K loop's wait counts only see
  // operand loads behind them (the block's last tile fetches its own again).
  auto after = [&](int t) { return t + nslots < run_end ? t + nslots : t; };
  fetch_rows(tile);
  setup(tile);
  fetch_rows(after(tile));
  load(R0{}, 0);
  load(R1{}, BK);
  if constexpr (EARLY) {
    // every tile starts with step 0 in stage 0 and step 2 in flight in set 0
    store(R0{}, 0);
    load(R0{}, 2 * BK);
  }
  for (;;) {
    // The stage memory is free (the previous tile's epilogue is done with it).
    // EARLY: stage 0 already holds step 0, written before this barrier, which
    // also makes it visible; step 1's first pairs go to stage 1 after it, and
    // are read only after the barrier inside step 0.
    lds_barrier();
    if constexpr (!EARLY) store(R0{}, 0);
    store_range(R1{}, 1, 0, 2);  // step 1's first pairs, as a step's last slice would have
#pragma unroll
    for (int i = 0; i < NAF; ++i)
#pragma unroll
      for (int j = 0; j < NBF; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;
    if constexpr (!EARLY) lds_barrier();
    read_frags(lds, 0, 0);
    if constexpr (EARLY) {
      // step 2's loads went out before the previous tile's output stores (the
      // vector memory counter retires in issue order, so a load issued behind
      // the stores could not be waited for before they completed)
      step(R0{}, 0, First{});
      step(R1{}, 3 * BK, Full{});
    }
    for (int kt = EARLY ? 2 : 0; kt < nk - 2; kt += 2) {
      step(R0{}, (kt + 2) * BK, Full{});
      step(R1{}, (kt + 3) * BK, Full{});
    }
    // The last two steps load the first two of the block's next tile (the last
    // tile re-loads itself: no load sits under a branch).
    const int e_row0 = row0, e_row_end = row_end, e_n0 = n0;
    const int next = tile + nslots;
    const bool more = next < run_end;
    setup(more ? next : tile);
    fetch_rows(after(more ? next : tile));
    step(R0{}, 0, Pre{});
    step(R1{}, BK, PreLast{});

    // Epilogue through LDS.  acc[i][j] element r of lane l: output row (m) = 32 i +
    // l % 32 of the wave's rows, output column (n) = 8 (r / 4) + 4 (l / 32) + r % 4 of
    // fragment j.  Stored straight to memory, each store instruction would touch 32
    // rows with 16 bytes apiece; instead the block's bf16 tile is written to LDS
    // (row-major, rows padded by 16 bytes) and then stored as whole rows, 16 bytes
    // per lane, so each instruction writes 8 full 128-byte lines.
    uint16_t* ot = EARLY ? lds + STAGE : lds;
    // Pass p writes fragments [p NAF / PASSES, (p + 1) NAF / PASSES) of every wave
    // to LDS: with two passes and BM = 256, tile rows [64 p, 64 p + 64) (waves
    // wm = 0) and [128 + 64 p, 192 + 64 p) (wm = 1) as LDS rows 0..127; with BM <
    // 256, tile rows [p PROWS, (p + 1) PROWS).
    constexpr int FPP = NAF / PASSES;  // fragments per wave and pass
    auto write_out = [&](auto pass) {
      constexpr int P = decltype(pass)::value;
#pragma unroll
      for (int i = P * FPP; i < (P + 1) * FPP; ++i) {
        const int r = (BM == 256 ? wm * (128 / PASSES) : 0) + (i - P * FPP) * 32 + frow;
#pragma unroll
        for (int j = 0; j < (DUAL ? NBF / 2 : NBF); ++j)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int c = (BM == 256 ? (DUAL ? wn * 64 : wn * 128) : (DUAL ? wave * 32 : wave * 64)) + j * 32 +
                          8 * q + 4 * half;
            float v[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const float x = acc[i][j][4 * q + e];
              v[e] = DUAL ? silu_bf16out(x) * acc[i][j + NBF / 2][4 * q + e] : x;
            }
            *reinterpret_cast<uint2*>(ot + r * OST + c) =
                make_uint2(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]));
          }
      }
    };
    // Thread tid stores 16-byte chunk tid % CPR of rows tid / CPR + RSTEP u of a
    // pass.  The stores are buffer stores whose range ends at the tile's last row
    // of the group; a chunk past that row, or (single) past column N, lies beyond
    // the range and is dropped, so the loop has no branch.  Its LDS reads go out
    // in groups of 8 ahead of their stores: one read, wait and store at a time
    // paid the LDS latency per chunk (about 5k cycles of a down tile's 128 KB).
    constexpr int CPR = TN / 8;             // 16-byte chunks per output row
    constexpr int RSTEP = 256 / CPR;        // rows between one thread's chunks
    constexpr int NST = PROWS * CPR / 256;  // chunks per thread and pass
    const int ncols = DUAL ? TN : min(TN, N - e_n0);
    const int sr = tid / CPR, sc = 8 * (tid % CPR);
    const uint32_t c_off = sc < ncols ? ((uint32_t)sr * (uint32_t)N + (uint32_t)(e_n0 + sc)) * 2u : 0x80000000u;
    const uint32_t c_step = (uint32_t)RSTEP * (uint32_t)N * 2u;
    const uint16_t* os = ot + sr * OST + sc;
    const int e_rows = min(e_row_end - e_row0, BM);
    const __amdgpu_buffer_rsrc_t rsrc_c = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(C + (size_t)e_row0 * N), (short)0, (int)((uint32_t)e_rows * (uint32_t)N * 2u), kBufferFlags);
    // LDS row lr of pass p is tile row lr + p PROWS, or with two passes and BM = 256,
    // 128 (lr / 64) + 64 p + lr % 64.
    auto store_out = [&](auto pass) {
      constexpr int P = decltype(pass)::value;
      constexpr int HALF = 64 / RSTEP;  // chunks per thread in LDS rows 0..63
#pragma unroll
      for (int u0 = 0; u0 < NST; u0 += 8) {
        u32x4 v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u)
          if (u0 + u < NST) v[u] = ld16(os + (u0 + u) * RSTEP * OST);
#pragma unroll
        for (int u = 0; u < 8; ++u)
          if (u0 + u < NST) {
            const int trow = BM == 256 && PASSES == 2 ? 64 * P + ((u0 + u) >= HALF ? 64 : 0) : P * PROWS;
            __builtin_amdgcn_raw_buffer_store_b128(
                v[u], rsrc_c, (int)(c_off + (uint32_t)(u0 + u) * c_step + (uint32_t)trow * (uint32_t)N * 2u), 0, 0);
          }
      }
    };
    // Scatter form: wave w takes LDS rows w, w + 4, ... of a pass; lane l < RPW
    // fetches the token and weight of the wave's row l, which every lane then
    // reads as scalars.  A row's columns go out as fp32 atomic adds with lane l
    // on columns l + 64 c, so that one instruction covers 256 contiguous bytes.
    auto scatter_out = [&](auto pass) {
      constexpr int P = decltype(pass)::value;
      constexpr int RPW = PROWS / 4;  // rows per wave and pass
      static_assert(RPW <= 64, "a row per lane");
      const int wv = __builtin_amdgcn_readfirstlane(wave);
      const int lr_l = wv + 4 * min(lane, RPW - 1);
      const int trow_l = BM == 256 && PASSES == 2 ? (lr_l >= 64 ? 128 : 0) + 64 * P + (lr_l & 63) : lr_l + P * PROWS;
      int tok_l = -1;
      float w_l = 0.f;
      if (lane < RPW && trow_l < e_rows) {
        tok_l = out_tok[e_row0 + trow_l];
        w_l = out_w[e_row0 + trow_l];
      }
#pragma unroll
      for (int i = 0; i < RPW; ++i) {
        const int tok = __builtin_amdgcn_readlane(tok_l, i);
        if (tok < 0 || tok >= T_out) continue;  // past the group, padding, or not a token
        const float w = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(w_l), i));
        const uint16_t* orow = ot + (wv + 4 * i) * OST;
        float* yr = y_acc + (size_t)tok * N + e_n0;
#pragma unroll
        for (int c = 0; c < TN / 64; ++c) {
          const int col = lane + 64 * c;
          if (col < ncols) atomic_add_f32(yr + col, w * bf16_to_f32(orow[col]));
        }
      }
    };
    auto emit = [&](auto pass) {
      if constexpr (SCATTER) scatter_out(pass); else store_out(pass);
    };
    using P0 = std::integral_constant<int, 0>;
    using P1 = std::integral_constant<int, 1>;
    // The next tile's step 0 goes to stage 0 and its step 2 is loaded ahead of
    // the stores; in one pass (dual), ahead of the SiLU*up conversion as well
    // (gate/up 1% faster; the two-pass single form measured 0.5-0.8% slower so).
    lds_barrier();  // every wave is done with the last stage
    if constexpr (EARLY && PASSES == 1) {
      store(R0{}, 0);
      load(R0{}, 2 * BK);
    }
    write_out(P0{});
    if constexpr (EARLY && PASSES == 2) store(R0{}, 0);
    lds_barrier();
    if constexpr (EARLY && PASSES == 2) load(R0{}, 2 * BK);
    emit(P0{});
    if constexpr (PASSES == 2) {
      lds_barrier();  // every wave has read the first pass
      write_out(P1{});
      lds_barrier();
      emit(P1{});
    }
    if (!more) break;
    tile = next;
  }
}

// Skinny variant for groups of a few rows (decode: about T k / E rows per expert).
// The weights are streamed once from HBM straight into MFMA operands (no LDS): one
// block per (group, 64 B rows; single: 128), each wave two 16-row B sets (dual: 16
// gate rows and the same 16 up rows; single: 32 consecutive rows) against 16-row
// token tiles, v_mfma_f32_16x16x32_bf16 with the weights as the "A" operand.  In
// k-step u of a 128-wide K chunk, lane group q = l / 16 holds k values
// 32 u + 8 q .. 32 u + 8 q + 7 of its row (the instruction's own order), so each
// 16-byte load instruction reads 64 contiguous bytes of 16 rows.  Two chunks are
// in flight per wave.  A weight pass serves TT 16-row token tiles (the launcher uses
// one, and gives groups of more rows to the tiled kernel).
constexpr int SK_ROWS = 16;   // B rows per MFMA tile
// B rows per block: dual, 4 waves x 16 rows (each with its gate and up rows);
// single, 4 waves x 32 rows (two 16-row sets).
__host__ __device__ constexpr int sk_bn(bool dual) { return dual ? 64 : 128; }
constexpr int SK_CHUNK = 128; // K per chunk
constexpr int64_t kSliceDealBytes = 16ll << 20;  // per expert weight matrix, for slice dealing

template <bool DUAL, bool GATHER, int TT, bool SCATTER = false>
__global__ __launch_bounds__(256) void grouped_gemm_skinny_kernel(
    const uint16_t* __restrict__ A, const int32_t* __restrict__ a_rows, int a_nrows,
    const int32_t* __restrict__ offsets, int G, int max_rows, int N, int K, const uint16_t* __restrict__ B0,
    const uint16_t* __restrict__ B1, uint16_t* __restrict__ C, const int32_t* __restrict__ out_tok,
    const float* __restrict__ out_w, float* __restrict__ y_acc, int T_out, int big_rows, int slice_deal) {
  static_assert(!(SCATTER && DUAL), "the scatter form is single");
  const int nblk_n = N / sk_bn(DUAL);
  // Each XCD streams one contiguous eighth of the weights (whole experts), or with
  // slice_deal (nblk_n a multiple of 8) one contiguous eighth of every expert's B
  // rows: then every touched expert loads the 8 XCDs evenly, however few are
  // touched, and for large experts the pages an XCD touches are as few.
  int g, nb;
  if (slice_deal) {
    const int per = nblk_n >> 3, slot = (int)blockIdx.x >> 3;
    g = slot / per;
    nb = ((int)blockIdx.x & 7) * per + slot % per;
  } else {
    const int lb = xcd_contiguous_block();
    g = lb / nblk_n;
    nb = lb % nblk_n;
  }
  const int lo = clamp_off(offsets[g], max_rows), hi = clamp_off(offsets[g + 1], max_rows);
  // empty groups, and groups of more than big_rows rows (the tiled kernel takes those)
  if (hi <= lo || hi - lo > big_rows) return;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int r16 = lane & 15, q = lane >> 4;
  const int n_base = nb * sk_bn(DUAL) + wave * (DUAL ? SK_ROWS : 2 * SK_ROWS);
  // the two B row sets: dual, gate and up rows n_base ..; single, rows n_base .. and
  // n_base + 16 ..
  const uint16_t* bg = B0 + ((size_t)g * N + n_base + r16) * K + 8 * q;
  const uint16_t* bu = DUAL ? B1 + ((size_t)g * N + n_base + r16) * K + 8 * q : bg + (size_t)SK_ROWS * K;
  const int nchunks = K / SK_CHUNK;
  constexpr int NB = 2;

  // Register sets 0 and 1 hold chunks 2p and 2p + 1, each issued as weights then
  // tokens, so that waiting for one set leaves the other in flight (the vector
  // memory counter retires in order).  The loop prefetches the next pair while a
  // pair is multiplied; the last pair is peeled off, so no load sits under a branch
  // and none is wasted (an odd chunk count re-loads the last chunk once, as a
  // second chunk multiplied with zeroed token values).  Each weight chunk serves
  // TT 16-row token tiles (rows past the group re-read its last row; their results
  // are not stored).
  u32x4 wa[2][NB][4], ta[2][TT][4];
  const uint16_t* ap[TT];
  auto load_w = [&](int buf, int c) {
    const int k0 = min(c, nchunks - 1) * SK_CHUNK;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      wa[buf][0][u] = ld16(bg + k0 + 32 * u);
      wa[buf][1][u] = ld16(bu + k0 + 32 * u);
    }
  };
  auto load_x = [&](int buf, int c) {
    const int k0 = min(c, nchunks - 1) * SK_CHUNK;
#pragma unroll
    for (int tt = 0; tt < TT; ++tt)
#pragma unroll
      for (int u = 0; u < 4; ++u) ta[buf][tt][u] = ld16(ap[tt] + k0 + 32 * u);
  };
  const int npairs = (nchunks + 1) / 2;
  for (int t0 = lo; t0 < hi; t0 += 16 * TT) {
    // an opaque zero keeps the first loads inside this loop (hoisted, they would be
    // drained by the first wait)
    int z;
    asm volatile("s_mov_b32 %0, 0" : "=s"(z));
    int m[TT], mg[TT];
#pragma unroll
    for (int tt = 0; tt < TT; ++tt) {
      m[tt] = min(t0 + 16 * tt + r16, hi - 1);
      mg[tt] = 0;
      if (GATHER) mg[tt] = a_rows[m[tt]];
    }
    load_w(0, z);
#pragma unroll
    for (int tt = 0; tt < TT; ++tt) {
      if (GATHER) m[tt] = min(max(mg[tt], 0), a_nrows - 1);
      ap[tt] = A + (size_t)m[tt] * K + 8 * q;
    }
    // issue order w0, x0, w1, x1 as in the loop (the scheduler would otherwise
    // reorder or sink the loads)
    __builtin_amdgcn_sched_barrier(0);
    load_x(0, z);
    int z1 = z + 1;
#pragma unroll
    for (int tt = 0; tt < TT; ++tt) asm volatile("" : "+s"(z1) : "v"(m[tt]));  // w1 after x0
    __builtin_amdgcn_sched_barrier(0);
    load_w(1, z1);
    load_x(1, z1);
    __builtin_amdgcn_sched_barrier(0);
    f32x4 acc[TT][NB];
#pragma unroll
    for (int tt = 0; tt < TT; ++tt)
#pragma unroll
      for (int b = 0; b < NB; ++b) acc[tt][b] = f32x4{0.f, 0.f, 0.f, 0.f};
    auto mma = [&](int buf, uint32_t keep) {
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int tt = 0; tt < TT; ++tt)
#pragma unroll
          for (int b = 0; b < NB; ++b)
            acc[tt][b] = mfma16x16x32(as_bf16x8(wa[buf][b][u]), as_bf16x8(ta[buf][tt][u] & keep), acc[tt][b]);
    };
    for (int p = 0; p + 1 < npairs; ++p) {
      mma(0, ~0u);
      __builtin_amdgcn_sched_barrier(0);
      load_w(0, 2 * p + 2);
      load_x(0, 2 * p + 2);
      __builtin_amdgcn_sched_barrier(0);
      mma(1, ~0u);
      __builtin_amdgcn_sched_barrier(0);
      load_w(1, 2 * p + 3);
      load_x(1, 2 * p + 3);
      __builtin_amdgcn_sched_barrier(0);
    }
    mma(0, ~0u);
    mma(1, 2 * npairs <= nchunks ? ~0u : 0u);  // uniform
    // acc[tt][b] element i of lane l: B row 4 (l / 16) + i of set b, token row
    // t0 + 16 tt + l % 16.
#pragma unroll
    for (int tt = 0; tt < TT; ++tt) {
      const int row = t0 + 16 * tt + r16;
      if (row < hi) {
        uint16_t* crow = C + (size_t)row * N + n_base + 4 * q;
        if (DUAL) {
          float v[4];
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const float x = acc[tt][0][i];
            v[i] = silu_bf16out(x) * acc[tt][1][i];
          }
          *reinterpret_cast<uint2*>(crow) = make_uint2(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]));
        } else if (SCATTER) {
          // the product rounded to bf16, as C would hold it, times the row's weight
          const int tok = out_tok[row];
          if (tok >= 0 && tok < T_out) {
            const float w = out_w[row];
            float* yr = y_acc + (size_t)tok * N + n_base + 4 * q;
#pragma unroll
            for (int b = 0; b < 2; ++b)
#pragma unroll
              for (int i = 0; i < 4; i += 2) {
                const uint32_t pk = pack_bf16x2(acc[tt][b][i], acc[tt][b][i + 1]);
                atomic_add_f32(yr + b * SK_ROWS + i, w * __uint_as_float(pk << 16));
                atomic_add_f32(yr + b * SK_ROWS + i + 1, w * __uint_as_float(pk & 0xffff0000u));
              }
          }
        } else {
#pragma unroll
          for (int b = 0; b < 2; ++b)
            *reinterpret_cast<uint2*>(crow + b * SK_ROWS) =
                make_uint2(pack_bf16x2(acc[tt][b][0], acc[tt][b][1]), pack_bf16x2(acc[tt][b][2], acc[tt][b][3]));
        }
      }
    }
  }
}

// fp32 path: one thread per output element, plain K loop.
template <bool DUAL>
__global__ __launch_bounds__(256) void grouped_gemm_f32_kernel(const float* __restrict__ A,
                                                                const int32_t* __restrict__ a_rows, int a_nrows,
                                                                const int32_t* __restrict__ offsets, int G,
                                                                int max_rows, int N, int K,
                                                                const float* __restrict__ B0,
                                                                const float* __restrict__ B1,
                                                                float* __restrict__ C,
                                                                const int32_t* __restrict__ out_tok,
                                                                const float* __restrict__ out_w,
                                                                float* __restrict__ y_acc, int T_out) {
  const int64_t id = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (id >= (int64_t)max_rows * N) return;
  const int row = (int)(id / N), n = (int)(id % N);
  int g = -1;
  for (int q = 0; q < G; ++q) {
    const int lo = clamp_off(offsets[q], max_rows), hi = clamp_off(offsets[q + 1], max_rows);
    if (row >= lo && row < hi) { g = q; break; }
  }
  if (g < 0) return;
  const int ar = a_rows != nullptr ? min(max(a_rows[row], 0), a_nrows - 1) : row;
  const float* a = A + (size_t)ar * K;
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
  if (y_acc != nullptr) {
    const int tok = out_tok[row];
    if (tok >= 0 && tok < T_out) atomic_add_f32(y_acc + (size_t)tok * N + n, out_w[row] * s0);
  } else {
    C[(size_t)row * N + n] = s0;
  }
}

}  // namespace

// Blocks of the persistent kernel: the current device's compute units, rounded
// down to a multiple of the XCD count (256 on MI355X), cached per device.
int persistent_blocks() {
  static int cached[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cached[dev] == 0) {
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < kXcds)
      cus = 256;
    cached[dev] = cus / kXcds * kXcds;
  }
  return cached[dev];
}

namespace {

// The tiled kernel with bm-row tiles over the groups of more than min_rows rows.
hipError_t launch_tiled(const GroupedGemmArgs& a, bool dual, int bm, int min_rows, hipStream_t stream) {
  const bool scatter = a.y_acc != nullptr;
  const int n_tiles = dual ? a.N / (BN / 2) : (a.N + BN - 1) / BN;
  // m-tiles: at most ceil(rows / bm) + 1 per group that holds tiles, and at most
  // max_rows / (min_rows + 1) groups hold more than min_rows rows
  const int64_t groups = std::min<int64_t>(a.G, (int64_t)a.max_rows / ((int64_t)min_rows + 1));
  const int64_t m_tiles = (a.max_rows + bm - 1) / bm + groups;
  // persistent grid: one block per CU (the LDS stages take a CU), a multiple of
  // the 8 XCDs, no more than the tiles there can be
  const int64_t max_tiles = m_tiles * n_tiles;
  if (max_tiles <= 0) return hipSuccess;
  const int64_t blocks = std::min<int64_t>(persistent_blocks(), (max_tiles + kXcds - 1) / kXcds * kXcds);
  // Step 2 of a tile can be loaded in the previous tile's epilogue when there is one (K >= 256).
  const bool early = a.K >= 4 * BK;
#define MOE_TILED_E(D, M, E, S)                                                                               \
  hipLaunchKernelGGL((grouped_gemm_bf16_kernel<D, M, E, S>), dim3((unsigned)blocks), dim3(256), 0, stream,   \
                     (const uint16_t*)a.A, a.a_rows, a.a_nrows, a.offsets, a.G, a.max_rows, a.N, a.K,         \
                     (const uint16_t*)a.B0, D ? (const uint16_t*)a.B1 : nullptr, (uint16_t*)a.C, n_tiles,     \
                     a.out_tok, a.out_w, a.y_acc, a.T, min_rows)
#define MOE_TILED(D, M)                                     \
  do {                                                      \
    if (early) {                                            \
      if (D) MOE_TILED_E(D, M, true, false);                \
      else if (scatter) MOE_TILED_E(false, M, true, true);  \
      else MOE_TILED_E(false, M, true, false);              \
    } else {                                                \
      if (D) MOE_TILED_E(D, M, false, false);               \
      else if (scatter) MOE_TILED_E(false, M, false, true); \
      else MOE_TILED_E(false, M, false, false);             \
    }                                                       \
  } while (0)
  if (bm == 128) {
    if (dual) MOE_TILED(true, 128); else MOE_TILED(false, 128);
  } else if (bm == 192) {
    if (dual) MOE_TILED(true, 192); else MOE_TILED(false, 192);
  } else {
    if (dual) MOE_TILED(true, 256); else MOE_TILED(false, 256);
  }
#undef MOE_TILED
#undef MOE_TILED_E
  return hipGetLastError();
}

}  // namespace

hipError_t launch_grouped_gemm(const GroupedGemmArgs& a, bool dual, hipStream_t stream) {
  const bool scatter = a.y_acc != nullptr;
  if (scatter && (dual || a.a_rows != nullptr)) return hipErrorInvalidValue;
  if (a.dtype == MOE_BF16 && (int64_t)a.max_rows <= (int64_t)kSkinnyRowsPerGroup * a.G) {
    // Few rows per group on average: the weight-streaming kernel takes the groups
    // of up to 16 rows (one 16-row token tile, one pass over their weights), and
    // the tiled kernel, with 128-row tiles, the larger ones.  Group sizes are known
    // only on the device, so both launches read the offsets; the second is issued
    // when some group can exceed 16 rows.  A skewed routing (a hot expert holding
    // most tokens) would otherwise stream the hot expert's weights once per 16 of
    // its rows, one pass after another in the same blocks.
    const int big = SK_ROWS;
    const int nblk_n = a.N / sk_bn(dual);
    // experts of 16 MB or more per weight matrix: deal each one's B rows to the XCDs
    const int slice_deal = nblk_n % kXcds == 0 && (int64_t)a.N * a.K * 2 >= (int64_t)kSliceDealBytes;
    const dim3 grid((unsigned)((int64_t)a.G * nblk_n)), block(256);
#define MOE_SKINNY(D, GA, S)                                                                                    \
  hipLaunchKernelGGL((grouped_gemm_skinny_kernel<D, GA, 1, S>), grid, block, 0, stream, (const uint16_t*)a.A, \
                     a.a_rows, a.a_nrows, a.offsets, a.G, a.max_rows, a.N, a.K, (const uint16_t*)a.B0,       \
                     D ? (const uint16_t*)a.B1 : nullptr, (uint16_t*)a.C, a.out_tok, a.out_w, a.y_acc, a.T, big,  \
                     slice_deal)
    const bool gather = a.a_rows != nullptr;
    if (scatter) MOE_SKINNY(false, false, true);
    else if (dual && gather) MOE_SKINNY(true, true, false);
    else if (dual) MOE_SKINNY(true, false, false);
    else if (gather) MOE_SKINNY(false, true, false);
    else MOE_SKINNY(false, false, false);
#undef MOE_SKINNY
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess || a.max_rows <= big) return e;
    return launch_tiled(a, dual, 128, big, stream);
  }
  if (a.dtype == MOE_BF16) {
    const int64_t rows_per_group = (a.max_rows + a.G - 1) / a.G;  // ceiling of the average
    const int bm = rows_per_group <= kSmallTileRowsPerGroup ? 128 : rows_per_group <= kMidTileRowsPerGroup ? 192 : 256;
    return launch_tiled(a, dual, bm, 0, stream);
  }
  const int64_t blocks = ((int64_t)a.max_rows * a.N + 255) / 256;
  if (blocks <= 0) return hipSuccess;
  if (dual)
    hipLaunchKernelGGL(grouped_gemm_f32_kernel<true>, dim3((unsigned)blocks), dim3(256), 0, stream,
                       (const float*)a.A, a.a_rows, a.a_nrows, a.offsets, a.G, a.max_rows, a.N, a.K,
                       (const float*)a.B0, (const float*)a.B1, (float*)a.C, nullptr, nullptr, nullptr, 0);
  else
    hipLaunchKernelGGL(grouped_gemm_f32_kernel<false>, dim3((unsigned)blocks), dim3(256), 0, stream,
                       (const float*)a.A, a.a_rows, a.a_nrows, a.offsets, a.G, a.max_rows, a.N, a.K,
                       (const float*)a.B0, nullptr, (float*)a.C, a.out_tok, a.out_w, a.y_acc, a.T);
  return hipGetLastError();
}

}  // namespace moe
