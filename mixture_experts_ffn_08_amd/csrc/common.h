// Device helpers shared by the MoE kernels (gfx950 / CDNA4, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;

__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float(uint32_t(b) << 16); }

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// Two float32 -> two bfloat16 (lo in bits 0..15), round to nearest, ties to even:
// one v_cvt_pk_bf16_f32 on gfx950.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{lo, hi}, bf16x2));
}

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

__device__ __forceinline__ u32x4 ld16(const void* p) { return *reinterpret_cast<const u32x4*>(p); }

// Fourth word of a gfx9-family buffer resource: raw (untyped) 32-bit access.
constexpr int kBufferFlags = 0x00020000;

// Block barrier without the memory fence of __syncthreads (which would also wait
// for the global loads still in flight): LDS writes are drained first, and the
// memory clobber keeps the compiler from moving LDS accesses across it.
// Hardware deals the blocks of a 1-D grid round-robin to the 8 XCDs (block b runs
// on XCD b % 8).  Block b's logical index here gives XCD x the contiguous run
// [x q + min(x, r), ..) of the n blocks (q = n / 8, r = n % 8), so a kernel whose
// blocks stream consecutive regions has each XCD stream one contiguous eighth:
// its address translation then covers only those pages.
__device__ __forceinline__ int xcd_contiguous(int b, int n) {
  const int q = n >> 3, r = n & 7, x = b & 7;
  return x * q + min(x, r) + (b >> 3);
}
__device__ __forceinline__ int xcd_contiguous_block() { return xcd_contiguous((int)blockIdx.x, (int)gridDim.x); }
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }
__device__ __forceinline__ void st16(void* p, u32x4 v) { *reinterpret_cast<u32x4*>(p) = v; }

// SiLU(g) = g / (1 + e^-g) for outputs that are rounded to bf16: the hardware
// reciprocal (v_rcp_f32, about 1 ulp) in place of a correctly rounded fp32
// division, which compiles to a dozen instructions.  Large |g| stays exact in
// the limit: e^-g = inf gives g * 0, e^-g = 0 gives g.
__device__ __forceinline__ float silu_bf16out(float g) { return g * __builtin_amdgcn_rcpf(1.f + __expf(-g)); }

// 32x32 output, K = 16 per instruction.  Lane l supplies A row (l % 32) and B
// column (l % 32), each with the 8 k values 8*(l/32) .. 8*(l/32)+7.
// Accumulator element i of lane l is row 8*(i/4) + 4*(l/32) + (i%4), column l % 32.
__device__ __forceinline__ f32x16 mfma32x32x16(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
// 16x16 output, K = 32 per instruction.  Lane l supplies A row (l % 16) and B
// column (l % 16) with k values 8*(l/16) .. 8*(l/16)+7.  Accumulator element i
// of lane l is row 4*(l/16) + i, column l % 16.
__device__ __forceinline__ f32x4 mfma16x16x32(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// Butterfly exchange inside each 32-lane half through ds_swizzle (bit mode:
// and-mask 0x1f, xor-mask X).
template <int X>
__device__ __forceinline__ uint32_t swz_xor(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_ds_swizzle((int)v, (X << 10) | 0x1f);
}
template <int X>
__device__ __forceinline__ float swz_xor(float v) {
  return __uint_as_float(swz_xor<X>(__float_as_uint(v)));
}

// Sum over the wave; every lane gets the same value (same tree on every lane).
__device__ __forceinline__ float wave_sum(float v) {
  v += swz_xor<1>(v);
  v += swz_xor<2>(v);
  v += swz_xor<4>(v);
  v += swz_xor<8>(v);
  v += swz_xor<16>(v);
  float a = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0));
  float b = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32));
  return a + b;
}

__device__ __forceinline__ float wave_max(float v) {
  v = fmaxf(v, swz_xor<1>(v));
  v = fmaxf(v, swz_xor<2>(v));
  v = fmaxf(v, swz_xor<4>(v));
  v = fmaxf(v, swz_xor<8>(v));
  v = fmaxf(v, swz_xor<16>(v));
  float a = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0));
  float b = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32));
  return fmaxf(a, b);
}

// Total order on float32 scores as uint32: larger float -> larger key; -0 and +0
// map to the same key.
__device__ __forceinline__ uint32_t order_key(float f) {
  uint32_t u = __float_as_uint(f + 0.0f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

}  // namespace moe

namespace moe {

// DPP lane permutations inside each row of 16 lanes (GFX9 encodings).
constexpr int kDppXor1 = 0xB1;        // quad_perm [1,0,3,2]
constexpr int kDppXor2 = 0x4E;        // quad_perm [2,3,0,1]
constexpr int kDppHalfMirror = 0x141; // lane i <-> 7-i within each 8
constexpr int kDppMirror = 0x140;     // lane i <-> 15-i within each 16

template <int CTRL>
__device__ __forceinline__ uint32_t dpp(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, CTRL, 0xf, 0xf, false);
}
template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xf, 0xf, false));
}

// Sum over each row of 16 lanes; every lane of the row gets the same value.
__device__ __forceinline__ float row16_sum(float v) {
  v += dpp<kDppXor1>(v);
  v += dpp<kDppXor2>(v);
  v += dpp<kDppHalfMirror>(v);
  v += dpp<kDppMirror>(v);
  return v;
}

__device__ __forceinline__ float row16_max(float v) {
  v = fmaxf(v, dpp<kDppXor1>(v));
  v = fmaxf(v, dpp<kDppXor2>(v));
  v = fmaxf(v, dpp<kDppHalfMirror>(v));
  v = fmaxf(v, dpp<kDppMirror>(v));
  return v;
}

// Inverse of order_key (-0 comes back as +0).
__device__ __forceinline__ float key_value(uint32_t o) {
  return __uint_as_float((o & 0x80000000u) ? (o & 0x7fffffffu) : ~o);
}

}  // namespace moe
