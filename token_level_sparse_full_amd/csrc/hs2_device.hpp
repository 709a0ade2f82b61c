// Device-side helpers shared by the gfx950 kernels of libhs2.
//
// Lane layouts used throughout (wave64, gfx950):
//  * v_mfma_f32_32x32x16_bf16: A lane l holds A[l%32][8*(l/32) + i], B lane l
//    holds B[8*(l/32) + i][l%32] (i = 0..7); C reg r of lane l is
//    C[8*(r/4) + 4*(l/32) + r%4][l%32].
//  * v_mfma_f32_16x16x32_bf16: A lane l holds A[l%16][8*(l/16) + i], B lane l
//    holds B[8*(l/16) + i][l%16]; C reg r of lane l is C[4*(l/16) + r][l%16].
//  * v_mfma_f32_16x16x4_f32:   A lane l holds A[l%16][l/16], B lane l holds
//    B[l/16][l%16]; C as for 16x16x32.
//  * ds_read_b64_tr_b16 works on groups of 16 lanes: lane i of a group receives
//    element (i%4) of the 4-element (8-byte) segments addressed by lanes
//    i/4 + 4e of its group, e = 0..3, as its elements e.  Pointing lane s of a
//    group at row (rbase + s/4), columns (cbase + 4*(s%4) .. +3) of a row-major
//    16-bit matrix therefore hands lane i the column (cbase + i) of rows
//    rbase..rbase+3: a transposed 4x16 read.
//  * v_permlane32_swap(x, y) returns (x with its upper half replaced by the
//    lower half of y, y with its lower half replaced by the upper half of x).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "hs2_internal.hpp"

namespace hs2 {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;
constexpr int kHeadDim = 256;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kNegInf = -__builtin_inff();

#define HS2_LDS __attribute__((address_space(3)))

__device__ __forceinline__ int lane_id() { return __builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u)); }

// ---------------------------------------------------------------- MFMA wrappers
__device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma16_f32(float a, float b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x16 mfma32_f32(float a, float b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
}

// ---------------------------------------------------------------- conversions
__device__ __forceinline__ bf16 to_bf16(float x) { return (bf16)x; }  // RNE on gfx950

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 u) { return __builtin_bit_cast(bf16x8, u); }
__device__ __forceinline__ u32x4 as_u32x4(bf16x8 v) { return __builtin_bit_cast(u32x4, v); }

// 8 OCP e4m3 codes (two dwords) -> 8 bf16 values, exactly (every e4m3 value
// is a bf16 value: 4 significant bits, exponents 2^-9 .. 2^8).
__device__ __forceinline__ bf16x8 e4m3x8_to_bf16(uint32_t lo, uint32_t hi) {
  f32x2 a = __builtin_amdgcn_cvt_pk_f32_fp8((int)lo, false);
  f32x2 b = __builtin_amdgcn_cvt_pk_f32_fp8((int)lo, true);
  f32x2 c = __builtin_amdgcn_cvt_pk_f32_fp8((int)hi, false);
  f32x2 d = __builtin_amdgcn_cvt_pk_f32_fp8((int)hi, true);
  bf16x8 r;
  r[0] = (bf16)a[0]; r[1] = (bf16)a[1]; r[2] = (bf16)b[0]; r[3] = (bf16)b[1];
  r[4] = (bf16)c[0]; r[5] = (bf16)c[1]; r[6] = (bf16)d[0]; r[7] = (bf16)d[1];
  return r;
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

// ---------------------------------------------------------------- LDS transposed read
__device__ __forceinline__ bf16x4 lds_tr16(const bf16* p) {
  i16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((i16x4 HS2_LDS*)(p));
  return __builtin_bit_cast(bf16x4, v);
}
__device__ __forceinline__ bf16x8 cat8(bf16x4 a, bf16x4 b) {
  bf16x8 r;
  r[0] = a[0]; r[1] = a[1]; r[2] = a[2]; r[3] = a[3];
  r[4] = b[0]; r[5] = b[1]; r[6] = b[2]; r[7] = b[3];
  return r;
}

// ---------------------------------------------------------------- cross-lane
__device__ __forceinline__ float shfl_xor(float v, int m) { return __shfl_xor(v, m, kWave); }

// Sum of x over lanes l and l^32, landing in lane l%32 for x and in lane
// 32+l%32 for y: returns x(l) + x(l+32) on lanes < 32 and y(l-32) + y(l) on
// lanes >= 32.
// Workgroup barrier for tiles filled by LDS DMA.  __syncthreads() carries a
// workgroup-scope fence, and the compiler implements that fence by waiting
// for every outstanding vector-memory operation (vmcnt(0)), which would also
// wait for the DMA of tiles further ahead.  This barrier waits only for the
// wave's own LDS operations; the caller first waits (vmcnt) for the DMA that
// must have landed.  The "memory" clobber keeps the compiler from moving
// memory accesses across it.
__device__ __forceinline__ void dma_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

__device__ __forceinline__ float halfwave_pair_sum(float x, float y) {
  auto r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(uint32_t, x), __builtin_bit_cast(uint32_t, y), false, false);
  return __builtin_bit_cast(float, (uint32_t)r[0]) + __builtin_bit_cast(float, (uint32_t)r[1]);
}

// ---------------------------------------------------------------- misc
// Blocks are dispatched round-robin over the 8 XCDs (block b -> XCD b % 8).
// This gives each XCD a contiguous range of logical block ids, so that blocks
// sharing data also share an L2.
__device__ __forceinline__ int xcd_remap(int bid, int nblk) {
  const int per = nblk / 8, rem = nblk % 8;
  const int x = bid % 8, j = bid / 8;
  return x * per + (x < rem ? x : rem) + j;
}

template <typename T>
__device__ __forceinline__ T ld_nt(const T* p) { return __builtin_nontemporal_load(p); }

}  // namespace hs2
