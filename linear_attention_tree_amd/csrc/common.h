// Device helpers shared by the gfx950 kernels of libbole.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "bole.h"

namespace bole {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint16_t u16x8 __attribute__((ext_vector_type(8)));
typedef uint16_t u16x4 __attribute__((ext_vector_type(4)));

constexpr int kMaxTree = BOLE_MAX_TREE;  // one wave64 lane / one mask bit per node
constexpr int kWave = 64;

// ---------------------------------------------------------------------------
// MFMA: v_mfma_f32_16x16x32_bf16 (CDNA4).  Lane layout, lane l in [0, 64):
//   A (16 x 32, row-major M x K): lane holds A[l % 16][8*(l/16) .. 8*(l/16)+7]
//   B (32 x 16, K x N):           lane holds B[8*(l/16) .. +7][l % 16]
//   D (16 x 16):                  lane holds D[4*(l/16) + r][l % 16], r = 0..3
__device__ __forceinline__ f32x4 mfma_bf16(const bf16x8& a, const bf16x8& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// v_mfma_f32_16x16x16_bf16.  Lane layout, lane l in [0, 64):
//   A (16 x 16): lane holds A[l % 16][4*(l/16) .. 4*(l/16)+3]
//   B (16 x 16): lane holds B[4*(l/16) .. +3][l % 16]
//   D (16 x 16): lane holds D[4*(l/16) + r][l % 16], r = 0..3
// D and B coincide, so a product's result feeds the next product's B operand
// without any data movement.
__device__ __forceinline__ f32x4 mfma16_bf16(const bf16x4& a, const bf16x4& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
}

// Round-to-nearest-even split x ~= hi + lo into bf16 parts (relative residual
// below 2^-16), using packed conversions (two elements per instruction).
__device__ __forceinline__ void split_bf16x4(const f32x4& x, bf16x4& hi, bf16x4& lo) {
  hi = __builtin_convertvector(x, bf16x4);
  lo = __builtin_convertvector(x - __builtin_convertvector(hi, f32x4), bf16x4);
}

// Vector stores at device scope (sc1): the line is written through the L2 at
// once rather than left dirty in it.  A kernel ends only once its dirty L2
// lines are written back, so output written late in a kernel would otherwise
// be written back after the last wave has finished.
__device__ __forceinline__ void store_sc1(float* p, const f32x4& v) {
  asm volatile("global_store_dwordx4 %0, %1, off sc1" : : "v"(p), "v"(v) : "memory");
}
__device__ __forceinline__ void store_sc1(uint16_t* p, const u16x4& v) {
  asm volatile("global_store_dwordx2 %0, %1, off sc1" : : "v"(p), "v"(v) : "memory");
}

__device__ __forceinline__ f32x4 zero_f32x4() { return f32x4{0.f, 0.f, 0.f, 0.f}; }

__device__ __forceinline__ bf16x8 zero_bf16x8() {
  bf16x8 z;
#pragma unroll
  for (int e = 0; e < 8; ++e) z[e] = (__bf16)0.0f;
  return z;
}

typedef float f32x8 __attribute__((ext_vector_type(8)));

// Round-to-nearest-even split of 8 floats into bf16 hi + lo parts, x ~= hi + lo
// (relative residual below 2^-16).
__device__ __forceinline__ void split_bf16x8(const float* x, bf16x8& hi, bf16x8& lo) {
  const f32x8 v = {x[0], x[1], x[2], x[3], x[4], x[5], x[6], x[7]};
  hi = __builtin_convertvector(v, bf16x8);
  lo = __builtin_convertvector(v - __builtin_convertvector(hi, f32x8), bf16x8);
}

__device__ __forceinline__ void load_f32x8(const float* __restrict__ p, float* x) {
  const float4 a = *reinterpret_cast<const float4*>(p);
  const float4 b = *reinterpret_cast<const float4*>(p + 4);
  x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
  x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
}

__device__ __forceinline__ bf16x8 load_bf16x8(const uint16_t* __restrict__ p) {
  const u16x8 u = *reinterpret_cast<const u16x8*>(p);
  return __builtin_bit_cast(bf16x8, u);
}

__device__ __forceinline__ float bf16_bits_to_float(uint16_t b) {
  return __uint_as_float(((uint32_t)b) << 16);
}

__device__ __forceinline__ uint16_t float_to_bf16_bits(float x) {
  return __builtin_bit_cast(uint16_t, (__bf16)x);
}

// Local node index read from a caller array, forced into [0, T) so that an
// inconsistent order/parent array can never address rows outside the tree.
__device__ __forceinline__ int clamp_node(int x, int T) {
  return (unsigned)x < (unsigned)T ? x : 0;
}

// Make a value provably wave-uniform for the compiler (scalar registers).
__device__ __forceinline__ int uniform(int x) { return __builtin_amdgcn_readfirstlane(x); }

__device__ __forceinline__ uint64_t uniform64(uint64_t x) {
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)x);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(x >> 32));
  return ((uint64_t)hi << 32) | lo;
}

__device__ __forceinline__ uint64_t ballot64(bool p) { return __ballot(p); }

__device__ __forceinline__ void report(uint32_t* err, uint32_t bits) {
  if (err) atomicOr(err, bits);
}

// Workgroup-id remap so that consecutive logical ids land on the same XCD.
// MI355X dispatches workgroup w to XCD (w mod 8); this returns the logical id
// whose XCD-local rank is w / 8, with XCD x owning a contiguous logical range.
// Gate ratio P_i / P_j = exp(logP_i - logP_j) from the sums prescaled to base 2
// (e2 = logP * log2(e), one rounding), as one hardware exp2.  Relative error
// about |logP| * 2^-24, against 1 ulp for expf; it feeds float32 products.
constexpr float kLog2e = 1.44269504088896341f;
__device__ __forceinline__ float gate_ratio(float e2_i, float e2_j) {
  return __builtin_amdgcn_exp2f(e2_i - e2_j);
}

// all-ones or zero: a mask applied to a loaded value (a select would let the
// compiler move the load behind a branch and wait for it there)
__device__ __forceinline__ uint32_t keep(bool b) { return 0u - (uint32_t)b; }

__device__ __forceinline__ int xcd_remap(int w, int total) {
  constexpr int kXcd = 8;
  const int x = w % kXcd, k = w / kXcd;
  const int q = total / kXcd, rem = total % kXcd;
  return x * q + (x < rem ? x : rem) + k;
}

}  // namespace bole
