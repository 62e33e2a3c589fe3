// common.hpp -- device-side building blocks shared by the gfx950 kernels.
//
// CDNA4 facts relied on here: 64-lane wavefronts; MFMA
// v_mfma_f32_32x32x16_bf16 / v_mfma_f32_16x16x32_bf16 with fp32
// accumulators; v_cvt_pk_bf16_f32 (round to nearest even); 160 KB of LDS per
// CU; workgroups dispatched round-robin over 8 XCDs, each with its own L2.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace da {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Strided tensor descriptors, element strides by role (batch, head, token);
// the head_dim axis is unit-stride.  Mirrors da_in / da_out of the C ABI.
struct TIn {
  const void* p;
  int64_t sb, sh, st;
};
struct TOut {
  void* p;
  int64_t sb, sh, st;
};

constexpr int kXcds = 8;

// Workgroups are dealt to XCDs round-robin (block b runs on XCD b % 8).  Map
// the hardware block id to a logical id so that each XCD receives one
// contiguous range of logical ids: neighbouring logical work items (which
// share K/V) then share that XCD's L2.  A bijection on [0, n).
__device__ __forceinline__ int xcd_logical_id(int bid, int n) {
  const int xcd = bid % kXcds, slot = bid / kXcds;
  const int base = n / kXcds, rem = n % kXcds;
  return xcd * base + (xcd < rem ? xcd : rem) + slot;
}

__device__ __forceinline__ f32x16 mfma32x32x16(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma16x16x32(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8 as_bf16x8(uint4 u) { return __builtin_bit_cast(bf16x8, u); }
__device__ __forceinline__ uint4 as_u4(bf16x8 v) { return __builtin_bit_cast(uint4, v); }

__device__ __forceinline__ bf16x8 join_bf16x8(uint2 lo, uint2 hi) {
  return as_bf16x8(make_uint4(lo.x, lo.y, hi.x, hi.y));
}

// Eight fp32 values -> eight bf16 (v_cvt_pk_bf16_f32, round to nearest even).
__device__ __forceinline__ bf16x8 cvt_bf16x8(f32x8 v) { return __builtin_convertvector(v, bf16x8); }

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __builtin_bit_cast(float, (uint32_t)b << 16);
}

// Round-to-nearest-even fp32 -> bf16 of two values packed in one word.
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  typedef float f2 __attribute__((ext_vector_type(2)));
  typedef __bf16 h2 __attribute__((ext_vector_type(2)));
  f2 v = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, h2));
}

// Logistic sigmoid of a logit, never overflowing; sigmoid(+-inf) = 1 / 0.
__device__ __forceinline__ float sigmoid_f32(float x) {
  if (x >= 0.f) return 1.f / (1.f + __expf(-x));
  const float e = __expf(x);
  return e / (1.f + e);
}

// max(x[l % 32], x[l % 32 + 32]) in every lane l, without an LDS round trip:
// v_permlane32_swap exchanges the upper half of one copy of x with the lower
// half of another, leaving each lane with x of both lane halves.  Written as
// inline asm: with both operands equal, the compiler's model of the builtin
// folds the two results into one and drops the upper half.  The s_nop covers
// the VALU-write -> permlane-read hazards on both sides of the swap.
__device__ __forceinline__ float max_across_halves(float x) {
  float a = x, b = x;
  asm volatile("s_nop 1\n\tv_permlane32_swap_b32 %0, %1\n\ts_nop 1\n\tv_max_f32 %0, %0, %1"
               : "+v"(a), "+v"(b));
  return a;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

}  // namespace da
