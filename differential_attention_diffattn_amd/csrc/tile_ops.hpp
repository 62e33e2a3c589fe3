// tile_ops.hpp -- LDS tile helpers shared by the prefill and backward
// kernels (gfx950): HBM -> LDS copies, transpose and 16-byte LDS reads, the
// XOR swizzles of tile rows, a compile-time loop.
#pragma once

#include <stdint.h>

#include <type_traits>

#include "kernels.hpp"

namespace da {

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4_t;

// 16 bytes per lane, HBM -> LDS (global_load_lds_dwordx4, "saddr" form: a
// wave-uniform 64-bit base in SGPRs plus a per-lane 32-bit byte offset):
// lane l's bytes land at LDS byte address lds_addr + 16 l; lds_addr must be
// wave-uniform.  Issued as inline asm so the compiler does not track it: it
// would otherwise make every LDS read wait for the copy in flight, although
// that copy only ever targets another LDS stage.  The kernel waits for it
// explicitly (vmcnt(0) + barrier) before the stage is read.  M0 is used by
// nothing else in these kernels.
__device__ __forceinline__ void dma16_sbase(const void* base, uint32_t off, uint32_t lds_addr) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1"
               :
               : "v"(off), "s"(base), "s"(__builtin_amdgcn_readfirstlane(lds_addr))
               : "memory");
}
// The same copy marked non-temporal ("nt"), for data read once (a stream):
// the caches do not keep it at the expense of data that is re-read.
__device__ __forceinline__ void dma16_sbase_nt(const void* base, uint32_t off, uint32_t lds_addr) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1 nt"
               :
               : "v"(off), "s"(base), "s"(__builtin_amdgcn_readfirstlane(lds_addr))
               : "memory");
}

// LDS transpose read: in each group of 16 lanes, lane j receives element
// (j & 3) of the 4-element rows addressed by lanes 4k + (j >> 2), k = 0..3.
__device__ __forceinline__ uint2 tr_read(uint32_t lds_addr) {
  const s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(uintptr_t)lds_addr);
  return __builtin_bit_cast(uint2, v);
}

// 16-byte LDS read (ds_read_b128) at an LDS byte address.
__device__ __forceinline__ bf16x8 lds_read16(uint32_t lds_addr) {
  return *(const __attribute__((address_space(3))) bf16x8*)(uintptr_t)lds_addr;
}

template <int I, int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (I < N) {
    f(std::integral_constant<int, I>{});
    static_for<I + 1, N>(f);
  }
}

// Sum of the eight bf16 values of x, accumulated onto acc in fp32
// (v_dot2_f32_bf16 against (1, 1)).
__device__ __forceinline__ float sum_bf16x8(bf16x8 x, float acc) {
  const uint4 u = as_u4(x);
  const bf16x2 one = __builtin_bit_cast(bf16x2, 0x3f803f80u);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, u.x), one, acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, u.y), one, acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, u.z), one, acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, u.w), one, acc, false);
  return acc;
}

// XOR swizzles of 16-byte chunks inside a tile row (measured conflict-free on
// gfx950, whose LDS serves 256 B per clock from 64 banks):
//   K rows (read by ds_read_b128, 16 rows per pass): rows of 256 B use
//   chunk ^ (r & 15); rows of 128 B use chunk ^ ((r & 7) ^ ((r >> 3) & 1)).
//   V rows (read by ds_read_b64_tr_b16, 4 rows x 32 B per 16 lanes):
//   chunk ^ 4 (r & 3) when a row has >= 16 chunks, else chunk ^ 2 (r & 3).
template <int D>
__device__ __forceinline__ int k_swizzle(int r) {
  return D >= 128 ? (r & 15) : ((r & 7) ^ ((r >> 3) & 1));
}
template <int DV>
__device__ __forceinline__ int v_swizzle(int r) {
  return (DV >= 128 ? 4 : 2) * (r & 3);
}
// One layout serving both read forms, for a tile that is read as rows and
// transposed (d = 64 or 128): the swizzle is a bijection on r mod 16 (so the
// 16 rows of a ds_read_b128 pass hit distinct chunks), gives each aligned
// group of 4 rows distinct bits 2-3 (d = 128; bit 2 between rows 2 apart at
// d = 64) (so a transpose read's 4 rows x 64 bytes per 32 lanes hit distinct
// banks), and satisfies u(r + 8) = u(r) ^ 4, u(r + 16) = u(r), so the
// transpose read 8 rows further down lands in column block cb ^ 1 of the
// same base.  Bits: r2, r1, r1 ^ r3 (and r0 at d = 128).  The bank behaviour
// of both read forms and the operands they deliver are checked on the CPU
// (tests/test_tile_layout.py).
template <int D>
__device__ __forceinline__ int u_swizzle(int r) {
  const int v = ((r >> 2) & 1) | (((r >> 1) & 1) << 1) | ((((r >> 1) ^ (r >> 3)) & 1) << 2);
  return D >= 128 ? v | ((r & 1) << 3) : v;
}
enum TileLayout { kRowLayout = 0, kTransLayout = 1, kBothLayout = 2 };
template <int D>
__device__ __forceinline__ int tile_swizzle(int layout, int r) {
  return layout == kRowLayout ? k_swizzle<D>(r) : layout == kTransLayout ? v_swizzle<D>(r) : u_swizzle<D>(r);
}

}  // namespace da
