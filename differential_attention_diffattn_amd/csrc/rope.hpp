// rope.hpp -- rotary position embedding on bf16 operand fragments (gfx950).
//
// Rotate-half arrangement (the rotary embedding that Wilsontomass's module in
// the nanoGPT issue "How best to implement a differential transformer?"
// applies to every q and k head): element c < d/2 pairs with c + d/2, and the
// pair turns by the angle t * w_c, w_c = theta^(-2c/d), at position t:
//   x'_c = x_c cos - x_{c+d/2} sin,   x'_{c+d/2} = x_{c+d/2} cos + x_c sin.
// w_c arrives as an unevaluated sum of two floats (host-computed in
// double).  The angle t * w_c is formed in fp32 as hi + lo (an fma recovers
// the main product's rounding error) and turned into revolutions with
// 1/(2 pi) split in two fp32 parts, the whole revolutions dropped inside one
// fma; the hardware sine and cosine (v_sin_f32 / v_cos_f32, argument in
// revolutions) then see |f| <= 1/2 plus a remainder accurate to ~1e-7
// revolutions at every position below 2^24.  The
// instructions' own error is ~1e-6; the rotated pair is rounded once to bf16
// (relative 2^-9).
#pragma once

#include <math.h>
#include <stdint.h>

#include "kernels.hpp"

namespace da {

// sin and cos of pos * (w_hi + w_lo) (pos < 2^24).
__device__ __forceinline__ void rope_sincos(int pos, float w_hi, float w_lo, float* sn, float* cs) {
  constexpr float kR = 1.591549367e-01f;     // 1/(2 pi), rounded to fp32
  constexpr float kRlo = 6.420638243e-09f;   // 1/(2 pi) - kR
  const float p = (float)pos;
  const float hi = p * w_hi;
  const float lo = fmaf(p, w_hi, -hi) + p * w_lo;  // p * w = hi + lo
  // whole revolutions n of hi * kR, then hi * kR - n in one fma: |result| <=
  // 1/2, rounded once (3e-8), whatever rounding hi * kR itself had
  const float n = rintf(hi * kR);
  const float f = fmaf(hi, kR, -n) + fmaf(hi, kRlo, lo * kR);  // revolutions mod 1
  *sn = __builtin_amdgcn_sinf(f);
  *cs = __builtin_amdgcn_cosf(f);
}

// Rotate the fragments of one row held as f[ks] = elements
// CS * ks + coff + 0..7 (ks = 0 .. KS-1, KS * CS = d): element c of f[ks]
// pairs with the same element of f[ks + KS/2].
template <int KS, int CS>
__device__ __forceinline__ void rope_rotate_frags(bf16x8* f, int coff, int pos, const RopeTab& w) {
  static_assert(KS % 2 == 0, "pairs c, c + d/2 sit in fragments ks, ks + KS/2");
#pragma unroll
  for (int ks = 0; ks < KS / 2; ++ks) {
    f32x8 a, b;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      float sn, cs;
      const int c = CS * ks + coff + e;
      rope_sincos(pos, w.hi[c], w.lo[c], &sn, &cs);
      const float x1 = (float)f[ks][e], x2 = (float)f[ks + KS / 2][e];
      a[e] = x1 * cs - x2 * sn;
      b[e] = x2 * cs + x1 * sn;
    }
    f[ks] = cvt_bf16x8(a);
    f[ks + KS / 2] = cvt_bf16x8(b);
  }
}

}  // namespace da
