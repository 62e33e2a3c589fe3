// rope.hpp -- rotary position embedding on bf16 operand fragments (gfx950).
//
// Rotate-half arrangement (the rotary embedding that Wilsontomass's module in
// the nanoGPT issue "How best to implement a differential transformer?"
// applies to every q and k head): element c < d/2 pairs with c + d/2, and the
// pair turns by the angle t * w_c, w_c = theta^(-2c/d), at position t:
//   x'_c = x_c cos - x_{c+d/2} sin,   x'_{c+d/2} = x_{c+d/2} cos + x_c sin.
// The angle t * w_c is formed in fp32 together with its rounding error (an
// fma recovers it exactly) and sine and cosine of the rounded angle are
// corrected to first order by it, so the product's rounding (up to ~5e-4 rad
// at t = 8192) does not reach the result; w_c itself comes from exp2f (its
// error moves the angle by < 2e-4 rad at t = 8192).  The rotated pair is
// rounded once to bf16 (relative 2^-9).
#pragma once

#include <math.h>
#include <stdint.h>

#include "kernels.hpp"

namespace da {

// Frequency w_c = theta^(-2c/d) = 2^(c * nl2t), nl2t = -2 log2(theta) / d.
__device__ __forceinline__ float rope_freq(int c, float nl2t) { return exp2f(nl2t * (float)c); }

// sin and cos of pos * w (pos < 2^24).
__device__ __forceinline__ void rope_sincos(int pos, float w, float* sn, float* cs) {
  const float p = (float)pos;
  const float hi = p * w;
  const float lo = fmaf(p, w, -hi);  // p * w - hi, exactly
  float s, c;
  sincosf(hi, &s, &c);
  *sn = fmaf(lo, c, s);
  *cs = fmaf(-lo, s, c);
}

// Rotate the fragments of one row held as f[ks] = elements
// CS * ks + coff + 0..7 (ks = 0 .. KS-1, KS * CS = d): element c of f[ks]
// pairs with the same element of f[ks + KS/2].
template <int KS, int CS>
__device__ __forceinline__ void rope_rotate_frags(bf16x8* f, int coff, int pos, float nl2t) {
  static_assert(KS % 2 == 0, "pairs c, c + d/2 sit in fragments ks, ks + KS/2");
#pragma unroll
  for (int ks = 0; ks < KS / 2; ++ks) {
    f32x8 a, b;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      float sn, cs;
      rope_sincos(pos, rope_freq(CS * ks + coff + e, nl2t), &sn, &cs);
      const float x1 = (float)f[ks][e], x2 = (float)f[ks + KS / 2][e];
      a[e] = x1 * cs - x2 * sn;
      b[e] = x2 * cs + x1 * sn;
    }
    f[ks] = cvt_bf16x8(a);
    f[ks + KS / 2] = cvt_bf16x8(b);
  }
}

}  // namespace da
