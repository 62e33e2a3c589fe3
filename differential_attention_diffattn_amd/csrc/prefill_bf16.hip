// prefill_bf16.hip -- fused causal differential-attention prefill, bf16 MFMA.
//
// What is computed ("Differential Transformer V2" article, DiffAttnV1 and
// DiffAttnV2 pseudo-code):
//   V1: per differential head, the two causal softmax maps
//       softmax(Q1 K1^T / sqrt d) and softmax(Q2 K2^T / sqrt d) applied to the
//       one shared V (width 2d), then A1 V - lam A2 V, RMSNorm over the 2d
//       channels (eps 1e-5, no weight) and the (1 - lambda_init) scale
//       (nanoGPT issue "How best to implement a differential transformer?",
//       Wilsontomass's module).
//   V2: per adjacent head pair (2p, 2p+1) of a GQA group, the two maps over
//       the group's shared K and V, then O_2p - sigmoid(lam[t, p]) O_2p+1
//       (no norm, no scale).
//
// Structure (designed for gfx950, not taken from any listing):
//   * A wave owns 32 query rows of ONE map (V1: map 1 or map 2 of a
//     differential head; V2: the even or the odd head of a pair).  Partner
//     waves (2k, 2k+1) hold the two maps of the same rows and are combined
//     through LDS in the epilogue.  For V2 the waves of a workgroup cover the
//     heads of one GQA group, so each K/V tile is loaded once for the group.
//   * K and V tiles go HBM -> LDS with global_load_lds_dwordx4 (no registers,
//     no VALU), double-buffered: the next tile streams in while the current
//     one is consumed; one barrier per tile.  In LDS both stay row-major with
//     an XOR swizzle of their 16-byte chunks, so the MFMA operand reads are
//     bank-conflict-free.  The LDS holds [K stage 0 | K stage 1 | V stage 0 |
//     V stage 1] and the key loop is unrolled by stage, so every operand
//     read is a per-lane base register plus an immediate offset.
//   * Scores are computed transposed, S^T = K Q^T, with
//     v_mfma_f32_32x32x16_bf16: Q fragments stay in registers for the whole
//     key loop, each lane holds 16 scores of ONE query row (softmax state is
//     per lane), and the probabilities convert in place to the bf16 B operand
//     of O^T = V^T P^T.  The V^T A operand comes straight from the row-major
//     V tile through ds_read_b64_tr_b16 (the LDS transpose read).
//   * Online softmax in the log2 domain against a per-row reference m that
//     only moves when it must.  The common path per 32-key sub-block is one
//     fma + one exp2 per score, a bf16 conversion, and the row sum taken with
//     v_dot2_f32_bf16 over the converted probabilities (so the sum is exactly
//     that of the P fed to the MFMA).  No row maximum is computed there: if
//     a lane's 16 probabilities sum past 2^10 (a score rose more than ~10
//     log2 units above m, or m is still unset), the wave takes the exact
//     path -- the row maximum over both lane halves, a rescale of O and l,
//     and the sub-block's exponentials again against the new m.  Every
//     probability fed to the MFMA is therefore <= 2^10, and the result is the
//     same softmax up to rounding.
//   * Causal skipping at 32-key granularity (mask only on diagonal
//     sub-blocks); heaviest tiles first; workgroups mapped onto XCDs so the
//     tiles of one head share an L2.
//   * V1 cancellation guard.  Each map's P enters its P.V product rounded to
//     bf16 (relative 2^-9), so A1 V and A2 V each carry an error of about
//     1e-3 of their size.  Where they nearly cancel (lambda near 1 and two
//     maps that nearly agree, e.g. a row with two visible keys) the RMSNorm
//     scales D = A1 V - lam A2 V back to O(1) and with it that error, by
//     the factor kappa = |(A1 V, lam A2 V)| / |D|.  A row with kappa > 8 is
//     recomputed by its map-1 wave from the definition in fp32 (both maps,
//     exact softmax, P unrounded): the fast path's error stays below ~1e-2
//     and a flagged row's below 1e-5.  Random inputs flag no rows.
#include <math.h>

#include <type_traits>

#include "kernels.hpp"
#include "rope.hpp"
#include "tile_ops.hpp"

namespace da {
namespace {

#ifndef DA_V2_BN
#define DA_V2_BN 128  // keys per LDS stage of the V2 kernel (64 or 128)
#endif
#ifndef DA_PIPE_VSTAGES
#define DA_PIPE_VSTAGES 3  // V stages of the pipelined loop (2: 80 KB of LDS at d = 64 / 128)
#endif
#ifndef DA_NO_HINTS
#define DA_NO_HINTS 0
#endif
#ifndef DA_HINT_LEAD
#define DA_HINT_LEAD 8  // LDS operand reads issued ahead of a step's first MFMA
#endif
#ifndef DA_HINT_VPER
#define DA_HINT_VPER 3  // vector instructions per MFMA slot of a step
#endif
#ifndef DA_SETPRIO
#define DA_SETPRIO 1  // raise wave priority while issuing MFMA sections
#endif

// A lane whose 16 probabilities of a sub-block sum past this takes the exact
// (row maximum + rescale) path.
constexpr float kSumCap = 1024.f;
// Reference before any key is seen: finite, so masked scores (-inf) still
// give fma(-inf, c, kMInit) = -inf rather than NaN, and every visible score
// overflows the cap on the first sub-block.
constexpr float kMInit = -1e30f;

template <int D, int DV, bool V2, int NW, int MPW, bool PIPE>
struct Cfg {
  static constexpr int KS = D / 16;   // k-steps of the score MFMA
  static constexpr int CB = DV / 32;  // 32-wide column blocks of O^T
  static constexpr int NK = V2 ? 1 : 2;
  // PIPE: 64-key tiles, K in a 3-stage ring and V in a DA_PIPE_VSTAGES-stage
  // ring (software-pipelined key loop: the scores of a tile's first
  // sub-block are computed one step before its V is needed, so V needs one
  // stage less); otherwise BN-key tiles with K and V double-buffered.
  static constexpr int NSTK = PIPE ? 3 : 2;
  static constexpr int NSTV = PIPE ? DA_PIPE_VSTAGES : 2;
  static_assert(NSTV == 2 || NSTV == 3, "V ring depth");
  static constexpr int BN = PIPE ? 64 : (V2 ? DA_V2_BN : 64);  // keys per tile
  static constexpr int NSB = BN / 32;            // 32-key sub-blocks per tile
  static constexpr int K_BYTES = BN * D * 2;     // one K tensor of one tile
  static constexpr int V_BYTES = BN * DV * 2;
  static constexpr int KREG = NK * K_BYTES;      // K tensors of one stage
  static constexpr int VBASE = NSTK * KREG;      // V stages follow all K stages
  static constexpr int TILE_SMEM = NSTK * KREG + NSTV * V_BYTES;
  static constexpr int KCH = NK * K_BYTES / 1024;  // 1 KB DMA instructions per tile: K
  static constexpr int VCH = V_BYTES / 1024;       // and V
  static constexpr int KPW = KCH / NW, VPW = VCH / NW;  // per wave
  static_assert(KCH % NW == 0 && VCH % NW == 0, "tile DMA split");
  static_assert(D >= 64 && DV >= 64, "swizzles assume >= 8 chunks per row");
  static_assert(MPW == 1 || MPW == 2, "maps per wave");
  static_assert(!PIPE || NSB >= 2, "the pipelined rings free a stage one sub-block before the tile ends");
  // Operand reads use 16-bit immediate offsets from a per-lane base.
  static_assert((NSTK - 1) * KREG + (NK - 1) * K_BYTES * (MPW - 1) + (BN - 32) * D * 2 < 65536, "K read offset range");
  static_assert((NSTV - 1) * V_BYTES + (BN - 8) * DV * 2 + (CB - 1) * 64 < 65536, "V read offset range");
  // MPW == 1 epilogue: one exchange slot per partner-wave pair (fp32, lane-native
  // order).  When the stages already take more than half the LDS (one
  // workgroup per CU) and the slots fit beside them (SEPX), they get LDS of
  // their own, so a map-2 wave writes its slot as soon as its own key loop
  // ends; otherwise they reuse the stages once every wave is done with them.
  static constexpr int XBYTES = MPW == 1 ? (NW / 2) * CB * 16 * 64 * 4 : 0;
  static constexpr bool SEPX = MPW == 1 && TILE_SMEM > 80 * 1024 && TILE_SMEM + XBYTES <= 160 * 1024;
  static constexpr int XBASE = SEPX ? TILE_SMEM : 0;
  static constexpr int SMEM = SEPX ? TILE_SMEM + XBYTES : (TILE_SMEM > XBYTES ? TILE_SMEM : XBYTES);
  static_assert(SMEM <= 160 * 1024, "LDS budget");
  // MPW == 1 with 4 waves: two workgroups (two waves per SIMD) per CU
  static constexpr int MIN_BLOCKS = (MPW == 1 && NW == 4) ? 2 : 1;
  static_assert(MIN_BLOCKS * SMEM <= 160 * 1024, "LDS budget for the intended occupancy");
};

// (clang tries to constant-evaluate a lambda call whose value initialises a
// variable or is returned, and that evaluation crashes on the vector element
// stores inside; the score lambda therefore starts with an empty asm
// statement, which ends any such evaluation at once.)
template <int MPW>
struct Scores {
  f32x16 s[MPW];
};
template <int MPW>
struct Probs {
  bf16x8 p[MPW][2];  // bf16 B operand of P.V, two 16-key halves
  float bs[MPW];     // this lane's sum of the block's probabilities
};

// kappa^2 above which a V1 row is recomputed exactly (kappa > 8).
constexpr float kCancel2 = 64.f;

// One V1 output row (batch b, differential head h, query row i) from the
// definition, in fp32 and with the whole wave: both maps' scores
// q_m . k_m,j / sqrt d for j <= i (lane = key, 64 keys per chunk), an online
// softmax over the chunks with the exact row maximum and no rounding of P,
// A_m V over the 2d channels (lane = DV/64 consecutive channels), then
// D = A1 V - lam A2 V, the RMSNorm and the scale, stored to out.  buf (LDS,
// 2D floats) holds the two q rows.  With rope, q and the keys as given are
// turned here in fp32 (the key loop reads keys rotated and rounded to bf16).
typedef __attribute__((address_space(3))) float lds_f32;
typedef const __attribute__((address_space(4))) PrefillArgs kargs_t;  // the kernel's argument in its segment
template <int D, int DV>
__device__ __forceinline__ void v1_exact_row(int b, int h, int i, float lam, lds_f32* buf, int lane) {
  constexpr int CPL = DV / 64;  // V channels per lane (2 or 4)
  // The arguments are read from the kernel argument segment (the kernel's
  // only argument sits at its start) through a pointer the compiler cannot
  // see through: none of them is then loaded at kernel entry and kept live
  // across the key loop for this rarely taken path.
  kargs_t* ap = (kargs_t*)__builtin_amdgcn_kernarg_segment_ptr();
  asm volatile("" : "+s"(ap));
  lds_f32* qs = buf;
  // keys as given (with rope: before rotation, turned below in fp32)
  const uint16_t* kq0 = (const uint16_t*)ap->k1o.p + b * ap->k1o.sb + h * ap->k1o.sh;
  const uint16_t* kq1 = (const uint16_t*)ap->k2o.p + b * ap->k2o.sb + h * ap->k2o.sh;
  const int64_t kst0 = ap->k1o.st, kst1 = ap->k2o.st;
  const int64_t vst = ap->v.st;
  const uint16_t* vb = (const uint16_t*)ap->v.p + b * ap->v.sb + h * ap->v.sh + lane * CPL;
  const int rope = ap->rope, softmax1 = ap->softmax1;
  const float sl2 = ap->sl2, lam_init = ap->lam_init;
#pragma unroll
  for (int m = 0; m < 2; ++m) {
    const uint16_t* qr = m ? (const uint16_t*)ap->q2.p + b * ap->q2.sb + h * ap->q2.sh + (int64_t)i * ap->q2.st
                           : (const uint16_t*)ap->q1.p + b * ap->q1.sb + h * ap->q1.sh + (int64_t)i * ap->q1.st;
    for (int c = lane; c < D / 2; c += 64) {
      float x1 = bf16_to_f32(qr[c]), x2 = bf16_to_f32(qr[c + D / 2]);
      if (rope) {
        float sn, cs;
        rope_sincos(i, ap->rope_w.hi[c], ap->rope_w.lo[c], &sn, &cs);
        const float y1 = x1 * cs - x2 * sn, y2 = x2 * cs + x1 * sn;
        x1 = y1;
        x2 = y2;
      }
      qs[m * D + c] = x1;
      qs[m * D + c + D / 2] = x2;
    }
  }
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  float M[2], Z[2], O[2][CPL];
#pragma unroll
  for (int m = 0; m < 2; ++m) {
    // off-by-one softmax: one more logit 0 with a zero value row
    M[m] = softmax1 ? 0.f : -INFINITY;
    Z[m] = softmax1 ? 1.f : 0.f;
#pragma unroll
    for (int e = 0; e < CPL; ++e) O[m][e] = 0.f;
  }
  for (int j0 = 0; j0 <= i; j0 += 64) {
    const int j = min(j0 + lane, i);  // lanes past the row read its last key (masked below)
    // opaque per chunk: the q reads are re-issued (broadcast LDS reads), not
    // hoisted out of the loop into 2d registers
    uint32_t qa = (uint32_t)(uintptr_t)qs;
    asm volatile("" : "+v"(qa));
    const lds_f32* qc = (const lds_f32*)(uintptr_t)qa;
    float p[2];
#pragma unroll
    for (int m = 0; m < 2; ++m) {
      const uint16_t* kr = m ? kq1 + (int64_t)j * kst1 : kq0 + (int64_t)j * kst0;
      float acc = 0.f;
      if (rope) {  // key j turned by j * w_c, pairs (c, c + d/2), in fp32
#pragma unroll 2
        for (int c = 0; c < D / 2; c += 8) {
          const uint4 wa = *(const uint4*)(kr + c), wb = *(const uint4*)(kr + c + D / 2);
          const uint32_t ua[4] = {wa.x, wa.y, wa.z, wa.w}, ub[4] = {wb.x, wb.y, wb.z, wb.w};
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const float x1 = __builtin_bit_cast(float, (e & 1) ? ua[e / 2] & 0xffff0000u : ua[e / 2] << 16);
            const float x2 = __builtin_bit_cast(float, (e & 1) ? ub[e / 2] & 0xffff0000u : ub[e / 2] << 16);
            float sn, cs;
            rope_sincos(j, ap->rope_w.hi[c + e], ap->rope_w.lo[c + e], &sn, &cs);
            acc += qc[m * D + c + e] * (x1 * cs - x2 * sn) + qc[m * D + c + e + D / 2] * (x2 * cs + x1 * sn);
          }
        }
      } else {
#pragma unroll 4
        for (int c = 0; c < D; c += 8) {
          const uint4 w = *(const uint4*)(kr + c);
          const uint32_t u[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            acc += __builtin_bit_cast(float, u[e] << 16) * qc[m * D + c + 2 * e];
            acc += __builtin_bit_cast(float, u[e] & 0xffff0000u) * qc[m * D + c + 2 * e + 1];
          }
        }
      }
      const float sc = j0 + lane <= i ? acc * sl2 : -INFINITY;  // log2 units
      float cm = sc;
#pragma unroll
      for (int o = 32; o >= 1; o >>= 1) cm = fmaxf(cm, __shfl_xor(cm, o, 64));
      const float nM = fmaxf(M[m], cm);
      const float al = exp2f(M[m] - nM);
      p[m] = exp2f(sc - nM);
      Z[m] = Z[m] * al + wave_sum(p[m]);
#pragma unroll
      for (int e = 0; e < CPL; ++e) O[m][e] *= al;
      M[m] = nM;
    }
    const int n = min(64, i + 1 - j0);
#pragma unroll 8
    for (int jj = 0; jj < n; ++jj) {
      const float p1 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, p[0]), jj));
      const float p2 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, p[1]), jj));
      const uint16_t* vr = vb + (int64_t)(j0 + jj) * vst;
      float x[CPL];
      if constexpr (CPL == 2) {
        const uint32_t w = *(const uint32_t*)vr;
        x[0] = __builtin_bit_cast(float, w << 16);
        x[1] = __builtin_bit_cast(float, w & 0xffff0000u);
      } else {
        const uint2 w = *(const uint2*)vr;
        x[0] = __builtin_bit_cast(float, w.x << 16);
        x[1] = __builtin_bit_cast(float, w.x & 0xffff0000u);
        x[2] = __builtin_bit_cast(float, w.y << 16);
        x[3] = __builtin_bit_cast(float, w.y & 0xffff0000u);
      }
#pragma unroll
      for (int e = 0; e < CPL; ++e) {
        O[0][e] = fmaf(p1, x[e], O[0][e]);
        O[1][e] = fmaf(p2, x[e], O[1][e]);
      }
    }
  }
  // D = A1 V - lam A2 V, RMSNorm over the 2d channels, (1 - lambda_init)
  const float r1 = 1.f / Z[0], r2 = lam / Z[1];
  float dd[CPL], ss = 0.f;
#pragma unroll
  for (int e = 0; e < CPL; ++e) {
    dd[e] = O[0][e] * r1 - O[1][e] * r2;
    ss += dd[e] * dd[e];
  }
  const float post = (1.f - lam_init) / sqrtf(wave_sum(ss) * (1.f / DV) + 1e-5f);
  uint16_t* dst = (uint16_t*)ap->out.p + b * ap->out.sb + (int64_t)i * ap->out.st + h * ap->out.sh + lane * CPL;
  if constexpr (CPL == 2) {
    *(uint32_t*)dst = pack_bf16x2(dd[0] * post, dd[1] * post);
  } else {
    *(uint2*)dst = make_uint2(pack_bf16x2(dd[0] * post, dd[1] * post), pack_bf16x2(dd[2] * post, dd[3] * post));
  }
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // the next row rewrites qs
}

template <int D, int DV, bool V2, int NW, int MPW, bool PIPE>
__global__ void __launch_bounds__(NW * 64, (Cfg<D, DV, V2, NW, MPW, PIPE>::MIN_BLOCKS))
    prefill_kernel(const PrefillArgs a) {
  using C = Cfg<D, DV, V2, NW, MPW, PIPE>;
  using Sc = Scores<MPW>;
  using Pr = Probs<MPW>;
  constexpr int kBN = C::BN;
  constexpr int KS = C::KS, CB = C::CB;
  __shared__ __attribute__((aligned(1024))) unsigned char smem[C::SMEM];

  // wave index in a scalar register: every per-wave condition derived from it
  // is then a uniform (scalar) branch and does not split basic blocks
  const int tid = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int li = lane & 31, hg = lane >> 5;

  // Work order.  Units (a head / group of one batch entry) are dealt to XCDs
  // round-robin; when every XCD gets the same number of units, each XCD runs
  // its units' tiles heaviest-first across all of them (longest causal rows
  // start first, the L2 still only holds those units' K/V).  Otherwise each
  // XCD gets a contiguous run of (unit, tile) pairs, heaviest tile first.
  int unit, tile;
  {
    const int units = a.nwg / a.tiles;
    if (units % kXcds == 0) {
      const int xcd = blockIdx.x % kXcds, slot = blockIdx.x / kXcds, nu = units / kXcds;
      tile = a.tiles - 1 - slot / nu;
      unit = xcd + kXcds * (slot % nu);
    } else {
      const int logical = xcd_logical_id(blockIdx.x, a.nwg);
      unit = logical / a.tiles;
      tile = a.tiles - 1 - logical % a.tiles;
    }
  }
  const int b = unit / a.units_per_b;
  const int u = unit % a.units_per_b;
  const int T = a.T;

  // ---- roles: which rows and which maps this wave owns ----------------------
  // MPW == 2: the wave holds both maps (V1) / both heads of a pair (V2).
  // MPW == 1: waves 2k (map 1 / even head) and 2k+1 (map 2 / odd head) are
  // partners holding the two maps of the same rows.
  constexpr int WPU = 2 / MPW;           // waves per (rows, map pair) unit
  const int m0 = MPW == 1 ? wave & 1 : 0;  // first map of this wave
  const int slot = wave / WPU;           // (rows, map pair) unit of the workgroup
  int rb, h = 0, pair = 0;
  const uint16_t* qp[MPW];
  int64_t qst[MPW];
  const uint16_t* kp[2];
  int64_t kst[2];
  const uint16_t* vp;
  int64_t vst;
  if constexpr (!V2) {
    h = u;
    rb = slot;
#pragma unroll
    for (int m = 0; m < MPW; ++m) {  // selects, not an indexed array: keeps args out of scratch
      const bool second = m0 + m == 1;
      qp[m] = second ? (const uint16_t*)a.q2.p + b * a.q2.sb + h * a.q2.sh
                     : (const uint16_t*)a.q1.p + b * a.q1.sb + h * a.q1.sh;
      qst[m] = second ? a.q2.st : a.q1.st;
    }
    kp[0] = (const uint16_t*)a.k1.p + b * a.k1.sb + h * a.k1.sh;
    kp[1] = (const uint16_t*)a.k2.p + b * a.k2.sb + h * a.k2.sh;
    kst[0] = a.k1.st;
    kst[1] = a.k2.st;
    vp = (const uint16_t*)a.v.p + b * a.v.sb + h * a.v.sh;
    vst = a.v.st;
  } else {
    // unit slot -> pair slot % pc of this chunk of the group, row block slot / pc
    const int npc = (a.G / 2) / a.pc;  // pair chunks per group
    const int g = u / npc, pcix = u % npc;
    rb = slot / a.pc;
    pair = g * (a.G / 2) + pcix * a.pc + slot % a.pc;
#pragma unroll
    for (int m = 0; m < MPW; ++m) {
      qp[m] = (const uint16_t*)a.q1.p + b * a.q1.sb + (2 * pair + m0 + m) * a.q1.sh;
      qst[m] = a.q1.st;
    }
    kp[0] = kp[1] = (const uint16_t*)a.k1.p + b * a.k1.sb + g * a.k1.sh;
    kst[0] = kst[1] = a.k1.st;
    vp = (const uint16_t*)a.v.p + b * a.v.sb + g * a.v.sh;
    vst = a.v.st;
  }
  const int RB = V2 ? (NW / WPU) / a.pc : NW / WPU;  // row blocks per workgroup
  const int BMT = 32 * RB;
  const int I0 = tile * BMT;
  const int i0w = I0 + 32 * rb;
  const bool active = i0w < T;
  const int kend = min(T, I0 + BMT);
  const int nkt = (kend + kBN - 1) / kBN;

  const uint32_t smem_lds = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) unsigned char*)smem;

  // ---- tile DMA ----------------------------------------------------------------
  // Each wave copies CPW 1 KB chunks per tile.  A chunk slot always covers the
  // same (tensor, rows, swizzled columns) relative to the tile start, so the
  // lane's byte offset is computed once; per tile only the scalar base moves.
  // Rows >= T (last tile only) are clamped to T-1: finite data for keys that
  // every valid query masks.
  uint32_t koff[C::KPW], voff[C::VPW];
#pragma unroll
  for (int i = 0; i < C::KPW; ++i) {
    const int ci = wave + NW * i;  // K chunk of the tile (wave-uniform)
    const int n = ci / (C::KCH / C::NK), cix = ci % (C::KCH / C::NK);
    const int pos = cix * 64 + lane;  // 16 B chunk index inside the K tensor's tile
    const int r = pos / (D / 8), sc = pos % (D / 8);
    koff[i] = (uint32_t)((r * (n ? kst[1] : kst[0]) + (sc ^ k_swizzle<D>(r)) * 8) * 2);
  }
#pragma unroll
  for (int i = 0; i < C::VPW; ++i) {
    const int cix = wave + NW * i;
    const int pos = cix * 64 + lane;
    const int r = pos / (DV / 8), sc = pos % (DV / 8);
    voff[i] = (uint32_t)((r * vst + (sc ^ v_swizzle<DV>(r)) * 8) * 2);
  }
  // K tensors of tile kt into K stage S.
  auto issue_k = [&](int kt, auto stage_c) {
    constexpr int S = decltype(stage_c)::value;
    const int j0 = kt * kBN;
    const bool tail = j0 + kBN > T;  // uniform: rows past the end need clamping
#pragma unroll
    for (int i = 0; i < C::KPW; ++i) {
      const int ci = wave + NW * i;
      const int n = ci / (C::KCH / C::NK), cix = ci % (C::KCH / C::NK);
      const int64_t tst = n ? kst[1] : kst[0];
      uint32_t off = koff[i];
      if (tail) {  // same chunk, row clamped to T-1 (offsets < 2^31: token stride < 2^24)
        const int pos = cix * 64 + lane;
        const int r = pos / (D / 8), sc = pos % (D / 8);
        off = ((uint32_t)min(r, T - 1 - j0) * (uint32_t)tst + (uint32_t)((sc ^ k_swizzle<D>(r)) * 8)) * 2u;
      }
      dma16_sbase((n ? kp[1] : kp[0]) + (int64_t)j0 * tst, off,
                  smem_lds + S * C::KREG + n * C::K_BYTES + cix * 1024);
    }
  };
  // V of tile kt into V stage S.
  auto issue_v = [&](int kt, auto stage_c) {
    constexpr int S = decltype(stage_c)::value;
    const int j0 = kt * kBN;
    const bool tail = j0 + kBN > T;
#pragma unroll
    for (int i = 0; i < C::VPW; ++i) {
      const int cix = wave + NW * i;
      uint32_t off = voff[i];
      if (tail) {
        const int pos = cix * 64 + lane;
        const int r = pos / (DV / 8), sc = pos % (DV / 8);
        off = ((uint32_t)min(r, T - 1 - j0) * (uint32_t)vst + (uint32_t)((sc ^ v_swizzle<DV>(r)) * 8)) * 2u;
      }
      dma16_sbase(vp + (int64_t)j0 * vst, off, smem_lds + C::VBASE + S * C::V_BYTES + cix * 1024);
    }
  };

  // ---- prologue loads, overlapped: the first K/V tile, Q, the V1 lambda
  // vectors / the V2 logit, then (pipelined loop) the second tile.  One wait
  // below retires all but the second tile's copies, so a compiler-placed wait
  // for Q inside the key loop (which would also wait for a tile copy in
  // flight) never happens, the latencies are paid once, and the second tile
  // keeps streaming until the first tile barrier.
  using std::integral_constant;
  issue_k(0, integral_constant<int, 0>{});
  // Q fragments (B operand of S^T = K Q^T): row i0w+li, cols 16ks+8hg
  bf16x8 qf[MPW][KS];
  {
    const int row = i0w + li;
#pragma unroll
    for (int m = 0; m < MPW; ++m)
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
        qf[m][ks] = as_bf16x8(row < T ? *(const uint4*)(qp[m] + (int64_t)row * qst[m] + 16 * ks + 8 * hg)
                                      : make_uint4(0, 0, 0, 0));
  }
  // V2: this row's lambda logit for the pair (used by the wave holding the odd head)
  float lgit = 0.f;
  if constexpr (V2) {
    const int row = i0w + li;
    if ((MPW == 2 || m0 == 1) && row < T)
      lgit = ((const float*)a.lam.p)[b * a.lam.sb + (int64_t)row * a.lam.st + pair * a.lam.sh];
  }
  constexpr int LPL = (D + 63) / 64;  // lambda vector elements per lane
  float lv[4][LPL];
  if constexpr (!V2) {
    const float* lp[4] = {a.lq1, a.lk1, a.lq2, a.lk2};
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int i = 0; i < LPL; ++i) lv[j][i] = lane + 64 * i < D ? lp[j][lane + 64 * i] : 0.f;
  }
  // V of tile 0 after Q: the pipelined loop's first P.V is the next step's
  // (after the first tile barrier), so outside the first row tile the wait
  // below leaves V(0) in flight too; then the copies of tile 1, issued last.
  issue_v(0, integral_constant<int, 0>{});
  constexpr int kT1 = PIPE ? C::KPW + (C::NSTV == 3 ? C::VPW : 0) : 0;
  // (in the first row tile a wave with one sub-block drains its P.V at step 0)
  const bool v0_in_flight = PIPE && nkt > 1 && I0 > 0;
  if constexpr (PIPE) {
    if (nkt > 1) {
      issue_k(1, integral_constant<int, 1>{});
      if constexpr (C::NSTV == 3) issue_v(1, integral_constant<int, 1>{});
    }
  }
  // Every value loaded above passes through one of these waits, so the
  // compiler sees it as available from here on and places no wait of its own
  // later (such a wait would also hold up tile 1's copies).
  auto retire = [&](auto& v) {
    if (v0_in_flight)
      asm volatile("s_waitcnt vmcnt(%1)" : "+v"(v) : "n"(kT1 + C::VPW));
    else if (PIPE && nkt > 1)
      asm volatile("s_waitcnt vmcnt(%1)" : "+v"(v) : "n"(kT1));
    else
      asm volatile("s_waitcnt vmcnt(0)" : "+v"(v));
  };
#pragma unroll
  for (int m = 0; m < MPW; ++m)
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) retire(qf[m][ks]);
  if constexpr (V2) {
    retire(lgit);
  } else {
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int i = 0; i < LPL; ++i) retire(lv[j][i]);
  }
  if (a.rope) {  // rotary embedding of this wave's q rows (row i0w + li, elements 16 ks + 8 hg + e)
#pragma unroll
    for (int m = 0; m < MPW; ++m) rope_rotate_frags<KS, 16>(qf[m], 8 * hg, i0w + li, a.rope_w);
  }

  // ---- per-lane LDS bases (every stage / sub-block / map offset is an immediate) ----
  // K chunk (2ks + hg) of tile row r = 32 sb + li sits at chunk (2ks + hg) ^ k_swizzle(li)
  // of the map's K tensor (V1: K2 follows K1 in a stage).
  uint32_t kbase[KS];  // LDS byte addresses
#pragma unroll
  for (int ks = 0; ks < KS; ++ks)
    kbase[ks] = smem_lds + (V2 ? 0 : m0 * C::K_BYTES) + li * (D * 2) + (((2 * ks + hg) ^ k_swizzle<D>(li)) << 4);
  // Opaque to the compiler: it would otherwise rebuild each base from shared
  // parts inside the key loop (one VALU add per operand read).
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) asm volatile("" : "+v"(kbase[ks]));
  // V^T operand via transpose reads: lane (G16 = lane>>4, l16 = lane&15) points at
  // row 4*(G16>>1) + (l16>>2) (+ sub-block, k-step), columns 32cb + 16(G16&1) + 4(l16&3),
  // i.e. chunk 4cb + cl.  The swizzle only permutes chunks within aligned groups of
  // 4*NV, so the per-lane offset depends on cb only through cb % NV.
  constexpr int NV = DV >= 128 ? 4 : 2;
  uint32_t vbase[NV];
  {
    const int l16 = lane & 15, g16 = lane >> 4;
    const int vr = 4 * (g16 >> 1) + (l16 >> 2);
    const int cl = 2 * (g16 & 1) + ((l16 & 3) >> 1);
    const int x = v_swizzle<DV>(vr);  // rows of one read share r & 3 = l16 >> 2
#pragma unroll
    for (int v = 0; v < NV; ++v)
      vbase[v] = smem_lds + C::VBASE + vr * (DV * 2) + (((4 * v + cl) ^ x) - 4 * v) * 16 + (l16 & 1) * 8;
#pragma unroll
    for (int v = 0; v < NV; ++v) asm volatile("" : "+v"(vbase[v]));
  }

  // ---- V1 lambda (one fp32 scalar per call) ----
  float lam = 0.f;
  if constexpr (!V2) {
    float pa = 0.f, pb = 0.f;
#pragma unroll
    for (int i = 0; i < LPL; ++i) {
      pa += lv[0][i] * lv[1][i];
      pb += lv[2][i] * lv[3][i];
    }
    pa = wave_sum(pa);
    pb = wave_sum(pb);
    lam = expf(pa) - expf(pb) + a.lam_init;
  }

  if constexpr (MPW == 2) {
    // With two maps per wave the working set exceeds 256 VGPRs.  An inline
    // asm operand in an AGPR makes the backend select the MFMA forms whose
    // accumulators live in AGPRs (O stays there between MFMAs) instead of
    // VGPR forms with AGPRs used as spill space.
    asm volatile("" ::"a"(0.f));
  }
  const float sl2 = a.sl2;
  float nm[MPW], lsum[MPW];  // minus the reference m of this lane's row (log2 units); row sum
  f32x16 o[MPW][CB];
#pragma unroll
  for (int m = 0; m < MPW; ++m) {
    nm[m] = -kMInit;
    lsum[m] = 0.f;
#pragma unroll
    for (int cb = 0; cb < CB; ++cb)
#pragma unroll
      for (int r = 0; r < 16; ++r) o[m][cb][r] = 0.f;
  }

  // ---- building blocks of one 32-key sub-block --------------------------------
  // (s_setprio around the MFMA sections only in the unpipelined loop: it
  // bounds the compiler's scheduling regions.)
  constexpr bool kPrio = DA_SETPRIO && !PIPE;
  // S^T (32 keys x 32 rows per map) of the sub-block at K offset KO.  V2: one
  // K fragment feeds every map of the wave.
  auto qk = [&](auto koffc) {
    constexpr int KO = decltype(koffc)::value;
    asm volatile("");  // not a constant expression (see the note above Scores)
    Sc r;
#pragma unroll
    for (int m = 0; m < MPW; ++m)
#pragma unroll
      for (int i = 0; i < 16; ++i) r.s[m][i] = 0.f;
    if (kPrio) __builtin_amdgcn_s_setprio(2);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      if constexpr (V2) {
        const bf16x8 ka = lds_read16(kbase[ks] + KO);
#pragma unroll
        for (int m = 0; m < MPW; ++m) r.s[m] = mfma32x32x16(ka, qf[m][ks], r.s[m]);
      } else {
#pragma unroll
        for (int m = 0; m < MPW; ++m)
          r.s[m] = mfma32x32x16(lds_read16(kbase[ks] + KO + m * C::K_BYTES), qf[m][ks], r.s[m]);
      }
    }
    if (kPrio) __builtin_amdgcn_s_setprio(0);
    return r;
  };
  // O^T += V^T P^T over the sub-block at V offset VO; one V fragment feeds
  // every map of the wave.
  auto pv = [&](auto voffc, const Pr& P) {
    constexpr int VO = decltype(voffc)::value;
    if (kPrio) __builtin_amdgcn_s_setprio(2);
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
#pragma unroll
      for (int cb = 0; cb < CB; ++cb) {
        const uint32_t q = vbase[cb % NV] + VO + 16 * kk * (DV * 2) + cb * 64;
        const bf16x8 va = join_bf16x8(tr_read(q), tr_read(q + 8 * (DV * 2)));
#pragma unroll
        for (int m = 0; m < MPW; ++m) o[m][cb] = mfma32x32x16(va, P.p[m][kk], o[m][cb]);
      }
    }
    if (kPrio) __builtin_amdgcn_s_setprio(0);
  };
  // Causal mask of the diagonal sub-block: key 8(r>>2) + 4hg + (r&3) is
  // masked for row li when 8(r>>2) + (r&3) > li - 4hg.  The threshold is
  // opaque so the 16 compares stay here instead of being hoisted into 32
  // live SGPRs.
  auto mask_diag = [&](Sc& S) {
    int t = li - 4 * hg;
    asm volatile("" : "+v"(t));
#pragma unroll
    for (int m = 0; m < MPW; ++m)
#pragma unroll
      for (int r = 0; r < 16; ++r)
        if (8 * (r >> 2) + (r & 3) > t) S.s[m][r] = -INFINITY;
  };
  // Probabilities as the bf16 B operand of P.V and the lane's block sums bs,
  // computed in place over the scores (no branch: part of the steady-state
  // scheduling region).
  auto softmax_exps = [&](Sc& S, Pr& P) {
#pragma unroll
    for (int m = 0; m < MPW; ++m) {
#pragma unroll
      for (int r = 0; r < 16; ++r) S.s[m][r] = __builtin_amdgcn_exp2f(fmaf(S.s[m][r], sl2, nm[m]));
      f32x8 e0, e1;
#pragma unroll
      for (int r = 0; r < 8; ++r) {
        e0[r] = S.s[m][r];
        e1[r] = S.s[m][r + 8];
      }
      P.p[m][0] = cvt_bf16x8(e0);
      P.p[m][1] = cvt_bf16x8(e1);
      P.bs[m] = sum_bf16x8(P.p[m][1], sum_bf16x8(P.p[m][0], 0.f));
    }
  };
  // The rare exact path, taken when some lane's block sum is above the cap:
  // the sub-block's scores again (rescore(): its K is still in LDS), each
  // map's m moved to its row maximum over both lane halves, O and l rescaled,
  // the exponentials redone.  Then the running sums.
  auto softmax_finish = [&](auto rescore, bool diag, Pr& P) {
    bool any = false;
#pragma unroll
    for (int m = 0; m < MPW; ++m) any |= !(P.bs[m] <= kSumCap);
    if (__builtin_amdgcn_ballot_w64(any)) {
      Sc S;
      S = rescore();
      if (diag) mask_diag(S);
#pragma unroll
      for (int m = 0; m < MPW; ++m) {
        float mx = S.s[m][0];
#pragma unroll
        for (int r = 1; r < 16; ++r) mx = fmaxf(mx, S.s[m][r]);
        const float mnew = fmaxf(-nm[m], max_across_halves(mx) * sl2);
        const float al = __builtin_amdgcn_exp2f(-nm[m] - mnew);
        nm[m] = -mnew;
        lsum[m] *= al;
#pragma unroll
        for (int cb = 0; cb < CB; ++cb)
#pragma unroll
          for (int r = 0; r < 16; ++r) o[m][cb][r] *= al;
      }
      softmax_exps(S, P);
    }
#pragma unroll
    for (int m = 0; m < MPW; ++m) lsum[m] += P.bs[m];
  };

  if constexpr (!PIPE) {
    // ---- key loop: 2-stage ring, unrolled by stage; each sub-block in order --
    auto tile_step = [&](int kt, auto stage_c) {
      constexpr int S = decltype(stage_c)::value;
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // this wave's part of tile kt landed
      __syncthreads();                                  // all parts landed; other stage free
      if (kt + 1 < nkt) {
        issue_k(kt + 1, integral_constant<int, 1 - S>{});
        issue_v(kt + 1, integral_constant<int, 1 - S>{});
      }
      if (!active) return;
      const int j0 = kt * kBN;
      static_for<0, C::NSB>([&](auto sbc) {
        constexpr int SB = decltype(sbc)::value;
        const int jb = j0 + 32 * SB;
        if (jb > i0w) return;  // sub-block entirely above this wave's diagonal
        using cur_k = integral_constant<int, S * C::KREG + 32 * SB * D * 2>;
        using cur_v = integral_constant<int, S * C::V_BYTES + 32 * SB * DV * 2>;
        const bool diag = jb == i0w;
        Sc Sb;
        Sb = qk(cur_k{});
        if (diag) mask_diag(Sb);
        Pr P;
        softmax_exps(Sb, P);
        softmax_finish([&]() { return qk(cur_k{}); }, diag, P);
        pv(cur_v{}, P);
      });
    };
    for (int kt = 0; kt < nkt; kt += 2) {  // (tile 0 was issued in the prologue)
      tile_step(kt, integral_constant<int, 0>{});
      if (kt + 1 >= nkt) break;
      tile_step(kt + 1, integral_constant<int, 1>{});
    }
  } else {
    // ---- key loop: K in a 3-stage ring, V in an NSTV-stage ring, software-
    // pipelined over sub-blocks.  Step n (this wave's n-th sub-block) issues,
    // in one basic block, the P.V MFMAs of sub-block n-1 and the score MFMAs
    // of sub-block n+1 alongside the exponentials of sub-block n, so matrix
    // and vector work of one wave overlap.
    // Tile kt's K sits in K stage kt % 3 and its V in V stage kt % NSTV.
    // Before the last sub-block of tile kt (whose step computes the scores of
    // tile kt+1) every wave waits for its copies and meets at a barrier; then:
    //   * K of tile kt+2 goes to K stage (kt+2) % 3, last read by the scores
    //     of tile kt-1's last sub-block (step (kt-1, NSB-2));
    //   * V of tile kt+NSTV-1 goes to V stage (kt-1) % NSTV, last read by the
    //     P.V of tile kt-1's last sub-block (step (kt, 0)).
    // Every wave has passed both steps at that barrier.  K lands two steps
    // before its first reader, V 2 (NSTV - 1) steps before.
    const int nsub = active ? i0w / 32 + 1 : 0;  // sub-blocks up to the diagonal
    // Scheduling of the steady-state step: NMF MFMAs (P.V of the previous
    // sub-block, scores of the next), NRD LDS operand reads and the
    // exponentials of this sub-block (~52 VALU instructions per map) dealt
    // out in turn: DA_HINT_LEAD reads first, then per MFMA DA_HINT_VPER
    // vector instructions and its share of the reads (8 and 3 measured ~2%
    // faster on the V2 prefill than two reads ahead and an even split of
    // the vector work).
    auto interleave_hints = [&]() {
      constexpr int NMF = MPW * (2 * CB + KS);
      constexpr int NRD = 4 * CB + (V2 ? 1 : MPW) * KS;
      constexpr int VPER = DA_HINT_VPER;
      constexpr int RPER = (NRD + NMF - 1) / NMF;
      __builtin_amdgcn_sched_group_barrier(0x100, DA_HINT_LEAD, 0);  // DS reads
      static_for<0, NMF>([&](auto) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);     // MFMA
        __builtin_amdgcn_sched_group_barrier(0x002, VPER, 0);  // VALU
        __builtin_amdgcn_sched_group_barrier(0x100, RPER, 0);  // DS reads
      });
    };
    Sc Scur;
    Pr pp;  // probabilities of the previous sub-block, P.V pending
#pragma unroll
    for (int m = 0; m < MPW; ++m) pp.p[m][0] = pp.p[m][1] = as_bf16x8(make_uint4(0, 0, 0, 0));
    {  // zero the V slot read as "the previous sub-block" at n = 0 (last V stage, last sub-block)
      constexpr int ZB = 32 * DV * 2, Z0 = C::VBASE + (C::NSTV - 1) * C::V_BYTES + 32 * (C::NSB - 1) * DV * 2;
      for (int i = tid * 16; i < ZB; i += NW * 64 * 16) *(uint4*)(smem + Z0 + i) = make_uint4(0, 0, 0, 0);
    }
    __syncthreads();  // K (and, in the first row tile, V) of tile 0 visible; the rest is waited for at the first tile barrier
    if (nsub > 0) Scur = qk(integral_constant<int, 0>{});
    auto tile_step = [&](int kt, auto kstage_c, auto vstage_c) {
      constexpr int SK = decltype(kstage_c)::value, SV = decltype(vstage_c)::value;
      static_for<0, C::NSB>([&](auto sbc) {
        constexpr int SB = decltype(sbc)::value;
        if constexpr (SB == C::NSB - 1) {
          if (kt + 1 < nkt) {
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // this wave's copies landed
            __syncthreads();
            if (kt + 2 < nkt) issue_k(kt + 2, integral_constant<int, (SK + 2) % 3>{});
            if (kt + C::NSTV - 1 < nkt)
              issue_v(kt + C::NSTV - 1, integral_constant<int, (SV + C::NSTV - 1) % C::NSTV>{});
          }
        }
        const int n = kt * C::NSB + SB;
        if (n >= nsub) return;
        constexpr int PSV = SB > 0 ? SV : (SV + C::NSTV - 1) % C::NSTV, PSB = SB > 0 ? SB - 1 : C::NSB - 1;  // prev
        constexpr int NSK = SB + 1 < C::NSB ? SK : (SK + 1) % 3, NSBI = SB + 1 < C::NSB ? SB + 1 : 0;  // next
        using prev_v = integral_constant<int, PSV * C::V_BYTES + 32 * PSB * DV * 2>;
        using next_k = integral_constant<int, NSK * C::KREG + 32 * NSBI * D * 2>;
        using cur_v = integral_constant<int, SV * C::V_BYTES + 32 * SB * DV * 2>;
        using cur_k = integral_constant<int, SK * C::KREG + 32 * SB * D * 2>;
        // One straight-line step for every n.  At n = 0 the P.V of "the
        // previous sub-block" multiplies zero probabilities with a zeroed V
        // slot; at the last step the score MFMAs of "the next sub-block" read
        // whatever that LDS holds and their result is dropped.
        const bool last = n + 1 == nsub;
        if (last) mask_diag(Scur);  // the diagonal is this wave's last sub-block
        pv(prev_v{}, pp);
        Sc Snext;
        Snext = qk(next_k{});
        softmax_exps(Scur, pp);
        if (!DA_NO_HINTS) interleave_hints();
        softmax_finish([&]() { return qk(cur_k{}); }, last, pp);
        if (last) pv(cur_v{}, pp);  // drain
        Scur = Snext;
      });
    };
    // unrolled over the period of the two rings
    constexpr int PER = C::NSTV == 3 ? 3 : 6;
    for (int kt0 = 0; kt0 < nkt; kt0 += PER) {
      bool done = false;
      static_for<0, PER>([&](auto ic) {
        constexpr int I = decltype(ic)::value;
        if (done || kt0 + I >= nkt) {
          done = true;
          return;
        }
        tile_step(kt0 + I, integral_constant<int, I % 3>{}, integral_constant<int, I % C::NSTV>{});
      });
    }
  }

  // ---- epilogue ----------------------------------------------------------------
  const int row = i0w + li;
  float inv[MPW];
#pragma unroll
  for (int m = 0; m < MPW; ++m) {
    // off-by-one softmax: one more logit 0, i.e. 2^(0 - m) against the row's reference m
    const float extra = a.softmax1 ? __builtin_amdgcn_exp2f(nm[m]) : 0.f;
    inv[m] = 1.f / (lsum[m] + __shfl_xor(lsum[m], 32, 64) + extra);
  }
  // Training forward: this wave's map (V1) / head (V2) output, normalised,
  // and the row's log2-sum-exp2, lse = m + log2(denominator) = -nm - log2(inv).
  // V1: map outputs in attn (map 1) and attn2 (map 2), lse [2][B][H][T];
  // V2: head outputs in attn, lse [B][Hq][T].
  if (a.lse != nullptr && active && row < T) {
#pragma unroll
    for (int m = 0; m < MPW; ++m) {
      const int mi = m0 + m;
      const int head = V2 ? 2 * pair + mi : h;
      const int64_t li_ = V2 ? ((int64_t)b * (a.H * a.G) + head) * T + row
                             : (((int64_t)mi * a.B + b) * a.H + h) * T + row;
      if (hg == 0) a.lse[li_] = -nm[m] - log2f(inv[m]);
      const TOut& at = (!V2 && mi == 1) ? a.attn2 : a.attn;
      uint16_t* ad = (uint16_t*)at.p + b * at.sb + (int64_t)row * at.st + (int64_t)head * at.sh;
#pragma unroll
      for (int cb = 0; cb < CB; ++cb)
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
          uint2 w;
          w.x = pack_bf16x2(o[m][cb][4 * g4 + 0] * inv[m], o[m][cb][4 * g4 + 1] * inv[m]);
          w.y = pack_bf16x2(o[m][cb][4 * g4 + 2] * inv[m], o[m][cb][4 * g4 + 3] * inv[m]);
          *(uint2*)(ad + 32 * cb + 8 * g4 + 4 * hg) = w;
        }
    }
  }
  // weight of the second map: lam / l2 (V1) or sigmoid(lam[t, p]) / l_odd (V2)
  auto second_weight = [&](float inv2) {
    if constexpr (V2) {
      return sigmoid_f32(lgit) * inv2;
    } else {
      return lam * inv2;
    }
  };
  float ss = 0.f, s12 = 0.f;  // sums of D^2 and of (A1 V)^2 + (lam A2 V)^2 (V1 cancellation guard)
  if constexpr (MPW == 1) {
    // map 2's wave hands its weighted O to its partner through LDS
    if constexpr (!C::SEPX) __syncthreads();  // every wave is done with the K/V stages
    // 16-byte chunks (four accumulator registers) in lane order: conflict-free
    f32x4* xch = (f32x4*)(smem + C::XBASE) + slot * (CB * 4 * 64);
    if (m0 == 1) {
      if (active) {
        const float w = second_weight(inv[0]);
#pragma unroll
        for (int cb = 0; cb < CB; ++cb)
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            f32x4 x;
#pragma unroll
            for (int j = 0; j < 4; ++j) x[j] = o[0][cb][4 * g + j] * w;
            xch[(cb * 4 + g) * 64 + lane] = x;
          }
      }
      __syncthreads();
      return;
    }
    __syncthreads();
    if (!active) return;
#pragma unroll
    for (int cb = 0; cb < CB; ++cb)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const f32x4 x = xch[(cb * 4 + g) * 64 + lane];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float a1 = o[0][cb][4 * g + j] * inv[0];
          const float dv = a1 - x[j];
          o[0][cb][4 * g + j] = dv;
          ss += dv * dv;
          if constexpr (!V2) s12 += a1 * a1 + x[j] * x[j];
        }
      }
  } else {
    static_assert(V2 || MPW == 1, "the V1 cancellation guard uses the partner exchange slots");
    if (!active) return;
    const float w = second_weight(inv[1]);
#pragma unroll
    for (int cb = 0; cb < CB; ++cb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float dv = o[0][cb][r] * inv[0] - w * o[1][cb][r];
        o[0][cb][r] = dv;
        ss += dv * dv;
      }
  }
  uint16_t* dst;
  float post = 1.f;
  uint64_t flagged = 0;  // V1: rows (bit li) whose maps cancel, recomputed exactly below
  if constexpr (!V2) {
    ss += __shfl_xor(ss, 32, 64);
    s12 += __shfl_xor(s12, 32, 64);
    flagged = __ballot(row < T && s12 > kCancel2 * ss) & 0xffffffffull;
    post = (1.f - a.lam_init) / sqrtf(ss * (1.f / DV) + 1e-5f);
    dst = (uint16_t*)a.out.p + b * a.out.sb + (int64_t)row * a.out.st + h * a.out.sh;
  } else {
    dst = (uint16_t*)a.out.p + b * a.out.sb + (int64_t)row * a.out.st + pair * a.out.sh;
  }
  if (row < T && !((flagged >> li) & 1)) {
#pragma unroll
    for (int cb = 0; cb < CB; ++cb)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const int c = 32 * cb + 8 * g4 + 4 * hg;
        uint2 w;
        w.x = pack_bf16x2(o[0][cb][4 * g4 + 0] * post, o[0][cb][4 * g4 + 1] * post);
        w.y = pack_bf16x2(o[0][cb][4 * g4 + 2] * post, o[0][cb][4 * g4 + 3] * post);
        *(uint2*)(dst + c) = w;
      }
  }
  if constexpr (!V2) {
    if (flagged) {
      // this slot's exchange area (map 2's values were read above) holds the q rows
      lds_f32* buf = (lds_f32*)(uintptr_t)(smem_lds + C::XBASE) + slot * (CB * 4 * 64 * 4);
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      while (flagged) {
        const int r = __builtin_ctzll(flagged);
        flagged &= flagged - 1;
        v1_exact_row<D, DV>(b, h, i0w + r, lam, buf, lane);
      }
    }
  }
}

template <int D, int DV, bool V2, int NW, int MPW, bool PIPE>
hipError_t launch(const PrefillArgs& a, hipStream_t s) {
  const void* args[] = {&a};
  return hipLaunchKernel((const void*)prefill_kernel<D, DV, V2, NW, MPW, PIPE>, dim3(a.nwg), dim3(NW * 64),
                         (void**)args, 0, s);
}

}  // namespace

// Kernel shape by workload: waves per workgroup (NW), maps per wave (MPW),
// pipelined key loop (PIPE).  Rows per workgroup = 32 * NW * MPW / 2 (V1).
#ifndef DA_V1_D64_NW
#define DA_V1_D64_NW 8
#endif
#ifndef DA_V1_D64_MPW
#define DA_V1_D64_MPW 1
#endif
#ifndef DA_V1_D64_PIPE
#define DA_V1_D64_PIPE true
#endif
#ifndef DA_V1_D128_NW
#define DA_V1_D128_NW 8
#endif
#ifndef DA_V1_D128_MPW
#define DA_V1_D128_MPW 1
#endif
#ifndef DA_V1_D128_PIPE
#define DA_V1_D128_PIPE false
#endif
#ifndef DA_V2_NW
#define DA_V2_NW 8
#endif
#ifndef DA_V2_MPW
#define DA_V2_MPW 1
#endif
#ifndef DA_V2_PIPE
#define DA_V2_PIPE true
#endif

hipError_t launch_prefill_v1_bf16(int d, const PrefillArgs& a0, hipStream_t s) {
  PrefillArgs a = a0;
  a.units_per_b = a.H;
  auto geom = [&](int nw, int mpw) {
    const int BMT = 32 * (nw * mpw / 2);  // rows per workgroup
    a.tiles = (a.T + BMT - 1) / BMT;
    a.nwg = a.B * a.H * a.tiles;
  };
  if (d == 64) {
    geom(DA_V1_D64_NW, DA_V1_D64_MPW);
    return launch<64, 128, false, DA_V1_D64_NW, DA_V1_D64_MPW, DA_V1_D64_PIPE>(a, s);
  }
  if (d == 128) {
    geom(DA_V1_D128_NW, DA_V1_D128_MPW);
    return launch<128, 256, false, DA_V1_D128_NW, DA_V1_D128_MPW, DA_V1_D128_PIPE>(a, s);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_prefill_v2_bf16(int d, const PrefillArgs& a0, hipStream_t s) {
  PrefillArgs a = a0;
  const int np = a.G / 2;
  const int units = DA_V2_NW * DA_V2_MPW / 2;  // (pair, row block) slots per workgroup
  a.pc = np % units == 0 ? units : np % 2 == 0 && units % 2 == 0 ? 2 : 1;
  if (a.pc > units) a.pc = 1;
  const int BMT = 32 * (units / a.pc);
  a.tiles = (a.T + BMT - 1) / BMT;
  a.units_per_b = a.H * (np / a.pc);
  a.nwg = a.B * a.units_per_b * a.tiles;
  if (d == 64) return launch<64, 64, true, DA_V2_NW, DA_V2_MPW, DA_V2_PIPE>(a, s);
  if (d == 128) return launch<128, 128, true, DA_V2_NW, DA_V2_MPW, DA_V2_PIPE>(a, s);
  return hipErrorInvalidValue;
}

}  // namespace da
