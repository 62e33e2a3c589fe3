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
//   * K and V tiles of 64 keys go HBM -> LDS with global_load_lds_dwordx4
//     (no registers, no VALU), double-buffered: the next tile streams in
//     while the current one is consumed; one barrier per tile.  In LDS both
//     stay row-major with an XOR swizzle of their 16-byte chunks, so the
//     MFMA operand reads are bank-conflict-free (256 B per clock).
//   * Scores are computed transposed, S^T = K Q^T, with
//     v_mfma_f32_32x32x16_bf16: Q fragments stay in registers for the whole
//     key loop, each lane holds 16 scores of ONE query row (softmax state is
//     per lane), and the fp32 score registers convert in place to the bf16 B
//     operand of O^T = V^T P^T.  The V^T A operand comes straight from the
//     row-major V tile through ds_read_b64_tr_b16 (the LDS transpose read).
//   * Online softmax in the log2 domain with a lazily updated reference max:
//     O and l are only rescaled when a row's max grows by more than 2^8,
//     which keeps every exponent <= 2^8 and the result exact up to rounding.
//   * Work split.  A wave owns 32 query rows.  MPW = 2: the wave carries
//     both maps (V1: map 1 and map 2 of one differential head; V2: the two
//     heads of a pair), so a V fragment read once feeds two MFMAs.  MPW = 1:
//     the two maps of the same rows sit in two partner waves (halving the
//     accumulator registers, so two waves fit per SIMD) and are combined
//     through LDS at the end.  For V2 the waves of a workgroup cover the
//     heads of one GQA group, so each K/V tile is loaded once for the whole
//     group.
//   * Causal skipping at 32-key granularity (mask only on diagonal
//     sub-blocks); heaviest tiles first; workgroups mapped onto XCDs so the
//     tiles of one head share an L2.
#include <math.h>

#include <type_traits>

#include "kernels.hpp"

namespace da {
namespace {

constexpr float kLazyLog2 = 8.f;  // rescale only when the max grows by > 2^8
#ifndef DA_V2_BN
#define DA_V2_BN 128  // keys per LDS stage of the V2 kernel (64 or 128)
#endif
#ifndef DA_TILE_SOFTMAX
#define DA_TILE_SOFTMAX 0  // one max/rescale decision per two visible sub-blocks (slower on MI355X)
#endif
#ifndef DA_SETPRIO
#define DA_SETPRIO 1  // raise wave priority while issuing MFMA sections
#endif

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(3))) s16x4 lds_s16x4_t;

// 16 bytes per lane, HBM -> LDS (global_load_lds_dwordx4): lane l's bytes
// land at LDS byte address lds_addr + 16 l; lds_addr must be wave-uniform.
// Issued as inline asm so the compiler does not track it: it would otherwise
// make every LDS read wait for the copy in flight, although that copy only
// ever targets the other LDS stage.  The kernel waits for it explicitly
// (vmcnt(0) + barrier) before the stage is read.  M0 is used by nothing else
// in these kernels.
__device__ __forceinline__ void dma16(const void* g, uint32_t lds_addr) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
               :
               : "v"(g), "s"(__builtin_amdgcn_readfirstlane(lds_addr))
               : "memory");
}

// Same copy with a wave-uniform 64-bit base in SGPRs and a per-lane 32-bit
// byte offset (the global_load "saddr" form): no per-lane address arithmetic.
__device__ __forceinline__ void dma16_sbase(const void* base, uint32_t off, uint32_t lds_addr) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1"
               :
               : "v"(off), "s"(base), "s"(__builtin_amdgcn_readfirstlane(lds_addr))
               : "memory");
}

// LDS transpose read: in each group of 16 lanes, lane j receives element
// (j & 3) of the 4-element rows addressed by lanes 4k + (j >> 2), k = 0..3.
__device__ __forceinline__ uint2 tr_read(const unsigned char* p) {
  const s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)p);
  return __builtin_bit_cast(uint2, v);
}

template <int I, int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (I < N) {
    f(std::integral_constant<int, I>{});
    static_for<I + 1, N>(f);
  }
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

template <int D, int DV, bool V2, int NW, int MPW, bool PIPE>
struct Cfg {
  static constexpr int NT = NW * 64;
  static constexpr int KS = D / 16;   // k-steps of the score MFMA
  static constexpr int CB = DV / 32;  // 32-wide column blocks of O^T
  static constexpr int NK = V2 ? 1 : 2;
  // PIPE: 32-key tiles in a 4-stage ring (software-pipelined key loop);
  // otherwise 64-key tiles, double-buffered.
  static constexpr int BN = PIPE ? 32 : (V2 ? DA_V2_BN : 64);
  static constexpr int NST = PIPE ? 4 : 2;
  static constexpr int K_BYTES = BN * D * 2;
  static constexpr int V_BYTES = BN * DV * 2;
  static constexpr int STAGE = NK * K_BYTES + V_BYTES;
  static constexpr int KCH = K_BYTES / 1024;  // 1 KB DMA instructions per K tensor
  static constexpr int VCH = V_BYTES / 1024;
  static constexpr int NCH = NK * KCH + VCH;
  static constexpr int CPW = NCH / NW;        // DMA instructions per wave per tile
  static_assert(NCH % NW == 0, "tile DMA split");
  static_assert(D >= 64 && DV >= 64, "swizzles assume >= 8 chunks per row");
  // MPW == 1: one exchange slot per partner-wave pair (fp32, lane-native order)
  static constexpr int XBYTES = MPW == 1 ? (NW / 2) * CB * 16 * 64 * 4 : 0;
  static constexpr int SMEM = NST * STAGE > XBYTES ? NST * STAGE : XBYTES;
  static constexpr int MIN_BLOCKS = NW == 4 ? 2 : 1;  // two waves per SIMD
  // sub-blocks per softmax group (registers permitting: two score tiles per wave)
  static constexpr int SMG = (DA_TILE_SOFTMAX && !PIPE && DV <= 128 && BN >= 64) ? 2 : 1;
};

template <int MPW>
struct Scores {
  f32x16 s[MPW];
};
template <int MPW>
struct Probs {
  bf16x8 p[MPW][2];
};

template <int D, int DV, bool V2, int NW, int MPW, bool PIPE>
__global__ void __launch_bounds__(NW * 64, (Cfg<D, DV, V2, NW, MPW, PIPE>::MIN_BLOCKS))
    prefill_kernel(const PrefillArgs a) {
  using C = Cfg<D, DV, V2, NW, MPW, PIPE>;
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

  // ---- roles: which rows and maps this wave owns ----------------------------
  int RB, rb, m0 = 0, h = 0, pair = 0;
  const uint16_t* qp[2];
  int64_t qst[2];
  const uint16_t* kp[2];
  int64_t kst[2];
  const uint16_t* vp;
  int64_t vst;
  if constexpr (!V2) {
    h = u;
    if constexpr (MPW == 2) {
      RB = NW;
      rb = wave;
    } else {
      RB = NW / 2;
      rb = wave >> 1;
      m0 = wave & 1;  // this wave's map
    }
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
    const int npc = (a.G / 2) / a.pc;  // pair chunks per group
    const int g = u / npc, pcix = u % npc;
    // MPW == 2: wave w -> pair w % pc, row block w / pc.
    // MPW == 1: waves 2k (even head) and 2k+1 (odd head) share pair k % pc and
    //           row block k / pc.
    const int pw = MPW == 2 ? wave : wave >> 1;
    if constexpr (MPW == 1) m0 = wave & 1;
    RB = (MPW == 2 ? NW : NW / 2) / a.pc;
    rb = pw / a.pc;
    pair = g * (a.G / 2) + pcix * a.pc + pw % a.pc;
#pragma unroll
    for (int m = 0; m < MPW; ++m) qp[m] = (const uint16_t*)a.q1.p + b * a.q1.sb + (2 * pair + m0 + m) * a.q1.sh;
    qst[0] = qst[1] = a.q1.st;
    kp[0] = kp[1] = (const uint16_t*)a.k1.p + b * a.k1.sb + g * a.k1.sh;
    kst[0] = kst[1] = a.k1.st;
    vp = (const uint16_t*)a.v.p + b * a.v.sb + g * a.v.sh;
    vst = a.v.st;
  }
  const int BMT = 32 * RB;
  const int I0 = tile * BMT;
  const int i0w = I0 + 32 * rb;
  const bool active = i0w < T;
  const int kend = min(T, I0 + BMT);
  const int nkt = (kend + kBN - 1) / kBN;

  const uint32_t smem_lds = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) unsigned char*)smem;

  // ---- tile DMA: wave issues CPW 1 KB chunks; rows >= T are clamped to T-1
  // (finite data; those keys are always masked for every valid query) ----
  // Each wave copies CPW 1 KB chunks per tile.  A chunk slot always covers the
  // same (tensor, rows, swizzled columns) relative to the tile start, so the
  // lane's byte offset is computed once; per tile only the scalar base moves.
  // Rows >= T (last tile only) are clamped to T-1: finite data for keys that
  // every valid query masks.
  uint32_t dma_off[C::CPW];
#pragma unroll
  for (int i = 0; i < C::CPW; ++i) {
    const int ci = wave + NW * i;  // chunk of the stage (wave-uniform)
    if (ci < C::NK * C::KCH) {
      const int n = ci / C::KCH, cix = ci % C::KCH;
      const int pos = cix * 64 + lane;  // 16 B chunk index inside the K tile
      const int r = pos / (D / 8), sc = pos % (D / 8);
      dma_off[i] = (uint32_t)((r * (n ? kst[1] : kst[0]) + (sc ^ k_swizzle<D>(r)) * 8) * 2);
    } else {
      const int cix = ci - C::NK * C::KCH;
      const int pos = cix * 64 + lane;
      const int r = pos / (DV / 8), sc = pos % (DV / 8);
      dma_off[i] = (uint32_t)((r * vst + (sc ^ v_swizzle<DV>(r)) * 8) * 2);
    }
  }
  auto issue_tile = [&](int kt, int stage) {
    const int j0 = kt * kBN;
    const uint32_t sbase = smem_lds + stage * C::STAGE;
    const bool tail = j0 + kBN > T;  // uniform: rows past the end need clamping
#pragma unroll
    for (int i = 0; i < C::CPW; ++i) {
      const int ci = wave + NW * i;
      const bool isk = ci < C::NK * C::KCH;
      const int n = isk ? ci / C::KCH : 0;
      const int cix = isk ? ci % C::KCH : ci - C::NK * C::KCH;
      const uint16_t* tp = isk ? (n ? kp[1] : kp[0]) : vp;
      const int64_t tst = isk ? (n ? kst[1] : kst[0]) : vst;
      const uint32_t dst = sbase + (isk ? n * C::K_BYTES : C::NK * C::K_BYTES) + cix * 1024;
      if (!tail) {
        dma16_sbase(tp + (int64_t)j0 * tst, dma_off[i], dst);
      } else {
        const int cols = isk ? D / 8 : DV / 8;
        const int pos = cix * 64 + lane;
        const int r = pos / cols, sc = pos % cols;
        const int c = sc ^ (isk ? k_swizzle<D>(r) : v_swizzle<DV>(r));
        dma16(tp + (int64_t)min(j0 + r, T - 1) * tst + c * 8, dst);
      }
    }
  };

  // ---- Q fragments (B operand of S^T = K Q^T): row i0w+li, cols 16ks+8hg ----
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

  // Retire the Q loads here.  The compiler cannot see the tile DMA, but the
  // hardware counter counts it: a compiler-placed vmcnt wait for Q inside the
  // key loop would also wait for the next tile's copy.
#pragma unroll
  for (int m = 0; m < MPW; ++m)
#pragma unroll
    for (int ks = 0; ks < KS; ks += 2)
      asm volatile("s_waitcnt vmcnt(0)" : "+v"(qf[m][ks]), "+v"(qf[m][ks + 1]));

  // ---- per-lane LDS offsets ----
  // K chunk (2ks + hg) of tile row r = 32 sb + li sits at chunk (2ks + hg) ^ k_swizzle(li).
  int koff[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) koff[ks] = li * (D * 2) + (((2 * ks + hg) ^ k_swizzle<D>(li)) << 4);
  // V^T operand via transpose reads: lane (G16 = lane>>4, l16 = lane&15) points at
  // row 4*(G16>>1) + (l16>>2) (+ sub-block, k-step), columns 32cb + 16(G16&1) + 4(l16&3),
  // i.e. chunk 4cb + cl.  The swizzle only permutes chunks within aligned groups of
  // 4*NV, so the per-lane offset depends on cb only through cb % NV.
  constexpr int NV = DV >= 128 ? 4 : 2;
  int voff[NV];
  {
    const int l16 = lane & 15, g16 = lane >> 4;
    const int vr = 4 * (g16 >> 1) + (l16 >> 2);
    const int cl = 2 * (g16 & 1) + ((l16 & 3) >> 1);
    const int x = v_swizzle<DV>(vr);  // rows of one read share r & 3 = l16 >> 2
#pragma unroll
    for (int v = 0; v < NV; ++v) voff[v] = vr * (DV * 2) + (((4 * v + cl) ^ x) - 4 * v) * 16 + (l16 & 1) * 8;
  }

  // ---- V1 lambda (one fp32 scalar per call) ----
  float lam = 0.f;
  if constexpr (!V2) {
    float pa = 0.f, pb = 0.f;
    for (int c = lane; c < D; c += 64) {
      pa += a.lq1[c] * a.lk1[c];
      pb += a.lq2[c] * a.lk2[c];
    }
    pa = wave_sum(pa);
    pb = wave_sum(pb);
    lam = expf(pa) - expf(pb) + a.lam_init;
  }

  const float sl2 = a.sl2;
  float mref[MPW], lsum[MPW];
  f32x16 o[MPW][CB];
#pragma unroll
  for (int m = 0; m < MPW; ++m) {
    mref[m] = -INFINITY;
    lsum[m] = 0.f;
#pragma unroll
    for (int cb = 0; cb < CB; ++cb)
#pragma unroll
      for (int r = 0; r < 16; ++r) o[m][cb][r] = 0.f;
  }
  // K tensor of each map inside a stage
  int kbyte[MPW];
#pragma unroll
  for (int m = 0; m < MPW; ++m) kbyte[m] = V2 ? 0 : (m0 + m) * C::K_BYTES;

  // ---- the arithmetic of one 32-key sub-block, shared by both loop forms ----
  // scores S^T[j][i] (32 keys x 32 rows per map) from K rows row0.. of a stage
  auto qk = [&](const unsigned char* st, int row0) {
    Scores<MPW> r;
#pragma unroll
    for (int m = 0; m < MPW; ++m)
#pragma unroll
      for (int i = 0; i < 16; ++i) r.s[m][i] = 0.f;
    const unsigned char* kr = st + row0 * (D * 2);
    if (DA_SETPRIO) __builtin_amdgcn_s_setprio(2);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      if constexpr (V2) {  // one K fragment feeds every map of the wave
        const bf16x8 ka = *(const bf16x8*)(kr + koff[ks]);
#pragma unroll
        for (int m = 0; m < MPW; ++m) r.s[m] = mfma32x32x16(ka, qf[m][ks], r.s[m]);
      } else {
#pragma unroll
        for (int m = 0; m < MPW; ++m)
          r.s[m] = mfma32x32x16(*(const bf16x8*)(kr + kbyte[m] + koff[ks]), qf[m][ks], r.s[m]);
      }
    }
    if (DA_SETPRIO) __builtin_amdgcn_s_setprio(0);
    return r;
  };
  // causal mask (diagonal sub-block only), row maxima, and whether any row's max
  // outgrew its reference by more than 2^8
  float mb[MPW];
  bool need[MPW];
  auto softmax_head = [&](Scores<MPW>& S, bool diag) {
    bool any = false;
#pragma unroll
    for (int m = 0; m < MPW; ++m) {
      if (diag) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = 8 * (r >> 2) + 4 * hg + (r & 3);
          if (key > li) S.s[m][r] = -INFINITY;
        }
      }
      float mx = S.s[m][0];
#pragma unroll
      for (int r = 1; r < 16; ++r) mx = fmaxf(mx, S.s[m][r]);
      mx = max_across_halves(mx);
      mb[m] = mx * sl2;
      need[m] = mb[m] > mref[m] + kLazyLog2;
      any |= need[m];
    }
    return any;
  };
  auto rescale = [&]() {
#pragma unroll
    for (int m = 0; m < MPW; ++m) {
      const float al = need[m] ? exp2f(mref[m] - mb[m]) : 1.f;
      if (need[m]) mref[m] = mb[m];
      lsum[m] *= al;
#pragma unroll
      for (int cb = 0; cb < CB; ++cb)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[m][cb][r] *= al;
    }
  };
  // probabilities -> bf16 B operand of O^T = V^T P^T
  auto softmax_exp = [&](const Scores<MPW>& S) {
    Probs<MPW> P;
#pragma unroll
    for (int m = 0; m < MPW; ++m) {
      f32x8 p0, p1;
      float acc = 0.f;
#pragma unroll
      for (int r = 0; r < 8; ++r) {
        p0[r] = __builtin_amdgcn_exp2f(fmaf(S.s[m][r], sl2, -mref[m]));
        p1[r] = __builtin_amdgcn_exp2f(fmaf(S.s[m][r + 8], sl2, -mref[m]));
        acc += p0[r] + p1[r];
      }
      lsum[m] += acc;
      P.p[m][0] = cvt_bf16x8(p0);
      P.p[m][1] = cvt_bf16x8(p1);
    }
    return P;
  };
  // O^T[c][i] += V^T[c][j] P^T[j][i] over V rows row0..row0+31 of a stage
  auto pv = [&](const unsigned char* st, int row0, const Probs<MPW>& P) {
    const unsigned char* vt = st + C::NK * C::K_BYTES;
    if (DA_SETPRIO) __builtin_amdgcn_s_setprio(2);
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
#pragma unroll
      for (int cb = 0; cb < CB; ++cb) {
        const unsigned char* q = vt + (row0 + 16 * kk) * (DV * 2) + cb * 64 + voff[cb % NV];
        const bf16x8 va = join_bf16x8(tr_read(q), tr_read(q + 8 * (DV * 2)));
#pragma unroll
        for (int m = 0; m < MPW; ++m) o[m][cb] = mfma32x32x16(va, P.p[m][kk], o[m][cb]);
      }
    }
    if (DA_SETPRIO) __builtin_amdgcn_s_setprio(0);
  };

  if constexpr (!PIPE) {
    // ---- 64-key tiles, double-buffered; sub-blocks processed in order ----
    issue_tile(0, 0);
    for (int kt = 0; kt < nkt; ++kt) {
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // this wave's part of tile kt landed
      __syncthreads();                                  // all parts landed; other stage free
      if (kt + 1 < nkt) issue_tile(kt + 1, (kt + 1) & 1);
      if (!active) continue;
      const unsigned char* st = smem + (kt & 1) * C::STAGE;
      constexpr int NSB = kBN / 32;
      constexpr int GS = C::SMG;  // sub-blocks sharing one max / rescale decision
#pragma unroll
      for (int g0 = 0; g0 < NSB; g0 += GS) {
        if (kt * kBN + 32 * g0 > i0w) break;  // group entirely above this wave's diagonal
        if (GS > 1 && kt * kBN + 32 * (g0 + GS - 1) <= i0w) {
          // The whole group is visible: its score MFMAs back to back, one max /
          // rescale decision, then the exponentials of sub-block s+1 alongside
          // the P.V MFMAs of sub-block s.
          Scores<MPW> S[GS];
#pragma unroll
          for (int j = 0; j < GS; ++j) S[j] = qk(st, 32 * (g0 + j));
          const bool diag_last = kt * kBN + 32 * (g0 + GS - 1) == i0w;
          bool any = false;
#pragma unroll
          for (int m = 0; m < MPW; ++m) {
            if (diag_last) {
#pragma unroll
              for (int r = 0; r < 16; ++r) {
                const int key = 8 * (r >> 2) + 4 * hg + (r & 3);
                if (key > li) S[GS - 1].s[m][r] = -INFINITY;
              }
            }
            float mx = S[0].s[m][0];
#pragma unroll
            for (int j = 0; j < GS; ++j)
#pragma unroll
              for (int r = 0; r < 16; ++r) mx = fmaxf(mx, S[j].s[m][r]);
            mx = max_across_halves(mx);
            mb[m] = mx * sl2;
            need[m] = mb[m] > mref[m] + kLazyLog2;
            any |= need[m];
          }
          if (__builtin_amdgcn_ballot_w64(any)) rescale();
          Probs<MPW> P = softmax_exp(S[0]);
#pragma unroll
          for (int j = 0; j < GS; ++j) {
            Probs<MPW> Pn;
            if (j + 1 < GS) Pn = softmax_exp(S[j + 1]);
            pv(st, 32 * (g0 + j), P);
            if (j + 1 < GS) P = Pn;
          }
        } else {
#pragma unroll
          for (int j = 0; j < GS; ++j) {
            const int jb = kt * kBN + 32 * (g0 + j);
            if (jb > i0w) break;  // sub-block entirely above this wave's diagonal
            Scores<MPW> S = qk(st, 32 * (g0 + j));
            if (__builtin_amdgcn_ballot_w64(softmax_head(S, jb == i0w))) rescale();
            pv(st, 32 * (g0 + j), softmax_exp(S));
          }
        }
      }
    }
  } else {
    // ---- 32-key tiles in a 4-stage ring, software-pipelined ----
    // Step n (tile n) issues the MFMAs of P.V for tile n-1 and of the scores
    // for tile n+1 in the same basic block as the exponentials of tile n, so
    // matrix and vector work overlap inside the wave.  Tile n+1 is waited for
    // (and made visible by a barrier) at step n; the copy of tile n+2 then
    // goes to stage (n+2)%4, whose last reader was step n-1.  A rescale (rare)
    // first flushes the pending P.V of tile n-1.
    const int dw = active ? i0w / 32 : -1;  // last tile this wave needs
    auto stage = [&](int n) { return smem + (n & 3) * C::STAGE; };
    issue_tile(0, 0);
    if (nkt > 1) issue_tile(1, 1);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    Scores<MPW> S;
    Probs<MPW> P;
    if (dw >= 0) S = qk(stage(0), 0);
    bool pending = false;  // P holds tile n-1's probabilities, its P.V not issued yet
    for (int n = 0; n < nkt; ++n) {
      const bool mine = n <= dw;
      if (mine && __builtin_amdgcn_ballot_w64(softmax_head(S, n == dw))) {
        if (pending) {
          pv(stage(n - 1), 0, P);
          pending = false;
        }
        rescale();
      }
      if (n + 1 < nkt) {
        if (n >= 1) {
          asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // tile n+1 landed (this wave's part)
          __syncthreads();
        }
        if (n + 2 < nkt) issue_tile(n + 2, (n + 2) & 3);
      }
      if (!mine) continue;
      if (n < dw) {
        if (pending) {  // steady state
          const Scores<MPW> Sn = qk(stage(n + 1), 0);
          const Probs<MPW> Pn = softmax_exp(S);
          pv(stage(n - 1), 0, P);
          S = Sn;
          P = Pn;
        } else {
          const Scores<MPW> Sn = qk(stage(n + 1), 0);
          P = softmax_exp(S);
          S = Sn;
        }
        pending = true;
      } else {  // n == dw: this wave's last tile
        if (pending) pv(stage(n - 1), 0, P);
        pv(stage(n), 0, softmax_exp(S));
        pending = false;
      }
    }
  }

  // ---- epilogue ----------------------------------------------------------------
  const int row = i0w + li;
  float inv[MPW];
#pragma unroll
  for (int m = 0; m < MPW; ++m) inv[m] = 1.f / (lsum[m] + __shfl_xor(lsum[m], 32, 64));

  uint16_t* dst;
  float post = 1.f;
  if constexpr (MPW == 1) {
    // map 2's wave hands lam * O2 / l2 to map 1's wave through LDS
    __syncthreads();  // every wave is done with the K/V stages
    float* xch = (float*)smem + (wave >> 1) * (CB * 16 * 64);  // one slot per partner pair
    if (m0 == 1) {
      if (active) {
        float w = lam * inv[0];
        if constexpr (V2) {
          float lg = 0.f;
          if (row < T) lg = ((const float*)a.lam.p)[b * a.lam.sb + (int64_t)row * a.lam.st + pair * a.lam.sh];
          w = sigmoid_f32(lg) * inv[0];
        }
#pragma unroll
        for (int cb = 0; cb < CB; ++cb)
#pragma unroll
          for (int r = 0; r < 16; ++r) xch[(cb * 16 + r) * 64 + lane] = o[0][cb][r] * w;
      }
      __syncthreads();
      return;
    }
    __syncthreads();
    if (!active) return;
    float ss = 0.f;
#pragma unroll
    for (int cb = 0; cb < CB; ++cb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float dv = o[0][cb][r] * inv[0] - xch[(cb * 16 + r) * 64 + lane];
        o[0][cb][r] = dv;
        ss += dv * dv;
      }
    if constexpr (!V2) {
      ss += __shfl_xor(ss, 32, 64);
      post = (1.f - a.lam_init) / sqrtf(ss * (1.f / DV) + 1e-5f);
      dst = (uint16_t*)a.out.p + b * a.out.sb + (int64_t)row * a.out.st + h * a.out.sh;
    } else {
      dst = (uint16_t*)a.out.p + b * a.out.sb + (int64_t)row * a.out.st + pair * a.out.sh;
    }
  } else {
    if (!active) return;
    if constexpr (!V2) {
      const float w1 = lam * inv[1];
      float ss = 0.f;
#pragma unroll
      for (int cb = 0; cb < CB; ++cb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float dv = o[0][cb][r] * inv[0] - w1 * o[1][cb][r];
          o[0][cb][r] = dv;
          ss += dv * dv;
        }
      ss += __shfl_xor(ss, 32, 64);
      post = (1.f - a.lam_init) / sqrtf(ss * (1.f / DV) + 1e-5f);
      dst = (uint16_t*)a.out.p + b * a.out.sb + (int64_t)row * a.out.st + h * a.out.sh;
    } else {
      float lg = 0.f;
      if (row < T) lg = ((const float*)a.lam.p)[b * a.lam.sb + (int64_t)row * a.lam.st + pair * a.lam.sh];
      const float w1 = sigmoid_f32(lg) * inv[1];
#pragma unroll
      for (int cb = 0; cb < CB; ++cb)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[0][cb][r] = o[0][cb][r] * inv[0] - w1 * o[1][cb][r];
      dst = (uint16_t*)a.out.p + b * a.out.sb + (int64_t)row * a.out.st + pair * a.out.sh;
    }
  }
  if (row < T) {
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
}

template <int D, int DV, bool V2, int NW, int MPW, bool PIPE>
hipError_t launch(const PrefillArgs& a, hipStream_t s) {
  const void* args[] = {&a};
  return hipLaunchKernel((const void*)prefill_kernel<D, DV, V2, NW, MPW, PIPE>, dim3(a.nwg), dim3(NW * 64),
                         (void**)args, 0, s);
}

}  // namespace

// Per-shape kernel variant: maps per wave (MPW) and waves per workgroup (NW).
#ifndef DA_V1_D64_MPW
#define DA_V1_D64_MPW 1
#endif
#ifndef DA_V1_D64_NW
#define DA_V1_D64_NW 4
#endif
#ifndef DA_V1_D128_MPW
#define DA_V1_D128_MPW 1
#endif
#ifndef DA_V2_MPW
#define DA_V2_MPW 1
#endif
#ifndef DA_V2_NW
#define DA_V2_NW 8
#endif
#ifndef DA_V1_D64_PIPE
#define DA_V1_D64_PIPE false
#endif
#ifndef DA_V2_PIPE
#define DA_V2_PIPE false
#endif

hipError_t launch_prefill_v1_bf16(int d, const PrefillArgs& a0, hipStream_t s) {
  PrefillArgs a = a0;
  a.units_per_b = a.H;
  auto geom = [&](int nw, int mpw) {
    const int BMT = 32 * (mpw == 2 ? nw : nw / 2);  // rows per workgroup
    a.tiles = (a.T + BMT - 1) / BMT;
    a.nwg = a.B * a.H * a.tiles;
  };
  if (d == 64) {
    geom(DA_V1_D64_NW, DA_V1_D64_MPW);
    return launch<64, 128, false, DA_V1_D64_NW, DA_V1_D64_MPW, DA_V1_D64_PIPE>(a, s);
  }
  if (d == 128) {
    geom(4 * (3 - DA_V1_D128_MPW), DA_V1_D128_MPW);
    return launch<128, 256, false, 4 * (3 - DA_V1_D128_MPW), DA_V1_D128_MPW, false>(a, s);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_prefill_v2_bf16(int d, const PrefillArgs& a0, hipStream_t s) {
  PrefillArgs a = a0;
  const int np = a.G / 2;
  const int units = DA_V2_MPW == 2 ? DA_V2_NW : DA_V2_NW / 2;  // (pair, row block) slots per workgroup
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
