// prefill_bf16.hip -- fused causal differential-attention prefill, bf16 MFMA.
//
// What one wave computes ("Differential Transformer V2" article, DiffAttnV1
// and DiffAttnV2 pseudo-code):
//   V1: for 32 query rows of one differential head, the two causal softmax
//       maps softmax(Q1 K1^T / sqrt d) and softmax(Q2 K2^T / sqrt d) applied to
//       the one shared V (width 2d), then A1 V - lam A2 V, RMSNorm over the 2d
//       channels (eps 1e-5, no weight) and the (1 - lambda_init) scale
//       (nanoGPT issue "How best to implement a differential transformer?",
//       Wilsontomass's module).
//   V2: for 32 tokens of one adjacent head pair (2p, 2p+1) of a GQA group,
//       the two maps over the group's shared K and V, then
//       O_2p - sigmoid(lam[t, p]) O_2p+1 (no norm, no scale).
//
// Structure (designed for gfx950, not taken from any listing):
//   * A workgroup of 4 waves streams 64-key tiles of K (two K tensors for
//     V1, one for V2) and V through LDS, double-buffered, so each tile is read
//     from HBM/L2 once per workgroup.  For V2 the 4 waves are the 4 pairs of
//     one 8-head GQA group, so a K/V tile is loaded once for the whole group.
//   * Scores are computed transposed, S^T = K Q^T, with
//     v_mfma_f32_32x32x16_bf16: the Q fragments stay in registers for the
//     whole key loop and each lane then holds 16 scores of ONE query row, so
//     the softmax row state (running max and sum) is per lane, and the fp32
//     score registers convert in place to the bf16 B operand of the P.V
//     product O^T = V^T P^T.  V is transposed once on its way into LDS.
//   * Online softmax in the log2 domain with a lazily updated reference max:
//     the running reference only moves (and O, l are rescaled) when a row's
//     max exceeds it by more than 2^8, which keeps every exponent <= 2^8 and
//     leaves the result exact up to rounding.
//   * Causal work skipping at 32-key granularity; the mask is only evaluated
//     on diagonal sub-blocks.  Workgroups run heaviest tiles first and map
//     onto XCDs so the tiles of one head share an L2.
#include <math.h>

#include "kernels.hpp"

namespace da {
namespace {

constexpr int kBN = 64;          // keys per LDS stage
constexpr int kKPad = 8;         // bf16 padding per K row  -> conflict-free 16 B reads
constexpr int kVPad = 4;         // bf16 padding per V^T row -> conflict-free 8 B reads/writes
constexpr float kLazyLog2 = 8.f; // rescale only when the max grows by > 2^8

template <int D, int DV, bool V2>
struct Layout {
  static constexpr int KROW = D + kKPad;
  static constexpr int VROW = kBN + kVPad;
  static constexpr int NK = V2 ? 1 : 2;
  static constexpr int KSZ = kBN * KROW;
  static constexpr int VSZ = DV * VROW;
  static constexpr int STAGE = NK * KSZ + VSZ;  // bf16 elements per stage
};

// Cooperative staging of one key tile: global -> registers -> LDS.
template <int D, int DV, bool V2, int NT>
struct Stage {
  using L = Layout<D, DV, V2>;
  static constexpr int KTOT = kBN * (D / 8);         // 16 B chunks per K tensor
  static constexpr int VTOT = (kBN / 4) * (DV / 8);  // 4-row x 8-col units of V
  static constexpr int KCH = (KTOT + NT - 1) / NT;
  static constexpr int VU = (VTOT + NT - 1) / NT;
  uint4 k[L::NK][KCH];
  uint4 v[VU][4];

  __device__ __forceinline__ void load(const uint16_t* const kp[2], const int64_t kst[2], const uint16_t* vp,
                                       int64_t vst, int j0, int T, int tid) {
#pragma unroll
    for (int n = 0; n < L::NK; ++n) {
#pragma unroll
      for (int u = 0; u < KCH; ++u) {
        const int c = tid + NT * u;
        const int row = c / (D / 8), col = (c % (D / 8)) * 8;
        const int key = j0 + row;
        k[n][u] = (KTOT % NT == 0 || c < KTOT) && key < T
                      ? *(const uint4*)(kp[n] + (int64_t)key * kst[n] + col)
                      : make_uint4(0, 0, 0, 0);
      }
    }
#pragma unroll
    for (int u = 0; u < VU; ++u) {
      const int c = tid + NT * u;
      const int rg = c % (kBN / 4), cc = c / (kBN / 4);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int key = j0 + 4 * rg + q;
        v[u][q] = (VTOT % NT == 0 || c < VTOT) && key < T ? *(const uint4*)(vp + (int64_t)key * vst + cc * 8)
                                                          : make_uint4(0, 0, 0, 0);
      }
    }
  }

  __device__ __forceinline__ void store(uint16_t* st, int tid) const {
#pragma unroll
    for (int n = 0; n < L::NK; ++n) {
#pragma unroll
      for (int u = 0; u < KCH; ++u) {
        const int c = tid + NT * u;
        const int row = c / (D / 8), col = (c % (D / 8)) * 8;
        if (KTOT % NT == 0 || c < KTOT) *(uint4*)(st + n * L::KSZ + row * L::KROW + col) = k[n][u];
      }
    }
    uint16_t* vt = st + L::NK * L::KSZ;
#pragma unroll
    for (int u = 0; u < VU; ++u) {
      const int c = tid + NT * u;
      const int rg = c % (kBN / 4), cc = c / (kBN / 4);
      if (VTOT % NT == 0 || c < VTOT) {
#pragma unroll
        for (int e = 0; e < 8; ++e)
          *(uint2*)(vt + (cc * 8 + e) * L::VROW + 4 * rg) = column4(v[u][0], v[u][1], v[u][2], v[u][3], e);
      }
    }
  }
};

template <int D, int DV, bool V2, int NW>
__global__ void __launch_bounds__(NW * 64, 1) prefill_kernel(const PrefillArgs a) {
  using L = Layout<D, DV, V2>;
  constexpr int NT = NW * 64;
  constexpr int KS = D / 16;   // k-steps of the score MFMA
  constexpr int CB = DV / 32;  // 32-wide column blocks of O^T
  __shared__ __attribute__((aligned(16))) uint16_t smem[2 * L::STAGE];

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int li = lane & 31, hg = lane >> 5;

  const int logical = xcd_logical_id(blockIdx.x, a.nwg);
  const int unit = logical / a.tiles;
  const int tile = a.tiles - 1 - logical % a.tiles;  // heaviest tiles first
  const int b = unit / a.units_per_b;
  const int u = unit % a.units_per_b;

  // --- this wave's two maps and its 32 rows --------------------------------
  int RB, rb, h = 0, pair = 0;
  const uint16_t *qA, *qB, *kp[2], *vp;
  int64_t qstA, qstB, kst[2], vst;
  if constexpr (!V2) {
    RB = NW;
    rb = wave;
    h = u;
    qA = (const uint16_t*)a.q1.p + b * a.q1.sb + h * a.q1.sh;
    qB = (const uint16_t*)a.q2.p + b * a.q2.sb + h * a.q2.sh;
    qstA = a.q1.st;
    qstB = a.q2.st;
    kp[0] = (const uint16_t*)a.k1.p + b * a.k1.sb + h * a.k1.sh;
    kp[1] = (const uint16_t*)a.k2.p + b * a.k2.sb + h * a.k2.sh;
    kst[0] = a.k1.st;
    kst[1] = a.k2.st;
    vp = (const uint16_t*)a.v.p + b * a.v.sb + h * a.v.sh;
    vst = a.v.st;
  } else {
    const int npc = (a.G / 2) / a.pc;  // pair chunks per group
    const int g = u / npc, pcix = u % npc;
    RB = NW / a.pc;
    rb = wave / a.pc;
    pair = g * (a.G / 2) + pcix * a.pc + wave % a.pc;
    qA = (const uint16_t*)a.q1.p + b * a.q1.sb + (2 * pair) * a.q1.sh;
    qB = (const uint16_t*)a.q1.p + b * a.q1.sb + (2 * pair + 1) * a.q1.sh;
    qstA = qstB = a.q1.st;
    kp[0] = kp[1] = (const uint16_t*)a.k1.p + b * a.k1.sb + g * a.k1.sh;
    kst[0] = kst[1] = a.k1.st;
    vp = (const uint16_t*)a.v.p + b * a.v.sb + g * a.v.sh;
    vst = a.v.st;
  }
  const int T = a.T;
  const int BMT = 32 * RB;
  const int I0 = tile * BMT;
  const int i0w = I0 + 32 * rb;
  const bool active = i0w < T;
  const int kend = min(T, I0 + BMT);
  const int nkt = (kend + kBN - 1) / kBN;

  // --- Q fragments (B operand of S^T = K Q^T): row i0w+li, cols 16ks+8hg.. --
  bf16x8 qf[2][KS];
  {
    const int row = i0w + li;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const uint4 z = make_uint4(0, 0, 0, 0);
      qf[0][ks] = as_bf16x8(row < T ? *(const uint4*)(qA + (int64_t)row * qstA + 16 * ks + 8 * hg) : z);
      qf[1][ks] = as_bf16x8(row < T ? *(const uint4*)(qB + (int64_t)row * qstB + 16 * ks + 8 * hg) : z);
    }
  }

  // --- V1 lambda: one scalar per call, fp32 ---------------------------------
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
  float mref[2] = {-INFINITY, -INFINITY};
  float lsum[2] = {0.f, 0.f};
  f32x16 o[2][CB];
#pragma unroll
  for (int m = 0; m < 2; ++m)
#pragma unroll
    for (int cb = 0; cb < CB; ++cb)
#pragma unroll
      for (int r = 0; r < 16; ++r) o[m][cb][r] = 0.f;

  Stage<D, DV, V2, NT> stg;
  stg.load(kp, kst, vp, vst, 0, T, tid);
  stg.store(smem, tid);
  __syncthreads();

  for (int kt = 0; kt < nkt; ++kt) {
    const uint16_t* cur = smem + (kt & 1) * L::STAGE;
    const bool has_next = kt + 1 < nkt;
    if (has_next) stg.load(kp, kst, vp, vst, (kt + 1) * kBN, T, tid);

    if (active) {
#pragma unroll
      for (int sb = 0; sb < kBN / 32; ++sb) {
        const int jb = kt * kBN + 32 * sb;
        if (jb > i0w) break;  // sub-block entirely above this wave's diagonal
        const bool diag = jb == i0w;
        const int kb0 = 32 * sb;

        // ---- scores, both maps: S^T[j][i] for 32 keys x 32 rows ----
        f32x16 s[2];
#pragma unroll
        for (int m = 0; m < 2; ++m)
#pragma unroll
          for (int r = 0; r < 16; ++r) s[m][r] = 0.f;
        const uint16_t* krow0 = cur + (kb0 + li) * L::KROW + 8 * hg;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          const bf16x8 ka = *(const bf16x8*)(krow0 + 16 * ks);
          s[0] = mfma32x32x16(ka, qf[0][ks], s[0]);
          if constexpr (V2) {
            s[1] = mfma32x32x16(ka, qf[1][ks], s[1]);
          } else {
            const bf16x8 kb = *(const bf16x8*)(krow0 + L::KSZ + 16 * ks);
            s[1] = mfma32x32x16(kb, qf[1][ks], s[1]);
          }
        }

        // ---- causal mask (diagonal sub-block only) and row maxima ----
        float mb[2];
#pragma unroll
        for (int m = 0; m < 2; ++m) {
          if (diag) {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              const int key = 8 * (r >> 2) + 4 * hg + (r & 3);
              if (key > li) s[m][r] = -INFINITY;
            }
          }
          float mx = s[m][0];
#pragma unroll
          for (int r = 1; r < 16; ++r) mx = fmaxf(mx, s[m][r]);
          mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
          mb[m] = mx * sl2;
        }

        // ---- lazy rescale: only when some row's max outgrew its reference ----
        const bool need0 = mb[0] > mref[0] + kLazyLog2;
        const bool need1 = mb[1] > mref[1] + kLazyLog2;
        if (__builtin_amdgcn_ballot_w64(need0 || need1)) {
          const float al0 = need0 ? exp2f(mref[0] - mb[0]) : 1.f;
          const float al1 = need1 ? exp2f(mref[1] - mb[1]) : 1.f;
          if (need0) mref[0] = mb[0];
          if (need1) mref[1] = mb[1];
          lsum[0] *= al0;
          lsum[1] *= al1;
#pragma unroll
          for (int cb = 0; cb < CB; ++cb)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              o[0][cb][r] *= al0;
              o[1][cb][r] *= al1;
            }
        }

        // ---- probabilities -> bf16 B operand of O^T = V^T P^T ----
        bf16x8 pk[2][2];
#pragma unroll
        for (int m = 0; m < 2; ++m) {
          f32x8 p0, p1;
          float acc = 0.f;
#pragma unroll
          for (int r = 0; r < 8; ++r) {
            p0[r] = __builtin_amdgcn_exp2f(fmaf(s[m][r], sl2, -mref[m]));
            p1[r] = __builtin_amdgcn_exp2f(fmaf(s[m][r + 8], sl2, -mref[m]));
            acc += p0[r] + p1[r];
          }
          lsum[m] += acc;
          pk[m][0] = cvt_bf16x8(p0);
          pk[m][1] = cvt_bf16x8(p1);
        }

        // ---- O^T[c][i] += V^T[c][j] P^T[j][i]; V^T fragment shared by both maps ----
        const uint16_t* vt = cur + L::NK * L::KSZ + li * L::VROW + kb0 + 4 * hg;
#pragma unroll
        for (int cb = 0; cb < CB; ++cb) {
#pragma unroll
          for (int kk = 0; kk < 2; ++kk) {
            const uint16_t* vr = vt + 32 * cb * L::VROW + 16 * kk;
            const bf16x8 va = join_bf16x8(*(const uint2*)vr, *(const uint2*)(vr + 8));
            o[0][cb] = mfma32x32x16(va, pk[0][kk], o[0][cb]);
            o[1][cb] = mfma32x32x16(va, pk[1][kk], o[1][cb]);
          }
        }
      }
    }

    if (has_next) stg.store(smem + ((kt + 1) & 1) * L::STAGE, tid);
    __syncthreads();
  }

  if (!active) return;

  // --- epilogue: normalise each map, combine, (V1) RMSNorm and scale ---------
  const float l0 = lsum[0] + __shfl_xor(lsum[0], 32, 64);
  const float l1 = lsum[1] + __shfl_xor(lsum[1], 32, 64);
  const float inv0 = 1.f / l0, inv1 = 1.f / l1;
  const int row = i0w + li;

  float w1;  // weight of map 2 in the combine
  float post = 1.f;
  uint16_t* dst;
  if constexpr (!V2) {
    w1 = lam * inv1;
    float ss = 0.f;
#pragma unroll
    for (int cb = 0; cb < CB; ++cb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float dv = o[0][cb][r] * inv0 - w1 * o[1][cb][r];
        o[0][cb][r] = dv;
        ss += dv * dv;
      }
    ss += __shfl_xor(ss, 32, 64);
    post = (1.f - a.lam_init) / sqrtf(ss * (1.f / DV) + 1e-5f);
    dst = (uint16_t*)a.out.p + b * a.out.sb + (int64_t)row * a.out.st + h * a.out.sh;
  } else {
    float lg = 0.f;
    if (row < T) lg = ((const float*)a.lam.p)[b * a.lam.sb + (int64_t)row * a.lam.st + pair * a.lam.sh];
    w1 = sigmoid_f32(lg) * inv1;
#pragma unroll
    for (int cb = 0; cb < CB; ++cb)
#pragma unroll
      for (int r = 0; r < 16; ++r) o[0][cb][r] = o[0][cb][r] * inv0 - w1 * o[1][cb][r];
    dst = (uint16_t*)a.out.p + b * a.out.sb + (int64_t)row * a.out.st + pair * a.out.sh;
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

template <int D, int DV, bool V2>
hipError_t launch(const PrefillArgs& a, hipStream_t s) {
  const void* args[] = {&a};
  return hipLaunchKernel((const void*)prefill_kernel<D, DV, V2, 4>, dim3(a.nwg), dim3(256), (void**)args, 0, s);
}

}  // namespace

hipError_t launch_prefill_v1_bf16(int d, const PrefillArgs& a0, hipStream_t s) {
  PrefillArgs a = a0;
  const int BMT = 32 * 4;
  a.tiles = (a.T + BMT - 1) / BMT;
  a.units_per_b = a.H;
  a.nwg = a.B * a.H * a.tiles;
  if (d == 64) return launch<64, 128, false>(a, s);
  if (d == 128) return launch<128, 256, false>(a, s);
  return hipErrorInvalidValue;
}

hipError_t launch_prefill_v2_bf16(int d, const PrefillArgs& a0, hipStream_t s) {
  PrefillArgs a = a0;
  const int np = a.G / 2;
  a.pc = np % 4 == 0 ? 4 : np % 2 == 0 ? 2 : 1;
  const int BMT = 32 * (4 / a.pc);
  a.tiles = (a.T + BMT - 1) / BMT;
  a.units_per_b = a.H * (np / a.pc);
  a.nwg = a.B * a.units_per_b * a.tiles;
  if (d == 64) return launch<64, 64, true>(a, s);
  if (d == 128) return launch<128, 128, true>(a, s);
  return hipErrorInvalidValue;
}

}  // namespace da
