// decode_bf16.hip -- DIFF V2 decode: one new query token per sequence against
// a long KV cache ("Differential Transformer V2" article: DiffAttnV2 at the
// newest position; the remark that decoding is memory-bound and that the
// paired heads of one GQA group share key and value).
//
// The cache is the only large operand (B*L*Hkv*d*2 bf16), so the kernel is
// built to stream it from HBM exactly once:
//   * split kernel: a workgroup owns (batch b, kv head g, one chunk of the
//     cache).  Its 4 waves take interleaved 32-token blocks.  For each block
//     a wave loads K straight from global memory into MFMA A-operand
//     registers (16-byte loads, 64 contiguous bytes per row per instruction)
//     and scores all G query heads of the group at once with
//     v_mfma_f32_16x16x32_bf16 (tokens x heads), keeps a lazily rescaled
//     online softmax per head, transposes the V block through a per-wave LDS
//     slice and accumulates O^T = V^T P^T with the same MFMA.  The four
//     waves' (max, sum, O) states are then merged in LDS (log-sum-exp) and
//     one partial per (b, g, chunk, head) goes to the caller's workspace.
//   * merge kernel: per (b, pair), the partials of both heads are merged in
//     split order (fixed, no atomics: deterministic), normalised and combined
//     as a_2p - sigmoid(lam[b, p]) a_2p+1.
#include <math.h>

#include "kernels.hpp"

namespace da {
namespace {

constexpr int kWaves = 4;
constexpr int kBlk = 32;          // tokens per wave step
constexpr int kVtPad = 4;         // bf16 padding of a V^T row (conflict-free 8 B reads)
constexpr float kLazyLog2 = 8.f;  // rescale only when a head's max grows by > 2^8

__device__ __forceinline__ void lds_fence() {
  // The LDS executes one wave's instructions in order; this waits for the
  // wave's outstanding LDS accesses and is a compiler barrier for memory, so
  // writes by some lanes are visible to reads by other lanes of the wave.
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
}

template <int D>
__global__ void __launch_bounds__(kWaves * 64) decode_split_kernel(const DecodeArgs a) {
  constexpr int KS = D / 32;   // k-steps of the score MFMA
  constexpr int CB = D / 16;   // 16-wide column blocks of O^T
  constexpr int VROW = kBlk + kVtPad;
  constexpr int VT_ELEMS = D * VROW;               // one wave's V^T slice
  constexpr int VU = (kBlk / 4) * (D / 8) / 64;    // 4x8 V units per lane
  static_assert(VU >= 1 && (kBlk / 4) * (D / 8) % 64 == 0, "V block split");
  constexpr int LDS_VT = kWaves * VT_ELEMS * 2;            // bytes
  constexpr int LDS_RED = kWaves * 16 * (D + 2) * 4;       // bytes
  constexpr int LDS_BYTES = LDS_VT > LDS_RED ? LDS_VT : LDS_RED;
  __shared__ __attribute__((aligned(16))) unsigned char smem[LDS_BYTES];

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int c16 = lane & 15, kg = lane >> 4;

  const int bid = blockIdx.x;
  const int s = bid % a.nsplit;
  const int g = (bid / a.nsplit) % a.Hkv;
  const int b = bid / (a.nsplit * a.Hkv);
  const int G = a.G, L = a.L;

  // q fragments: B operand of S = K q^T.  Lane column = head (c16 < G).
  bf16x8 qf[KS];
  {
    const uint16_t* qrow = (const uint16_t*)a.q.p + b * a.q.sb + (int64_t)(g * G + c16) * a.q.sh;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      qf[ks] = as_bf16x8(c16 < G ? *(const uint4*)(qrow + 32 * ks + 8 * kg) : make_uint4(0, 0, 0, 0));
  }
  const uint16_t* kbase = (const uint16_t*)a.k.p + b * a.k.sb + g * a.k.sh;
  const uint16_t* vbase = (const uint16_t*)a.v.p + b * a.v.sb + g * a.v.sh;
  const int64_t kst = a.k.st, vst = a.v.st;

  uint16_t* vt = (uint16_t*)smem + wave * VT_ELEMS;
  const float sl2 = a.sl2;
  float mref = -INFINITY, lsum = 0.f;
  f32x4 o[CB];
#pragma unroll
  for (int cb = 0; cb < CB; ++cb) o[cb] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int t0 = s * a.chunk, t1 = min(L, t0 + a.chunk);
  for (int blk = t0 + kBlk * wave; blk < t1; blk += kBlk * kWaves) {
    // ---- issue the block's K (A operand) and V (transpose units) loads ----
    uint4 kr[2][KS];
#pragma unroll
    for (int sub = 0; sub < 2; ++sub) {
      const int tok = blk + 16 * sub + c16;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
        kr[sub][ks] = tok < L ? load_nt16(kbase + (int64_t)tok * kst + 32 * ks + 8 * kg)
                              : make_uint4(0, 0, 0, 0);
    }
    uint4 vr[VU][4];
#pragma unroll
    for (int u = 0; u < VU; ++u) {
      const int unit = lane + 64 * u;
      const int rg = unit % (kBlk / 4), cc = unit / (kBlk / 4);
#pragma unroll
      for (int qq = 0; qq < 4; ++qq) {
        const int tok = blk + 4 * rg + qq;
        vr[u][qq] = tok < L ? load_nt16(vbase + (int64_t)tok * vst + cc * 8)
                            : make_uint4(0, 0, 0, 0);
      }
    }

    // ---- scores: S[tok][head], two 16-token sub-blocks ----
    f32x4 sc[2];
#pragma unroll
    for (int sub = 0; sub < 2; ++sub) {
      sc[sub] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) sc[sub] = mfma16x16x32(as_bf16x8(kr[sub][ks]), qf[ks], sc[sub]);
    }
    // lane (head c16, kg) holds tokens blk + 16*sub + 4*kg + r
    float mx = -INFINITY;
#pragma unroll
    for (int sub = 0; sub < 2; ++sub)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        if (blk + 16 * sub + 4 * kg + r >= L) sc[sub][r] = -INFINITY;
        mx = fmaxf(mx, sc[sub][r]);
      }
    mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    const float mb = mx * sl2;  // finite: token blk < L is in every block
    const bool need = mb > mref + kLazyLog2;
    if (__builtin_amdgcn_ballot_w64(need)) {
      const float al = need ? exp2f(mref - mb) : 1.f;
      if (need) mref = mb;
      lsum *= al;
#pragma unroll
      for (int cb = 0; cb < CB; ++cb) o[cb] *= al;
    }
    f32x8 p;
    float ps = 0.f;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      p[r] = __builtin_amdgcn_exp2f(fmaf(sc[0][r], sl2, -mref));
      p[r + 4] = __builtin_amdgcn_exp2f(fmaf(sc[1][r], sl2, -mref));
      ps += p[r] + p[r + 4];
    }
    lsum += ps;
    const bf16x8 pk = cvt_bf16x8(p);  // slot t: token 4kg+t (t<4), 16+4kg+t-4 (t>=4)

    // ---- V block -> V^T in this wave's LDS slice ----
#pragma unroll
    for (int u = 0; u < VU; ++u) {
      const int unit = lane + 64 * u;
      const int rg = unit % (kBlk / 4), cc = unit / (kBlk / 4);
#pragma unroll
      for (int e = 0; e < 8; ++e)
        *(uint2*)(vt + (cc * 8 + e) * VROW + 4 * rg) = column4(vr[u][0], vr[u][1], vr[u][2], vr[u][3], e);
    }
    lds_fence();
    // ---- O^T[c][head] += V^T[c][tok] P^T[tok][head] ----
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) {
      const uint16_t* row = vt + (16 * cb + c16) * VROW + 4 * kg;
      const bf16x8 va = join_bf16x8(*(const uint2*)row, *(const uint2*)(row + 16));
      o[cb] = mfma16x16x32(va, pk, o[cb]);
    }
    lds_fence();
  }

  // ---- per-wave state -> LDS, then a log-sum-exp merge across the 4 waves ----
  lsum += __shfl_xor(lsum, 16, 64);
  lsum += __shfl_xor(lsum, 32, 64);
  __syncthreads();  // all waves are done with their V^T slices
  float* red = (float*)smem;  // [wave][head 16][D + 2]: m, l, O[D]
  {
    float* mine = red + (wave * 16 + c16) * (D + 2);
    if (kg == 0) {
      mine[0] = mref;
      mine[1] = lsum;
    }
#pragma unroll
    for (int cb = 0; cb < CB; ++cb)
#pragma unroll
      for (int r = 0; r < 4; ++r) mine[2 + 16 * cb + 4 * kg + r] = o[cb][r];
  }
  __syncthreads();
  float* out = a.ws + (((int64_t)b * a.Hkv + g) * a.nsplit + s) * (int64_t)G * (D + 2);
  for (int e = tid; e < G * (D + 2); e += kWaves * 64) {
    const int hh = e / (D + 2), c = e % (D + 2);
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) M = fmaxf(M, red[(w * 16 + hh) * (D + 2)]);
    float acc = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const float mw = red[(w * 16 + hh) * (D + 2)];
      const float f = mw == -INFINITY ? 0.f : exp2f(mw - M);
      acc += (c == 0 ? 0.f : red[(w * 16 + hh) * (D + 2) + c]) * f;
    }
    out[hh * (D + 2) + c] = c == 0 ? M : acc;
  }
}

template <int D>
__global__ void __launch_bounds__(D) decode_merge_kernel(const DecodeArgs a) {
  const int P = a.Hq / 2;
  const int b = blockIdx.x / P, p = blockIdx.x % P;
  const int c = threadIdx.x;
  const int G = a.G;
  float res[2];
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const int head = 2 * p + k;
    const int g = head / G, hh = head % G;
    const float* base = a.ws + ((int64_t)b * a.Hkv + g) * a.nsplit * (int64_t)G * (D + 2) + hh * (D + 2);
    const int64_t sstride = (int64_t)G * (D + 2);
    float M = -INFINITY;
    for (int s = 0; s < a.nsplit; ++s) M = fmaxf(M, base[s * sstride]);
    float l = 0.f, acc = 0.f;
    for (int s = 0; s < a.nsplit; ++s) {
      const float f = exp2f(base[s * sstride] - M);
      l += base[s * sstride + 1] * f;
      acc += base[s * sstride + 2 + c] * f;
    }
    // off-by-one softmax: one more logit 0, i.e. 2^(0 - M) against the merged max
    res[k] = acc / (l + (a.softmax1 ? exp2f(-M) : 0.f));
  }
  const float lg = ((const float*)a.lam.p)[b * a.lam.sb + p * a.lam.sh];
  const float val = res[0] - sigmoid_f32(lg) * res[1];
  uint16_t* dst = (uint16_t*)a.out.p + b * a.out.sb + p * a.out.sh;
  const uint32_t w = pack_bf16x2(val, 0.f);
  dst[c] = (uint16_t)(w & 0xffffu);
}

template <int D>
hipError_t launch(const DecodeArgs& a, hipStream_t st) {
  const void* args[] = {&a};
  hipError_t e = hipLaunchKernel((const void*)decode_split_kernel<D>, dim3(a.B * a.Hkv * a.nsplit),
                                 dim3(kWaves * 64), (void**)args, 0, st);
  if (e != hipSuccess) return e;
  return hipLaunchKernel((const void*)decode_merge_kernel<D>, dim3(a.B * (a.Hq / 2)), dim3(D), (void**)args, 0,
                         st);
}

}  // namespace

DecodeSplit decode_split(int B, int L, int Hkv) {
  // Aim for >= 2048 workgroups (8 per CU) and chunks of <= 2048 tokens; a
  // chunk is a multiple of the 4 waves x 32 tokens one step consumes.
  const int step = kWaves * kBlk;
  const long units = (long)B * Hkv;
  long ns = (L + 2047) / 2048;
  const long want = (2048 + units - 1) / units;
  if (ns < want) ns = want;
  const long maxns = (L + step - 1) / step;
  if (ns > maxns) ns = maxns;
  if (ns < 1) ns = 1;
  long chunk = (L + ns - 1) / ns;
  chunk = (chunk + step - 1) / step * step;
  DecodeSplit r;
  r.chunk = (int)chunk;
  r.nsplit = (int)((L + chunk - 1) / chunk);
  return r;
}

hipError_t launch_decode_bf16(int d, const DecodeArgs& a, hipStream_t s) {
  if (d == 64) return launch<64>(a, s);
  if (d == 128) return launch<128>(a, s);
  return hipErrorInvalidValue;
}

}  // namespace da
