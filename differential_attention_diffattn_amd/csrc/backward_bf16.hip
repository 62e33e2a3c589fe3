// backward_bf16.hip -- DIFF V2 backward (gradients of the prefill), bf16 MFMA.
//
// What is differentiated ("Differential Transformer V2" article, DiffAttnV2
// pseudo-code): attn_h = causal softmax(q_h k_g^T / sqrt d) v_g for every
// query head h of kv group g, out_p = attn_2p - sigmoid(lam_p) attn_2p+1.
// Chain rule, in the forward's order reversed:
//   d attn_2p = dout_p, d attn_2p+1 = -sigmoid(lam_p) dout_p,
//   d lam_p = -sigmoid(lam_p)(1 - sigmoid(lam_p)) <dout_p, attn_2p+1>,
//   per head: P = exp2(s log2(e)/sqrt(d) - lse) (rebuilt from the forward's
//   log-sum-exp), dP = d attn_h v^T, dS = P o (dP - D) with
//   D = rowsum(d attn_h o attn_h), dq = dS k / sqrt d, dk += dS^T q / sqrt d,
//   dv += P^T d attn_h.  (With the off-by-one softmax P carries the extra
//   term in lse, and the same steps hold.)  Since d attn of both heads of a
//   pair is a row multiple of dout, the pair's dP are row multiples of the
//   one G = dout v^T and D_h = c_h E_h with E_h = rowsum(dout o attn_h).
//
// Three kernels (designed for gfx950):
//   * bwd_pre: 16 lanes per (b, token, pair): E of both heads, d lam, and a
//     copy of lse padded to a multiple of 128 rows (so row blocks read whole
//     float4 groups), the odd head's as lse - log2(sigmoid(lam)) so that the
//     P rebuilt from it carries the factor -c.
//   * bwd_dq: the forward's structure with the key loop kept: a wave owns 32
//     query rows of one head, K/V tiles of 32 keys stream through LDS
//     (global_load_lds), S^T = K Q^T and G^T = V dout^T come from
//     v_mfma_f32_32x32x16_bf16 with Q / dout fragments held in registers,
//     and dQ^T += K^T dS^T takes K^T through ds_read_b64_tr_b16 (K is copied
//     to LDS once, in a layout that serves both reads); the odd head's dQ
//     takes the sign of -c at the store.
//   * bwd_dkdv: the mirror image: two waves own 32 keys of one kv head and
//     loop over the query rows at or after their keys and the group's head
//     pairs, forming S of each head, G and dV once per pair, and dK of each
//     head, from K / V fragments in registers and transpose reads of the Q
//     and dout tiles.  The gradients of a kv head are summed over its query
//     heads inside the workgroup, so nothing is reduced across workgroups
//     (no atomics: deterministic).
#include <math.h>

#include <type_traits>

#include "kernels.hpp"
#include "tile_ops.hpp"

namespace da {
namespace {

constexpr int kNW = 4;   // waves per workgroup of bwd_dq; bwd_dkdv has 2 kNW (two per key block)
constexpr int kBT = 32;  // rows / keys per streamed tile

// ---- pre-pass -----------------------------------------------------------------
// Sum over the 16 lanes of a row (lanes 16k .. 16k + 15).
__device__ __forceinline__ float row16_sum(float v) {
#pragma unroll
  for (int o = 8; o >= 1; o >>= 1) v += __shfl_xor(v, o, 16);
  return v;
}

// Sixteen lanes per (b, t, p), t < Tp: each lane holds d/16 consecutive
// channels (16-byte accesses at d = 128, 8-byte at d = 64), four pairs per
// wave, so a wave reads and writes contiguous spans.
template <int D>
__global__ void __launch_bounds__(256) bwd_pre_kernel(const BwdArgs a) {
  constexpr int EL = D / 16;  // channels per lane
  using Vec = typename std::conditional<EL == 8, uint4, uint2>::type;
  const int lane = threadIdx.x & 63, l16 = lane & 15;
  const int P = a.Hq / 2;
  const long long item = ((long long)blockIdx.x * 4 + (threadIdx.x >> 6)) * 4 + (lane >> 4);  // (b, t, p)
  if (item >= (long long)a.B * a.Tp * P) return;  // whole rows of 16 lanes
  const int p = (int)(item % P);
  const int t = (int)((item / P) % a.Tp);
  const int b = (int)(item / ((long long)P * a.Tp));
  const int64_t r0 = ((int64_t)b * a.Hq + 2 * p) * a.Tp + t, r1 = r0 + a.Tp;  // rows of heads 2p, 2p+1
  if (t >= a.T) {  // padding rows: zero E and lse (masked where read)
    if (l16 == 0) a.Dw[r0] = a.Dw[r1] = a.lsew[r0] = a.lsew[r1] = 0.f;
    return;
  }
  const int c = EL * l16;
  const uint16_t* dop = (const uint16_t*)a.dout.p + b * a.dout.sb + (int64_t)t * a.dout.st + p * a.dout.sh;
  const uint16_t* a0 = (const uint16_t*)a.attn.p + b * a.attn.sb + (int64_t)t * a.attn.st + (2 * p) * a.attn.sh;
  const uint16_t* a1 = a0 + a.attn.sh;
  const Vec gv = *(const Vec*)(dop + c), x0v = *(const Vec*)(a0 + c), x1v = *(const Vec*)(a1 + c);
  const uint32_t* gw = (const uint32_t*)&gv;
  const uint32_t* w0 = (const uint32_t*)&x0v;
  const uint32_t* w1 = (const uint32_t*)&x1v;
  auto lo = [](uint32_t w) { return __builtin_bit_cast(float, w << 16); };
  auto hi = [](uint32_t w) { return __builtin_bit_cast(float, w & 0xffff0000u); };
  const float lg = ((const float*)a.lam.p)[b * a.lam.sb + (int64_t)t * a.lam.st + p * a.lam.sh];
  const float s = sigmoid_f32(lg);
  // E_2p = <dout, attn_2p> and E_2p+1 = <dout, attn_2p+1>; the second also
  // feeds d lam.  The odd head's d attn is c dout with c = -s: its lse is
  // kept as lse - log2(s), so the P rebuilt from it is s P = -c P (0 where
  // s is 0), and the kernels fold the sign in.
  float x = 0.f, y = 0.f;
#pragma unroll
  for (int i = 0; i < EL / 2; ++i) {
    x += lo(gw[i]) * lo(w0[i]) + hi(gw[i]) * hi(w0[i]);
    y += lo(gw[i]) * lo(w1[i]) + hi(gw[i]) * hi(w1[i]);
  }
  x = row16_sum(x);
  y = row16_sum(y);
  if (l16 == 0) {
    a.Dw[r0] = x;
    a.Dw[r1] = y;
    a.lsew[r0] = a.lse[((int64_t)b * a.Hq + 2 * p) * a.T + t];
    a.lsew[r1] = a.lse[((int64_t)b * a.Hq + 2 * p + 1) * a.T + t] - log2f(s);
    ((float*)a.dlam.p)[b * a.dlam.sb + (int64_t)t * a.dlam.st + p * a.dlam.sh] = -s * (1.f - s) * y;
  }
}

// ---- shared tile machinery -------------------------------------------------
// A streamed tile is kBT rows of D bf16 of one tensor (row stride `st`
// elements), copied HBM -> LDS in 1 KB chunks, its 16-byte chunks
// XOR-swizzled for the reads it serves (TileLayout: ds_read_b128 row reads,
// ds_read_b64_tr_b16 transpose reads, or both).  Rows past the end are
// clamped to the last row (finite data; masked where used).
template <int D, int NW = kNW>
struct TileDma {
  static constexpr int BYTES = kBT * D * 2;
  static constexpr int CH = BYTES / 1024;  // 1 KB copies per tensor tile
  // issue this wave's copies of chunks wave, wave + NW, ... of one tensor tile
  __device__ static void issue(const uint16_t* base, int64_t st, int row0, int T, int layout, uint32_t lds,
                               int wave, int lane) {
    const bool tail = row0 + kBT > T;
    for (int ci = wave; ci < CH; ci += NW) {
      const int pos = ci * 64 + lane;
      const int r = pos / (D / 8), sc = pos % (D / 8);
      const int sw = tile_swizzle<D>(layout, r);
      const int rr = tail ? min(r, T - 1 - row0) : r;
      const uint32_t off = ((uint32_t)rr * (uint32_t)st + (uint32_t)((sc ^ sw) * 8)) * 2u;
      dma16_sbase(base + (int64_t)row0 * st, off, lds + ci * 1024);
    }
  }
};

// The same copies with the per-lane source offsets of a full tile computed
// once: wave w moves chunks w, w + NW, ... (PER of them); a ragged tile (rows
// past T) goes through TileDma::issue instead.
template <int D, int NW>
struct TileCopy {
  static constexpr int CH = TileDma<D, NW>::CH;
  static constexpr int PER = (CH + NW - 1) / NW;
  uint32_t off[PER];
  __device__ void init(int64_t st, int layout, int wave, int lane) {
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int pos = (wave + i * NW) * 64 + lane;
      const int r = pos / (D / 8), sc = pos % (D / 8);
      const int sw = tile_swizzle<D>(layout, r);
      off[i] = ((uint32_t)r * (uint32_t)st + (uint32_t)((sc ^ sw) * 8)) * 2u;
    }
  }
  // the copies of a full tile whose row 0 starts at `base` (wave-uniform)
  __device__ void issue(const uint16_t* base, uint32_t lds, int wave) const {
#pragma unroll
    for (int i = 0; i < PER; ++i)
      if (wave + i * NW < CH) dma16_sbase(base, off[i], lds + (wave + i * NW) * 1024);
  }
};

// Per-lane LDS byte offsets of the transpose reads giving A operands
// X^T[c][rows of k-chunk kk] from a tile in the transpose (BOTH = false) or
// the both-ways (BOTH = true) layout (rows in the order the P-like B operands
// hold them: 16kk + 4hg + 0..3, then + 8).  base(v) + v * 64 addresses
// column block v of the lane's first row; off(cb, kk, h) is the byte offset
// of column block cb in rows + 16 kk + 8 h from the base it uses, which is
// base(cb % NV) (both-ways layout, h = 1: base((cb ^ 1) % NV), since the
// swizzle of the row 8 further down flips bit 2 of the chunk).
template <int D, bool BOTH = false>
struct TrBases {
  static constexpr int NV = D >= 128 ? 4 : 2;
  uint32_t b[NV];
  __device__ void init(int lane) {
    const int l16 = lane & 15, g16 = lane >> 4;
    const int vr = 4 * (g16 >> 1) + (l16 >> 2);
    const int cl = 2 * (g16 & 1) + ((l16 & 3) >> 1);
    const int x = BOTH ? u_swizzle<D>(vr) : v_swizzle<D>(vr);
#pragma unroll
    for (int v = 0; v < NV; ++v) b[v] = vr * (D * 2) + (((4 * v + cl) ^ x) - 4 * v) * 16 + (l16 & 1) * 8;
  }
  static constexpr int src(int cb, int h) { return ((BOTH && h) ? (cb ^ 1) : cb) % NV; }
  static constexpr int off(int cb, int kk, int h) {
    return ((BOTH && h) ? (cb ^ 1) : cb) * 64 + (16 * kk + 8 * h) * (D * 2);
  }
};

__device__ __forceinline__ void wait_copies() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// Wait for every read in flight and pass a loaded register through the
// wait: the compiler then sees the value as available from here on and puts
// no wait of its own before a later use (such a wait, vmcnt(0) inside the
// loop, would also hold up the tile copies issued ahead of their use).
__device__ __forceinline__ void retire(bf16x8& x) {
  uint4 u = as_u4(x);
  asm volatile("s_waitcnt vmcnt(0)" : "+v"(u.x), "+v"(u.y), "+v"(u.z), "+v"(u.w));
  x = as_bf16x8(u);
}
__device__ __forceinline__ void retire(float& x) { asm volatile("s_waitcnt vmcnt(0)" : "+v"(x)); }

// s_waitcnt vmcnt(n) for a wave-uniform n in [0, 31] (the count is an
// instruction immediate): wait until at most n of this wave's memory reads
// are in flight.
__device__ __forceinline__ void wait_vmcnt(int n) {
  static_for<0, 32>([&](auto c) {
    constexpr int C = decltype(c)::value;
    if (n == C) asm volatile("s_waitcnt vmcnt(%0)" ::"n"(C) : "memory");
  });
}

// ---- dQ ------------------------------------------------------------------------
// Workgroup: (b, head h, 32 kNW query rows); wave w owns rows i0 + 32 w.  D:
// q/k head dim; DV: v head dim (V2: D; V1: 2D, one launch per map).
template <int D, int DV>
struct DqCfg {
  static constexpr int STAGE = TileDma<D>::BYTES + TileDma<DV>::BYTES;  // [K (both ways) | V (rows)]
  static constexpr int SMEM = 2 * STAGE;
};
// `bid`: the workgroup's index in the dQ grid order; `smem`: DqCfg::SMEM bytes
// of LDS, 1 KB aligned.
//
// As in the dK/dV kernel, the accumulators take one path through the loop
// body (key tiles after a wave's rows skip the scores and accumulate zeros),
// the mask is applied only on the diagonal tile, and E is folded into the G
// accumulator: the dout fragments are negated once and the accumulator
// starts at E, so the MFMAs leave E - G, P (E - G) = -dS (the odd head: +dS,
// its P being -c P), and dQ takes the sign when stored.
template <int D, int DV>
__device__ __forceinline__ void bwd_dq_body(const BwdArgs& a, int bid, unsigned char* smem) {
  constexpr int KS = D / 16, KSV = DV / 16, CB = D / 32;
  constexpr int KM = KS > KSV ? KS : KSV;
  using Dma = TileDma<D>;
  using DmaV = TileDma<DV>;
  constexpr int TB = Dma::BYTES;
  constexpr int STAGE = DqCfg<D, DV>::STAGE;
  static_assert(STAGE % (2 * DV) == 0 && TB % (2 * DV) == 0 && TB % (2 * D) == 0,
                "tile bases leave a row's chunk bits free");
  const uint32_t lds0 = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) unsigned char*)smem;

  const int tid = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int li = lane & 31, hg = lane >> 5;
  const int T = a.T, BM = 32 * kNW;
  const int tiles = (T + BM - 1) / BM;
  // heaviest row tiles first; within a tile index the kv group varies
  // fastest, so the workgroups on one XCD (id mod 8) share kv groups and
  // stream the same K/V tiles through its L2
  const int units = a.B * a.Hq;
  const int unit = bid % units, tile = tiles - 1 - bid / units;
  const int g = unit % a.Hkv, jq = unit / a.Hkv;
  const int b = jq / a.G, h = g * a.G + jq % a.G;
  const int i0w = tile * BM + 32 * wave;
  const bool active = i0w < T;
  const int kend = min(T, tile * BM + BM);
  const int nkt = (kend + kBT - 1) / kBT;
  const int row = i0w + li;

  const uint16_t* kp = (const uint16_t*)a.k.p + b * a.k.sb + g * a.k.sh;
  const uint16_t* vp = (const uint16_t*)a.v.p + b * a.v.sb + g * a.v.sh;
  // K is read as rows (S^T = K Q^T) and transposed (dQ += dS K): one copy in
  // the both-ways layout; V as rows only.
  TileCopy<D, kNW> ck;
  TileCopy<DV, kNW> cv;
  ck.init(a.k.st, kBothLayout, wave, lane);
  cv.init(a.v.st, kRowLayout, wave, lane);
  auto issue = [&](int kt, int stage) {
    const uint32_t st = lds0 + stage * STAGE;
    const int r0 = kt * kBT;
    if (r0 + kBT > T) {  // ragged last tile
      Dma::issue(kp, a.k.st, r0, T, kBothLayout, st, wave, lane);
      DmaV::issue(vp, a.v.st, r0, T, kRowLayout, st + TB, wave, lane);
    } else {
      ck.issue(kp + (int64_t)r0 * a.k.st, st, wave);
      cv.issue(vp + (int64_t)r0 * a.v.st, st + TB, wave);
    }
  };
  issue(0, 0);

  // B operands: Q^T and -dout^T of this wave's rows; the row's lse and E
  // (the odd head's lse carries -log2(s), so its P is s P = -c P and its dQ
  // takes the opposite sign at the store)
  bf16x8 qf[KS], af[KSV];
  {
    const uint16_t* qr = (const uint16_t*)a.q.p + b * a.q.sb + (int64_t)row * a.q.st + h * a.q.sh;
    const uint16_t* ar = (const uint16_t*)a.dout.p + b * a.dout.sb + (int64_t)row * a.dout.st + (h >> 1) * a.dout.sh;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      qf[ks] = as_bf16x8(row < T ? *(const uint4*)(qr + 16 * ks + 8 * hg) : make_uint4(0, 0, 0, 0));
#pragma unroll
    for (int ks = 0; ks < KSV; ++ks)
      af[ks] = as_bf16x8(row < T ? *(const uint4*)(ar + 16 * ks + 8 * hg) : make_uint4(0, 0, 0, 0));
  }
  const int64_t rr = ((int64_t)b * a.Hq + h) * a.Tp + min(row, a.Tp - 1);
  float lse_r = a.lsew[rr], D_r = a.Dw[rr];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) retire(qf[ks]);
#pragma unroll
  for (int ks = 0; ks < KSV; ++ks) {
    retire(af[ks]);
    const uint4 u = as_u4(af[ks]);  // sign flip of every bf16 (exact)
    af[ks] = as_bf16x8(make_uint4(u.x ^ 0x80008000u, u.y ^ 0x80008000u, u.z ^ 0x80008000u, u.w ^ 0x80008000u));
  }
  retire(lse_r);
  retire(D_r);
  // Row reads (K rows for S^T, V rows for dP^T): chunk (2 ks + hg) ^
  // swizzle(li) = 2 ks ^ (hg ^ swizzle(li)), so the address is
  // (tile base + lane part) ^ 32 ks.
  const uint32_t kxs = (uint32_t)(li * (2 * D) + ((hg ^ u_swizzle<D>(li)) << 4));
  const uint32_t vxs = (uint32_t)(li * (2 * DV) + ((hg ^ k_swizzle<DV>(li)) << 4));
  using TrB = TrBases<D, true>;
  TrB tb;
  tb.init(lane);
  const float sl2 = a.sl2;
  f32x16 acc[CB];  // -dQ^T
#pragma unroll
  for (int cb = 0; cb < CB; ++cb)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[cb][r] = 0.f;

  for (int kt = 0; kt < nkt; ++kt) {
    const int stage = kt & 1;
    wait_copies();
    __syncthreads();  // tile kt visible; the other stage is free
    if (kt + 1 < nkt) issue(kt + 1, stage ^ 1);
    const int j0 = kt * kBT;
    const uint32_t st = lds0 + stage * STAGE;
    uint32_t krow = st + kxs, vrow = st + TB + vxs;
    uint32_t tbase[TrB::NV];
#pragma unroll
    for (int v = 0; v < TrB::NV; ++v) tbase[v] = st + tb.b[v];
    asm volatile("" : "+v"(krow), "+v"(vrow));
#pragma unroll
    for (int v = 0; v < TrB::NV; ++v) asm volatile("" : "+v"(tbase[v]));
    // Key tiles entirely after this wave's rows (the last 3 at most) skip the
    // scores and accumulate zeros: the accumulators then take one path.
    bf16x8 dsk[2] = {};
    if (j0 <= i0w) {
      bf16x8 ka[KS], va[KSV];
#pragma unroll
      for (int ks = 0; ks < KM; ++ks) {
        if (ks < KS) ka[ks] = lds_read16(krow ^ (32u * ks));
        if (ks < KSV) va[ks] = lds_read16(vrow ^ (32u * ks));
      }
      f32x16 s, dp;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        s[r] = 0.f;
        dp[r] = D_r;
      }
#pragma unroll
      for (int ks = 0; ks < KM; ++ks) {
        if (ks < KS) s = mfma32x32x16(ka[ks], qf[ks], s);     // S^T = K Q^T
        if (ks < KSV) dp = mfma32x32x16(va[ks], af[ks], dp);  // E - G^T = E + V (-dout)^T
      }
      constexpr int NMF = KS + KSV;
      __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
      for (int i = 0; i < NMF; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        if (i + 4 < NMF) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      }
      // lane: row li; register r: key j0 + 8(r>>2) + 4hg + (r&3)
      float x[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) x[r] = fmaf(s[r], sl2, -lse_r);
      if (j0 == i0w) {  // the diagonal tile: keys after the row masked
        int lim = li - 4 * hg;  // kept: key offset 4hg + c <= li
        asm volatile("" : "+v"(lim));
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int c = 8 * (r >> 2) + (r & 3);
          x[r] = c <= lim ? x[r] : -INFINITY;
        }
      }
      f32x8 e0, e1;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float ds = __builtin_amdgcn_exp2f(x[r]) * dp[r];  // P (D - dP) = -dS
        if (r < 8) e0[r] = ds; else e1[r - 8] = ds;
      }
      dsk[0] = cvt_bf16x8(e0);
      dsk[1] = cvt_bf16x8(e1);
    }
#pragma unroll
    for (int kk = 0; kk < 2; ++kk)
#pragma unroll
      for (int cb = 0; cb < CB; ++cb) {
        const bf16x8 ka = join_bf16x8(tr_read(tbase[TrB::src(cb, 0)] + TrB::off(cb, kk, 0)),
                                      tr_read(tbase[TrB::src(cb, 1)] + TrB::off(cb, kk, 1)));
        acc[cb] = mfma32x32x16(ka, dsk[kk], acc[cb]);
      }
  }
  if (!active || row >= T) return;
  // dQ^T[c][row]: c = 32 cb + 8 (r>>2) + 4 hg + (r&3); dq = dS k / sqrt d
  uint16_t* dst = (uint16_t*)a.dq.p + b * a.dq.sb + (int64_t)row * a.dq.st + h * a.dq.sh;
  const float sc = (h & 1) ? a.scale : -a.scale;
#pragma unroll
  for (int cb = 0; cb < CB; ++cb)
#pragma unroll
    for (int g4 = 0; g4 < 4; ++g4) {
      uint2 w;
      w.x = pack_bf16x2(acc[cb][4 * g4 + 0] * sc, acc[cb][4 * g4 + 1] * sc);
      w.y = pack_bf16x2(acc[cb][4 * g4 + 2] * sc, acc[cb][4 * g4 + 3] * sc);
      *(uint2*)(dst + 32 * cb + 8 * g4 + 4 * hg) = w;
    }
}

template <int D, int DV>
__global__ void __launch_bounds__(kNW * 64, 2) bwd_dq_kernel(const BwdArgs a) {
  __shared__ __attribute__((aligned(1024))) unsigned char smem[DqCfg<D, DV>::SMEM];
  bwd_dq_body<D, DV>(a, blockIdx.x, smem);
}

// ---- dK, dV ------------------------------------------------------------------
// The two heads of a pair share dout: d attn of head 2p is dout and of head
// 2p+1 is c dout with c = -sigmoid(lam) per row, so both heads' dP come from
// the one product G = dout v^T (the odd head's is c G, its row term c E_odd
// with E_h = rowsum(dout * attn_h)), dS_2p = P_2p (G - E_2p), dS_2p+1 =
// c P_2p+1 (G - E_2p+1), and the pair's share of dV is the one product
// (P_2p + c P_2p+1)^T dout.
// Workgroup: (b, kv head g, 32 kNW keys), 2 kNW waves: waves m (A) and
// m + kNW (B) own keys j0 + 32 m (on one SIMD: wave w runs on SIMD w mod 4)
// and loop over the row tiles at or after their keys (rows descending) and,
// per row tile, the group's head pairs, one (row tile, pair) per period:
//   phase 1: A computes S and P of head 2p and -G = dout (-v)^T (its v
//            fragments negated once) and writes P_2p (bf16) and -G (fp32)
//            to LDS; B computes S and c P of head 2p+1;
//   barrier;
//   phase 2: A forms P_2p (E_2p - G) = -dS_2p and accumulates its part of
//            -dK^T += Q_2p^T (-dS_2p); B reads -G and P_2p, forms
//            c P_2p+1 (E_2p+1 - G) = -dS_2p+1, accumulates its part of
//            -dK^T += Q_2p+1^T (-dS_2p+1) and dV^T += dout^T (P_2p + c P_2p+1).
// Each wave issues 3 d / 16 MFMAs per pair (one S, G or dV, one dK) and
// one head's exponentials (6 products per pair instead of 8).  The two
// waves' dK parts are added in one order at the end.  A second barrier per
// period (before the next period's slots are written) is the stage barrier
// the copy ring needs anyway.  Masks (diagonal tile, rows past T) are
// applied only where needed; tiles of rows before the wave's keys skip the
// scores and accumulate zeros, so the accumulators take one path through
// the loop.  Copy pointers advance by running (pair, row) counters.
template <int D>
__global__ void __launch_bounds__(2 * kNW * 64, 1) bwd_dkdv_kernel(const BwdArgs a) {
  constexpr int NW = 2 * kNW;
  constexpr int KS = D / 16, CB = D / 32;
  constexpr int TB = kBT * 2 * D;      // bytes of one tensor tile
  constexpr int STAGE = 3 * TB + 512;  // [Q_2p | Q_2p+1 | dout (both ways) | lse x 2, E x 2 of the 32 rows]
  static_assert(STAGE % 256 == 0 && TB % 256 == 0, "tile bases leave the row's chunk bits free");
  constexpr int PSLOT = 2 * 1024;      // P_2p of one key block: 64 lanes x 2 x 16 bytes
  constexpr int GSLOT = 4 * 1024;      // -G of one key block: 64 lanes x 4 x 16 bytes
  constexpr int XBASE = 2 * STAGE;
  constexpr int SMEM_LOOP = XBASE + kNW * (PSLOT + GSLOT);
  constexpr int SMEM_END = kNW * CB * 16 * 64 * 4;  // B's dK parts, after the loop
  constexpr int SMEM = SMEM_LOOP > SMEM_END ? SMEM_LOOP : SMEM_END;
  __shared__ __attribute__((aligned(1024))) unsigned char smem[SMEM];
  static_assert(SMEM <= 160 * 1024, "LDS budget");
  const uint32_t lds0 = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) unsigned char*)smem;

  const int tid = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int li = lane & 31, hg = lane >> 5;
  const int kb = wave % kNW;
  const bool bwave = wave >= kNW;  // wave B (head 2p+1, dV), else wave A (head 2p, G)
  const int T = a.T, G = a.G, NP = a.G / 2, BK = 32 * kNW;
  const int units = a.B * a.Hkv;
  const int unit = blockIdx.x % units, kt = blockIdx.x / units;  // low key tiles (most rows) first
  const int b = unit / a.Hkv, g = unit % a.Hkv;
  const int J0 = kt * BK, j0w = J0 + 32 * kb;
  const bool active = j0w < T;
  const int key = j0w + li;
  const int nrt = (T + kBT - 1) / kBT;  // row tiles of 32
  const int rt0 = J0 / kBT;
  const int nit = NP * (nrt - rt0);    // (row tile, pair) iterations
  // Iteration it: row tile nrt-1 - it/NP (rows descending), pair g*NP + it%NP.
  // Every workgroup starts at the last row tile and they step down in
  // lockstep, so the workgroups of one kv group (one XCD: the group varies
  // fastest in the grid order) read the same Q / dout tiles at about the
  // same time, from that XCD's L2; a workgroup stops at its own first keys.

  // B operands: K^T of this wave's keys (both waves); -V^T (wave A only)
  bf16x8 kf[KS], vf[KS];
  {
    const uint16_t* r = (const uint16_t*)a.k.p + b * a.k.sb + (int64_t)key * a.k.st + g * a.k.sh;
    const uint16_t* rv = (const uint16_t*)a.v.p + b * a.v.sb + (int64_t)key * a.v.st + g * a.v.sh;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      kf[ks] = as_bf16x8(key < T ? *(const uint4*)(r + 16 * ks + 8 * hg) : make_uint4(0, 0, 0, 0));
      vf[ks] = as_bf16x8(key < T && !bwave ? *(const uint4*)(rv + 16 * ks + 8 * hg) : make_uint4(0, 0, 0, 0));
    }
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      retire(kf[ks]);
      retire(vf[ks]);
      const uint4 u = as_u4(vf[ks]);  // sign flip of every bf16 of V (exact)
      vf[ks] = as_bf16x8(make_uint4(u.x ^ 0x80008000u, u.y ^ 0x80008000u, u.z ^ 0x80008000u, u.w ^ 0x80008000u));
    }
  }

  // Copies.  Q of both heads and dout are each read as rows and transposed:
  // one copy each in the both-ways layout.  Waves 4-7 copy the rows' lse and
  // E of both heads (padded arrays: always in bounds).
  TileCopy<D, NW> cq0, cq1, co;
  cq0.init(a.q.st, kBothLayout, wave, lane);
  cq1.init(a.q.st, kBothLayout, wave, lane);
  co.init(a.dout.st, kBothLayout, wave, lane);
  const uint16_t* qg = (const uint16_t*)a.q.p + b * a.q.sb + (int64_t)g * G * a.q.sh;  // head g G, row 0
  const uint16_t* og = (const uint16_t*)a.dout.p + b * a.dout.sb + (int64_t)g * NP * a.dout.sh;
  const int rw = wave - (NW - 4);  // 0..3 on the row copiers
  // rows of head g G + 2p (lse, E) or + 1: base at row 0, step per pair
  const float* rsrc = rw <= 1 ? a.lsew + ((int64_t)b * a.Hq + g * G + rw) * a.Tp
                              : a.Dw + ((int64_t)b * a.Hq + g * G + rw - 2) * a.Tp;
  const int64_t rstep = 2 * (int64_t)a.Tp;
  // the next iteration to copy: pair, first row, and the pair's head-2p / dout bases
  int iss_p = 0, iss_r0 = (nrt - 1) * kBT;
  const uint16_t* iss_q = qg;
  const uint16_t* iss_o = og;
  const float* iss_rs = rsrc;
  auto issue = [&](int stage) {
    const uint32_t st = lds0 + stage * STAGE;
    const int i0 = iss_r0;
    const uint16_t* qh = iss_q;
    const uint16_t* oh = iss_o;
    const float* rs = iss_rs;
    if (++iss_p == NP) {
      iss_p = 0;
      iss_r0 -= kBT;
      iss_q = qg;
      iss_o = og;
      iss_rs = rsrc;
    } else {
      iss_q += 2 * a.q.sh;
      iss_o += a.dout.sh;
      iss_rs += rstep;
    }
    if (i0 + kBT > T) {  // ragged last row tile: rows past T repeat row T - 1
      TileDma<D, NW>::issue(qh, a.q.st, i0, T, kBothLayout, st, wave, lane);
      TileDma<D, NW>::issue(qh + a.q.sh, a.q.st, i0, T, kBothLayout, st + TB, wave, lane);
      TileDma<D, NW>::issue(oh, a.dout.st, i0, T, kBothLayout, st + 2 * TB, wave, lane);
    } else {
      cq0.issue(qh + (int64_t)i0 * a.q.st, st, wave);
      cq1.issue(qh + a.q.sh + (int64_t)i0 * a.q.st, st + TB, wave);
      co.issue(oh + (int64_t)i0 * a.dout.st, st + 2 * TB, wave);
    }
    if (rw >= 0 && lane < 8) dma16_sbase(rs + i0, lane * 16, st + 3 * TB + 128 * rw);
  };
  issue(0);

  // Row reads of A operands X[row li][16 ks + 8 hg ..]: chunk (2 ks + hg) ^
  // swizzle(li) = 2 ks ^ (hg ^ swizzle(li)); tile bases are multiples of 256,
  // so the read address is (tile base + rxs) ^ 32 ks.
  const uint32_t rxs = (uint32_t)(li * (2 * D) + ((hg ^ u_swizzle<D>(li)) << 4));
  using TrB = TrBases<D, true>;
  TrB tb;
  tb.init(lane);
  const float sl2 = a.sl2;
  // Exchange slots of key block kb (16-byte chunks, chunk-major: conflict-free)
  const uint32_t pslot = lds0 + XBASE + kb * (PSLOT + GSLOT) + lane * 16, gslot = pslot + PSLOT;
  f32x16 acc[CB], accv[CB];  // -dK^T part (both waves); dV^T (wave B) [c][key]
#pragma unroll
  for (int cb = 0; cb < CB; ++cb)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[cb][r] = accv[cb][r] = 0.f;
  // A += X^T Y over the tile's 32 rows (X^T by transpose reads of the tile at `tile`)
  auto accumulate = [&](f32x16 (&A)[CB], uint32_t tile, const bf16x8 (&y)[2]) {
    uint32_t tbase[TrB::NV];
#pragma unroll
    for (int v = 0; v < TrB::NV; ++v) tbase[v] = tile + tb.b[v];
#pragma unroll
    for (int v = 0; v < TrB::NV; ++v) asm volatile("" : "+v"(tbase[v]));
#pragma unroll
    for (int kk = 0; kk < 2; ++kk)
#pragma unroll
      for (int cb = 0; cb < CB; ++cb) {
        const bf16x8 xa = join_bf16x8(tr_read(tbase[TrB::src(cb, 0)] + TrB::off(cb, kk, 0)),
                                      tr_read(tbase[TrB::src(cb, 1)] + TrB::off(cb, kk, 1)));
        A[cb] = mfma32x32x16(xa, y[kk], A[cb]);
      }
  };
  auto rows4 = [&](uint32_t at, f32x4 (&v)[4]) {  // 16 row values of the lane: rows 8(r>>2) + 4hg + (r&3)
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) v[q4] = *(const __attribute__((address_space(3))) f32x4*)(uintptr_t)(at + 32 * q4);
  };

  int cmp_p = 0, cmp_r0 = (nrt - 1) * kBT;  // the next iteration to compute
  auto next_row0 = [&]() {
    const int i0 = cmp_r0;
    if (++cmp_p == NP) {
      cmp_p = 0;
      cmp_r0 -= kBT;
    }
    return i0;
  };
  // S and P of head e (0: 2p; 1: 2p+1, times -c) of the tile at sb, rows i0
  auto probs = [&](uint32_t sb, int i0, int e, f32x8& p0, f32x8& p1) {
    bf16x8 qa[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) qa[ks] = lds_read16((sb + e * TB + rxs) ^ (32u * ks));
    f32x4 lq[4];
    rows4(sb + 3 * TB + 128 * e + 16 * hg, lq);
    f32x16 sc;
#pragma unroll
    for (int r = 0; r < 16; ++r) sc[r] = 0.f;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) sc = mfma32x32x16(qa[ks], kf[ks], sc);  // S = Q K^T
    __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
    for (int i = 0; i < KS; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      if (i + 4 < KS) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
    // lane: key li; register r: row i0 + 8(r>>2) + 4hg + (r&3)
    float x[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) x[r] = fmaf(sc[r], sl2, -lq[r >> 2][r & 3]);
    if (i0 == j0w || i0 + kBT > T) {  // diagonal tile or rows past T
      // row offset ro = 4 hg + cc (cc = 8(r>>2) + (r&3)) is kept if ro < T - i0
      // and ro >= li (the key's offset) on the diagonal
      int lim = T - i0 - 4 * hg, dlo = i0 == j0w ? li - 4 * hg : -64;
      asm volatile("" : "+v"(lim), "+v"(dlo));
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int cc = 8 * (r >> 2) + (r & 3);
        x[r] = (cc < lim && cc >= dlo) ? x[r] : -INFINITY;
      }
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const float pr = __builtin_amdgcn_exp2f(x[r]);  // P_2p, or -c P_2p+1 (its lse carries -log2(s))
      if (r < 8) p0[r] = pr; else p1[r - 8] = pr;
    }
  };
  if (!bwave) {
    for (int it = 0; it < nit; ++it) {
      const int stage = it & 1;
      wait_copies();
      __syncthreads();  // tile it visible; the other stage and the slots are free
      if (it + 1 < nit) issue(stage ^ 1);
      const int i0 = next_row0();
      uint32_t sb = lds0 + stage * STAGE;
      asm volatile("" : "+v"(sb));
      f32x8 p0, p1;
      f32x16 ng;
      if (i0 >= j0w) {  // (else: rows before this wave's keys, or an inactive wave)
        bf16x8 oa[KS];
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) oa[ks] = lds_read16((sb + 2 * TB + rxs) ^ (32u * ks));
#pragma unroll
        for (int r = 0; r < 16; ++r) ng[r] = 0.f;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) ng = mfma32x32x16(oa[ks], vf[ks], ng);  // -G = dout (-V)^T
        probs(sb, i0, 0, p0, p1);
        *(__attribute__((address_space(3))) bf16x8*)(uintptr_t)pslot = cvt_bf16x8(p0);
        *(__attribute__((address_space(3))) bf16x8*)(uintptr_t)(pslot + 1024) = cvt_bf16x8(p1);
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          f32x4 v4;
#pragma unroll
          for (int e = 0; e < 4; ++e) v4[e] = ng[4 * q4 + e];
          *(__attribute__((address_space(3))) f32x4*)(uintptr_t)(gslot + 1024 * q4) = v4;
        }
      }
      __syncthreads();  // P_2p and -G in LDS
      bf16x8 y[2] = {};
      if (i0 >= j0w) {
        f32x4 ev[4];
        rows4(sb + 3 * TB + 256 + 16 * hg, ev);
        f32x8 d0, d1;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float p = r < 8 ? p0[r] : p1[r - 8];
          const float ds = p * (ev[r >> 2][r & 3] + ng[r]);  // P (E - G) = -dS
          if (r < 8) d0[r] = ds; else d1[r - 8] = ds;
        }
        y[0] = cvt_bf16x8(d0);
        y[1] = cvt_bf16x8(d1);
      }
      accumulate(acc, sb, y);  // -dK^T += Q_2p^T (-dS_2p)
    }
  } else {
    for (int it = 0; it < nit; ++it) {
      const int stage = it & 1;
      wait_copies();
      __syncthreads();
      if (it + 1 < nit) issue(stage ^ 1);
      const int i0 = next_row0();
      uint32_t sb = lds0 + stage * STAGE;
      asm volatile("" : "+v"(sb));
      f32x8 p0, p1;
      if (i0 >= j0w) probs(sb, i0, 1, p0, p1);
      __syncthreads();  // P_2p and -G in LDS
      bf16x8 y[2] = {}, pc[2] = {};
      if (i0 >= j0w) {
        f32x4 ev[4], gv[4];
        rows4(sb + 3 * TB + 384 + 16 * hg, ev);
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4)
          gv[q4] = *(const __attribute__((address_space(3))) f32x4*)(uintptr_t)(gslot + 1024 * q4);
        const uint4 w0 = as_u4(*(const __attribute__((address_space(3))) bf16x8*)(uintptr_t)pslot);
        const uint4 w1 = as_u4(*(const __attribute__((address_space(3))) bf16x8*)(uintptr_t)(pslot + 1024));
        const uint32_t pw[8] = {w0.x, w0.y, w0.z, w0.w, w1.x, w1.y, w1.z, w1.w};
        f32x8 d0, d1, c0, c1;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float p = r < 8 ? p0[r] : p1[r - 8];  // -c P_2p+1
          const uint32_t w = pw[r >> 1];  // P_2p: bf16 r of the 16 (element r & 1 of word r >> 1)
          const float pe = __builtin_bit_cast(float, (r & 1) ? (w & 0xffff0000u) : (w << 16));
          const float ds = p * (ev[r >> 2][r & 3] + gv[r >> 2][r & 3]);  // -c P (E - G) = dS
          if (r < 8) {
            d0[r] = ds, c0[r] = pe - p;  // P_2p + c P_2p+1
          } else {
            d1[r - 8] = ds, c1[r - 8] = pe - p;
          }
        }
        y[0] = cvt_bf16x8(d0);
        y[1] = cvt_bf16x8(d1);
        pc[0] = cvt_bf16x8(c0);
        pc[1] = cvt_bf16x8(c1);
      }
      accumulate(acc, sb + TB, y);       // B's part: dK^T += Q_2p+1^T dS_2p+1
      accumulate(accv, sb + 2 * TB, pc);  // dV^T += dout^T (P_2p + c P_2p+1)
    }
  }
  // -dK^T = A's part - B's part (one order), through LDS once every wave is done
  __syncthreads();
  f32x4* xk = (f32x4*)smem + (size_t)kb * CB * 4 * 64 + lane;  // [kb][cb][q4][lane]
  if (bwave) {
#pragma unroll
    for (int cb = 0; cb < CB; ++cb)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        f32x4 v4;
#pragma unroll
        for (int e = 0; e < 4; ++e) v4[e] = acc[cb][4 * q4 + e];
        xk[(cb * 4 + q4) * 64] = v4;
      }
  }
  __syncthreads();
  if (!bwave) {
#pragma unroll
    for (int cb = 0; cb < CB; ++cb)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const f32x4 v4 = xk[(cb * 4 + q4) * 64];
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[cb][4 * q4 + e] -= v4[e];
      }
  }
  if (!active || key >= T) return;
  const TOut& o = bwave ? a.dv : a.dk;
  const float sc = bwave ? 1.f : -a.scale;
  uint16_t* dst = (uint16_t*)o.p + b * o.sb + (int64_t)key * o.st + g * o.sh;
#pragma unroll
  for (int cb = 0; cb < CB; ++cb)
#pragma unroll
    for (int g4 = 0; g4 < 4; ++g4) {
      const f32x16& A = bwave ? accv[cb] : acc[cb];
      uint2 w;
      w.x = pack_bf16x2(A[4 * g4 + 0] * sc, A[4 * g4 + 1] * sc);
      w.y = pack_bf16x2(A[4 * g4 + 2] * sc, A[4 * g4 + 3] * sc);
      *(uint2*)(dst + 32 * cb + 8 * g4 + 4 * hg) = w;
    }
}

template <int D>
hipError_t launch(const BwdArgs& a, hipStream_t st) {
  const void* args[] = {&a};
  const long long items = (long long)a.B * a.Tp * (a.Hq / 2);
  hipError_t e = hipLaunchKernel((const void*)bwd_pre_kernel<D>, dim3((unsigned)((items + 15) / 16)), dim3(256),
                                 (void**)args, 0, st);
  if (e != hipSuccess) return e;
  const int qt = (a.T + 32 * kNW - 1) / (32 * kNW);
  e = hipLaunchKernel((const void*)bwd_dq_kernel<D, D>, dim3(a.B * a.Hq * qt), dim3(kNW * 64), (void**)args, 0, st);
  if (e != hipSuccess) return e;
  return hipLaunchKernel((const void*)bwd_dkdv_kernel<D>, dim3(a.B * a.Hkv * qt), dim3(2 * kNW * 64), (void**)args,
                         0, st);
}


// ==== DIFF V1 =======================================================================
//
// ("Differential Transformer V2" article, DiffAttnV1 pseudo-code; the RMSNorm
// arguments of Wilsontomass's module in the nanoGPT issue "How best to
// implement a differential transformer?")  Forward: a_m = causal softmax
// attention of map m over the shared 2d-wide v, D = a_1 - lam a_2,
// r = (mean D^2 + 1e-5)^(-1/2), out = (1 - lam_init) r D.  Backward:
//   dD = (1 - lam_init) r (dout - r^2 D mean(dout D)),  da_1 = dD,
//   da_2 = -lam dD,  dlam = -sum over rows of <dD, a_2>, and per map the
//   softmax-attention gradients (dv summed over both maps); the lambda
//   vectors get dlam times the derivative of exp(<lq, lk>).
// Since da_2 = c dD with c = -lam, both maps' softmax gradients come from the
// one product G = dD v^T:  dS_1 = P_1 (G - E_1),  dS_2 = c P_2 (G - E_2)
// with E_m = rowsum(dD * a_m), and dv = (P_1 + c P_2)^T dD is one product.
// Kernels: a pre-pass per (b, token, head) writes dD, E_1, E_2 and the
// padded lse rows; then one grid holds the dlam reduction (one workgroup,
// fixed order, writes the four vector gradients), dQ of both maps (the two
// maps' waves of the same rows sharing G) and dK of both maps with dv (four
// waves per 32-key block sharing S, G and P).

// lam = exp(<lq1, lk1>) - exp(<lq2, lk2>) + lam_init, the same bits in every
// wave that computes it (the pre-pass and the main grid)
template <int D>
__device__ __forceinline__ float v1_lambda(const V1BwdArgs& a) {
  const int lane = threadIdx.x & 63;
  float pa = 0.f, pb = 0.f;
#pragma unroll
  for (int i = 0; i < D / 64; ++i) {
    const int c = lane + 64 * i;
    pa += a.lq1[c] * a.lk1[c];
    pb += a.lq2[c] * a.lk2[c];
  }
  return expf(wave_sum(pa)) - expf(wave_sum(pb)) + a.lam_init;
}

// Sixteen lanes per (b, h, t), t < Tp: each lane holds 2d/16 consecutive
// channels (16-byte loads and stores), four items per wave with consecutive
// tokens, so each item's rows of [B, T, H, 2d] are whole 16-byte spans and
// the per-row arrays ([B][H][Tp], lse [2][B][H][T]) are written and read in
// runs (8% faster than consecutive heads at the GPT-2-small shape).
template <int D>
__global__ void __launch_bounds__(256) bwd_v1_pre_kernel(const V1BwdArgs a) {
  constexpr int DV = 2 * D, NV = DV / 128;  // 16-byte vectors (8 channels) per lane
  const int lane = threadIdx.x & 63, l16 = lane & 15;
  const float lam = v1_lambda<D>(a);  // once per wave
  const long long item = ((long long)blockIdx.x * 4 + (threadIdx.x >> 6)) * 4 + (lane >> 4);  // (b, h, t)
  if (item >= (long long)a.B * a.Tp * a.H) return;  // whole rows of 16 lanes
  const int t = (int)(item % a.Tp);
  const int h = (int)((item / a.Tp) % a.H);
  const int b = (int)(item / ((long long)a.H * a.Tp));
  const int64_t rw = ((int64_t)b * a.H + h) * a.Tp + t;
  if (t >= a.T) {  // padding rows: zero D and lse (masked where read)
    if (l16 == 0) a.Dw[0][rw] = a.Dw[1][rw] = a.lsew[0][rw] = a.lsew[1][rw] = 0.f;
    return;
  }
  const uint16_t* gp = (const uint16_t*)a.dout.p + b * a.dout.sb + (int64_t)t * a.dout.st + h * a.dout.sh;
  const uint16_t* a0 = (const uint16_t*)a.a[0].p + b * a.a[0].sb + (int64_t)t * a.a[0].st + h * a.a[0].sh;
  const uint16_t* a1 = (const uint16_t*)a.a[1].p + b * a.a[1].sb + (int64_t)t * a.a[1].st + h * a.a[1].sh;
  uint4 gv[NV], xv0[NV], xv1[NV];
#pragma unroll
  for (int v = 0; v < NV; ++v) {  // channels 128 v + 8 l16 .. + 7
    const int c = 128 * v + 8 * l16;
    gv[v] = *(const uint4*)(gp + c);
    xv0[v] = *(const uint4*)(a0 + c);
    xv1[v] = *(const uint4*)(a1 + c);
  }
  auto elem = [](const uint4& u, int e) {  // channel e of a 16-byte vector
    const uint32_t w = e < 2 ? u.x : e < 4 ? u.y : e < 6 ? u.z : u.w;
    return __builtin_bit_cast(float, (e & 1) ? (w & 0xffff0000u) : (w << 16));
  };
  float dd[NV][8], ss = 0.f, gd = 0.f;
#pragma unroll
  for (int v = 0; v < NV; ++v)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      dd[v][e] = elem(xv0[v], e) - lam * elem(xv1[v], e);  // D
      ss += dd[v][e] * dd[v][e];
      gd += elem(gv[v], e) * dd[v][e];
    }
  const float r = rsqrtf(row16_sum(ss) * (1.f / DV) + 1e-5f);
  const float pm = r * r * row16_sum(gd) * (1.f / DV);
  const float cr = (1.f - a.lam_init) * r;
  uint16_t* d0 = a.dD + (((int64_t)b * a.T + t) * a.H + h) * DV;
  float s0 = 0.f, s1 = 0.f, sl = 0.f;
#pragma unroll
  for (int v = 0; v < NV; ++v) {
    uint32_t w0[4];
#pragma unroll
    for (int e = 0; e < 8; e += 2) {
      const float dA = cr * (elem(gv[v], e) - dd[v][e] * pm), dB = cr * (elem(gv[v], e + 1) - dd[v][e + 1] * pm);
      w0[e / 2] = pack_bf16x2(dA, dB);
      // E_m from the rounded dD the MFMAs see
      const uint4 r0 = make_uint4(w0[e / 2], 0, 0, 0);
      s0 += elem(r0, 0) * elem(xv0[v], e) + elem(r0, 1) * elem(xv0[v], e + 1);
      s1 += elem(r0, 0) * elem(xv1[v], e) + elem(r0, 1) * elem(xv1[v], e + 1);
      sl -= dA * elem(xv1[v], e) + dB * elem(xv1[v], e + 1);
    }
    const int c = 128 * v + 8 * l16;
    *(uint4*)(d0 + c) = make_uint4(w0[0], w0[1], w0[2], w0[3]);
  }
  s0 = row16_sum(s0);
  s1 = row16_sum(s1);
  sl = row16_sum(sl);
  if (l16 == 0) {
    a.Dw[0][rw] = s0;
    a.Dw[1][rw] = s1;
    a.lsew[0][rw] = a.lse[(((int64_t)0 * a.B + b) * a.H + h) * a.T + t];
    a.lsew[1][rw] = a.lse[(((int64_t)1 * a.B + b) * a.H + h) * a.T + t];
    a.lamrow[((int64_t)b * a.T + t) * a.H + h] = sl;
  }
}

// One workgroup of NT threads: dlam = sum of the row terms, in a fixed order
// (thread t adds rows t + NT j into accumulator j mod 8, the eight are added
// in order, then a fixed tree), then the four vector gradients.  `part`: NT
// floats of LDS.
template <int D, int NT>
__device__ __forceinline__ void bwd_v1_lam_body(const V1BwdArgs& a, float* part) {
  const int tid = threadIdx.x;
  const long long n = (long long)a.B * a.T * a.H;
  float acc[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) acc[j] = 0.f;
  for (long long i0 = 0; i0 < n; i0 += 8LL * NT) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const long long i = i0 + (long long)j * NT + tid;
      acc[j] += i < n ? a.lamrow[i] : 0.f;
    }
  }
  float tot = 0.f;
#pragma unroll
  for (int j = 0; j < 8; ++j) tot += acc[j];
  part[tid] = tot;
  __syncthreads();
  for (int w = NT / 2; w > 0; w >>= 1) {
    if (tid < w) part[tid] += part[tid + w];
    __syncthreads();
  }
  const float dl = part[0];
  // e1 = exp(<lq1, lk1>), e2 = exp(<lq2, lk2>): every wave computes them
  float pa = 0.f, pb = 0.f;
  const int lane = tid & 63;
#pragma unroll
  for (int i = 0; i < D / 64; ++i) {
    const int c = lane + 64 * i;
    pa += a.lq1[c] * a.lk1[c];
    pb += a.lq2[c] * a.lk2[c];
  }
  const float e1 = expf(wave_sum(pa)), e2 = expf(wave_sum(pb));
  for (int c = tid; c < D; c += NT) {
    a.dlq1[c] = dl * e1 * a.lk1[c];
    a.dlk1[c] = dl * e1 * a.lq1[c];
    a.dlq2[c] = -dl * e2 * a.lk2[c];
    a.dlk2[c] = -dl * e2 * a.lq2[c];
  }
}

// dK of both maps and dv: workgroup (b, h, 32 NKB keys), four waves per
// 32-key block kb (wave w: kb = w % NKB, role w / NKB), over the row tiles at
// or after the keys, rows descending, one 32-row tile per step:
//   role 0 / 1 (map m = role): S_m = Q_m K_m^T with K_m^T of its keys in
//     registers, P_m (map 2: c P_2) in bf16 to LDS; after the barrier the
//     other map's P from LDS, P_1 + c P_2, and the d-wide half m of
//     dv^T += dD^T (P_1 + c P_2) by transpose reads of the dD tile;
//   role 2 / 3 (half m): the half-m part of -G = -dD v^T (channels m d ..
//     m d + d - 1 of dD rows, -v^T of its keys in registers) to LDS; after
//     the barrier -G = both halves (added in one order by both waves),
//     P_m (E_m - G) = -dS_m with P_m (c P_2 for map 2) from LDS, and
//     -dK_m^T += Q_m^T (-dS_m) by transpose reads of the Q_m tile.
// Each wave issues 2 d / 16 MFMAs per tile and each product is formed once
// (S of each map, G, dv, dK of each map).  With two key blocks, roles 0 and
// 2 (1 and 3) of one key block share a SIMD.  Q_1, Q_2 and dD are each read
// as rows and transposed: one copy each in the both-ways layout.
template <int D, int NKB>
struct V1DkvCfg {
  static constexpr int TB = TileDma<D>::BYTES;       // a Q_m tile (32 x d bf16)
  static constexpr int TBD = TileDma<2 * D>::BYTES;  // the dD tile (32 x 2d)
  // [Q_1 | Q_2 | dD | lse_1, lse_2, E_1, E_2 of the 32 rows]
  static constexpr int STAGE = 2 * TB + TBD + 512;
  static constexpr int PSLOT = 2048;  // a tile's P of one map: 64 lanes x 2 x 16 bytes
  static constexpr int GSLOT = 4096;  // a half of -G: 64 lanes x 4 x 16 bytes
  static constexpr int XKB = 2 * PSLOT + 2 * GSLOT;  // exchange slots of one key block
  static constexpr int XBASE = 2 * STAGE;
  static constexpr int SMEM = XBASE + NKB * XKB;
  static_assert(STAGE % (4 * D) == 0 && TB % (4 * D) == 0, "tile bases leave a row's chunk bits free");
};
template <int D, int NKB>
__device__ __forceinline__ void bwd_v1_dkv_body(const V1BwdArgs& a, int bid, float c, unsigned char* smem) {
  constexpr int DV = 2 * D;
  constexpr int KS = D / 16, CB = D / 32;
  constexpr int NW = 4 * NKB;
  using Cfg = V1DkvCfg<D, NKB>;
  constexpr int TB = Cfg::TB, STAGE = Cfg::STAGE, PSLOT = Cfg::PSLOT, GSLOT = Cfg::GSLOT;
  const uint32_t lds0 = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) unsigned char*)smem;

  const int tid = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int li = lane & 31, hg = lane >> 5;
  const int kb = wave % NKB, role = wave / NKB, m = role & 1;
  const bool pwave = role < 2;
  const int T = a.T;
  const int units = a.B * a.H;
  const int unit = bid % units, kt = bid / units;  // key tiles, low ones (most rows) first
  const int b = unit / a.H, h = unit % a.H;
  const int J0 = kt * 32 * NKB, j0w = J0 + 32 * kb;
  const int nrt = (T + kBT - 1) / kBT;
  const int nit = nrt - J0 / kBT;  // row tiles from the last down to J0
  if (nit <= 0) return;            // (keys past T: the whole workgroup)
  const bool active = j0w < T;
  const int key = j0w + li;
  auto it_row0 = [&](int it) { return (nrt - 1 - it) * kBT; };

  // B operands: K_m^T (role 0 / 1) or -v^T of half m (role 2 / 3) of this wave's keys
  bf16x8 fr[KS];
  {
    const TIn& t = pwave ? a.k[m] : a.v;
    const uint16_t* r = (const uint16_t*)t.p + b * t.sb + (int64_t)key * t.st + h * t.sh + (pwave ? 0 : m * D);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      fr[ks] = as_bf16x8(key < T ? *(const uint4*)(r + 16 * ks + 8 * hg) : make_uint4(0, 0, 0, 0));
    const uint32_t flip = pwave ? 0u : 0x80008000u;  // sign flip of every bf16 of v (exact)
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      retire(fr[ks]);
      const uint4 u = as_u4(fr[ks]);
      fr[ks] = as_bf16x8(make_uint4(u.x ^ flip, u.y ^ flip, u.z ^ flip, u.w ^ flip));
    }
  }

  // Copies: Q_1, Q_2 and dD tiles in the both-ways layout; the last four
  // waves copy the rows' lse_1, lse_2, E_1, E_2 (padded arrays: always in
  // bounds).
  const uint16_t* qb0 = (const uint16_t*)a.q[0].p + b * a.q[0].sb + h * a.q[0].sh;
  const uint16_t* qb1 = (const uint16_t*)a.q[1].p + b * a.q[1].sb + h * a.q[1].sh;
  const uint16_t* db = a.dD + ((int64_t)b * T * a.H + h) * DV;
  const int64_t dst_ = (int64_t)a.H * DV;
  const int rw4 = wave - (NW - 4);  // 0..3 on the row copiers
  const float* rowsrc = rw4 == 0 ? a.lsew[0] : rw4 == 1 ? a.lsew[1] : rw4 == 2 ? a.Dw[0] : a.Dw[1];
  rowsrc += ((int64_t)b * a.H + h) * a.Tp;
  TileCopy<D, NW> cq0, cq1;
  TileCopy<DV, NW> cd;
  cq0.init(a.q[0].st, kBothLayout, wave, lane);
  cq1.init(a.q[1].st, kBothLayout, wave, lane);
  cd.init(dst_, kBothLayout, wave, lane);
  auto issue = [&](int it, int stage) {
    const int i0 = it_row0(it);
    const uint32_t st = lds0 + stage * STAGE;
    if (i0 + kBT > T) {  // ragged last row tile: rows past T repeat row T - 1
      TileDma<D, NW>::issue(qb0, a.q[0].st, i0, T, kBothLayout, st, wave, lane);
      TileDma<D, NW>::issue(qb1, a.q[1].st, i0, T, kBothLayout, st + TB, wave, lane);
      TileDma<DV, NW>::issue(db, dst_, i0, T, kBothLayout, st + 2 * TB, wave, lane);
    } else {
      cq0.issue(qb0 + (int64_t)i0 * a.q[0].st, st, wave);
      cq1.issue(qb1 + (int64_t)i0 * a.q[1].st, st + TB, wave);
      cd.issue(db + (int64_t)i0 * dst_, st + 2 * TB, wave);
    }
    if (rw4 >= 0 && lane < 8) dma16_sbase(rowsrc + i0, lane * 16, st + 4 * TB + 128 * rw4);
  };
  issue(0, 0);

  // Row reads: chunk (2 ks + hg) ^ swizzle(li) = 2 ks ^ (hg ^ swizzle(li)),
  // so the address is (tile base + lane part) ^ 32 ks; half m of a dD row
  // starts at k-step m KS, i.e. XOR 32 m KS.
  const uint32_t qxs = (uint32_t)(li * (2 * D) + ((hg ^ u_swizzle<D>(li)) << 4));
  const uint32_t dxs = (uint32_t)(li * (2 * DV) + ((hg ^ u_swizzle<DV>(li)) << 4)) ^ (uint32_t)(32 * m * KS);
  // exchange slots of this key block: P of map mm at pslot(mm), half mm of -G at gslot(mm)
  const uint32_t xb = lds0 + Cfg::XBASE + kb * Cfg::XKB + lane * 16;
  auto pslot = [&](int mm) { return xb + mm * PSLOT; };
  auto gslot = [&](int mm) { return xb + 2 * PSLOT + mm * GSLOT; };
  const float sl2 = a.sl2;
  f32x16 acc[CB];  // dv^T of half m (roles 0 / 1) or -dK_m^T (roles 2 / 3) [c][key]
#pragma unroll
  for (int cb = 0; cb < CB; ++cb)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[cb][r] = 0.f;
  auto bf16_at = [](const uint32_t (&w)[8], int r) {  // bf16 r of 16 packed pairs, as fp32
    return __builtin_bit_cast(float, (r & 1) ? (w[r >> 1] & 0xffff0000u) : (w[r >> 1] << 16));
  };
  auto load_p = [&](uint32_t at, uint32_t (&w)[8]) {
    const uint4 p0 = as_u4(*(const __attribute__((address_space(3))) bf16x8*)(uintptr_t)at);
    const uint4 p1 = as_u4(*(const __attribute__((address_space(3))) bf16x8*)(uintptr_t)(at + 1024));
    w[0] = p0.x, w[1] = p0.y, w[2] = p0.z, w[3] = p0.w, w[4] = p1.x, w[5] = p1.y, w[6] = p1.z, w[7] = p1.w;
  };

  if (pwave) {
    using TrD = TrBases<DV, true>;
    TrD td;
    td.init(lane);
    // Column block cb of half m is block m CB + cb of the dD row: its lane
    // base is base((m CB + cb) % NV), so the bases are rotated by m CB.
    uint32_t tdb[TrD::NV];
#pragma unroll
    for (int v = 0; v < TrD::NV; ++v) tdb[v] = m ? td.b[(v + CB) % TrD::NV] : td.b[v];
    for (int it = 0; it < nit; ++it) {
      const int stage = it & 1;
      wait_copies();
      __syncthreads();  // tile it visible; the other stage and the exchange slots are free
      if (it + 1 < nit) issue(it + 1, stage ^ 1);
      const int i0 = it_row0(it);
      const uint32_t st = lds0 + stage * STAGE;
      uint32_t qrow = st + m * TB + qxs, rowst = st + 4 * TB + 128 * m + 16 * hg;
      uint32_t tbase[TrD::NV];
#pragma unroll
      for (int v = 0; v < TrD::NV; ++v) tbase[v] = st + 2 * TB + m * (CB * 64) + tdb[v];
      asm volatile("" : "+v"(qrow), "+v"(rowst));
#pragma unroll
      for (int v = 0; v < TrD::NV; ++v) asm volatile("" : "+v"(tbase[v]));
      const bool vis = i0 >= j0w;  // (else: rows before this wave's keys, or an inactive wave)
      if (vis) {
        bf16x8 qa[KS];
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) qa[ks] = lds_read16(qrow ^ (32u * ks));
        f32x4 lq[4];
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4)
          lq[q4] = *(const __attribute__((address_space(3))) f32x4*)(uintptr_t)(rowst + 32 * q4);
        f32x16 s;
#pragma unroll
        for (int r = 0; r < 16; ++r) s[r] = 0.f;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) s = mfma32x32x16(qa[ks], fr[ks], s);  // S = Q K^T
        __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
        for (int i = 0; i < KS; ++i) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        }
        // lane: key li; register r: row i0 + 8(r>>2) + 4hg + (r&3)
        float x[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) x[r] = fmaf(s[r], sl2, -lq[r >> 2][r & 3]);
        if (i0 == j0w || i0 + kBT > T) {  // diagonal tile or rows past T
          int lim = T - i0 - 4 * hg, dlo = i0 == j0w ? li - 4 * hg : -64;
          asm volatile("" : "+v"(lim), "+v"(dlo));
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int cc = 8 * (r >> 2) + (r & 3);
            x[r] = (cc < lim && cc >= dlo) ? x[r] : -INFINITY;
          }
        }
        const float pm = m ? c : 1.f;
        f32x8 e0, e1;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float pr = __builtin_amdgcn_exp2f(x[r]) * pm;  // P_1, or c P_2
          if (r < 8) e0[r] = pr; else e1[r - 8] = pr;
        }
        const uint32_t pw = pslot(m);
        *(__attribute__((address_space(3))) bf16x8*)(uintptr_t)pw = cvt_bf16x8(e0);
        *(__attribute__((address_space(3))) bf16x8*)(uintptr_t)(pw + 1024) = cvt_bf16x8(e1);
      }
      __syncthreads();  // P of both maps in LDS
      bf16x8 pc[2] = {};
      if (vis) {
        uint32_t w1[8], w2[8];
        load_p(pslot(0), w1);
        load_p(pslot(1), w2);
        f32x8 e0, e1;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float v = bf16_at(w1, r) + bf16_at(w2, r);  // P_1 + c P_2
          if (r < 8) e0[r] = v; else e1[r - 8] = v;
        }
        pc[0] = cvt_bf16x8(e0);
        pc[1] = cvt_bf16x8(e1);
      }
#pragma unroll
      for (int kk = 0; kk < 2; ++kk)
#pragma unroll
        for (int cb = 0; cb < CB; ++cb) {
          const bf16x8 xa = join_bf16x8(tr_read(tbase[TrD::src(cb, 0)] + TrD::off(cb, kk, 0)),
                                        tr_read(tbase[TrD::src(cb, 1)] + TrD::off(cb, kk, 1)));
          acc[cb] = mfma32x32x16(xa, pc[kk], acc[cb]);  // dv^T += dD^T (P_1 + c P_2)
        }
    }
  } else {
    using TrQ = TrBases<D, true>;
    TrQ tq;
    tq.init(lane);
    for (int it = 0; it < nit; ++it) {
      const int stage = it & 1;
      wait_copies();
      __syncthreads();
      if (it + 1 < nit) issue(it + 1, stage ^ 1);
      const int i0 = it_row0(it);
      const uint32_t st = lds0 + stage * STAGE;
      uint32_t drow = st + 2 * TB + dxs, rowst = st + 4 * TB + 256 + 128 * m + 16 * hg;
      uint32_t tbase[TrQ::NV];
#pragma unroll
      for (int v = 0; v < TrQ::NV; ++v) tbase[v] = st + m * TB + tq.b[v];
      asm volatile("" : "+v"(drow), "+v"(rowst));
#pragma unroll
      for (int v = 0; v < TrQ::NV; ++v) asm volatile("" : "+v"(tbase[v]));
      const bool vis = i0 >= j0w;
      f32x16 g;
      if (vis) {
        bf16x8 da[KS];
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) da[ks] = lds_read16(drow ^ (32u * ks));
#pragma unroll
        for (int r = 0; r < 16; ++r) g[r] = 0.f;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) g = mfma32x32x16(da[ks], fr[ks], g);  // half m of -G = dD (-v)^T
        __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
        for (int i = 0; i < KS; ++i) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          if (i + 4 < KS) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        }
        const uint32_t gw = gslot(m);
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          f32x4 v4;
#pragma unroll
          for (int e = 0; e < 4; ++e) v4[e] = g[4 * q4 + e];
          *(__attribute__((address_space(3))) f32x4*)(uintptr_t)(gw + 1024 * q4) = v4;
        }
      }
      __syncthreads();  // both halves of -G and P of both maps in LDS
      bf16x8 y[2] = {};
      if (vis) {
        f32x4 go[4], e4[4];
        const uint32_t gr = gslot(m ^ 1);
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          go[q4] = *(const __attribute__((address_space(3))) f32x4*)(uintptr_t)(gr + 1024 * q4);
          e4[q4] = *(const __attribute__((address_space(3))) f32x4*)(uintptr_t)(rowst + 32 * q4);
        }
        uint32_t w[8];
        load_p(pslot(m), w);
        f32x8 e0, e1;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float own = g[r], oth = go[r >> 2][r & 3];
          const float ng = m ? oth + own : own + oth;   // -G, the halves in one order
          const float ds = bf16_at(w, r) * (e4[r >> 2][r & 3] + ng);  // P_m (E_m - G) = -dS_m
          if (r < 8) e0[r] = ds; else e1[r - 8] = ds;
        }
        y[0] = cvt_bf16x8(e0);
        y[1] = cvt_bf16x8(e1);
      }
#pragma unroll
      for (int kk = 0; kk < 2; ++kk)
#pragma unroll
        for (int cb = 0; cb < CB; ++cb) {
          const bf16x8 xa = join_bf16x8(tr_read(tbase[TrQ::src(cb, 0)] + TrQ::off(cb, kk, 0)),
                                        tr_read(tbase[TrQ::src(cb, 1)] + TrQ::off(cb, kk, 1)));
          acc[cb] = mfma32x32x16(xa, y[kk], acc[cb]);  // -dK_m^T += Q_m^T (-dS_m)
        }
    }
  }
  if (!active || key >= T) return;
  const TOut& o = pwave ? a.dv : a.dk[m];
  const float sc = pwave ? 1.f : -a.scale;
  uint16_t* dst = (uint16_t*)o.p + b * o.sb + (int64_t)key * o.st + h * o.sh + (pwave ? m * D : 0);
#pragma unroll
  for (int cb = 0; cb < CB; ++cb)
#pragma unroll
    for (int g4 = 0; g4 < 4; ++g4) {
      uint2 w;
      w.x = pack_bf16x2(acc[cb][4 * g4 + 0] * sc, acc[cb][4 * g4 + 1] * sc);
      w.y = pack_bf16x2(acc[cb][4 * g4 + 2] * sc, acc[cb][4 * g4 + 3] * sc);
      *(uint2*)(dst + 32 * cb + 8 * g4 + 4 * hg) = w;
    }
}

// dQ of both maps: workgroup (b, h, 32 NRB rows), wave w: map m = w / NRB,
// rows i0 + 32 (w % NRB); the waves of the two maps of the same rows share
// the product G = dD v^T.  Per 32-key tile (K_1, K_2 in the both-ways
// layout, v in the row layout): S_m^T = K_m Q_m^T with Q_m^T of its rows in
// registers, and half m of -G^T (v channels m d .. m d + d - 1 against the
// same channels of -dD^T, in registers) to LDS; after the barrier -G^T =
// both halves (one order), P_m (E_m - G) = -dS_m (the map-2 factor c goes
// into the output scale), dQ_m^T += K_m^T (-dS_m^T) by transpose reads.
// 3 d / 16 MFMAs per wave and tile instead of 4 d / 16 with G formed per map.
template <int D, int NRB>
struct V1DqCfg {
  static constexpr int TB = TileDma<D>::BYTES, TBV = TileDma<2 * D>::BYTES;
  static constexpr int STAGE = 2 * TB + TBV;  // [K_1 | K_2 (both ways) | v (rows)]
  static constexpr int GSLOT = 4096;           // a half of -G^T: 64 lanes x 4 x 16 bytes
  static constexpr int XBASE = 2 * STAGE;
  static constexpr int SMEM = XBASE + NRB * 2 * GSLOT;
  static_assert(STAGE % (4 * D) == 0 && TB % (4 * D) == 0, "tile bases leave a row's chunk bits free");
};
template <int D, int NRB>
__device__ __forceinline__ void bwd_v1_dq_body(const V1BwdArgs& a, int tile, int unit, float c, unsigned char* smem) {
  constexpr int DV = 2 * D;
  constexpr int KS = D / 16, CB = D / 32;
  constexpr int NW = 2 * NRB;
  using Cfg = V1DqCfg<D, NRB>;
  constexpr int TB = Cfg::TB, STAGE = Cfg::STAGE, GSLOT = Cfg::GSLOT;
  const uint32_t lds0 = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) unsigned char*)smem;

  const int tid = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int li = lane & 31, hg = lane >> 5;
  const int rb = wave % NRB, m = wave / NRB;
  const int T = a.T, BM = 32 * NRB;
  if (tile * BM >= T) return;  // (rows past T: the whole workgroup)
  const int b = unit / a.H, h = unit % a.H;
  const int i0w = tile * BM + 32 * rb;
  const bool active = i0w < T;
  const int kend = min(T, tile * BM + BM);
  const int nkt = (kend + kBT - 1) / kBT;
  const int row = i0w + li;

  const uint16_t* kp0 = (const uint16_t*)a.k[0].p + b * a.k[0].sb + h * a.k[0].sh;
  const uint16_t* kp1 = (const uint16_t*)a.k[1].p + b * a.k[1].sb + h * a.k[1].sh;
  const uint16_t* vp = (const uint16_t*)a.v.p + b * a.v.sb + h * a.v.sh;
  TileCopy<D, NW> ck0, ck1;
  TileCopy<DV, NW> cv;
  ck0.init(a.k[0].st, kBothLayout, wave, lane);
  ck1.init(a.k[1].st, kBothLayout, wave, lane);
  cv.init(a.v.st, kRowLayout, wave, lane);
  auto issue = [&](int kt, int stage) {
    const uint32_t st = lds0 + stage * STAGE;
    const int r0 = kt * kBT;
    if (r0 + kBT > T) {  // ragged last tile
      TileDma<D, NW>::issue(kp0, a.k[0].st, r0, T, kBothLayout, st, wave, lane);
      TileDma<D, NW>::issue(kp1, a.k[1].st, r0, T, kBothLayout, st + TB, wave, lane);
      TileDma<DV, NW>::issue(vp, a.v.st, r0, T, kRowLayout, st + 2 * TB, wave, lane);
    } else {
      ck0.issue(kp0 + (int64_t)r0 * a.k[0].st, st, wave);
      ck1.issue(kp1 + (int64_t)r0 * a.k[1].st, st + TB, wave);
      cv.issue(vp + (int64_t)r0 * a.v.st, st + 2 * TB, wave);
    }
  };
  issue(0, 0);

  // B operands: Q_m^T and half m of -dD^T of this wave's rows; the row's lse and E_m
  bf16x8 qf[KS], af[KS];
  {
    const TIn& tq = a.q[m];
    const uint16_t* qr = (const uint16_t*)tq.p + b * tq.sb + (int64_t)row * tq.st + h * tq.sh;
    const uint16_t* ar = a.dD + (((int64_t)b * T + row) * a.H + h) * DV + m * D;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      qf[ks] = as_bf16x8(row < T ? *(const uint4*)(qr + 16 * ks + 8 * hg) : make_uint4(0, 0, 0, 0));
      af[ks] = as_bf16x8(row < T ? *(const uint4*)(ar + 16 * ks + 8 * hg) : make_uint4(0, 0, 0, 0));
    }
  }
  const int64_t rr = ((int64_t)b * a.H + h) * a.Tp + min(row, a.Tp - 1);
  float lse_r = a.lsew[m][rr], E_r = a.Dw[m][rr];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    retire(qf[ks]);
    retire(af[ks]);
    const uint4 u = as_u4(af[ks]);  // sign flip of every bf16 (exact)
    af[ks] = as_bf16x8(make_uint4(u.x ^ 0x80008000u, u.y ^ 0x80008000u, u.z ^ 0x80008000u, u.w ^ 0x80008000u));
  }
  retire(lse_r);
  retire(E_r);
  // Row reads: chunk (2 ks + hg) ^ swizzle(li) = 2 ks ^ (hg ^ swizzle(li)),
  // so the address is (tile base + lane part) ^ 32 ks; half m of a v row
  // starts at k-step m KS (XOR 32 m KS).
  const uint32_t kxs = (uint32_t)(li * (2 * D) + ((hg ^ u_swizzle<D>(li)) << 4));
  const uint32_t vxs = (uint32_t)(li * (2 * DV) + ((hg ^ k_swizzle<DV>(li)) << 4)) ^ (uint32_t)(32 * m * KS);
  using TrB = TrBases<D, true>;
  TrB tb;
  tb.init(lane);
  const uint32_t xs = lds0 + Cfg::XBASE + rb * 2 * GSLOT + lane * 16;  // slots of this row block
  const float sl2 = a.sl2;
  f32x16 acc[CB];  // -dQ_m^T (up to c)
#pragma unroll
  for (int cb = 0; cb < CB; ++cb)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[cb][r] = 0.f;

  for (int kt = 0; kt < nkt; ++kt) {
    const int stage = kt & 1;
    wait_copies();
    __syncthreads();  // tile kt visible; the other stage and the slots are free
    if (kt + 1 < nkt) issue(kt + 1, stage ^ 1);
    const int j0 = kt * kBT;
    const uint32_t st = lds0 + stage * STAGE;
    uint32_t krow = st + m * TB + kxs, vrow = st + 2 * TB + vxs;
    uint32_t tbase[TrB::NV];
#pragma unroll
    for (int v = 0; v < TrB::NV; ++v) tbase[v] = st + m * TB + tb.b[v];
    asm volatile("" : "+v"(krow), "+v"(vrow));
#pragma unroll
    for (int v = 0; v < TrB::NV; ++v) asm volatile("" : "+v"(tbase[v]));
    // Key tiles entirely after this row block's rows skip the scores and
    // accumulate zeros (the same for both maps' waves of the rows).
    const bool vis = j0 <= i0w;
    f32x16 s, gp;
    if (vis) {
      bf16x8 ka[KS], va[KS];
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        ka[ks] = lds_read16(krow ^ (32u * ks));
        va[ks] = lds_read16(vrow ^ (32u * ks));
      }
#pragma unroll
      for (int r = 0; r < 16; ++r) s[r] = gp[r] = 0.f;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        s = mfma32x32x16(ka[ks], qf[ks], s);    // S^T = K Q^T
        gp = mfma32x32x16(va[ks], af[ks], gp);  // half m of -G^T = v (-dD)^T
      }
      __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
      for (int i = 0; i < 2 * KS; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        if (i + 4 < 2 * KS) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      }
      const uint32_t gw = xs + m * GSLOT;
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        f32x4 v4;
#pragma unroll
        for (int e = 0; e < 4; ++e) v4[e] = gp[4 * q4 + e];
        *(__attribute__((address_space(3))) f32x4*)(uintptr_t)(gw + 1024 * q4) = v4;
      }
    }
    __syncthreads();  // both halves of -G^T of every row block in LDS
    bf16x8 dsk[2] = {};
    if (vis) {
      f32x4 go[4];
      const uint32_t gr = xs + (m ^ 1) * GSLOT;
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4)
        go[q4] = *(const __attribute__((address_space(3))) f32x4*)(uintptr_t)(gr + 1024 * q4);
      // lane: row li; register r: key j0 + 8(r>>2) + 4hg + (r&3)
      float x[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) x[r] = fmaf(s[r], sl2, -lse_r);
      if (j0 == i0w) {  // the diagonal tile: keys after the row masked
        int lim = li - 4 * hg;  // kept: key offset 4hg + c <= li
        asm volatile("" : "+v"(lim));
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int cc = 8 * (r >> 2) + (r & 3);
          x[r] = cc <= lim ? x[r] : -INFINITY;
        }
      }
      f32x8 e0, e1;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float own = gp[r], oth = go[r >> 2][r & 3];
        const float ng = m ? oth + own : own + oth;  // -G^T, the halves in one order
        const float ds = __builtin_amdgcn_exp2f(x[r]) * (E_r + ng);  // P (E - G) = -dS
        if (r < 8) e0[r] = ds; else e1[r - 8] = ds;
      }
      dsk[0] = cvt_bf16x8(e0);
      dsk[1] = cvt_bf16x8(e1);
    }
#pragma unroll
    for (int kk = 0; kk < 2; ++kk)
#pragma unroll
      for (int cb = 0; cb < CB; ++cb) {
        const bf16x8 ka = join_bf16x8(tr_read(tbase[TrB::src(cb, 0)] + TrB::off(cb, kk, 0)),
                                      tr_read(tbase[TrB::src(cb, 1)] + TrB::off(cb, kk, 1)));
        acc[cb] = mfma32x32x16(ka, dsk[kk], acc[cb]);
      }
  }
  if (!active || row >= T) return;
  // dQ^T[c][row]: c = 32 cb + 8 (r>>2) + 4 hg + (r&3); dq_m = c_m dS_m k_m / sqrt d
  const TOut& o = a.dq[m];
  uint16_t* dst = (uint16_t*)o.p + b * o.sb + (int64_t)row * o.st + h * o.sh;
  const float sc = -a.scale * (m ? c : 1.f);
#pragma unroll
  for (int cb = 0; cb < CB; ++cb)
#pragma unroll
    for (int g4 = 0; g4 < 4; ++g4) {
      uint2 w;
      w.x = pack_bf16x2(acc[cb][4 * g4 + 0] * sc, acc[cb][4 * g4 + 1] * sc);
      w.y = pack_bf16x2(acc[cb][4 * g4 + 2] * sc, acc[cb][4 * g4 + 3] * sc);
      *(uint2*)(dst + 32 * cb + 8 * g4 + 4 * hg) = w;
    }
}

// The dQ, dK and dv work of the V1 backward in one grid, so no workgroup
// waits for another kernel's tail: level L = 0, 1, ... (heaviest first) holds
// the dQ work of the 128 rows qt-1-L of both maps and the dK / dv work of
// the 128 keys 128 L .. (each a causal trapezoid of about the same size).
// NKB = 2 (d = 128): 512-thread workgroups, per level one dQ workgroup (128
// rows) and two 64-key dK / dv workgroups.  NKB = 1 (d = 64, where three
// 256-thread workgroups fit a CU): two 64-row dQ workgroups and four 32-key
// dK / dv workgroups.  The
// hardware deals consecutive workgroups to the 8 XCDs in turn (XCD = id mod
// 8); when the (batch, head) units divide by 8, XCD x takes the units u = x
// mod 8 only (its work in level order, then unit, then role), so the
// workgroups running together on one XCD stream the tiles of a few heads
// through its L2 instead of every head's.
#ifndef DA_V1_D64_NKB
#define DA_V1_D64_NKB 1
#endif
#ifndef DA_V1_D128_NKB
#define DA_V1_D128_NKB 2
#endif
template <int D>
struct V1MainCfg {
  static constexpr int NKB = D == 64 ? DA_V1_D64_NKB : DA_V1_D128_NKB;  // 32-key blocks per dK / dv workgroup
  static_assert(NKB == 1 || NKB == 2, "key blocks per workgroup");
  static constexpr int THREADS = NKB * kNW * 64;
  static constexpr int NRB = 2 * NKB;                 // 32-row blocks per dQ workgroup
  static constexpr int NQ = 4 / NRB;                  // dQ workgroups per level (128 rows)
  static constexpr int NKT = 4 / NKB;                 // dK / dv workgroups per level (128 keys)
  static constexpr int ROLES = NQ + NKT;
  static constexpr int a_ = V1DqCfg<D, NRB>::SMEM, b_ = V1DkvCfg<D, NKB>::SMEM, c_ = THREADS * 4;
  static constexpr int SMEM = a_ > b_ ? (a_ > c_ ? a_ : c_) : (b_ > c_ ? b_ : c_);
  static_assert(SMEM <= 160 * 1024, "LDS budget");
};
template <int D>
__global__ void __launch_bounds__(V1MainCfg<D>::THREADS, 3 - V1MainCfg<D>::NKB) bwd_v1_main_kernel(const V1BwdArgs a) {
  using Cfg = V1MainCfg<D>;
  __shared__ __attribute__((aligned(1024))) unsigned char smem[Cfg::SMEM];
  if (blockIdx.x == 0) {  // the dlam reduction, first so that it overlaps the rest
    bwd_v1_lam_body<D, Cfg::THREADS>(a, (float*)smem);
    return;
  }
  const int bh = a.B * a.H;
  const int id = blockIdx.x - 1;
  int level, u, role;  // role < NQ: dQ; then the dK / dv key tiles of the level
  if (bh % 8 == 0) {
    const int per = Cfg::ROLES * (bh / 8);  // one XCD's workgroups per level
    const int sx = id / 8, w = sx % per;
    level = sx / per;
    u = id % 8 + 8 * (w / Cfg::ROLES);
    role = w % Cfg::ROLES;
  } else {
    const int r = id % (Cfg::ROLES * bh);
    level = id / (Cfg::ROLES * bh);
    role = r / bh;
    u = r % bh;
  }
  const float c = -v1_lambda<D>(a);  // d a_2 = c dD
  if (role < Cfg::NQ) {  // rows 128 (qt-1-level) .., the later (heavier) row tile first
    const int qt = (a.T + 127) / 128;
    bwd_v1_dq_body<D, Cfg::NRB>(a, Cfg::NQ * (qt - 1 - level) + (Cfg::NQ - 1 - role), u, c, smem);
  } else {
    bwd_v1_dkv_body<D, Cfg::NKB>(a, (Cfg::NKT * level + role - Cfg::NQ) * bh + u, c, smem);
  }
}

template <int D>
hipError_t launch_v1(const V1BwdArgs& a, hipStream_t st) {
  using Cfg = V1MainCfg<D>;
  const void* args[] = {&a};
  const long long items = (long long)a.B * a.Tp * a.H;
  hipError_t e = hipLaunchKernel((const void*)bwd_v1_pre_kernel<D>, dim3((unsigned)((items + 15) / 16)), dim3(256),
                                 (void**)args, 0, st);
  if (e != hipSuccess) return e;
  const int qt = (a.T + 32 * kNW - 1) / (32 * kNW);
  return hipLaunchKernel((const void*)bwd_v1_main_kernel<D>, dim3(1 + Cfg::ROLES * a.B * a.H * qt),
                         dim3(Cfg::THREADS), (void**)args, 0, st);
}

}  // namespace

int backward_padded_rows(int T) { return (T + 127) / 128 * 128; }

hipError_t launch_backward_v2_bf16(int d, const BwdArgs& a, hipStream_t s) {
  if (d == 64) return launch<64>(a, s);
  if (d == 128) return launch<128>(a, s);
  return hipErrorInvalidValue;
}

hipError_t launch_backward_v1_bf16(int d, const V1BwdArgs& a, hipStream_t s) {
  if (d == 64) return launch_v1<64>(a, s);
  if (d == 128) return launch_v1<128>(a, s);
  return hipErrorInvalidValue;
}

}  // namespace da
