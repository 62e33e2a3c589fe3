// decode_bf16.hip -- DIFF V2 decode: one (or nq) new query tokens per
// sequence against a long KV cache ("Differential Transformer V2" article:
// DiffAttnV2 at the newest positions; the remark that decoding is
// memory-bound and that the paired heads of one GQA group share key and
// value).
//
// The cache is the only large operand (B*L*Hkv*d*2 bf16), so the kernel is
// built to stream it from HBM exactly once:
//   * split kernel: a workgroup owns (batch b, kv head g, one chunk of the
//     cache).  Its 4 waves take interleaved 32-token blocks.  Each block's K
//     and V rows are copied HBM -> the wave's LDS slot (global_load_lds,
//     16 bytes per lane, marked non-temporal: read once), the next block's
//     copy in flight while this one is computed by the other workgroup on
//     the CU.  The wave scores all G query heads of the group at once with
//     v_mfma_f32_16x16x32_bf16 (tokens x heads, K read back from LDS as the
//     operand), keeps a lazily rescaled online softmax per head and
//     accumulates O^T = V^T P^T with the same MFMA (V^T by transpose reads).
//     The four waves' (max, sum, O) states are then merged in LDS
//     (log-sum-exp) and one partial per (b, g, chunk, head) goes to the
//     caller's workspace.
//   * merge kernel: per (b, pair), the partials of both heads are merged in
//     split order (fixed, no atomics: deterministic), normalised and combined
//     as a_2p - sigmoid(lam[b, p]) a_2p+1.
// The paged variant (PAGED) reads the cache through a per-sequence page table
// and stops at each sequence's own length; splits past that length leave an
// empty partial (max -inf), which the merges skip.
// Several new tokens (nq > 1, the last nq cache entries): the MFMA columns
// are (query token, head) pairs instead of heads, 16 per column block and
// NCB = 1 or 2 blocks per workgroup, so one pass over the cache serves up to
// 32 of them; new token i masks the entries after its own position.
#include <math.h>

#include "kernels.hpp"
#include "rope.hpp"
#include "tile_ops.hpp"

namespace da {
namespace {

constexpr int kWaves = 4;         // split geometry: chunks are multiples of kWaves x kBlk tokens
constexpr int kBlk = 32;          // tokens per wave step
constexpr float kLazyLog2 = 8.f;  // rescale only when a head's max grows by > 2^8

// LDS slots per wave of the copy path: one (64 KB per workgroup at d = 128,
// two workgroups per CU, so while one computes a block the other's copy is
// in flight, and a CU whose split ends early takes another).  With the
// copies marked non-temporal, one slot per wave and two workgroups per CU
// measured 3% faster on the 4-token decode than two slots and one workgroup
// (DA_DEC_DENSE_SLOTS = 2); the paged decode was faster with one slot
// before as well.  The slot count changes only when copies are issued, not
// the arithmetic, so a paged cache whose pages lie in order gives the dense
// result bit for bit.
#ifndef DA_DEC_DENSE_SLOTS
#define DA_DEC_DENSE_SLOTS 1
#endif
template <bool PAGED>
constexpr int dec_slots() { return PAGED ? 1 : DA_DEC_DENSE_SLOTS; }
static_assert(2 * kPagedMaxChunk / (kBlk * kWaves) <= 64, "a paged wave holds its split's page-table entries one per lane");

// 16-byte chunk c of row r of a K or V block sits at chunk c ^ dec_swizzle(r)
// of its LDS row: the K operand reads (16 rows x one chunk per 16 lanes) and
// the V^T transpose reads (8 rows x 32 bytes per 32 lanes) then touch every
// bank once.  Depends on r & 15 only.
template <int D>
__device__ __forceinline__ int dec_swizzle(int r) {
  return D >= 128 ? (((r & 7) << 1) | ((r >> 3) & 1)) : ((((r >> 1) & 3) << 1) | ((r >> 3) & 1));
}

__device__ __forceinline__ void lds_fence() {
  // The LDS executes one wave's instructions in order; this waits for the
  // wave's outstanding LDS accesses and is a compiler barrier for memory, so
  // writes by some lanes are visible to reads by other lanes of the wave.
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
}

template <int D, bool PAGED, int NCB>
__global__ void __launch_bounds__(kWaves * 64, 2) decode_split_kernel(const DecodeArgs a) {
  constexpr int W = kWaves;  // waves per workgroup
  constexpr int KS = D / 32;   // k-steps of the score MFMA
  constexpr int CB = D / 16;   // 16-wide column blocks of O^T
  static_assert(kBlk == 32, "a step is two 16-token sub-blocks");
  constexpr int NST = dec_slots<PAGED>();
  static_assert(NST >= 1 && NST <= 3, "LDS slots per wave");
  constexpr int RB = D * 2;                 // bytes of a K / V row
  constexpr int TBYTES = kBlk * RB;         // one tensor's block
  constexpr int SLOT = 2 * TBYTES;          // [K block | V block]
  constexpr int RPI = 1024 / RB;            // rows per 1 KB copy instruction
  constexpr int NI = kBlk / RPI;            // copy instructions per tensor and block
  constexpr int CPR = D / 8;                // 16-byte chunks per row
  static_assert(16 % RPI == 0, "a copy instruction's rows lie in one 16-token sub-block");
  // K and V blocks are copied into per-wave LDS slots by global_load_lds;
  // K is read back as the MFMA operand, V^T by transpose reads.
  constexpr int LDS_STG = W * NST * SLOT;  // bytes
  constexpr int LDS_RED = W * 16 * (D + 2) * 4;       // bytes (one column block at a time)
  constexpr int LDS_BYTES = LDS_STG > LDS_RED ? LDS_STG : LDS_RED;
  __shared__ __attribute__((aligned(1024))) unsigned char smem[LDS_BYTES];
  const uint32_t lds_base = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) unsigned char*)smem;

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int c16 = lane & 15, kg = lane >> 4;

  // Workgroup -> (sequence b, column group cg, kv head g, split s).  A
  // "column" is one (query token, head of the group) pair; a workgroup scores
  // 16 NCB of them (column group cg), the pair (b, cg) acting as one virtual
  // sequence vb.  The hardware deals consecutive workgroups to the 8 XCDs in
  // turn (XCD = id mod 8).
  //  * dense (every sequence L long, uniform work): split fastest, then kv
  //    head, then virtual sequence (with nsplit a multiple of 8, XCD x takes
  //    the splits s = x mod 8 of every (vb, g)).
  //  * paged (ragged lengths: the late splits of short sequences are empty):
  //    only the non-empty splits get workgroups.  They are numbered in one
  //    packed list, virtual sequence by virtual sequence (split s of vb is
  //    unit prefix(vb) + s, prefix = the number of non-empty splits before
  //    vb, found from the lengths with a wave-wide scan); unit u takes
  //    workgroups Hkv u .. Hkv u + Hkv - 1, one per kv head, and the
  //    workgroups past the last unit exit at once.  So the workgroups with
  //    work are the first ones dispatched, dealt evenly over XCDs and CUs.
  const int bid = blockIdx.x;
  const int VB = a.B * a.ncg;
  int vb, g, s;
  if constexpr (PAGED) {
    const int u = bid / a.Hkv;
    g = bid % a.Hkv;
    vb = -1;
    s = 0;
    int done = 0;  // units in the virtual sequences before this 64-wide window
    for (int base = 0; base < VB; base += 64) {
      const int v = base + lane;
      int ns = 0;
      if (v < VB) ns = (min(max(a.seq_lens[v / a.ncg], 0), a.L) + a.chunk - 1) / a.chunk;
      int inc = ns;  // inclusive scan over the window
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const int t = __shfl_up(inc, o, 64);
        if (lane >= o) inc += t;
      }
      const int first = done + inc - ns;  // this lane's first unit
      const unsigned long long hit = __ballot(u >= first && u < first + ns);
      if (hit) {  // wave-uniform
        const int l = __ffsll((long long)hit) - 1;
        vb = base + l;
        s = u - __shfl(first, l, 64);
        break;
      }
      done += __shfl(inc, 63, 64);
    }
    if (vb < 0) return;  // past the last unit (uniform over the workgroup)
  } else {
    if (bid >= VB * a.Hkv * a.nsplit) return;  // padding
    s = bid % a.nsplit;
    g = (bid / a.nsplit) % a.Hkv;
    vb = bid / (a.nsplit * a.Hkv);
  }
  // (uniform by construction; in scalar registers, as the copies' bases must be)
  vb = __builtin_amdgcn_readfirstlane(vb);
  s = __builtin_amdgcn_readfirstlane(s);
  const int b = vb / a.ncg, cg = vb % a.ncg;
  const int G = a.G, NQ = a.nq, NC = NQ * G;
  // tokens of this sequence (paged: its own length, at most the longest)
  const int L = __builtin_amdgcn_readfirstlane(PAGED ? min(max(a.seq_lens[b], 0), a.L) : a.L);

  // q fragments: B operand of S = K q^T.  Column n*16 + c16 of the group is
  // query token qi, head hh; it sees cache entries t < lim (the new tokens
  // are the last NQ entries, each seeing itself and what precedes it).
  bf16x8 qf[NCB][KS];
  int lim[NCB];
#pragma unroll
  for (int n = 0; n < NCB; ++n) {
    const int col = (cg * NCB + n) * 16 + c16;
    const bool valid = col < NC;
    const int qi = valid ? col / G : 0, hh = valid ? col % G : 0;
    lim[n] = valid ? L - NQ + 1 + qi : L;
    const uint16_t* qrow =
        (const uint16_t*)a.q.p + b * a.q.sb + (int64_t)qi * a.q.st + (int64_t)(g * G + hh) * a.q.sh;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      qf[n][ks] = as_bf16x8(valid ? *(const uint4*)(qrow + 32 * ks + 8 * kg) : make_uint4(0, 0, 0, 0));
    // rotary embedding of the new token at its cache position (elements 32 ks + 8 kg + e)
    if (a.rope) rope_rotate_frags<KS, 32>(qf[n], 8 * kg, max(L - NQ + qi, 0), a.rope_w);
  }
  const uint16_t* kbase = (const uint16_t*)a.k.p + (PAGED ? 0 : b * a.k.sb) + g * a.k.sh;
  const uint16_t* vbase = (const uint16_t*)a.v.p + (PAGED ? 0 : b * a.v.sb) + g * a.v.sh;
  const int64_t kst = a.k.st, vst = a.v.st;
  // Paged cache: pages hold a power of two >= 16 tokens, so each 16-token
  // sub-block of a block lies in one page and one table entry locates it.  A
  // wave's split holds at most 32 steps, i.e. 64 sub-blocks: lane e holds the
  // entry of the wave's sub-block e (step e/2), loaded once, read per step
  // with readlane.  A sub-block past the sequence's end takes the entry of its
  // last token (its rows are masked); entries outside [0, num_pages) are
  // clamped.
  const int pmask = PAGED ? a.page_mask : 0;
  const int t0 = s * a.chunk, t1 = min(L, t0 + a.chunk);
  const int wv = __builtin_amdgcn_readfirstlane(wave);
  const int blk0 = t0 + kBlk * wv;
  const int nsteps = blk0 < t1 ? (t1 - blk0 + kBlk * W - 1) / (kBlk * W) : 0;
  int ent = 0;
  if constexpr (PAGED) {
    if (L > 0) {
      const int tok = min(blk0 + kBlk * W * (lane >> 1) + 16 * (lane & 1), L - 1);
      ent = a.block_table[(int64_t)b * a.bt_stride + (tok >> a.page_shift)];
    }
  }
  // q fragments and table entries have landed before the first copy is issued
  // (no compiler-placed wait inside the loop, which would also wait for copies)
#pragma unroll
  for (int n = 0; n < NCB; ++n)
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) asm volatile("s_waitcnt vmcnt(0)" : "+v"(qf[n][ks]));
  asm volatile("s_waitcnt vmcnt(0)" : "+v"(ent));

  // ---- copies: this wave's block -> its LDS slot (global_load_lds) ----------
  // Copy i of a tensor moves rows i*RPI .. i*RPI + RPI-1; the lane moves
  // source chunk (lane % CPR) ^ swizzle(row) of row i*RPI + lane / CPR into
  // slot chunk lane % CPR.  A block is two 16-row halves (each in one page of
  // a paged cache); copy i = h * CPH + j of half h moves rows 16 h + j*RPI ..,
  // and its per-lane source offset from the half's first row depends on j
  // only (the swizzle depends on the row mod 16), so CPH offsets per tensor
  // are computed once.  Rows past the sequence's end repeat its last row
  // (finite data; their scores are masked to -inf below): a block holding
  // them takes the per-copy path.
  constexpr int CPH = 16 / RPI;  // copies per 16-row half
  const int r_in = lane / CPR;
  uint32_t choff[NI];  // the lane's chunk byte offset in copy i (same for K and V)
#pragma unroll
  for (int i = 0; i < NI; ++i) choff[i] = (uint32_t)(((lane % CPR) ^ dec_swizzle<D>(i * RPI + r_in)) * 16);
  const uint32_t krow = (uint32_t)(r_in * kst * 2), vrow = (uint32_t)(r_in * vst * 2);
  uint32_t kho[CPH], vho[CPH];  // full half: offsets of its copies from the half's first row
#pragma unroll
  for (int j = 0; j < CPH; ++j) {
    kho[j] = krow + (uint32_t)(j * RPI * kst * 2) + choff[j];
    vho[j] = vrow + (uint32_t)(j * RPI * vst * 2) + choff[j];
  }
  const uint32_t slot0 = lds_base + wv * (NST * SLOT);
  auto issue = [&](int n, int slot) {
    const int blk = blk0 + kBlk * W * n;
    const uint32_t dst = slot0 + slot * SLOT;
    if (blk + kBlk <= L) {  // full block (uniform)
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const uint16_t *kb, *vb;  // the half's first row
        if constexpr (PAGED) {
          const int raw = __builtin_amdgcn_readlane(ent, 2 * n + h);
          const int pg = min(max(raw, 0), a.num_pages - 1);
          const int prow = (blk + 16 * h) & pmask;
          kb = kbase + (int64_t)pg * a.k.sb + (int64_t)prow * kst;
          vb = vbase + (int64_t)pg * a.v.sb + (int64_t)prow * vst;
        } else {
          kb = kbase + (int64_t)(blk + 16 * h) * kst;
          vb = vbase + (int64_t)(blk + 16 * h) * vst;
        }
#pragma unroll
        for (int j = 0; j < CPH; ++j) {
          dma16_sbase_nt(kb, kho[j], dst + (h * CPH + j) * 1024);
          dma16_sbase_nt(vb, vho[j], dst + TBYTES + (h * CPH + j) * 1024);
        }
      }
      return;
    }
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int sub = (i * RPI) / 16;
      int64_t kb, vb;  // element offsets of the copy's anchor row
      int anchor;      // token of that row
      if constexpr (PAGED) {
        anchor = min(blk + 16 * sub, L - 1);
        const int raw = __builtin_amdgcn_readlane(ent, 2 * n + sub);
        const int pg = min(max(raw, 0), a.num_pages - 1);
        kb = (int64_t)pg * a.k.sb + (int64_t)(anchor & pmask) * kst;
        vb = (int64_t)pg * a.v.sb + (int64_t)(anchor & pmask) * vst;
      } else {
        anchor = blk;
        kb = (int64_t)blk * kst;
        vb = (int64_t)blk * vst;
      }
      const int tok = min(blk + i * RPI + r_in, L - 1);
      const uint32_t ko = (uint32_t)((tok - anchor) * kst * 2) + choff[i];
      const uint32_t vo = (uint32_t)((tok - anchor) * vst * 2) + choff[i];
      dma16_sbase_nt(kbase + kb, ko, dst + i * 1024);
      dma16_sbase_nt(vbase + vb, vo, dst + TBYTES + i * 1024);
    }
  };

  // Per-lane LDS read addresses within a slot, as a base XOR a constant:
  //   K operand of S = K q^T: lane (c16, kg) reads row 16 sub + c16, chunk
  //   (4 ks + kg) ^ swizzle(c16) = 4 ks ^ (kg ^ swizzle(c16)): base kxb
  //   (sub 0) XOR 64 ks, + 16 RB for sub 1 (the swizzle depends on the row
  //   mod 16, and rows are RB >= 128 bytes: the XOR stays inside a row).
  //   V^T operand (transpose read): lane (L = lane & 15, kg) points at row
  //   vr = 4 kg + (L >> 2) (+ 16 for the second read), chunk (2 cb + b0) ^
  //   swizzle(vr) = 2 cb ^ (b0 ^ swizzle(vr)), b0 = (L & 3) >> 1, plus 8 bytes
  //   for odd L: base vxb XOR 32 cb; it receives channel 16 cb + L of tokens
  //   4 kg .. 4 kg + 3 (16 + ...)
  const uint32_t kxb = (uint32_t)(c16 * RB + ((kg ^ dec_swizzle<D>(c16)) << 4));
  uint32_t vxb;
  {
    const int l16 = lane & 15, vr = 4 * kg + (l16 >> 2);
    vxb = (uint32_t)(TBYTES + vr * RB + ((((l16 & 3) >> 1) ^ dec_swizzle<D>(vr)) << 4) + 8 * (l16 & 1));
  }

  const float sl2 = a.sl2;
  float mref[NCB], lsum[NCB];
  f32x4 o[NCB][CB];
#pragma unroll
  for (int n = 0; n < NCB; ++n) {
    mref[n] = -INFINITY;
    lsum[n] = 0.f;
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) o[n][cb] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  // Softmax state of column block n2 over one block's scores sc (lane (column
  // c16, kg) holds tokens blk + 16 sub + 4 kg + r): mask, lazy rescale,
  // probabilities as the bf16 B operand of P.V (slot t: token 4 kg + t for
  // t < 4, 16 + 4 kg + t - 4 for t >= 4).
  // Only a block reaching the first masked entry (past the sequence's end,
  // or after a new token's own position) applies the mask (a uniform test).
  const int mask_from = L - NQ + 1;
  auto softmax_block = [&](f32x4* sc, int blk, int n2) -> bf16x8 {
    if (blk + kBlk > mask_from) {
#pragma unroll
      for (int sub = 0; sub < 2; ++sub)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (blk + 16 * sub + 4 * kg + r >= lim[n2]) sc[sub][r] = -INFINITY;
    }
    float mx = -INFINITY;
#pragma unroll
    for (int sub = 0; sub < 2; ++sub)
#pragma unroll
      for (int r = 0; r < 4; ++r) mx = fmaxf(mx, sc[sub][r]);
    mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    // -inf when the whole block is masked for this column (a later query
    // token's entries only); then nothing changes below
    const float mb = mx * sl2;
    const bool need = mb > mref[n2] + kLazyLog2;
    if (__builtin_amdgcn_ballot_w64(need)) {
      const float al = need ? exp2f(mref[n2] - mb) : 1.f;
      if (need) mref[n2] = mb;
      lsum[n2] *= al;
#pragma unroll
      for (int cb = 0; cb < CB; ++cb) o[n2][cb] *= al;
    }
    // a column that has seen no visible entry yet has every score -inf:
    // use 0 for its reference so the probabilities are 0, not NaN
    const float nm = mref[n2] == -INFINITY ? 0.f : -mref[n2];
    f32x8 p;
    float ps = 0.f;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      p[r] = __builtin_amdgcn_exp2f(fmaf(sc[0][r], sl2, nm));
      p[r + 4] = __builtin_amdgcn_exp2f(fmaf(sc[1][r], sl2, nm));
      ps += p[r] + p[r + 4];
    }
    lsum[n2] += ps;
    return cvt_bf16x8(p);
  };

  // Block n goes to slot n % NST, issued NST - 1 steps ahead (NST = 1: right
  // after the previous block's reads); the slot it overwrites was last read
  // at the end of the step before.
  if (NST == 1) {
    if (nsteps > 0) issue(0, 0);
  } else {
#pragma unroll
    for (int p = 0; p < NST - 1; ++p)
      if (p < nsteps) issue(p, p);
  }
  for (int n = 0; n < nsteps; ++n) {
    const int blk = blk0 + kBlk * W * n;
    const int cur = n % NST;
    if (NST > 1 && n + NST - 1 < nsteps) issue(n + NST - 1, (n + NST - 1) % NST);
    // block n's copies have landed once at most the later blocks' remain
    const int later = NST == 1 ? 0 : min(NST - 1, nsteps - 1 - n);
    if (NST > 2 && later >= 2) {
      asm volatile("s_waitcnt vmcnt(%0)" ::"n"(4 * NI) : "memory");
    } else if (NST > 1 && later >= 1) {
      asm volatile("s_waitcnt vmcnt(%0)" ::"n"(2 * NI) : "memory");
    } else {
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    }
    const uint32_t sb = slot0 + cur * SLOT;
    // (opaque to the compiler: otherwise it keeps base + constant for every
    // read in a register of its own)
    uint32_t kb0 = sb + kxb, vb0 = sb + vxb;
    asm volatile("" : "+v"(kb0), "+v"(vb0));

    // ---- scores S[tok][col], softmax state per column ----
    bf16x8 pk[NCB];  // slot t: token 4kg+t (t<4), 16+4kg+t-4 (t>=4)
    f32x4 sc[NCB][2];
#pragma unroll
    for (int n2 = 0; n2 < NCB; ++n2) sc[n2][0] = sc[n2][1] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const uint32_t ka_addr = kb0 ^ (64u * ks);
#pragma unroll
      for (int sub = 0; sub < 2; ++sub) {
        const bf16x8 ka = lds_read16(ka_addr + sub * 16 * RB);
#pragma unroll
        for (int n2 = 0; n2 < NCB; ++n2) sc[n2][sub] = mfma16x16x32(ka, qf[n2][ks], sc[n2][sub]);
      }
    }
#pragma unroll
    for (int n2 = 0; n2 < NCB; ++n2) pk[n2] = softmax_block(sc[n2], blk, n2);

    // ---- O^T[c][col] += V^T[c][tok] P^T[tok][col] (V^T by transpose reads) ----
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) {
      const uint32_t va_addr = vb0 ^ (32u * cb);
      const bf16x8 va = join_bf16x8(tr_read(va_addr), tr_read(va_addr + 16 * RB));
#pragma unroll
      for (int n2 = 0; n2 < NCB; ++n2) o[n2][cb] = mfma16x16x32(va, pk[n2], o[n2][cb]);
    }
    lds_fence();  // this slot's reads are done before a later copy rewrites it
    if (NST == 1 && n + 1 < nsteps) issue(n + 1, 0);
  }

  // ---- per column block: per-wave state -> LDS, then a log-sum-exp merge
  // across the 4 waves; one partial per (b, g, split, column) ----
  float* red = (float*)smem;  // [wave][column 16][D + 2]: m, l, O[D]
  float* out = a.ws + (((int64_t)b * a.Hkv + g) * a.nsplit + s) * (int64_t)NC * (D + 2);
#pragma unroll
  for (int n = 0; n < NCB; ++n) {
    float l = lsum[n];
    l += __shfl_xor(l, 16, 64);
    l += __shfl_xor(l, 32, 64);
    __syncthreads();  // all waves are done with their V^T slices / the previous block's reads
    {
      float* mine = red + (wave * 16 + c16) * (D + 2);
      if (kg == 0) {
        mine[0] = mref[n];
        mine[1] = l;
      }
#pragma unroll
      for (int cb = 0; cb < CB; ++cb)
#pragma unroll
        for (int r = 0; r < 4; ++r) mine[2 + 16 * cb + 4 * kg + r] = o[n][cb][r];
    }
    __syncthreads();
    const int col0 = (cg * NCB + n) * 16;
    const int ncols = min(16, NC - col0);
    for (int e = tid; e < ncols * (D + 2); e += W * 64) {
      const int hh = e / (D + 2), c = e % (D + 2);
      float M = -INFINITY;
#pragma unroll
      for (int w = 0; w < W; ++w) M = fmaxf(M, red[(w * 16 + hh) * (D + 2)]);
      float acc = 0.f;
#pragma unroll
      for (int w = 0; w < W; ++w) {
        const float mw = red[(w * 16 + hh) * (D + 2)];
        const float f = mw == -INFINITY ? 0.f : exp2f(mw - M);
        acc += (c == 0 ? 0.f : red[(w * 16 + hh) * (D + 2) + c]) * f;
      }
      out[(int64_t)(col0 + hh) * (D + 2) + c] = c == 0 ? M : acc;
    }
  }
}

template <int D>
__global__ void __launch_bounds__(D) decode_merge_kernel(const DecodeArgs a) {
  // workgroup -> (sequence b, query token qi, pair p)
  const int P = a.Hq / 2;
  const int p = blockIdx.x % P;
  const int qi = (blockIdx.x / P) % a.nq;
  const int b = blockIdx.x / (P * a.nq);
  const int c = threadIdx.x;
  const int G = a.G, NC = a.nq * G;
  float res[2];
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const int head = 2 * p + k;
    const int g = head / G, col = qi * G + head % G;
    const float* base = a.ws + ((int64_t)b * a.Hkv + g) * a.nsplit * (int64_t)NC * (D + 2) + (int64_t)col * (D + 2);
    const int64_t sstride = (int64_t)NC * (D + 2);
    // splits of this sequence that hold entries (paged: the others have no
    // workgroup and no partial)
    const int ns = a.block_table ? (min(max(a.seq_lens[b], 0), a.L) + a.chunk - 1) / a.chunk : a.nsplit;
    // (loops unrolled by 8: a batch's loads are in flight together instead of
    // one memory latency per split)
    float M = -INFINITY;
#pragma unroll 8
    for (int s = 0; s < ns; ++s) M = fmaxf(M, base[s * sstride]);
    if (M == -INFINITY) {  // no visible entry at all (e.g. a paged sequence of length 0): no contribution
      res[k] = 0.f;
      continue;
    }
    float l = 0.f, acc = 0.f;
#pragma unroll 8
    for (int s = 0; s < ns; ++s) {
      const float f = exp2f(base[s * sstride] - M);
      l += base[s * sstride + 1] * f;
      acc += base[s * sstride + 2 + c] * f;
    }
    // off-by-one softmax: one more logit 0, i.e. 2^(0 - M) against the merged max
    res[k] = acc / (l + (a.softmax1 ? exp2f(-M) : 0.f));
  }
  const float lg = ((const float*)a.lam.p)[b * a.lam.sb + (int64_t)qi * a.lam.st + p * a.lam.sh];
  const float val = res[0] - sigmoid_f32(lg) * res[1];
  uint16_t* dst = (uint16_t*)a.out.p + b * a.out.sb + (int64_t)qi * a.out.st + p * a.out.sh;
  const uint32_t w = pack_bf16x2(val, 0.f);
  dst[c] = (uint16_t)(w & 0xffffu);
}

template <int D, int NCB>
hipError_t launch(const DecodeArgs& a, hipStream_t st) {
  const void* args[] = {&a};
  const void* split = a.block_table ? (const void*)decode_split_kernel<D, true, NCB>
                                    : (const void*)decode_split_kernel<D, false, NCB>;
  hipError_t e = hipLaunchKernel(split, dim3(decode_split_grid(a.B * a.ncg, a.Hkv, a.nsplit)), dim3(kWaves * 64),
                                 (void**)args, 0, st);
  if (e != hipSuccess) return e;
  return hipLaunchKernel((const void*)decode_merge_kernel<D>, dim3(a.B * a.nq * (a.Hq / 2)), dim3(D), (void**)args,
                         0, st);
}

}  // namespace

DecodeSplit decode_split(int B, int L, int Hkv, int max_chunk, int max_splits) {
  // Aim for >= 2048 workgroups (8 per CU) and chunks of <= max_chunk tokens,
  // with at most max_splits splits; a chunk is a multiple of the 4 waves x 32
  // tokens one step consumes.
  const int step = kWaves * kBlk;
  const long units = (long)B * Hkv;
  long ns = (L + max_chunk - 1) / max_chunk;
  const long want = (2048 + units - 1) / units;
  if (ns < want) ns = want;
  const long maxns = (L + step - 1) / step;
  if (ns > maxns) ns = maxns;
  if (ns > max_splits) ns = max_splits;
  if (ns < 1) ns = 1;
  long chunk = (L + ns - 1) / ns;
  chunk = (chunk + step - 1) / step * step;
  DecodeSplit r;
  r.chunk = (int)chunk;
  r.nsplit = (int)((L + chunk - 1) / chunk);
  return r;
}

long long decode_split_grid(int B, int Hkv, int nsplit) {
  const long long units = (long long)B * nsplit;
  return (units + 7) / 8 * 8 * Hkv;
}

int decode_column_blocks(int nq, int G) { return nq * G <= 16 ? 1 : 2; }

int decode_column_groups(int nq, int G) {
  const int per = 16 * decode_column_blocks(nq, G);
  return (nq * G + per - 1) / per;
}

hipError_t launch_decode_bf16(int d, const DecodeArgs& a, hipStream_t s) {
  const int ncb = decode_column_blocks(a.nq, a.G);
  if (a.ncg != decode_column_groups(a.nq, a.G)) return hipErrorInvalidValue;
  if (d == 64) return ncb == 1 ? launch<64, 1>(a, s) : launch<64, 2>(a, s);
  if (d == 128) return ncb == 1 ? launch<128, 1>(a, s) : launch<128, 2>(a, s);
  return hipErrorInvalidValue;
}

}  // namespace da
