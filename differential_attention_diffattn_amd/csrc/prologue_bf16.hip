// prologue_bf16.hip -- the steps just upstream of the attention: the rotary
// embedding of a q or k tensor, and the V2 lambda projection (gfx950).
//
// Rotary embedding (rope.hpp: the rotate-half arrangement Wilsontomass's
// module in the nanoGPT issue "How best to implement a differential
// transformer?" applies to every q and k head): an HBM-bound pass, one thread
// per eight consecutive pairs (c .. c+7) <-> (c + d/2 .. c + d/2 + 7) with
// 16-byte loads and stores (two pairs and 4-byte accesses when d/2 is not a
// multiple of 8); in place or out of place.  The prefill and decode kernels rotate q
// themselves (prologue, registers); this pass is for k, whose tiles go from
// HBM straight to LDS and are read by several workgroups each.
//
// Lambda projection ("Differential Transformer V2" article: a projected
// lambda for each token and head): logits[b,t,p] = <x[b,t,:], w[p,:]>, w laid
// out like a linear layer's weight [P, dm].  A workgroup owns 32 tokens x 32
// pairs; its 8 waves split dm in eight and each runs v_mfma_f32_32x32x16_bf16
// over its part (A = 32 token rows of x, B = 32 rows of w, both 16-byte
// loads straight from HBM / L2); the eight partial tiles are added in a fixed
// order through LDS (deterministic).  It reads x once: HBM-bound.
#include <math.h>

#include <type_traits>

#include "kernels.hpp"
#include "rope.hpp"
#include "tile_ops.hpp"

namespace da {
namespace {

// VW consecutive pairs per thread: elements c .. c + VW - 1 and the same
// span of the second half (16-byte loads and stores when VW = 8).
template <int VW>
__global__ void __launch_bounds__(256) rope_kernel(const RopeArgs a) {
  using Vec = typename std::conditional<VW == 8, uint4, uint32_t>::type;
  const int half = a.d / 2;
  const int tpr = half / VW;  // threads per row
  const long long gid = (long long)blockIdx.x * 256 + threadIdx.x;
  const long long row = gid / tpr;
  if (row >= (long long)a.B * a.T * a.H) return;
  const int c = VW * (int)(gid % tpr);
  const int h = (int)(row % a.H);
  const int t = (int)((row / a.H) % a.T);
  const int b = (int)(row / ((long long)a.H * a.T));
  const uint16_t* xr = (const uint16_t*)a.x.p + b * a.x.sb + (int64_t)t * a.x.st + (int64_t)h * a.x.sh;
  uint16_t* orow = (uint16_t*)a.out.p + b * a.out.sb + (int64_t)t * a.out.st + (int64_t)h * a.out.sh;
  const Vec lo = *(const Vec*)(xr + c), hi = *(const Vec*)(xr + c + half);
  const uint32_t* lw = (const uint32_t*)&lo;
  const uint32_t* hw = (const uint32_t*)&hi;
  uint32_t y1w[VW / 2], y2w[VW / 2];
#pragma unroll
  for (int j = 0; j < VW; j += 2) {
    float y1[2], y2[2];
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const float x1 = bf16_to_f32((uint16_t)(e ? lw[j / 2] >> 16 : lw[j / 2] & 0xffffu));
      const float x2 = bf16_to_f32((uint16_t)(e ? hw[j / 2] >> 16 : hw[j / 2] & 0xffffu));
      float sn, cs;
      rope_sincos(a.pos0 + t, a.w.hi[c + j + e], a.w.lo[c + j + e], &sn, &cs);
      y1[e] = x1 * cs - x2 * sn;
      y2[e] = x2 * cs + x1 * sn;
    }
    y1w[j / 2] = pack_bf16x2(y1[0], y1[1]);
    y2w[j / 2] = pack_bf16x2(y2[0], y2[1]);
  }
  *(Vec*)(orow + c) = *(const Vec*)y1w;
  *(Vec*)(orow + c + half) = *(const Vec*)y2w;
}

constexpr int kProjWaves = 8;

__global__ void __launch_bounds__(kProjWaves * 64) lambda_proj_kernel(const LamProjArgs a) {
  __shared__ f32x16 part[kProjWaves - 1][64];
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int li = lane & 31, hg = lane >> 5;
  const int ptiles = (a.P + 31) / 32;
  const long long r0 = (long long)(blockIdx.x / ptiles) * 32;  // first token (flattened b * T + t)
  const int p0 = (blockIdx.x % ptiles) * 32;
  const long long ntok = (long long)a.B * a.T;
  // this lane's A row (token) and B row (pair), clamped into range (masked at the store)
  const long long r = min(r0 + li, ntok - 1);
  const int rb = (int)(r / a.T), rt = (int)(r % a.T);
  const uint16_t* xr = (const uint16_t*)a.x.p + rb * a.x.sb + (int64_t)rt * a.x.st;
  const uint16_t* wr = (const uint16_t*)a.w.p + (int64_t)min(p0 + li, a.P - 1) * a.w.sh;
  const int kq = a.dm / kProjWaves;  // this wave's part of dm (a multiple of 16)
  const int k0 = wave * kq;
  f32x16 acc;
#pragma unroll
  for (int i = 0; i < 16; ++i) acc[i] = 0.f;
  int k = k0;
  for (; k + 128 <= k0 + kq; k += 128) {  // eight k-steps per round: sixteen 16-byte loads in flight
    bf16x8 xa[8], wb[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      xa[j] = as_bf16x8(*(const uint4*)(xr + k + 16 * j + 8 * hg));
      wb[j] = as_bf16x8(*(const uint4*)(wr + k + 16 * j + 8 * hg));
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) acc = mfma32x32x16(xa[j], wb[j], acc);
  }
  for (; k < k0 + kq; k += 16)
    acc = mfma32x32x16(as_bf16x8(*(const uint4*)(xr + k + 8 * hg)), as_bf16x8(*(const uint4*)(wr + k + 8 * hg)),
                       acc);
  if (wave > 0) part[wave - 1][lane] = acc;
  __syncthreads();
  if (wave != 0) return;
#pragma unroll
  for (int w = 0; w < kProjWaves - 1; ++w) {
    const f32x16 x = part[w][lane];
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[i] += x[i];
  }
  // register i: token r0 + 8(i>>2) + 4hg + (i&3), pair p0 + li
  const int p = p0 + li;
  if (p >= a.P) return;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const long long tok = r0 + 8 * (i >> 2) + 4 * hg + (i & 3);
    if (tok < ntok) {
      const int ob = (int)(tok / a.T), ot = (int)(tok % a.T);
      ((float*)a.out.p)[ob * a.out.sb + (int64_t)ot * a.out.st + (int64_t)p * a.out.sh] = acc[i];
    }
  }
}

// Streaming form for dm a multiple of 256: a workgroup (4 waves) owns 32
// tokens x 32 pairs and walks dm in 256-wide chunks.  Each chunk's x rows
// (32 x 512 B) and w rows (32 x 512 B) go HBM -> LDS by global_load_lds, two
// whole rows per 1 KB instruction (fully coalesced), into a 3-stage ring with
// two chunks in flight (three or four in flight measured 1-3% slower); 16-byte
// chunk c of a row lands at chunk c ^ (row & 15), so the MFMA operand reads
// (ds_read_b128, 16 rows per pass) hit distinct banks.  Wave w runs k-steps
// 4w .. 4w+3 of each chunk; the four partial tiles are added in a fixed order
// at the end.  Workgroups walk the chunks in rotated order (workgroup k of
// an XCD starts at chunk k mod n): when every workgroup read the same columns
// at the same time, the rows' 8 KB stride kept the reads on a few memory
// channels and the kernel ran at two thirds of the rate it reaches rotated.
#ifndef DA_PS_STAGES
#define DA_PS_STAGES 3  // ring depth of the streaming projection (stages - 1 chunks in flight)
#endif
#ifndef DA_PS_NT
#define DA_PS_NT 0  // x copies with the non-temporal policy
#endif
#ifndef DA_PS_CHUNK
#define DA_PS_CHUNK 256  // dm per chunk of the streaming projection (256 or 512)
#endif
constexpr int kPsWaves = 4, kPsChunk = DA_PS_CHUNK, kPsStages = DA_PS_STAGES;  // dm per chunk
constexpr int kPsRowBytes = kPsChunk * 2;    // 512 B or 1 KB
constexpr int kPsRPI = 1024 / kPsRowBytes;   // rows per 1 KB copy (2 or 1)
constexpr int kPsTile = 32 * kPsRowBytes;    // one operand tile of a chunk
constexpr int kPsStage = 2 * kPsTile;        // x tile, w tile
constexpr int kPsNIW = 32 / kPsRPI / kPsWaves;  // 1 KB copies per wave per tensor and chunk
constexpr int kPsCopies = 2 * kPsNIW;        // per wave and chunk
constexpr int kPsKW = kPsChunk / 16 / kPsWaves;  // k-steps per wave and chunk
static_assert(kPsChunk == 256 || kPsChunk == 512, "projection chunk");
static_assert(kPsStages >= 2 && kPsStages <= 5 && kPsStages * kPsStage <= 160 * 1024, "projection ring");

__global__ void __launch_bounds__(kPsWaves * 64) lambda_proj_stream_kernel(const LamProjArgs a) {
  __shared__ __attribute__((aligned(1024))) unsigned char smem[kPsStages * kPsStage];
  const uint32_t lds0 = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) unsigned char*)smem;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int li = lane & 31, hg = lane >> 5;
  const int ptiles = (a.P + 31) / 32;
  const long long r0 = (long long)(blockIdx.x / ptiles) * 32;  // first token (flattened b * T + t)
  const int p0 = (blockIdx.x % ptiles) * 32;
  const long long ntok = (long long)a.B * a.T;
  const int nch = a.dm / kPsChunk;
  const int rot = (int)((blockIdx.x / 8) % (unsigned)nch);  // workgroups of one XCD: consecutive k
  // Copy i of wave w moves rows 2(4w + i) and 2(4w + i) + 1 (lanes 0-31 and
  // 32-63) of the x tile and of the w tile (rows past the end clamped to the
  // last token / pair: finite, masked at the store).  The two rows' bases
  // differ per lane half: a copy takes the lower one as its scalar base and
  // adds each half's distance to the lane offset (the launcher uses this
  // kernel only when every distance between rows fits in 31 bits).  Bases and
  // distances do not depend on the chunk, so they are formed once.
  // (With 1 KB rows, copy i of wave w moves row NIW w + i whole.)
  const char* xb[kPsNIW];
  const char* wb[kPsNIW];
  uint32_t xd[kPsNIW], wd[kPsNIW];
#pragma unroll
  for (int i = 0; i < kPsNIW; ++i) {
    const int rp = kPsRPI * (kPsNIW * wave + i);  // first row of the copy (uniform)
    const int r1 = kPsRPI == 2 ? rp + 1 : rp;
    const long long t0 = min(r0 + rp, ntok - 1), t1 = min(r0 + r1, ntok - 1);
    const char* x0 = (const char*)((const uint16_t*)a.x.p + (t0 / a.T) * a.x.sb + (int64_t)(t0 % a.T) * a.x.st);
    const char* x1 = (const char*)((const uint16_t*)a.x.p + (t1 / a.T) * a.x.sb + (int64_t)(t1 % a.T) * a.x.st);
    xb[i] = x0 < x1 ? x0 : x1;
    xd[i] = (uint32_t)((hg ? x1 : x0) - xb[i]);
    wb[i] = (const char*)((const uint16_t*)a.w.p + (int64_t)min(p0 + rp, a.P - 1) * a.w.sh);
    const char* w1 = (const char*)((const uint16_t*)a.w.p + (int64_t)min(p0 + r1, a.P - 1) * a.w.sh);
    wd[i] = (uint32_t)((hg ? w1 : wb[i]) - wb[i]);
  }
  auto issue = [&](int ch, int stage) {
    const uint32_t st = lds0 + stage * kPsStage;
#pragma unroll
    for (int i = 0; i < kPsNIW; ++i) {
      const int rp = kPsRPI * (kPsNIW * wave + i);
      const int chr = ch + rot < nch ? ch + rot : ch + rot - nch;  // chunk of the rotated order
      // lane's destination chunk of its row: li (two rows per copy) or lane (one)
      const int dchunk = kPsRPI == 2 ? li : lane, drow = kPsRPI == 2 ? rp + hg : rp;
      const uint32_t off = (uint32_t)chr * kPsRowBytes + (uint32_t)((dchunk ^ (drow & 15)) << 4);
      if (DA_PS_NT)
        dma16_sbase_nt(xb[i], off + xd[i], st + rp * kPsRowBytes);
      else
        dma16_sbase(xb[i], off + xd[i], st + rp * kPsRowBytes);
      dma16_sbase(wb[i], off + wd[i], st + kPsTile + rp * kPsRowBytes);
    }
  };
  for (int c = 0; c < kPsStages - 1 && c < nch; ++c) issue(c, c);
  f32x16 acc;
#pragma unroll
  for (int i = 0; i < 16; ++i) acc[i] = 0.f;
  const uint32_t rrow = li * kPsRowBytes;
  for (int ch = 0; ch < nch; ++ch) {
    const int stage = ch % kPsStages;
    // this wave's copies of chunk ch landed (later chunks may stay in flight)
    const int later = min(kPsStages - 2, nch - 1 - ch);
    if (later >= 3)
      asm volatile("s_waitcnt vmcnt(%0)" ::"n"(3 * kPsCopies) : "memory");
    else if (later == 2)
      asm volatile("s_waitcnt vmcnt(%0)" ::"n"(2 * kPsCopies) : "memory");
    else if (later == 1)
      asm volatile("s_waitcnt vmcnt(%0)" ::"n"(kPsCopies) : "memory");
    else
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();  // every wave's copies of chunk ch landed; stage (ch - 1) % 4 is free
    if (ch + kPsStages - 1 < nch) issue(ch + kPsStages - 1, (ch + kPsStages - 1) % kPsStages);
    const uint32_t st = lds0 + stage * kPsStage;
#pragma unroll
    for (int j = 0; j < kPsKW; ++j) {
      const int q = 2 * (kPsKW * wave + j) + hg;  // 16-byte chunk of the row this lane's half reads
      const uint32_t o = rrow + (uint32_t)((q ^ (li & 15)) << 4);
      acc = mfma32x32x16(lds_read16(st + o), lds_read16(st + kPsTile + o), acc);
    }
  }
  // fixed-order reduction of the four partial tiles through LDS
  __syncthreads();  // every wave is done with the stages
  f32x16* part = (f32x16*)smem;
  if (wave > 0) part[(wave - 1) * 64 + lane] = acc;
  __syncthreads();
  if (wave != 0) return;
#pragma unroll
  for (int w = 0; w < kPsWaves - 1; ++w) {
    const f32x16 x = part[w * 64 + lane];
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[i] += x[i];
  }
  // register i: token r0 + 8(i>>2) + 4hg + (i&3), pair p0 + li
  const int p = p0 + li;
  if (p >= a.P) return;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const long long tok = r0 + 8 * (i >> 2) + 4 * hg + (i & 3);
    if (tok < ntok) {
      const int ob = (int)(tok / a.T), ot = (int)(tok % a.T);
      ((float*)a.out.p)[ob * a.out.sb + (int64_t)ot * a.out.st + (int64_t)p * a.out.sh] = acc[i];
    }
  }
}

}  // namespace

hipError_t launch_rope_bf16(const RopeArgs& a, hipStream_t s) {
  const void* args[] = {&a};
  const int vw = a.d % 16 == 0 ? 8 : 2;  // pairs per thread (d % 8 == 0 always)
  const long long threads = (long long)a.B * a.T * a.H * (a.d / 2 / vw);
  return hipLaunchKernel(vw == 8 ? (const void*)rope_kernel<8> : (const void*)rope_kernel<2>,
                         dim3((unsigned)((threads + 255) / 256)), dim3(256), (void**)args, 0, s);
}

hipError_t launch_lambda_proj_bf16(const LamProjArgs& a, hipStream_t s) {
  const void* args[] = {&a};
  const long long tiles = ((long long)a.B * a.T + 31) / 32 * ((a.P + 31) / 32);
  // the streaming kernel addresses rows of x and of w by 32-bit byte
  // distances from a per-copy base
  const long long xspan = ((long long)(a.B - 1) * a.x.sb + (long long)(a.T - 1) * a.x.st + a.dm) * 2;
  const long long wspan = ((long long)(a.P - 1) * a.w.sh + a.dm) * 2;
  if (a.dm % kPsChunk == 0 && xspan < (1LL << 31) && wspan < (1LL << 31))
    return hipLaunchKernel((const void*)lambda_proj_stream_kernel, dim3((unsigned)tiles), dim3(kPsWaves * 64),
                           (void**)args, 0, s);
  return hipLaunchKernel((const void*)lambda_proj_kernel, dim3((unsigned)tiles), dim3(kProjWaves * 64),
                         (void**)args, 0, s);
}

}  // namespace da
