// kernels.hpp -- internal interface between the C-ABI front end (api.cpp) and
// the kernel translation units.  Every function here enqueues work on
// `stream` and returns the hipError_t of the launch; arguments have already
// been validated by the front end.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "common.hpp"

namespace da {

// Rotary-embedding frequencies w_c = theta^(-2c/d), c < d/2 (d <= 256), each
// as an unevaluated sum hi + lo of two floats (computed on the host in
// double), so a position times w_c keeps ~48 bits.
struct RopeTab {
  float hi[128], lo[128];
};

// Two causal softmax maps per wave over one shared V (V1), or one GQA
// attention whose adjacent query heads are paired (V2).
struct PrefillArgs {
  TIn q1, q2, k1, k2, v;  // V2: q1 == q2 == q (heads selected by pair), k1 == k2 == k
  TIn lam;                // V2: fp32 logits [B,T,Hq/2] (roles b, pair, t)
  TOut out;
  const float* lq1;  // V1 lambda vectors (device, [d])
  const float* lk1;
  const float* lq2;
  const float* lk2;
  float lam_init;  // V1: 0.8 - 0.6 exp(-0.3 layer)
  float sl2;       // log2(e) / sqrt(d)
  int B, T;
  int H;           // V1: differential heads; V2: kv heads
  int G;           // V2: query heads per kv head (even)
  int pc;          // V2: pairs per workgroup (1, 2 or 4)
  int units_per_b; // work units per batch entry
  int tiles;       // token tiles per unit
  int nwg;         // workgroups in the grid
  int softmax1;    // 1: off-by-one softmax (each map's denominator + exp(0))
  // Training forward (lse non-null): the log2 of each row's softmax
  // denominator of the log2(e)/sqrt(d)-scaled scores and the normalised
  // attention outputs.  V2: each head's output attn [B,T,Hq,d] (roles b,
  // head, t), lse [B][Hq][T].  V1: map 1's output in attn and map 2's in
  // attn2, both [B,T,H,2d] (roles b, differential head, t), lse [2][B][H][T].
  TOut attn, attn2;
  float* lse;
  // rotary embedding of q in the prologue (rope != 0): row t of q turns by
  // t * w_c
  int rope;
  RopeTab rope_w;
  // V1 with rope: the keys before rotation (k1, k2 then hold them rotated
  // and rounded to bf16); the cancellation guard's exact rows rotate these
  // in fp32.  Without rope the same as k1, k2.
  TIn k1o, k2o;
};

hipError_t launch_prefill_v1_bf16(int d, const PrefillArgs& a, hipStream_t s);
hipError_t launch_prefill_v2_bf16(int d, const PrefillArgs& a, hipStream_t s);

// Plain fp32 V1 forward (VALU, LDS tiled).
struct V1F32Args {
  TIn q1, q2, k1, k2, v;
  TOut out;
  const float* lq1;
  const float* lk1;
  const float* lq2;
  const float* lk2;
  float lam_init;
  float sl2;
  int B, H, T;
  int tiles;
  int softmax1;  // 1: off-by-one softmax (each map's denominator + exp(0))
};
hipError_t launch_v1_fp32(int d, const V1F32Args& a, hipStream_t s);

// DIFF V2 backward: pre-pass, dQ kernel, dK/dV kernel.
struct BwdArgs {
  TIn q, k, v;     // [B,T,Hq,d] / [B,T,Hkv,d] bf16
  TIn lam;         // [B,T,Hq/2] fp32 logits (roles b, pair, t)
  TIn attn;        // [B,T,Hq,d] bf16 per-head forward outputs
  TIn dout;        // [B,T,Hq/2,d] bf16
  const float* lse;  // [B][Hq][T] log2 softmax denominators (training forward)
  TOut dq, dk, dv;   // bf16, layouts of q / k / v
  TOut dlam;         // [B,T,Hq/2] fp32
  float* Dw;         // workspace [B][Hq][Tp]: E_h = rowsum(dout * attn_h)
  float* lsew;       // workspace [B][Hq][Tp]: lse (odd heads: lse - log2 sigmoid(lam)), padded with zeros
  float sl2;         // log2(e) / sqrt(d)
  float scale;       // 1 / sqrt(d)
  int B, T, Hq, Hkv, G, Tp;
};
int backward_padded_rows(int T);
hipError_t launch_backward_v2_bf16(int d, const BwdArgs& a, hipStream_t s);

// DIFF V1 backward (map m = 0, 1 for the pages' maps 1, 2; dv = 2d).
struct V1BwdArgs {
  TIn q[2], k[2], v;  // [B,H,T,d] / v [B,H,T,2d] bf16 (roles b, differential head, t)
  TIn a[2];           // training forward's map outputs [B,T,H,2d] bf16
  TIn dout;           // [B,T,H,2d] bf16
  const float* lse;   // [2][B][H][T] (training forward)
  const float *lq1, *lk1, *lq2, *lk2;  // lambda vectors [d]
  TOut dq[2], dk[2], dv;               // bf16, layouts of q / k / v
  float *dlq1, *dlk1, *dlq2, *dlk2;    // [d] fp32
  uint16_t* dD;       // workspace [B][T][H][2d] bf16: dD (d a_1 = dD, d a_2 = -lam dD)
  float* Dw[2];       // workspace [B][H][Tp]: E_m = rowsum(dD * a_m)
  float* lsew[2];     // workspace [B][H][Tp]: lse of map m, padded with zeros
  float* lamrow;      // workspace [B][T][H]: each row's term of d lambda
  float lam_init, sl2, scale;
  int B, T, H, Tp;
};
hipError_t launch_backward_v1_bf16(int d, const V1BwdArgs& a, hipStream_t s);

// Split-K decode over a KV cache, then a deterministic merge.
struct DecodeArgs {
  TIn q, k, v, lam;
  TOut out;
  float* ws;  // [B][Hkv][nsplit][G][d + 2] fp32 partials (m, l, O)
  float sl2;
  int B, L, Hq, Hkv, G;
  int chunk;   // tokens per split (multiple of 128)
  int nsplit;
  int nq;      // query tokens per sequence (the last nq cache entries; q/lam/out token stride st)
  int ncg;     // column groups: (query token, head) columns are scored 16 or 32 per workgroup
  int softmax1;  // 1: off-by-one softmax (each head's denominator + exp(0))
  // Paged cache (null block_table: the dense [B, L, Hkv, d] cache of k / v):
  // token t of sequence b is row (t & page_mask) of page
  // block_table[b * bt_stride + (t >> page_shift)] (clamped to [0, num_pages)),
  // with k.sb / v.sb the stride between pages; the sequence has seq_lens[b]
  // tokens (clamped to [0, L]; L is the longest).
  const int32_t* block_table;
  int64_t bt_stride;
  const int32_t* seq_lens;
  int page_shift, page_mask, num_pages;
  // rotary embedding of q (rope != 0): new token i sits at cache position
  // L_b - nq + i; the cache holds its keys rotated
  int rope;
  RopeTab rope_w;
};
hipError_t launch_decode_bf16(int d, const DecodeArgs& a, hipStream_t s);

// Rotary embedding of a [B,T,H,d] bf16 tensor (rows at positions pos0 + t),
// out-of-place or in place; and the V2 lambda projection
// logits[b,t,p] = <x[b,t,:], w[p,:]> (x [B,T,dm] bf16, w [P,dm] bf16, fp32 out).
struct RopeArgs {
  TIn x;
  TOut out;
  int B, T, H, d, pos0;
  RopeTab w;
};
hipError_t launch_rope_bf16(const RopeArgs& a, hipStream_t s);
struct LamProjArgs {
  TIn x;       // roles b, -, t
  TIn w;       // roles -, p (sh), -
  TOut out;    // fp32, roles b, p, t
  int B, T, dm, P;
};
hipError_t launch_lambda_proj_bf16(const LamProjArgs& a, hipStream_t s);
// workgroups of the decode split kernel (B * nsplit units padded to a multiple of 8, times Hkv)
long long decode_split_grid(int B, int Hkv, int nsplit);
// 16-wide column blocks per workgroup (1 or 2) and column groups for nq query tokens x G heads
int decode_column_blocks(int nq, int G);
int decode_column_groups(int nq, int G);

// Decode split geometry, shared by the workspace query and the launcher.
struct DecodeSplit {
  int chunk, nsplit;
};
DecodeSplit decode_split(int B, int L, int Hkv, int max_chunk = 2048, int max_splits = 0x7fffffff);
#ifndef DA_PAGED_CHUNK
#define DA_PAGED_CHUNK 4096
#endif
constexpr int kPagedMaxChunk = DA_PAGED_CHUNK;  // paged decode: tokens per split at most
#ifndef DA_DENSE_CHUNK
#define DA_DENSE_CHUNK 4096
#endif
constexpr int kDenseMaxChunk = DA_DENSE_CHUNK;  // dense decode: tokens per split at most

}  // namespace da
