/*
 * diffattn_oracle.h -- plain, slow, fp64 CPU reference for differential attention.
 *
 * TEST INFRASTRUCTURE ONLY.  Only tests/, __graft_entry__.smoke() and the
 * cpu_baseline leg of bench.py may load or call this library.  It shares no
 * code, header, table or helper with the HIP library under
 * differential_attention_diffattn_amd/csrc/, and the product path never
 * routes through it.
 *
 * Every array is host memory, fp64, densely packed in the layout stated at
 * each function ("[B][H][T][d]" means the last index is fastest).  Inputs are
 * the exact values given to the GPU (bf16 / fp32 widened to double), so a
 * comparison measures the kernel's error only.
 *
 * Sources (the pages):
 *   [V2A]  "Differential Transformer V2" article: the DiffAttnV1 and
 *          DiffAttnV2 pseudo-code, the GQA-layout note above them, and the
 *          paragraph on decoding below them.
 *   [NGI]  nanoGPT issue "How best to implement a differential
 *          transformer?": Wilsontomass's module (lambda vectors drawn
 *          N(0, 0.1), subln = RMSNorm(2*head_dim, eps=1e-5, no affine),
 *          output scale 1 - lambda_init, causal SDPA with default scale) and
 *          notlober's module (explicit masked score maps, adjacent heads
 *          paired, one V of width 2*head_dim per differential head).
 *   [HN]   Hacker News item 41780844 comments: the lambda_init expression
 *          0.8 - 0.6*exp(-0.3*depth), and a comment proposing a softmax
 *          whose denominator gains an extra 1 (the "off-by-one" softmax,
 *          the same as one extra logit 0).
 *
 * softmax1 (every attention function): 0 = the standard softmax; 1 = the
 * off-by-one softmax, each map's denominator gaining exp(0) -- equivalently
 * one more key at logit 0 whose value row is 0.
 */
#ifndef DIFFATTN_ORACLE_H
#define DIFFATTN_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* lambda_init(layer) = 0.8 - 0.6*exp(-0.3*layer), layer counted from 0.
 * [V2A] DiffAttnV1 (lam_init line); [HN] quoted constant. */
double da_oracle_lambda_init(int layer);

/* V1 lambda = exp(sum_c lq1[c]*lk1[c]) - exp(sum_c lq2[c]*lk2[c]) + lambda_init.
 * One scalar per layer, shared by every head.  [V2A] DiffAttnV1 (lam1, lam2,
 * lam lines); [NGI] Wilsontomass's lambda_1/lambda_2/lambda_full. */
double da_oracle_v1_lambda(int d, const double* lq1, const double* lk1,
                           const double* lq2, const double* lk2, int layer);

/* DIFF V1 forward, every row.
 *   q1, q2, k1, k2 : [B][H][T][d]      (H = differential heads)
 *   v              : [B][H][T][2d]     (one V shared by both maps)
 *   lq1..lk2       : [d]
 *   out            : [B][T][H][2d]
 * out[b,i,h,:] = (1-li) * RMSNorm_{2d, eps 1e-5}( A1 v - lambda * A2 v )[i]
 * with A_m the causal softmax of q_m k_m^T / sqrt(d).  [V2A] DiffAttnV1;
 * [NGI] both modules. */
void da_oracle_v1_fwd(int B, int H, int T, int d,
                      const double* q1, const double* q2,
                      const double* k1, const double* k2, const double* v,
                      const double* lq1, const double* lk1,
                      const double* lq2, const double* lk2,
                      int layer, int softmax1, double* out);

/* DIFF V1 forward for selected rows only: row r is (b, h, i) =
 * (bhi[3r], bhi[3r+1], bhi[3r+2]); out_rows is [n][2d].  Same layouts as
 * da_oracle_v1_fwd.  Lets a test check sampled outputs at full size. */
void da_oracle_v1_rows(int B, int H, int T, int d,
                       const double* q1, const double* q2,
                       const double* k1, const double* k2, const double* v,
                       const double* lq1, const double* lk1,
                       const double* lq2, const double* lk2,
                       int layer, int softmax1, int64_t n, const int64_t* bhi,
                       double* out_rows);

/* DIFF V2 prefill, every row.
 *   q   : [B][T][Hq][d]   (heads of one GQA group are contiguous)
 *   k, v: [B][T][Hkv][d]
 *   lam : [B][T][Hq/2]    (logits; sigmoid applied here)
 *   out : [B][T][Hq/2][d]
 * a_h = causal softmax(q_h k_g^T / sqrt(d)) v_g with g = h / (Hq/Hkv);
 * out[b,t,p,:] = a_{2p} - sigmoid(lam[b,t,p]) * a_{2p+1}.
 * [V2A] DiffAttnV2 and the GQA-layout note. */
void da_oracle_v2_fwd(int B, int T, int Hq, int Hkv, int d,
                      const double* q, const double* k, const double* v,
                      const double* lam, int softmax1, double* out);

/* DIFF V2 prefill for selected rows: row r is (b, t, p) = btp[3r..3r+2];
 * out_rows is [n][d]. */
void da_oracle_v2_rows(int B, int T, int Hq, int Hkv, int d,
                       const double* q, const double* k, const double* v,
                       const double* lam, int softmax1, int64_t n, const int64_t* btp,
                       double* out_rows);

/* DIFF V2 decode: one new query token per sequence against a cache that
 * already holds it at position L-1; the query sees all L entries.
 *   q   : [B][Hq][d]
 *   k, v: [B][L][Hkv][d]
 *   lam : [B][Hq/2]
 *   out : [B][Hq/2][d]
 * [V2A] DiffAttnV2 applied to the last position (the decoding paragraph). */
void da_oracle_v2_decode(int B, int L, int Hq, int Hkv, int d,
                         const double* q, const double* k, const double* v,
                         const double* lam, int softmax1, double* out);

/* Every query head's own causal attention rows, before the pairs combine,
 * and each row's log-sum-exp (what a training forward keeps):
 *   q   : [B][T][Hq][d];  k, v: [B][T][Hkv][d]
 *   attn: [B][T][Hq][d];  lse : [B][Hq][T] (natural log of the row's
 *         softmax denominator, the off-by-one term included when softmax1)
 * [V2A] DiffAttnV2: the attention call over all Hq heads. */
void da_oracle_v2_heads(int B, int T, int Hq, int Hkv, int d, const double* q,
                        const double* k, const double* v, int softmax1,
                        double* attn, double* lse);

/* Threads the library's OpenMP loops may use (0 = OpenMP default).  Returns
 * the count that will be used. */
int da_oracle_set_threads(int n);

#ifdef __cplusplus
}
#endif
#endif /* DIFFATTN_ORACLE_H */
