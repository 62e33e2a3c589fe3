/*
 * diffattn.h -- C ABI of libdiffattn.so: differential-attention forward on
 * AMD Instinct MI355X (gfx950).
 *
 * What is computed (the pages this follows):
 *   "Differential Transformer V2" article -- the DiffAttnV1 and DiffAttnV2
 *     pseudo-code, the note that heads of one GQA group are contiguous and
 *     that the two heads subtracted share key and value, and the paragraph
 *     on memory-bound decoding.
 *   nanoGPT issue "How best to implement a differential transformer?" --
 *     Wilsontomass's module: causal attention with the default 1/sqrt(d)
 *     scale, one V of width 2*head_dim shared by both maps, the lambda
 *     vectors, subln = RMSNorm(2*head_dim, eps 1e-5, no affine) and the
 *     (1 - lambda_init) output scale.
 *   Hacker News item 41780844 -- lambda_init = 0.8 - 0.6*exp(-0.3*depth).
 *
 * Conventions shared by every entry point
 *   Memory    Every tensor pointer is DEVICE memory, allocated and owned by
 *             the caller; the library allocates nothing, keeps no state
 *             between calls and never frees caller memory.  The one
 *             exception is diffattn_v2_decode_noalloc, whose scratch is a
 *             static device array of the library (see there).
 *   Layout    A tensor is described by da_in / da_out: a base pointer and
 *             element strides for its batch, head and token axes (the
 *             "role" strides).  The head_dim axis is always unit-stride.
 *             Any permutation of those axes (e.g. [B,T,H,d] or [B,H,T,d])
 *             is accepted without a copy.  Base pointers must be 16-byte
 *             aligned and every role stride a multiple of 8 elements (bf16)
 *             or 4 elements (fp32), so rows can be moved with 128-bit loads.
 *             Lambda tensors (fp32, no head_dim axis) only need 4-byte
 *             alignment and have no stride-multiple rule.  For the bf16
 *             prefill entry points, and for the dense decode caches, the key/value
 *             token strides must be below 2^24 elements (DA_E_UNSUPPORTED
 *             otherwise).
 *   Stream    Work is enqueued on `stream` (a hipStream_t; NULL = the
 *             default stream) and the call returns without synchronising.
 *   Errors    Status codes only; nothing is thrown, nothing aborts.  All
 *             arguments are validated on the host before anything is
 *             enqueued: on any error other than DA_E_LAUNCH nothing has been
 *             enqueued and `out` is untouched.  DA_E_LAUNCH reports a launch
 *             failure from the HIP runtime.  Faults during execution surface
 *             at the caller's next synchronisation, as for any HIP kernel.
 *   Threads   Entry points are reentrant and may be called concurrently
 *             from several host threads (on different or the same stream).
 *   Numerics  bf16 inputs, fp32 accumulation and softmax, fp32 lambda,
 *             combine and norm; one round-to-nearest-even store to the
 *             output dtype.  Results are bitwise reproducible run to run.
 */
#ifndef DIFFATTN_H
#define DIFFATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    DA_OK = 0,
    DA_E_NULL = 1,        /* a required pointer is NULL                         */
    DA_E_DTYPE = 2,       /* unknown dtype value                                */
    DA_E_SHAPE = 3,       /* a size is < 1, or sizes are inconsistent           */
    DA_E_LAYOUT = 4,      /* misaligned pointer or a stride breaks the rules    */
    DA_E_UNSUPPORTED = 5, /* valid arguments the library has no kernel for     */
    DA_E_WORKSPACE = 6,   /* decode workspace missing or too small              */
    DA_E_LAUNCH = 7,      /* the HIP runtime rejected a kernel launch           */
    DA_E_SCRATCH = 8      /* diffattn_v2_decode_noalloc: sizes need more than   */
                          /* the library's static scratch                       */
} da_status;

/* Element types.  Entry points take the dtype as a plain int holding one of
 * these values, so any other value a caller passes is reported as
 * DA_E_DTYPE (an out-of-range enum argument would be undefined in C++). */
typedef enum { DA_FP32 = 0, DA_BF16 = 1 } da_dtype;

/* Read-only device tensor: base pointer + element strides by role. */
typedef struct {
    const void* ptr;
    int64_t sb; /* stride between batch entries   */
    int64_t sh; /* stride between heads (or pairs) */
    int64_t st; /* stride between tokens           */
} da_in;

/* Writable device tensor: same meaning as da_in. */
typedef struct {
    void* ptr;
    int64_t sb;
    int64_t sh;
    int64_t st;
} da_out;

/*
 * DIFF V1 forward ("Differential Transformer V2" article, DiffAttnV1;
 * nanoGPT issue, Wilsontomass's module).  For every batch b, differential
 * head h and token i:
 *   A_m     = causal softmax_j( q_m[b,h,i] . k_m[b,h,j] / sqrt(d) ),  j <= i
 *   lam     = exp(sum_c lam_q1[c]*lam_k1[c]) - exp(sum_c lam_q2[c]*lam_k2[c])
 *             + lambda_init,  lambda_init = 0.8 - 0.6*exp(-0.3*layer_index)
 *   D       = (A_1 - lam*A_2) V[b,h]                (width 2d)
 *   out[b,i,h,:] = D / sqrt(mean_c D^2 + 1e-5) * (1 - lambda_init)
 *
 *   dtype        DA_BF16 (d in {64, 128}) or DA_FP32 (d in {32, 64, 128}).
 *   B, H, T, d   batch, differential heads, tokens, q/k head_dim; >= 1.
 *   q1,q2,k1,k2  logical [B,H,T,d] of `dtype` (roles b, h, t).
 *   v            logical [B,H,T,2d] of `dtype`; one V shared by both maps.
 *   lam_q1..lam_k2  device fp32 vectors of length d, contiguous.
 *   layer_index  0-based depth of the layer (any int >= 0).
 *   out          logical [B,T,H,2d] of `dtype` (roles b, h, t).
 * lam is one scalar per call shared by every head, computed on the device
 * in fp32; it may take any real value (no clamp).
 */
da_status diffattn_v1_fwd(int dtype, int B, int H, int T, int d,
                          da_in q1, da_in q2, da_in k1, da_in k2, da_in v,
                          const float* lam_q1, const float* lam_k1,
                          const float* lam_q2, const float* lam_k2,
                          int layer_index, da_out out, void* stream);

/*
 * DIFF V2 prefill ("Differential Transformer V2" article, DiffAttnV2 and
 * the GQA-layout note).  Query heads of one GQA group are contiguous, so
 * query head h reads kv head g = h / (Hq/Hkv); the two heads of a pair
 * (2p, 2p+1) always fall in one group.  For every b, token t, pair p:
 *   a_h = causal softmax_j( q[b,t,h] . k[b,j,g] / sqrt(d) ) v[b,:,g],  j <= t
 *   out[b,t,p,:] = a_{2p} - sigmoid(lam[b,t,p]) * a_{2p+1}
 * No norm, no scale.
 *
 *   dtype   DA_BF16 only (DA_FP32 -> DA_E_UNSUPPORTED).
 *   d       128 or 64.   Hq % Hkv == 0 and (Hq/Hkv) even.
 *   q       logical [B,T,Hq,d]   (roles b, h, t)
 *   k, v    logical [B,T,Hkv,d]  (roles b, h, t)
 *   lam     logical [B,T,Hq/2] fp32 logits (roles b, h = pair, t); +-inf allowed.
 *   out     logical [B,T,Hq/2,d] bf16 (roles b, h = pair, t).
 */
da_status diffattn_v2_fwd(int dtype, int B, int T, int Hq, int Hkv, int d,
                          da_in q, da_in k, da_in v, da_in lam,
                          da_out out, void* stream);

/*
 * Bytes of device workspace diffattn_v2_decode needs for these sizes
 * (0 if the sizes are invalid).  The split of the cache length, and hence
 * the size, depends only on (B, L, Hq, Hkv, d).
 */
size_t diffattn_v2_decode_workspace_bytes(int B, int L, int Hq, int Hkv, int d);

/*
 * DIFF V2 decode ("Differential Transformer V2" article: DiffAttnV2 at the
 * newest position; decoding is memory-bound).  One new query token per
 * sequence against a KV cache of L entries that already holds that token at
 * position L-1; the query attends to all L entries:
 *   a_h = softmax_j( q[b,h] . k[b,j,g] / sqrt(d) ) v[b,:,g],  j < L
 *   out[b,p,:] = a_{2p} - sigmoid(lam[b,p]) * a_{2p+1}
 * The cache is split along L; each piece is reduced to a partial (max, sum,
 * weighted V) per head and the pieces are merged in a fixed order (no
 * atomics, so results are deterministic).
 *
 *   dtype      DA_BF16 only.   d in {64, 128}.  Hq % Hkv == 0, (Hq/Hkv) even.
 *   q          logical [B,Hq,d]      (roles b, h; st ignored)
 *   k_cache    logical [B,L,Hkv,d]   (roles b, h, t)
 *   v_cache    logical [B,L,Hkv,d]   (roles b, h, t)
 *   lam        logical [B,Hq/2] fp32 logits (roles b, h = pair; st ignored)
 *   out        logical [B,Hq/2,d] bf16 (roles b, h = pair; st ignored)
 *   workspace  device scratch of at least
 *              diffattn_v2_decode_workspace_bytes(B,L,Hq,Hkv,d) bytes,
 *              16-byte aligned, owned by the caller; its contents on entry
 *              do not matter and on return are unspecified.
 * Two kernels are enqueued on `stream` (split, then merge).
 */
da_status diffattn_v2_decode(int dtype, int B, int L, int Hq, int Hkv, int d,
                             da_in q, da_in k_cache, da_in v_cache, da_in lam,
                             da_out out, void* workspace, size_t workspace_bytes,
                             void* stream);

/*
 * Off-by-one softmax variants (Hacker News item 41780844, a comment
 * proposing that the softmax denominator gain an extra 1, equivalently an
 * extra logit of value 0 among the inputs).  Each
 * entry point computes exactly what its namesake above computes, with every
 * softmax map replaced by
 *     softmax1_j(x) = exp(x_j) / (1 + sum_k exp(x_k))
 * over the same visible keys -- the same as one more key whose logit is 0
 * for every query and whose value row is 0.  A row's attention weights then
 * sum to less than 1 and tend to 0 when every logit is very negative.
 * Arguments, layouts, validation, workspace and errors are those of the
 * namesake.
 */
da_status diffattn_v1_fwd_softmax1(int dtype, int B, int H, int T, int d,
                                   da_in q1, da_in q2, da_in k1, da_in k2, da_in v,
                                   const float* lam_q1, const float* lam_k1,
                                   const float* lam_q2, const float* lam_k2,
                                   int layer_index, da_out out, void* stream);
da_status diffattn_v2_fwd_softmax1(int dtype, int B, int T, int Hq, int Hkv, int d,
                                   da_in q, da_in k, da_in v, da_in lam,
                                   da_out out, void* stream);
da_status diffattn_v2_decode_softmax1(int dtype, int B, int L, int Hq, int Hkv, int d,
                                      da_in q, da_in k_cache, da_in v_cache, da_in lam,
                                      da_out out, void* workspace, size_t workspace_bytes,
                                      void* stream);

/*
 * DIFF V2 decode of nq new tokens per sequence at once (multi-token, e.g.
 * speculative, decoding).  The cache of L entries already holds the nq new
 * tokens at positions L-nq .. L-1; new token i (0-based) attends, causally,
 * to entries j <= L-nq+i -- the last nq rows of DiffAttnV2 over the cache
 * ("Differential Transformer V2" article, DiffAttnV2 pseudo-code; decoding
 * is memory-bound, so the cache is streamed once for all nq tokens):
 *   a_{i,h} = softmax_{j <= L-nq+i}( q[b,i,h] . k[b,j,g] / sqrt(d) ) v[b,:,g]
 *   out[b,i,p,:] = a_{i,2p} - sigmoid(lam[b,i,p]) * a_{i,2p+1}
 * With nq = 1 this is diffattn_v2_decode.
 *
 *   dtype, d, Hq, Hkv   as for diffattn_v2_decode.   1 <= nq <= L.
 *   q          logical [B,nq,Hq,d]   (roles b, h, t = new token)
 *   k_cache    logical [B,L,Hkv,d]   (roles b, h, t)
 *   v_cache    logical [B,L,Hkv,d]   (roles b, h, t)
 *   lam        logical [B,nq,Hq/2] fp32 logits (roles b, h = pair, t)
 *   out        logical [B,nq,Hq/2,d] bf16 (roles b, h = pair, t)
 *   workspace  at least diffattn_v2_decode_multi_workspace_bytes(B, L, nq,
 *              Hq, Hkv, d) bytes, 16-byte aligned, owned by the caller.
 * The cache is read once per group of 16 (Hq/Hkv*nq <= 16) or 32 (query
 * token, head) pairs of a kv head.  Two kernels are enqueued on `stream`.
 */
size_t diffattn_v2_decode_multi_workspace_bytes(int B, int L, int nq, int Hq, int Hkv, int d);
da_status diffattn_v2_decode_multi(int dtype, int B, int L, int nq, int Hq, int Hkv, int d,
                                   da_in q, da_in k_cache, da_in v_cache, da_in lam,
                                   da_out out, void* workspace, size_t workspace_bytes,
                                   void* stream);
/* Off-by-one softmax variant of diffattn_v2_decode_multi. */
da_status diffattn_v2_decode_multi_softmax1(int dtype, int B, int L, int nq, int Hq, int Hkv,
                                            int d, da_in q, da_in k_cache, da_in v_cache,
                                            da_in lam, da_out out, void* workspace,
                                            size_t workspace_bytes, void* stream);

/*
 * Bytes of device workspace diffattn_v2_decode_paged (and its _softmax1
 * variant) needs for these sizes (0 if the sizes are invalid); it depends
 * only on (B, max_len, nq, Hq, Hkv, d).
 */
size_t diffattn_v2_decode_paged_workspace_bytes(int B, int max_len, int nq, int Hq, int Hkv, int d);

/*
 * DIFF V2 decode over a paged, ragged KV cache.  Per sequence b it computes
 * exactly what diffattn_v2_decode_multi computes ("Differential Transformer
 * V2" article: DiffAttnV2 at the newest positions) with L = seq_lens[b]; only
 * the storage of the cache differs (nq = 1: one new token per sequence).  The pages define the attention, not this
 * layout: it is the serving layout in which sequences of different lengths
 * share one pool of fixed-size cache pages.
 *
 *   dtype        DA_BF16 only.   d in {64, 128}.  Hq % Hkv == 0, (Hq/Hkv)
 *                even and <= 16.
 *   max_len      the longest sequence allowed (>= 1); sets the split of the
 *                cache and the workspace size.
 *   nq           new tokens per sequence (>= 1), the last nq of its entries.
 *   q, lam, out  as for diffattn_v2_decode_multi (token axis used when
 *                nq > 1).
 *   k_pages      logical [num_pages, page_size, Hkv, d] bf16 with roles
 *   v_pages      b = page, h = kv head, t = row within the page.
 *   num_pages    pages in the pool (>= 1).
 *   page_size    tokens per page: a power of two, >= 16.
 *   block_table  DEVICE int32 [B][bt_stride], bt_stride >=
 *                ceil(max_len / page_size): token t of sequence b is row
 *                t % page_size of page block_table[b*bt_stride + t/page_size].
 *                Only the entries that cover t < seq_lens[b] are read.  An
 *                entry outside [0, num_pages) is clamped into it (wrong
 *                values, never an access outside the pool).
 *   seq_lens     DEVICE int32 [B]: cache entries of each sequence, the new
 *                token's included (the query attends to all of them).
 *                Values are clamped to [0, max_len]; a new token that sees
 *                no entry (a sequence shorter than nq, or of length 0) gets
 *                an output of 0.
 *   workspace    at least diffattn_v2_decode_paged_workspace_bytes(B,
 *                max_len, nq, Hq, Hkv, d) bytes, 16-byte aligned, owned by
 *                the caller; contents on entry do not matter.
 * Errors: DA_E_SHAPE also for a page_size that is not a power of two >= 16,
 * num_pages < 1 or a bt_stride too small; DA_E_UNSUPPORTED if page_size times
 * a token stride of k_pages / v_pages reaches 2^31 elements (rows within a
 * page are addressed with 32-bit offsets); DA_E_NULL for a NULL block_table or
 * seq_lens; DA_E_LAYOUT if either is not 4-byte aligned.  The table and the
 * lengths live on the device and are not checked on the host.
 * Two kernels are enqueued on `stream` (split, then merge).
 */
da_status diffattn_v2_decode_paged(int dtype, int B, int max_len, int nq, int Hq, int Hkv, int d,
                                   da_in q, da_in k_pages, da_in v_pages,
                                   int num_pages, int page_size,
                                   const int32_t* block_table, int64_t bt_stride,
                                   const int32_t* seq_lens, da_in lam, da_out out,
                                   void* workspace, size_t workspace_bytes, void* stream);
/* Off-by-one softmax variant of diffattn_v2_decode_paged (see the
 * *_softmax1 entry points above); a sequence of length 0 also gets 0. */
da_status diffattn_v2_decode_paged_softmax1(int dtype, int B, int max_len, int nq, int Hq,
                                            int Hkv, int d, da_in q, da_in k_pages, da_in v_pages,
                                            int num_pages, int page_size,
                                            const int32_t* block_table, int64_t bt_stride,
                                            const int32_t* seq_lens, da_in lam, da_out out,
                                            void* workspace, size_t workspace_bytes,
                                            void* stream);

/*
 * DIFF V2 training forward: diffattn_v2_fwd (or its off-by-one softmax
 * variant) that also keeps what diffattn_v2_bwd needs.
 *   attn   logical [B,T,Hq,d] bf16 (roles b, h = query head, t): each head's
 *          attention output before the pair combine (the pseudo-code's attn
 *          of "Differential Transformer V2", DiffAttnV2, before the 0::2 /
 *          1::2 split), normalised, rounded once to bf16.
 *   lse    DEVICE fp32 [B][Hq][T], contiguous: for each row, log2 of the
 *          softmax denominator of the scores scaled by log2(e)/sqrt(d), so a
 *          probability is exp2(q.k log2(e)/sqrt(d) - lse) (with the
 *          off-by-one softmax the denominator holds its extra term).
 * Other arguments, layouts and errors as for diffattn_v2_fwd; DA_E_NULL for
 * a NULL lse, DA_E_LAYOUT for a misaligned one.
 */
da_status diffattn_v2_fwd_train(int dtype, int B, int T, int Hq, int Hkv, int d,
                                da_in q, da_in k, da_in v, da_in lam,
                                da_out out, da_out attn, float* lse, void* stream);
da_status diffattn_v2_fwd_train_softmax1(int dtype, int B, int T, int Hq, int Hkv, int d,
                                         da_in q, da_in k, da_in v, da_in lam,
                                         da_out out, da_out attn, float* lse, void* stream);

/*
 * Bytes of device workspace diffattn_v2_bwd needs (0 if the sizes are
 * invalid): two fp32 arrays of B*Hq rows, each row padded to a multiple of
 * 128 tokens.
 */
size_t diffattn_v2_bwd_workspace_bytes(int B, int T, int Hq, int Hkv, int d);

/*
 * DIFF V2 backward ("Differential Transformer V2" article, DiffAttnV2
 * pseudo-code, differentiated): given dout = dL/dout, the gradients of the
 * prefill's inputs, from the training forward's attn and lse:
 *   d attn_2p = dout_p,   d attn_2p+1 = -sigmoid(lam_p) dout_p,
 *   dlam_p    = -sigmoid(lam_p) (1 - sigmoid(lam_p)) <dout_p, attn_2p+1>,
 *   and for every head the softmax-attention gradients dq, dk, dv (dk and
 *   dv of a kv head summed over the query heads of its group).
 *   dtype      DA_BF16 only; d in {64, 128}; Hq % Hkv == 0, (Hq/Hkv) even.
 *   q, k, v, lam   the forward's inputs (layouts as for diffattn_v2_fwd).
 *   attn, lse      the training forward's outputs for the same inputs.
 *   dout       logical [B,T,Hq/2,d] bf16.
 *   dq         logical [B,T,Hq,d] bf16;  dk, dv  logical [B,T,Hkv,d] bf16.
 *   dlam       logical [B,T,Hq/2] fp32 (roles b, h = pair, t).
 *   workspace  at least diffattn_v2_bwd_workspace_bytes(B,T,Hq,Hkv,d) bytes,
 *              256-byte aligned, owned by the caller.
 * Three kernels are enqueued on `stream` (a pre-pass, dq, then dk/dv); the
 * sums over heads and keys are taken in a fixed order (deterministic).
 * Token strides of q, k, v and dout must be below 2^24 elements
 * (DA_E_UNSUPPORTED).
 */
da_status diffattn_v2_bwd(int dtype, int B, int T, int Hq, int Hkv, int d,
                          da_in q, da_in k, da_in v, da_in lam, da_in attn,
                          const float* lse, da_in dout, da_out dq, da_out dk, da_out dv,
                          da_out dlam, void* workspace, size_t workspace_bytes, void* stream);

/*
 * DIFF V1 training forward: diffattn_v1_fwd (or its off-by-one softmax
 * variant) that also keeps what diffattn_v1_bwd needs.
 *   attn1, attn2  logical [B,T,H,2d] bf16 (roles b, h = differential head,
 *          t): each map's attention output softmax(q_m k_m^T / sqrt d) v,
 *          normalised, rounded once to bf16 (the two flash-attention outputs
 *          that "Differential Transformer V2" article's DiffAttnV1 pseudo-code
 *          combines).
 *   lse    DEVICE fp32 [2][B][H][T], contiguous: for map m (0: q1/k1,
 *          1: q2/k2) and each row, log2 of the softmax denominator of the
 *          scores scaled by log2(e)/sqrt(d) (with the off-by-one softmax the
 *          denominator holds its extra term).
 * Other arguments, layouts and errors as for diffattn_v1_fwd; bf16 only
 * (DA_E_UNSUPPORTED for fp32); DA_E_NULL for a NULL lse, DA_E_LAYOUT for a
 * misaligned one.
 */
da_status diffattn_v1_fwd_train(int dtype, int B, int H, int T, int d, da_in q1, da_in q2, da_in k1, da_in k2,
                                da_in v, const float* lam_q1, const float* lam_k1, const float* lam_q2,
                                const float* lam_k2, int layer_index, da_out out, da_out attn1, da_out attn2,
                                float* lse, void* stream);
da_status diffattn_v1_fwd_train_softmax1(int dtype, int B, int H, int T, int d, da_in q1, da_in q2,
                                         da_in k1, da_in k2, da_in v, const float* lam_q1, const float* lam_k1,
                                         const float* lam_q2, const float* lam_k2, int layer_index, da_out out,
                                         da_out attn1, da_out attn2, float* lse, void* stream);

/*
 * Bytes of device workspace diffattn_v1_bwd needs (0 if the sizes are
 * invalid): dD in bf16 (B*T*H*2d), four fp32 arrays of B*H rows padded to
 * a multiple of 128 tokens, and one fp32 value per (b, t, h).
 */
size_t diffattn_v1_bwd_workspace_bytes(int B, int H, int T, int d);

/*
 * DIFF V1 backward ("Differential Transformer V2" article, DiffAttnV1
 * pseudo-code, with the RMSNorm of Wilsontomass's module in the nanoGPT
 * issue "How best to implement a differential transformer?",
 * differentiated): given dout = dL/dout, the gradients of the forward's
 * inputs from the training forward's attn1, attn2 and lse.  With
 * D = a_1 - lam a_2 and r = (mean D^2 + 1e-5)^(-1/2) per (token, head):
 *   dD = (1 - lam_init) r (dout - r^2 D mean(dout D)),
 *   d a_1 = dD,  d a_2 = -lam dD,  dlam = -sum over (b, t, h) of <dD, a_2>,
 *   per map the softmax-attention gradients dq_m, dk_m and dv (dv summed
 *   over both maps), and the lambda vectors' gradients
 *   dlam_q1 = dlam e1 lam_k1, dlam_k1 = dlam e1 lam_q1,
 *   dlam_q2 = -dlam e2 lam_k2, dlam_k2 = -dlam e2 lam_q2,
 *   e1 = exp(<lam_q1, lam_k1>), e2 = exp(<lam_q2, lam_k2>).
 *   dtype      DA_BF16 only; d in {64, 128}.
 *   q1 .. v, lam vectors, layer_index   the forward's inputs (layouts as for
 *              diffattn_v1_fwd).
 *   attn1, attn2, lse   the training forward's outputs for the same inputs.
 *   dout       logical [B,T,H,2d] bf16.
 *   dq1, dq2, dk1, dk2  logical [B,H,T,d] bf16;  dv  logical [B,H,T,2d] bf16.
 *   dlam_q1 .. dlam_k2  DEVICE fp32 [d] each.
 *   workspace  at least diffattn_v1_bwd_workspace_bytes(B,H,T,d) bytes,
 *              256-byte aligned, owned by the caller.
 * Two kernels are enqueued on `stream` (a pre-pass, then one grid with the
 * dlam reduction, dq of both maps, dk of both maps and dv); every sum is
 * taken in a fixed order (deterministic).  Token strides of q1 .. v must be below 2^24 elements
 * (DA_E_UNSUPPORTED).
 */
da_status diffattn_v1_bwd(int dtype, int B, int H, int T, int d, da_in q1, da_in q2, da_in k1, da_in k2,
                          da_in v, const float* lam_q1, const float* lam_k1, const float* lam_q2,
                          const float* lam_k2, int layer_index, da_in attn1, da_in attn2, const float* lse,
                          da_in dout, da_out dq1, da_out dq2, da_out dk1, da_out dk2, da_out dv, float* dlam_q1,
                          float* dlam_k1, float* dlam_q2, float* dlam_k2, void* workspace, size_t workspace_bytes,
                          void* stream);

/*
 * Rotary position embedding (Wilsontomass's module in the nanoGPT issue "How
 * best to implement a differential transformer?" rotates every q and k head
 * before the attention; the rotate-half arrangement): element c < d/2 of a
 * head vector pairs with c + d/2 and the pair turns by t * theta^(-2c/d) at
 * position t:  x'_c = x_c cos - x_{c+d/2} sin,  x'_{c+d/2} = x_{c+d/2} cos +
 * x_c sin.  theta: a finite float > 0 (10000 in the usual setting).
 *
 * diffattn_rope: rotate x, logical [B,T,H,d] bf16 (roles b, h, t), row t at
 *   position pos0 + t, into out (same logical shape; out == x rotates in
 *   place).  d a multiple of 8, at most 256; pos0 >= 0 and pos0 + T < 2^24.  One
 *   HBM-bound kernel.  Use it for keys written into a cache, which the
 *   decode entry points below expect rotated.
 */
da_status diffattn_rope(int dtype, int B, int T, int H, int d, da_in x, da_out out, float theta, int pos0,
                        void* stream);

/*
 * DIFF V1 / V2 prefill with the rotary embedding applied to q and k first
 * (positions 0 .. T-1): q is rotated inside the attention kernel's prologue,
 * k by diffattn_rope into the caller's workspace (k's tiles are read by
 * several workgroups each, so it is rotated once), then the attention reads
 * it.  Arguments, layouts and errors as for diffattn_v1_fwd /
 * diffattn_v2_fwd, plus theta and a workspace of at least
 * diffattn_v1_fwd_rope_workspace_bytes(B,H,T,d) /
 * diffattn_v2_fwd_rope_workspace_bytes(B,T,Hkv,d) bytes, 256-byte aligned
 * (DA_E_WORKSPACE otherwise).  bf16 only; T < 2^24.
 */
size_t diffattn_v1_fwd_rope_workspace_bytes(int B, int H, int T, int d);
da_status diffattn_v1_fwd_rope(int dtype, int B, int H, int T, int d, da_in q1, da_in q2, da_in k1, da_in k2,
                               da_in v, const float* lam_q1, const float* lam_k1, const float* lam_q2,
                               const float* lam_k2, int layer_index, float theta, da_out out, void* workspace,
                               size_t workspace_bytes, void* stream);
size_t diffattn_v2_fwd_rope_workspace_bytes(int B, int T, int Hkv, int d);
da_status diffattn_v2_fwd_rope(int dtype, int B, int T, int Hq, int Hkv, int d, da_in q, da_in k, da_in v,
                               da_in lam, float theta, da_out out, void* workspace, size_t workspace_bytes,
                               void* stream);

/*
 * DIFF V2 decode with the new token's q rotated to its cache position inside
 * the decode kernel: L - 1 (dense), seq_lens[b] - nq + i (paged, new token
 * i).  The cache must hold its keys already rotated, each at its own
 * position (as diffattn_rope with pos0 = the first row's position writes
 * them).  Arguments, workspace and errors as for diffattn_v2_decode /
 * diffattn_v2_decode_paged, plus theta (DA_E_SHAPE unless finite and > 0).
 */
da_status diffattn_v2_decode_rope(int dtype, int B, int L, int Hq, int Hkv, int d, da_in q, da_in k_cache,
                                  da_in v_cache, da_in lam, float theta, da_out out, void* workspace,
                                  size_t workspace_bytes, void* stream);
da_status diffattn_v2_decode_paged_rope(int dtype, int B, int max_len, int nq, int Hq, int Hkv, int d, da_in q,
                                        da_in k_pages, da_in v_pages, int num_pages, int page_size,
                                        const int32_t* block_table, int64_t bt_stride, const int32_t* seq_lens,
                                        da_in lam, float theta, da_out out, void* workspace,
                                        size_t workspace_bytes, void* stream);

/*
 * The four rotary-embedding entry points above with every softmax map
 * replaced by the off-by-one softmax (as the *_softmax1 entry points do):
 * identical arguments, checks and workspaces.
 */
da_status diffattn_v1_fwd_softmax1_rope(int dtype, int B, int H, int T, int d, da_in q1, da_in q2, da_in k1,
                                       da_in k2, da_in v, const float* lam_q1, const float* lam_k1,
                                       const float* lam_q2, const float* lam_k2, int layer_index, float theta,
                                       da_out out, void* workspace, size_t workspace_bytes, void* stream);
da_status diffattn_v2_fwd_softmax1_rope(int dtype, int B, int T, int Hq, int Hkv, int d, da_in q, da_in k,
                                       da_in v, da_in lam, float theta, da_out out, void* workspace,
                                       size_t workspace_bytes, void* stream);
da_status diffattn_v2_decode_softmax1_rope(int dtype, int B, int L, int Hq, int Hkv, int d, da_in q,
                                          da_in k_cache, da_in v_cache, da_in lam, float theta, da_out out,
                                          void* workspace, size_t workspace_bytes, void* stream);
da_status diffattn_v2_decode_paged_softmax1_rope(int dtype, int B, int max_len, int nq, int Hq, int Hkv, int d,
                                                da_in q, da_in k_pages, da_in v_pages, int num_pages, int page_size,
                                                const int32_t* block_table, int64_t bt_stride,
                                                const int32_t* seq_lens, da_in lam, float theta, da_out out,
                                                void* workspace, size_t workspace_bytes, void* stream);

/*
 * diffattn_v2_decode without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc).  Same arguments, checks and result as
 * diffattn_v2_decode (within the bf16 tolerance: the split of the cache may
 * differ, so the last bits may), but the split partials go to a static
 * device array of the library, diffattn_v2_decode_noalloc_max_bytes() = 16 MiB
 * per GPU, allocated when the library is loaded and held until the process
 * ends.  The call lowers the number of cache splits until the partials
 * (B * Hkv * splits * Hq/Hkv * (d + 2) * 4 bytes) fit; if one split does
 * not fit (B * Hq * (d + 2) * 4 > 16 MiB) it returns DA_E_SCRATCH and
 * enqueues nothing.  It calls no allocating routine.
 * Every call on one GPU uses that GPU's one array: calls that overlap in
 * time on one GPU (different streams, or threads without ordering) race and
 * give wrong results; calls on one stream are ordered and safe.
 */
da_status diffattn_v2_decode_noalloc(int dtype, int B, int L, int Hq, int Hkv, int d, da_in q,
                                     da_in k_cache, da_in v_cache, da_in lam, da_out out, void* stream);
size_t diffattn_v2_decode_noalloc_max_bytes(void);

/*
 * DIFF V2 lambda projection ("Differential Transformer V2" article: lambda
 * is computed per token and per head by a projection the article does not
 * show; read here as a linear map without bias of the token's hidden state):
 *   out[b,t,p] = sum_c x[b,t,c] w[p,c]   (fp32 logits; the sigmoid stays in
 *   diffattn_v2_fwd, which takes these logits as lam).
 *   x    logical [B,T,dm] bf16 (roles b, t; sh unused), 16-byte rows.
 *   w    logical [P,dm] bf16, a linear layer's weight (the pair stride in sh;
 *        sb, st unused).
 *   out  logical [B,T,P] fp32 (roles b, h = pair, t), 4-byte aligned.
 *   dm a multiple of 128 (DA_E_UNSUPPORTED otherwise).  One kernel, MFMA,
 *   reads x once; sums over dm in a fixed order (deterministic).
 */
da_status diffattn_v2_lambda_proj(int dtype, int B, int T, int dm, int P, da_in x, da_in w, da_in out,
                                  void* stream);

/* lambda_init = 0.8 - 0.6*exp(-0.3*layer_index), as the V1 kernels use it
 * (computed on the host in double, handed to the device as float). */
double diffattn_lambda_init(int layer_index);

/* Static, NUL-terminated description of a status code. */
const char* diffattn_status_string(da_status s);

#ifdef __cplusplus
}
#endif
#endif /* DIFFATTN_H */
