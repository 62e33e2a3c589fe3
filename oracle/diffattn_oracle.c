/*
 * diffattn_oracle.c -- plain fp64 CPU reference for differential attention.
 *
 * TEST INFRASTRUCTURE ONLY (see diffattn_oracle.h).  Scalar loops, no
 * blocking, no fusion, no online softmax: each output row is computed from
 * the definition, one causal softmax row at a time.  OpenMP only spreads
 * independent rows over threads.
 */
#include "diffattn_oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* [V2A] DiffAttnV1: lam_init = 0.8 - 0.6 * exp(-0.3 * layer_index). */
double da_oracle_lambda_init(int layer) {
    return 0.8 - 0.6 * exp(-0.3 * (double)layer);
}

static double dot(int n, const double* a, const double* b) {
    double s = 0.0;
    for (int c = 0; c < n; ++c) s += a[c] * b[c];
    return s;
}

/* [V2A] DiffAttnV1: lam1 = exp(sum(lam_q1*lam_k1)), lam2 likewise,
 * lam = lam1 - lam2 + lam_init. */
double da_oracle_v1_lambda(int d, const double* lq1, const double* lk1,
                           const double* lq2, const double* lk2, int layer) {
    return exp(dot(d, lq1, lk1)) - exp(dot(d, lq2, lk2)) +
           da_oracle_lambda_init(layer);
}

/* Logistic sigmoid, in the branch that never overflows; sigmoid(-inf) = 0
 * and sigmoid(+inf) = 1 exactly.  [V2A] DiffAttnV2 (lam_val = sigmoid(lam)). */
static double sigmoid(double x) {
    if (x >= 0.0) return 1.0 / (1.0 + exp(-x));
    double e = exp(x);
    return e / (1.0 + e);
}

/*
 * One causal softmax-attention row (the flash_attn_func / causal SDPA call
 * of [V2A] and [NGI], written out):
 *   s_j = q . k_j / sqrt(d)          for j = 0 .. nkeys-1 (the caller passes
 *                                    only the keys the query may see)
 *   w_j = exp(s_j - M),  Z = sum_j w_j,  M = max_j s_j
 *   out[c] = sum_j w_j v_j[c] / Z    for c < dv
 * With softmax1 set, the off-by-one softmax proposed in a comment of
 * Hacker News item 41780844: one is added to the softmax denominator, which
 * is the same as one more logit 0 whose value row is 0.  M then also covers
 * that logit, M = max(0, max_j s_j), and Z gains exp(0 - M).
 * k_j is at k + j*kstride, v_j at v + j*vstride.  w is caller scratch of
 * nkeys doubles.  If lse is not NULL it receives M + log(Z), the natural log
 * of the row's softmax denominator.
 */
static void softmax_attention_row(int d, int dv, int nkeys, const double* q,
                                  const double* k, int64_t kstride,
                                  const double* v, int64_t vstride,
                                  int softmax1, double* w, double* out, double* lse) {
    const double scale = 1.0 / sqrt((double)d);
    double m = softmax1 ? 0.0 : -INFINITY;
    for (int j = 0; j < nkeys; ++j) {
        w[j] = dot(d, q, k + (int64_t)j * kstride) * scale;
        if (w[j] > m) m = w[j];
    }
    double z = softmax1 ? exp(0.0 - m) : 0.0;
    for (int j = 0; j < nkeys; ++j) {
        w[j] = exp(w[j] - m);
        z += w[j];
    }
    for (int c = 0; c < dv; ++c) out[c] = 0.0;
    for (int j = 0; j < nkeys; ++j) {
        const double* vj = v + (int64_t)j * vstride;
        for (int c = 0; c < dv; ++c) out[c] += w[j] * vj[c];
    }
    for (int c = 0; c < dv; ++c) out[c] /= z;
    if (lse) *lse = m + log(z);
}

/*
 * One V1 output row (b, h, i), the steps of [V2A] DiffAttnV1 in their order:
 *   attn1 = attention(q1, k1, v), attn2 = attention(q2, k2, v)   (causal)
 *   attn  = attn1 - lam * attn2
 *   attn  = rmsnorm(attn)     -- over the 2d channels, eps 1e-5 inside the
 *                                root, no weight ([NGI] subln definition)
 *   attn  = attn * (1 - lam_init)
 */
static void v1_row(int H, int T, int d, const double* q1, const double* q2,
                   const double* k1, const double* k2, const double* v,
                   double lam, double lam_init, int softmax1, int b, int h, int i,
                   double* w, double* a1, double* a2, double* dst) {
    const int dv = 2 * d;
    const int64_t bh = (int64_t)b * H + h;
    const double* q1i = q1 + (bh * T + i) * d;
    const double* q2i = q2 + (bh * T + i) * d;
    const double* k1h = k1 + bh * T * d;
    const double* k2h = k2 + bh * T * d;
    const double* vh = v + bh * T * dv;
    softmax_attention_row(d, dv, i + 1, q1i, k1h, d, vh, dv, softmax1, w, a1, NULL);
    softmax_attention_row(d, dv, i + 1, q2i, k2h, d, vh, dv, softmax1, w, a2, NULL);
    double ms = 0.0;
    for (int c = 0; c < dv; ++c) {
        a1[c] = a1[c] - lam * a2[c];
        ms += a1[c] * a1[c];
    }
    ms /= dv;
    const double r = 1.0 / sqrt(ms + 1e-5);
    for (int c = 0; c < dv; ++c) dst[c] = a1[c] * r * (1.0 - lam_init);
}

void da_oracle_v1_fwd(int B, int H, int T, int d, const double* q1,
                      const double* q2, const double* k1, const double* k2,
                      const double* v, const double* lq1, const double* lk1,
                      const double* lq2, const double* lk2, int layer,
                      int softmax1, double* out) {
    const double lam = da_oracle_v1_lambda(d, lq1, lk1, lq2, lk2, layer);
    const double li = da_oracle_lambda_init(layer);
    const int dv = 2 * d;
    const int64_t nrows = (int64_t)B * H * T;
#pragma omp parallel
    {
        double* w = (double*)malloc(sizeof(double) * (size_t)(T > 0 ? T : 1));
        double* a1 = (double*)malloc(sizeof(double) * (size_t)dv);
        double* a2 = (double*)malloc(sizeof(double) * (size_t)dv);
#pragma omp for schedule(dynamic, 16)
        for (int64_t r = 0; r < nrows; ++r) {
            const int i = (int)(r % T);
            const int h = (int)((r / T) % H);
            const int b = (int)(r / ((int64_t)T * H));
            double* dst = out + (((int64_t)b * T + i) * H + h) * dv;
            v1_row(H, T, d, q1, q2, k1, k2, v, lam, li, softmax1, b, h, i, w, a1, a2, dst);
        }
        free(w);
        free(a1);
        free(a2);
    }
}

void da_oracle_v1_rows(int B, int H, int T, int d, const double* q1,
                       const double* q2, const double* k1, const double* k2,
                       const double* v, const double* lq1, const double* lk1,
                       const double* lq2, const double* lk2, int layer,
                       int softmax1, int64_t n, const int64_t* bhi, double* out_rows) {
    (void)B;
    const double lam = da_oracle_v1_lambda(d, lq1, lk1, lq2, lk2, layer);
    const double li = da_oracle_lambda_init(layer);
    const int dv = 2 * d;
#pragma omp parallel
    {
        double* w = (double*)malloc(sizeof(double) * (size_t)(T > 0 ? T : 1));
        double* a1 = (double*)malloc(sizeof(double) * (size_t)dv);
        double* a2 = (double*)malloc(sizeof(double) * (size_t)dv);
#pragma omp for schedule(dynamic, 1)
        for (int64_t r = 0; r < n; ++r) {
            v1_row(H, T, d, q1, q2, k1, k2, v, lam, li, softmax1, (int)bhi[3 * r],
                   (int)bhi[3 * r + 1], (int)bhi[3 * r + 2], w, a1, a2,
                   out_rows + r * dv);
        }
        free(w);
        free(a1);
        free(a2);
    }
}

/*
 * One V2 output row (b, t, p), the steps of [V2A] DiffAttnV2: one attention
 * over all Hq query heads, heads of a GQA group contiguous so head h reads
 * kv head g = h / (Hq/Hkv); the output pairs adjacent heads,
 *   attn1 = attn[:, 0::2], attn2 = attn[:, 1::2]
 *   attn  = attn1 - sigmoid(lam) * attn2.
 * nkeys = number of keys visible to the query (t + 1 for causal prefill,
 * L for decode); qrow points at q[b, t, 0, 0]; kb, vb at k[b, 0, 0, 0].
 */
static void v2_row(int Hq, int Hkv, int d, int nkeys, const double* qrow,
                   const double* kb, const double* vb, double lam_logit,
                   int p, int softmax1, double* w, double* a_even, double* a_odd,
                   double* dst) {
    const int group = Hq / Hkv;
    const int he = 2 * p, ho = 2 * p + 1;
    const int ge = he / group, go = ho / group;
    const int64_t kvstride = (int64_t)Hkv * d; /* token stride in k, v */
    softmax_attention_row(d, d, nkeys, qrow + (int64_t)he * d, kb + (int64_t)ge * d,
                          kvstride, vb + (int64_t)ge * d, kvstride, softmax1, w, a_even, NULL);
    softmax_attention_row(d, d, nkeys, qrow + (int64_t)ho * d, kb + (int64_t)go * d,
                          kvstride, vb + (int64_t)go * d, kvstride, softmax1, w, a_odd, NULL);
    const double s = sigmoid(lam_logit);
    for (int c = 0; c < d; ++c) dst[c] = a_even[c] - s * a_odd[c];
}

void da_oracle_v2_fwd(int B, int T, int Hq, int Hkv, int d, const double* q,
                      const double* k, const double* v, const double* lam,
                      int softmax1, double* out) {
    const int P = Hq / 2;
    const int64_t nrows = (int64_t)B * T * P;
#pragma omp parallel
    {
        double* w = (double*)malloc(sizeof(double) * (size_t)(T > 0 ? T : 1));
        double* ae = (double*)malloc(sizeof(double) * (size_t)d);
        double* ao = (double*)malloc(sizeof(double) * (size_t)d);
#pragma omp for schedule(dynamic, 16)
        for (int64_t r = 0; r < nrows; ++r) {
            const int p = (int)(r % P);
            const int t = (int)((r / P) % T);
            const int b = (int)(r / ((int64_t)P * T));
            const double* qrow = q + ((int64_t)b * T + t) * Hq * d;
            const double* kb = k + (int64_t)b * T * Hkv * d;
            const double* vb = v + (int64_t)b * T * Hkv * d;
            const double lg = lam[((int64_t)b * T + t) * P + p];
            v2_row(Hq, Hkv, d, t + 1, qrow, kb, vb, lg, p, softmax1, w, ae, ao,
                   out + (((int64_t)b * T + t) * P + p) * d);
        }
        free(w);
        free(ae);
        free(ao);
    }
}

void da_oracle_v2_rows(int B, int T, int Hq, int Hkv, int d, const double* q,
                       const double* k, const double* v, const double* lam,
                       int softmax1, int64_t n, const int64_t* btp, double* out_rows) {
    (void)B;
    const int P = Hq / 2;
#pragma omp parallel
    {
        double* w = (double*)malloc(sizeof(double) * (size_t)(T > 0 ? T : 1));
        double* ae = (double*)malloc(sizeof(double) * (size_t)d);
        double* ao = (double*)malloc(sizeof(double) * (size_t)d);
#pragma omp for schedule(dynamic, 1)
        for (int64_t r = 0; r < n; ++r) {
            const int b = (int)btp[3 * r], t = (int)btp[3 * r + 1],
                      p = (int)btp[3 * r + 2];
            const double* qrow = q + ((int64_t)b * T + t) * Hq * d;
            const double* kb = k + (int64_t)b * T * Hkv * d;
            const double* vb = v + (int64_t)b * T * Hkv * d;
            const double lg = lam[((int64_t)b * T + t) * P + p];
            v2_row(Hq, Hkv, d, t + 1, qrow, kb, vb, lg, p, softmax1, w, ae, ao,
                   out_rows + r * d);
        }
        free(w);
        free(ae);
        free(ao);
    }
}

void da_oracle_v2_decode(int B, int L, int Hq, int Hkv, int d,
                         const double* q, const double* k, const double* v,
                         const double* lam, int softmax1, double* out) {
    const int P = Hq / 2;
    const int64_t nrows = (int64_t)B * P;
#pragma omp parallel
    {
        double* w = (double*)malloc(sizeof(double) * (size_t)(L > 0 ? L : 1));
        double* ae = (double*)malloc(sizeof(double) * (size_t)d);
        double* ao = (double*)malloc(sizeof(double) * (size_t)d);
#pragma omp for schedule(dynamic, 1)
        for (int64_t r = 0; r < nrows; ++r) {
            const int p = (int)(r % P);
            const int b = (int)(r / P);
            const double* qrow = q + (int64_t)b * Hq * d;
            const double* kb = k + (int64_t)b * L * Hkv * d;
            const double* vb = v + (int64_t)b * L * Hkv * d;
            v2_row(Hq, Hkv, d, L, qrow, kb, vb, lam[(int64_t)b * P + p], p, softmax1, w,
                   ae, ao, out + ((int64_t)b * P + p) * d);
        }
        free(w);
        free(ae);
        free(ao);
    }
}

/*
 * Every query head's own causal attention, before the pairs are combined
 * ([V2A] DiffAttnV2: the single attention call over all Hq heads, head h
 * reading kv head h / (Hq/Hkv)):
 *   attn[b, t, h, :] = softmax_j(q_h . k_g(h),j / sqrt d) v_g(h),j   (j <= t)
 *   lse[b, h, t]     = natural log of that row's softmax denominator
 * What a backward pass keeps from the forward; rows computed one at a time.
 */
void da_oracle_v2_heads(int B, int T, int Hq, int Hkv, int d, const double* q,
                        const double* k, const double* v, int softmax1,
                        double* attn, double* lse) {
    const int group = Hq / Hkv;
    const int64_t nrows = (int64_t)B * T * Hq;
    const int64_t kvstride = (int64_t)Hkv * d;
#pragma omp parallel
    {
        double* w = (double*)malloc(sizeof(double) * (size_t)(T > 0 ? T : 1));
#pragma omp for schedule(dynamic, 16)
        for (int64_t r = 0; r < nrows; ++r) {
            const int h = (int)(r % Hq);
            const int t = (int)((r / Hq) % T);
            const int b = (int)(r / ((int64_t)Hq * T));
            const int g = h / group;
            const double* qrow = q + (((int64_t)b * T + t) * Hq + h) * d;
            const double* kb = k + (int64_t)b * T * kvstride + (int64_t)g * d;
            const double* vb = v + (int64_t)b * T * kvstride + (int64_t)g * d;
            softmax_attention_row(d, d, t + 1, qrow, kb, kvstride, vb, kvstride, softmax1, w,
                                  attn + r * d, lse + ((int64_t)b * Hq + h) * T + t);
        }
        free(w);
    }
}

int da_oracle_set_threads(int n) {
#ifdef _OPENMP
    if (n > 0) omp_set_num_threads(n);
    return omp_get_max_threads();
#else
    (void)n;
    return 1;
#endif
}
