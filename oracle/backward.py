"""fp64 oracle for the DIFF V2 and DIFF V1 training steps: forward with the
quantities a backward pass keeps, and the gradients -- TEST INFRASTRUCTURE
ONLY (the same rule as the rest of ``oracle/``: only ``tests/``,
``__graft_entry__.smoke()`` and ``bench.py``'s ``cpu_baseline`` use it).
The V1 part follows the V2 part below.

What is differentiated ("Differential Transformer V2" article, DiffAttnV2
pseudo-code; the paragraph on the per-token projected lambda):

    attn[:, h]    = softmax_j( q_h . k_g(h) / sqrt(d) ) v_g(h),  j <= i (causal)
    out[:, p]     = attn[:, 2p] - sigmoid(lam[:, p]) * attn[:, 2p+1]

with g(h) = h // (Hq / Hkv).  The gradients follow from the chain rule, step
by step in the forward's order reversed (plain dense matrices per head, numpy
fp64, no blocking):

    d attn_2p     = dout_p
    d attn_2p+1   = -sigmoid(lam_p) * dout_p               (per token)
    d lam_p       = -sigmoid(lam_p) (1 - sigmoid(lam_p)) <dout_p, attn_2p+1>
    per head h:   dP = d attn_h  v_g^T
                  dS = P o (dP - rowsum(P o dP))          (softmax Jacobian)
                  dq_h  = dS k_g / sqrt(d)
                  dk_g += dS^T q_h / sqrt(d)
                  dv_g += P^T d attn_h

With the off-by-one softmax (an extra logit 0 in every row, Hacker News item
41780844) P is exp(S_ij) / (1 + sum_j exp(S_ij)); its Jacobian has the same
form, so the same steps apply with that P.

``lse`` is what a kernel keeps per (b, head, row) to rebuild P without the
row's running statistics: log2 of the row's softmax denominator of the
log2(e)-scaled scores, i.e. P_ij = exp2(S_ij log2(e) - lse_i).
"""
from __future__ import annotations

import math

import numpy as np

from . import _f64, lambda_init


def _rows(q, k, v, softmax1):
    """Per-head causal attention of one batch entry: q [T,Hq,d], k/v [T,Hkv,d]
    -> P [Hq,T,T], attn [T,Hq,d], lse2 [Hq,T]."""
    T, Hq, d = q.shape
    Hkv = k.shape[1]
    G = Hq // Hkv
    P = np.zeros((Hq, T, T))
    attn = np.zeros((T, Hq, d))
    lse2 = np.zeros((Hq, T))
    mask = np.triu(np.ones((T, T), dtype=bool), k=1)
    for h in range(Hq):
        g = h // G
        S = q[:, h] @ k[:, g].T / math.sqrt(d)
        S = np.where(mask, -np.inf, S)
        m = S.max(axis=1, keepdims=True)
        if softmax1:
            m = np.maximum(m, 0.0)  # the extra logit 0 takes part in the max
        e = np.exp(S - m)
        z = e.sum(axis=1, keepdims=True) + (np.exp(-m) if softmax1 else 0.0)
        P[h] = e / z
        attn[:, h] = P[h] @ v[:, g]
        lse2[h] = (m[:, 0] + np.log(z[:, 0])) / math.log(2.0)
    return P, attn, lse2


def v2_fwd_train(q, k, v, lam, softmax1: bool = False):
    """DIFF V2 prefill keeping what the backward needs.

    q [B,T,Hq,d], k/v [B,T,Hkv,d], lam [B,T,Hq/2] -> (out [B,T,Hq/2,d],
    attn [B,T,Hq,d], lse2 [B,Hq,T]), all float64.
    """
    q, k, v, lam = [_f64(x) for x in (q, k, v, lam)]
    B, T, Hq, d = q.shape
    out = np.zeros((B, T, Hq // 2, d))
    attn = np.zeros((B, T, Hq, d))
    lse2 = np.zeros((B, Hq, T))
    for b in range(B):
        _, attn[b], lse2[b] = _rows(q[b], k[b], v[b], softmax1)
        sig = 1.0 / (1.0 + np.exp(-lam[b]))  # [T, Hq/2]
        out[b] = attn[b][:, 0::2] - sig[..., None] * attn[b][:, 1::2]
    return out, attn, lse2


def v2_bwd(q, k, v, lam, dout, softmax1: bool = False):
    """Gradients of sum(dout * out) for DIFF V2 prefill.

    Returns (dq [B,T,Hq,d], dk [B,T,Hkv,d], dv [B,T,Hkv,d], dlam [B,T,Hq/2]),
    float64.
    """
    q, k, v, lam, dout = [_f64(x) for x in (q, k, v, lam, dout)]
    B, T, Hq, d = q.shape
    Hkv = k.shape[2]
    G = Hq // Hkv
    dq, dk, dv = np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)
    dlam = np.zeros_like(lam)
    for b in range(B):
        P, attn, _ = _rows(q[b], k[b], v[b], softmax1)
        sig = 1.0 / (1.0 + np.exp(-lam[b]))  # [T, Hq/2]
        da = np.zeros((T, Hq, d))
        da[:, 0::2] = dout[b]
        da[:, 1::2] = -sig[..., None] * dout[b]
        dlam[b] = -sig * (1.0 - sig) * np.einsum("tpc,tpc->tp", dout[b], attn[:, 1::2])
        for h in range(Hq):
            g = h // G
            dP = da[:, h] @ v[b][:, g].T
            dS = P[h] * (dP - (P[h] * dP).sum(axis=1, keepdims=True))
            dq[b][:, h] = dS @ k[b][:, g] / math.sqrt(d)
            dk[b][:, g] += dS.T @ q[b][:, h] / math.sqrt(d)
            dv[b][:, g] += P[h].T @ da[:, h]
    return dq, dk, dv, dlam


def v2_bwd_rounding_bounds(q, k, v, lam, dout, softmax1: bool = False):
    """Per-element scale of what bf16 rounding can move in each gradient of
    :func:`v2_bwd`, for a path that holds P, dS, d attn and attn in bf16
    (relative rounding u = 2^-9 each) and accumulates in fp32.

    Each bound is u times the sum of the absolute values of the terms that a
    rounded factor enters, following the same steps as :func:`v2_bwd`:
      E_i     = sum_c |d attn_ic| |attn_ic|     (what rounding attn moves in D_i)
      dq_ic  <- sum_j (P_ij E_i + |dS_ij|) |k_jc| / sqrt d
      dk_jc  <- sum_{h,i} (P_ij E_i + |dS_ij|) |q_ic| / sqrt d
      dv_jc  <- 2 sum_{h,i} P_ij |d attn_ic|
      dlam   <- 2 s (1 - s) sum_c |dout_c| |attn_odd,c|
    Returns (bq, bk, bv, blam) shaped like the gradients.
    """
    q, k, v, lam, dout = [_f64(x) for x in (q, k, v, lam, dout)]
    u = 2.0 ** -9
    B, T, Hq, d = q.shape
    G = Hq // k.shape[2]
    bq, bk, bv = np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)
    blam = np.zeros_like(lam)
    for b in range(B):
        P, attn, _ = _rows(q[b], k[b], v[b], softmax1)
        sig = 1.0 / (1.0 + np.exp(-lam[b]))
        da = np.zeros((T, Hq, d))
        da[:, 0::2] = dout[b]
        da[:, 1::2] = -sig[..., None] * dout[b]
        blam[b] = 2 * u * sig * (1.0 - sig) * np.einsum("tpc,tpc->tp", np.abs(dout[b]), np.abs(attn[:, 1::2]))
        for h in range(Hq):
            g = h // G
            dP = da[:, h] @ v[b][:, g].T
            dS = P[h] * (dP - (P[h] * dP).sum(axis=1, keepdims=True))
            E = (np.abs(da[:, h]) * np.abs(attn[:, h])).sum(axis=1, keepdims=True)
            W = P[h] * E + np.abs(dS)
            bq[b][:, h] = u * (W @ np.abs(k[b][:, g])) / math.sqrt(d)
            bk[b][:, g] += u * (W.T @ np.abs(q[b][:, h])) / math.sqrt(d)
            bv[b][:, g] += 2 * u * (P[h].T @ np.abs(da[:, h]))
    return bq, bk, bv, blam


# ---- DIFF V1 ---------------------------------------------------------------------
#
# What is differentiated ("Differential Transformer V2" article, DiffAttnV1
# pseudo-code; nanoGPT issue "How best to implement a differential
# transformer?", Wilsontomass's module for the RMSNorm arguments):
#
#     a_m    = causal softmax(q_m k_m^T / sqrt(d)) v        (m = 1, 2; v is 2d wide)
#     lam    = exp(<lq1, lk1>) - exp(<lq2, lk2>) + lam_init(layer)
#     D      = a_1 - lam a_2
#     r      = (mean_c D_c^2 + 1e-5)^(-1/2)                 (per token and head)
#     out    = (1 - lam_init) r D
#
# Backward, the forward's steps reversed (n = 2d channels per row):
#
#     dD     = (1 - lam_init) r (dout - r^2 D mean_c(dout_c D_c))
#     da_1   = dD,    da_2 = -lam dD,    dlam = -sum_rows <dD, a_2>
#     per map: the softmax-attention gradients of q_m, k_m and v (dv summed
#     over the two maps)
#     dlq1 = dlam e1 lk1,  dlk1 = dlam e1 lq1,  dlq2 = -dlam e2 lk2,
#     dlk2 = -dlam e2 lq2,   with e1 = exp(<lq1, lk1>), e2 = exp(<lq2, lk2>).


def _causal_map(q, k, softmax1):
    """One causal softmax map: q, k [T, d] -> P [T, T], lse2 [T] (log2 of the
    denominator of the log2(e)-scaled scores, max-shifted)."""
    T, d = q.shape
    S = q @ k.T / math.sqrt(d)
    S = np.where(np.triu(np.ones((T, T), dtype=bool), k=1), -np.inf, S)
    m = S.max(axis=1, keepdims=True)
    if softmax1:
        m = np.maximum(m, 0.0)
    e = np.exp(S - m)
    z = e.sum(axis=1, keepdims=True) + (np.exp(-m) if softmax1 else 0.0)
    return e / z, (m[:, 0] + np.log(z[:, 0])) / math.log(2.0)


def _v1_args(q1, q2, k1, k2, v, lq1, lk1, lq2, lk2, layer):
    t = [_f64(x) for x in (q1, q2, k1, k2, v, lq1, lk1, lq2, lk2)]
    li = lambda_init(layer)
    e1, e2 = math.exp(float(t[5] @ t[6])), math.exp(float(t[7] @ t[8]))
    return t, li, e1, e2, e1 - e2 + li


def v1_fwd_train(q1, q2, k1, k2, v, lq1, lk1, lq2, lk2, layer: int, softmax1: bool = False):
    """DIFF V1 forward keeping what the backward needs.

    q1, q2, k1, k2 [B,H,T,d], v [B,H,T,2d], lambda vectors [d] ->
    (out [B,T,H,2d], a1 [B,T,H,2d], a2 [B,T,H,2d], lse2 [2,B,H,T]), float64;
    a_m is map m's normalised attention output, lse2[m-1] its rows' log2
    denominators.
    """
    (q1, q2, k1, k2, v, *_), li, _, _, lam = _v1_args(q1, q2, k1, k2, v, lq1, lk1, lq2, lk2, layer)
    B, H, T, d = q1.shape
    a = np.zeros((2, B, T, H, 2 * d))
    lse2 = np.zeros((2, B, H, T))
    for b in range(B):
        for h in range(H):
            for m, (q, k) in enumerate(((q1, k1), (q2, k2))):
                P, lse2[m, b, h] = _causal_map(q[b, h], k[b, h], softmax1)
                a[m, b, :, h] = P @ v[b, h]
    D = a[0] - lam * a[1]
    r = 1.0 / np.sqrt((D * D).mean(axis=-1, keepdims=True) + 1e-5)
    return (1.0 - li) * r * D, a[0], a[1], lse2


def v1_bwd(q1, q2, k1, k2, v, lq1, lk1, lq2, lk2, layer: int, dout, softmax1: bool = False):
    """Gradients of sum(dout * out) for DIFF V1.

    Returns (dq1, dq2, dk1, dk2 [B,H,T,d], dv [B,H,T,2d], dlq1, dlk1, dlq2,
    dlk2 [d]), float64.
    """
    t, li, e1, e2, lam = _v1_args(q1, q2, k1, k2, v, lq1, lk1, lq2, lk2, layer)
    q1, q2, k1, k2, v, lq1, lk1, lq2, lk2 = t
    dout = _f64(dout)
    B, H, T, d = q1.shape
    qs, ks = (q1, q2), (k1, k2)
    dq = [np.zeros_like(q1), np.zeros_like(q2)]
    dk = [np.zeros_like(k1), np.zeros_like(k2)]
    dv = np.zeros_like(v)
    dlam = 0.0
    for b in range(B):
        for h in range(H):
            P, a = [], []
            for m in range(2):
                Pm, _ = _causal_map(qs[m][b, h], ks[m][b, h], softmax1)
                P.append(Pm)
                a.append(Pm @ v[b, h])
            D = a[0] - lam * a[1]                                    # [T, 2d]
            r = 1.0 / np.sqrt((D * D).mean(axis=1, keepdims=True) + 1e-5)
            g = dout[b, :, h]                                        # [T, 2d]
            dD = (1.0 - li) * r * (g - r * r * D * (g * D).mean(axis=1, keepdims=True))
            dlam -= float((dD * a[1]).sum())
            for m, da in enumerate((dD, -lam * dD)):
                dP = da @ v[b, h].T
                dS = P[m] * (dP - (P[m] * dP).sum(axis=1, keepdims=True))
                dq[m][b, h] = dS @ ks[m][b, h] / math.sqrt(d)
                dk[m][b, h] = dS.T @ qs[m][b, h] / math.sqrt(d)
                dv[b, h] += P[m].T @ da
    return (dq[0], dq[1], dk[0], dk[1], dv,
            dlam * e1 * lk1, dlam * e1 * lq1, -dlam * e2 * lk2, -dlam * e2 * lq2)


def v1_bwd_rounding_bounds(q1, q2, k1, k2, v, lq1, lk1, lq2, lk2, layer: int, dout, softmax1: bool = False,
                           rss: bool = True):
    """Per-element scale of what bf16 rounding can move in each gradient of
    :func:`v1_bwd`, for a path that keeps a_1, a_2 in bf16 (the training
    forward's outputs), rebuilds D from them, holds da_m, P and dS in bf16
    and accumulates in fp32 (relative rounding u = 2^-9 per rounded value).

    Followed through the same steps, to first order:
      dD_e   <- the RMSNorm backward's derivative with respect to D applied
                to |delta D| = u (|a_1| + |lam| |a_2|), plus u |dD| (rounding)
      da_m   <- eps_m = (1, |lam|)_m times that
      D_m,i  <- <eps_m,i, |a_m,i|> + u <|da_m,i|, |a_m,i|>
      dS_ij  <- P_ij (<eps_m,i, |v_j|> + err D_m,i) + u |dS_ij|
      dq, dk <- |err dS| times |k| or |q| over sqrt d;  dv <- P^T (eps_m + 2u |da_m|)
      dlam   <- sum_rows <|err dD|, |a_2|> + u <|dD|, |a_2|>;  the vectors scale by e |lambda vector|
    With ``rss=False`` every sum over an index adds absolute values (a
    worst case: all roundings aligned); with ``rss=True`` (default) it takes
    the root of the sum of squares, the typical size when the roundings are
    independent (each contraction then grows like sqrt(n), not n).
    Returns arrays shaped like :func:`v1_bwd`'s results.
    """
    t, li, e1, e2, lam = _v1_args(q1, q2, k1, k2, v, lq1, lk1, lq2, lk2, layer)
    q1, q2, k1, k2, v, lq1, lk1, lq2, lk2 = t
    dout = _f64(dout)
    u = 2.0 ** -9
    B, H, T, d = q1.shape
    n = 2 * d
    c = 1.0 - li
    if rss:
        agg = lambda x: np.sqrt((x * x).sum(axis=1, keepdims=True))
        mm = lambda x, y: np.sqrt((x * x) @ (y * y))
        tot = lambda x: float(np.sqrt((x * x).sum()))
    else:
        agg = lambda x: x.sum(axis=1, keepdims=True)
        mm = lambda x, y: x @ y
        tot = lambda x: float(x.sum())
    qs, ks = (q1, q2), (k1, k2)
    bq = [np.zeros_like(q1), np.zeros_like(q2)]
    bk = [np.zeros_like(k1), np.zeros_like(k2)]
    bv = [np.zeros_like(v) for _ in range(B * H)]
    lam_terms = []
    for b in range(B):
        for h in range(H):
            P, a = [], []
            for m in range(2):
                Pm, _ = _causal_map(qs[m][b, h], ks[m][b, h], softmax1)
                P.append(Pm)
                a.append(Pm @ v[b, h])
            D = a[0] - lam * a[1]
            r = 1.0 / np.sqrt((D * D).mean(axis=1, keepdims=True) + 1e-5)
            g = dout[b, :, h]
            gm = (g * D).mean(axis=1, keepdims=True)
            dD = c * r * (g - r * r * D * gm)
            dlt = u * (np.abs(a[0]) + abs(lam) * np.abs(a[1]))      # |delta D|
            S1 = agg(np.abs(D) * dlt)
            S2 = agg(np.abs(g) * dlt)
            r3 = r ** 3
            err_dD = (c * r3 * np.abs(g) * S1 / n + 3 * c * r ** 5 * np.abs(D) * np.abs(gm) * S1 / n
                      + c * r3 * np.abs(gm) * dlt + c * r3 * np.abs(D) * S2 / n)
            lam_terms.append(err_dD * np.abs(a[1]) + u * np.abs(dD) * np.abs(a[1]))
            acc_v = np.zeros_like(v[b, h]) if not rss else None
            sq_v = np.zeros_like(v[b, h])
            for m, (wt, da) in enumerate(((1.0, dD), (abs(lam), -lam * dD))):
                eps = wt * (err_dD + u * np.abs(dD))
                dP = da @ v[b, h].T
                dS = P[m] * (dP - (P[m] * dP).sum(axis=1, keepdims=True))
                errD = agg(eps * np.abs(a[m])) + u * agg(np.abs(da) * np.abs(a[m]))
                W = P[m] * (mm(eps, np.abs(v[b, h]).T) + errD) + u * np.abs(dS)
                bq[m][b, h] = mm(W, np.abs(ks[m][b, h])) / math.sqrt(d)
                bk[m][b, h] = mm(W.T, np.abs(qs[m][b, h])) / math.sqrt(d)
                x = mm(P[m].T, eps + 2 * u * np.abs(da))
                if rss:
                    sq_v += x * x
                else:
                    acc_v += x
            bv[b * H + h] = np.sqrt(sq_v) if rss else acc_v
    dvb = np.stack(bv).reshape(v.shape)
    blam = tot(np.stack(lam_terms))
    return (bq[0], bq[1], bk[0], bk[1], dvb,
            blam * e1 * np.abs(lk1), blam * e1 * np.abs(lq1), blam * e2 * np.abs(lk2), blam * e2 * np.abs(lq2))
