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


def v2_bwd_sampled(q, k, v, lam, dout, rows, keys, softmax1: bool = False):
    """The gradients of :func:`v2_bwd` at chosen places, for sizes where the
    dense per-head matrices are too slow: dq of the rows ``rows`` (an
    ``[n, 3]`` array of (b, t, query head)), dk and dv of the keys ``keys``
    (``[m, 3]`` of (b, j, kv head)), and dlam everywhere.

    The same chain rule, one row or one key at a time.  Each head's rows and
    log-sum-exp come from :func:`oracle.v2_heads` (the C forward), so that
    P_tj = exp(q_t . k_j / sqrt d - lse_t) for j <= t, and with
    d attn as in :func:`v2_bwd` and D_t = <d attn_t, attn_t> (= rowsum(P o dP)):
        dq_t  = sum_{j <= t} P_tj (d attn_t . v_j - D_t) k_j / sqrt d
        dk_j  = sum_{h in g} sum_{t >= j} P_tj (d attn_t . v_j - D_t) q_t / sqrt d
        dv_j  = sum_{h in g} sum_{t >= j} P_tj d attn_t
    Returns (dq [n, d], dk [m, d], dv [m, d], dlam [B, T, Hq/2]).
    """
    from . import v2_heads

    q, k, v, lam, dout = [_f64(x) for x in (q, k, v, lam, dout)]
    B, T, Hq, d = q.shape
    G = Hq // k.shape[2]
    rows = np.asarray(rows, dtype=np.int64).reshape(-1, 3)
    keys = np.asarray(keys, dtype=np.int64).reshape(-1, 3)
    attn, lse = v2_heads(q, k, v, softmax1=softmax1)
    sig = 1.0 / (1.0 + np.exp(-lam))  # [B, T, Hq/2]
    dlam = -sig * (1.0 - sig) * np.einsum("btpc,btpc->btp", dout, attn[:, :, 1::2])

    def d_attn(b, t, h):  # d attn of head h at rows t (t: int or array)
        g = dout[b, t, h // 2]
        return g if h % 2 == 0 else -sig[b, t, h // 2][..., None] * g

    sc = 1.0 / math.sqrt(d)
    dq = np.zeros((rows.shape[0], d))
    for n, (b, t, h) in enumerate(rows):
        g = h // G
        kj, vj = k[b, :t + 1, g], v[b, :t + 1, g]
        P = np.exp(kj @ q[b, t, h] * sc - lse[b, h, t])
        da = d_attn(b, t, h)
        dS = P * (vj @ da - da @ attn[b, t, h])
        dq[n] = dS @ kj * sc
    dk = np.zeros((keys.shape[0], d))
    dv = np.zeros((keys.shape[0], d))
    for n, (b, j, g) in enumerate(keys):
        for h in range(g * G, (g + 1) * G):
            ts = np.arange(j, T)
            qt = q[b, j:, h]
            P = np.exp(qt @ k[b, j, g] * sc - lse[b, h, j:])
            da = d_attn(b, ts, h)
            D = np.einsum("tc,tc->t", da, attn[b, j:, h])
            dS = P * (da @ v[b, j, g] - D)
            dk[n] += dS @ qt * sc
            dv[n] += P @ da
    return dq, dk, dv, dlam


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
