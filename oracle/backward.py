"""fp64 oracle for the DIFF V2 training step: forward with the quantities a
backward pass keeps, and the gradients -- TEST INFRASTRUCTURE ONLY (the same
rule as the rest of ``oracle/``: only ``tests/``, ``__graft_entry__.smoke()``
and ``bench.py``'s ``cpu_baseline`` use it).

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

from . import _f64


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
