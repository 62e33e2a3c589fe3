"""Brute-force fp64 differential attention with explicit T x T maps (numpy).

A second, independent formulation used only to pin the oracle on tiny
inputs.  V1 works on whole maps: the two maps of a differential head are
stacked along a map axis and softmaxed together (scores masked with -inf
above the diagonal), their combination is a contraction of that axis with
the coefficient vector (1, -lambda) -- so the combined weights exist BEFORE
they meet V, as in the explicit-map form of notlober's module in the nanoGPT
issue "How best to implement a differential transformer?" -- and the RMSNorm
is written with a vector norm.  Two deviations of that module are not taken,
because the "Differential Transformer V2" article (DiffAttnV1 pseudo-code) is
the authority: the norm is RMSNorm (not LayerNorm with affine), and
lambda_init uses the layer's own index (not the layer count).

This shares no code with ``oracle/`` (which computes one softmax row at a
time, maps separately, and combines after P.V).
"""
import math

import numpy as np
from scipy.special import expit


def _causal_softmax(s: np.ndarray) -> np.ndarray:
    """Row softmax of ``s[..., T, T]`` with keys j > i masked to -inf."""
    T = s.shape[-1]
    mask = np.triu(np.ones((T, T), dtype=bool), k=1)
    s = np.where(mask, -np.inf, s)
    s = s - s.max(axis=-1, keepdims=True)
    e = np.exp(s)
    return e / e.sum(axis=-1, keepdims=True)


def v1(q1, q2, k1, k2, v, lq1, lk1, lq2, lk2, layer):
    """q*, k* [B,H,T,d]; v [B,H,T,2d]; returns [B,T,H,2d]."""
    d = q1.shape[-1]
    n = v.shape[-1]  # 2d channels
    li = 0.8 - 0.6 * math.exp(-0.3 * layer)
    coef = np.array([1.0, -(math.exp(float(lq1 @ lk1)) - math.exp(float(lq2 @ lk2)) + li)])
    Q = np.stack([q1, q2], axis=2)  # [B,H,2,T,d]: the maps side by side
    K = np.stack([k1, k2], axis=2)
    A = _causal_softmax(np.einsum("bhmic,bhmjc->bhmij", Q, K) / math.sqrt(d))
    W = np.einsum("m,bhmij->bhij", coef, A)  # differential weights, [B,H,T,T]
    D = np.einsum("bhij,bhjc->bihc", W, v)  # [B,T,H,2d]
    rms = np.linalg.norm(D, axis=-1, keepdims=True) / math.sqrt(n)
    return (1.0 - li) * D / np.sqrt(rms * rms + 1e-5)


def _gqa_attention(q, k, v, causal=True):
    """q [B,Tq,Hq,d], k/v [B,Tk,Hkv,d] -> [B,Tq,Hq,d]; head h uses kv head
    h // (Hq/Hkv).  causal masks j > i (Tq == Tk); otherwise all keys."""
    B, Tq, Hq, d = q.shape
    Hkv = k.shape[2]
    G = Hq // Hkv
    kr = np.repeat(k, G, axis=2)  # [B,Tk,Hq,d]
    vr = np.repeat(v, G, axis=2)
    qh = np.transpose(q, (0, 2, 1, 3))
    kh = np.transpose(kr, (0, 2, 1, 3))
    vh = np.transpose(vr, (0, 2, 1, 3))
    s = qh @ np.swapaxes(kh, -1, -2) / math.sqrt(d)
    if causal:
        a = _causal_softmax(s)
    else:
        s = s - s.max(axis=-1, keepdims=True)
        e = np.exp(s)
        a = e / e.sum(axis=-1, keepdims=True)
    return np.transpose(a @ vh, (0, 2, 1, 3))


def v2(q, k, v, lam):
    """q [B,T,Hq,d], k/v [B,T,Hkv,d], lam [B,T,Hq/2] -> [B,T,Hq/2,d]."""
    a = _gqa_attention(q, k, v, causal=True)
    return a[:, :, 0::2] - expit(lam)[..., None] * a[:, :, 1::2]


def v2_decode(q, k, v, lam):
    """q [B,Hq,d], k/v [B,L,Hkv,d], lam [B,Hq/2] -> [B,Hq/2,d]; the query
    sees every cache entry."""
    a = _gqa_attention(q[:, None], k, v, causal=False)[:, 0]
    return a[:, 0::2] - expit(lam)[..., None] * a[:, 1::2]


def v2_decode_paged(q, k_pages, v_pages, block_table, seq_lens, lam):
    """Paged decode, one sequence and one token at a time: walk the page
    table entry by entry (page j holds tokens j*P .. j*P + P - 1), copy each
    stored row out, then decode the dense copy with :func:`v2_decode`.
    A sequence of length 0 gives 0."""
    B, Hq, d = q.shape
    P, Hkv = k_pages.shape[1], k_pages.shape[2]
    out = np.zeros((B, Hq // 2, d))
    for b in range(B):
        L = int(seq_lens[b])
        if L == 0:
            continue
        k = np.zeros((L, Hkv, d))
        v = np.zeros((L, Hkv, d))
        for j in range((L + P - 1) // P):
            page = int(block_table[b][j])
            for r in range(P):
                t = j * P + r
                if t < L:
                    k[t] = k_pages[page][r]
                    v[t] = v_pages[page][r]
        out[b] = v2_decode(q[b:b + 1], k[None], v[None], lam[b:b + 1])[0]
    return out
