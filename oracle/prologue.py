"""fp64 oracle for the steps just upstream of the attention that the library
fuses or runs next to it -- TEST INFRASTRUCTURE ONLY (the same rule as the
rest of ``oracle/``: only ``tests/``, ``__graft_entry__.smoke()`` and
``bench.py``'s ``cpu_baseline`` use it).

Rotary position embedding.  Wilsontomass's module in the nanoGPT issue "How
best to implement a differential transformer?" applies
``RotaryEmbedding(dim=head_dim)`` with ``apply_rotary_pos_emb`` to every q and
k head (both halves of each differential head) before the attention; the
bodies are not on the pages.  The plainest reading is the rotary embedding in
the rotate-half arrangement: element c < d/2 pairs with c + d/2 and the pair
turns by the angle t * w_c, w_c = theta^(-2c/d), at position t:

    x'_c       = x_c cos(t w_c) - x_{c+d/2} sin(t w_c)
    x'_{c+d/2} = x_{c+d/2} cos(t w_c) + x_c sin(t w_c)

(theta = 10000 unless given).  A score between positions s and t then
depends on s - t only.

V2 lambda projection.  The "Differential Transformer V2" article computes
lambda per token and per head with a projection it does not show; the
plainest reading is a linear map (no bias) of the token's
hidden state to one logit per output pair, ``logits[b, t, p] = <x[b, t, :],
W[p, :]>`` with W laid out like a linear layer's weight [pairs, d_model]; the
sigmoid stays where the DiffAttnV2 pseudo-code puts it.
"""
from __future__ import annotations

import numpy as np

from . import _f64, v1_fwd, v2_decode, v2_decode_paged, v2_fwd


def rope(x, theta: float = 10000.0, pos0: int = 0, axis_t: int = 1, positions=None):
    """Rotate the last axis (d, even) of x by position: token i of axis
    ``axis_t`` sits at position pos0 + i (or ``positions[i]``)."""
    x = _f64(x)
    d = x.shape[-1]
    h = d // 2
    T = x.shape[axis_t]
    pos = np.arange(T, dtype=np.float64) + pos0 if positions is None else np.asarray(positions, np.float64)
    w = theta ** (-2.0 * np.arange(h) / d)                  # [d/2]
    ang = pos[:, None] * w[None, :]                          # [T, d/2]
    shape = [1] * x.ndim
    shape[axis_t] = T
    shape[-1] = h
    c, s = np.cos(ang).reshape(shape), np.sin(ang).reshape(shape)
    x1, x2 = x[..., :h], x[..., h:]
    return np.concatenate([x1 * c - x2 * s, x2 * c + x1 * s], axis=-1)


def v1_fwd_rope(q1, q2, k1, k2, v, lq1, lk1, lq2, lk2, layer: int, theta: float = 10000.0, pos0: int = 0,
                softmax1: bool = False):
    """DIFF V1 forward with q1, q2, k1, k2 ([B,H,T,d]) rotated first."""
    r = lambda x: rope(x, theta, pos0, axis_t=2)
    return v1_fwd(r(q1), r(q2), r(k1), r(k2), v, lq1, lk1, lq2, lk2, layer, softmax1=softmax1)


def v2_fwd_rope(q, k, v, lam, theta: float = 10000.0, pos0: int = 0, softmax1: bool = False):
    """DIFF V2 prefill with q and k ([B,T,H,d]) rotated first."""
    return v2_fwd(rope(q, theta, pos0), rope(k, theta, pos0), v, lam, softmax1=softmax1)


def v2_decode_rope(q, k_cache, v_cache, lam, theta: float = 10000.0, softmax1: bool = False):
    """DIFF V2 decode of one new token per sequence whose q ([B,Hq,d]) is
    rotated to its position L - 1; the cache keys are taken as stored
    rotated (each at its own position), as a cache holds them."""
    L = k_cache.shape[1]
    qr = rope(_f64(q)[:, None], theta, L - 1, axis_t=1)[:, 0]
    return v2_decode(qr, k_cache, v_cache, lam, softmax1=softmax1)


def v2_decode_paged_rope(q, k_pages, v_pages, block_table, seq_lens, lam, theta: float = 10000.0,
                         softmax1: bool = False):
    """Paged decode with each sequence's nq new tokens ([B,Hq,d] or
    [B,nq,Hq,d]) rotated to their positions seq_len - nq + i."""
    q = _f64(q)
    q4 = q[:, None] if q.ndim == 3 else q
    nq = q4.shape[1]
    lens = np.asarray(seq_lens).astype(np.int64)
    qr = np.stack([rope(q4[b:b + 1], theta, axis_t=1, positions=lens[b] - nq + np.arange(nq))[0]
                   for b in range(q4.shape[0])])
    return v2_decode_paged(qr[:, 0] if q.ndim == 3 else qr, k_pages, v_pages, block_table, seq_lens, lam,
                           softmax1=softmax1)


def lambda_proj(x, w):
    """V2 lambda logits: x [B,T,dm], w [P,dm] -> [B,T,P] float64."""
    return _f64(x) @ _f64(w).T
