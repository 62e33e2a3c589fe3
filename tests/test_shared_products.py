"""The backward kernels' reformulation, checked in fp64 on the CPU against
the oracle's chain rule (oracle/backward.py).

The kernels do not form d attn / dP per head or map.  They use that the
attention outputs enter the result linearly:

* DIFF V2 ("Differential Transformer V2" article, DiffAttnV2 pseudo-code):
  d attn_2p = dout_p and d attn_2p+1 = c dout_p with c = -sigmoid(lam) per
  row, so with G = dout_p v^T and E_h = rowsum(dout_p o attn_h)
      dS_2p = P_2p (G - E_2p),   dS_2p+1 = c P_2p+1 (G - E_2p+1),
      dv   += (P_2p + c P_2p+1)^T dout_p    (one product per pair).
* DIFF V1 (the same article, DiffAttnV1 pseudo-code, with the RMSNorm of
  Wilsontomass's module in the nanoGPT issue "How best to implement a
  differential transformer?"): d a_1 = dD and d a_2 = c dD with c = -lam, so
  with G = dD v^T (over the 2d channels) and E_m = rowsum(dD o a_m)
      dS_1 = P_1 (G - E_1),   dS_2 = c P_2 (G - E_2),
      dv = (P_1 + c P_2)^T dD.
P is rebuilt from the kept log-sum-exp (P = exp2(S log2(e)/sqrt(d) - lse)),
as the kernels do.  Both sides are fp64, so they agree to rounding.
"""
import math

import numpy as np
import pytest

from oracle import backward as ob
from oracle import lambda_init

rng = np.random.default_rng(20261202)


def _p_from_lse(q, k, lse2):
    T, d = q.shape
    s = q @ k.T / math.sqrt(d)
    p = np.exp2(s * math.log2(math.e) - lse2[:, None])
    return np.where(np.tril(np.ones((T, T), dtype=bool)), p, 0.0)


@pytest.mark.parametrize("softmax1", [False, True])
def test_v2_pair_shares_g_and_dv(softmax1):
    B, T, Hq, Hkv, d = 2, 9, 8, 2, 8
    G_ = Hq // Hkv
    q = rng.standard_normal((B, T, Hq, d))
    k = rng.standard_normal((B, T, Hkv, d))
    v = rng.standard_normal((B, T, Hkv, d))
    lam = rng.standard_normal((B, T, Hq // 2))
    dout = rng.standard_normal((B, T, Hq // 2, d))
    ref = ob.v2_bwd(q, k, v, lam, dout, softmax1=softmax1)
    _, attn, lse2 = ob.v2_fwd_train(q, k, v, lam, softmax1=softmax1)
    dq, dk, dv = np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)
    for b in range(B):
        for p in range(Hq // 2):
            g = (2 * p) // G_
            c = -1.0 / (1.0 + np.exp(-lam[b, :, p]))                   # [T]
            Gm = dout[b, :, p] @ v[b, :, g].T                            # one product per pair
            Pp = [_p_from_lse(q[b, :, 2 * p + e], k[b, :, g], lse2[b, 2 * p + e]) for e in range(2)]
            E = [(dout[b, :, p] * attn[b, :, 2 * p + e]).sum(axis=1) for e in range(2)]
            dS = [Pp[0] * (Gm - E[0][:, None]), c[:, None] * Pp[1] * (Gm - E[1][:, None])]
            for e in range(2):
                dq[b, :, 2 * p + e] = dS[e] @ k[b, :, g] / math.sqrt(d)
                dk[b, :, g] += dS[e].T @ q[b, :, 2 * p + e] / math.sqrt(d)
            dv[b, :, g] += (Pp[0] + c[:, None] * Pp[1]).T @ dout[b, :, p]
    for got, want in zip((dq, dk, dv), ref[:3]):
        np.testing.assert_allclose(got, want, rtol=1e-10, atol=1e-12)


@pytest.mark.parametrize("softmax1", [False, True])
def test_v1_maps_share_g_and_dv(softmax1):
    B, H, T, d, layer = 2, 2, 9, 8, 5
    q1, q2, k1, k2 = (rng.standard_normal((B, H, T, d)) for _ in range(4))
    v = rng.standard_normal((B, H, T, 2 * d))
    lq1, lk1, lq2, lk2 = (0.1 * rng.standard_normal(d) for _ in range(4))
    dout = rng.standard_normal((B, T, H, 2 * d))
    ref = ob.v1_bwd(q1, q2, k1, k2, v, lq1, lk1, lq2, lk2, layer, dout, softmax1=softmax1)
    _, a1, a2, lse2 = ob.v1_fwd_train(q1, q2, k1, k2, v, lq1, lk1, lq2, lk2, layer, softmax1=softmax1)
    li = lambda_init(layer)
    lam = math.exp(lq1 @ lk1) - math.exp(lq2 @ lk2) + li
    c = -lam
    qs, ks = (q1, q2), (k1, k2)
    dq = [np.zeros_like(q1), np.zeros_like(q2)]
    dk = [np.zeros_like(k1), np.zeros_like(k2)]
    dv = np.zeros_like(v)
    for b in range(B):
        for h in range(H):
            a = (a1[b, :, h], a2[b, :, h])
            D = a[0] - lam * a[1]
            r = 1.0 / np.sqrt((D * D).mean(axis=1, keepdims=True) + 1e-5)
            g = dout[b, :, h]
            dD = (1.0 - li) * r * (g - r * r * D * (g * D).mean(axis=1, keepdims=True))
            Gm = dD @ v[b, h].T                                          # one product for both maps
            P = [_p_from_lse(qs[m][b, h], ks[m][b, h], lse2[m, b, h]) for m in range(2)]
            E = [(dD * a[m]).sum(axis=1) for m in range(2)]
            dS = [P[0] * (Gm - E[0][:, None]), c * P[1] * (Gm - E[1][:, None])]
            for m in range(2):
                dq[m][b, h] = dS[m] @ ks[m][b, h] / math.sqrt(d)
                dk[m][b, h] = dS[m].T @ qs[m][b, h] / math.sqrt(d)
            dv[b, h] = (P[0] + c * P[1]).T @ dD
    for got, want in zip((dq[0], dq[1], dk[0], dk[1], dv), ref[:5]):
        np.testing.assert_allclose(got, want, rtol=1e-10, atol=1e-12)
