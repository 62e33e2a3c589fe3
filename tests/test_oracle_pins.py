"""Pins for the fp64 oracle: checks against things other than the oracle itself.

The pages print no worked numerical example for this method, so every pin is
constructed from what the pages and the mathematics fix:

* brute force: an independent explicit-map formulation (tests/bruteforce.py)
  on tiny hypothesis-drawn shapes;
* library routines: torch's scaled_dot_product_attention and rms_norm (fp64,
  CPU) where the method reduces to plain causal attention (lambda = 0,
  sigmoid = 0, identical branches);
* closed forms: T = 1, uniform attention (Q = 0 gives prefix means), needle
  keys on and just past the diagonal, lambda_init special values;
* invariants: odd symmetry in V, linearity of V2 in V, batch permutation,
  GQA group mapping.
"""
import math
from decimal import Decimal, getcontext

import numpy as np
import pytest
import torch
import torch.nn.functional as F
from hypothesis import given, settings, strategies as st

import bruteforce
import oracle

RTOL = 1e-12


def _rng(seed):
    return np.random.default_rng(seed)


def _v1_case(rng, B, H, T, d, lam_std=0.1):
    q1, q2, k1, k2 = (rng.standard_normal((B, H, T, d)) for _ in range(4))
    v = rng.standard_normal((B, H, T, 2 * d))
    lams = [lam_std * rng.standard_normal(d) for _ in range(4)]
    return q1, q2, k1, k2, v, lams


def _v2_case(rng, B, T, Hq, Hkv, d):
    q = rng.standard_normal((B, T, Hq, d))
    k = rng.standard_normal((B, T, Hkv, d))
    v = rng.standard_normal((B, T, Hkv, d))
    lam = rng.standard_normal((B, T, Hq // 2))
    return q, k, v, lam


def _close(a, b, rtol=RTOL, atol=1e-13):
    np.testing.assert_allclose(a, b, rtol=rtol, atol=atol)


# --------------------------------------------------------------------------
# lambda_init = 0.8 - 0.6 exp(-0.3 layer)  ("Differential Transformer V2",
# DiffAttnV1; Hacker News item 41780844, the quoted constant)
# --------------------------------------------------------------------------

def test_lambda_init_special_values():
    assert abs(oracle.lambda_init(0) - 0.2) < 1e-15  # 0.8 - 0.6 * e^0
    assert abs(oracle.lambda_init(400) - 0.8) < 1e-15  # decays to 0.8
    vals = [oracle.lambda_init(l) for l in range(40)]
    assert all(a < b for a, b in zip(vals, vals[1:]))  # increasing in depth
    assert all(0.2 <= x < 0.8 for x in vals)


def test_lambda_init_geometric_gap_decimal():
    """The gap to 0.8 shrinks by e^-0.3 per layer; e^-0.3 comes from Python's
    decimal module, an exp implementation independent of libm."""
    getcontext().prec = 40
    ratio = float(Decimal("-0.3").exp())
    for l in range(30):
        g0 = 0.8 - oracle.lambda_init(l)
        g1 = 0.8 - oracle.lambda_init(l + 1)
        assert abs(g1 / g0 - ratio) < 1e-12
    for l in range(16):
        ref = Decimal("0.8") - Decimal("0.6") * (Decimal(-3 * l) / Decimal(10)).exp()
        assert abs(oracle.lambda_init(l) - float(ref)) < 1e-15


def test_v1_lambda_special_cases():
    rng = _rng(0)
    d = 8
    z = np.zeros(d)
    for layer in (0, 3, 11):
        li = oracle.lambda_init(layer)
        # all-zero vectors: exp(0) - exp(0) + li
        assert abs(oracle.v1_lambda(z, z, z, z, layer) - li) < 1e-15
        # identical pairs cancel
        a, b = rng.standard_normal(d), rng.standard_normal(d)
        assert abs(oracle.v1_lambda(a, b, a, b, layer) - li) < 1e-14
    # one active coordinate: exp(2*3) - exp(0) + li(2)
    a = np.zeros(d); a[5] = 2.0
    b = np.zeros(d); b[5] = 3.0
    assert abs(oracle.v1_lambda(a, b, z, z, 2) - (math.exp(6.0) - 1.0 + oracle.lambda_init(2))) < 1e-11
    # sign: the second exponential is subtracted
    assert abs(oracle.v1_lambda(z, z, a, b, 2) - (1.0 - math.exp(6.0) + oracle.lambda_init(2))) < 1e-11


# --------------------------------------------------------------------------
# brute force on tiny shapes
# --------------------------------------------------------------------------

@settings(max_examples=40, deadline=None)
@given(B=st.integers(1, 2), H=st.integers(1, 3), T=st.sampled_from([1, 2, 3, 7, 16, 33]),
       d=st.sampled_from([4, 8, 32]), layer=st.integers(0, 20), seed=st.integers(0, 10**6))
def test_v1_matches_bruteforce(B, H, T, d, layer, seed):
    q1, q2, k1, k2, v, lams = _v1_case(_rng(seed), B, H, T, d, lam_std=0.3)
    got = oracle.v1_fwd(q1, q2, k1, k2, v, *lams, layer)
    ref = bruteforce.v1(q1, q2, k1, k2, v, *lams, layer)
    _close(got, ref, rtol=1e-10, atol=1e-11)


@settings(max_examples=40, deadline=None)
@given(B=st.integers(1, 2), T=st.sampled_from([1, 2, 5, 16, 33]), Hkv=st.integers(1, 3),
       G=st.sampled_from([2, 4]), d=st.sampled_from([4, 8, 16]), seed=st.integers(0, 10**6))
def test_v2_matches_bruteforce(B, T, Hkv, G, d, seed):
    q, k, v, lam = _v2_case(_rng(seed), B, T, G * Hkv, Hkv, d)
    _close(oracle.v2_fwd(q, k, v, lam), bruteforce.v2(q, k, v, lam))


@settings(max_examples=30, deadline=None)
@given(B=st.integers(1, 3), L=st.sampled_from([1, 2, 9, 64, 100]), Hkv=st.integers(1, 3),
       G=st.sampled_from([2, 4, 8]), d=st.sampled_from([4, 16]), seed=st.integers(0, 10**6))
def test_decode_matches_bruteforce(B, L, Hkv, G, d, seed):
    rng = _rng(seed)
    Hq = G * Hkv
    q = rng.standard_normal((B, Hq, d))
    k = rng.standard_normal((B, L, Hkv, d))
    v = rng.standard_normal((B, L, Hkv, d))
    lam = rng.standard_normal((B, Hq // 2))
    _close(oracle.v2_decode(q, k, v, lam), bruteforce.v2_decode(q, k, v, lam))


# --------------------------------------------------------------------------
# reductions to plain causal attention (torch SDPA + rms_norm, fp64, CPU)
# --------------------------------------------------------------------------

def _sdpa(q, k, v):
    """Causal SDPA with torch's default 1/sqrt(E) scale; q,k [.., T, E], v [.., T, Ev]."""
    t = [torch.from_numpy(np.ascontiguousarray(x)) for x in (q, k, v)]
    return F.scaled_dot_product_attention(*t, is_causal=True).numpy()


def _rmsnorm(x):
    t = torch.from_numpy(np.ascontiguousarray(x))
    return F.rms_norm(t, (t.shape[-1],), eps=1e-5).numpy()


@pytest.mark.parametrize("layer", [0, 3, 14])
def test_v1_lambda_zero_is_plain_attention(layer):
    """lambda = 0 (lq1 = 0, lq2 = lk2 = c*1 with d c^2 = ln(1 + li)): the
    output is (1 - li) * RMSNorm(SDPA(Q1, K1, V))."""
    rng = _rng(1 + layer)
    B, H, T, d = 2, 3, 29, 16
    q1, q2, k1, k2, v, lams = _v1_case(rng, B, H, T, d)
    li = oracle.lambda_init(layer)
    c = math.sqrt(math.log(1.0 + li) / d)
    lq1, lk1 = np.zeros(d), rng.standard_normal(d)
    lq2 = lk2 = np.full(d, c)
    assert abs(oracle.v1_lambda(lq1, lk1, lq2, lk2, layer)) < 1e-14
    got = oracle.v1_fwd(q1, q2, k1, k2, v, lq1, lk1, lq2, lk2, layer)
    ref = (1.0 - li) * _rmsnorm(_sdpa(q1, k1, v))  # [B,H,T,2d]
    _close(got, np.transpose(ref, (0, 2, 1, 3)), rtol=1e-10, atol=1e-12)


def test_v1_identical_branches():
    """Q2 = Q1, K2 = K1: the two maps coincide and A - lambda*A = (1 - lambda)*A
    (Hacker News "Differential Transformer" board, post #131), so the output is
    (1 - li) * RMSNorm((1 - lambda) * SDPA(Q1, K1, V))."""
    rng = _rng(7)
    B, H, T, d, layer = 1, 2, 40, 8, 5
    q1, _, k1, _, v, lams = _v1_case(rng, B, H, T, d, lam_std=0.4)
    lam = oracle.v1_lambda(*lams, layer)
    assert abs(1.0 - lam) > 0.05
    li = oracle.lambda_init(layer)
    got = oracle.v1_fwd(q1, q1, k1, k1, v, *lams, layer)
    ref = (1.0 - li) * _rmsnorm((1.0 - lam) * _sdpa(q1, k1, v))
    _close(got, np.transpose(ref, (0, 2, 1, 3)), rtol=1e-10, atol=1e-12)


def test_v2_sigmoid_zero_is_plain_gqa_attention():
    """lam = -inf gives sigmoid = 0 exactly: out[:, :, p] = SDPA(q_{2p}, K_g, V_g)
    with g = 2p // (Hq/Hkv)."""
    rng = _rng(3)
    B, T, Hq, Hkv, d = 2, 23, 8, 2, 16
    q, k, v, _ = _v2_case(rng, B, T, Hq, Hkv, d)
    lam = np.full((B, T, Hq // 2), -np.inf)
    got = oracle.v2_fwd(q, k, v, lam)
    G = Hq // Hkv
    for p in range(Hq // 2):
        h, g = 2 * p, (2 * p) // G
        ref = _sdpa(q[:, :, h].transpose(0, 1, 2)[:, None], k[:, :, g][:, None], v[:, :, g][:, None])[:, 0]
        _close(got[:, :, p], ref)


def test_v2_identical_heads_and_full_gate():
    """q_{2p+1} = q_{2p}: out = (1 - sigmoid(lam)) * a_{2p}; with lam = +inf the
    pair cancels to exactly zero."""
    rng = _rng(4)
    B, T, Hq, Hkv, d = 1, 17, 4, 1, 8
    q, k, v, lam = _v2_case(rng, B, T, Hq, Hkv, d)
    q[:, :, 1::2] = q[:, :, 0::2]
    got = oracle.v2_fwd(q, k, v, lam)
    a = np.stack([_sdpa(q[:, None, :, 2 * p], k[:, None, :, 0], v[:, None, :, 0])[:, 0]
                  for p in range(Hq // 2)], axis=2)
    sig = 1.0 / (1.0 + np.exp(-lam))
    _close(got, (1.0 - sig)[..., None] * a)
    zero = oracle.v2_fwd(q, k, v, np.full_like(lam, np.inf))
    assert np.array_equal(zero, np.zeros_like(zero))


# --------------------------------------------------------------------------
# closed forms
# --------------------------------------------------------------------------

def test_t1_closed_forms():
    """T = 1: each map returns v_0, so V1 gives (1-li)(1-lam)v0 /
    sqrt((1-lam)^2 mean(v0^2) + 1e-5) and V2 gives (1 - sigmoid) v0."""
    rng = _rng(5)
    d, layer = 16, 9
    q1, q2, k1, k2, v, lams = _v1_case(rng, 2, 3, 1, d, lam_std=0.5)
    lam = oracle.v1_lambda(*lams, layer)
    li = oracle.lambda_init(layer)
    got = oracle.v1_fwd(q1, q2, k1, k2, v, *lams, layer)[:, 0]  # [B,H,2d]
    v0 = v[:, :, 0]
    ref = (1 - li) * (1 - lam) * v0 / np.sqrt((1 - lam) ** 2 * np.mean(v0 * v0, -1, keepdims=True) + 1e-5)
    _close(got, ref)
    q, k, vv, lg = _v2_case(rng, 2, 1, 8, 2, d)
    got2 = oracle.v2_fwd(q, k, vv, lg)[:, 0]  # [B,P,d]
    sig = 1.0 / (1.0 + np.exp(-lg[:, 0]))
    ref2 = (1 - sig)[..., None] * np.repeat(vv[:, 0], 2, axis=1)  # pairs 0,1 -> group 0; 2,3 -> 1
    _close(got2, ref2)


def test_uniform_attention_prefix_mean():
    """Q = 0: every visible score is 0, each row is uniform over j <= i and A.V
    is the prefix mean of V."""
    rng = _rng(6)
    B, H, T, d, layer = 1, 2, 50, 8, 4
    _, _, k1, k2, v, lams = _v1_case(rng, B, H, T, d, lam_std=0.3)
    z = np.zeros((B, H, T, d))
    lam = oracle.v1_lambda(*lams, layer)
    li = oracle.lambda_init(layer)
    pm = np.cumsum(v, axis=2) / np.arange(1, T + 1)[None, None, :, None]
    D = (1 - lam) * pm
    ref = (1 - li) * D / np.sqrt(np.mean(D * D, -1, keepdims=True) + 1e-5)
    _close(oracle.v1_fwd(z, z, k1, k2, v, *lams, layer), np.transpose(ref, (0, 2, 1, 3)))
    q, k, vv, lg = _v2_case(rng, 2, 37, 8, 2, d)
    pm2 = np.cumsum(vv, axis=1) / np.arange(1, 38)[None, :, None, None]  # [B,T,Hkv,d]
    sig = 1.0 / (1.0 + np.exp(-lg))
    ref2 = (1 - sig)[..., None] * np.repeat(pm2, 2, axis=2)
    _close(oracle.v2_fwd(np.zeros_like(q), k, vv, lg), ref2)


@pytest.mark.parametrize("offset,visible", [(0, True), (1, False)])
def test_needle_on_and_past_the_diagonal(offset, visible):
    """Query i = a*e0, key i+offset = e0, every other key has coordinate 0 = 0.
    On the diagonal (offset 0) the map is one-hot at key i (error ~e^-40);
    one past it (offset 1) the key is masked and the row is uniform."""
    d, T = 8, 24
    rng = _rng(10 + offset)
    alpha = 40.0 * math.sqrt(d)
    q = np.zeros((1, 1, T, d)); k = rng.standard_normal((1, 1, T, d)); k[..., 0] = 0.0
    v = rng.standard_normal((1, 1, T, 2 * d))
    i = 11
    q[0, 0, i, 0] = alpha
    k[0, 0, i + offset] = 0.0
    k[0, 0, i + offset, 0] = 1.0
    z = np.zeros(d)
    li = oracle.lambda_init(0)
    # lambda = li with zero vectors; second map uses q2 = 0 (uniform)
    out = oracle.v1_fwd(q, np.zeros_like(q), k, k, v, z, z, z, z, 0)[0, i, 0]
    a1 = v[0, 0, i] if visible else v[0, 0, : i + 1].mean(axis=0)
    D = a1 - li * v[0, 0, : i + 1].mean(axis=0)
    ref = (1 - li) * D / math.sqrt(np.mean(D * D) + 1e-5)
    _close(out, ref, rtol=1e-9, atol=1e-12)


# --------------------------------------------------------------------------
# invariants
# --------------------------------------------------------------------------

def test_v1_odd_symmetry_and_scale():
    rng = _rng(8)
    q1, q2, k1, k2, v, lams = _v1_case(rng, 1, 2, 20, 8)
    a = oracle.v1_fwd(q1, q2, k1, k2, v, *lams, 2)
    b = oracle.v1_fwd(q1, q2, k1, k2, -v, *lams, 2)
    assert np.array_equal(a, -b)  # exact: every step is odd in V
    # RMSNorm removes the scale of V up to eps: at x1000 and x2000 the eps
    # term is ~1e-11 of mean(D^2), so the two agree to ~1e-11.
    c = oracle.v1_fwd(q1, q2, k1, k2, 1000.0 * v, *lams, 2)
    e = oracle.v1_fwd(q1, q2, k1, k2, 2000.0 * v, *lams, 2)
    _close(c, e, rtol=1e-9, atol=1e-10)
    assert np.max(np.abs(c - a)) > 1e-7  # while at scale 1 eps is visible


def test_v2_linear_in_v():
    rng = _rng(9)
    q, k, v, lam = _v2_case(rng, 1, 19, 4, 2, 8)
    w = rng.standard_normal(v.shape)
    lhs = oracle.v2_fwd(q, k, 2.0 * v - 3.0 * w, lam)
    rhs = 2.0 * oracle.v2_fwd(q, k, v, lam) - 3.0 * oracle.v2_fwd(q, k, w, lam)
    _close(lhs, rhs, rtol=1e-10, atol=1e-12)


def test_v2_gqa_group_mapping():
    """Heads of one GQA group are contiguous: with V_g = (g+1) everywhere and
    sigmoid = 0, pair p reads group (2p) // (Hq/Hkv)."""
    rng = _rng(11)
    B, T, Hq, Hkv, d = 1, 9, 12, 3, 4
    q, k, _, _ = _v2_case(rng, B, T, Hq, Hkv, d)
    v = np.ones((B, T, Hkv, d)) * (np.arange(Hkv) + 1.0)[None, None, :, None]
    out = oracle.v2_fwd(q, k, v, np.full((B, T, Hq // 2), -np.inf))
    G = Hq // Hkv
    for p in range(Hq // 2):
        _close(out[:, :, p], np.full((B, T, d), (2 * p) // G + 1.0))


def test_batch_permutation():
    rng = _rng(12)
    q1, q2, k1, k2, v, lams = _v1_case(rng, 3, 2, 12, 8)
    perm = [2, 0, 1]
    a = oracle.v1_fwd(q1, q2, k1, k2, v, *lams, 1)
    b = oracle.v1_fwd(q1[perm], q2[perm], k1[perm], k2[perm], v[perm], *lams, 1)
    assert np.array_equal(a[perm], b)


def test_decode_equals_last_prefill_row():
    rng = _rng(13)
    q, k, v, lam = _v2_case(rng, 2, 31, 8, 2, 8)
    full = oracle.v2_fwd(q, k, v, lam)
    dec = oracle.v2_decode(q[:, -1], k, v, lam[:, -1])
    _close(dec, full[:, -1])


def test_row_variants_match_full():
    rng = _rng(14)
    q1, q2, k1, k2, v, lams = _v1_case(rng, 2, 3, 21, 8)
    full = oracle.v1_fwd(q1, q2, k1, k2, v, *lams, 6)
    idx = np.array([[0, 0, 0], [1, 2, 20], [0, 1, 7], [1, 0, 13]])
    rows = oracle.v1_rows(q1, q2, k1, k2, v, *lams, 6, idx)
    for r, (b, h, i) in enumerate(idx):
        assert np.array_equal(rows[r], full[b, i, h])
    q, k, vv, lam = _v2_case(rng, 2, 15, 8, 2, 8)
    full2 = oracle.v2_fwd(q, k, vv, lam)
    idx2 = np.array([[0, 0, 0], [1, 14, 3], [0, 7, 2]])
    rows2 = oracle.v2_rows(q, k, vv, lam, idx2)
    for r, (b, t, p) in enumerate(idx2):
        assert np.array_equal(rows2[r], full2[b, t, p])


# --------------------------------------------------------------------------
# Off-by-one softmax exp(x_j) / (1 + sum_j exp(x_j)) (Hacker News item
# 41780844: a comment proposing an extra 1 in the softmax denominator, which
# is the same as an extra logit 0 among the inputs)
# --------------------------------------------------------------------------

def _prepend_zero_token(x, axis):
    """x with one all-zero entry inserted at index 0 of the token axis."""
    shape = list(x.shape)
    shape[axis] = 1
    return np.concatenate([np.zeros(shape), x], axis=axis)


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_softmax1_is_an_extra_zero_key(seed):
    """Off-by-one attention over T keys equals standard attention over T+1
    keys whose first key is the zero vector (logit exactly 0 for every
    query) with a zero value row: prepend that token, drop its output row."""
    rng = _rng(200 + seed)
    B, H, T, d, layer = 2, 2, 19, 8, 3
    q1, q2, k1, k2, v, lams = _v1_case(rng, B, H, T, d, lam_std=0.4)
    got = oracle.v1_fwd(q1, q2, k1, k2, v, *lams, layer, softmax1=True)
    aug = [_prepend_zero_token(x, 2) for x in (q1, q2, k1, k2, v)]
    ref = oracle.v1_fwd(*aug, *lams, layer)[:, 1:]
    _close(got, ref, rtol=1e-11, atol=1e-12)
    q, k, vv, lg = _v2_case(rng, 2, 23, 8, 2, d)
    got2 = oracle.v2_fwd(q, k, vv, lg, softmax1=True)
    ref2 = oracle.v2_fwd(*[_prepend_zero_token(x, 1) for x in (q, k, vv, lg)])[:, 1:]
    _close(got2, ref2, rtol=1e-11, atol=1e-12)
    qd = rng.standard_normal((2, 8, d))
    kd, vd = rng.standard_normal((2, 30, 2, d)), rng.standard_normal((2, 30, 2, d))
    lgd = rng.standard_normal((2, 4))
    got3 = oracle.v2_decode(qd, kd, vd, lgd, softmax1=True)
    ref3 = oracle.v2_decode(qd, _prepend_zero_token(kd, 1), _prepend_zero_token(vd, 1), lgd)
    _close(got3, ref3, rtol=1e-11, atol=1e-12)


@pytest.mark.parametrize("s", [-2.0, 1.5])
def test_softmax1_equal_scores_closed_form(s):
    """Every visible score equal to s: each of the n = i+1 keys gets weight
    e^s / (1 + n e^s), so A.V = n e^s / (1 + n e^s) * prefix-mean(V)."""
    rng = _rng(210)
    B, T, Hq, Hkv, d = 1, 40, 4, 2, 8
    u = np.zeros(d)
    u[0] = 1.0
    q = np.broadcast_to(s * math.sqrt(d) * u, (B, T, Hq, d)).copy()
    k = np.broadcast_to(u, (B, T, Hkv, d)).copy()
    v = rng.standard_normal((B, T, Hkv, d))
    lg = rng.standard_normal((B, T, Hq // 2))
    n = np.arange(1, T + 1)[None, :, None, None]
    frac = n * math.exp(s) / (1.0 + n * math.exp(s))
    pm = np.cumsum(v, axis=1) / n  # [B,T,Hkv,d]
    a = np.repeat(frac * pm, 2, axis=2)  # heads 2p, 2p+1 share the group's K/V here (G = 2)
    sig = 1.0 / (1.0 + np.exp(-lg))
    _close(oracle.v2_fwd(q, k, v, lg, softmax1=True), (1 - sig)[..., None] * a[:, :, 0::2])
    # V1 with both maps on the same scores: D = (1 - lam) frac * prefix-mean(V)
    H, layer = 1, 6
    q1 = np.broadcast_to(s * math.sqrt(d) * u, (B, H, T, d)).copy()
    k1 = np.broadcast_to(u, (B, H, T, d)).copy()
    v1 = rng.standard_normal((B, H, T, 2 * d))
    lams = [0.3 * rng.standard_normal(d) for _ in range(4)]
    lam, li = oracle.v1_lambda(*lams, layer), oracle.lambda_init(layer)
    n1 = np.arange(1, T + 1)[None, None, :, None]
    D = (1 - lam) * (n1 * math.exp(s) / (1 + n1 * math.exp(s))) * np.cumsum(v1, axis=2) / n1
    ref = (1 - li) * D / np.sqrt(np.mean(D * D, -1, keepdims=True) + 1e-5)
    _close(oracle.v1_fwd(q1, q1, k1, k1, v1, *lams, layer, softmax1=True), np.transpose(ref, (0, 2, 1, 3)))


# --------------------------------------------------------------------------
# V2 decode over a paged, ragged cache: a storage layout of the same decode
# ("Differential Transformer V2" article, DiffAttnV2 at the newest position)
# --------------------------------------------------------------------------

def _paged_case(rng, lens, page, Hkv, G, d, spare=3):
    """Random pages for sequences of lengths ``lens``: every page a sequence
    uses is drawn without replacement from a shuffled pool with ``spare``
    unused pages; returns (q, k_pages, v_pages, table, lens, lam)."""
    B = len(lens)
    npp = [max(1, (L + page - 1) // page) for L in lens]
    width = max(npp)
    pool = sum(npp) + spare
    order = rng.permutation(pool)
    table = np.full((B, width), -1, dtype=np.int64)
    at = 0
    for b in range(B):
        table[b, :npp[b]] = order[at:at + npp[b]]
        at += npp[b]
    Hq = G * Hkv
    q = rng.standard_normal((B, Hq, d))
    kp = rng.standard_normal((pool, page, Hkv, d))
    vp = rng.standard_normal((pool, page, Hkv, d))
    lam = rng.standard_normal((B, Hq // 2))
    return q, kp, vp, table, np.array(lens, dtype=np.int64), lam


@settings(max_examples=30, deadline=None)
@given(lens=st.lists(st.integers(0, 40), min_size=1, max_size=4), page=st.sampled_from([1, 2, 4, 16]),
       Hkv=st.integers(1, 2), G=st.sampled_from([2, 4]), d=st.sampled_from([4, 8]), seed=st.integers(0, 10**6))
def test_paged_decode_matches_bruteforce(lens, page, Hkv, G, d, seed):
    q, kp, vp, table, ln, lam = _paged_case(_rng(seed), lens, page, Hkv, G, d)
    got = oracle.v2_decode_paged(q, kp, vp, table, ln, lam)
    _close(got, bruteforce.v2_decode_paged(q, kp, vp, table, ln, lam))


def test_paged_identity_table_is_the_dense_cache():
    """Pages laid end to end in sequence order (table[b, j] = b*n + j) are a
    reshaped dense cache: the result is the dense decode's."""
    rng = _rng(220)
    B, L, Hkv, G, d, page = 3, 48, 2, 4, 8, 16
    q = rng.standard_normal((B, G * Hkv, d))
    k = rng.standard_normal((B, L, Hkv, d))
    v = rng.standard_normal((B, L, Hkv, d))
    lam = rng.standard_normal((B, G * Hkv // 2))
    n = L // page
    table = np.arange(B * n).reshape(B, n)
    kp, vp = k.reshape(B * n, page, Hkv, d), v.reshape(B * n, page, Hkv, d)
    got = oracle.v2_decode_paged(q, kp, vp, table, np.full(B, L), lam)
    assert np.array_equal(got, oracle.v2_decode(q, k, v, lam))


def test_paged_pool_permutation_invariance():
    """Moving pages around the pool and rewriting the table to match leaves
    every result bit-identical."""
    rng = _rng(221)
    q, kp, vp, table, ln, lam = _paged_case(rng, [37, 1, 64, 0, 16], 16, 2, 4, 8)
    perm = rng.permutation(kp.shape[0])  # new slot of old page i is perm[i]
    kq, vq = np.empty_like(kp), np.empty_like(vp)
    kq[perm], vq[perm] = kp, vp
    t2 = np.where(table >= 0, perm[np.maximum(table, 0)], -1)
    a = oracle.v2_decode_paged(q, kp, vp, table, ln, lam)
    assert np.array_equal(a, oracle.v2_decode_paged(q, kq, vq, t2, ln, lam))


def test_paged_ragged_lengths_are_dense_prefixes():
    """A sequence of length L_b decodes exactly the first L_b cache entries
    (dense decode of the prefix); length 0 gives 0."""
    rng = _rng(222)
    lens = [1, 17, 32, 0, 45]
    B, Lmax, Hkv, G, d, page = len(lens), 48, 2, 2, 8, 16
    q = rng.standard_normal((B, G * Hkv, d))
    k = rng.standard_normal((B, Lmax, Hkv, d))
    v = rng.standard_normal((B, Lmax, Hkv, d))
    lam = rng.standard_normal((B, G * Hkv // 2))
    n = Lmax // page
    table = np.arange(B * n).reshape(B, n)
    got = oracle.v2_decode_paged(q, k.reshape(B * n, page, Hkv, d), v.reshape(B * n, page, Hkv, d),
                                 table, np.array(lens), lam)
    for b, L in enumerate(lens):
        if L == 0:
            assert np.array_equal(got[b], np.zeros_like(got[b]))
        else:
            ref = oracle.v2_decode(q[b:b + 1], k[b:b + 1, :L], v[b:b + 1, :L], lam[b:b + 1])[0]
            assert np.array_equal(got[b], ref)


# --------------------------------------------------------------------------
# Multi-token decode: the last nq rows of causal DiffAttnV2 over the cache
# --------------------------------------------------------------------------

def _as_prefill(rng, q_new, lam_new, L):
    """Embed the nq decode queries as the last nq rows of a length-L prefill
    (random queries and logits for the rows before them)."""
    B, nq, Hq, d = q_new.shape
    q = rng.standard_normal((B, L, Hq, d))
    lam = rng.standard_normal((B, L, Hq // 2))
    q[:, L - nq:] = q_new
    lam[:, L - nq:] = lam_new
    return q, lam


@settings(max_examples=25, deadline=None)
@given(B=st.integers(1, 2), L=st.sampled_from([1, 2, 5, 17, 40]), nq=st.integers(1, 6), Hkv=st.integers(1, 2),
       G=st.sampled_from([2, 4]), d=st.sampled_from([4, 8]), seed=st.integers(0, 10**6))
def test_multi_decode_is_the_last_prefill_rows_bruteforce(B, L, nq, Hkv, G, d, seed):
    """Brute force (explicit masked maps over the whole sequence): the nq new
    tokens' outputs are the last nq rows of causal DiffAttnV2."""
    nq = min(nq, L)
    rng = _rng(seed)
    Hq = G * Hkv
    qn, ln = rng.standard_normal((B, nq, Hq, d)), rng.standard_normal((B, nq, Hq // 2))
    k, v = rng.standard_normal((B, L, Hkv, d)), rng.standard_normal((B, L, Hkv, d))
    q, lam = _as_prefill(rng, qn, ln, L)
    _close(oracle.v2_decode_multi(qn, k, v, ln), bruteforce.v2(q, k, v, lam)[:, L - nq:])


def test_multi_decode_matches_prefill_oracle_and_single_token():
    rng = _rng(230)
    B, L, nq, Hq, Hkv, d = 2, 50, 5, 16, 2, 16
    qn, ln = rng.standard_normal((B, nq, Hq, d)), rng.standard_normal((B, nq, Hq // 2))
    k, v = rng.standard_normal((B, L, Hkv, d)), rng.standard_normal((B, L, Hkv, d))
    q, lam = _as_prefill(rng, qn, ln, L)
    got = oracle.v2_decode_multi(qn, k, v, ln)
    _close(got, oracle.v2_fwd(q, k, v, lam)[:, L - nq:])
    # the newest token sees the whole cache: the single-token decode
    assert np.array_equal(got[:, -1], oracle.v2_decode(qn[:, -1], k, v, ln[:, -1]))
    # off-by-one softmax: the same rows of the off-by-one prefill
    _close(oracle.v2_decode_multi(qn, k, v, ln, softmax1=True),
           oracle.v2_fwd(q, k, v, lam, softmax1=True)[:, L - nq:])


def test_paged_multi_decode_matches_dense_multi():
    rng = _rng(231)
    lens, nq, page, Hkv, G, d = [30, 5, 64, 17], 4, 16, 2, 4, 8
    q, kp, vp, table, ln, lam = _paged_case(rng, lens, page, Hkv, G, d)
    B, Hq = len(lens), G * Hkv
    qn, lmn = rng.standard_normal((B, nq, Hq, d)), rng.standard_normal((B, nq, Hq // 2))
    got = oracle.v2_decode_paged(qn, kp, vp, table, ln, lmn)
    for b, L in enumerate(lens):
        t = np.arange(L)
        k, v = kp[table[b, t // page], t % page], vp[table[b, t // page], t % page]
        ref = oracle.v2_decode_multi(qn[b:b + 1], k[None], v[None], lmn[b:b + 1])[0]
        assert np.array_equal(got[b], ref)
    # a sequence shorter than nq: its first new tokens see nothing and give 0
    short = oracle.v2_decode_paged(qn[:1], kp, vp, table[:1], np.array([2]), lmn[:1])
    assert np.array_equal(short[0, :2], np.zeros_like(short[0, :2]))
    assert np.abs(short[0, 2:]).max() > 0
