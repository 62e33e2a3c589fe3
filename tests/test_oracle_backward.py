"""Pins of the DIFF V2 backward oracle (oracle/backward.py), on the CPU.

The gradient oracle is pinned to things other than itself: central finite
differences of the (pinned) forward in random directions, torch autograd
through an independently written fp64 forward, and an exact invariant of
the softmax (each row of P sums to one).  The mutants at the end plant one
plausible mistake at a time in the oracle's source and check a pin fails.
"""
import inspect
import math

import numpy as np
import pytest
import torch
from hypothesis import given, settings, strategies as st

import oracle
from oracle import backward as ob


def _case(seed, B, T, Hkv, G, d):
    rng = np.random.default_rng(seed)
    Hq = G * Hkv
    return (rng.standard_normal((B, T, Hq, d)), rng.standard_normal((B, T, Hkv, d)),
            rng.standard_normal((B, T, Hkv, d)), rng.standard_normal((B, T, Hq // 2)),
            rng.standard_normal((B, T, Hq // 2, d)), rng)


def test_fwd_train_matches_the_forward_oracle():
    q, k, v, lam, _, _ = _case(1, 2, 13, 2, 4, 8)
    for s1 in (False, True):
        out, attn, lse2 = ob.v2_fwd_train(q, k, v, lam, softmax1=s1)
        assert np.abs(out - oracle.v2_fwd(q, k, v, lam, softmax1=s1)).max() < 1e-12
        sig = 1.0 / (1.0 + np.exp(-lam))
        assert np.abs(out - (attn[:, :, 0::2] - sig[..., None] * attn[:, :, 1::2])).max() < 1e-12
        # lse2 rebuilds the row's probabilities: they sum to 1 (standard) or
        # to 1 - 2^(-lse2) (off-by-one: the extra logit 0 takes the rest)
        B, T, Hq, d = q.shape
        G = Hq // k.shape[2]
        for h in (0, Hq - 1):
            S = q[0][:, h] @ k[0][:, h // G].T / math.sqrt(d) * math.log2(math.e)
            S = np.where(np.triu(np.ones((T, T), bool), 1), -np.inf, S)
            rows = np.exp2(S - lse2[0, h][:, None]).sum(axis=1)
            want = 1.0 - (np.exp2(-lse2[0, h]) if s1 else 0.0)
            assert np.abs(rows - want).max() < 1e-12


@settings(max_examples=20, deadline=None)
@given(B=st.integers(1, 2), T=st.sampled_from([1, 2, 5, 12]), Hkv=st.integers(1, 2), G=st.sampled_from([2, 4]),
       d=st.sampled_from([4, 8]), s1=st.booleans(), seed=st.integers(0, 10**6))
def test_bwd_matches_central_differences(B, T, Hkv, G, d, s1, seed):
    """<grad, u> equals the central difference of sum(dout * out) along a
    random direction u, for each input."""
    q, k, v, lam, dout, rng = _case(seed, B, T, Hkv, G, d)
    grads = dict(zip(("q", "k", "v", "lam"), ob.v2_bwd(q, k, v, lam, dout, softmax1=s1)))
    args = dict(q=q, k=k, v=v, lam=lam)
    f = lambda **a: float((ob.v2_fwd_train(**a, softmax1=s1)[0] * dout).sum())
    eps = 1e-5
    for name, x in args.items():
        u = rng.standard_normal(x.shape)
        fd = (f(**{**args, name: x + eps * u}) - f(**{**args, name: x - eps * u})) / (2 * eps)
        an = float((grads[name] * u).sum())
        assert abs(fd - an) <= 1e-6 * (1.0 + abs(an)), (name, fd, an)


def _torch_forward(q, k, v, lam, softmax1):
    """An independent fp64 forward in torch ops (explicit masked maps per
    kv group, heads repeated), differentiated by autograd."""
    B, T, Hq, d = q.shape
    G = Hq // k.shape[2]
    kr, vr = k.repeat_interleave(G, dim=2), v.repeat_interleave(G, dim=2)
    s = torch.einsum("bthc,bjhc->bhtj", q, kr) / math.sqrt(d)
    s = s.masked_fill(torch.ones(T, T, dtype=torch.bool).triu(1), -math.inf)
    if softmax1:
        s = torch.cat([s, torch.zeros(B, Hq, T, 1, dtype=s.dtype)], dim=-1)
        p = torch.softmax(s, dim=-1)[..., :T]
    else:
        p = torch.softmax(s, dim=-1)
    a = torch.einsum("bhtj,bjhc->bthc", p, vr)
    return a[:, :, 0::2] - torch.sigmoid(lam)[..., None] * a[:, :, 1::2]


@pytest.mark.parametrize("s1", [False, True])
def test_bwd_matches_torch_autograd(s1):
    q, k, v, lam, dout, _ = _case(7, 2, 17, 2, 4, 8)
    ts = [torch.tensor(x, requires_grad=True) for x in (q, k, v, lam)]
    (_torch_forward(*ts, s1) * torch.tensor(dout)).sum().backward()
    for got, t in zip(ob.v2_bwd(q, k, v, lam, dout, softmax1=s1), ts):
        assert np.abs(got - t.grad.numpy()).max() < 1e-10


def test_bwd_dv_column_sums():
    """Rows of P sum to one, so summing dv over the keys gives the sum over
    rows and over the group's heads of d attn (dout for even heads,
    -sigmoid(lam) dout for odd heads)."""
    q, k, v, lam, dout, _ = _case(8, 2, 11, 2, 4, 8)
    dv = ob.v2_bwd(q, k, v, lam, dout)[2]
    sig = 1.0 / (1.0 + np.exp(-lam))
    da = np.zeros(q.shape)
    da[:, :, 0::2] = dout
    da[:, :, 1::2] = -sig[..., None] * dout
    G = q.shape[2] // k.shape[2]
    for g in range(k.shape[2]):
        want = da[:, :, g * G:(g + 1) * G].sum(axis=(1, 2))
        assert np.abs(dv[:, :, g].sum(axis=1) - want).max() < 1e-12


BWD_SRC = inspect.getsource(ob.v2_bwd)

BWD_MUTATIONS = {
    "odd_head_sign": ("da[:, 1::2] = -sig[..., None] * dout[b]", "da[:, 1::2] = sig[..., None] * dout[b]"),
    "dlam_no_derivative": ("dlam[b] = -sig * (1.0 - sig) *", "dlam[b] = -sig *"),
    "dlam_even_head": ('np.einsum("tpc,tpc->tp", dout[b], attn[:, 1::2])',
                       'np.einsum("tpc,tpc->tp", dout[b], attn[:, 0::2])'),
    "softmax_jacobian_no_rowsum": ("dS = P[h] * (dP - (P[h] * dP).sum(axis=1, keepdims=True))", "dS = P[h] * dP"),
    "dk_unscaled": ("dk[b][:, g] += dS.T @ q[b][:, h] / math.sqrt(d)", "dk[b][:, g] += dS.T @ q[b][:, h]"),
    "dv_untransposed": ("dv[b][:, g] += P[h].T @ da[:, h]", "dv[b][:, g] += P[h] @ da[:, h]"),
    "dq_wrong_group": ("dq[b][:, h] = dS @ k[b][:, g] / math.sqrt(d)",
                       "dq[b][:, h] = dS @ k[b][:, (g + 1) % Hkv] / math.sqrt(d)"),
}

BWD_PINS = [
    lambda: test_bwd_matches_central_differences.hypothesis.inner_test(
        B=1, T=6, Hkv=2, G=2, d=4, s1=False, seed=11),
    lambda: test_bwd_matches_torch_autograd(False),
    test_bwd_dv_column_sums,
]


@pytest.mark.parametrize("name", sorted(BWD_MUTATIONS))
def test_backward_mutant_is_caught(name, monkeypatch):
    old, new = BWD_MUTATIONS[name]
    assert BWD_SRC.count(old) == 1, f"mutation {name} no longer matches the oracle source"
    ns = dict(vars(ob))
    exec(compile(BWD_SRC.replace(old, new), "<mutant>", "exec"), ns)
    monkeypatch.setattr(ob, "v2_bwd", ns["v2_bwd"])
    failed = 0
    for pin in BWD_PINS:
        try:
            with np.errstate(all="ignore"):
                pin()
        except AssertionError:
            failed += 1
    assert failed >= 1, f"no pin catches mutation {name}"


# ---- sampled V2 backward (rows and keys, for full-size GPU checks) -----------------

@pytest.mark.parametrize("s1", [False, True])
def test_v2_heads_matches_fwd_train(s1):
    """The C per-head forward gives the dense numpy training forward's attn and
    lse (natural log here, log2 there)."""
    q, k, v, lam, _, _ = _case(21, 2, 19, 2, 4, 8)
    attn, lse = oracle.v2_heads(q, k, v, softmax1=s1)
    _, attn2, lse2 = ob.v2_fwd_train(q, k, v, lam, softmax1=s1)
    assert np.abs(attn - attn2).max() < 1e-12
    assert np.abs(lse - lse2 * math.log(2.0)).max() < 1e-12


@settings(max_examples=15, deadline=None)
@given(B=st.integers(1, 2), T=st.sampled_from([1, 2, 7, 20]), Hkv=st.integers(1, 2), G=st.sampled_from([2, 4]),
       d=st.sampled_from([4, 8]), s1=st.booleans(), seed=st.integers(0, 10**6))
def test_bwd_sampled_matches_dense(B, T, Hkv, G, d, s1, seed):
    """dq of every row and dk, dv of every key, one at a time, equal the dense
    per-head gradients."""
    q, k, v, lam, dout, _ = _case(seed, B, T, Hkv, G, d)
    dq, dk, dv, dlam = ob.v2_bwd(q, k, v, lam, dout, softmax1=s1)
    Hq = G * Hkv
    rows = [(b, t, h) for b in range(B) for t in range(T) for h in range(Hq)]
    keys = [(b, j, g) for b in range(B) for j in range(T) for g in range(Hkv)]
    sq, sk, sv, sl = ob.v2_bwd_sampled(q, k, v, lam, dout, rows, keys, softmax1=s1)
    scale = lambda x: max(1.0, np.abs(x).max())
    assert np.abs(sq - dq.reshape(-1, d)).max() < 1e-12 * scale(dq)
    assert np.abs(sk - dk.reshape(-1, d)).max() < 1e-12 * scale(dk)
    assert np.abs(sv - dv.reshape(-1, d)).max() < 1e-12 * scale(dv)
    assert np.abs(sl - dlam).max() < 1e-12


SAMPLED_SRC = inspect.getsource(ob.v2_bwd_sampled)

SAMPLED_MUTATIONS = {
    "odd_head_sign": ("return g if h % 2 == 0 else -sig", "return g if h % 2 == 0 else sig"),
    "no_D_in_dq": ("dS = P * (vj @ da - da @ attn[b, t, h])", "dS = P * (vj @ da)"),
    "rows_from_next_key": ("ts = np.arange(j, T)", "ts = np.arange(j + 1, T)"),
    "dk_unscaled": ("dk[n] += dS @ qt * sc", "dk[n] += dS @ qt"),
    "dq_sees_masked_key": ("kj, vj = k[b, :t + 1, g], v[b, :t + 1, g]", "kj, vj = k[b, :t + 2, g], v[b, :t + 2, g]"),
    "wrong_group_heads": ("for h in range(g * G, (g + 1) * G):", "for h in range(g, g + G):"),
}


@pytest.mark.parametrize("name", sorted(SAMPLED_MUTATIONS))
def test_sampled_mutant_is_caught(name, monkeypatch):
    old, new = SAMPLED_MUTATIONS[name]
    assert SAMPLED_SRC.count(old) == 1, f"mutation {name} no longer matches the oracle source"
    ns = dict(vars(ob))
    exec(compile(SAMPLED_SRC.replace(old, new), "<mutant>", "exec"), ns)
    monkeypatch.setattr(ob, "v2_bwd_sampled", ns["v2_bwd_sampled"])
    with pytest.raises((AssertionError, ValueError, IndexError)):
        with np.errstate(all="ignore"):
            test_bwd_sampled_matches_dense.hypothesis.inner_test(B=2, T=9, Hkv=2, G=2, d=4, s1=False, seed=5)


# ---- DIFF V1 ---------------------------------------------------------------------

def _v1_case(seed, B, H, T, d):
    rng = np.random.default_rng(seed)
    qk = [rng.standard_normal((B, H, T, d)) for _ in range(4)]
    v = rng.standard_normal((B, H, T, 2 * d))
    lams = [0.1 * rng.standard_normal(d) for _ in range(4)]
    dout = rng.standard_normal((B, T, H, 2 * d))
    return qk, v, lams, dout, rng


V1_NAMES = ("q1", "q2", "k1", "k2", "v", "lq1", "lk1", "lq2", "lk2")


def test_v1_fwd_train_matches_the_forward_oracle():
    (q1, q2, k1, k2), v, lams, _, _ = _v1_case(3, 2, 2, 11, 8)
    layer = 5
    lam = oracle.v1_lambda(*lams, layer)
    li = oracle.lambda_init(layer)
    for s1 in (False, True):
        out, a1, a2, lse2 = ob.v1_fwd_train(q1, q2, k1, k2, v, *lams, layer, softmax1=s1)
        assert np.abs(out - oracle.v1_fwd(q1, q2, k1, k2, v, *lams, layer, softmax1=s1)).max() < 1e-12
        D = a1 - lam * a2
        assert np.abs(out - (1 - li) * D / np.sqrt((D * D).mean(-1, keepdims=True) + 1e-5)).max() < 1e-12
        T, d = q1.shape[2], q1.shape[3]
        for m, (q, k, a) in enumerate(((q1, k1, a1), (q2, k2, a2))):
            S = q[1, 0] @ k[1, 0].T / math.sqrt(d) * math.log2(math.e)
            S = np.where(np.triu(np.ones((T, T), bool), 1), -np.inf, S)
            P = np.exp2(S - lse2[m, 1, 0][:, None])
            want = 1.0 - (np.exp2(-lse2[m, 1, 0]) if s1 else 0.0)
            assert np.abs(P.sum(axis=1) - want).max() < 1e-12
            assert np.abs(P @ v[1, 0] - a[1, :, 0]).max() < 1e-12


@settings(max_examples=15, deadline=None)
@given(B=st.integers(1, 2), H=st.integers(1, 2), T=st.sampled_from([1, 2, 5, 12]), d=st.sampled_from([2, 4, 8]),
       layer=st.integers(0, 14), s1=st.booleans(), seed=st.integers(0, 10**6))
def test_v1_bwd_matches_central_differences(B, H, T, d, layer, s1, seed):
    """<grad, u> equals the central difference of sum(dout * out) along a
    random direction u, for each of the nine inputs."""
    qk, v, lams, dout, rng = _v1_case(seed, B, H, T, d)
    args = dict(zip(V1_NAMES, qk + [v] + lams))
    grads = dict(zip(V1_NAMES, ob.v1_bwd(**args, layer=layer, dout=dout, softmax1=s1)))
    f = lambda **a: float((ob.v1_fwd_train(**a, layer=layer, softmax1=s1)[0] * dout).sum())
    # Richardson extrapolation of central differences at steps h and h/2
    # (truncation O(h^4) instead of O(h^2)): a row whose D is near 0 puts the
    # RMSNorm near its eps, where the curvature is large enough that a plain
    # central difference at 1e-5 misses the tolerance
    h = 1e-5
    cd = lambda name, x, u, e: (f(**{**args, name: x + e * u}) - f(**{**args, name: x - e * u})) / (2 * e)
    for name, x in args.items():
        u = rng.standard_normal(x.shape)
        fd = (4 * cd(name, x, u, h / 2) - cd(name, x, u, h)) / 3
        an = float((grads[name] * u).sum())
        assert abs(fd - an) <= 1e-6 * (1.0 + abs(an)), (name, fd, an)


def _torch_v1_forward(q1, q2, k1, k2, v, lq1, lk1, lq2, lk2, layer, softmax1):
    """An independent fp64 forward from torch library routines: causal
    scaled_dot_product_attention per map (the off-by-one softmax as one extra
    zero key and zero value row in front, unmasked) and rms_norm."""
    import torch.nn.functional as F
    li = 0.8 - 0.6 * math.exp(-0.3 * layer)
    lam = torch.exp((lq1 * lk1).sum()) - torch.exp((lq2 * lk2).sum()) + li
    B, H, T, d = q1.shape

    def attend(q, k):
        if not softmax1:
            return F.scaled_dot_product_attention(q, k, v, is_causal=True)
        z = lambda x: torch.cat([torch.zeros(B, H, 1, x.shape[-1], dtype=x.dtype), x], dim=2)
        mask = torch.ones(T, T + 1, dtype=torch.bool).tril(1)
        return F.scaled_dot_product_attention(q, z(k), z(v), attn_mask=mask)

    D = attend(q1, k1) - lam * attend(q2, k2)                     # [B, H, T, 2d]
    y = F.rms_norm(D, (2 * d,), eps=1e-5) * (1 - li)
    return y.transpose(1, 2)                                       # [B, T, H, 2d]


@pytest.mark.parametrize("s1", [False, True])
def test_v1_bwd_matches_torch_autograd(s1):
    qk, v, lams, dout, _ = _v1_case(9, 2, 2, 13, 8)
    ts = [torch.tensor(x, requires_grad=True) for x in qk + [v] + lams]
    (_torch_v1_forward(*ts, 7, s1) * torch.tensor(dout)).sum().backward()
    for name, got, t in zip(V1_NAMES, ob.v1_bwd(*qk, v, *lams, 7, dout, softmax1=s1), ts):
        assert np.abs(got - t.grad.numpy()).max() < 1e-10, name


def test_v1_bwd_lambda_vector_structure():
    """d lam / d lq1 = e1 lk1 and d lam / d lk1 = e1 lq1 (same for map 2 with
    a minus sign): the four vector gradients share one scalar, so
    dlq1 / lk1 = dlk1 / lq1 = -(dlq2 / lk2) e1 / e2 elementwise."""
    qk, v, lams, dout, _ = _v1_case(10, 1, 2, 9, 4)
    g = ob.v1_bwd(*qk, v, *lams, 2, dout)
    lq1, lk1, lq2, lk2 = lams
    e1, e2 = math.exp(lq1 @ lk1), math.exp(lq2 @ lk2)
    s = g[5] / lk1
    assert np.abs(s - s[0]).max() < 1e-12 * abs(s[0])
    assert np.abs(g[6] / lq1 - s[0]).max() < 1e-12 * abs(s[0])
    assert np.abs(-g[7] / lk2 * e1 / e2 - s[0]).max() < 1e-12 * abs(s[0])
    assert np.abs(-g[8] / lq2 * e1 / e2 - s[0]).max() < 1e-12 * abs(s[0])


V1_BWD_SRC = inspect.getsource(ob.v1_bwd)

V1_BWD_MUTATIONS = {
    "second_map_sign": ("for m, da in enumerate((dD, -lam * dD)):", "for m, da in enumerate((dD, lam * dD)):"),
    "norm_no_projection": ("dD = (1.0 - li) * r * (g - r * r * D * (g * D).mean(axis=1, keepdims=True))",
                           "dD = (1.0 - li) * r * g"),
    "norm_missing_r2": ("(g - r * r * D * (g * D).mean(axis=1, keepdims=True))",
                        "(g - D * (g * D).mean(axis=1, keepdims=True))"),
    "no_output_scale": ("dD = (1.0 - li) * r *", "dD = r *"),
    "dlam_from_first_map": ("dlam -= float((dD * a[1]).sum())", "dlam -= float((dD * a[0]).sum())"),
    "dv_one_map": ("dv[b, h] += P[m].T @ da", "dv[b, h] = P[m].T @ da"),
    "swapped_lambda_pair": ("-dlam * e2 * lk2, -dlam * e2 * lq2", "-dlam * e2 * lq2, -dlam * e2 * lk2"),
    "dk_unscaled": ("dk[m][b, h] = dS.T @ qs[m][b, h] / math.sqrt(d)", "dk[m][b, h] = dS.T @ qs[m][b, h]"),
}

V1_BWD_PINS = [
    lambda: test_v1_bwd_matches_central_differences.hypothesis.inner_test(
        B=1, H=2, T=6, d=4, layer=3, s1=False, seed=12),
    lambda: test_v1_bwd_matches_torch_autograd(False),
]


@pytest.mark.parametrize("name", sorted(V1_BWD_MUTATIONS))
def test_v1_backward_mutant_is_caught(name, monkeypatch):
    old, new = V1_BWD_MUTATIONS[name]
    assert V1_BWD_SRC.count(old) == 1, f"mutation {name} no longer matches the oracle source"
    ns = dict(vars(ob))
    exec(compile(V1_BWD_SRC.replace(old, new), "<mutant>", "exec"), ns)
    monkeypatch.setattr(ob, "v1_bwd", ns["v1_bwd"])
    failed = 0
    for pin in V1_BWD_PINS:
        try:
            with np.errstate(all="ignore"):
                pin()
        except AssertionError:
            failed += 1
    assert failed >= 1, f"no pin catches mutation {name}"
