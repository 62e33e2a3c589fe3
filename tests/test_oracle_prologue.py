"""Pins of the RoPE and lambda-projection oracle (oracle/prologue.py), on the CPU.

No page prints a rotary example, so the rotation is pinned by what defines it:
the d = 2 case is multiplication by e^{it} (fixes the sign), a unit vector
at one index traces the circle at that index's frequency (fixes the pairing
c <-> c + d/2 and the exponent -2c/d), rotations compose by adding positions,
preserve each pair's length, and a score then depends on the position
difference only -- so a causal prefill is unchanged when every position is
shifted.  The projection is a linear layer without bias (torch's F.linear,
fp64).  Mutants plant one plausible mistake at a time in the source.
"""
import inspect
import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F
from hypothesis import given, settings, strategies as st

import oracle
from oracle import prologue as op


def test_rope_d2_is_complex_rotation():
    t = np.arange(7.0)
    x = np.array([0.3, -1.2])
    got = op.rope(np.broadcast_to(x, (1, 7, 2)), theta=10000.0)[0]
    z = (x[0] + 1j * x[1]) * np.exp(1j * t)  # w_0 = theta^0 = 1
    assert np.abs(got[:, 0] - z.real).max() < 1e-13
    assert np.abs(got[:, 1] - z.imag).max() < 1e-13


@pytest.mark.parametrize("d,c", [(4, 1), (8, 3), (64, 17), (128, 63)])
def test_rope_unit_vector_traces_its_frequency(d, c):
    theta = 500.0
    e = np.zeros(d)
    e[c] = 1.0
    T = 9
    got = op.rope(np.broadcast_to(e, (1, T, d)), theta=theta)[0]
    w = theta ** (-2.0 * c / d)
    t = np.arange(T)
    want = np.zeros((T, d))
    want[:, c] = np.cos(t * w)
    want[:, c + d // 2] = np.sin(t * w)
    assert np.abs(got - want).max() < 1e-13


@settings(max_examples=20, deadline=None)
@given(a=st.integers(0, 5000), b=st.integers(0, 5000), seed=st.integers(0, 10**6))
def test_rope_composes_and_preserves_pair_lengths(a, b, seed):
    x = np.random.default_rng(seed).standard_normal((1, 3, 2, 16))
    pa, pb = np.array([a, a + 7, 2 * a]), np.array([b, 3, b + 1])
    ra = op.rope(x, positions=pa)
    rab = op.rope(ra, positions=pb)
    assert np.abs(rab - op.rope(x, positions=pa + pb)).max() < 1e-9  # angles add
    assert np.abs(op.rope(x, pos0=a) - op.rope(x, positions=a + np.arange(3))).max() == 0
    pl = lambda y: y[..., :8] ** 2 + y[..., 8:] ** 2
    assert np.abs(pl(ra) - pl(x)).max() < 1e-12


@settings(max_examples=15, deadline=None)
@given(s=st.integers(0, 3000), t=st.integers(0, 3000), u=st.integers(0, 3000), seed=st.integers(0, 10**6))
def test_rope_scores_depend_on_position_difference(s, t, u, seed):
    rng = np.random.default_rng(seed)
    q, k = rng.standard_normal(32), rng.standard_normal(32)
    at = lambda x, p: op.rope(x[None, None], pos0=p)[0, 0]
    assert abs(at(q, s) @ at(k, t) - at(q, s - t + u + 3000) @ at(k, u + 3000)) < 1e-9


def test_prefill_is_invariant_to_a_position_shift():
    rng = np.random.default_rng(5)
    B, T, Hq, Hkv, d = 1, 23, 4, 2, 8
    q, k, v = rng.standard_normal((B, T, Hq, d)), rng.standard_normal((B, T, Hkv, d)), rng.standard_normal((B, T, Hkv, d))
    lam = rng.standard_normal((B, T, Hq // 2))
    a = op.v2_fwd_rope(q, k, v, lam, pos0=0)
    b = op.v2_fwd_rope(q, k, v, lam, pos0=777)
    assert np.abs(a - b).max() < 1e-12
    # and rotation changes the result (it is not skipped)
    assert np.abs(a - oracle.v2_fwd(q, k, v, lam)).max() > 1e-3


def test_v1_rope_rotates_both_maps_at_the_same_positions():
    rng = np.random.default_rng(6)
    B, H, T, d = 1, 2, 17, 8
    q1, q2, k1, k2 = [rng.standard_normal((B, H, T, d)) for _ in range(4)]
    v = rng.standard_normal((B, H, T, 2 * d))
    lams = [0.1 * rng.standard_normal(d) for _ in range(4)]
    a = op.v1_fwd_rope(q1, q2, k1, k2, v, *lams, 3, pos0=0)
    b = op.v1_fwd_rope(q1, q2, k1, k2, v, *lams, 3, pos0=400)
    assert np.abs(a - b).max() < 1e-12
    # identical branches stay identical after rotation: D = (1 - lambda) A1 V (page [HN2] #131's case)
    c = op.v1_fwd_rope(q1, q1, k1, k1, v, *lams, 3)
    d_ = oracle.v1_fwd(*(op.rope(x, axis_t=2) for x in (q1, q1, k1, k1)), v, *lams, 3)
    assert np.abs(c - d_).max() < 1e-12


def test_decode_rope_is_the_last_row_of_the_rotated_prefill():
    rng = np.random.default_rng(7)
    B, L, Hq, Hkv, d = 2, 19, 4, 2, 8
    q = rng.standard_normal((B, L, Hq, d))
    k, v = rng.standard_normal((B, L, Hkv, d)), rng.standard_normal((B, L, Hkv, d))
    lam = rng.standard_normal((B, L, Hq // 2))
    pre = op.v2_fwd_rope(q, k, v, lam)
    dec = op.v2_decode_rope(q[:, -1], op.rope(k), v, lam[:, -1])
    assert np.abs(dec - pre[:, -1]).max() < 1e-12


def test_lambda_proj_is_a_linear_layer():
    rng = np.random.default_rng(8)
    x, w = rng.standard_normal((2, 5, 48)), rng.standard_normal((6, 48))
    want = F.linear(torch.tensor(x), torch.tensor(w)).numpy()
    assert np.abs(op.lambda_proj(x, w) - want).max() < 1e-12


ROPE_SRC = inspect.getsource(op.rope)
ROPE_MUTATIONS = {
    "sign": ("x1 * c - x2 * s, x2 * c + x1 * s", "x1 * c + x2 * s, x2 * c - x1 * s"),
    "exponent": ("w = theta ** (-2.0 * np.arange(h) / d)", "w = theta ** (-1.0 * np.arange(h) / d)"),
    "position_off_by_one": ("np.arange(T, dtype=np.float64) + pos0", "np.arange(T, dtype=np.float64) + pos0 + 1"),
    "interleaved_pairs": ("x1, x2 = x[..., :h], x[..., h:]", "x1, x2 = x[..., 0::2], x[..., 1::2]"),
}
ROPE_PINS = [test_rope_d2_is_complex_rotation, lambda: test_rope_unit_vector_traces_its_frequency(8, 3)]


@pytest.mark.parametrize("name", sorted(ROPE_MUTATIONS))
def test_rope_mutant_is_caught(name, monkeypatch):
    old, new = ROPE_MUTATIONS[name]
    assert ROPE_SRC.count(old) == 1, name
    ns = dict(vars(op))
    exec(compile(ROPE_SRC.replace(old, new), "<mutant>", "exec"), ns)
    monkeypatch.setattr(op, "rope", ns["rope"])
    failed = 0
    for pin in ROPE_PINS:
        try:
            pin()
        except AssertionError:
            failed += 1
    assert failed >= 1, f"no pin catches mutation {name}"
