"""DIFF V2 training forward and backward (HIP, through the C ABI) against the
fp64 oracle in oracle/backward.py.

Tolerance.  Every gradient is a sum over rows (and heads) of products whose
factors the kernels hold in bf16 (P and dS as MFMA operands, d attn, attn
and hence D = rowsum(d attn * attn)), each with a relative rounding of at
most u = 2^-9, accumulated in fp32.  Where the terms cancel (dq of a row
that sees one key is exactly 0) the error is set by the terms, not by the
result, so each element is bounded by 2e-2 |ref| (the forward's bf16 bar)
plus 4x the sum of |terms| times u that oracle.backward.v2_bwd_rounding_bounds
follows through the same steps, plus 1e-4.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from oracle import backward as ob
from differential_attention_diffattn_amd import binding, workloads
from gpu_util import assert_bf16_close, host64

pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a visible MI355X"
    binding.load_library()
    yield
    torch.cuda.synchronize()


def assert_grad_close(got, ref, bound, what):
    g = host64(got) if isinstance(got, torch.Tensor) else np.asarray(got, np.float64)
    assert g.shape == ref.shape, (g.shape, ref.shape)
    assert np.all(np.isfinite(g)), f"{what}: non-finite"
    excess = np.abs(g - ref) - (2e-2 * np.abs(ref) + 4.0 * bound + 1e-4)
    worst = np.unravel_index(np.argmax(excess), excess.shape)
    assert excess.max() <= 0, (f"{what}: element {worst} got {g[worst]:.5f} ref {ref[worst]:.5f} "
                               f"(excess {excess.max():.3e}, bound {bound[worst]:.3e})")


def _check_grads(grads, ins, what, softmax1=False):
    ref = ob.v2_bwd(*ins, softmax1=softmax1)
    bnd = ob.v2_bwd_rounding_bounds(*ins, softmax1=softmax1)
    for name, got, r, bd in zip(("dq", "dk", "dv", "dlam"), grads, ref, bnd):
        assert_grad_close(got, r, bd, f"{name} {what}")


def _inputs(B, T, Hq, Hkv, d, seed):
    y = workloads.v2_inputs(B, T, Hq, Hkv, d, torch.bfloat16, seed=seed, device=DEV)
    g = torch.Generator(device=DEV).manual_seed(seed + 99)
    dout = torch.randn((B, T, Hq // 2, d), generator=g, device=DEV).to(torch.bfloat16)
    return y, dout


def _cpu(*ts):
    return [t.cpu() for t in ts]


@pytest.mark.parametrize("s1", [False, True])
@pytest.mark.parametrize("T,G,d", [(1, 2, 64), (33, 8, 128), (300, 2, 64), (257, 8, 64), (200, 4, 128)])
def test_fwd_train(T, G, d, s1):
    """out is the inference forward's, bit for bit; attn and lse match the oracle."""
    Hkv = 2
    y, _ = _inputs(2, T, G * Hkv, Hkv, d, seed=700 + T + G + d)
    out, attn, lse = binding.v2_fwd_train(y["q"], y["k"], y["v"], y["lam"], softmax1=s1)
    inf = binding.v2_fwd(y["q"], y["k"], y["v"], y["lam"], softmax1=s1)
    torch.cuda.synchronize()
    assert torch.equal(out, inf)
    r_out, r_attn, r_lse = ob.v2_fwd_train(*_cpu(y["q"], y["k"], y["v"], y["lam"]), softmax1=s1)
    assert_bf16_close(attn, r_attn, f"attn T{T} G{G} d{d}")
    # lse in log2 units; fp32 sums of bf16-rounded probabilities: relative 2^-8 of the sum
    assert np.abs(host64(lse) - r_lse).max() < 1e-2


@pytest.mark.parametrize("T", [1, 31, 32, 33, 100, 300])
@pytest.mark.parametrize("G,d", [(2, 64), (8, 128), (4, 64), (2, 128)])
def test_backward(T, G, d):
    Hkv = 2
    B = 2 if T < 200 else 1
    y, dout = _inputs(B, T, G * Hkv, Hkv, d, seed=800 + T + G + d)
    _, attn, lse = binding.v2_fwd_train(y["q"], y["k"], y["v"], y["lam"])
    grads = binding.v2_bwd(y["q"], y["k"], y["v"], y["lam"], attn, lse, dout)
    torch.cuda.synchronize()
    _check_grads(grads, _cpu(y["q"], y["k"], y["v"], y["lam"], dout), f"T{T} G{G} d{d}")


def test_backward_softmax1():
    """The off-by-one training forward's lse carries the extra term; the
    backward is the same code and must give the off-by-one gradients."""
    y, dout = _inputs(1, 150, 8, 2, 128, seed=900)
    _, attn, lse = binding.v2_fwd_train(y["q"], y["k"], y["v"], y["lam"], softmax1=True)
    grads = binding.v2_bwd(y["q"], y["k"], y["v"], y["lam"], attn, lse, dout)
    torch.cuda.synchronize()
    _check_grads(grads, _cpu(y["q"], y["k"], y["v"], y["lam"], dout), "softmax1", softmax1=True)


def test_backward_deterministic_and_strided():
    """Two runs give identical bits; q/k/v/dout given as [B,H,T,d] views give
    the same gradients as contiguous [B,T,H,d]."""
    y, dout = _inputs(1, 200, 16, 2, 64, seed=910)
    _, attn, lse = binding.v2_fwd_train(y["q"], y["k"], y["v"], y["lam"])
    g1 = binding.v2_bwd(y["q"], y["k"], y["v"], y["lam"], attn, lse, dout)
    g2 = binding.v2_bwd(y["q"], y["k"], y["v"], y["lam"], attn, lse, dout)
    tr = lambda x: x.transpose(1, 2).contiguous().transpose(1, 2)
    g3 = binding.v2_bwd(tr(y["q"]), tr(y["k"]), tr(y["v"]), y["lam"], tr(attn), lse, tr(dout))
    torch.cuda.synchronize()
    for a, b, c in zip(g1, g2, g3):
        assert torch.equal(a, b)
        assert torch.equal(a, c)


def test_backward_full_size_properties():
    """The V2 prefill workload (T = 8192, 64 query heads, 8 kv heads): the sum
    of dv over the keys equals the sum over rows and the group's heads of
    d attn (rows of P sum to one), and sampled dlam entries equal
    -s(1-s)<dout, attn_odd> from the training forward's attn."""
    w = workloads.WORKLOADS["v2_prefill_B1_T8192_Hq64_Hkv8_d128"]
    y = workloads.inputs_for(w, DEV)
    g = torch.Generator(device=DEV).manual_seed(4321)
    dout = torch.randn((w.B, w.T, w.Hq // 2, w.d), generator=g, device=DEV).to(torch.bfloat16)
    _, attn, lse = binding.v2_fwd_train(y["q"], y["k"], y["v"], y["lam"])
    dq, dk, dv, dlam = binding.v2_bwd(y["q"], y["k"], y["v"], y["lam"], attn, lse, dout)
    torch.cuda.synchronize()
    s = torch.sigmoid(y["lam"].double())
    da = torch.zeros((w.B, w.T, w.Hq, w.d), dtype=torch.float64, device=DEV)
    da[:, :, 0::2] = dout.double()
    da[:, :, 1::2] = -s[..., None] * dout.double()
    G = w.Hq // w.Hkv
    want = da.reshape(w.B, w.T, w.Hkv, G, w.d).sum(dim=(1, 3))  # [B, Hkv, d]
    got = dv.double().sum(dim=1)
    err = (got - want).abs() / (want.abs() + want.abs().mean())
    assert err.max().item() < 2e-2, err.max().item()
    want_l = -s * (1 - s) * (dout.double() * attn[:, :, 1::2].double()).sum(-1)
    assert (dlam.double() - want_l).abs().max().item() < 1e-2 * max(1.0, want_l.abs().max().item())
    for t in (0, 4097, 8191):  # sampled attn rows against the oracle's forward rows
        idx = np.array([[0, t, p] for p in (0, 17)])
        ra = oracle.v2_rows(*_cpu(y["q"], y["k"], y["v"], y["lam"]), idx)
        sg = 1.0 / (1.0 + np.exp(-y["lam"][0, t, [0, 17]].double().cpu().numpy()))
        got_out = attn[0, t, [0, 34]].double().cpu().numpy() - sg[:, None] * attn[0, t, [1, 35]].double().cpu().numpy()
        assert np.abs(got_out - ra).max() < 3e-2
    del y, dq, dk, dv, attn
    torch.cuda.empty_cache()
