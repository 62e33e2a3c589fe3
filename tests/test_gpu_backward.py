"""DIFF V2 and DIFF V1 training forward and backward (HIP, through the C ABI)
against the fp64 oracle in oracle/backward.py.

Tolerance (gpu_util.assert_grad_close): every element within the forward's
bf16 bar, 2e-2 + 1e-2 |ref| (+ 1e-4, the fp32 bar, for exact zeros), whose
absolute part grows with the gradient tensor's RMS once that passes 1 and is
raised to twice the worst error of the pages' module run in bf16 by PyTorch
(tests/bf16_module.py) where bf16 arithmetic itself costs more than that;
and every tensor within a relative L2 error of 1e-2.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from oracle import backward as ob
from differential_attention_diffattn_amd import binding, workloads
import bf16_module
from gpu_util import assert_bf16_close, assert_grad_close, host64

pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a visible MI355X"
    binding.load_library()
    yield
    torch.cuda.synchronize()


def _check_grads(grads, ins, what, softmax1=False):
    ref = ob.v2_bwd(*ins, softmax1=softmax1)
    yard = bf16_module.v2_grads(*ins, softmax1=softmax1)
    for name, got, r, y in zip(("dq", "dk", "dv", "dlam"), grads, ref, yard):
        assert_grad_close(got, r, f"{name} {what}", yard=y)


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
@pytest.mark.parametrize("G,d", [(2, 64), (8, 128), (4, 64), (2, 128), (6, 64)])
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


# ==== DIFF V1 =======================================================================
#
V1_GRADS = ("dq1", "dq2", "dk1", "dk2", "dv", "dlq1", "dlk1", "dlq2", "dlk2")


def _v1_in(B, H, T, d, seed):
    x = workloads.v1_inputs(B, H, T, d, torch.bfloat16, seed=seed, device=DEV)
    g = torch.Generator(device=DEV).manual_seed(seed + 99)
    dout = torch.randn((B, T, H, 2 * d), generator=g, device=DEV).to(torch.bfloat16)
    args = [x[k] for k in ("q1", "q2", "k1", "k2", "v", "lq1", "lk1", "lq2", "lk2")]
    return args, dout


def _v1_check(grads, args, layer, dout, what, softmax1=False):
    cpu = [a.cpu() for a in args]
    ref = ob.v1_bwd(*cpu, layer, dout.cpu(), softmax1=softmax1)
    yard = bf16_module.v1_grads(*cpu, layer, dout.cpu(), softmax1=softmax1)
    for name, got, r, y in zip(V1_GRADS, grads, ref, yard):
        assert_grad_close(got, r, f"{name} {what}", yard=y)


@pytest.mark.parametrize("s1", [False, True])
@pytest.mark.parametrize("T,d", [(1, 64), (33, 128), (300, 64), (200, 128)])
def test_v1_fwd_train(T, d, s1):
    """out is the inference forward's, bit for bit; attn1, attn2 and lse match the oracle."""
    args, _ = _v1_in(2, 2, T, d, seed=1000 + T + d)
    layer = 4
    out, a1, a2, lse = binding.v1_fwd_train(*args, layer, softmax1=s1)
    inf = binding.v1_fwd(*args, layer, softmax1=s1)
    torch.cuda.synchronize()
    assert torch.equal(out, inf)
    r_out, r_a1, r_a2, r_lse = ob.v1_fwd_train(*[a.cpu() for a in args], layer, softmax1=s1)
    assert_bf16_close(a1, r_a1, f"attn1 T{T} d{d}")
    assert_bf16_close(a2, r_a2, f"attn2 T{T} d{d}")
    assert np.abs(host64(lse) - r_lse).max() < 1e-2


@pytest.mark.parametrize("T", [1, 31, 33, 100, 300])
@pytest.mark.parametrize("d,layer", [(64, 0), (128, 14), (64, 11)])
def test_v1_backward(T, d, layer):
    B = 2 if T < 200 else 1
    args, dout = _v1_in(B, 2, T, d, seed=1100 + T + d + layer)
    _, a1, a2, lse = binding.v1_fwd_train(*args, layer)
    grads = binding.v1_bwd(*args, layer, a1, a2, lse, dout)
    torch.cuda.synchronize()
    _v1_check(grads, args, layer, dout, f"T{T} d{d} layer{layer}")


@pytest.mark.parametrize("d", [64, 128])
def test_v1_backward_xcd_grouped_ragged(d):
    """(batch, head) units divisible by 8 (the grid groups a head's work on
    one XCD) with a ragged T, every gradient element against the oracle."""
    args, dout = _v1_in(2, 4, 300, d, seed=1150 + d)
    _, a1, a2, lse = binding.v1_fwd_train(*args, 3)
    grads = binding.v1_bwd(*args, 3, a1, a2, lse, dout)
    torch.cuda.synchronize()
    _v1_check(grads, args, 3, dout, f"B2 H4 T300 d{d}")


def test_v1_backward_softmax1():
    args, dout = _v1_in(1, 2, 150, 64, seed=1200)
    _, a1, a2, lse = binding.v1_fwd_train(*args, 2, softmax1=True)
    grads = binding.v1_bwd(*args, 2, a1, a2, lse, dout)
    torch.cuda.synchronize()
    _v1_check(grads, args, 2, dout, "softmax1", softmax1=True)


def test_v1_backward_deterministic_and_strided():
    """Two runs give identical bits; q/k/v given as [B,T,H,d] storage (strided
    [B,H,T,d] views) give the same gradients as contiguous inputs."""
    args, dout = _v1_in(2, 3, 160, 64, seed=1300)
    _, a1, a2, lse = binding.v1_fwd_train(*args, 1)
    g1 = binding.v1_bwd(*args, 1, a1, a2, lse, dout)
    g2 = binding.v1_bwd(*args, 1, a1, a2, lse, dout)
    tr = lambda x: x.transpose(1, 2).contiguous().transpose(1, 2)
    g3 = binding.v1_bwd(*[tr(a) for a in args[:5]], *args[5:], 1, a1, a2, lse, dout)
    torch.cuda.synchronize()
    for a, b, c in zip(g1, g2, g3):
        assert torch.equal(a, b)
        assert torch.equal(a, c)


def test_v1_backward_headline_shape():
    """The GPT-2-small V1 shape (B 8, 6 differential heads, T 1024, d 64),
    every gradient element against the oracle."""
    w = workloads.WORKLOADS["v1_gpt2small_B8_H6_T1024_d64"]
    x = workloads.inputs_for(w, DEV)
    args = [x[k] for k in ("q1", "q2", "k1", "k2", "v", "lq1", "lk1", "lq2", "lk2")]
    g = torch.Generator(device=DEV).manual_seed(5555)
    dout = torch.randn((w.B, w.T, w.H, 2 * w.d), generator=g, device=DEV).to(torch.bfloat16)
    _, a1, a2, lse = binding.v1_fwd_train(*args, 6)
    grads = binding.v1_bwd(*args, 6, a1, a2, lse, dout)
    torch.cuda.synchronize()
    _v1_check(grads, args, 6, dout, "headline shape")


def test_v1_backward_3b_shape_sampled_heads():
    """The 3B-class V1 shape (B 2, 12 differential heads, T 4096, d 128):
    dq, dk, dv of two (b, h) heads against the oracle run on those heads
    alone (each head's gradients depend only on its own inputs and lambda)."""
    w = workloads.WORKLOADS["v1_3b_B2_H12_T4096_d128"]
    x = workloads.inputs_for(w, DEV)
    args = [x[k] for k in ("q1", "q2", "k1", "k2", "v", "lq1", "lk1", "lq2", "lk2")]
    g = torch.Generator(device=DEV).manual_seed(5556)
    dout = torch.randn((w.B, w.T, w.H, 2 * w.d), generator=g, device=DEV).to(torch.bfloat16)
    _, a1, a2, lse = binding.v1_fwd_train(*args, 14)
    grads = binding.v1_bwd(*args, 14, a1, a2, lse, dout)
    torch.cuda.synchronize()
    for b, h in ((0, 0), (1, 11)):
        sub = [a[b:b + 1, h:h + 1].cpu() for a in args[:5]] + [a.cpu() for a in args[5:]]
        dsub = dout[b:b + 1, :, h:h + 1].cpu()
        ref = ob.v1_bwd(*sub, 14, dsub)
        yard = bf16_module.v1_grads(*sub, 14, dsub)
        for name, got, r, y in list(zip(V1_GRADS, grads, ref, yard))[:5]:
            assert_grad_close(got[b:b + 1, h:h + 1], r, f"{name} b{b} h{h}", yard=y)


# ==== regressions and full-size checks ==================================================

@pytest.mark.parametrize("G,d", [(2, 64), (8, 128)])
def test_v2_row0_dq_is_zero(G, d):
    """Row 0 of every head sees one key, so its P is 1 and dS = dP - D = 0:
    dq there is exactly 0.  The kernels form G = dout v^T and E = <dout,
    attn> from the same bf16 dout and apply the odd head's -sigmoid(lam) in
    fp32 to both, so what is left is fp32 summation order."""
    y, dout = _inputs(2, 300, G * 2, 2, d, seed=930 + G)
    _, attn, lse = binding.v2_fwd_train(y["q"], y["k"], y["v"], y["lam"])
    dq = binding.v2_bwd(y["q"], y["k"], y["v"], y["lam"], attn, lse, dout)[0]
    torch.cuda.synchronize()
    assert dq[:, 0].abs().max().item() <= 1e-4, dq[:, 0].abs().max().item()


def test_v1_row0_dq_is_zero():
    args, dout = _v1_in(2, 3, 200, 64, seed=940)
    _, a1, a2, lse = binding.v1_fwd_train(*args, 5)
    grads = binding.v1_bwd(*args, 5, a1, a2, lse, dout)
    torch.cuda.synchronize()
    for g in grads[:2]:
        assert g[:, :, 0].abs().max().item() <= 1e-4, g[:, :, 0].abs().max().item()


def test_backward_full_size_sampled():
    """The V2 prefill workload (B 1, T 8192, 64 query heads, 8 kv heads):
    for two kv groups, dq of sampled rows of all 8 heads, dk and dv of
    sampled keys and every dlam of the group's pairs, against the sampled
    oracle run on that group's inputs alone (a group's gradients depend only
    on its own q heads, k, v, lambda logits and dout)."""
    w = workloads.WORKLOADS["v2_prefill_B1_T8192_Hq64_Hkv8_d128"]
    y = workloads.inputs_for(w, DEV)
    g = torch.Generator(device=DEV).manual_seed(4321)
    dout = torch.randn((w.B, w.T, w.Hq // 2, w.d), generator=g, device=DEV).to(torch.bfloat16)
    _, attn, lse = binding.v2_fwd_train(y["q"], y["k"], y["v"], y["lam"])
    dq, dk, dv, dlam = binding.v2_bwd(y["q"], y["k"], y["v"], y["lam"], attn, lse, dout)
    torch.cuda.synchronize()
    G = w.Hq // w.Hkv
    ts = [0, 1, 2, 31, 32, 127, 128, 1000, 4095, 4096, 8190, 8191]
    js = [0, 1, 31, 32, 2047, 4096, 8000, 8191]
    for grp in (0, 5):
        hs, ps = slice(grp * G, (grp + 1) * G), slice(grp * G // 2, (grp + 1) * G // 2)
        sub = [y["q"][:, :, hs], y["k"][:, :, grp:grp + 1], y["v"][:, :, grp:grp + 1], y["lam"][:, :, ps],
               dout[:, :, ps]]
        rows = [(0, t, h) for t in ts for h in range(G)]
        keys = [(0, j, 0) for j in js]
        rq, rk, rv, rl = ob.v2_bwd_sampled(*_cpu(*sub), rows, keys)
        got_q = torch.stack([dq[0, t, grp * G + h] for _, t, h in rows])
        got_k = torch.stack([dk[0, j, grp] for _, j, _ in keys])
        got_v = torch.stack([dv[0, j, grp] for _, j, _ in keys])
        assert_grad_close(got_q, rq, f"dq group {grp}")
        assert_grad_close(got_k, rk, f"dk group {grp}")
        assert_grad_close(got_v, rv, f"dv group {grp}")
        assert_grad_close(dlam[:, :, ps], rl, f"dlam group {grp}")
        assert dq[0, 0, hs].abs().max().item() <= 1e-4  # row 0: exactly 0
    del y, dq, dk, dv, attn
    torch.cuda.empty_cache()
