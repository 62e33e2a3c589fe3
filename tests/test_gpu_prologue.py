"""Rotary embedding and the V2 lambda projection on the GPU (through the C
ABI) against the fp64 oracle in oracle/prologue.py.

Tolerances.  diffattn_rope rounds each rotated value once to bf16 (relative
2^-9) after an fp32 rotation whose angle is exact to ~2e-4 rad at the
positions tested, so every element must satisfy |x - ref| <= 2^-8 |ref| +
1e-3 max|x|.  The fused prefill and decode paths round the rotated q and k
to bf16 once each, an input-sized rounding, and are held to the forward's
bf16 bar (2e-2 + 1e-2 |ref|).  The projection's products are exact (bf16 x
bf16) and summed in fp32 over dm: |x - ref| <= 2e-5 sum_c |x_c w_c| + 1e-6.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from oracle import prologue as op
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


def _bf16(shape, seed, std=1.0):
    g = torch.Generator(device=DEV).manual_seed(seed)
    return (std * torch.randn(shape, generator=g, device=DEV)).to(torch.bfloat16)


@pytest.mark.parametrize("d,theta,pos0", [(64, 1e4, 0), (128, 1e4, 12345), (128, 5e5, 3), (8, 10.0, 100000),
                                         (24, 1e4, 7), (256, 1e4, 0)])
def test_rope_kernel(d, theta, pos0):
    x = _bf16((2, 300, 3, d), seed=2000 + d)
    got = binding.rope(x, theta=theta, pos0=pos0)
    inplace = x.clone()
    binding.rope(inplace, theta=theta, pos0=pos0, out=inplace)
    torch.cuda.synchronize()
    assert torch.equal(got, inplace)
    ref = op.rope(x.cpu(), theta=theta, pos0=pos0)
    g = host64(got)
    tol = 2.0 ** -8 * np.abs(ref) + 1e-3 * np.abs(host64(x)).max()
    assert np.all(np.abs(g - ref) <= tol), np.abs(g - ref).max()


def test_rope_kernel_strided():
    """[B,H,T,d] storage passed as a strided [B,T,H,d] view."""
    x = _bf16((2, 3, 77, 64), seed=2100).transpose(1, 2)
    got = binding.rope(x, theta=1e4, pos0=5)
    torch.cuda.synchronize()
    ref = op.rope(x.cpu(), theta=1e4, pos0=5)
    assert np.all(np.abs(host64(got) - ref) <= 2.0 ** -8 * np.abs(ref) + 1e-3 * np.abs(ref).max())


@pytest.mark.parametrize("T,G,d", [(1, 2, 128), (77, 8, 128), (300, 2, 64), (1029, 4, 128)])
def test_v2_prefill_rope(T, G, d):
    Hkv = 2
    y = workloads.v2_inputs(1, T, G * Hkv, Hkv, d, torch.bfloat16, seed=2200 + T, device=DEV)
    got = binding.v2_fwd(y["q"], y["k"], y["v"], y["lam"], theta=1e4)
    plain = binding.v2_fwd(y["q"], y["k"], y["v"], y["lam"])
    torch.cuda.synchronize()
    ref = op.v2_fwd_rope(*[y[n].cpu() for n in ("q", "k", "v", "lam")], theta=1e4)
    assert_bf16_close(got, ref, f"v2 rope T{T} G{G} d{d}")
    if T > 1:  # the rotation is applied (not a no-op)
        assert not torch.equal(got, plain)


@pytest.mark.parametrize("T,d,layer", [(1, 64, 0), (130, 64, 5), (257, 128, 14)])
def test_v1_prefill_rope(T, d, layer):
    x = workloads.v1_inputs(2, 2, T, d, torch.bfloat16, seed=2300 + T, device=DEV)
    args = [x[n] for n in ("q1", "q2", "k1", "k2", "v", "lq1", "lk1", "lq2", "lk2")]
    got = binding.v1_fwd(*args, layer, theta=1e4)
    torch.cuda.synchronize()
    ref = op.v1_fwd_rope(*[a.cpu() for a in args], layer, theta=1e4)
    assert_bf16_close(got, ref, f"v1 rope T{T} d{d}")


def test_decode_rope_dense():
    B, L, Hq, Hkv, d = 3, 1500, 16, 2, 128
    g = torch.Generator(device=DEV).manual_seed(2400)
    q = torch.randn((B, Hq, d), generator=g, device=DEV).to(torch.bfloat16)
    k = torch.randn((B, L, Hkv, d), generator=g, device=DEV).to(torch.bfloat16)
    v = torch.randn((B, L, Hkv, d), generator=g, device=DEV).to(torch.bfloat16)
    lam = torch.randn((B, Hq // 2), generator=g, device=DEV)
    # the cache holds rotated keys: rotated here by the oracle, then stored as bf16
    k_rot = torch.tensor(op.rope(k.cpu(), theta=1e4)).to(torch.bfloat16).to(DEV)
    got = binding.v2_decode(q, k_rot, v, lam, theta=1e4)
    torch.cuda.synchronize()
    ref = op.v2_decode_rope(q.cpu(), k_rot.cpu(), v.cpu(), lam.cpu(), theta=1e4)
    assert_bf16_close(got, ref, "decode rope")


def test_decode_rope_paged_multi():
    B, max_len, page, nq, Hq, Hkv, d = 4, 700, 16, 3, 16, 2, 128
    x = workloads.paged_decode_inputs(B, max_len, page, Hq, Hkv, d, torch.bfloat16, seed=2500, device=DEV, nq=nq)
    lens = x["seq_lens"].cpu().numpy()
    table = x["block_table"].cpu().numpy()
    # rotate each stored key at its position in its sequence (oracle), as a cache append would
    kp = x["k_pages"].cpu().double().numpy().copy()
    for b in range(B):
        for t in range(int(lens[b])):
            pg, row = table[b, t // page], t % page
            kp[pg, row] = op.rope(kp[pg, row][None, None], theta=1e4, pos0=t)[0, 0]
    k_rot = torch.tensor(kp).to(torch.bfloat16).to(DEV)
    got = binding.v2_decode_paged(x["q"], k_rot, x["v_pages"], x["block_table"], x["seq_lens"], x["lam"], max_len,
                                  theta=1e4)
    torch.cuda.synchronize()
    ref = op.v2_decode_paged_rope(x["q"].cpu(), k_rot.cpu(), x["v_pages"].cpu(), table, lens, x["lam"].cpu(),
                                  theta=1e4)
    assert_bf16_close(got, ref, "paged multi decode rope")


def test_decode_rope_matches_rope_kernel_cache():
    """A cache written by diffattn_rope (the GPU's own rotation) gives the
    same decode as the oracle over that cache."""
    B, L, Hq, Hkv, d = 2, 333, 8, 2, 64
    g = torch.Generator(device=DEV).manual_seed(2600)
    q = torch.randn((B, Hq, d), generator=g, device=DEV).to(torch.bfloat16)
    k = torch.randn((B, L, Hkv, d), generator=g, device=DEV).to(torch.bfloat16)
    v = torch.randn((B, L, Hkv, d), generator=g, device=DEV).to(torch.bfloat16)
    lam = torch.randn((B, Hq // 2), generator=g, device=DEV)
    k_rot = binding.rope(k, theta=1e4)
    got = binding.v2_decode(q, k_rot, v, lam, theta=1e4)
    torch.cuda.synchronize()
    ref = op.v2_decode_rope(q.cpu(), op.rope(k.cpu(), theta=1e4), v.cpu(), lam.cpu(), theta=1e4)
    assert_bf16_close(got, ref, "decode over a diffattn_rope cache")


@pytest.mark.parametrize("B,T,dm,P", [(1, 8192, 4096, 32), (2, 77, 256, 20), (1, 33, 128, 70)])
def test_lambda_proj(B, T, dm, P):
    x = _bf16((B, T, dm), seed=2700 + dm)
    w = _bf16((P, dm), seed=2701 + dm, std=1.0 / math.sqrt(dm))
    got = binding.v2_lambda_proj(x, w)
    torch.cuda.synchronize()
    xd, wd = host64(x), host64(w)
    ref = op.lambda_proj(x.cpu(), w.cpu())
    scale = np.abs(xd) @ np.abs(wd).T
    assert np.all(np.abs(host64(got) - ref) <= 2e-5 * scale + 1e-6), np.abs(host64(got) - ref).max()


def test_lambda_proj_feeds_the_prefill():
    """x -> logits on the GPU -> V2 prefill equals the oracle's projection
    followed by the oracle prefill."""
    B, T, Hq, Hkv, d, dm = 1, 200, 8, 2, 128, 512
    y = workloads.v2_inputs(B, T, Hq, Hkv, d, torch.bfloat16, seed=2800, device=DEV)
    x = _bf16((B, T, dm), seed=2801)
    w = _bf16((Hq // 2, dm), seed=2802, std=1.0 / math.sqrt(dm))
    lam = binding.v2_lambda_proj(x, w)
    got = binding.v2_fwd(y["q"], y["k"], y["v"], lam)
    torch.cuda.synchronize()
    ref = oracle.v2_fwd(*[y[n].cpu() for n in ("q", "k", "v")], op.lambda_proj(x.cpu(), w.cpu()))
    assert_bf16_close(got, ref, "projection + prefill")


# ---- the off-by-one softmax with the rotary embedding ----------------------------

@pytest.mark.parametrize("kind", ["v1", "v2"])
def test_prefill_rope_softmax1(kind):
    if kind == "v1":
        x = workloads.v1_inputs(2, 2, 200, 64, torch.bfloat16, seed=2900, device=DEV)
        args = [x[n] for n in ("q1", "q2", "k1", "k2", "v", "lq1", "lk1", "lq2", "lk2")]
        got = binding.v1_fwd(*args, 3, theta=1e4, softmax1=True)
        plain = binding.v1_fwd(*args, 3, theta=1e4)
        ref = op.v1_fwd_rope(*[a.cpu() for a in args], 3, theta=1e4, softmax1=True)
    else:
        y = workloads.v2_inputs(1, 300, 8, 2, 128, torch.bfloat16, seed=2901, device=DEV)
        got = binding.v2_fwd(y["q"], y["k"], y["v"], y["lam"], theta=1e4, softmax1=True)
        plain = binding.v2_fwd(y["q"], y["k"], y["v"], y["lam"], theta=1e4)
        ref = op.v2_fwd_rope(*[y[n].cpu() for n in ("q", "k", "v", "lam")], theta=1e4, softmax1=True)
    torch.cuda.synchronize()
    assert_bf16_close(got, ref, f"{kind} rope softmax1")
    assert not torch.equal(got, plain)


def test_decode_rope_softmax1_dense_and_paged():
    B, L, Hq, Hkv, d = 2, 900, 8, 2, 128
    g = torch.Generator(device=DEV).manual_seed(2902)
    q = torch.randn((B, Hq, d), generator=g, device=DEV).to(torch.bfloat16)
    k = torch.randn((B, L, Hkv, d), generator=g, device=DEV).to(torch.bfloat16)
    v = torch.randn((B, L, Hkv, d), generator=g, device=DEV).to(torch.bfloat16)
    lam = torch.randn((B, Hq // 2), generator=g, device=DEV)
    got = binding.v2_decode(q, k, v, lam, theta=1e4, softmax1=True)
    # the same cache as 16-token pages laid end to end
    page = 16
    npg = (L + page - 1) // page
    pool_k = torch.zeros((B * npg, page, Hkv, d), dtype=torch.bfloat16, device=DEV)
    pool_v = torch.zeros_like(pool_k)
    for b in range(B):
        pool_k.view(B, npg * page, Hkv, d)[b, :L] = k[b]
        pool_v.view(B, npg * page, Hkv, d)[b, :L] = v[b]
    table = torch.arange(B * npg, dtype=torch.int32, device=DEV).reshape(B, npg)
    lens = torch.full((B,), L, dtype=torch.int32, device=DEV)
    gotp = binding.v2_decode_paged(q, pool_k, pool_v, table, lens, lam, L, theta=1e4, softmax1=True)
    torch.cuda.synchronize()
    ref = op.v2_decode_rope(q.cpu(), k.cpu(), v.cpu(), lam.cpu(), theta=1e4, softmax1=True)
    assert_bf16_close(got, ref, "decode rope softmax1")
    assert_bf16_close(gotp, ref, "paged decode rope softmax1")


# ---- the benchmarked RoPE workloads at full size ------------------------------------

def test_v2_prefill_rope_full_sampled():
    """The V2 prefill workload with the rotary embedding (B 1, T 8192, 64 / 8
    heads, d 128): sampled rows, including the last positions, against the
    oracle's rotation (fp64) and prefill rows."""
    w = workloads.WORKLOADS["v2_prefill_rope_B1_T8192_Hq64_Hkv8_d128"]
    y = workloads.inputs_for(w, DEV)
    got = binding.v2_fwd(y["q"], y["k"], y["v"], y["lam"], theta=1e4)
    torch.cuda.synchronize()
    rng = np.random.default_rng(4)
    idx = np.stack([np.zeros(64, np.int64), rng.integers(0, w.T, 64), rng.integers(0, w.Hq // 2, 64)], 1)
    idx[:6, 1] = [0, 1, 4095, 4096, 8190, 8191]
    q, k = op.rope(y["q"].cpu(), 1e4), op.rope(y["k"].cpu(), 1e4)
    ref = oracle.v2_rows(q, k, y["v"].cpu(), y["lam"].cpu(), idx)
    assert_bf16_close(host64(got)[idx[:, 0], idx[:, 1], idx[:, 2]], ref, "v2 rope prefill T8192 sampled rows")


def test_decode_rope_full_sampled():
    """The V2 decode workload with q rotated to position 32767 in the kernel
    (B 64, L 32768, 64 / 8 heads, d 128): three sequences against the
    oracle (the cache read as holding rotated keys)."""
    w = workloads.WORKLOADS["v2_decode_rope_B64_L32768_Hq64_Hkv8_d128"]
    x = workloads.inputs_for(w, DEV)
    got = binding.v2_decode(x["q"], x["k"], x["v"], x["lam"], theta=1e4)
    torch.cuda.synchronize()
    bs = [0, 31, 63]
    ref = op.v2_decode_rope(*[x[n][bs].cpu() for n in ("q", "k", "v", "lam")], theta=1e4)
    assert_bf16_close(host64(got)[bs], ref, "decode rope L32768 sampled sequences")
    del x
    torch.cuda.empty_cache()
