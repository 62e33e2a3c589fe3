"""Parity of the HIP path (through the C ABI) against the fp64 oracle.

Small cases compare every element; full-size workloads (the shapes and the
launch configuration the benchmark times) compare sampled rows, which the
oracle computes one by one, plus closed forms that hold at any size.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from differential_attention_diffattn_amd import binding, workloads
from differential_attention_diffattn_amd.workloads import WORKLOADS
from gpu_util import assert_bf16_close, assert_fp32_close, host64, rel_l2

pytestmark = pytest.mark.gpu
DEV = "cuda"
V1_NAMES = ("q1", "q2", "k1", "k2", "v", "lq1", "lk1", "lq2", "lk2")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a visible MI355X"
    binding.load_library()
    yield
    torch.cuda.synchronize()


def _v1_run(x, layer, out=None, softmax1=False):
    o = binding.v1_fwd(*[x[n] for n in V1_NAMES], layer, out=out, softmax1=softmax1)
    torch.cuda.synchronize()
    return o


def _v1_cpu(x):
    return [x[n].cpu() for n in V1_NAMES]


# ------------------------------------------------------------------ V1 fp32

def test_v1_fp32_workload_full():
    w = WORKLOADS["v1_fp32_B1_H2_T128_d32"]
    x = workloads.inputs_for(w, DEV)
    out = _v1_run(x, w.layers[0])
    ref = oracle.v1_fwd(*_v1_cpu(x), w.layers[0])
    assert_fp32_close(out, ref, w.name)


@pytest.mark.parametrize("d", [32, 64, 128])
@pytest.mark.parametrize("T", [1, 33, 200])
def test_v1_fp32_shapes(d, T):
    x = workloads.v1_inputs(2, 3, T, d, torch.float32, seed=100 + d + T, device=DEV)
    out = _v1_run(x, 7)
    assert_fp32_close(out, oracle.v1_fwd(*_v1_cpu(x), 7), f"fp32 d{d} T{T}")


# ------------------------------------------------------------------ V1 bf16

@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("T", [1, 31, 32, 33, 129, 300])
def test_v1_bf16_ragged(d, T):
    x = workloads.v1_inputs(2, 3, T, d, torch.bfloat16, seed=200 + d + T, device=DEV)
    out = _v1_run(x, 4)
    assert_bf16_close(out, oracle.v1_fwd(*_v1_cpu(x), 4), f"bf16 d{d} T{T}")


@pytest.mark.parametrize("d", [64, 128])
def test_v1_bf16_peaked_scores(d):
    """Scores spread over hundreds of log2 units: every row's maximum must be
    taken over all of its keys (both lane halves of a score tile), or the
    exponentials overflow."""
    x = workloads.v1_inputs(2, 3, 300, d, torch.bfloat16, seed=250 + d, device=DEV)
    for n in ("q1", "q2", "k1", "k2"):
        x[n].mul_(6)
    out = _v1_run(x, 2)
    assert_bf16_close(out, oracle.v1_fwd(*_v1_cpu(x), 2), f"peaked d{d}")


def test_v1_fp32_peaked_scores():
    x = workloads.v1_inputs(1, 2, 200, 64, torch.float32, seed=260, device=DEV)
    for n in ("q1", "q2", "k1", "k2"):
        x[n].mul_(6)
    out = _v1_run(x, 2)
    assert_fp32_close(out, oracle.v1_fwd(*_v1_cpu(x), 2), "fp32 peaked")


def _rising(k, slope):
    """k[..., j, 0] = slope * j along the token axis (axis -2 of [.., T, d])."""
    T = k.shape[-2]
    k[..., 0] = (slope * torch.arange(T, device=k.device, dtype=torch.float32)).to(k.dtype)


@pytest.mark.parametrize("d", [64, 128])
def test_v1_rising_scores_rescale_every_block(d):
    """Scores that grow with the key index: every 32-key block raises each
    row's maximum by ~12 log2 units, so the exact rescale path runs on
    nearly every block (and on both lane halves)."""
    x = workloads.v1_inputs(2, 2, 300, d, torch.bfloat16, seed=270 + d, device=DEV)
    s = math.sqrt(d) / 8.0
    for n in ("q1", "q2"):
        x[n][..., 0] = 8.0 * s
    for n in ("k1", "k2"):
        _rising(x[n], 0.26)
    out = _v1_run(x, 5)
    assert_bf16_close(out, oracle.v1_fwd(*_v1_cpu(x), 5), f"rising d{d}")


def test_v1_bf16_gpt2small_full():
    """GPT-2-small shape, every element of layer 0, then sampled rows of
    every layer of the 0..11 sweep (only lambda_init changes)."""
    w = WORKLOADS["v1_gpt2small_B8_H6_T1024_d64"]
    x = workloads.inputs_for(w, DEV)
    xc = _v1_cpu(x)
    out = _v1_run(x, 0)
    assert_bf16_close(out, oracle.v1_fwd(*xc, 0), "gpt2small layer 0")
    rng = np.random.default_rng(0)
    bhi = np.stack([rng.integers(0, w.B, 48), rng.integers(0, w.H, 48), rng.integers(0, w.T, 48)], 1)
    bhi[:4, 2] = [0, 31, 1022, 1023]
    for layer in w.layers[1:]:
        out = _v1_run(x, layer)
        ref = oracle.v1_rows(*xc, layer, bhi)
        got = host64(out)[bhi[:, 0], bhi[:, 2], bhi[:, 1]]
        assert_bf16_close(got, ref, f"gpt2small layer {layer}")


def _v1_rows_sample(w, rng, n):
    b = rng.integers(0, w.B, n)
    h = rng.integers(0, w.H, n)
    i = rng.integers(0, w.T, n)
    fixed = [0, 1, 31, 32, 127, 128, w.T - 2, w.T - 1]
    i[: len(fixed)] = fixed
    return np.stack([b, h, i], 1)


def test_v1_bf16_3b_sampled():
    w = WORKLOADS["v1_3b_B2_H12_T4096_d128"]
    x = workloads.inputs_for(w, DEV)
    out = _v1_run(x, w.layers[0])
    bhi = _v1_rows_sample(w, np.random.default_rng(1), 96)
    ref = oracle.v1_rows(*_v1_cpu(x), w.layers[0], bhi)
    got = host64(out)[bhi[:, 0], bhi[:, 2], bhi[:, 1]]
    assert_bf16_close(got, ref, w.name)


# ------------------------------------------------- V1 cancellation regime
# Hacker News "Differential Transformer" board, posts #131 and #135: with
# identical maps A1 = A2 the method gives (1 - lam) A, and lam may take any
# sign.  Where the two maps nearly agree and lam is near 1, D = A1 V - lam A2 V
# cancels and the RMSNorm scales it back to O(1); the kernel recomputes such
# rows exactly, so every case below holds the bf16 bar.

def _set_lambda(x, layer, target):
    """Rewrite the four lambda vectors (fp32, constant) so that
    exp(lq1.lk1) - exp(lq2.lk2) + lambda_init = target."""
    d = x["lq1"].numel()
    li = oracle.lambda_init(layer)
    for n in ("lq1", "lk1", "lq2", "lk2"):
        x[n].zero_()
    if target >= li:  # exp(a) = 1 + target - li, exp(b) = 1
        c = math.sqrt(math.log1p(target - li) / d)
        x["lq1"].fill_(c), x["lk1"].fill_(c)
    else:             # exp(a) = 1, exp(b) = 1 + li - target
        c = math.sqrt(math.log1p(li - target) / d)
        x["lq2"].fill_(c), x["lk2"].fill_(c)
    got = oracle.v1_lambda(*[x[n].cpu() for n in ("lq1", "lk1", "lq2", "lk2")], layer)
    assert abs(got - target) < 1e-6, (got, target)


def _sdpa_rmsnorm(q, k, v, lam, li):
    """(1 - lambda_init) RMSNorm((1 - lam) causal_attention(q, k, v)), fp64 on
    the CPU with torch's SDPA: identical branches in closed form."""
    qd, kd, vd = [t.cpu().double() for t in (q, k, v)]
    a = torch.nn.functional.scaled_dot_product_attention(qd, kd, vd, is_causal=True)  # [B,H,T,2d]
    D = (1.0 - lam) * a
    y = D / torch.sqrt((D * D).mean(-1, keepdim=True) + 1e-5) * (1.0 - li)
    return y.transpose(1, 2).numpy()  # [B,T,H,2d]


@pytest.mark.parametrize("target", [None, 0.95, 1.0, 1.05, -0.5])
@pytest.mark.parametrize("d", [64, 128])
def test_v1_identical_branches(d, target):
    """Q2 = Q1, K2 = K1: out = (1 - li) RMSNorm((1 - lam) A V) (post #131),
    for the drawn lambda and for lambda built to 0.95, 1, 1.05 and -0.5."""
    layer = 6
    x = workloads.v1_inputs(2, 3, 300, d, torch.bfloat16, seed=1400 + d, device=DEV)
    x["q2"].copy_(x["q1"]), x["k2"].copy_(x["k1"])
    if target is not None:
        _set_lambda(x, layer, target)
    lam = oracle.v1_lambda(*[x[n].cpu() for n in ("lq1", "lk1", "lq2", "lk2")], layer)
    out = _v1_run(x, layer)
    assert_bf16_close(out, oracle.v1_fwd(*_v1_cpu(x), layer), f"identical d{d} lam {lam:.4f}")
    ref = _sdpa_rmsnorm(x["q1"], x["k1"], x["v"], lam, oracle.lambda_init(layer))
    assert_bf16_close(out, ref, f"identical d{d} lam {lam:.4f} vs SDPA closed form")


@pytest.mark.parametrize("d", [64, 128])
def test_v1_lambda_zero_reduces_to_attention(d):
    """lambda built to 0 from the vectors: out = (1 - li) RMSNorm(A1 V), the
    standard causal attention of the first map (torch SDPA, fp64)."""
    layer = 3
    x = workloads.v1_inputs(2, 3, 257, d, torch.bfloat16, seed=1500 + d, device=DEV)
    _set_lambda(x, layer, 0.0)
    out = _v1_run(x, layer)
    assert_bf16_close(out, oracle.v1_fwd(*_v1_cpu(x), layer), f"lam 0 d{d}")
    ref = _sdpa_rmsnorm(x["q1"], x["k1"], x["v"], 0.0, oracle.lambda_init(layer))
    assert_bf16_close(out, ref, f"lam 0 d{d} vs SDPA")


@pytest.mark.parametrize("s1", [False, True])
@pytest.mark.parametrize("eps", [0.02, 0.2])
@pytest.mark.parametrize("target", [0.95, 1.0, 1.05])
@pytest.mark.parametrize("d", [64, 128])
def test_v1_near_identical_branches(d, target, eps, s1):
    """Q2 = Q1 + eps N(0,1), K2 = K1 + eps N(0,1) with lambda near 1: the maps
    nearly agree on every row and D cancels by factors of ~10 to ~1000."""
    layer = 9
    x = workloads.v1_inputs(1, 2, 300, d, torch.bfloat16, seed=1600 + d, device=DEV)
    g = torch.Generator(device=DEV).manual_seed(1601 + d)
    for a, b in (("q2", "q1"), ("k2", "k1")):
        x[a].copy_((x[b].float() + eps * torch.randn(x[b].shape, generator=g, device=DEV)).to(torch.bfloat16))
    _set_lambda(x, layer, target)
    out = _v1_run(x, layer, softmax1=s1)
    assert_bf16_close(out, oracle.v1_fwd(*_v1_cpu(x), layer, softmax1=s1),
                      f"near-identical d{d} lam {target} eps {eps} softmax1 {s1}")


@pytest.mark.parametrize("d", [64, 128])
def test_v1_near_identical_branches_training_forward_and_rope(d):
    """The training forward's out is the inference forward's bit for bit, and
    the RoPE entry point recomputes cancelling rows with q rotated."""
    layer = 9
    x = workloads.v1_inputs(1, 2, 200, d, torch.bfloat16, seed=1700 + d, device=DEV)
    g = torch.Generator(device=DEV).manual_seed(1701 + d)
    for a, b in (("q2", "q1"), ("k2", "k1")):
        x[a].copy_((x[b].float() + 0.02 * torch.randn(x[b].shape, generator=g, device=DEV)).to(torch.bfloat16))
    _set_lambda(x, layer, 1.0)
    args = [x[n] for n in V1_NAMES]
    out, _, _, _ = binding.v1_fwd_train(*args, layer)
    inf = binding.v1_fwd(*args, layer)
    rot = binding.v1_fwd(*args, layer, theta=10000.0)
    torch.cuda.synchronize()
    assert torch.equal(out, inf)
    assert_bf16_close(inf, oracle.v1_fwd(*_v1_cpu(x), layer), f"near-identical d{d}")
    from oracle import prologue as op
    assert_bf16_close(rot, op.v1_fwd_rope(*_v1_cpu(x), layer), f"near-identical rope d{d}")


def test_v1_strided_layouts_are_bitwise_equal():
    """The interleaved layout of Wilsontomass's module (q viewed as
    [B,T,nh,2,hd], q1 = q[..., 0, :]) is passed as strided views; the
    result must equal the contiguous [B,H,T,d] call bit for bit."""
    B, H, T, d = 2, 3, 150, 64
    g = torch.Generator(device=DEV).manual_seed(5)
    q = torch.randn(B, T, H, 2, d, generator=g, device=DEV).bfloat16()
    k = torch.randn(B, T, H, 2, d, generator=g, device=DEV).bfloat16()
    v = torch.randn(B, T, H, 2 * d, generator=g, device=DEV).bfloat16()
    lam = [0.1 * torch.randn(d, generator=g, device=DEV) for _ in range(4)]
    views = [q[:, :, :, 0].transpose(1, 2), q[:, :, :, 1].transpose(1, 2),
             k[:, :, :, 0].transpose(1, 2), k[:, :, :, 1].transpose(1, 2), v.transpose(1, 2)]
    a = binding.v1_fwd(*views, *lam, 3)
    b = binding.v1_fwd(*[t.contiguous() for t in views], *lam, 3)
    out_t = torch.empty(B, H, T, 2 * d, device=DEV, dtype=torch.bfloat16).transpose(1, 2)  # strided out
    c = binding.v1_fwd(*views, *lam, 3, out=out_t)
    torch.cuda.synchronize()
    assert torch.equal(a, b) and torch.equal(a, c)
    ref = oracle.v1_fwd(*[t.cpu() for t in views], *[t.cpu() for t in lam], 3)
    assert_bf16_close(a, ref, "strided")


def test_v1_needle_on_and_past_the_diagonal():
    """Query i = a e0 and key i (visible) or i+1 (masked) = e0: the first map
    is one-hot on v_i or uniform over j <= i."""
    B, H, T, d = 1, 1, 96, 64
    x = workloads.v1_inputs(B, H, T, d, torch.bfloat16, seed=9, device=DEV)
    for name in ("q1", "q2"):
        x[name].zero_()
    x["k1"][..., 0] = 0
    for n in ("lq1", "lk1", "lq2", "lk2"):
        x[n].zero_()
    i = 45
    x["q1"][0, 0, i, 0] = 40.0 * math.sqrt(d)
    for off in (0, 1):
        k1 = x["k1"].clone()
        k1[0, 0, i + off] = 0
        k1[0, 0, i + off, 0] = 1.0
        y = dict(x, k1=k1)
        out = _v1_run(y, 0)
        ref = oracle.v1_fwd(*_v1_cpu(y), 0)
        assert_bf16_close(out, ref, f"needle offset {off}")


def test_v1_prefix_mean_closed_form_full_size():
    """Q1 = Q2 = 0 at the 3B-class shape: every visible score is 0, so
    D = (1 - lam) * prefix-mean(V) and the output has a closed form."""
    w = WORKLOADS["v1_3b_B2_H12_T4096_d128"]
    x = workloads.inputs_for(w, DEV)
    x["q1"].zero_()
    x["q2"].zero_()
    layer = w.layers[0]
    out = _v1_run(x, layer)
    lam = oracle.v1_lambda(*[x[n].cpu() for n in ("lq1", "lk1", "lq2", "lk2")], layer)
    li = oracle.lambda_init(layer)
    v = host64(x["v"])  # [B,H,T,2d]
    pm = np.cumsum(v, axis=2) / np.arange(1, w.T + 1)[None, None, :, None]
    D = (1 - lam) * pm
    ref = (1 - li) * D / np.sqrt(np.mean(D * D, -1, keepdims=True) + 1e-5)
    assert_bf16_close(out, np.transpose(ref, (0, 2, 1, 3)), "v1 prefix mean")


def test_v1_deterministic():
    w = WORKLOADS["v1_gpt2small_B8_H6_T1024_d64"]
    x = workloads.inputs_for(w, DEV)
    a = _v1_run(x, 3).clone()
    b = _v1_run(x, 3)
    assert torch.equal(a, b)


def test_v1_error_leaves_output_untouched():
    x = workloads.v1_inputs(1, 2, 64, 64, torch.bfloat16, seed=3, device=DEV)
    out = torch.full((1, 64, 2, 128), 7.0, device=DEV, dtype=torch.bfloat16)
    with pytest.raises(binding.DiffAttnError) as e:
        binding.v1_fwd(x["q1"][..., 1:], x["q2"][..., 1:], x["k1"][..., 1:], x["k2"][..., 1:],
                       torch.zeros(1, 2, 64, 126, device=DEV, dtype=torch.bfloat16),
                       *[torch.zeros(63, device=DEV) for _ in range(4)], 0, out=out[..., :126])
    assert e.value.name in ("DA_E_LAYOUT", "DA_E_UNSUPPORTED")
    torch.cuda.synchronize()
    assert torch.all(out == 7.0)


# ------------------------------------------------------------------ V2 prefill

def _v2_run(y, out=None, softmax1=False):
    o = binding.v2_fwd(y["q"], y["k"], y["v"], y["lam"], out=out, softmax1=softmax1)
    torch.cuda.synchronize()
    return o


def _v2_cpu(y):
    return [y[n].cpu() for n in ("q", "k", "v", "lam")]


@pytest.mark.parametrize("G", [2, 4, 6, 8])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("T", [1, 33, 150])
def test_v2_ragged(G, d, T):
    Hkv = 2
    y = workloads.v2_inputs(2, T, G * Hkv, Hkv, d, torch.bfloat16, seed=300 + G + d + T, device=DEV)
    out = _v2_run(y)
    assert_bf16_close(out, oracle.v2_fwd(*_v2_cpu(y)), f"v2 G{G} d{d} T{T}")


@pytest.mark.parametrize("d", [64, 128])
def test_v2_peaked_scores(d):
    y = workloads.v2_inputs(1, 300, 8, 1, d, torch.bfloat16, seed=350 + d, device=DEV)
    y["q"].mul_(6)
    y["k"].mul_(6)
    out = _v2_run(y)
    assert_bf16_close(out, oracle.v2_fwd(*_v2_cpu(y)), f"v2 peaked d{d}")


@pytest.mark.parametrize("d", [64, 128])
def test_v2_rising_scores_rescale_every_block(d):
    y = workloads.v2_inputs(1, 300, 8, 2, d, torch.bfloat16, seed=370 + d, device=DEV)
    y["q"][..., 0] = 12.0 * math.sqrt(d) / math.sqrt(128)
    k = y["k"].transpose(1, 2)  # [B, Hkv, T, d] view
    _rising(k, 0.26)
    out = _v2_run(y)
    assert_bf16_close(out, oracle.v2_fwd(*_v2_cpu(y)), f"v2 rising d{d}")


def test_v2_gate_limits():
    """Logits -inf / +inf give sigmoid 0 / 1 exactly."""
    y = workloads.v2_inputs(1, 80, 8, 1, 128, torch.bfloat16, seed=31, device=DEV)
    for val in (-math.inf, math.inf):
        y["lam"].fill_(val)
        out = _v2_run(y)
        assert_bf16_close(out, oracle.v2_fwd(*_v2_cpu(y)), f"gate {val}")


def test_v2_prefill_full_sampled():
    w = WORKLOADS["v2_prefill_B1_T8192_Hq64_Hkv8_d128"]
    y = workloads.inputs_for(w, DEV)
    out = _v2_run(y)
    rng = np.random.default_rng(2)
    n = 128
    btp = np.stack([np.zeros(n, dtype=np.int64), rng.integers(0, w.T, n), rng.integers(0, w.Hq // 2, n)], 1)
    btp[:6, 1] = [0, 1, 31, 32, w.T - 2, w.T - 1]
    ref = oracle.v2_rows(*_v2_cpu(y), btp)
    got = host64(out)[btp[:, 0], btp[:, 1], btp[:, 2]]
    assert_bf16_close(got, ref, w.name)
    # the absolute tolerance is loose for long rows (outputs shrink like
    # sqrt(e/n)); the per-row relative L2 error must stay at bf16 level
    assert rel_l2(got, ref, axis=-1).max() < 3e-2


def test_v2_prefix_mean_closed_form_full_size():
    w = WORKLOADS["v2_prefill_B1_T8192_Hq64_Hkv8_d128"]
    y = workloads.inputs_for(w, DEV)
    y["q"].zero_()
    out = _v2_run(y)
    v = host64(y["v"])  # [B,T,Hkv,d]
    pm = np.cumsum(v, axis=1) / np.arange(1, w.T + 1)[None, :, None, None]
    sig = 1.0 / (1.0 + np.exp(-host64(y["lam"])))
    G = w.Hq // w.Hkv
    ref = (1 - sig)[..., None] * np.repeat(pm, G // 2, axis=2)
    assert_bf16_close(out, ref, "v2 prefix mean")


# ------------------------------------------------------------------ V2 decode

def _dec_run(z, out=None, ws=None, softmax1=False):
    o = binding.v2_decode(z["q"], z["k"], z["v"], z["lam"], out=out, workspace=ws, softmax1=softmax1)
    torch.cuda.synchronize()
    return o


def _dec_cpu(z):
    return [z[n].cpu() for n in ("q", "k", "v", "lam")]


@pytest.mark.parametrize("L", [1, 31, 32, 33, 300, 1000, 5000])
@pytest.mark.parametrize("G,d", [(2, 128), (8, 128), (8, 64), (16, 128)])
def test_decode_ragged(L, G, d):
    Hkv = 2
    z = workloads.decode_inputs(3, L, G * Hkv, Hkv, d, torch.bfloat16, seed=400 + L + G + d, device=DEV)
    out = _dec_run(z)
    assert_bf16_close(out, oracle.v2_decode(*_dec_cpu(z)), f"decode L{L} G{G} d{d}")


@pytest.mark.parametrize("d", [64, 128])
def test_decode_peaked_scores(d):
    z = workloads.decode_inputs(2, 1000, 16, 2, d, torch.bfloat16, seed=450 + d, device=DEV)
    z["q"].mul_(6)
    z["k"].mul_(6)
    out = _dec_run(z)
    assert_bf16_close(out, oracle.v2_decode(*_dec_cpu(z)), f"decode peaked d{d}")


@pytest.mark.parametrize("d", [64, 128])
def test_decode_rising_scores_rescale_every_block(d):
    z = workloads.decode_inputs(2, 1000, 16, 2, d, torch.bfloat16, seed=470 + d, device=DEV)
    z["q"][..., 0] = 12.0 * math.sqrt(d) / math.sqrt(128)
    _rising(z["k"].transpose(1, 2), 0.26)
    out = _dec_run(z)
    assert_bf16_close(out, oracle.v2_decode(*_dec_cpu(z)), f"decode rising d{d}")


def test_decode_equals_last_prefill_row():
    B, L, Hq, Hkv, d = 2, 700, 16, 2, 128
    y = workloads.v2_inputs(B, L, Hq, Hkv, d, torch.bfloat16, seed=17, device=DEV)
    pre = _v2_run(y)
    z = {"q": y["q"][:, -1].contiguous(), "k": y["k"], "v": y["v"], "lam": y["lam"][:, -1].contiguous()}
    dec = _dec_run(z)
    ref = oracle.v2_decode(*_dec_cpu(z))
    assert_bf16_close(dec, ref, "decode vs oracle")
    assert_bf16_close(pre[:, -1], ref, "prefill last row vs oracle")
    assert_bf16_close(dec, host64(pre[:, -1]), "decode vs prefill last row")


def test_decode_full_sampled():
    w = WORKLOADS["v2_decode_B64_L32768_Hq64_Hkv8_d128"]
    z = workloads.inputs_for(w, DEV)
    out = _dec_run(z)
    again = _dec_run(z)
    assert torch.equal(out, again)  # fixed merge order: bitwise deterministic
    for b in (0, 17, 63):
        zb = {n: z[n][b:b + 1].cpu() for n in ("q", "k", "v", "lam")}
        ref = oracle.v2_decode(zb["q"], zb["k"], zb["v"], zb["lam"])
        got = host64(out[b:b + 1])
        assert_bf16_close(got, ref, f"{w.name} b{b}")
        assert rel_l2(got, ref, axis=-1).max() < 3e-2
    del z
    torch.cuda.empty_cache()


def test_decode_prefix_mean_closed_form_full_size():
    """q = 0: every score is 0 and each head returns the mean of its group's
    V over the whole cache: out = (1 - sigmoid) * mean(V_g)."""
    w = WORKLOADS["v2_decode_B64_L32768_Hq64_Hkv8_d128"]
    z = workloads.inputs_for(w, DEV)
    z["q"].zero_()
    out = _dec_run(z)
    mean = z["v"].double().mean(dim=1).cpu().numpy()  # [B,Hkv,d], fp64 on the device
    sig = 1.0 / (1.0 + np.exp(-host64(z["lam"])))
    G = w.Hq // w.Hkv
    ref = (1 - sig)[..., None] * np.repeat(mean, G // 2, axis=1)
    assert_bf16_close(out, ref, "decode mean")
    del z
    torch.cuda.empty_cache()


# ------------------------------------------------- V2 decode, paged and ragged

def _paged_run(z, max_len, out=None, ws=None, softmax1=False):
    o = binding.v2_decode_paged(z["q"], z["k_pages"], z["v_pages"], z["block_table"], z["seq_lens"], z["lam"],
                                max_len, out=out, workspace=ws, softmax1=softmax1)
    torch.cuda.synchronize()
    return o


def _paged_ref(z, softmax1=False):
    c = {n: z[n].cpu() for n in z}
    return oracle.v2_decode_paged(c["q"], c["k_pages"], c["v_pages"], c["block_table"].numpy(),
                                  c["seq_lens"].numpy(), c["lam"], softmax1=softmax1)


PAGED_LENS = [1, 15, 16, 17, 127, 128, 129, 640, 2047, 3001]


@pytest.mark.parametrize("page", [16, 32, 64, 256])
@pytest.mark.parametrize("G,d", [(2, 128), (8, 128), (8, 64), (16, 64)])
def test_paged_decode_ragged(page, G, d):
    Hkv = 2
    z = workloads.paged_decode_inputs(len(PAGED_LENS), 3072, page, G * Hkv, Hkv, d, torch.bfloat16,
                                      seed=500 + page + G + d, device=DEV, lens=PAGED_LENS)
    out = _paged_run(z, 3072)
    assert_bf16_close(out, _paged_ref(z), f"paged P{page} G{G} d{d}")


def test_paged_identity_table_matches_dense_decode_bitwise():
    """Pages laid end to end in sequence order and every length = L: the
    paged kernel visits the same rows in the same order as the dense one, so
    the outputs are bit-identical."""
    B, L, Hq, Hkv, d, page = 3, 1000, 16, 2, 128, 16
    z = workloads.decode_inputs(B, L, Hq, Hkv, d, torch.bfloat16, seed=520, device=DEV)
    Lp = (L + page - 1) // page * page
    pad = torch.zeros((B, Lp - L, Hkv, d), dtype=torch.bfloat16, device=DEV)
    kp = torch.cat([z["k"], pad], 1).reshape(B * Lp // page, page, Hkv, d)
    vp = torch.cat([z["v"], pad], 1).reshape(B * Lp // page, page, Hkv, d)
    table = torch.arange(B * Lp // page, dtype=torch.int32, device=DEV).reshape(B, Lp // page)
    lens = torch.full((B,), L, dtype=torch.int32, device=DEV)
    pz = {"q": z["q"], "k_pages": kp, "v_pages": vp, "block_table": table, "seq_lens": lens, "lam": z["lam"]}
    assert torch.equal(_paged_run(pz, L), _dec_run(z))


def test_paged_max_len_beyond_every_sequence():
    """A max_len far above the lengths only adds empty splits."""
    lens = [3, 200, 1]
    z = workloads.paged_decode_inputs(3, 20000, 32, 16, 2, 128, torch.bfloat16, seed=530, device=DEV, lens=lens)
    ref = _paged_ref(z)
    assert_bf16_close(_paged_run(z, 20000), ref, "paged, long max_len")
    z2 = dict(z, block_table=z["block_table"][:, :7].contiguous())  # 7 pages of 32 cover max_len 224
    assert_bf16_close(_paged_run(z2, 224), ref, "paged, tight max_len")


def test_paged_strided_pool_and_table():
    """Pages stored head-major ([num_pages, Hkv, page, d], viewed as
    [num_pages, page, Hkv, d]) and a table that is a column slice of a wider
    one: the kernel follows the role strides."""
    lens = [77, 500, 16, 1]
    z = workloads.paged_decode_inputs(4, 512, 16, 8, 2, 64, torch.bfloat16, seed=540, device=DEV, lens=lens)
    kp = z["k_pages"].transpose(1, 2).contiguous().transpose(1, 2)
    vp = z["v_pages"].transpose(1, 2).contiguous().transpose(1, 2)
    wide = torch.full((4, 64), -1, dtype=torch.int32, device=DEV)
    wide[:, 5:5 + z["block_table"].shape[1]] = z["block_table"]
    zs = dict(z, k_pages=kp, v_pages=vp, block_table=wide[:, 5:5 + z["block_table"].shape[1]])
    assert zs["block_table"].stride(0) == 64 and kp.stride(1) == 64
    assert_bf16_close(_paged_run(zs, 512), _paged_ref(z), "paged strided")


def test_paged_length_zero_and_clamping():
    """Documented edge cases: a length of 0 (or below) gives 0, a length
    above max_len counts as max_len, a table entry outside the pool reads
    the nearest page of the pool."""
    lens = [0, 40, 64, 33]
    z = workloads.paged_decode_inputs(4, 64, 16, 8, 2, 128, torch.bfloat16, seed=550, device=DEV, lens=lens)
    n = z["k_pages"].shape[0]
    bad = z["block_table"].clone()
    bad[1, 0] = -5          # clamps to page 0
    bad[2, 3] = n + 3       # clamps to page n-1
    # sequence 3 (33 tokens, 3 pages) is given length 90: it reads 64 tokens,
    # its fourth table entry (-1) included, which clamps to page 0
    zc = dict(z, block_table=bad, seq_lens=torch.tensor([-4, 40, 64, 90], dtype=torch.int32, device=DEV))
    out = _paged_run(zc, 64)
    ref = _paged_ref(dict(z, block_table=bad.clamp(0, n - 1),
                          seq_lens=torch.tensor([0, 40, 64, 64], dtype=torch.int32)))
    assert torch.all(out[0] == 0)
    assert_bf16_close(out, ref, "paged clamping")


@pytest.mark.parametrize("d", [64, 128])
def test_paged_softmax1(d):
    z = workloads.paged_decode_inputs(len(PAGED_LENS), 3072, 64, 16, 2, d, torch.bfloat16, seed=560 + d,
                                      device=DEV, lens=PAGED_LENS)
    out = _paged_run(z, 3072, softmax1=True)
    assert_bf16_close(out, _paged_ref(z, softmax1=True), f"paged softmax1 d{d}")


def test_paged_full_sampled():
    """The benchmarked ragged batch (64 sequences, lengths uniform in
    [1, 32768], 64-token pages in a shuffled pool): sampled sequences against
    the oracle, and bitwise determinism."""
    w = WORKLOADS["v2_decode_paged_B64_Lmax32768_P64_Hq64_Hkv8_d128"]
    z = workloads.inputs_for(w, DEV)
    out = _paged_run(z, w.T)
    assert torch.equal(out, _paged_run(z, w.T))
    lens = z["seq_lens"].cpu()
    picks = [int(lens.argmin()), int(lens.argmax()), 5, 40]
    for b in picks:
        L = int(lens[b])
        pages = z["block_table"][b, :(L + w.page - 1) // w.page].long()
        zb = {"q": z["q"][b:b + 1].cpu(), "k_pages": z["k_pages"][pages].cpu(), "v_pages": z["v_pages"][pages].cpu(),
              "lam": z["lam"][b:b + 1].cpu()}
        table = np.arange(len(pages))[None]
        ref = oracle.v2_decode_paged(zb["q"], zb["k_pages"], zb["v_pages"], table, np.array([L]), zb["lam"])
        got = host64(out[b:b + 1])
        assert_bf16_close(got, ref, f"{w.name} b{b} L{L}")
    del z
    torch.cuda.empty_cache()


# ------------------------------------------------- V2 decode, several new tokens

def _multi_cpu(z):
    return [z[n].cpu() for n in ("q", "k", "v", "lam")]


@pytest.mark.parametrize("L,nq", [(4, 4), (33, 3), (300, 2), (1000, 4), (2100, 8), (5000, 5)])
@pytest.mark.parametrize("G,d", [(2, 128), (8, 128), (8, 64), (16, 64)])
def test_multi_decode(L, nq, G, d):
    """nq x G columns: 16 or fewer (one column block), up to 32 (two), more
    (several column groups, each streaming the cache)."""
    Hkv = 2
    z = workloads.decode_multi_inputs(2, L, nq, G * Hkv, Hkv, d, torch.bfloat16, seed=600 + L + nq + G + d,
                                      device=DEV)
    out = binding.v2_decode_multi(z["q"], z["k"], z["v"], z["lam"])
    torch.cuda.synchronize()
    assert_bf16_close(out, oracle.v2_decode_multi(*_multi_cpu(z)), f"multi L{L} nq{nq} G{G} d{d}")


def test_multi_decode_one_token_is_the_single_token_path():
    z = workloads.decode_inputs(3, 777, 16, 2, 128, torch.bfloat16, seed=620, device=DEV)
    single = _dec_run(z)
    multi = binding.v2_decode_multi(z["q"][:, None], z["k"], z["v"], z["lam"][:, None])
    torch.cuda.synchronize()
    assert torch.equal(multi[:, 0], single)


def test_multi_decode_equals_prefill_last_rows():
    """The new tokens' outputs are the last nq rows of the prefill over the
    cache (both kernels against each other, and against the oracle)."""
    B, L, nq, Hq, Hkv, d = 2, 600, 4, 16, 2, 128
    y = workloads.v2_inputs(B, L, Hq, Hkv, d, torch.bfloat16, seed=630, device=DEV)
    pre = _v2_run(y)
    dec = binding.v2_decode_multi(y["q"][:, L - nq:], y["k"], y["v"], y["lam"][:, L - nq:])
    torch.cuda.synchronize()
    ref = oracle.v2_decode_multi(y["q"][:, L - nq:].cpu(), y["k"].cpu(), y["v"].cpu(), y["lam"][:, L - nq:].cpu())
    assert_bf16_close(dec, ref, "multi decode vs oracle")
    assert_bf16_close(pre[:, L - nq:], ref, "prefill last rows vs oracle")


@pytest.mark.parametrize("d", [64, 128])
def test_multi_decode_softmax1(d):
    z = workloads.decode_multi_inputs(2, 1500, 4, 16, 2, d, torch.bfloat16, seed=640 + d, device=DEV)
    out = binding.v2_decode_multi(z["q"], z["k"], z["v"], z["lam"], softmax1=True)
    torch.cuda.synchronize()
    assert_bf16_close(out, oracle.v2_decode_multi(*_multi_cpu(z), softmax1=True), f"multi softmax1 d{d}")


@pytest.mark.parametrize("nq", [2, 4, 7])
def test_paged_multi_decode(nq):
    """Ragged lengths, some shorter than nq (their first new tokens see no
    entry and give 0), shuffled pages."""
    lens = [1, 3, 16, 17, 200, 2047, 3001]
    z = workloads.paged_decode_inputs(len(lens), 3072, 32, 16, 2, 128, torch.bfloat16, seed=650 + nq,
                                      device=DEV, lens=lens, nq=nq)
    out = _paged_run(z, 3072)
    assert out.shape == (len(lens), nq, 8, 128)
    assert_bf16_close(out, _paged_ref(z), f"paged multi nq{nq}")


def test_multi_decode_full_sampled():
    """The speculative-decoding shape: 64 sequences of 32768 entries, 4 new
    tokens each; sampled sequences against the oracle, and determinism."""
    w = WORKLOADS["v2_decode_multi_B64_L32768_nq4_Hq64_Hkv8_d128"]
    z = workloads.inputs_for(w, DEV)
    out = binding.v2_decode_multi(z["q"], z["k"], z["v"], z["lam"])
    again = binding.v2_decode_multi(z["q"], z["k"], z["v"], z["lam"])
    torch.cuda.synchronize()
    assert torch.equal(out, again)
    for b in (0, 41):
        ref = oracle.v2_decode_multi(*[z[n][b:b + 1].cpu() for n in ("q", "k", "v", "lam")])
        assert_bf16_close(out[b:b + 1], ref, f"{w.name} b{b}")
    del z
    torch.cuda.empty_cache()


# ------------------------------------------------------------------ HIP graphs

# ------------------------------------------------------- off-by-one softmax
# (every map's denominator + exp(0); Hacker News item 41780844)

@pytest.mark.parametrize("layer", [0, 4])
@pytest.mark.parametrize("d,T", [(64, 1), (64, 33), (64, 300), (128, 33), (128, 300)])
def test_softmax1_v1_bf16(d, T, layer):
    """(At layer 4, d 128, T 300 this seed draws lambda = 1.006, and row 1 of
    one head has two maps that nearly agree: D cancels by a factor of ~51,
    a row the cancellation guard recomputes exactly.)"""
    x = workloads.v1_inputs(2, 3, T, d, torch.bfloat16, seed=500 + d + T, device=DEV)
    out = _v1_run(x, layer, softmax1=True)
    assert_bf16_close(out, oracle.v1_fwd(*_v1_cpu(x), layer, softmax1=True), f"softmax1 v1 d{d} T{T} layer {layer}")


@pytest.mark.parametrize("d", [64, 128])
def test_softmax1_v1_bf16_peaked_and_rising(d):
    x = workloads.v1_inputs(2, 2, 300, d, torch.bfloat16, seed=520 + d, device=DEV)
    for n in ("q1", "q2", "k1", "k2"):
        x[n].mul_(6)
    assert_bf16_close(_v1_run(x, 2, softmax1=True), oracle.v1_fwd(*_v1_cpu(x), 2, softmax1=True), "peaked")
    x = workloads.v1_inputs(2, 2, 300, d, torch.bfloat16, seed=530 + d, device=DEV)
    for n in ("q1", "q2"):
        x[n][..., 0] = math.sqrt(d)
    for n in ("k1", "k2"):
        _rising(x[n], 0.26)
    assert_bf16_close(_v1_run(x, 5, softmax1=True), oracle.v1_fwd(*_v1_cpu(x), 5, softmax1=True), "rising")


@pytest.mark.parametrize("d,T", [(32, 33), (64, 200), (128, 33)])
def test_softmax1_v1_fp32(d, T):
    x = workloads.v1_inputs(2, 2, T, d, torch.float32, seed=540 + d + T, device=DEV)
    out = _v1_run(x, 7, softmax1=True)
    assert_fp32_close(out, oracle.v1_fwd(*_v1_cpu(x), 7, softmax1=True), f"softmax1 fp32 d{d} T{T}")


@pytest.mark.parametrize("G,d,T", [(2, 128, 1), (8, 128, 150), (8, 64, 150), (4, 128, 33)])
def test_softmax1_v2(G, d, T):
    y = workloads.v2_inputs(2, T, 2 * G, 2, d, torch.bfloat16, seed=550 + G + d + T, device=DEV)
    out = _v2_run(y, softmax1=True)
    assert_bf16_close(out, oracle.v2_fwd(*_v2_cpu(y), softmax1=True), f"softmax1 v2 G{G} d{d} T{T}")


def test_softmax1_v2_very_negative_logits():
    """Every visible score strongly negative: the off-by-one weights (and the
    output) shrink towards 0 while the standard softmax still averages V."""
    y = workloads.v2_inputs(1, 150, 8, 1, 128, torch.bfloat16, seed=560, device=DEV)
    y["k"].zero_()
    y["k"][..., 0] = 1.0
    y["q"].zero_()
    y["q"][..., 0] = -6.0 * math.sqrt(128)  # score -6 everywhere
    out = _v2_run(y, softmax1=True)
    ref = oracle.v2_fwd(*_v2_cpu(y), softmax1=True)
    assert_bf16_close(out, ref, "softmax1 negative logits")
    assert np.abs(ref[:, :8]).max() < 0.05  # first rows: n e^-6 / (1 + n e^-6) is small


def test_softmax1_v2_full_sampled():
    w = WORKLOADS["v2_prefill_B1_T8192_Hq64_Hkv8_d128"]
    y = workloads.inputs_for(w, DEV)
    out = _v2_run(y, softmax1=True)
    rng = np.random.default_rng(3)
    n = 64
    btp = np.stack([np.zeros(n, dtype=np.int64), rng.integers(0, w.T, n), rng.integers(0, w.Hq // 2, n)], 1)
    btp[:4, 1] = [0, 1, 32, w.T - 1]
    ref = oracle.v2_rows(*_v2_cpu(y), btp, softmax1=True)
    got = host64(out)[btp[:, 0], btp[:, 1], btp[:, 2]]
    assert_bf16_close(got, ref, "softmax1 " + w.name)
    assert rel_l2(got, ref, axis=-1).max() < 3e-2


@pytest.mark.parametrize("L,G,d", [(1, 8, 128), (33, 2, 128), (1000, 8, 64), (5000, 16, 128)])
def test_softmax1_decode(L, G, d):
    z = workloads.decode_inputs(2, L, G * 2, 2, d, torch.bfloat16, seed=570 + L + G + d, device=DEV)
    out = _dec_run(z, softmax1=True)
    assert_bf16_close(out, oracle.v2_decode(*_dec_cpu(z), softmax1=True), f"softmax1 decode L{L}")


def test_softmax1_decode_equals_last_prefill_row():
    B, L, Hq, Hkv, d = 1, 600, 16, 2, 128
    y = workloads.v2_inputs(B, L, Hq, Hkv, d, torch.bfloat16, seed=580, device=DEV)
    pre = _v2_run(y, softmax1=True)
    z = {"q": y["q"][:, -1].contiguous(), "k": y["k"], "v": y["v"], "lam": y["lam"][:, -1].contiguous()}
    dec = _dec_run(z, softmax1=True)
    assert_bf16_close(dec, host64(pre[:, -1]), "softmax1 decode vs prefill last row")


def test_v2_fused_qkv_and_head_major_cache_layouts_are_bitwise_equal():
    """Layouts callers hand over as views: V2 q, k, v sliced out of one fused
    projection output [B, T, Hq + 2 Hkv, d] (token stride (Hq + 2 Hkv) d), an
    output written into a wider buffer, and a decode cache stored head-major
    [B, Hkv, L, d] passed as a [B, L, Hkv, d] view.  The kernels read the same
    values in the same order, so the results equal the contiguous ones bit
    for bit; the contiguous ones are checked against the oracle."""
    B, T, Hq, Hkv, d = 2, 190, 8, 2, 128
    g = torch.Generator(device=DEV).manual_seed(4300)
    qkv = torch.randn((B, T, Hq + 2 * Hkv, d), generator=g, device=DEV).to(torch.bfloat16)
    lam = torch.randn((B, T, Hq // 2), generator=g, device=DEV)
    q, k, v = qkv[:, :, :Hq], qkv[:, :, Hq:Hq + Hkv], qkv[:, :, Hq + Hkv:]
    wide = torch.zeros((B, T, Hq // 2 + 3, d), dtype=torch.bfloat16, device=DEV)
    a = binding.v2_fwd(q, k, v, lam, out=wide[:, :, 1:1 + Hq // 2])
    torch.cuda.synchronize()
    c = _v2_run({"q": q.contiguous(), "k": k.contiguous(), "v": v.contiguous(), "lam": lam})
    assert torch.equal(a, c)
    assert torch.count_nonzero(wide[:, :, 0]) == 0 and torch.count_nonzero(wide[:, :, 1 + Hq // 2:]) == 0
    assert_bf16_close(c, oracle.v2_fwd(q.cpu(), k.cpu(), v.cpu(), lam.cpu()), "contiguous V2")

    Bd, L = 3, 2500
    kh = torch.randn((Bd, Hkv, L, d), generator=g, device=DEV).to(torch.bfloat16)
    vh = torch.randn((Bd, Hkv, L, d), generator=g, device=DEV).to(torch.bfloat16)
    z = {"q": torch.randn((Bd, Hq, d), generator=g, device=DEV).to(torch.bfloat16),
         "k": kh.transpose(1, 2), "v": vh.transpose(1, 2),
         "lam": torch.randn((Bd, Hq // 2), generator=g, device=DEV)}
    a = _dec_run(z)
    zc = dict(z, k=z["k"].contiguous(), v=z["v"].contiguous())
    c = _dec_run(zc)
    assert torch.equal(a, c)
    assert_bf16_close(c, oracle.v2_decode(*[zc[n].cpu() for n in ("q", "k", "v", "lam")]), "contiguous decode")


def test_graph_replay_matches_eager():
    """The benchmark replays one step captured as a HIP graph (12 V1 layer
    calls, a V2 prefill and a decode).  Every replay, with eager work and a
    clearing of the outputs in between, must equal the eager results bit for
    bit."""
    w = WORKLOADS["v1_gpt2small_B8_H6_T1024_d64"]
    x = workloads.inputs_for(w, DEV)
    y = workloads.v2_inputs(1, 300, 16, 2, 128, torch.bfloat16, seed=41, device=DEV)
    z = workloads.decode_inputs(4, 3000, 16, 2, 128, torch.bfloat16, seed=42, device=DEV)
    outs = [torch.empty((w.B, w.T, w.H, 2 * w.d), device=DEV, dtype=torch.bfloat16) for _ in w.layers]
    out2 = torch.empty((1, 300, 8, 128), device=DEV, dtype=torch.bfloat16)
    out3 = torch.empty((4, 8, 128), device=DEV, dtype=torch.bfloat16)
    ws = torch.empty(binding.v2_decode_workspace_bytes(4, 3000, 16, 2, 128), device=DEV, dtype=torch.uint8)

    def step():
        for layer, o in zip(w.layers, outs):
            binding.v1_fwd(*[x[n] for n in V1_NAMES], layer, out=o)
        binding.v2_fwd(y["q"], y["k"], y["v"], y["lam"], out=out2)
        binding.v2_decode(z["q"], z["k"], z["v"], z["lam"], out=out3, workspace=ws)

    step()
    torch.cuda.synchronize()
    ref = [o.clone() for o in outs] + [out2.clone(), out3.clone()]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()
    for rep in range(4):
        for o in outs + [out2, out3]:
            o.zero_()
        _v1_run(workloads.v1_inputs(1, 2, 64, 64, torch.bfloat16, seed=rep, device=DEV), rep)  # eager work
        g.replay()
        torch.cuda.synchronize()
        for got, want in zip(outs + [out2, out3], ref):
            assert torch.equal(got, want), f"replay {rep} differs"
