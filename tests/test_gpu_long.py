"""Long contexts and large tensors: the HIP path at sizes where byte offsets
pass 2^31 and rows run over tens of thousands of keys.

* decode over a cache of 2^20 + 64 tokens x 8 kv heads x 128 (each of K and V
  is 2 GiB + 128 KiB), dense and paged (pool > 2 GiB), with a needle key
  near the end: every other key has coordinate 0 equal to 0, the queries
  point along coordinate 0, so every score but the needle's is exactly 0 and
  the exact result is a closed form of two sums;
* causal prefill at T = 65536 + 5 (V2) and T = 32768 + 3 (V1): rows sampled
  near the end, against the oracle row by row.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from differential_attention_diffattn_amd import binding, workloads
from gpu_util import assert_bf16_close, host64, rel_l2

pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a visible MI355X"
    binding.load_library()
    yield
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def _needle_cache(L, Hkv, d, needle, alpha, seed):
    g = torch.Generator(device=DEV).manual_seed(seed)
    k = torch.randn((1, L, Hkv, d), generator=g, device=DEV, dtype=torch.bfloat16)
    v = torch.randn((1, L, Hkv, d), generator=g, device=DEV, dtype=torch.bfloat16)
    k[..., 0] = 0
    k[0, needle, :, 0] = alpha
    return k, v


def _needle_ref(v, needle, alpha, d, lam, G):
    """Exact decode output: scores are alpha^2/sqrt(d) at the needle and 0
    elsewhere, so head h of group g returns (W v_n + S) / (W + L - 1) with
    W = e^(alpha^2/sqrt(d)) and S the sum of the group's other V rows; both
    heads of a pair see the same, and out_p = (1 - sigmoid(lam_p)) a."""
    L = v.shape[1]
    S = torch.zeros(v.shape[2], v.shape[3], dtype=torch.float64, device=v.device)
    for i in range(0, L, 1 << 17):  # fp64 sums on the device in slices (bounded temporaries)
        S += v[0, i:i + (1 << 17)].double().sum(0)
    vn = v[0, needle].double()
    S = (S - vn).cpu().numpy()
    vn = vn.cpu().numpy()
    W = math.exp(alpha * alpha / math.sqrt(d))
    a = (W * vn + S) / (W + (L - 1))                      # [Hkv, d]
    sig = 1.0 / (1.0 + np.exp(-host64(lam)[0]))            # [Hq/2]
    grp = (2 * np.arange(sig.shape[0])) // G
    return ((1.0 - sig)[:, None] * a[grp])[None]         # [1, Hq/2, d]


def test_decode_needle_cache_past_2gib_dense_and_paged():
    L, Hq, Hkv, d, page = (1 << 20) + 64, 16, 8, 128, 64
    needle, alpha = L - 3, 16.0
    assert L * Hkv * d * 2 > (1 << 31)
    k, v = _needle_cache(L, Hkv, d, needle, alpha, seed=9100)
    q = torch.zeros((1, Hq, d), dtype=torch.bfloat16, device=DEV)
    q[..., 0] = alpha
    lam = torch.randn((1, Hq // 2), generator=torch.Generator(device=DEV).manual_seed(9101), device=DEV)
    ref = _needle_ref(v, needle, alpha, d, lam, Hq // Hkv)
    out = binding.v2_decode(q, k, v, lam)
    torch.cuda.synchronize()
    assert_bf16_close(out, ref, "dense decode, 2^20 + 64 tokens")
    assert rel_l2(out, ref, axis=-1).max() < 1e-2
    # the same cache as a pool of 64-token pages (16385 pages, > 2 GiB each
    # for K and V), table in sequence order, one sequence of length L
    kp = k.view(L // page, page, Hkv, d)
    vp = v.view(L // page, page, Hkv, d)
    table = torch.arange(L // page, dtype=torch.int32, device=DEV).reshape(1, -1)
    lens = torch.full((1,), L, dtype=torch.int32, device=DEV)
    outp = binding.v2_decode_paged(q, kp, vp, table, lens, lam, L)
    torch.cuda.synchronize()
    assert_bf16_close(outp, ref, "paged decode, pool > 2 GiB")
    assert rel_l2(outp, ref, axis=-1).max() < 1e-2
    del k, v, kp, vp
    torch.cuda.empty_cache()


def test_decode_needle_in_the_last_page_of_a_shuffled_pool():
    """Paged: the needle's page sits at the end of a pool > 2 GiB and the
    table visits pages in a shuffled order."""
    L, Hq, Hkv, d, page = (1 << 20) + 64, 16, 8, 128, 64
    npg = L // page
    needle, alpha = 5 * page + 7, 16.0  # logical position: early in the sequence
    k, v = _needle_cache(L, Hkv, d, needle, alpha, seed=9200)
    q = torch.zeros((1, Hq, d), dtype=torch.bfloat16, device=DEV)
    q[..., 0] = alpha
    lam = torch.randn((1, Hq // 2), generator=torch.Generator(device=DEV).manual_seed(9201), device=DEV)
    ref = _needle_ref(v, needle, alpha, d, lam, Hq // Hkv)
    # perm[i]: physical page of logical page i, shuffled, with logical page 5
    # (the needle's) at the last physical page
    perm = np.random.default_rng(9202).permutation(npg)
    j = int(np.where(perm == npg - 1)[0][0])
    perm[j], perm[5] = perm[5], perm[j]
    perm_t = torch.from_numpy(perm).to(DEV)
    kp = torch.empty((npg, page, Hkv, d), dtype=torch.bfloat16, device=DEV)
    kp[perm_t] = k.view(npg, page, Hkv, d)
    del k
    vp = torch.empty_like(kp)
    vp[perm_t] = v.view(npg, page, Hkv, d)
    del v
    table = perm_t.to(torch.int32).reshape(1, -1)
    lens = torch.full((1,), L, dtype=torch.int32, device=DEV)
    assert int(table[0, 5]) == npg - 1
    out = binding.v2_decode_paged(q, kp, vp, table, lens, lam, L)
    torch.cuda.synchronize()
    assert_bf16_close(out, ref, "paged decode, shuffled pool > 2 GiB")
    assert rel_l2(out, ref, axis=-1).max() < 1e-2
    del kp, vp
    torch.cuda.empty_cache()


def test_v2_prefill_long_sequence_sampled():
    B, T, Hq, Hkv, d = 1, 65536 + 5, 4, 2, 128
    y = workloads.v2_inputs(B, T, Hq, Hkv, d, torch.bfloat16, seed=9300, device=DEV)
    out = binding.v2_fwd(y["q"], y["k"], y["v"], y["lam"])
    torch.cuda.synchronize()
    rows = np.array([0, 1, 4095, 32768, T - 33, T - 32, T - 2, T - 1], dtype=np.int64)
    btp = np.stack([np.zeros(rows.size * 2, dtype=np.int64), np.repeat(rows, 2), np.tile([0, 1], rows.size)], 1)
    ref = oracle.v2_rows(*[y[n].cpu() for n in ("q", "k", "v", "lam")], btp)
    got = host64(out)[btp[:, 0], btp[:, 1], btp[:, 2]]
    assert_bf16_close(got, ref, "V2 prefill T = 65541")
    assert rel_l2(got, ref, axis=-1).max() < 3e-2


def test_v1_prefill_long_sequence_sampled():
    B, H, T, d, layer = 1, 2, 32768 + 3, 64, 7
    x = workloads.v1_inputs(B, H, T, d, torch.bfloat16, seed=9400, device=DEV)
    names = ("q1", "q2", "k1", "k2", "v", "lq1", "lk1", "lq2", "lk2")
    out = binding.v1_fwd(*[x[n] for n in names], layer)
    torch.cuda.synchronize()
    rows = np.array([0, 31, 8191, T - 35, T - 3, T - 1], dtype=np.int64)
    bhi = np.stack([np.zeros(rows.size * 2, dtype=np.int64), np.tile([0, 1], rows.size), np.repeat(rows, 2)], 1)
    ref = oracle.v1_rows(*[x[n].cpu() for n in names], layer, bhi)
    got = host64(out)[bhi[:, 0], bhi[:, 2], bhi[:, 1]]
    assert_bf16_close(got, ref, "V1 prefill T = 32771")
