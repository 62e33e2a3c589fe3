"""The decode entry point that allocates nothing (diffattn_v2_decode_noalloc,
static scratch) against diffattn_v2_decode on the same inputs, through the C
ABI: two calls in a row, the second smaller, so the second reads a scratch
the first has written."""
import numpy as np
import pytest
import torch

import oracle
from differential_attention_diffattn_amd import binding, workloads
from gpu_util import assert_bf16_close, host64

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _case(B, L, Hq, Hkv, d, seed):
    g = torch.Generator(device=DEV).manual_seed(seed)
    r = lambda *s: torch.randn(s, generator=g, device=DEV)
    return (r(B, Hq, d).to(torch.bfloat16), r(B, L, Hkv, d).to(torch.bfloat16), r(B, L, Hkv, d).to(torch.bfloat16),
            r(B, Hq // 2))


def test_noalloc_decode_matches_the_workspace_entry_point():
    assert torch.cuda.is_available(), "GPU tests need a visible MI355X"
    binding.load_library()
    # 1: the decode workload, B 64 x L 32768, Hq 64 / Hkv 8, d 128 (7 splits in 16 MiB instead of 16)
    w = workloads.WORKLOADS["v2_decode_B64_L32768_Hq64_Hkv8_d128"]
    x = workloads.inputs_for(w, DEV)
    ref = binding.v2_decode(x["q"], x["k"], x["v"], x["lam"])
    got = torch.full_like(ref, float("nan"))
    binding.v2_decode_noalloc(x["q"], x["k"], x["v"], x["lam"], got)
    torch.cuda.synchronize()
    assert_bf16_close(got, host64(ref), "noalloc vs workspace decode, B64 L32768")
    # the split into 7 chunks changes only the order of the sums
    assert (got.float() - ref.float()).abs().max().item() < 2e-3
    del x
    torch.cuda.empty_cache()
    # 2: smaller, right after: d 128, Hq 16 / Hkv 2, B 3, L 3000
    q, k, v, lam = _case(3, 3000, 16, 2, 128, seed=77)
    ref2 = binding.v2_decode(q, k, v, lam)
    got2 = torch.full_like(ref2, float("nan"))
    binding.v2_decode_noalloc(q, k, v, lam, got2)
    torch.cuda.synchronize()
    assert_bf16_close(got2, host64(ref2), "noalloc vs workspace decode, B3 L3000")
    assert_bf16_close(got2, oracle.v2_decode(q.cpu(), k.cpu(), v.cpu(), lam.cpu()), "noalloc vs oracle")
    # 3: sizes whose partials do not fit: an error, nothing written
    q3, k3, v3, lam3 = _case(2048, 1, 16, 2, 128, seed=78)
    out3 = torch.zeros((2048, 8, 128), dtype=torch.bfloat16, device=DEV)
    with pytest.raises(binding.DiffAttnError):
        binding.v2_decode_noalloc(q3, k3, v3, lam3, out3)
    torch.cuda.synchronize()
    assert out3.abs().max().item() == 0
