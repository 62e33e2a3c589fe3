"""Seeded synthetic workloads for differential attention.

This module only draws random tensors and names shapes; it holds none of the
method's arithmetic.  Both the HIP path (tests, bench) and the fp64 oracle
(tests) take their inputs from here, so the two sides see identical values.

Distributions follow the pages: activations N(0, 1); the four V1 lambda
vectors N(0, 0.1) in fp32 (nanoGPT issue "How best to implement a
differential transformer?", Wilsontomass's module, the lambda parameter
initialisation); V2 lambda logits N(0, 1) in fp32.  Values are drawn in fp32
with a seeded ``torch.Generator`` and then rounded (RNE) to the working dtype;
the order of draws is fixed per workload.

Paged decode: sequence lengths uniform in [1, max_len] and the page table a
seeded random permutation of the page pool (a pool shared by a ragged batch,
pages handed out in no particular order), both drawn on the CPU so the sizes
are known without touching the device.

Shapes: the workloads below.  The GPT-2-small and 3B-class shapes stand
in for the models the pages name (a GPT-2 124M nanoGPT run; a 3B model with
28 layers, hidden 3072, 12 heads); no dataset, checkpoint or real activation
is available, so seeded N(0, 1) tensors stand in for them.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Dict, Tuple

import torch


@dataclass(frozen=True)
class Workload:
    name: str
    kind: str  # "v1", "v2", "v2_rope", "v1_bwd", "v2_bwd", "decode", "decode_rope", "decode_paged",
    #           "decode_multi", "lam_proj"
    dtype: str  # "fp32" or "bf16"
    B: int
    H: int = 0  # V1: differential heads
    T: int = 0  # V1/V2: tokens; decode: cache length L
    d: int = 0
    Hq: int = 0
    Hkv: int = 0
    layers: Tuple[int, ...] = ()
    seed: int = 0
    page: int = 0  # decode_paged: tokens per cache page (T is then the longest length)
    nq: int = 0    # decode_multi: new tokens per sequence (the last nq of the T cache entries)

    def seq_lens(self) -> torch.Tensor:
        """decode_paged: the seeded sequence lengths (CPU int32 [B])."""
        return draw_seq_lens(self.B, self.T, self.seed)

    @property
    def torch_dtype(self):
        return torch.float32 if self.dtype == "fp32" else torch.bfloat16

    def flops(self) -> float:
        """Algorithmic flops of one call, counting only unmasked (i, j<=i)
        pairs: V1 = 2 maps x (QK^T over d + PV over 2d) = 6*B*H*d*T(T+1);
        V2 prefill = 2*B*Hq*d*T(T+1); decode = 4*B*Hq*d*L (paged: the sum of
        the sequences' lengths in place of B*L)."""
        if self.kind == "v1":
            return 6.0 * self.B * self.H * self.d * self.T * (self.T + 1)
        if self.kind in ("v2", "v2_rope"):
            return 2.0 * self.B * self.Hq * self.d * self.T * (self.T + 1)
        if self.kind == "lam_proj":  # x [B,T,dm] . w [P,dm]; here H holds dm and Hq holds P
            return 2.0 * self.B * self.T * self.H * self.Hq
        if self.kind == "v2_bwd":  # 5 products (S, dP, dV, dK, dQ) over the unmasked pairs
            return 5.0 * self.B * self.Hq * self.d * self.T * (self.T + 1)
        if self.kind == "v1_bwd":  # per map S, dK, dQ over d and dP, dV over 2d: 14 d flops per pair and map
            return 14.0 * self.B * self.H * self.d * self.T * (self.T + 1)
        if self.kind == "decode_paged":
            return 4.0 * self.Hq * self.d * int(self.seq_lens().sum())
        if self.kind == "decode_multi":  # new token i sees T - nq + i + 1 entries
            return 4.0 * self.B * self.Hq * self.d * sum(self.T - self.nq + i + 1 for i in range(self.nq))
        return 4.0 * self.B * self.Hq * self.d * self.T

    def compulsory_bytes(self) -> int:
        """Bytes every call must move between HBM and the chip at least once:
        each input read once, the output written once."""
        e = 4 if self.dtype == "fp32" else 2
        if self.kind == "v1":
            B, H, T, d = self.B, self.H, self.T, self.d
            return e * (4 * B * H * T * d + B * H * T * 2 * d + B * T * H * 2 * d) + 4 * 4 * d
        if self.kind in ("v2", "v2_rope"):
            B, T, Hq, Hkv, d = self.B, self.T, self.Hq, self.Hkv, self.d
            return e * (B * T * Hq * d + 2 * B * T * Hkv * d + B * T * (Hq // 2) * d) + 4 * B * T * (Hq // 2)
        if self.kind == "lam_proj":  # x and w read once, fp32 logits written once
            return e * (self.B * self.T * self.H + self.Hq * self.H) + 4 * self.B * self.T * self.Hq
        if self.kind == "v1_bwd":  # q1 q2 k1 k2 v, attn1 attn2, dout, lse, 4 lambda vectors in; 5 grads + 4 out
            B, H, T, d = self.B, self.H, self.T, self.d
            return (e * (4 * B * H * T * d + B * H * T * 2 * d + 3 * B * T * H * 2 * d + 4 * B * H * T * d
                         + B * H * T * 2 * d) + 4 * 2 * B * H * T + 4 * 8 * d)
        if self.kind == "v2_bwd":  # q, k, v, attn, dout, lam, lse in; dq, dk, dv, dlam out
            B, T, Hq, Hkv, d = self.B, self.T, self.Hq, self.Hkv, self.d
            return (e * (2 * B * T * Hq * d + 4 * B * T * Hkv * d + 2 * B * T * Hq * d + B * T * (Hq // 2) * d)
                    + 4 * (2 * B * T * (Hq // 2) + B * Hq * T))
        B, L, Hq, Hkv, d = self.B, self.T, self.Hq, self.Hkv, self.d
        if self.kind == "decode_paged":
            lens = self.seq_lens().long()
            tokens = int(lens.sum())
            table = 4 * int(((lens + self.page - 1) // self.page).sum())  # the entries a call reads
            return (e * (B * Hq * d + 2 * tokens * Hkv * d + B * (Hq // 2) * d) + 4 * B * (Hq // 2) + table
                    + 4 * B)
        if self.kind == "decode_multi":
            nq = self.nq
            return e * (B * nq * Hq * d + 2 * B * L * Hkv * d + B * nq * (Hq // 2) * d) + 4 * B * nq * (Hq // 2)
        return e * (B * Hq * d + 2 * B * L * Hkv * d + B * (Hq // 2) * d) + 4 * B * (Hq // 2)


WORKLOADS: Dict[str, Workload] = {
    w.name: w
    for w in [
        Workload("v1_fp32_B1_H2_T128_d32", "v1", "fp32", B=1, H=2, T=128, d=32, layers=(3,), seed=1),
        Workload("v1_gpt2small_B8_H6_T1024_d64", "v1", "bf16", B=8, H=6, T=1024, d=64,
                 layers=tuple(range(12)), seed=2),
        Workload("v1_3b_B2_H12_T4096_d128", "v1", "bf16", B=2, H=12, T=4096, d=128, layers=(14,), seed=3),
        Workload("v2_prefill_B1_T8192_Hq64_Hkv8_d128", "v2", "bf16", B=1, T=8192, d=128, Hq=64, Hkv=8, seed=4),
        Workload("v2_decode_B64_L32768_Hq64_Hkv8_d128", "decode", "bf16", B=64, T=32768, d=128, Hq=64,
                 Hkv=8, seed=5),
        Workload("v2_backward_B1_T8192_Hq64_Hkv8_d128", "v2_bwd", "bf16", B=1, T=8192, d=128, Hq=64, Hkv=8, seed=4),
        Workload("v1_backward_B8_H6_T1024_d64", "v1_bwd", "bf16", B=8, H=6, T=1024, d=64, layers=(6,), seed=2),
        Workload("v1_backward_B2_H12_T4096_d128", "v1_bwd", "bf16", B=2, H=12, T=4096, d=128, layers=(14,),
                 seed=3),
        Workload("v2_decode_paged_B64_Lmax32768_P64_Hq64_Hkv8_d128", "decode_paged", "bf16", B=64, T=32768,
                 d=128, Hq=64, Hkv=8, seed=6, page=64),
        Workload("v2_decode_multi_B64_L32768_nq4_Hq64_Hkv8_d128", "decode_multi", "bf16", B=64, T=32768, d=128,
                 Hq=64, Hkv=8, seed=7, nq=4),
        # rotary embedding fused (q in the kernel's prologue; prefill k rotated by a pass into a workspace)
        Workload("v2_prefill_rope_B1_T8192_Hq64_Hkv8_d128", "v2_rope", "bf16", B=1, T=8192, d=128, Hq=64, Hkv=8,
                 seed=4),
        Workload("v2_decode_rope_B64_L32768_Hq64_Hkv8_d128", "decode_rope", "bf16", B=64, T=32768, d=128, Hq=64,
                 Hkv=8, seed=5),
        # V2 lambda projection at the V2 prefill shape: d_model = 32 pairs x 128 = 4096 (H = dm, Hq = pairs)
        Workload("v2_lambda_proj_B1_T8192_dm4096_P32", "lam_proj", "bf16", B=1, T=8192, H=4096, Hq=32, seed=8),
    ]
}


def _gen(seed: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return g


def _randn(shape, g, device, dtype, std: float = 1.0, chunk_rows: int = 0) -> torch.Tensor:
    """fp32 N(0, std^2) draws rounded to ``dtype``.  With ``chunk_rows`` the
    draw is made in slices of the leading dimension to bound the fp32
    temporary (used for multi-GB KV caches)."""
    if chunk_rows <= 0 or shape[0] <= chunk_rows:
        x = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
        if std != 1.0:
            x.mul_(std)
        return x.to(dtype)
    out = torch.empty(shape, device=device, dtype=dtype)
    for s in range(0, shape[0], chunk_rows):
        e = min(shape[0], s + chunk_rows)
        x = torch.randn((e - s,) + tuple(shape[1:]), generator=g, device=device, dtype=torch.float32)
        if std != 1.0:
            x.mul_(std)
        out[s:e].copy_(x)
        del x
    return out


def v1_inputs(B: int, H: int, T: int, d: int, dtype=torch.bfloat16, seed: int = 0,
              device="cpu") -> Dict[str, torch.Tensor]:
    """q1, q2, k1, k2 ``[B, H, T, d]``; v ``[B, H, T, 2d]`` (dtype);
    lq1, lk1, lq2, lk2 ``[d]`` fp32 ~ N(0, 0.1)."""
    g = _gen(seed, device)
    out = {}
    for name in ("q1", "q2", "k1", "k2"):
        out[name] = _randn((B, H, T, d), g, device, dtype)
    out["v"] = _randn((B, H, T, 2 * d), g, device, dtype)
    for name in ("lq1", "lk1", "lq2", "lk2"):
        out[name] = _randn((d,), g, device, torch.float32, std=0.1)
    return out


def v2_inputs(B: int, T: int, Hq: int, Hkv: int, d: int, dtype=torch.bfloat16, seed: int = 0,
              device="cpu") -> Dict[str, torch.Tensor]:
    """q ``[B, T, Hq, d]``; k, v ``[B, T, Hkv, d]`` (dtype); lam ``[B, T, Hq/2]``
    fp32 logits ~ N(0, 1)."""
    g = _gen(seed, device)
    return {
        "q": _randn((B, T, Hq, d), g, device, dtype),
        "k": _randn((B, T, Hkv, d), g, device, dtype),
        "v": _randn((B, T, Hkv, d), g, device, dtype),
        "lam": _randn((B, T, Hq // 2), g, device, torch.float32),
    }


def decode_inputs(B: int, L: int, Hq: int, Hkv: int, d: int, dtype=torch.bfloat16, seed: int = 0,
                  device="cpu") -> Dict[str, torch.Tensor]:
    """q ``[B, Hq, d]``; k_cache, v_cache ``[B, L, Hkv, d]`` (dtype, contiguous);
    lam ``[B, Hq/2]`` fp32 logits ~ N(0, 1)."""
    g = _gen(seed, device)
    return {
        "q": _randn((B, Hq, d), g, device, dtype),
        "k": _randn((B, L, Hkv, d), g, device, dtype, chunk_rows=4),
        "v": _randn((B, L, Hkv, d), g, device, dtype, chunk_rows=4),
        "lam": _randn((B, Hq // 2), g, device, torch.float32),
    }


def decode_multi_inputs(B: int, L: int, nq: int, Hq: int, Hkv: int, d: int, dtype=torch.bfloat16, seed: int = 0,
                        device="cpu") -> Dict[str, torch.Tensor]:
    """Multi-token decode: q ``[B, nq, Hq, d]``; k_cache, v_cache ``[B, L, Hkv, d]``
    (the nq new tokens are the last nq entries); lam ``[B, nq, Hq/2]`` fp32."""
    g = _gen(seed, device)
    return {
        "q": _randn((B, nq, Hq, d), g, device, dtype),
        "k": _randn((B, L, Hkv, d), g, device, dtype, chunk_rows=4),
        "v": _randn((B, L, Hkv, d), g, device, dtype, chunk_rows=4),
        "lam": _randn((B, nq, Hq // 2), g, device, torch.float32),
    }


def lambda_proj_inputs(B: int, T: int, dm: int, P: int, dtype=torch.bfloat16, seed: int = 0,
                       device="cpu") -> Dict[str, torch.Tensor]:
    """x ``[B, T, dm]`` ~ N(0, 1) (a hidden state); w ``[P, dm]`` ~ N(0, 1/dm)
    (a linear layer's weight at the usual initialisation scale)."""
    g = _gen(seed, device)
    return {"x": _randn((B, T, dm), g, device, dtype),
            "w": _randn((P, dm), g, device, dtype, std=1.0 / dm ** 0.5)}


def draw_seq_lens(B: int, max_len: int, seed: int) -> torch.Tensor:
    """Lengths uniform in [1, max_len], CPU int32 [B]."""
    g = torch.Generator().manual_seed(int(seed) + 7919)
    return torch.randint(1, max_len + 1, (B,), generator=g, dtype=torch.int32)


def paged_decode_inputs(B: int, max_len: int, page: int, Hq: int, Hkv: int, d: int, dtype=torch.bfloat16,
                        seed: int = 0, device="cpu", lens=None, spare_pages: int = 3,
                        nq: int = 0) -> Dict[str, torch.Tensor]:
    """Decode over a paged cache.  lens: the sequence lengths (default: uniform
    in [1, max_len]); q ``[B, Hq, d]``; k_pages, v_pages ``[num_pages, page,
    Hkv, d]`` (dtype) with num_pages = the pages the sequences need +
    ``spare_pages``; block_table int32 ``[B, ceil(max_len / page)]``: the
    sequences' pages in a seeded random order of the pool, -1 past each
    sequence's last page; seq_lens int32 ``[B]``; lam ``[B, Hq/2]`` fp32.
    nq > 0: q ``[B, nq, Hq, d]`` and lam ``[B, nq, Hq/2]`` (nq new tokens)."""
    lens = draw_seq_lens(B, max_len, seed) if lens is None else torch.tensor(list(lens), dtype=torch.int32)
    width = (max_len + page - 1) // page
    need = [(int(L) + page - 1) // page for L in lens]
    num_pages = sum(need) + spare_pages
    gc = torch.Generator().manual_seed(int(seed) + 104729)
    order = torch.randperm(num_pages, generator=gc).to(torch.int32)
    table = torch.full((B, width), -1, dtype=torch.int32)
    at = 0
    for b, n in enumerate(need):
        table[b, :n] = order[at:at + n]
        at += n
    g = _gen(seed, device)
    rows = max(1, (64 << 20) // (page * Hkv * d * 4))  # bound the fp32 temporary to ~64 MB
    tok = (nq,) if nq > 0 else ()
    return {
        "q": _randn((B,) + tok + (Hq, d), g, device, dtype),
        "k_pages": _randn((num_pages, page, Hkv, d), g, device, dtype, chunk_rows=rows),
        "v_pages": _randn((num_pages, page, Hkv, d), g, device, dtype, chunk_rows=rows),
        "block_table": table.to(device),
        "seq_lens": lens.to(device),
        "lam": _randn((B,) + tok + (Hq // 2,), g, device, torch.float32),
    }


def inputs_for(w: Workload, device="cpu") -> Dict[str, torch.Tensor]:
    if w.kind == "v1":
        return v1_inputs(w.B, w.H, w.T, w.d, w.torch_dtype, w.seed, device)
    if w.kind == "v1_bwd":  # the V1 forward's inputs plus an output gradient dout ~ N(0, 1)
        x = v1_inputs(w.B, w.H, w.T, w.d, w.torch_dtype, w.seed, device)
        x["dout"] = _randn((w.B, w.T, w.H, 2 * w.d), _gen(w.seed + 99, device), device, w.torch_dtype)
        return x
    if w.kind in ("v2", "v2_rope"):
        return v2_inputs(w.B, w.T, w.Hq, w.Hkv, w.d, w.torch_dtype, w.seed, device)
    if w.kind == "lam_proj":
        return lambda_proj_inputs(w.B, w.T, w.H, w.Hq, w.torch_dtype, w.seed, device)
    if w.kind == "v2_bwd":  # the prefill's inputs plus an output gradient dout ~ N(0, 1)
        x = v2_inputs(w.B, w.T, w.Hq, w.Hkv, w.d, w.torch_dtype, w.seed, device)
        x["dout"] = _randn((w.B, w.T, w.Hq // 2, w.d), _gen(w.seed + 99, device), device, w.torch_dtype)
        return x
    if w.kind == "decode_paged":
        return paged_decode_inputs(w.B, w.T, w.page, w.Hq, w.Hkv, w.d, w.torch_dtype, w.seed, device)
    if w.kind == "decode_multi":
        return decode_multi_inputs(w.B, w.T, w.nq, w.Hq, w.Hkv, w.d, w.torch_dtype, w.seed, device)
    return decode_inputs(w.B, w.T, w.Hq, w.Hkv, w.d, w.torch_dtype, w.seed, device)
