"""fp64 CPU oracle for differential attention -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The product (the HIP library and its
binding in ``differential_attention_diffattn_amd``) never imports it and
shares no code with it.

The arithmetic lives in ``diffattn_oracle.c`` (plain C, fp64, one causal
softmax row at a time); this module only compiles it with gcc and marshals
numpy float64 arrays through ctypes.  Layouts are dense, as documented in
``diffattn_oracle.h``:

* V1: q1, q2, k1, k2 ``[B, H, T, d]``; v ``[B, H, T, 2d]``; out ``[B, T, H, 2d]``.
* V2 prefill: q ``[B, T, Hq, d]``; k, v ``[B, T, Hkv, d]``; lam ``[B, T, Hq/2]``;
  out ``[B, T, Hq/2, d]``.
* V2 decode: q ``[B, Hq, d]``; k, v ``[B, L, Hkv, d]``; lam ``[B, Hq/2]``;
  out ``[B, Hq/2, d]``.
* V2 decode over a paged cache: k, v pages ``[num_pages, page_size, Hkv, d]``,
  an int page table ``[B, >= ceil(L_b / page_size)]`` and lengths ``[B]``.

``oracle.backward`` (numpy, fp64) holds the V2 and V1 training steps: the
forward with what a backward pass keeps (per-head or per-map attention
outputs, log-sum-exp) and the gradients.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from pathlib import Path

import numpy as np

_HERE = Path(__file__).resolve().parent
_SRC = _HERE / "diffattn_oracle.c"
_LIB = _HERE / "liboracle.so"
# A prebuilt copy of this same source to load instead (the sanitizer test
# builds one with -fsanitize=address,undefined); never built here.
_LIB_OVERRIDE = os.environ.get("DIFFATTN_ORACLE_LIBRARY")

_lib = None


def build(force: bool = True) -> Path:
    """Compile the oracle into ``oracle/liboracle.so`` with gcc + OpenMP.

    No -ffast-math: the C code is evaluated with IEEE fp64 semantics.
    """
    if force or not _LIB.exists():
        tmp = _LIB.with_suffix(".so.tmp%d" % os.getpid())
        cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp",
               str(_SRC), "-o", str(tmp), "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if _LIB_OVERRIDE:
        _lib = _configure(ctypes.CDLL(_LIB_OVERRIDE))
        return _lib
    if not _LIB.exists() or _LIB.stat().st_mtime < _SRC.stat().st_mtime:
        build(force=True)
    _lib = _configure(ctypes.CDLL(str(_LIB)))
    return _lib


def _configure(lib):
    """Declare the C signatures on a loaded oracle library."""
    dp = ctypes.POINTER(ctypes.c_double)
    ip = ctypes.POINTER(ctypes.c_int64)
    i = ctypes.c_int
    lib.da_oracle_lambda_init.argtypes = [i]
    lib.da_oracle_lambda_init.restype = ctypes.c_double
    lib.da_oracle_v1_lambda.argtypes = [i, dp, dp, dp, dp, i]
    lib.da_oracle_v1_lambda.restype = ctypes.c_double
    lib.da_oracle_v1_fwd.argtypes = [i, i, i, i] + [dp] * 9 + [i, i, dp]
    lib.da_oracle_v1_fwd.restype = None
    lib.da_oracle_v1_rows.argtypes = [i, i, i, i] + [dp] * 9 + [i, i, ctypes.c_int64, ip, dp]
    lib.da_oracle_v1_rows.restype = None
    lib.da_oracle_v2_fwd.argtypes = [i, i, i, i, i] + [dp] * 4 + [i, dp]
    lib.da_oracle_v2_fwd.restype = None
    lib.da_oracle_v2_rows.argtypes = [i, i, i, i, i] + [dp] * 4 + [i, ctypes.c_int64, ip, dp]
    lib.da_oracle_v2_rows.restype = None
    lib.da_oracle_v2_decode.argtypes = [i, i, i, i, i] + [dp] * 4 + [i, dp]
    lib.da_oracle_v2_decode.restype = None
    lib.da_oracle_v2_heads.argtypes = [i, i, i, i, i] + [dp] * 3 + [i, dp, dp]
    lib.da_oracle_v2_heads.restype = None
    lib.da_oracle_set_threads.argtypes = [i]
    lib.da_oracle_set_threads.restype = i
    return lib


def _f64(a) -> np.ndarray:
    """Dense float64 copy (or view) of a numpy array or a CPU torch tensor."""
    if hasattr(a, "detach"):  # torch tensor: widen exactly on the CPU
        a = a.detach().to("cpu").double().numpy()
    return np.ascontiguousarray(a, dtype=np.float64)


def _p(a: np.ndarray):
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def set_threads(n: int = 0) -> int:
    """Set the OpenMP thread count (0 keeps the default); returns the count used."""
    return _load().da_oracle_set_threads(int(n))


def lambda_init(layer: int) -> float:
    return _load().da_oracle_lambda_init(int(layer))


def v1_lambda(lq1, lk1, lq2, lk2, layer: int) -> float:
    a = [_f64(x) for x in (lq1, lk1, lq2, lk2)]
    return _load().da_oracle_v1_lambda(a[0].size, *[_p(x) for x in a], int(layer))


def _v1_check(q1, q2, k1, k2, v, lams):
    B, H, T, d = q1.shape
    for x in (q2, k1, k2):
        assert x.shape == (B, H, T, d), x.shape
    assert v.shape == (B, H, T, 2 * d), v.shape
    for x in lams:
        assert x.shape == (d,), x.shape
    return B, H, T, d


def v1_fwd(q1, q2, k1, k2, v, lq1, lk1, lq2, lk2, layer: int, softmax1: bool = False) -> np.ndarray:
    """DIFF V1 forward, all rows; returns ``[B, T, H, 2d]`` float64.
    ``softmax1``: the off-by-one softmax (denominator + exp(0)) in both maps."""
    t = [_f64(x) for x in (q1, q2, k1, k2, v, lq1, lk1, lq2, lk2)]
    B, H, T, d = _v1_check(*t[:5], t[5:])
    out = np.zeros((B, T, H, 2 * d), dtype=np.float64)
    _load().da_oracle_v1_fwd(B, H, T, d, *[_p(x) for x in t], int(layer), int(bool(softmax1)), _p(out))
    return out


def v1_rows(q1, q2, k1, k2, v, lq1, lk1, lq2, lk2, layer: int, bhi, softmax1: bool = False) -> np.ndarray:
    """DIFF V1 forward for rows ``bhi`` (an ``[n, 3]`` array of (b, h, i));
    returns ``[n, 2d]`` float64."""
    t = [_f64(x) for x in (q1, q2, k1, k2, v, lq1, lk1, lq2, lk2)]
    B, H, T, d = _v1_check(*t[:5], t[5:])
    idx = np.ascontiguousarray(np.asarray(bhi, dtype=np.int64).reshape(-1, 3))
    assert (idx[:, 0] < B).all() and (idx[:, 1] < H).all() and (idx[:, 2] < T).all()
    out = np.zeros((idx.shape[0], 2 * d), dtype=np.float64)
    _load().da_oracle_v1_rows(B, H, T, d, *[_p(x) for x in t], int(layer), int(bool(softmax1)), idx.shape[0],
                              idx.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)), _p(out))
    return out


def _v2_check(q, k, v, lam, decode: bool):
    if decode:
        B, Hq, d = q.shape
        _, L, Hkv, _ = k.shape
        assert k.shape == (B, L, Hkv, d) and v.shape == k.shape
        assert lam.shape == (B, Hq // 2)
        T = L
    else:
        B, T, Hq, d = q.shape
        Hkv = k.shape[2]
        assert k.shape == (B, T, Hkv, d) and v.shape == k.shape
        assert lam.shape == (B, T, Hq // 2)
    assert Hq % Hkv == 0 and (Hq // Hkv) % 2 == 0, (Hq, Hkv)
    return B, T, Hq, Hkv, d


def v2_fwd(q, k, v, lam, softmax1: bool = False) -> np.ndarray:
    """DIFF V2 prefill, all rows; returns ``[B, T, Hq/2, d]`` float64."""
    t = [_f64(x) for x in (q, k, v, lam)]
    B, T, Hq, Hkv, d = _v2_check(*t, decode=False)
    out = np.zeros((B, T, Hq // 2, d), dtype=np.float64)
    _load().da_oracle_v2_fwd(B, T, Hq, Hkv, d, *[_p(x) for x in t], int(bool(softmax1)), _p(out))
    return out


def v2_rows(q, k, v, lam, btp, softmax1: bool = False) -> np.ndarray:
    """DIFF V2 prefill for rows ``btp`` (``[n, 3]`` of (b, t, pair))."""
    t = [_f64(x) for x in (q, k, v, lam)]
    B, T, Hq, Hkv, d = _v2_check(*t, decode=False)
    idx = np.ascontiguousarray(np.asarray(btp, dtype=np.int64).reshape(-1, 3))
    assert (idx[:, 0] < B).all() and (idx[:, 1] < T).all() and (idx[:, 2] < Hq // 2).all()
    out = np.zeros((idx.shape[0], d), dtype=np.float64)
    _load().da_oracle_v2_rows(B, T, Hq, Hkv, d, *[_p(x) for x in t], int(bool(softmax1)), idx.shape[0],
                              idx.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)), _p(out))
    return out


def v2_heads(q, k, v, softmax1: bool = False):
    """Every query head's causal attention before the pairs combine: q
    ``[B, T, Hq, d]``, k, v ``[B, T, Hkv, d]`` -> (attn ``[B, T, Hq, d]``, lse
    ``[B, Hq, T]``, the natural log of each row's softmax denominator)."""
    q, k, v = [_f64(x) for x in (q, k, v)]
    B, T, Hq, d = q.shape
    Hkv = k.shape[2]
    assert k.shape == (B, T, Hkv, d) and v.shape == k.shape and Hq % Hkv == 0
    attn = np.zeros((B, T, Hq, d), dtype=np.float64)
    lse = np.zeros((B, Hq, T), dtype=np.float64)
    _load().da_oracle_v2_heads(B, T, Hq, Hkv, d, _p(q), _p(k), _p(v), int(bool(softmax1)), _p(attn), _p(lse))
    return attn, lse


def v2_decode(q, k, v, lam, softmax1: bool = False) -> np.ndarray:
    """DIFF V2 decode; returns ``[B, Hq/2, d]`` float64."""
    t = [_f64(x) for x in (q, k, v, lam)]
    B, L, Hq, Hkv, d = _v2_check(*t, decode=True)
    out = np.zeros((B, Hq // 2, d), dtype=np.float64)
    _load().da_oracle_v2_decode(B, L, Hq, Hkv, d, *[_p(x) for x in t], int(bool(softmax1)), _p(out))
    return out


def v2_decode_multi(q, k, v, lam, softmax1: bool = False) -> np.ndarray:
    """DIFF V2 decode of nq new tokens per sequence; q ``[B, nq, Hq, d]``, k, v
    ``[B, L, Hkv, d]`` (the new tokens are the last nq entries), lam
    ``[B, nq, Hq/2]``; returns ``[B, nq, Hq/2, d]`` float64.

    New token i sits at cache position L - nq + i and, as a row of causal
    DiffAttnV2 ("Differential Transformer V2" article, DiffAttnV2
    pseudo-code), attends to positions 0 .. L - nq + i: it is the single-token
    decode over that prefix of the cache.
    """
    q, k, v, lam = [_f64(x) for x in (q, k, v, lam)]
    B, nq, Hq, d = q.shape
    L = k.shape[1]
    assert 1 <= nq <= L and lam.shape == (B, nq, Hq // 2)
    out = np.zeros((B, nq, Hq // 2, d), dtype=np.float64)
    for i in range(nq):
        n = L - nq + i + 1  # visible entries of new token i
        out[:, i] = v2_decode(q[:, i], k[:, :n], v[:, :n], lam[:, i], softmax1=softmax1)
    return out


def v2_decode_paged(q, k_pages, v_pages, block_table, seq_lens, lam, softmax1: bool = False) -> np.ndarray:
    """DIFF V2 decode over a paged, ragged cache; returns ``[B, Hq/2, d]`` float64.

    A page table only says where the cache entries are stored: token t of
    sequence b is row ``t % page_size`` of page ``block_table[b, t // page_size]``
    and the sequence holds ``seq_lens[b]`` entries.  Each sequence's entries
    are gathered into a dense ``[L_b, Hkv, d]`` cache and decoded by
    :func:`v2_decode` ("Differential Transformer V2" article, DiffAttnV2 at
    the newest position), or by :func:`v2_decode_multi` when q is
    ``[B, nq, Hq, d]`` (lam ``[B, nq, Hq/2]``, result ``[B, nq, Hq/2, d]``).
    The pages define no attention over an empty set: a new token that sees
    no entry (a sequence of length 0, or new token i of a sequence shorter
    than nq with L_b - nq + i < 0) is given the output 0 (with the off-by-one
    softmax that is also the limit, an extra zero key with a zero value).
    """
    q, kp, vp, lam = [_f64(x) for x in (q, k_pages, v_pages, lam)]
    table = np.asarray(block_table, dtype=np.int64)
    lens = np.asarray(seq_lens, dtype=np.int64)
    if q.ndim == 4:
        return _paged_multi(q, kp, vp, table, lens, lam, softmax1)
    B, Hq, d = q.shape
    num_pages, page, Hkv, _ = kp.shape
    assert vp.shape == kp.shape and kp.shape[3] == d
    assert table.ndim == 2 and table.shape[0] == B and lens.shape == (B,)
    assert lam.shape == (B, Hq // 2)
    out = np.zeros((B, Hq // 2, d), dtype=np.float64)
    for b in range(B):
        L = int(lens[b])
        if L == 0:
            continue
        t = np.arange(L)
        pg = table[b, t // page]
        assert ((pg >= 0) & (pg < num_pages)).all(), "page index outside the pool"
        k = kp[pg, t % page]  # [L, Hkv, d]
        v = vp[pg, t % page]
        out[b] = v2_decode(q[b:b + 1], k[None], v[None], lam[b:b + 1], softmax1=softmax1)[0]
    return out


def _paged_multi(q, kp, vp, table, lens, lam, softmax1):
    B, nq, Hq, d = q.shape
    page = kp.shape[1]
    assert lam.shape == (B, nq, Hq // 2)
    out = np.zeros((B, nq, Hq // 2, d), dtype=np.float64)
    for b in range(B):
        L = int(lens[b])
        if L == 0:
            continue
        t = np.arange(L)
        pg = table[b, t // page]
        assert ((pg >= 0) & (pg < kp.shape[0])).all(), "page index outside the pool"
        k, v = kp[pg, t % page], vp[pg, t % page]
        for i in range(nq):
            n = L - nq + i + 1  # visible entries of new token i
            if n > 0:
                out[b, i] = v2_decode(q[b:b + 1, i], k[None, :n], v[None, :n], lam[b:b + 1, i],
                                      softmax1=softmax1)[0]
    return out

