"""ctypes binding over libdiffattn.so (include/diffattn.h).

Argument marshalling only: tensors are passed as (data_ptr, role strides);
every step of the computation runs in the library's HIP kernels.  torch is
used for device memory, strides and the current stream.  If the library is
not built the calls raise -- there is no fallback path.

Logical layouts (any strided view with a unit-stride last axis is accepted):
  v1_fwd     q1, q2, k1, k2 [B,H,T,d]; v [B,H,T,2d]; lambda vectors [d] fp32;
             returns / writes out [B,T,H,2d]
  v2_fwd     q [B,T,Hq,d]; k, v [B,T,Hkv,d]; lam [B,T,Hq/2] fp32 logits;
             returns / writes out [B,T,Hq/2,d]
  v2_decode  q [B,Hq,d]; k_cache, v_cache [B,L,Hkv,d]; lam [B,Hq/2] fp32;
             returns / writes out [B,Hq/2,d]
  v2_decode_multi
             q [B,nq,Hq,d]; k_cache, v_cache [B,L,Hkv,d] holding the nq new tokens
             last; lam [B,nq,Hq/2] fp32; returns / writes out [B,nq,Hq/2,d]
  v2_decode_paged
             q [B,Hq,d] or [B,nq,Hq,d]; k_pages, v_pages [num_pages,page_size,Hkv,d];
             block_table int32 [B, >= ceil(max_len/page_size)]; seq_lens
             int32 [B]; lam [B,Hq/2] fp32; returns / writes out [B,Hq/2,d]
  v1_fwd_train  as v1_fwd, also returning attn1, attn2 [B,T,H,2d] and lse fp32 [2,B,H,T]
  v1_bwd     gradients dq1, dq2, dk1, dk2 [B,H,T,d], dv [B,H,T,2d] and the four
             lambda vectors' gradients fp32 [d] from dout [B,T,H,2d] and the
             training forward's attn1, attn2, lse
  v2_fwd_train  as v2_fwd, also returning attn [B,T,Hq,d] and lse fp32 [B,Hq,T]
  v2_bwd     gradients dq [B,T,Hq,d], dk, dv [B,T,Hkv,d], dlam fp32 [B,T,Hq/2]
             from dout [B,T,Hq/2,d] and the training forward's attn, lse
  rope       x [B,T,H,d] rotated (rotary embedding, rows at positions pos0 + t)
  v2_lambda_proj  x [B,T,dm], w [P,dm] -> fp32 logits [B,T,P]
Each takes ``softmax1=True`` for the off-by-one softmax entry points
(``diffattn_*_softmax1``: every map's denominator gains exp(0)).  v1_fwd,
v2_fwd, v2_decode and v2_decode_paged take ``theta=`` for the rotary-embedding
entry points (``diffattn_*_rope``: q rotated in the kernel, prefill k rotated
into a workspace, decode caches holding rotated keys).
"""
from __future__ import annotations

import ctypes
import os
from pathlib import Path

import torch

# DIFFATTN_LIBRARY names another build of the same sources to load (the
# host-sanitizer test links one); by default the in-tree libdiffattn.so.
_LIB_PATH = Path(os.environ.get("DIFFATTN_LIBRARY") or Path(__file__).resolve().parent / "libdiffattn.so")
_lib = None

DA_FP32, DA_BF16 = 0, 1
_STATUS = {0: "DA_OK", 1: "DA_E_NULL", 2: "DA_E_DTYPE", 3: "DA_E_SHAPE", 4: "DA_E_LAYOUT",
           5: "DA_E_UNSUPPORTED", 6: "DA_E_WORKSPACE", 7: "DA_E_LAUNCH", 8: "DA_E_SCRATCH"}


class DiffAttnError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        self.name = _STATUS.get(status, str(status))
        msg = load_library().diffattn_status_string(status).decode()
        super().__init__(f"{where}: {self.name} ({msg})")


class DaIn(ctypes.Structure):
    _fields_ = [("ptr", ctypes.c_void_p), ("sb", ctypes.c_int64), ("sh", ctypes.c_int64), ("st", ctypes.c_int64)]


class DaOut(ctypes.Structure):
    _fields_ = [("ptr", ctypes.c_void_p), ("sb", ctypes.c_int64), ("sh", ctypes.c_int64), ("st", ctypes.c_int64)]


def library_path() -> Path:
    return _LIB_PATH


def load_library():
    """Load libdiffattn.so; raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not _LIB_PATH.exists():
        raise RuntimeError(f"{_LIB_PATH} is not built: run `python -m differential_attention_diffattn_amd.build` "
                           "(or __graft_entry__.build())")
    lib = ctypes.CDLL(str(_LIB_PATH))
    i, vp, fp = ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p
    for sfx in ("", "_softmax1"):
        f = getattr(lib, "diffattn_v1_fwd" + sfx)
        f.argtypes = [i, i, i, i, i, DaIn, DaIn, DaIn, DaIn, DaIn, fp, fp, fp, fp, i, DaOut, vp]
        f.restype = i
        f = getattr(lib, "diffattn_v2_fwd" + sfx)
        f.argtypes = [i, i, i, i, i, i, DaIn, DaIn, DaIn, DaIn, DaOut, vp]
        f.restype = i
        f = getattr(lib, "diffattn_v2_decode" + sfx)
        f.argtypes = [i, i, i, i, i, i, DaIn, DaIn, DaIn, DaIn, DaOut, vp, ctypes.c_size_t, vp]
        f.restype = i
        f = getattr(lib, "diffattn_v2_decode_multi" + sfx)
        f.argtypes = [i, i, i, i, i, i, i, DaIn, DaIn, DaIn, DaIn, DaOut, vp, ctypes.c_size_t, vp]
        f.restype = i
        f = getattr(lib, "diffattn_v2_decode_paged" + sfx)
        f.argtypes = [i, i, i, i, i, i, i, DaIn, DaIn, DaIn, i, i, vp, ctypes.c_int64, vp, DaIn, DaOut, vp,
                      ctypes.c_size_t, vp]
        f.restype = i
    lib.diffattn_v2_decode_noalloc.argtypes = [i, i, i, i, i, i, DaIn, DaIn, DaIn, DaIn, DaOut, vp]
    lib.diffattn_v2_decode_noalloc.restype = i
    lib.diffattn_v2_decode_noalloc_max_bytes.argtypes = []
    lib.diffattn_v2_decode_noalloc_max_bytes.restype = ctypes.c_size_t
    fl = ctypes.c_float
    lib.diffattn_rope.argtypes = [i, i, i, i, i, DaIn, DaOut, fl, i, vp]
    lib.diffattn_rope.restype = i
    for sfx in ("_rope", "_softmax1_rope"):
        f = getattr(lib, "diffattn_v1_fwd" + sfx)
        f.argtypes = [i, i, i, i, i, DaIn, DaIn, DaIn, DaIn, DaIn, fp, fp, fp, fp, i, fl, DaOut, vp, ctypes.c_size_t,
                      vp]
        f.restype = i
        f = getattr(lib, "diffattn_v2_fwd" + sfx)
        f.argtypes = [i, i, i, i, i, i, DaIn, DaIn, DaIn, DaIn, fl, DaOut, vp, ctypes.c_size_t, vp]
        f.restype = i
        f = getattr(lib, "diffattn_v2_decode" + sfx)
        f.argtypes = [i, i, i, i, i, i, DaIn, DaIn, DaIn, DaIn, fl, DaOut, vp, ctypes.c_size_t, vp]
        f.restype = i
        f = getattr(lib, "diffattn_v2_decode_paged" + sfx)
        f.argtypes = [i, i, i, i, i, i, i, DaIn, DaIn, DaIn, i, i, vp, ctypes.c_int64, vp, DaIn, fl, DaOut, vp,
                      ctypes.c_size_t, vp]
        f.restype = i
    for f in (lib.diffattn_v1_fwd_rope_workspace_bytes, lib.diffattn_v2_fwd_rope_workspace_bytes):
        f.argtypes = [i, i, i, i]
        f.restype = ctypes.c_size_t
    lib.diffattn_v2_lambda_proj.argtypes = [i, i, i, i, i, DaIn, DaIn, DaIn, vp]
    lib.diffattn_v2_lambda_proj.restype = i
    for sfx in ("", "_softmax1"):
        f = getattr(lib, "diffattn_v1_fwd_train" + sfx)
        f.argtypes = [i, i, i, i, i, DaIn, DaIn, DaIn, DaIn, DaIn, fp, fp, fp, fp, i, DaOut, DaOut, DaOut, vp, vp]
        f.restype = i
    lib.diffattn_v1_bwd.argtypes = [i, i, i, i, i, DaIn, DaIn, DaIn, DaIn, DaIn, fp, fp, fp, fp, i, DaIn, DaIn, vp,
                                    DaIn, DaOut, DaOut, DaOut, DaOut, DaOut, vp, vp, vp, vp, vp, ctypes.c_size_t, vp]
    lib.diffattn_v1_bwd.restype = i
    lib.diffattn_v1_bwd_workspace_bytes.argtypes = [i, i, i, i]
    lib.diffattn_v1_bwd_workspace_bytes.restype = ctypes.c_size_t
    for sfx in ("", "_softmax1"):
        f = getattr(lib, "diffattn_v2_fwd_train" + sfx)
        f.argtypes = [i, i, i, i, i, i, DaIn, DaIn, DaIn, DaIn, DaOut, DaOut, vp, vp]
        f.restype = i
    lib.diffattn_v2_bwd.argtypes = [i, i, i, i, i, i, DaIn, DaIn, DaIn, DaIn, DaIn, vp, DaIn, DaOut, DaOut, DaOut,
                                    DaOut, vp, ctypes.c_size_t, vp]
    lib.diffattn_v2_bwd.restype = i
    lib.diffattn_v2_bwd_workspace_bytes.argtypes = [i, i, i, i, i]
    lib.diffattn_v2_bwd_workspace_bytes.restype = ctypes.c_size_t
    lib.diffattn_v2_decode_workspace_bytes.argtypes = [i, i, i, i, i]
    lib.diffattn_v2_decode_workspace_bytes.restype = ctypes.c_size_t
    for f in (lib.diffattn_v2_decode_multi_workspace_bytes, lib.diffattn_v2_decode_paged_workspace_bytes):
        f.argtypes = [i, i, i, i, i, i]
        f.restype = ctypes.c_size_t
    lib.diffattn_lambda_init.argtypes = [i]
    lib.diffattn_lambda_init.restype = ctypes.c_double
    lib.diffattn_status_string.argtypes = [i]
    lib.diffattn_status_string.restype = ctypes.c_char_p
    _lib = lib
    return lib


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return DA_BF16
    if t.dtype == torch.float32:
        return DA_FP32
    raise TypeError(f"unsupported dtype {t.dtype}")


def _in(t: torch.Tensor, b, h, tok) -> DaIn:
    """Role strides of a tensor whose axes b/h/tok (None = absent) are given."""
    s = t.stride()
    return DaIn(t.data_ptr(), s[b] if b is not None else 0, s[h] if h is not None else 0,
                s[tok] if tok is not None else 0)


def _out(t: torch.Tensor, b, h, tok) -> DaOut:
    s = t.stride()
    return DaOut(t.data_ptr(), s[b] if b is not None else 0, s[h] if h is not None else 0,
                 s[tok] if tok is not None else 0)


def _stream(t: torch.Tensor):
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _check_device(*ts):
    dev = ts[0].device
    for t in ts:
        if t.device.type != "cuda" or t.device != dev:
            raise ValueError("all tensors must be on the same CUDA (HIP) device")
        if t.stride(-1) != 1 and t.shape[-1] > 1:
            raise ValueError("the last (head_dim) axis must be unit-stride")


def lambda_init(layer: int) -> float:
    return load_library().diffattn_lambda_init(int(layer))


def v1_fwd(q1, q2, k1, k2, v, lq1, lk1, lq2, lk2, layer: int, out: torch.Tensor | None = None,
           softmax1: bool = False, theta: float | None = None, workspace: torch.Tensor | None = None):
    """DIFF V1 forward; q*/k* [B,H,T,d], v [B,H,T,2d]; returns out [B,T,H,2d].
    ``theta``: rotary embedding of q1, q2, k1, k2 first (positions 0..T-1)."""
    lib = load_library()
    B, H, T, d = q1.shape
    for x in (q2, k1, k2):
        if tuple(x.shape) != (B, H, T, d):
            raise ValueError(f"q/k shape mismatch: {tuple(x.shape)} vs {(B, H, T, d)}")
    if tuple(v.shape) != (B, H, T, 2 * d):
        raise ValueError(f"v must be {(B, H, T, 2 * d)}, got {tuple(v.shape)}")
    for x in (q2, k1, k2, v):
        if x.dtype != q1.dtype:
            raise TypeError("q1, q2, k1, k2, v must share one dtype")
    lams = [x.contiguous() for x in (lq1, lk1, lq2, lk2)]
    for x in lams:
        if x.dtype != torch.float32 or tuple(x.shape) != (d,):
            raise ValueError("lambda vectors must be fp32 of shape [d]")
    if out is None:
        out = torch.empty((B, T, H, 2 * d), dtype=q1.dtype, device=q1.device)
    _check_device(q1, q2, k1, k2, v, out, *lams)
    if theta is not None:
        need = int(lib.diffattn_v1_fwd_rope_workspace_bytes(B, H, T, d))
        if workspace is None:
            workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=q1.device)
        name = "diffattn_v1_fwd" + ("_softmax1" if softmax1 else "") + "_rope"
        st = getattr(lib, name)(_dtype_code(q1), B, H, T, d, _in(q1, 0, 1, 2), _in(q2, 0, 1, 2),
                                      _in(k1, 0, 1, 2), _in(k2, 0, 1, 2), _in(v, 0, 1, 2),
                                      *[x.data_ptr() for x in lams], int(layer), float(theta), _out(out, 0, 2, 1),
                                      workspace.data_ptr(), workspace.numel() * workspace.element_size(),
                                      _stream(q1))
        if st != 0:
            raise DiffAttnError(st, name)
        return out
    name = "diffattn_v1_fwd" + ("_softmax1" if softmax1 else "")
    st = getattr(lib, name)(_dtype_code(q1), B, H, T, d,
                             _in(q1, 0, 1, 2), _in(q2, 0, 1, 2), _in(k1, 0, 1, 2), _in(k2, 0, 1, 2),
                             _in(v, 0, 1, 2), *[x.data_ptr() for x in lams], int(layer),
                             _out(out, 0, 2, 1), _stream(q1))
    if st != 0:
        raise DiffAttnError(st, name)
    return out


def _v1_shapes(q1, q2, k1, k2, v, lams):
    B, H, T, d = q1.shape
    for x in (q2, k1, k2):
        if tuple(x.shape) != (B, H, T, d):
            raise ValueError(f"q/k shape mismatch: {tuple(x.shape)} vs {(B, H, T, d)}")
    if tuple(v.shape) != (B, H, T, 2 * d):
        raise ValueError(f"v must be {(B, H, T, 2 * d)}, got {tuple(v.shape)}")
    for x in lams:
        if x.dtype != torch.float32 or tuple(x.shape) != (d,) or not x.is_contiguous():
            raise ValueError("lambda vectors must be contiguous fp32 of shape [d]")
    return B, H, T, d


def v1_fwd_train(q1, q2, k1, k2, v, lq1, lk1, lq2, lk2, layer: int, out=None, attn1=None, attn2=None, lse=None,
                 softmax1: bool = False):
    """DIFF V1 training forward; returns (out [B,T,H,2d], attn1, attn2 [B,T,H,2d], lse fp32 [2,B,H,T])."""
    lib = load_library()
    lams = [x.contiguous() for x in (lq1, lk1, lq2, lk2)]
    B, H, T, d = _v1_shapes(q1, q2, k1, k2, v, lams)
    mk = lambda: torch.empty((B, T, H, 2 * d), dtype=q1.dtype, device=q1.device)
    out = mk() if out is None else out
    attn1 = mk() if attn1 is None else attn1
    attn2 = mk() if attn2 is None else attn2
    lse = torch.empty((2, B, H, T), dtype=torch.float32, device=q1.device) if lse is None else lse
    if lse.dtype != torch.float32 or tuple(lse.shape) != (2, B, H, T) or not lse.is_contiguous():
        raise ValueError("lse must be a contiguous fp32 [2,B,H,T]")
    _check_device(q1, q2, k1, k2, v, out, attn1, attn2, *lams)
    name = "diffattn_v1_fwd_train" + ("_softmax1" if softmax1 else "")
    st = getattr(lib, name)(_dtype_code(q1), B, H, T, d, _in(q1, 0, 1, 2), _in(q2, 0, 1, 2), _in(k1, 0, 1, 2),
                            _in(k2, 0, 1, 2), _in(v, 0, 1, 2), *[x.data_ptr() for x in lams], int(layer),
                            _out(out, 0, 2, 1), _out(attn1, 0, 2, 1), _out(attn2, 0, 2, 1), lse.data_ptr(),
                            _stream(q1))
    if st != 0:
        raise DiffAttnError(st, name)
    return out, attn1, attn2, lse


def v1_bwd_workspace_bytes(B: int, H: int, T: int, d: int) -> int:
    return int(load_library().diffattn_v1_bwd_workspace_bytes(B, H, T, d))


def v1_bwd(q1, q2, k1, k2, v, lq1, lk1, lq2, lk2, layer: int, attn1, attn2, lse, dout, grads=None,
           workspace: torch.Tensor | None = None):
    """DIFF V1 backward; returns (dq1, dq2, dk1, dk2 [B,H,T,d], dv [B,H,T,2d],
    dlq1, dlk1, dlq2, dlk2 fp32 [d]); ``grads`` may supply those nine outputs."""
    lib = load_library()
    lams = [x.contiguous() for x in (lq1, lk1, lq2, lk2)]
    B, H, T, d = _v1_shapes(q1, q2, k1, k2, v, lams)
    for x in (attn1, attn2, dout):
        if tuple(x.shape) != (B, T, H, 2 * d):
            raise ValueError("attn1, attn2 and dout must be [B,T,H,2d]")
    if lse.dtype != torch.float32 or tuple(lse.shape) != (2, B, H, T) or not lse.is_contiguous():
        raise ValueError("lse must be a contiguous fp32 [2,B,H,T]")
    if grads is None:
        grads = [torch.empty_like(x) for x in (q1, q2, k1, k2, v)] + \
                [torch.empty(d, dtype=torch.float32, device=q1.device) for _ in range(4)]
    need = v1_bwd_workspace_bytes(B, H, T, d)
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=q1.device)
    _check_device(q1, q2, k1, k2, v, attn1, attn2, dout, *grads)
    st = lib.diffattn_v1_bwd(_dtype_code(q1), B, H, T, d, _in(q1, 0, 1, 2), _in(q2, 0, 1, 2), _in(k1, 0, 1, 2),
                             _in(k2, 0, 1, 2), _in(v, 0, 1, 2), *[x.data_ptr() for x in lams], int(layer),
                             _in(attn1, 0, 2, 1), _in(attn2, 0, 2, 1), lse.data_ptr(), _in(dout, 0, 2, 1),
                             *[_out(g, 0, 1, 2) for g in grads[:5]], *[g.data_ptr() for g in grads[5:]],
                             workspace.data_ptr(), workspace.numel() * workspace.element_size(), _stream(q1))
    if st != 0:
        raise DiffAttnError(st, "diffattn_v1_bwd")
    return tuple(grads)


def v2_fwd(q, k, v, lam, out: torch.Tensor | None = None, softmax1: bool = False, theta: float | None = None,
           workspace: torch.Tensor | None = None):
    """DIFF V2 prefill; q [B,T,Hq,d], k/v [B,T,Hkv,d], lam [B,T,Hq/2]; returns [B,T,Hq/2,d].
    ``theta``: rotary embedding of q and k first (positions 0..T-1)."""
    lib = load_library()
    B, T, Hq, d = q.shape
    Hkv = k.shape[2]
    if tuple(k.shape) != (B, T, Hkv, d) or tuple(v.shape) != (B, T, Hkv, d):
        raise ValueError("k, v must be [B,T,Hkv,d]")
    if tuple(lam.shape) != (B, T, Hq // 2) or lam.dtype != torch.float32:
        raise ValueError("lam must be fp32 [B,T,Hq/2]")
    if out is None:
        out = torch.empty((B, T, Hq // 2, d), dtype=q.dtype, device=q.device)
    _check_device(q, k, v, out)
    if theta is not None:
        need = int(lib.diffattn_v2_fwd_rope_workspace_bytes(B, T, Hkv, d))
        if workspace is None:
            workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=q.device)
        name = "diffattn_v2_fwd" + ("_softmax1" if softmax1 else "") + "_rope"
        st = getattr(lib, name)(_dtype_code(q), B, T, Hq, Hkv, d, _in(q, 0, 2, 1), _in(k, 0, 2, 1),
                                _in(v, 0, 2, 1), _in(lam, 0, 2, 1), float(theta), _out(out, 0, 2, 1),
                                workspace.data_ptr(), workspace.numel() * workspace.element_size(), _stream(q))
        if st != 0:
            raise DiffAttnError(st, name)
        return out
    name = "diffattn_v2_fwd" + ("_softmax1" if softmax1 else "")
    st = getattr(lib, name)(_dtype_code(q), B, T, Hq, Hkv, d, _in(q, 0, 2, 1), _in(k, 0, 2, 1),
                            _in(v, 0, 2, 1), _in(lam, 0, 2, 1), _out(out, 0, 2, 1), _stream(q))
    if st != 0:
        raise DiffAttnError(st, name)
    return out


def v2_fwd_train(q, k, v, lam, out=None, attn=None, lse=None, softmax1: bool = False):
    """DIFF V2 training forward; returns (out [B,T,Hq/2,d], attn [B,T,Hq,d], lse fp32 [B,Hq,T])."""
    lib = load_library()
    B, T, Hq, d = q.shape
    Hkv = k.shape[2]
    if tuple(k.shape) != (B, T, Hkv, d) or tuple(v.shape) != (B, T, Hkv, d):
        raise ValueError("k, v must be [B,T,Hkv,d]")
    if tuple(lam.shape) != (B, T, Hq // 2) or lam.dtype != torch.float32:
        raise ValueError("lam must be fp32 [B,T,Hq/2]")
    out = torch.empty((B, T, Hq // 2, d), dtype=q.dtype, device=q.device) if out is None else out
    attn = torch.empty((B, T, Hq, d), dtype=q.dtype, device=q.device) if attn is None else attn
    lse = torch.empty((B, Hq, T), dtype=torch.float32, device=q.device) if lse is None else lse
    if lse.dtype != torch.float32 or tuple(lse.shape) != (B, Hq, T) or not lse.is_contiguous():
        raise ValueError("lse must be a contiguous fp32 [B,Hq,T]")
    _check_device(q, k, v, out, attn)
    name = "diffattn_v2_fwd_train" + ("_softmax1" if softmax1 else "")
    st = getattr(lib, name)(_dtype_code(q), B, T, Hq, Hkv, d, _in(q, 0, 2, 1), _in(k, 0, 2, 1), _in(v, 0, 2, 1),
                            _in(lam, 0, 2, 1), _out(out, 0, 2, 1), _out(attn, 0, 2, 1), lse.data_ptr(), _stream(q))
    if st != 0:
        raise DiffAttnError(st, name)
    return out, attn, lse


def v2_bwd_workspace_bytes(B: int, T: int, Hq: int, Hkv: int, d: int) -> int:
    return int(load_library().diffattn_v2_bwd_workspace_bytes(B, T, Hq, Hkv, d))


def v2_bwd(q, k, v, lam, attn, lse, dout, dq=None, dk=None, dv=None, dlam=None,
           workspace: torch.Tensor | None = None):
    """DIFF V2 backward; returns (dq [B,T,Hq,d], dk, dv [B,T,Hkv,d], dlam fp32 [B,T,Hq/2])."""
    lib = load_library()
    B, T, Hq, d = q.shape
    Hkv = k.shape[2]
    if tuple(attn.shape) != (B, T, Hq, d) or tuple(dout.shape) != (B, T, Hq // 2, d):
        raise ValueError("attn must be [B,T,Hq,d] and dout [B,T,Hq/2,d]")
    if lse.dtype != torch.float32 or tuple(lse.shape) != (B, Hq, T) or not lse.is_contiguous():
        raise ValueError("lse must be a contiguous fp32 [B,Hq,T]")
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    dlam = torch.empty_like(lam) if dlam is None else dlam
    need = v2_bwd_workspace_bytes(B, T, Hq, Hkv, d)
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=q.device)
    _check_device(q, k, v, attn, dout, dq, dk, dv)
    st = lib.diffattn_v2_bwd(_dtype_code(q), B, T, Hq, Hkv, d, _in(q, 0, 2, 1), _in(k, 0, 2, 1), _in(v, 0, 2, 1),
                             _in(lam, 0, 2, 1), _in(attn, 0, 2, 1), lse.data_ptr(), _in(dout, 0, 2, 1),
                             _out(dq, 0, 2, 1), _out(dk, 0, 2, 1), _out(dv, 0, 2, 1), _out(dlam, 0, 2, 1),
                             workspace.data_ptr(), workspace.numel() * workspace.element_size(), _stream(q))
    if st != 0:
        raise DiffAttnError(st, "diffattn_v2_bwd")
    return dq, dk, dv, dlam


def v2_decode_workspace_bytes(B: int, L: int, Hq: int, Hkv: int, d: int) -> int:
    return int(load_library().diffattn_v2_decode_workspace_bytes(B, L, Hq, Hkv, d))


def v2_decode_multi_workspace_bytes(B: int, L: int, nq: int, Hq: int, Hkv: int, d: int) -> int:
    return int(load_library().diffattn_v2_decode_multi_workspace_bytes(B, L, nq, Hq, Hkv, d))


def v2_decode_paged_workspace_bytes(B: int, max_len: int, nq: int, Hq: int, Hkv: int, d: int) -> int:
    return int(load_library().diffattn_v2_decode_paged_workspace_bytes(B, max_len, nq, Hq, Hkv, d))


def v2_decode(q, k_cache, v_cache, lam, out: torch.Tensor | None = None,
              workspace: torch.Tensor | None = None, softmax1: bool = False, theta: float | None = None):
    """DIFF V2 decode; q [B,Hq,d], caches [B,L,Hkv,d], lam [B,Hq/2]; returns [B,Hq/2,d].
    ``theta``: q rotated to position L-1 in the kernel (the cache holds rotated keys)."""
    lib = load_library()
    B, Hq, d = q.shape
    L, Hkv = k_cache.shape[1], k_cache.shape[2]
    if tuple(k_cache.shape) != (B, L, Hkv, d) or tuple(v_cache.shape) != (B, L, Hkv, d):
        raise ValueError("caches must be [B,L,Hkv,d]")
    if tuple(lam.shape) != (B, Hq // 2) or lam.dtype != torch.float32:
        raise ValueError("lam must be fp32 [B,Hq/2]")
    if out is None:
        out = torch.empty((B, Hq // 2, d), dtype=q.dtype, device=q.device)
    need = v2_decode_workspace_bytes(B, L, Hq, Hkv, d)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    _check_device(q, k_cache, v_cache, out)
    name = "diffattn_v2_decode" + ("_softmax1" if softmax1 else "") + ("_rope" if theta is not None else "")
    extra = (ctypes.c_float(theta),) if theta is not None else ()
    st = getattr(lib, name)(_dtype_code(q), B, L, Hq, Hkv, d, _in(q, 0, 1, None),
                            _in(k_cache, 0, 2, 1), _in(v_cache, 0, 2, 1), _in(lam, 0, 1, None), *extra,
                            _out(out, 0, 1, None), workspace.data_ptr(),
                            workspace.numel() * workspace.element_size(), _stream(q))
    if st != 0:
        raise DiffAttnError(st, name)
    return out


def v2_decode_noalloc(q, k_cache, v_cache, lam, out: torch.Tensor):
    """DIFF V2 decode into a caller-given ``out`` [B,Hq/2,d] without any device
    allocation (the library's static scratch holds the split partials);
    q [B,Hq,d], caches [B,L,Hkv,d], lam [B,Hq/2]."""
    lib = load_library()
    B, Hq, d = q.shape
    L, Hkv = k_cache.shape[1], k_cache.shape[2]
    if tuple(k_cache.shape) != (B, L, Hkv, d) or tuple(v_cache.shape) != (B, L, Hkv, d):
        raise ValueError("caches must be [B,L,Hkv,d]")
    if tuple(lam.shape) != (B, Hq // 2) or lam.dtype != torch.float32:
        raise ValueError("lam must be fp32 [B,Hq/2]")
    if tuple(out.shape) != (B, Hq // 2, d):
        raise ValueError("out must be [B,Hq/2,d]")
    _check_device(q, k_cache, v_cache, out)
    st = lib.diffattn_v2_decode_noalloc(_dtype_code(q), B, L, Hq, Hkv, d, _in(q, 0, 1, None), _in(k_cache, 0, 2, 1),
                                        _in(v_cache, 0, 2, 1), _in(lam, 0, 1, None), _out(out, 0, 1, None),
                                        _stream(q))
    if st != 0:
        raise DiffAttnError(st, "diffattn_v2_decode_noalloc")
    return out


def v2_decode_multi(q, k_cache, v_cache, lam, out: torch.Tensor | None = None,
                    workspace: torch.Tensor | None = None, softmax1: bool = False):
    """DIFF V2 decode of nq new tokens; q [B,nq,Hq,d], caches [B,L,Hkv,d] (the new tokens are the
    last nq entries), lam [B,nq,Hq/2]; returns [B,nq,Hq/2,d]."""
    lib = load_library()
    B, nq, Hq, d = q.shape
    L, Hkv = k_cache.shape[1], k_cache.shape[2]
    if tuple(k_cache.shape) != (B, L, Hkv, d) or tuple(v_cache.shape) != (B, L, Hkv, d):
        raise ValueError("caches must be [B,L,Hkv,d]")
    if tuple(lam.shape) != (B, nq, Hq // 2) or lam.dtype != torch.float32:
        raise ValueError("lam must be fp32 [B,nq,Hq/2]")
    if out is None:
        out = torch.empty((B, nq, Hq // 2, d), dtype=q.dtype, device=q.device)
    need = v2_decode_multi_workspace_bytes(B, L, nq, Hq, Hkv, d)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    _check_device(q, k_cache, v_cache, out)
    name = "diffattn_v2_decode_multi" + ("_softmax1" if softmax1 else "")
    st = getattr(lib, name)(_dtype_code(q), B, L, nq, Hq, Hkv, d, _in(q, 0, 2, 1), _in(k_cache, 0, 2, 1),
                            _in(v_cache, 0, 2, 1), _in(lam, 0, 2, 1), _out(out, 0, 2, 1), workspace.data_ptr(),
                            workspace.numel() * workspace.element_size(), _stream(q))
    if st != 0:
        raise DiffAttnError(st, name)
    return out


def v2_decode_paged(q, k_pages, v_pages, block_table, seq_lens, lam, max_len: int,
                    out: torch.Tensor | None = None, workspace: torch.Tensor | None = None,
                    softmax1: bool = False, theta: float | None = None):
    """DIFF V2 decode over a paged cache; q [B,Hq,d] (one new token, returns [B,Hq/2,d]) or
    [B,nq,Hq,d] (nq new tokens, the last nq entries of each sequence; lam [B,nq,Hq/2]; returns
    [B,nq,Hq/2,d]); pages [num_pages,page_size,Hkv,d], block_table int32
    [B, >= ceil(max_len/page_size)], seq_lens int32 [B]."""
    lib = load_library()
    multi = q.dim() == 4
    if multi:
        B, nq, Hq, d = q.shape
    else:
        (B, Hq, d), nq = q.shape, 1
    num_pages, page_size, Hkv = k_pages.shape[0], k_pages.shape[1], k_pages.shape[2]
    if tuple(k_pages.shape) != (num_pages, page_size, Hkv, d) or tuple(v_pages.shape) != tuple(k_pages.shape):
        raise ValueError("k_pages, v_pages must be [num_pages,page_size,Hkv,d]")
    if block_table.dtype != torch.int32 or block_table.dim() != 2 or block_table.shape[0] != B:
        raise ValueError("block_table must be int32 [B, pages per sequence]")
    if block_table.stride(1) != 1:
        raise ValueError("block_table rows must be unit-stride")
    if seq_lens.dtype != torch.int32 or tuple(seq_lens.shape) != (B,) or seq_lens.stride(0) != 1:
        raise ValueError("seq_lens must be a contiguous int32 [B]")
    if block_table.shape[1] * page_size < max_len:
        raise ValueError("block_table has too few columns for max_len")
    lam_shape = (B, nq, Hq // 2) if multi else (B, Hq // 2)
    if tuple(lam.shape) != lam_shape or lam.dtype != torch.float32:
        raise ValueError(f"lam must be fp32 {list(lam_shape)}")
    if out is None:
        out = torch.empty(((B, nq) if multi else (B,)) + (Hq // 2, d), dtype=q.dtype, device=q.device)
    need = v2_decode_paged_workspace_bytes(B, max_len, nq, Hq, Hkv, d)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    _check_device(q, k_pages, v_pages, out, block_table, seq_lens)
    name = "diffattn_v2_decode_paged" + ("_softmax1" if softmax1 else "") + ("_rope" if theta is not None else "")
    extra = (ctypes.c_float(theta),) if theta is not None else ()
    ax = (0, 2, 1) if multi else (0, 1, None)  # (b, h, t) axes of q / lam / out
    st = getattr(lib, name)(_dtype_code(q), B, int(max_len), nq, Hq, Hkv, d, _in(q, *ax),
                            _in(k_pages, 0, 2, 1), _in(v_pages, 0, 2, 1), num_pages, page_size,
                            block_table.data_ptr(), block_table.stride(0), seq_lens.data_ptr(),
                            _in(lam, *ax), *extra, _out(out, *ax), workspace.data_ptr(),
                            workspace.numel() * workspace.element_size(), _stream(q))
    if st != 0:
        raise DiffAttnError(st, name)
    return out


def rope(x, theta: float = 10000.0, pos0: int = 0, out: torch.Tensor | None = None):
    """Rotary embedding of x [B,T,H,d] bf16, row t at position pos0 + t (out may be x: in place)."""
    lib = load_library()
    B, T, H, d = x.shape
    out = torch.empty_like(x) if out is None else out
    if tuple(out.shape) != (B, T, H, d):
        raise ValueError("out must have x's shape")
    _check_device(x, out)
    st = lib.diffattn_rope(_dtype_code(x), B, T, H, d, _in(x, 0, 2, 1), _out(out, 0, 2, 1), float(theta),
                           int(pos0), _stream(x))
    if st != 0:
        raise DiffAttnError(st, "diffattn_rope")
    return out


def v2_lambda_proj(x, w, out: torch.Tensor | None = None):
    """V2 lambda logits: x [B,T,dm] bf16, w [P,dm] bf16 (a linear layer's weight) -> fp32 [B,T,P]."""
    lib = load_library()
    B, T, dm = x.shape
    P = w.shape[0]
    if tuple(w.shape) != (P, dm):
        raise ValueError("w must be [P, dm]")
    out = torch.empty((B, T, P), dtype=torch.float32, device=x.device) if out is None else out
    if tuple(out.shape) != (B, T, P) or out.dtype != torch.float32:
        raise ValueError("out must be fp32 [B,T,P]")
    _check_device(x, w)
    st = lib.diffattn_v2_lambda_proj(_dtype_code(x), B, T, dm, P, DaIn(x.data_ptr(), x.stride(0), 0, x.stride(1)),
                                     DaIn(w.data_ptr(), 0, w.stride(0), 0), _in(out, 0, 2, 1), _stream(x))
    if st != 0:
        raise DiffAttnError(st, "diffattn_v2_lambda_proj")
    return out
