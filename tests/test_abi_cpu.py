"""The C-ABI library without a GPU: it loads, exports every symbol the header
declares, and every validation error is returned before anything is
enqueued (no HIP call happens on these paths, so they run on any host)."""
import ctypes
import re
from pathlib import Path

import pytest

ROOT = Path(__file__).resolve().parents[1]
HEADER = ROOT / "include" / "diffattn.h"


@pytest.fixture(scope="module")
def lib():
    from differential_attention_diffattn_amd import binding

    if not binding.library_path().exists():
        from differential_attention_diffattn_amd.build import build_library

        build_library()
    return binding.load_library()


def _declared_symbols():
    text = HEADER.read_text()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(diffattn_\w+)\s*\(", text)))


def test_header_declares_the_entry_points():
    syms = _declared_symbols()
    for need in ("diffattn_v1_fwd", "diffattn_v2_fwd", "diffattn_v2_decode",
                 "diffattn_v1_fwd_softmax1", "diffattn_v2_fwd_softmax1", "diffattn_v2_decode_softmax1",
                 "diffattn_v2_decode_paged", "diffattn_v2_decode_paged_softmax1",
                 "diffattn_v2_decode_paged_workspace_bytes", "diffattn_v2_decode_multi",
                 "diffattn_v2_decode_multi_softmax1", "diffattn_v2_decode_multi_workspace_bytes",
                 "diffattn_v2_decode_workspace_bytes", "diffattn_status_string"):
        assert need in syms


def test_library_exports_every_declared_symbol(lib):
    for name in _declared_symbols():
        assert hasattr(lib, name), name


def test_status_strings(lib):
    for code in range(9):
        s = lib.diffattn_status_string(code)
        assert s and len(s) > 1
    assert lib.diffattn_status_string(0) == b"ok"


def test_lambda_init_matches_oracle(lib):
    import oracle

    for layer in range(20):
        assert abs(lib.diffattn_lambda_init(layer) - oracle.lambda_init(layer)) < 1e-15


# ----- validation -----------------------------------------------------------
from differential_attention_diffattn_amd.binding import DaIn, DaOut  # noqa: E402

OK = 0
E_NULL, E_DTYPE, E_SHAPE, E_LAYOUT, E_UNSUP, E_WS = 1, 2, 3, 4, 5, 6
FAKE = 0x10000  # aligned, never dereferenced: validation fails before any launch


def _t(ptr=FAKE, sb=8 * 1024, sh=8 * 64, st=64, out=False):
    return (DaOut if out else DaIn)(ptr, sb, sh, st)


def _v1(lib, dtype=1, B=1, H=2, T=16, d=64, q1=None, v=None, out=None, lam=FAKE, layer=0):
    q = q1 or _t()
    return lib.diffattn_v1_fwd(dtype, B, H, T, d, q, _t(), _t(), _t(), v or _t(), lam, FAKE, FAKE, FAKE,
                               layer, out or _t(out=True), None)


def test_v1_validation(lib):
    assert _v1(lib, dtype=7) == E_DTYPE
    assert _v1(lib, T=0) == E_SHAPE
    assert _v1(lib, B=0) == E_SHAPE
    assert _v1(lib, layer=-1) == E_SHAPE
    assert _v1(lib, q1=_t(ptr=0)) == E_NULL
    assert _v1(lib, lam=0) == E_NULL
    assert _v1(lib, out=_t(ptr=0, out=True)) == E_NULL
    assert _v1(lib, q1=_t(ptr=FAKE + 2)) == E_LAYOUT        # not 16-byte aligned
    assert _v1(lib, v=_t(st=68)) == E_LAYOUT                # stride not a multiple of 8 bf16
    assert _v1(lib, q1=_t(sh=-64)) == E_LAYOUT              # negative stride
    assert _v1(lib, lam=FAKE + 2) == E_LAYOUT
    assert _v1(lib, d=96) == E_UNSUP                        # bf16 d in {64, 128}
    assert _v1(lib, dtype=0, d=16) == E_UNSUP               # fp32 d in {32, 64, 128}
    assert _v1(lib, dtype=0, v=_t(st=66)) == E_LAYOUT       # fp32: multiples of 4
    assert _v1(lib, v=_t(st=1 << 24)) == E_UNSUP            # token stride beyond 32-bit tile offsets


def _v2(lib, dtype=1, B=1, T=16, Hq=8, Hkv=2, d=128, lam=None, q=None):
    return lib.diffattn_v2_fwd(dtype, B, T, Hq, Hkv, d, q or _t(), _t(), _t(), lam or _t(), _t(out=True), None)


def test_v2_validation(lib):
    assert _v2(lib, dtype=3) == E_DTYPE
    assert _v2(lib, T=0) == E_SHAPE
    assert _v2(lib, Hq=8, Hkv=3) == E_SHAPE                  # not a multiple
    assert _v2(lib, Hq=6, Hkv=2) == E_SHAPE                  # odd group: a pair would straddle groups
    assert _v2(lib, q=_t(ptr=0)) == E_NULL
    assert _v2(lib, lam=_t(ptr=FAKE + 2)) == E_LAYOUT        # logits need 4-byte alignment
    assert _v2(lib, dtype=0) == E_UNSUP                      # fp32 V2 has no kernel
    assert _v2(lib, d=96) == E_UNSUP


def test_decode_workspace_query(lib):
    n = lib.diffattn_v2_decode_workspace_bytes(64, 32768, 64, 8, 128)
    # 64 batch x 8 groups x 8 splits (chunks of at most 4096 tokens) x 8 heads x (128 + 2) floats
    assert n == 64 * 8 * 8 * 8 * 130 * 4
    assert lib.diffattn_v2_decode_workspace_bytes(1, 1, 2, 1, 128) > 0
    assert lib.diffattn_v2_decode_workspace_bytes(0, 10, 8, 2, 128) == 0
    assert lib.diffattn_v2_decode_workspace_bytes(1, 10, 6, 2, 128) == 0


def _dec(lib, B=2, L=100, Hq=8, Hkv=2, d=128, ws=FAKE, wsb=None, dtype=1):
    need = lib.diffattn_v2_decode_workspace_bytes(B, L, Hq, Hkv, d)
    return lib.diffattn_v2_decode(dtype, B, L, Hq, Hkv, d, _t(), _t(), _t(), _t(), _t(out=True), ws,
                                  need if wsb is None else wsb, None)


def test_decode_validation(lib):
    assert _dec(lib, L=0) == E_SHAPE
    assert _dec(lib, Hq=10, Hkv=2) == E_SHAPE
    assert _dec(lib, dtype=0) == E_UNSUP
    assert _dec(lib, Hq=64, Hkv=2) == E_UNSUP                # 32 heads per group > one 16-wide block
    assert _dec(lib, ws=0) == E_WS
    assert _dec(lib, ws=FAKE + 4) == E_WS
    assert _dec(lib, wsb=100) == E_WS


def test_noalloc_decode_validation(lib):
    """The no-alloc decode checks its arguments like diffattn_v2_decode (all
    before it touches a device), and rejects sizes whose split partials do
    not fit its static scratch."""
    assert lib.diffattn_v2_decode_noalloc_max_bytes() == 16 << 20
    f = lambda B=2, L=100, Hq=8, Hkv=2, d=128, dtype=1, out=None: lib.diffattn_v2_decode_noalloc(
        dtype, B, L, Hq, Hkv, d, _t(), _t(), _t(), _t(), out if out is not None else _t(out=True), None)
    assert f(L=0) == E_SHAPE
    assert f(Hq=10, Hkv=2) == E_SHAPE
    assert f(dtype=0) == E_UNSUP
    assert f(Hq=64, Hkv=2) == E_UNSUP
    # one split of B x Hq x (d + 2) fp32 over 16 MiB
    assert f(B=2048, Hq=16, Hkv=2) == 8
    assert lib.diffattn_status_string(8) != lib.diffattn_status_string(7)


def test_softmax1_entry_points_validate_like_their_namesakes(lib):
    """The off-by-one softmax entry points share their namesakes' argument
    checks: the same invalid calls return the same status, before any launch."""
    v1 = lambda f, **kw: f(kw.get("dtype", 1), 1, 2, kw.get("T", 16), kw.get("d", 64), _t(), _t(), _t(), _t(),
                           _t(), kw.get("lam", FAKE), FAKE, FAKE, FAKE, 0, _t(out=True), None)
    for kw in ({"dtype": 7}, {"T": 0}, {"lam": 0}, {"d": 96}):
        assert v1(lib.diffattn_v1_fwd_softmax1, **kw) == v1(lib.diffattn_v1_fwd, **kw) != OK
    v2 = lambda f, **kw: f(kw.get("dtype", 1), 1, 16, kw.get("Hq", 8), 2, 128, _t(), _t(), _t(), _t(),
                           _t(out=True), None)
    for kw in ({"dtype": 3}, {"Hq": 6}, {"dtype": 0}):
        assert v2(lib.diffattn_v2_fwd_softmax1, **kw) == v2(lib.diffattn_v2_fwd, **kw) != OK
    need = lib.diffattn_v2_decode_workspace_bytes(2, 100, 8, 2, 128)
    dec = lambda f, ws: f(1, 2, 100, 8, 2, 128, _t(), _t(), _t(), _t(), _t(out=True), ws, need, None)
    assert dec(lib.diffattn_v2_decode_softmax1, 0) == dec(lib.diffattn_v2_decode, 0) == E_WS


def _paged(lib, f=None, B=2, max_len=100, Hq=8, Hkv=2, d=128, num_pages=20, page=16, table=FAKE,
           bt_stride=None, lens=FAKE, ws=FAKE, wsb=None, dtype=1, kst=None, nq=1):
    need = lib.diffattn_v2_decode_paged_workspace_bytes(B, max_len, nq, Hq, Hkv, d)
    bt = (max_len + page - 1) // page if bt_stride is None else bt_stride
    kp = _t(sb=page * Hkv * d, sh=d, st=Hkv * d if kst is None else kst)
    return (f or lib.diffattn_v2_decode_paged)(dtype, B, max_len, nq, Hq, Hkv, d, _t(), kp, _t(sb=page * Hkv * d),
                                               num_pages, page, table, bt, lens, _t(), _t(out=True), ws,
                                               need if wsb is None else wsb, None)


def test_paged_decode_validation(lib):
    assert _paged(lib, max_len=0) == E_SHAPE
    assert _paged(lib, num_pages=0) == E_SHAPE
    assert _paged(lib, page=8) == E_SHAPE                    # below 16
    assert _paged(lib, page=48) == E_SHAPE                   # not a power of two
    assert _paged(lib, bt_stride=6) == E_SHAPE               # 100 tokens need 7 pages of 16
    assert _paged(lib, Hq=10, Hkv=2) == E_SHAPE
    assert _paged(lib, table=0) == E_NULL
    assert _paged(lib, lens=0) == E_NULL
    assert _paged(lib, table=FAKE + 2) == E_LAYOUT
    assert _paged(lib, lens=FAKE + 1) == E_LAYOUT
    assert _paged(lib, dtype=0) == E_UNSUP
    assert _paged(lib, d=96) == E_UNSUP
    assert _paged(lib, Hq=64, Hkv=2) == E_UNSUP
    assert _paged(lib, page=1 << 16, kst=1 << 15) == E_UNSUP  # rows within a page need 32-bit offsets
    assert _paged(lib, ws=0) == E_WS
    assert _paged(lib, wsb=100) == E_WS
    assert _paged(lib, nq=0) == E_SHAPE
    assert _paged(lib, nq=3, wsb=lib.diffattn_v2_decode_paged_workspace_bytes(2, 100, 2, 8, 2, 128)) == E_WS
    for kw in ({"page": 8}, {"table": 0}, {"dtype": 0}, {"ws": 0}):
        assert _paged(lib, lib.diffattn_v2_decode_paged_softmax1, **kw) == _paged(lib, **kw) != OK


def _multi(lib, f=None, B=2, L=100, nq=4, Hq=8, Hkv=2, d=128, ws=FAKE, wsb=None, dtype=1, q=None):
    need = lib.diffattn_v2_decode_multi_workspace_bytes(B, L, nq, Hq, Hkv, d)
    return (f or lib.diffattn_v2_decode_multi)(dtype, B, L, nq, Hq, Hkv, d, q or _t(), _t(), _t(), _t(),
                                               _t(out=True), ws, need if wsb is None else wsb, None)


def test_multi_decode_workspace_and_validation(lib):
    one = lib.diffattn_v2_decode_workspace_bytes(64, 32768, 64, 8, 128)
    assert lib.diffattn_v2_decode_multi_workspace_bytes(64, 32768, 1, 64, 8, 128) == one
    # 4 tokens x 8 heads = 32 columns: one workgroup column group, 4x the partial columns
    assert lib.diffattn_v2_decode_multi_workspace_bytes(64, 32768, 4, 64, 8, 128) == 4 * one
    assert lib.diffattn_v2_decode_multi_workspace_bytes(2, 10, 0, 8, 2, 128) == 0
    assert _multi(lib, nq=0) == E_SHAPE
    assert _multi(lib, nq=101) == E_SHAPE                    # more new tokens than cache entries
    assert _multi(lib, q=_t(st=68)) == E_LAYOUT              # token stride of q checked when nq > 1
    assert _multi(lib, wsb=100) == E_WS
    assert _multi(lib, dtype=0) == E_UNSUP
    for kw in ({"nq": 0}, {"ws": 0}, {"dtype": 0}):
        assert _multi(lib, lib.diffattn_v2_decode_multi_softmax1, **kw) == _multi(lib, **kw) != OK



# ----- training forward and backward ---------------------------------------------

def test_training_entry_points_are_declared():
    syms = _declared_symbols()
    for need in ("diffattn_v1_fwd_train", "diffattn_v1_fwd_train_softmax1", "diffattn_v1_bwd",
                 "diffattn_v1_bwd_workspace_bytes", "diffattn_v2_fwd_train", "diffattn_v2_fwd_train_softmax1",
                 "diffattn_v2_bwd", "diffattn_v2_bwd_workspace_bytes"):
        assert need in syms


def _v1_train(lib, fn=None, dtype=1, d=64, attn2=None, lse=FAKE):
    fn = fn or lib.diffattn_v1_fwd_train
    return fn(dtype, 1, 2, 16, d, _t(), _t(), _t(), _t(), _t(), FAKE, FAKE, FAKE, FAKE, 0, _t(out=True),
              _t(out=True), attn2 or _t(out=True), lse, None)


def test_v1_fwd_train_validation(lib):
    for fn in (lib.diffattn_v1_fwd_train, lib.diffattn_v1_fwd_train_softmax1):
        assert _v1_train(lib, fn, lse=0) == E_NULL
        assert _v1_train(lib, fn, lse=FAKE + 2) == E_LAYOUT
        assert _v1_train(lib, fn, attn2=_t(ptr=0, out=True)) == E_NULL
        assert _v1_train(lib, fn, attn2=_t(st=68, out=True)) == E_LAYOUT
        assert _v1_train(lib, fn, dtype=0, d=64) == E_UNSUP    # the training forward is bf16 only
        assert _v1_train(lib, fn, d=96) == E_UNSUP


def test_v1_bwd_workspace_query(lib):
    B, H, T, d = 8, 6, 1024, 64
    Tp = 1024
    want = B * T * H * 2 * d * 2 + 4 * B * H * Tp * 4 + B * T * H * 4
    assert lib.diffattn_v1_bwd_workspace_bytes(B, H, T, d) == want
    # padded rows and 256-byte aligned regions
    # B=H=1, T=3, d=64: dD 3*128*2 = 768 B, rows padded to 128 (512 B each), 12 B of row terms -> 256
    assert lib.diffattn_v1_bwd_workspace_bytes(1, 1, 3, 64) == 768 + 4 * 512 + 256
    assert lib.diffattn_v1_bwd_workspace_bytes(0, 1, 3, 64) == 0


def _v1_bwd(lib, dtype=1, B=1, H=2, T=16, d=64, ws=FAKE, wsb=1 << 30, lse=FAKE, dl=FAKE, q1=None, dv=None):
    return lib.diffattn_v1_bwd(dtype, B, H, T, d, q1 or _t(), _t(), _t(), _t(), _t(), FAKE, FAKE, FAKE, FAKE, 0,
                               _t(), _t(), lse, _t(), _t(out=True), _t(out=True), _t(out=True), _t(out=True),
                               dv or _t(out=True), dl, FAKE, FAKE, FAKE, ws, wsb, None)


def test_v1_bwd_validation(lib):
    assert _v1_bwd(lib, dtype=5) == E_DTYPE
    assert _v1_bwd(lib, T=0) == E_SHAPE
    assert _v1_bwd(lib, q1=_t(ptr=0)) == E_NULL
    assert _v1_bwd(lib, lse=0) == E_NULL
    assert _v1_bwd(lib, dl=0) == E_NULL
    assert _v1_bwd(lib, dl=FAKE + 2) == E_LAYOUT
    assert _v1_bwd(lib, dv=_t(st=68, out=True)) == E_LAYOUT
    assert _v1_bwd(lib, dtype=0) == E_UNSUP                   # bf16 only
    assert _v1_bwd(lib, d=32) == E_UNSUP
    assert _v1_bwd(lib, ws=0) == E_WS
    assert _v1_bwd(lib, ws=FAKE + 16) == E_WS                 # 256-byte alignment
    assert _v1_bwd(lib, wsb=lib.diffattn_v1_bwd_workspace_bytes(1, 2, 16, 64) - 1) == E_WS


def _v2_bwd(lib, dtype=1, Hq=8, Hkv=2, d=128, ws=FAKE, wsb=1 << 30, lse=FAKE):
    return lib.diffattn_v2_bwd(dtype, 1, 16, Hq, Hkv, d, _t(), _t(), _t(), _t(), _t(), lse, _t(), _t(out=True),
                               _t(out=True), _t(out=True), _t(out=True), ws, wsb, None)


def test_v2_training_validation(lib):
    assert lib.diffattn_v2_bwd_workspace_bytes(1, 8192, 64, 8, 128) == 2 * 64 * 8192 * 4
    assert lib.diffattn_v2_bwd_workspace_bytes(1, 16, 6, 2, 128) == 0   # odd group
    assert _v2_bwd(lib, Hq=6) == E_SHAPE
    assert _v2_bwd(lib, lse=0) == E_NULL
    assert _v2_bwd(lib, dtype=0) == E_UNSUP
    assert _v2_bwd(lib, ws=0) == E_WS
    assert _v2_bwd(lib, wsb=100) == E_WS
    for fn in (lib.diffattn_v2_fwd_train, lib.diffattn_v2_fwd_train_softmax1):
        assert fn(1, 1, 16, 8, 2, 128, _t(), _t(), _t(), _t(), _t(out=True), _t(out=True), 0, None) == E_NULL


# ----- rotary embedding and lambda projection ------------------------------------

def test_prologue_entry_points_are_declared(lib):
    syms = _declared_symbols()
    for need in ("diffattn_rope", "diffattn_v1_fwd_rope", "diffattn_v1_fwd_rope_workspace_bytes",
                 "diffattn_v2_fwd_rope", "diffattn_v2_fwd_rope_workspace_bytes", "diffattn_v2_decode_rope",
                 "diffattn_v2_decode_paged_rope", "diffattn_v2_lambda_proj", "diffattn_v1_fwd_softmax1_rope",
                 "diffattn_v2_fwd_softmax1_rope", "diffattn_v2_decode_softmax1_rope",
                 "diffattn_v2_decode_paged_softmax1_rope"):
        assert need in syms and hasattr(lib, need)


def test_rope_validation(lib):
    f = lambda **k: lib.diffattn_rope(k.get("dtype", 1), 1, k.get("T", 16), 2, k.get("d", 64), _t(),
                                      k.get("out", _t(out=True)), ctypes.c_float(k.get("theta", 1e4)),
                                      k.get("pos0", 0), None)
    assert f(theta=0.0) == E_SHAPE
    assert f(theta=-1.0) == E_SHAPE
    assert f(theta=float("inf")) == E_SHAPE
    assert f(pos0=-1) == E_SHAPE
    assert f(pos0=(1 << 24) - 8) == E_SHAPE                  # positions must stay exact in fp32
    assert f(T=0) == E_SHAPE
    assert f(out=_t(ptr=0, out=True)) == E_NULL
    assert f(dtype=0) == E_UNSUP
    assert f(d=12) == E_UNSUP                                 # multiples of 8
    assert f(d=264) == E_UNSUP                                # at most 256 (128 frequencies)


def test_prefill_rope_validation(lib):
    assert lib.diffattn_v2_fwd_rope_workspace_bytes(1, 8192, 8, 128) == 8192 * 8 * 128 * 2
    assert lib.diffattn_v1_fwd_rope_workspace_bytes(8, 6, 1024, 64) == 2 * 8 * 6 * 1024 * 64 * 2
    v2 = lambda ws=FAKE, wsb=1 << 30, theta=1e4: lib.diffattn_v2_fwd_rope(
        1, 1, 16, 8, 2, 128, _t(), _t(), _t(), _t(), ctypes.c_float(theta), _t(out=True), ws, wsb, None)
    assert v2(ws=0) == E_WS
    assert v2(ws=FAKE + 16) == E_WS
    assert v2(wsb=100) == E_WS
    assert v2(theta=0.0) == E_SHAPE
    v1 = lambda dtype=1, ws=FAKE, wsb=1 << 30: lib.diffattn_v1_fwd_rope(
        dtype, 1, 2, 16, 64, _t(), _t(), _t(), _t(), _t(), FAKE, FAKE, FAKE, FAKE, 0, ctypes.c_float(1e4),
        _t(out=True), ws, wsb, None)
    assert v1(dtype=0) == E_UNSUP
    assert v1(wsb=lib.diffattn_v1_fwd_rope_workspace_bytes(1, 2, 16, 64) - 1) == E_WS


def test_decode_rope_validation(lib):
    f = lambda theta=1e4, wsb=1 << 30: lib.diffattn_v2_decode_rope(
        1, 2, 100, 8, 2, 128, _t(), _t(), _t(), _t(), ctypes.c_float(theta), _t(out=True), FAKE, wsb, None)
    assert f(theta=0.0) == E_SHAPE
    assert f(theta=float("nan")) == E_SHAPE
    assert f(wsb=100) == E_WS


def test_lambda_proj_validation(lib):
    f = lambda dtype=1, dm=4096, out=FAKE: lib.diffattn_v2_lambda_proj(dtype, 1, 16, dm, 32, _t(), _t(),
                                                                        DaIn(out, 0, 4, 128), None)
    assert f(dm=100) == E_UNSUP                               # multiples of 128
    assert f(dm=192) == E_UNSUP
    assert f(dtype=0) == E_UNSUP
    assert f(out=0) == E_NULL
    assert f(out=FAKE + 2) == E_LAYOUT
