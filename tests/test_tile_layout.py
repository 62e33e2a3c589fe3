"""LDS tile layouts of the backward kernels, checked on the CPU.

A tile of 32 rows x d bf16 is copied into LDS with its 16-byte chunks
XOR-swizzled per row, and read back either as rows (ds_read_b128: lane
(li = lane & 31, hg = lane >> 5) reads row li, chunk (2 ks + hg), 16 lanes
per LDS pass) or transposed (ds_read_b64_tr_b16: in each group of 16 lanes,
lane j receives element j & 3 of the 8-byte rows addressed by lanes
4k + (j >> 2), k = 0..3; the per-lane addresses are those of the kernels'
TrBases).  These tests restate the three swizzles of
csrc/tile_ops.hpp (row, transpose, both ways) and the kernels' address
formulas, and check that
  * each layout's reads touch every bank at most once per pass (LDS: 64 banks
    of 4 bytes; 16-lane passes for the 16-byte reads; the transpose reads are
    checked for 16- and 32-lane passes);
  * the both-ways layout delivers, lane by lane, the same registers as the
    row layout (row reads) and the transpose layout (transpose reads), so one
    copy can serve both, and the row reads deliver the expected elements.
"""
import pytest


def k_sw(d, r):
    return (r & 15) if d >= 128 else ((r & 7) ^ ((r >> 3) & 1))


def v_sw(d, r):
    return (4 if d >= 128 else 2) * (r & 3)


def u_sw(d, r):
    v = ((r >> 2) & 1) | (((r >> 1) & 1) << 1) | ((((r >> 1) ^ (r >> 3)) & 1) << 2)
    return v | ((r & 1) << 3) if d >= 128 else v


def place(d, sw):
    """LDS image (bf16 elements) of a 32 x d tile whose element (r, c) = r*1000 + c."""
    nch, row = d // 8, d
    lds = [0] * (32 * row)
    for r in range(32):
        for c in range(nch):
            dst = r * row + ((c ^ sw(d, r)) % nch) * 8
            lds[dst:dst + 8] = [r * 1000 + 8 * c + e for e in range(8)]
    return lds


def worst_bank_use(addrs, nbytes, group):
    worst = 0
    for g0 in range(0, 64, group):
        use = {}
        for a in addrs[g0:g0 + group]:
            for i in range(nbytes // 4):
                b = (a // 4 + i) % 64
                use[b] = use.get(b, 0) + 1
        worst = max(worst, max(use.values()))
    return worst


def row_addrs(d, sw, ks):
    # lane part (li * RB + ((hg ^ sw(li)) << 4)) XOR 32 ks, as in the kernels
    return [((l & 31) * 2 * d + (((l >> 5) ^ sw(d, l & 31)) << 4)) ^ (32 * ks) for l in range(64)]


def trbase(d, sw, lane):
    nv = 4 if d >= 128 else 2
    l16, g16 = lane & 15, lane >> 4
    vr = 4 * (g16 >> 1) + (l16 >> 2)
    cl = 2 * (g16 & 1) + ((l16 & 3) >> 1)
    x = sw(d, vr)
    return [vr * 2 * d + (((4 * v + cl) ^ x) - 4 * v) * 16 + (l16 & 1) * 8 for v in range(nv)]


def tr_addrs(d, sw, both, cb, kk, h):
    nv = 4 if d >= 128 else 2
    c = (cb ^ 1) if (both and h) else cb
    return [trbase(d, sw, l)[c % nv] + c * 64 + (16 * kk + 8 * h) * 2 * d for l in range(64)]


def tr_read(lds, addrs):
    out = []
    for lane in range(64):
        g0, j = lane & ~15, lane & 15
        out.append([lds[addrs[g0 + 4 * k + (j >> 2)] // 2 + (j & 3)] for k in range(4)])
    return out


@pytest.mark.parametrize("d", [64, 128, 256])
def test_both_ways_swizzle_properties(d):
    rows = [u_sw(d, r) for r in range(16)]
    if d >= 128:
        assert sorted(rows) == list(range(16))
    else:  # 128-byte rows: two rows share a bank window, so each parity is a bijection
        assert sorted(rows[0::2]) == list(range(8)) and sorted(rows[1::2]) == list(range(8))
    for r in range(8):
        assert u_sw(d, r + 8) == u_sw(d, r) ^ 4
    for r in range(16):
        assert u_sw(d, r + 16) == u_sw(d, r)


@pytest.mark.parametrize("d", [64, 128, 256])
@pytest.mark.parametrize("layout", ["row", "both"])
def test_row_reads_conflict_free_and_exact(d, layout):
    sw = k_sw if layout == "row" else u_sw
    lds = place(d, sw)
    for ks in range(d // 16):
        addrs = row_addrs(d, sw, ks)
        assert worst_bank_use(addrs, 16, 16) == 1
        for l in range(64):
            got = lds[addrs[l] // 2: addrs[l] // 2 + 8]
            assert got == [(l & 31) * 1000 + 16 * ks + 8 * (l >> 5) + e for e in range(8)]


@pytest.mark.parametrize("d", [64, 128, 256])
def test_transpose_reads_conflict_free_and_equal(d):
    old, new = place(d, v_sw), place(d, u_sw)
    for kk in range(2):
        for cb in range(d // 32):
            for h in range(2):
                a_old = tr_addrs(d, v_sw, False, cb, kk, h)
                a_new = tr_addrs(d, u_sw, True, cb, kk, h)
                for group in (16, 32):
                    assert worst_bank_use(a_old, 8, group) == 1
                    assert worst_bank_use(a_new, 8, group) == 1
                assert tr_read(new, a_new) == tr_read(old, a_old)


@pytest.mark.parametrize("d", [64, 128, 256])
def test_single_layouts_conflict_in_the_other_read(d):
    # why the both-ways layout exists: the row swizzle conflicts in transpose
    # reads and the transpose swizzle in row reads
    assert worst_bank_use(tr_addrs(d, k_sw, False, 0, 0, 0), 8, 32) > 1
    assert worst_bank_use(row_addrs(d, v_sw, 0), 16, 16) > 1


@pytest.mark.parametrize("dv", [128, 256])
def test_half_width_transpose_reads(dv):
    # the V1 dK/dv kernel reads the transposed dD tile (dv = 2d wide) one
    # d-wide half m at a time: column block cb of half m is block m CB + cb,
    # read from the lane bases rotated by m CB plus m CB column blocks
    nv = 4 if dv >= 128 else 2
    cbh = dv // 64  # column blocks of a half
    for m in range(2):
        for lane in range(64):
            b = trbase(dv, u_sw, lane)
            rot = [b[(v + m * cbh) % nv] for v in range(nv)]
            for cb in range(cbh):
                for kk in range(2):
                    for h in range(2):
                        c = (cb ^ 1) if h else cb
                        got = rot[c % nv] + m * cbh * 64 + c * 64 + (16 * kk + 8 * h) * 2 * dv
                        want = tr_addrs(dv, u_sw, True, m * cbh + cb, kk, h)[lane]
                        assert got == want, (m, lane, cb, kk, h)
