"""The oracle against the fixtures in tests/golden/: the pages' definitions
evaluated in 40-digit decimal arithmetic on tiny hand-chosen inputs
(tests/golden/make_golden.py; no page prints a worked numerical example, so
these are the definitions evaluated, not printed values)."""
from __future__ import annotations

from pathlib import Path

import numpy as np
import pytest

import oracle

G = Path(__file__).resolve().parent / "golden"


def _rows(name):
    for line in (G / name).read_text().splitlines():
        if line and not line.startswith("#"):
            yield line.split()


def test_lambda_init_fixture():
    n = 0
    for layer, val in _rows("lambda_init.txt"):
        assert abs(oracle.lambda_init(int(layer)) - float(val)) < 2e-16
        n += 1
    assert n == 28


def test_v1_tiny_fixture():
    T, d = 3, 2
    arr = {k: np.zeros((1, 1, T, d if k != "v" else 2 * d)) for k in ("q1", "k1", "q2", "k2", "v")}
    lams, out_ref, lam_ref, layer = {}, np.zeros((1, T, 1, 2 * d)), None, None
    for r in _rows("v1_tiny.txt"):
        if r[0] in arr:
            arr[r[0]][0, 0, int(r[1])] = [float(x) for x in r[2:]]
        elif r[0] in ("lq1", "lk1", "lq2", "lk2"):
            lams[r[0]] = np.array([float(x) for x in r[1:]])
        elif r[0] == "layer":
            layer = int(r[1])
        elif r[0] == "lam":
            lam_ref = float(r[1])
        elif r[0] == "out":
            out_ref[0, int(r[1]), 0] = [float(x) for x in r[2:]]
    lam = oracle.v1_lambda(lams["lq1"], lams["lk1"], lams["lq2"], lams["lk2"], layer)
    assert abs(lam - lam_ref) < 1e-14
    got = oracle.v1_fwd(arr["q1"], arr["q2"], arr["k1"], arr["k2"], arr["v"],
                        lams["lq1"], lams["lk1"], lams["lq2"], lams["lk2"], layer)
    np.testing.assert_allclose(got, out_ref, rtol=0, atol=1e-13)


def test_v2_tiny_fixture():
    T = 3
    q, k, v = np.zeros((1, T, 4, 2)), np.zeros((1, T, 1, 2)), np.zeros((1, T, 1, 2))
    lam, out_ref = np.zeros((1, T, 2)), np.zeros((1, T, 2, 2))
    for r in _rows("v2_tiny.txt"):
        if r[0] == "q":
            q[0, int(r[1]), int(r[2])] = [float(x) for x in r[3:]]
        elif r[0] in ("k", "v"):
            (k if r[0] == "k" else v)[0, int(r[1]), 0] = [float(x) for x in r[2:]]
        elif r[0] == "lam":
            lam[0, int(r[1])] = [float(x) for x in r[2:]]
        elif r[0] == "out":
            out_ref[0, int(r[1]), int(r[2])] = [float(x) for x in r[3:]]
    got = oracle.v2_fwd(q, k, v, lam)
    np.testing.assert_allclose(got, out_ref, rtol=0, atol=1e-13)
    # the last row is the decode of the newest token over the whole cache
    dec = oracle.v2_decode(q[:, T - 1], k, v, lam[:, T - 1])
    np.testing.assert_allclose(dec, out_ref[:, T - 1], rtol=0, atol=1e-13)
