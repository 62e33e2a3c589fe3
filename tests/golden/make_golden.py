"""Write the fixtures in this folder: the pages' definitions evaluated in
decimal arithmetic (40 significant digits) on tiny hand-chosen inputs.

    python tests/golden/make_golden.py

Nothing here imports the oracle or the GPU library: every value is computed
step by step from the definitions, with Python's ``decimal`` module for exp,
ln and sqrt, so the fixtures are independent of libm and of fp64 rounding.

Definitions followed ("Differential Transformer V2" article, DiffAttnV1 and
DiffAttnV2 pseudo-code; nanoGPT issue "How best to implement a differential
transformer?", Wilsontomass's module):
* lambda_init = 0.8 - 0.6 exp(-0.3 layer);
* V1: per map m, causal softmax(Q_m K_m^T / sqrt d) applied to the shared V
  (width 2d); D = A1 V - lam A2 V with lam = exp(lq1.lk1) - exp(lq2.lk2) +
  lambda_init; out = D / sqrt(mean(D^2) + 1e-5) * (1 - lambda_init);
* V2: per adjacent head pair (2p, 2p+1) of a GQA group, out = A_2p V -
  sigmoid(lam[t, p]) A_2p+1 V, no norm.
Inputs are short decimal fractions, so the fp64 values the oracle receives
are the nearest doubles to them (an input error below 1e-16 relative).
"""
from __future__ import annotations

from decimal import Decimal as Dd, getcontext
from pathlib import Path

getcontext().prec = 40
HERE = Path(__file__).resolve().parent


def softmax_rows(scores):
    mx = max(scores)
    w = [(s - mx).exp() for s in scores]
    z = sum(w)
    return [x / z for x in w]


def attend(qrow, keys, vals, i):
    """Causal attention of one query row over keys 0..i (scale 1/sqrt d)."""
    d = len(qrow)
    sc = Dd(d).sqrt()
    s = [sum(qrow[c] * keys[j][c] for c in range(d)) / sc for j in range(i + 1)]
    p = softmax_rows(s)
    return [sum(p[j] * vals[j][c] for j in range(i + 1)) for c in range(len(vals[0]))]


def lambda_init(layer):
    return Dd("0.8") - Dd("0.6") * (Dd("-0.3") * layer).exp()


def v1_case():
    T, d = 3, 2
    q1 = [["0.5", "-1.25"], ["1.5", "0.25"], ["-0.75", "2.0"]]
    k1 = [["1.0", "0.5"], ["-0.5", "1.5"], ["0.25", "-1.0"]]
    q2 = [["-1.0", "0.75"], ["0.125", "-0.5"], ["1.25", "1.0"]]
    k2 = [["0.5", "0.5"], ["1.75", "-0.25"], ["-1.5", "0.375"]]
    v = [["1.0", "-2.0", "0.5", "0.25"], ["-0.5", "1.5", "2.0", "-1.0"], ["0.75", "0.125", "-1.25", "3.0"]]
    lq1, lk1, lq2, lk2 = ["0.1", "-0.2"], ["0.05", "0.15"], ["-0.1", "0.3"], ["0.2", "0.1"]
    layer = 4
    D = lambda rows: [[Dd(x) for x in r] for r in rows]
    Q1, K1, Q2, K2, V = D(q1), D(k1), D(q2), D(k2), D(v)
    vec = lambda xs: [Dd(x) for x in xs]
    li = lambda_init(layer)
    lam = (sum(a * b for a, b in zip(vec(lq1), vec(lk1)))).exp() - \
          (sum(a * b for a, b in zip(vec(lq2), vec(lk2)))).exp() + li
    out = []
    for i in range(T):
        a1 = attend(Q1[i], K1, V, i)
        a2 = attend(Q2[i], K2, V, i)
        Dv = [x - lam * y for x, y in zip(a1, a2)]
        rms = (sum(x * x for x in Dv) / len(Dv) + Dd("1e-5")).sqrt()
        out.append([x / rms * (1 - li) for x in Dv])
    inputs = {"T": T, "d": d, "layer": layer, "q1": q1, "k1": k1, "q2": q2, "k2": k2, "v": v,
              "lq1": lq1, "lk1": lk1, "lq2": lq2, "lk2": lk2}
    return inputs, lam, out


def v2_case():
    # B 1, T 3, Hq 4 (two pairs), Hkv 1 (one group of 4 heads sharing K, V), d 2
    T = 3
    q = [[["0.5", "1.0"], ["-1.0", "0.25"], ["1.5", "-0.5"], ["0.0", "2.0"]],
         [["-0.25", "0.75"], ["1.0", "1.0"], ["0.5", "-1.5"], ["2.0", "0.125"]],
         [["1.25", "-1.0"], ["-0.5", "-0.5"], ["0.75", "0.25"], ["-1.0", "1.5"]]]
    k = [["1.0", "-0.5"], ["0.25", "1.25"], ["-1.5", "0.5"]]
    v = [["2.0", "-1.0"], ["0.5", "0.75"], ["-1.25", "1.5"]]
    lam = [["0.5", "-2.0"], ["1.5", "0.0"], ["-0.75", "3.0"]]
    D = lambda rows: [[Dd(x) for x in r] for r in rows]
    K, V = D(k), D(v)
    out = []
    for t in range(T):
        row = []
        for p in range(2):
            ae = attend([Dd(x) for x in q[t][2 * p]], K, V, t)
            ao = attend([Dd(x) for x in q[t][2 * p + 1]], K, V, t)
            sg = 1 / (1 + (-Dd(lam[t][p])).exp())
            row.append([x - sg * y for x, y in zip(ae, ao)])
        out.append(row)
    return {"T": T, "q": q, "k": k, "v": v, "lam": lam}, out


def main():
    lines = ["# lambda_init = 0.8 - 0.6 exp(-0.3 layer), 40-digit decimal, layers 0..27",
             "# (\"Differential Transformer V2\" article, DiffAttnV1 pseudo-code; the 3B-class",
             "#  model of Hacker News item 41780844 has 28 layers)"]
    lines += [f"{l} {lambda_init(l)}" for l in range(28)]
    (HERE / "lambda_init.txt").write_text("\n".join(lines) + "\n")

    inp, lam, out = v1_case()
    lines = ["# DIFF V1 forward, B 1, H 1, T 3, d 2 (V width 4), layer 4: inputs then lam then out[t][c],",
             "# 40-digit decimal (\"Differential Transformer V2\" article, DiffAttnV1 pseudo-code;",
             "#  nanoGPT issue \"How best to implement a differential transformer?\", RMSNorm eps 1e-5)"]
    for key in ("q1", "k1", "q2", "k2", "v"):
        lines += [f"{key} {t} " + " ".join(inp[key][t]) for t in range(inp["T"])]
    for key in ("lq1", "lk1", "lq2", "lk2"):
        lines.append(f"{key} " + " ".join(inp[key]))
    lines.append(f"layer {inp['layer']}")
    lines.append(f"lam {lam}")
    lines += [f"out {t} " + " ".join(str(x) for x in out[t]) for t in range(inp["T"])]
    (HERE / "v1_tiny.txt").write_text("\n".join(lines) + "\n")

    inp, out = v2_case()
    lines = ["# DIFF V2 prefill, B 1, T 3, Hq 4, Hkv 1, d 2: inputs then out[t][p][c], 40-digit decimal",
             "# (\"Differential Transformer V2\" article, DiffAttnV2 pseudo-code: heads 2p and 2p+1",
             "#  of one GQA group share K and V; out = A_2p V - sigmoid(lam[t, p]) A_2p+1 V)"]
    for t in range(inp["T"]):
        lines += [f"q {t} {h} " + " ".join(inp["q"][t][h]) for h in range(4)]
    lines += [f"k {t} " + " ".join(inp["k"][t]) for t in range(inp["T"])]
    lines += [f"v {t} " + " ".join(inp["v"][t]) for t in range(inp["T"])]
    lines += [f"lam {t} " + " ".join(inp["lam"][t]) for t in range(inp["T"])]
    lines += [f"out {t} {p} " + " ".join(str(x) for x in out[t][p]) for t in range(inp["T"]) for p in range(2)]
    (HERE / "v2_tiny.txt").write_text("\n".join(lines) + "\n")


if __name__ == "__main__":
    main()
