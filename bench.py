#!/usr/bin/env python3
"""Benchmark of the differential-attention forward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--only NAME] [--no-cpu-baseline] [--softmax1]

Headline workload (the `value`): the DIFF V2 causal GQA prefill of the
"Differential Transformer V2" article's DiffAttnV2 at B=1, T=8192, 64 query
heads (32 differential pairs), 8 kv heads, head_dim 128, bf16 -- the largest
configuration of the metric that fits one GPU.  One step = one call; up to
10 consecutive steps are captured in one HIP graph and replayed together
(the timed region still runs exactly K calls).  value =
algorithmic TFLOP/s over the K timed steps (only unmasked (i, j<=i) pairs are
counted: 2*B*Hq*d*T(T+1) per call).  Inputs are seeded synthetic N(0,1)
tensors (lambda logits N(0,1) fp32) already resident in HBM.

The JSON line also carries:
  roofline      the prefill kernel's per-launch duration (HIP events on the
                stream the library launches on) against the bf16 dense MFMA
                peak;
  cpu_baseline  the fp64 oracle timed on a bounded sample of rows of the same
                workload on this host's cores (the oracle leg);
  parity        the oracle leg's check of the timed output: sampled rows of
                every workload against the oracle (outside the timed region);
  secondary     the other full-size workloads (V1 at the GPT-2-small and
                3B-class shapes, the V1 backward at both shapes and the V2
                backward (each timed without its training forward), V2
                decode, V2 decode of a ragged batch over a paged cache, V2
                decode of 4 new tokens per sequence, V2 prefill and decode
                with the rotary embedding, the V2 lambda projection),
                each with its own roofline and parity; a secondary step is
                8 launches of the workload (warm-up ~0.3 s of its own calls;
                the GPT-2-small V1 step is its 12 layer calls 0..11).
Logs go to stderr; stdout holds exactly one JSON line.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "diff-attn causal fwd TFLOP/s (bf16, % MFMA peak); V2 decode HBM GB/s (% peak)"
PEAK_BF16_TFLOPS = 2500.0  # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0      # MI355X HBM3E
HEADLINE = "v2_prefill_B1_T8192_Hq64_Hkv8_d128"
SECONDARY = ["v1_gpt2small_B8_H6_T1024_d64", "v1_3b_B2_H12_T4096_d128", "v1_backward_B8_H6_T1024_d64",
             "v1_backward_B2_H12_T4096_d128", "v2_backward_B1_T8192_Hq64_Hkv8_d128",
             "v2_decode_B64_L32768_Hq64_Hkv8_d128", "v2_decode_paged_B64_Lmax32768_P64_Hq64_Hkv8_d128",
             "v2_decode_multi_B64_L32768_nq4_Hq64_Hkv8_d128", "v2_prefill_rope_B1_T8192_Hq64_Hkv8_d128",
             "v2_decode_rope_B64_L32768_Hq64_Hkv8_d128", "v2_lambda_proj_B1_T8192_dm4096_P32"]


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def _caller(w, x, binding, torch, softmax1=False):
    """Return (fn(layer) -> None that enqueues one call of workload w, dict of
    the tensors that call writes) (softmax1: the off-by-one softmax entry
    points)."""
    if w.kind == "v1":
        out = torch.empty((w.B, w.T, w.H, 2 * w.d), dtype=w.torch_dtype, device=x["v"].device)
        args = [x[n] for n in ("q1", "q2", "k1", "k2", "v", "lq1", "lk1", "lq2", "lk2")]
        return (lambda layer: binding.v1_fwd(*args, layer, out=out, softmax1=softmax1)), {"out": out}
    if w.kind == "v2":
        out = torch.empty((w.B, w.T, w.Hq // 2, w.d), dtype=w.torch_dtype, device=x["v"].device)
        return (lambda layer: binding.v2_fwd(x["q"], x["k"], x["v"], x["lam"], out=out, softmax1=softmax1)), \
            {"out": out}
    if w.kind == "v2_rope":  # rotary embedding: k rotation pass + prefill with q rotated in its prologue
        out = torch.empty((w.B, w.T, w.Hq // 2, w.d), dtype=w.torch_dtype, device=x["v"].device)
        ws = torch.empty(int(binding.load_library().diffattn_v2_fwd_rope_workspace_bytes(w.B, w.T, w.Hkv, w.d)),
                         dtype=torch.uint8, device=x["v"].device)
        return (lambda layer: binding.v2_fwd(x["q"], x["k"], x["v"], x["lam"], out=out, theta=1e4, workspace=ws)), \
            {"out": out}
    if w.kind == "lam_proj":
        out = torch.empty((w.B, w.T, w.Hq), dtype=torch.float32, device=x["x"].device)
        return (lambda layer: binding.v2_lambda_proj(x["x"], x["w"], out=out)), {"out": out}
    if w.kind == "v1_bwd":  # the timed call is the backward; the training forward runs once, untimed
        args = [x[n] for n in ("q1", "q2", "k1", "k2", "v", "lq1", "lk1", "lq2", "lk2")]
        layer0 = w.layers[0]
        _, a1, a2, lse = binding.v1_fwd_train(*args, layer0, softmax1=softmax1)
        grads = [torch.empty_like(x[n]) for n in ("q1", "q2", "k1", "k2", "v", "lq1", "lk1", "lq2", "lk2")]
        ws = torch.empty(binding.v1_bwd_workspace_bytes(w.B, w.H, w.T, w.d), dtype=torch.uint8, device=x["v"].device)
        return (lambda layer: binding.v1_bwd(*args, layer, a1, a2, lse, x["dout"], grads=grads, workspace=ws)), \
            {"grads": grads}
    if w.kind == "v2_bwd":  # the timed call is the backward; the training forward runs once, untimed
        _, attn, lse = binding.v2_fwd_train(x["q"], x["k"], x["v"], x["lam"], softmax1=softmax1)
        grads = [torch.empty_like(x[n]) for n in ("q", "k", "v", "lam")]
        ws = torch.empty(binding.v2_bwd_workspace_bytes(w.B, w.T, w.Hq, w.Hkv, w.d), dtype=torch.uint8,
                         device=x["v"].device)
        return (lambda layer: binding.v2_bwd(x["q"], x["k"], x["v"], x["lam"], attn, lse, x["dout"], *grads,
                                             workspace=ws)), {"grads": grads}
    dev = x["q"].device
    out = torch.empty((w.B, w.Hq // 2, w.d), dtype=w.torch_dtype, device=dev)
    if w.kind == "decode_paged":
        ws = torch.empty(binding.v2_decode_paged_workspace_bytes(w.B, w.T, 1, w.Hq, w.Hkv, w.d), dtype=torch.uint8,
                         device=dev)
        return (lambda layer: binding.v2_decode_paged(x["q"], x["k_pages"], x["v_pages"], x["block_table"],
                                                      x["seq_lens"], x["lam"], w.T, out=out, workspace=ws,
                                                      softmax1=softmax1)), {"out": out}
    if w.kind == "decode_multi":
        out = torch.empty((w.B, w.nq, w.Hq // 2, w.d), dtype=w.torch_dtype, device=dev)
        ws = torch.empty(binding.v2_decode_multi_workspace_bytes(w.B, w.T, w.nq, w.Hq, w.Hkv, w.d), dtype=torch.uint8,
                         device=dev)
        return (lambda layer: binding.v2_decode_multi(x["q"], x["k"], x["v"], x["lam"], out=out, workspace=ws,
                                                      softmax1=softmax1)), {"out": out}
    ws = torch.empty(binding.v2_decode_workspace_bytes(w.B, w.T, w.Hq, w.Hkv, w.d), dtype=torch.uint8, device=dev)
    if w.kind == "decode_rope":  # q rotated in the kernel; the cache is read as holding rotated keys
        return (lambda layer: binding.v2_decode(x["q"], x["k"], x["v"], x["lam"], out=out, workspace=ws,
                                                theta=1e4)), {"out": out}
    return (lambda layer: binding.v2_decode(x["q"], x["k"], x["v"], x["lam"], out=out, workspace=ws,
                                            softmax1=softmax1)), {"out": out}


def _timed(torch, call, layers, steps, warmup, graph=True, group=1):
    """Run `warmup` untimed steps, then exactly `steps` timed steps (one step
    = one call per layer).  With `graph`, `group` consecutive steps (their
    group * len(layers) calls) are captured once as a HIP graph and replayed
    steps / group times, so host launch overhead does not gap the GPU
    (`group` must divide `steps`; otherwise 1).  Returns (elapsed_s, per-call
    ms list) where a call's time is its replay's event-timed duration / calls
    per replay (graph) or the events around that one call (eager)."""
    if not graph or group < 1 or steps % group:
        group = 1
    for l in layers:  # eager first: any lazy initialisation happens outside capture
        call(l)
    torch.cuda.synchronize()
    g = None
    if graph:
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for _ in range(group):
                for l in layers:
                    call(l)
        torch.cuda.synchronize()
    for _ in range((warmup + group - 1) // group):
        if g is not None:
            g.replay()
        else:
            for l in layers:
                call(l)
    torch.cuda.synchronize()
    per = 1 if g is not None else len(layers)
    reps = steps // group
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps * per)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    k = 0
    for _ in range(reps):
        if g is not None:
            ev[k][0].record()
            g.replay()
            ev[k][1].record()
            k += 1
        else:
            for l in layers:
                ev[k][0].record()
                call(l)
                ev[k][1].record()
                k += 1
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    ms = [a.elapsed_time(b) for a, b in ev]
    if g is not None:
        n = group * len(layers)
        ms = [m / n for m in ms for _ in range(n)]
    return elapsed, ms


def _roofline(w, launch_ms):
    avg_s = sum(launch_ms) / len(launch_ms) / 1e3
    if w.kind in ("decode", "decode_rope", "decode_paged", "decode_multi", "lam_proj"):
        a = w.compulsory_bytes() / avg_s / 1e9
        return {"bound": "hbm", "achieved": round(a, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": round(a / PEAK_HBM_GBS, 4), "traffic": None,
                "kernel_ms": round(avg_s * 1e3, 5)}
    a = w.flops() / avg_s / 1e12
    return {"bound": "mfma", "achieved": round(a, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
            "frac": round(a / PEAK_BF16_TFLOPS, 4), "traffic": None, "kernel_ms": round(avg_s * 1e3, 5)}


# ---- the oracle leg: the fp64 oracle timed on the host, and its sampled
# rows compared with what the GPU wrote (test infrastructure; never on the
# timed path, and skipped with --no-cpu-baseline).

def _host(t):
    import numpy as np

    return np.ascontiguousarray(t.detach().to("cpu").double().numpy())


def _cpu_baseline(w, x, softmax1=False, min_seconds=10.0, max_seconds=30.0, batch=2048, seed=11):
    """Time the fp64 oracle on a bounded sample of rows of the headline V2
    prefill: batches of (t, pair) rows drawn uniformly (so the mean causal row
    length is the workload's), oracle.v2_rows over each batch, until at least
    `min_seconds` of work (stopping before `max_seconds`).  The rate counts
    each sampled row's own algorithmic flops (two heads x (QK^T + PV) over
    its t+1 visible keys: 8 d (t+1))."""
    import numpy as np

    import oracle

    cores = oracle.set_threads(len(os.sched_getaffinity(0)))
    q, k, v, lam = (_host(x[n]) for n in ("q", "k", "v", "lam"))
    rng = np.random.default_rng(seed)
    rows, flops, t = 0, 0.0, 0.0
    while t < min_seconds:
        idx = np.stack([np.zeros(batch, np.int64), rng.integers(0, w.T, batch), rng.integers(0, w.Hq // 2, batch)], 1)
        t0 = time.perf_counter()
        oracle.v2_rows(q, k, v, lam, idx, softmax1=softmax1)
        dt = time.perf_counter() - t0
        t += dt
        rows += batch
        flops += float(8.0 * w.d * (idx[:, 1] + 1).sum())
        if t + dt > max_seconds:
            break
    return {"value": round(flops / t / 1e12, 6), "unit": "TFLOP/s", "cores": cores, "kind": "oracle",
            "seconds": round(t, 3),
            "sample": f"{rows} random (token, pair) rows of {w.name} (of {w.T * w.Hq // 2}), fp64 C + OpenMP; "
                      f"rate = the sampled rows' own causal flops / time"}


def _oracle_parity(w, x, outs, softmax1=False, layer=0, n=16, seed=3):
    """Sampled outputs of one timed call against the oracle: rows of the
    prefills, batch entries of the decodes, tokens of the projection, rows /
    keys of one unit of the backward passes.  Forward outputs: max |err| and
    the bf16 bar 2e-2 + 1e-2 |ref|; gradients: max |err| and the relative L2
    error (bar 1e-2)."""
    import numpy as np

    import oracle
    from oracle import backward as ob
    from oracle import prologue as op

    rng = np.random.default_rng(seed)
    decode = w.kind.startswith("decode")
    # host fp64 copies of what the sample needs (the decode caches are sliced
    # to the sampled sequences on the device first)
    H = {} if decode else {n_: _host(t) for n_, t in x.items()}
    s1 = dict(softmax1=softmax1)
    got = ref = None
    if w.kind == "v1":
        idx = np.stack([rng.integers(0, w.B, n), rng.integers(0, w.H, n), rng.integers(0, w.T, n)], 1)
        idx[:3, 2] = [0, 1, w.T - 1]
        ref = oracle.v1_rows(*[H[k] for k in ("q1", "q2", "k1", "k2", "v", "lq1", "lk1", "lq2", "lk2")], layer, idx,
                             **s1)
        got = _host(outs["out"])[idx[:, 0], idx[:, 2], idx[:, 1]]
    elif w.kind in ("v2", "v2_rope"):
        idx = np.stack([rng.integers(0, w.B, n), rng.integers(0, w.T, n), rng.integers(0, w.Hq // 2, n)], 1)
        idx[:3, 1] = [0, 1, w.T - 1]
        q, k = H["q"], H["k"]
        if w.kind == "v2_rope":
            q, k = op.rope(q, 1e4), op.rope(k, 1e4)
        ref = oracle.v2_rows(q, k, H["v"], H["lam"], idx, **(s1 if w.kind == "v2" else {}))
        got = _host(outs["out"])[idx[:, 0], idx[:, 1], idx[:, 2]]
    elif w.kind in ("decode", "decode_rope", "decode_multi"):
        bs = np.sort(rng.choice(w.B, 2, replace=False))
        sub = [_host(x[k][bs]) for k in ("q", "k", "v", "lam")]
        if w.kind == "decode":
            ref = oracle.v2_decode(*sub, **s1)
        elif w.kind == "decode_rope":
            ref = op.v2_decode_rope(*sub, theta=1e4)
        else:
            ref = oracle.v2_decode_multi(*sub, **s1)
        got = _host(outs["out"])[bs]
    elif w.kind == "decode_paged":  # the sampled sequences' own pages, renumbered
        bs = np.sort(rng.choice(w.B, 2, replace=False))
        table, lens = x["block_table"].cpu().numpy()[bs], x["seq_lens"].cpu().numpy()[bs]
        npg = [(int(L) + w.page - 1) // w.page for L in lens]
        used = np.unique(np.concatenate([table[i, :npg[i]] for i in range(len(bs))]))
        remap = {int(pg): i for i, pg in enumerate(used)}
        t2 = np.zeros((len(bs), max(npg)), np.int64)
        for i in range(len(bs)):
            t2[i, :npg[i]] = [remap[int(pg)] for pg in table[i, :npg[i]]]
        sel = __import__("torch").as_tensor(used, device=x["k_pages"].device)
        ref = oracle.v2_decode_paged(_host(x["q"][bs]), _host(x["k_pages"][sel]), _host(x["v_pages"][sel]), t2, lens,
                                     _host(x["lam"][bs]), **s1)
        got = _host(outs["out"])[bs]
    elif w.kind == "lam_proj":
        ts = rng.integers(0, w.T, n)
        ref = op.lambda_proj(H["x"][:, ts], H["w"])
        got = _host(outs["out"])[:, ts]
    if got is not None:
        err = np.abs(got - ref)
        return {"sample": f"{ref.shape[0]} x {ref[0].size}", "max_abs_err": float(err.max()),
                "ok": bool((err <= 2e-2 + 1e-2 * np.abs(ref)).all())}
    grads = [_host(g) for g in outs["grads"]]
    if w.kind == "v2_bwd":  # one GQA group: dq of sampled rows, dk/dv of sampled keys, all its dlam
        G = w.Hq // w.Hkv
        g0 = int(rng.integers(0, w.Hkv))
        hs, ps = slice(g0 * G, (g0 + 1) * G), slice(g0 * G // 2, (g0 + 1) * G // 2)
        ts, js = rng.integers(0, w.T, 4), rng.integers(0, w.T, 4)
        rows = [(0, int(t), h) for t in ts for h in range(G)]
        keys = [(0, int(j), 0) for j in js]
        rq, rk, rv, rl = ob.v2_bwd_sampled(H["q"][:, :, hs], H["k"][:, :, g0:g0 + 1], H["v"][:, :, g0:g0 + 1],
                                           H["lam"][:, :, ps], H["dout"][:, :, ps], rows, keys, **s1)
        pairs = [(np.stack([grads[0][0, t, g0 * G + h] for _, t, h in rows]), rq),
                 (np.stack([grads[1][0, j, g0] for _, j, _ in keys]), rk),
                 (np.stack([grads[2][0, j, g0] for _, j, _ in keys]), rv), (grads[3][:, :, ps], rl)]
        what = f"kv group {g0}: dq of {len(rows)} rows, dk/dv of {len(keys)} keys, dlam of its pairs"
    else:  # v1_bwd: one (batch, differential head) unit, every gradient element of it
        b, h = int(rng.integers(0, w.B)), int(rng.integers(0, w.H))
        sub = [H[k][b:b + 1, h:h + 1] for k in ("q1", "q2", "k1", "k2", "v")]
        ref = ob.v1_bwd(*sub, *[H[k] for k in ("lq1", "lk1", "lq2", "lk2")], w.layers[0],
                        H["dout"][b:b + 1, :, h:h + 1], **s1)
        pairs = [(grads[i][b:b + 1, h:h + 1], ref[i]) for i in range(5)]
        what = f"(b {b}, head {h}): dq1, dq2, dk1, dk2, dv"
    rl2 = [float(np.sqrt(((g - r) ** 2).sum() / (r * r).sum())) for g, r in pairs]
    return {"sample": what, "max_abs_err": max(float(np.abs(g - r).max()) for g, r in pairs),
            "max_rel_l2": max(rl2), "ok": bool(max(rl2) <= 1e-2)}


def _source_sha(kind):
    """sha256 of the HIP source(s) a workload's kernels are built from; a
    traffic figure taken from hardware counters only applies to the kernels it
    was measured on."""
    import hashlib

    src = {"v1": ["prefill_bf16.hip"], "v2": ["prefill_bf16.hip"],
           "v2_rope": ["prologue_bf16.hip", "rope.hpp", "prefill_bf16.hip"],
           "v1_bwd": ["backward_bf16.hip"], "v2_bwd": ["backward_bf16.hip"], "decode": ["decode_bf16.hip"],
           "decode_rope": ["rope.hpp", "decode_bf16.hip"], "lam_proj": ["prologue_bf16.hip"],
           "decode_paged": ["decode_bf16.hip"], "decode_multi": ["decode_bf16.hip"]}[kind]
    h = hashlib.sha256()
    for f in src:
        h.update(open(os.path.join(ROOT, "differential_attention_diffattn_amd", "csrc", f), "rb").read())
    return h.hexdigest()


def _traffic(w):
    """HBM bytes per launch of the workload's dominant kernel from the committed
    counter summary (FETCH_SIZE + WRITE_SIZE, each scaled by what the same
    counters read for a plain copy of known size), or None when absent or
    taken on a different kernel source."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path)).get(w.name)
    if not rec or rec.get("kernel_source_sha256") != _source_sha(w.kind):
        return None
    return rec.get("traffic_bytes_per_launch")


def _copy_calibration(torch, steps):
    """A plain device copy of known size (reads and writes 1 GiB), the reference
    for scaling the FETCH_SIZE / WRITE_SIZE counters."""
    n = 1 << 29  # bf16 elements = 1 GiB
    src = torch.empty(n, dtype=torch.bfloat16, device="cuda").normal_()
    dst = torch.empty_like(src)
    for _ in range(2):
        dst.copy_(src)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        dst.copy_(src)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    return {"workload": "copy_1GiB", "bytes_read": 2 * n, "bytes_written": 2 * n, "ms": round(ms, 4),
            "GB_per_s": round(4 * n / ms / 1e6, 1)}


V1_BWD_KERNELS = "bwd_v1_pre_kernel|bwd_v1_main_kernel"


def write_traffic(pmc_dir):
    """Turn FETCH_SIZE / WRITE_SIZE counter runs into profiles/traffic.json.

    Expects rocprofv3 CSV output in <pmc_dir>/pmc_<workload>_<COUNTER>/ for the
    'copy' calibration and each workload (bench.py --only <workload>).  Each
    counter is scaled by bytes_moved / counter_reading of the 1 GiB copy."""
    import csv
    from collections import defaultdict

    from differential_attention_diffattn_amd import workloads

    def per_dispatch(work, counter, match):
        """Counter per call: mean over dispatches of each kernel matching one of
        the `|`-separated names (`name*n`: launched n times per call), summed
        over those kernels."""
        f = os.path.join(pmc_dir, f"pmc_{work}_{counter}", "run_counter_collection.csv")
        total = 0.0
        for m in match.split("|"):
            m, _, times = m.partition("*")
            acc = defaultdict(float)
            for r in csv.DictReader(open(f)):
                if m in r["Kernel_Name"]:
                    acc[r["Dispatch_Id"]] += float(r["Counter_Value"])
            total += sum(acc.values()) / len(acc) * int(times or 1)
        return total

    copy_bytes = 1 << 30
    f_scale = copy_bytes / (1024 * per_dispatch("copy", "FETCH_SIZE", "copyBuffer"))
    w_scale = copy_bytes / (1024 * per_dispatch("copy", "WRITE_SIZE", "copyBuffer"))
    out = {"_calibration": {"copy_bytes_each_way": copy_bytes, "fetch_scale": round(f_scale, 4),
                            "write_scale": round(w_scale, 4)}}
    for name, match in [("v1_gpt2small_B8_H6_T1024_d64", "prefill_kernel"), ("v1_3b_B2_H12_T4096_d128", "prefill_kernel"),
                        ("v2_prefill_B1_T8192_Hq64_Hkv8_d128", "prefill_kernel"),
                        ("v2_backward_B1_T8192_Hq64_Hkv8_d128", "bwd_pre_kernel|bwd_dq_kernel|bwd_dkdv_kernel"),
                        ("v1_backward_B8_H6_T1024_d64", V1_BWD_KERNELS), ("v1_backward_B2_H12_T4096_d128", V1_BWD_KERNELS),
                        ("v2_decode_B64_L32768_Hq64_Hkv8_d128", "decode_split_kernel"),
                        ("v2_decode_paged_B64_Lmax32768_P64_Hq64_Hkv8_d128", "decode_split_kernel"),
                        ("v2_decode_multi_B64_L32768_nq4_Hq64_Hkv8_d128", "decode_split_kernel"),
                        ("v2_prefill_rope_B1_T8192_Hq64_Hkv8_d128", "rope_kernel|prefill_kernel"),
                        ("v2_decode_rope_B64_L32768_Hq64_Hkv8_d128", "decode_split_kernel"),
                        ("v2_lambda_proj_B1_T8192_dm4096_P32", "lambda_proj")]:
        w = workloads.WORKLOADS[name]
        fk = per_dispatch(name, "FETCH_SIZE", match)
        wk = per_dispatch(name, "WRITE_SIZE", match)
        traffic = fk * 1024 * f_scale + wk * 1024 * w_scale
        out[name] = {"kernel": match, "kernel_source_sha256": _source_sha(w.kind),
                     "fetch_kib_per_dispatch": round(fk, 1), "write_kib_per_dispatch": round(wk, 1),
                     "traffic_bytes_per_launch": int(traffic), "algorithmic_bytes_per_launch": w.compulsory_bytes(),
                     "traffic_over_algorithmic": round(traffic / w.compulsory_bytes(), 3)}
    path = os.path.join(ROOT, "profiles", "traffic.json")
    with open(path, "w") as fh:
        json.dump(out, fh, indent=1)
        fh.write("\n")
    return out


def summarize(path, match):
    """Summarise rocprofv3 CSV output under `path` for kernels whose name
    contains `match`: kernel-trace durations and/or per-dispatch counters."""
    import csv
    import glob
    from collections import defaultdict

    out = {}
    for f in sorted(glob.glob(os.path.join(path, "**", "*kernel_trace.csv"), recursive=True)):
        durs = defaultdict(list)
        for r in csv.DictReader(open(f)):
            if match in r["Kernel_Name"]:
                durs[r["Kernel_Name"]].append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
        for k, v in durs.items():
            out.setdefault("kernels", {})[k] = {"dispatches": len(v), "avg_us": round(sum(v) / len(v), 3),
                                                 "min_us": round(min(v), 3), "max_us": round(max(v), 3)}
    acc = defaultdict(lambda: defaultdict(float))
    for f in sorted(glob.glob(os.path.join(path, "**", "*counter_collection.csv"), recursive=True)):
        for r in csv.DictReader(open(f)):
            if match in r["Kernel_Name"]:
                acc[r["Counter_Name"]][(f, r["Dispatch_Id"])] += float(r["Counter_Value"])
    for k, v in acc.items():
        out.setdefault("counters_per_dispatch", {})[k] = sum(v.values()) / len(v)
    return out


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=int(os.environ.get("WORLD_SIZE", "1")))
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=300)
    ap.add_argument("--only", default=None,
                    help="time a single workload by name, or 'copy' for the 1 GiB copy calibration")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-secondary", action="store_true")
    ap.add_argument("--eager", action="store_true", help="launch every call from Python instead of replaying "
                    "a captured HIP graph of one step")
    ap.add_argument("--softmax1", action="store_true",
                    help="time the off-by-one softmax entry points (diffattn_*_softmax1) instead")
    ap.add_argument("--summarize", default=None, metavar="DIR",
                    help="summarise rocprofv3 CSV output in DIR (kernels matching --kernel) and exit")
    ap.add_argument("--kernel", default="", help="kernel-name substring for --summarize")
    ap.add_argument("--write-traffic", default=None, metavar="DIR",
                    help="turn FETCH_SIZE/WRITE_SIZE runs in DIR into profiles/traffic.json and exit")
    args = ap.parse_args()
    if args.write_traffic:
        print(json.dumps(write_traffic(args.write_traffic), indent=1))
        return
    if args.summarize:
        print(json.dumps(summarize(args.summarize, args.kernel), indent=1))
        return
    if args.gpus != 1:
        print(f"bench.py: measures one GPU only (--gpus {args.gpus} requested); the kernels shard "
              "by head/group with no exchange, so the 1-GPU figure is the per-GPU figure.", file=sys.stderr)
        sys.exit(2)

    import torch

    from differential_attention_diffattn_amd import binding, workloads

    if not binding.library_path().exists():
        import __graft_entry__

        __graft_entry__.build()
    binding.load_library()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    def measure(name, steps, warmup, calls_per_step=None, group=1):
        w = workloads.WORKLOADS[name]
        x = workloads.inputs_for(w, dev)
        call, outs = _caller(w, x, binding, torch, softmax1=args.softmax1)
        layers = list(w.layers) if w.layers else [0]
        if calls_per_step:  # repeat the layer list so one step holds several launches
            layers = (layers * calls_per_step)[:max(calls_per_step, len(layers))]
        elapsed, launch_ms = _timed(torch, call, layers, steps, warmup, graph=not args.eager, group=group)
        per_call_s = elapsed / (steps * len(layers))
        roof = _roofline(w, launch_ms)
        roof["traffic"] = _traffic(w)
        res = {"workload": name, "steps": steps, "warmup": warmup, "calls_per_step": len(layers),
               "launch": "eager" if args.eager else f"hip_graph ({group} steps per replay)" if group > 1 else "hip_graph",
               "ms_per_step": round(elapsed / steps * 1e3, 5), "roofline": roof}
        if w.kind == "decode":
            res.update(metric="V2 decode HBM GB/s", unit="GB/s",
                       value=round(w.compulsory_bytes() / per_call_s / 1e9, 1))
        elif w.kind == "decode_paged":
            res.update(metric="V2 paged ragged decode HBM GB/s (bytes of the sequences' own lengths)",
                       unit="GB/s", value=round(w.compulsory_bytes() / per_call_s / 1e9, 1))
        elif w.kind == "decode_multi":
            res.update(metric=f"V2 decode of {w.nq} new tokens per sequence, HBM GB/s", unit="GB/s",
                       value=round(w.compulsory_bytes() / per_call_s / 1e9, 1))
        elif w.kind == "v2_bwd":
            res.update(metric="causal bwd TFLOP/s (5 products over unmasked pairs)", unit="TFLOP/s",
                       value=round(w.flops() / per_call_s / 1e12, 3))
        elif w.kind == "decode_rope":
            res.update(metric="V2 decode HBM GB/s, q rotated (rotary embedding) in the kernel", unit="GB/s",
                       value=round(w.compulsory_bytes() / per_call_s / 1e9, 1))
        elif w.kind == "lam_proj":
            res.update(metric="V2 lambda projection HBM GB/s (x, w read once; logits written once)", unit="GB/s",
                       value=round(w.compulsory_bytes() / per_call_s / 1e9, 1))
        elif w.kind == "v2_rope":
            res.update(metric="causal fwd TFLOP/s with the rotary embedding (k pass + prefill)", unit="TFLOP/s",
                       value=round(w.flops() / per_call_s / 1e12, 3))
        elif w.kind == "v1_bwd":
            res.update(metric="causal bwd TFLOP/s (5 products per map over unmasked pairs)", unit="TFLOP/s",
                       value=round(w.flops() / per_call_s / 1e12, 3))
        else:
            res.update(metric="causal fwd TFLOP/s", unit="TFLOP/s", value=round(w.flops() / per_call_s / 1e12, 3))
        if not args.no_cpu_baseline:  # the oracle leg: sampled outputs of the last timed call
            torch.cuda.synchronize()
            res["parity"] = _oracle_parity(w, x, outs, softmax1=args.softmax1, layer=layers[-1])
        log(json.dumps(res))
        return w, x, res

    if args.only == "copy":
        print(json.dumps(_copy_calibration(torch, args.steps)))
        return
    if args.only:  # at least 8 launches per step, as in the default run
        _, _, res = measure(args.only, args.steps, args.warmup, calls_per_step=8)
        print(json.dumps(res))
        return

    # headline: one step = one call; up to 10 consecutive steps share one graph
    # replay (the gap between replays is host launch time, not the kernel's)
    group = max(g for g in range(1, 11) if args.steps % g == 0)
    w, x, head = measure(HEADLINE, args.steps, args.warmup, group=group)
    secondary = []
    if not args.no_secondary:
        for name in SECONDARY:
            # warm-up sized to ~0.3 s of this workload's own calls, so the
            # GPU clock has settled under its load before the timed steps
            ws = workloads.WORKLOADS[name]
            est_s = (ws.flops() / 1e15 if ws.kind in ("v1", "v2", "v2_rope", "v1_bwd", "v2_bwd")
                     else ws.compulsory_bytes() / 5.5e12)
            # 8 launches per step: the events around a graph replay then time
            # the kernels, not the replay's launch
            _, xs, r = measure(name, max(10, args.steps), max(3, int(0.3 / (8 * est_s))), calls_per_step=8)
            secondary.append(r)
            del xs
            torch.cuda.empty_cache()
    # context for the MFMA roofline: the vendor GEMM (torch.matmul, hipBLASLt)
    # on a large square bf16 product on the same card and clock
    ref = None
    if not args.no_secondary:
        import torch
        n = 8192
        g = torch.Generator(device="cuda").manual_seed(7)
        a_ = torch.randn((n, n), generator=g, device="cuda").to(torch.bfloat16)
        b_ = torch.randn((n, n), generator=g, device="cuda").to(torch.bfloat16)
        for _ in range(10):
            c_ = torch.matmul(a_, b_)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(20):
            c_ = torch.matmul(a_, b_)
        e1.record()
        torch.cuda.synchronize()
        tf = 2.0 * n ** 3 / (e0.elapsed_time(e1) / 20 * 1e-3) / 1e12
        ref = {"kind": f"torch.matmul bf16 [{n}x{n}] x [{n}x{n}] (vendor GEMM library)",
               "tflops": round(tf, 1), "frac_of_peak": round(tf / 2500.0, 4)}
        del a_, b_, c_
        torch.cuda.empty_cache()
        log(json.dumps({"mfma_reference": ref}))
    cpu = None
    if not args.no_cpu_baseline:
        cpu = _cpu_baseline(w, x, softmax1=args.softmax1)
        log(json.dumps({"cpu_baseline": cpu}))

    line = {
        "metric": METRIC,
        "value": head["value"],
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": head["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic: seeded N(0,1) q/k/v, lambda logits N(0,1) fp32; resident in HBM",
        "config": {"workload": HEADLINE, "kind": "DIFF V2 causal GQA prefill", "B": w.B, "T": w.T, "Hq": w.Hq,
                   "Hkv": w.Hkv, "pairs": w.Hq // 2, "d": w.d, "step": "one call", "launch": head["launch"], "parallelism": "none",
                   "softmax": "off_by_one" if args.softmax1 else "standard"},
        "roofline": head["roofline"],
        "cpu_baseline": cpu,
        "parity": head.get("parity"),
        "mfma_reference": ref,
        "secondary": secondary,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
