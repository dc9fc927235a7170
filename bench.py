#!/usr/bin/env python3
"""Benchmark of the DFlash 2 path selector on one MI355X.

One step = one dflash2_select call over one batch (two launches: the scan
with the row merges, then the pair scores and walks): top-K of every logits
row, the gate projection, all pair scores and the walk.  Inputs are seeded
synthetic data resident in HBM; several copies of the per-cycle inputs
(logits, hidden) are rotated so that the 256 MB Infinity Cache cannot serve
them from the previous step.

Prints ONE JSON line:
  value       drafted positions/s (B*P per step) on the concurrency-32 workload
              (B=32, P=7, V=151936, d=5120, K=16, bf16), wall clock over the
              timed steps;
  us_per_cycle / b1   the same for the batch-1 Qwen3-4B-shaped workload
              (B=1, P=7, V=151936, d=2560, K=16, bf16), as microseconds per
              draft-verify cycle;
  roofline    algorithmic bytes per launch / average launch time (HIP events on
              the launch stream) against the 8 TB/s HBM peak;
  greedy      the same workloads with the greedy walk in place of the max-sum
              walk, and how often the two walks' paths differ (on the timed
              workload and on its pair-dominant variant);
  sample      the same workloads with the sampling walk (temperature 1,
              seeded uniforms resident on the device); beside it the device
              generator of those uniforms (dflash2_philox_uniforms) alone, at
              B*P uniforms per call and in bulk, and the cycle with both (the
              uniforms drawn on the device, then the sampling select);
  conv        the drafter's two-tap dynamic convolution (dflash2_conv2) at
              the two drafter shapes: µs per call (HIP events) and % of HBM
              peak for its algorithmic bytes, input copies rotated;
  c2, stress  the batch-8 workload (B=8, P=7, V=151936, d=5120) and the
              stress workload (B=256, P=15, V=262144, d=5120, K=32): µs per
              call and % of HBM peak;
  b1.graph    the batch-1 select over every rotated input set captured in one
              HIP graph and replayed (µs per call), replays checked against
              the eager outputs;
  project     the gate projection alone at the timed workload's shape: µs per
              call and TFLOP/s against the bf16 matrix-core peak;
  lmhead      the drafter's LM head fused with top-K (dflash2_lmhead_topk) at
              the concurrency-32 and batch-1 shapes: µs per call (HIP events,
              both launches), its roofline on the bytes it must read (the
              V x d bf16 weight once, plus hidden states and outputs) and
              TFLOP/s against the bf16 matrix-core peak, with the CPU oracle
              on a few sampled rows;
  cpu_baseline  the CPU oracle on a bounded sample of the same workload, one
              thread per usable host core (at most 16), and single-threaded.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "path-select µs/cycle at B=1, drafted positions/s at B=32; % HBM peak"
HBM_PEAK_GBS = 8000.0
MFMA_BF16_PEAK_TFLOPS = 2500.0
PROFILES = os.path.join(ROOT, "profiles")
KERNEL_SOURCES = ("common.hpp", "topk.hpp", "gate.hpp", "pairs.hpp", "walk.hpp", "dflash2.hip")
LMHEAD_SOURCES = ("common.hpp", "lmhead.hpp")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def algorithmic_bytes(wl) -> int:
    """Bytes the method must move once per cycle: every logit, every hidden
    value, W_H, the gathered A/B embedding rows ((2P-1)K+1 per sequence: K
    candidate rows B(.) at each of P positions, K predecessor rows A(.) at
    P-1 positions plus prev_tok's row), and the outputs."""
    esz = 2 if wl.dtype == "bf16" else 4
    logits = wl.B * wl.P * wl.V * esz
    hidden = wl.B * wl.P * wl.d * esz
    w = wl.r * wl.d * esz
    rows = wl.B * ((2 * wl.P - 1) * wl.K + 1) * wl.r * esz
    out = wl.B * wl.P * 4 + wl.B * 4
    return logits + hidden + w + rows + out


def _code_only(text: str) -> str:
    """C++ source without its comments and with whitespace runs collapsed
    (string literals kept as they are)."""
    out, i, n = [], 0, len(text)
    while i < n:
        c = text[i]
        if c == '"':
            j = i + 1
            while j < n and text[j] != '"':
                j += 2 if text[j] == "\\" else 1
            out.append(text[i:j + 1])
            i = j + 1
        elif text.startswith("//", i):
            j = text.find("\n", i)
            i = n if j < 0 else j
        elif text.startswith("/*", i):
            j = text.find("*/", i + 2)
            i = n if j < 0 else j + 2
            out.append(" ")
        else:
            out.append(c)
            i += 1
    return " ".join("".join(out).split())


def kernel_source_hash(family: str = "select") -> str:
    """Hash of the device code a family of kernels is built from (for the
    selector, dflash2.hip up to its host-side part; comments and layout
    ignored), so that counter runs are only reused while that code is
    unchanged."""
    files = {"select": KERNEL_SOURCES, "lmhead": LMHEAD_SOURCES}[family]
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(ROOT, "draft_selection_topk16_amd", "csrc", f), encoding="utf-8") as fh:
            data = fh.read()
        if f == "dflash2.hip":
            data = data.split("// Host side.")[0]
        h.update(_code_only(data).encode())
    return h.hexdigest()[:16]


def traffic_for(workload: str, family: str = "select"):
    """HBM bytes per launch from the committed rocprofv3 counter runs, if they
    were taken on the current kernel sources; else None.  LM-head entries are
    keyed "lmhead/<workload>"."""
    path = os.path.join(PROFILES, "traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        t = json.load(f)
    entry = t.get(workload if family == "select" else "lmhead/" + workload)
    if not entry or entry.get("kernel_source_sha") != kernel_source_hash(family):
        return None
    return entry.get("hbm_bytes_per_launch")


def time_workload(wl, steps: int, warmup: int, rotate_mb: float, walks=("viterbi",), graph=False):
    """Times dflash2_select_walk on `wl` for each walk in `walks` (same inputs);
    returns (inputs, {walk: timings}, {walk: path of the first input set}).
    With graph=True the Viterbi select over every rotated input set is also
    captured once into a HIP graph (on a stream warmed first, so that no
    allocation or memset is captured) and replayed; each replay's outputs are
    checked against the eager results."""
    import torch
    import draft_selection_topk16_amd as df2
    from draft_selection_topk16_amd import synth
    import numpy as np

    t0 = time.perf_counter()
    x = synth.make_inputs(wl)
    log("  inputs for %s drawn in %.1f s" % (wl.name, time.perf_counter() - t0))

    def dev(a, dt):
        a = np.ascontiguousarray(a)
        if dt == "bf16":
            return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()
        return torch.from_numpy(a).cuda()

    dt = wl.dtype
    logits, hidden = dev(x.logits, dt), dev(x.hidden, dt)
    A, Bt, W = dev(x.A, dt), dev(x.Bt, dt), dev(x.W, dt)
    prev = torch.from_numpy(x.prev).cuda()
    per_set = logits.nbytes + hidden.nbytes
    nsets = max(1, int(math.ceil(rotate_mb * 1e6 / per_set)))
    sets = [(logits, hidden)] + [(logits.clone(), hidden.clone()) for _ in range(nsets - 1)]
    stream = torch.cuda.current_stream()
    results, paths = {}, {}
    g = torch.Generator().manual_seed(0xDF2)
    u = torch.rand((wl.B, wl.P), generator=g, dtype=torch.float32).cuda()
    off = torch.zeros((1,), dtype=torch.int64, device="cuda")
    for walk in walks:
        calls = [df2.PreparedSelect(l, h, A, Bt, W, prev, wl.K,
                                    walk="sample" if walk == "sample_dev" else walk, u=u,
                                    temperature=1.0)
                 for (l, h) in sets]
        if walk == "sample_dev":
            calls = [_DrawThenSelect(c, u, off, stream) for c in calls]
        torch.cuda.synchronize()
        results[walk] = _time_calls(calls, nsets, steps, warmup, stream)
        results[walk].update(rotation_sets=nsets, rotation_mb=nsets * per_set / 1e6)
        calls[0]()
        torch.cuda.synchronize()
        paths[walk] = calls[0].out_path.cpu().numpy().copy()
        del calls
    if graph:
        results["graph"] = _time_graph(sets, A, Bt, W, prev, wl, steps)
    del sets
    torch.cuda.empty_cache()
    return x, results, paths


class _DrawThenSelect:
    """One serving-loop cycle of the sampling walk: the cycle's uniforms drawn
    on the device (dflash2_philox_uniforms_next, offset in device memory),
    then the prepared sampling select that reads them.  The generator's
    arguments are marshalled once."""

    def __init__(self, call, u, off, stream):
        import draft_selection_topk16_amd as df2
        self.call = call
        self.out_path = call.out_path
        self._fn = df2.load().dflash2_philox_uniforms_next
        self._args = (0xD1F1A5, off.data_ptr(), u.numel(), u.data_ptr(), stream.cuda_stream)

    def __call__(self):
        st = self._fn(*self._args)
        if st != 0:
            raise RuntimeError("dflash2_philox_uniforms_next failed: %d" % st)
        self.call()


def _time_graph(sets, A, Bt, W, prev, wl, steps: int):
    """One HIP graph holding a select call per rotated input set, replayed;
    per-call time = replay wall time / calls.  Every replay is checked
    against the eager outputs of the same calls."""
    import torch
    import draft_selection_topk16_amd as df2
    gs = torch.cuda.Stream()
    with torch.cuda.stream(gs):
        calls = [df2.PreparedSelect(l, h, A, Bt, W, prev, wl.K) for (l, h) in sets]
        for c in calls:
            c()
    gs.synchronize()
    eager = [(c.out_path.clone(), c.out_score.clone()) for c in calls]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=gs):
        for c in calls:
            c()
    reps = max(2, steps // len(calls))
    ok = True
    for _ in range(2):
        for c in calls:
            c.out_path.zero_()
        g.replay()
        torch.cuda.synchronize()
        ok &= all(torch.equal(c.out_path, e[0]) and torch.equal(c.out_score, e[1]) for c, e in zip(calls, eager))
    t0 = time.perf_counter()
    for _ in range(reps):
        g.replay()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ok &= all(torch.equal(c.out_path, e[0]) and torch.equal(c.out_score, e[1]) for c, e in zip(calls, eager))
    del g, calls
    return {"us_per_cycle": wall * 1e6 / (reps * len(sets)), "calls_per_graph": len(sets), "replays": reps,
            "replays_equal_eager": bool(ok)}


def _time_calls(calls, nsets: int, steps: int, warmup: int, stream):
    import torch
    for i in range(warmup):
        calls[i % nsets]()
    torch.cuda.synchronize()
    # whole-job throughput: the K timed launches back to back, nothing else
    # on the stream, synchronised on both sides
    t0 = time.perf_counter()
    for i in range(steps):
        calls[(warmup + i) % nsets]()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    # per-launch duration for the roofline: the same launches again, each
    # between two HIP events on the launch stream
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(steps)]
    for i in range(steps):
        ev[i][0].record(stream)
        calls[(warmup + i) % nsets]()
        ev[i][1].record(stream)
    torch.cuda.synchronize()
    ks = sorted(a.elapsed_time(b) for a, b in ev)      # ms per launch
    res = dict(ms_per_step=wall * 1e3 / steps,
               kernel_ms_avg=statistics.fmean(ks),
               kernel_ms_p10=ks[len(ks) // 10], kernel_ms_p50=ks[len(ks) // 2],
               kernel_ms_p90=ks[(9 * len(ks)) // 10])
    # warm (same buffers every step) for reference only
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        calls[0]()
    torch.cuda.synchronize()
    res["warm_ms_per_step"] = (time.perf_counter() - t0) * 1e3 / steps
    return res


def conv_bytes(B: int, P: int, d: int, esz: int) -> int:
    """x, x_prev, base and W_c read once, y written once."""
    return esz * (B * P * d + B * d + 2 * d + 2 * (d // 16) * d + B * P * d)


def time_conv(name: str, steps: int, warmup: int, rotate_mb: float):
    import torch
    import numpy as np
    import draft_selection_topk16_amd as df2
    from draft_selection_topk16_amd import synth
    shp = synth.CONV_WORKLOADS[name]
    B, P, d = shp["B"], shp["P"], shp["d"]
    c = synth.make_conv_inputs(B, P, d, "bf16")

    def dev(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()

    one = (dev(c.x), dev(c.x_prev), dev(c.base), dev(c.W_c))
    per = sum(t.nbytes for t in one) + one[0].nbytes
    nsets = max(1, int(math.ceil(rotate_mb * 1e6 / per)))
    sets = [one] + [tuple(t.clone() for t in one) for _ in range(nsets - 1)]
    outs = [torch.empty_like(s[0]) for s in sets]
    for i in range(warmup):
        k = i % nsets
        df2.conv2(*sets[k], out=outs[k])
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(steps)]
    for i in range(steps):
        k = (warmup + i) % nsets
        ev[i][0].record(stream)
        df2.conv2(*sets[k], out=outs[k])
        ev[i][1].record(stream)
    torch.cuda.synchronize()
    us = statistics.fmean(a.elapsed_time(b) for a, b in ev) * 1e3
    ab = conv_bytes(B, P, d, 2)
    del sets, outs
    torch.cuda.empty_cache()
    return {"workload": "%s: B=%d P=%d d=%d bf16" % (name, B, P, d), "us_per_call": us,
            "algorithmic_bytes": ab, "hbm_frac": ab / (us * 1e-6) / 1e9 / HBM_PEAK_GBS,
            "rotation_sets": nsets}


def _differ(paths):
    """Sequences whose greedy path differs from the Viterbi path."""
    import numpy as np
    g, v = paths["greedy"], paths["viterbi"]
    n = int(np.sum(np.any(g != v, axis=1)))
    pos = int(np.sum(g != v))
    return {"sequences": n, "of_sequences": int(g.shape[0]), "positions": pos,
            "of_positions": int(g.size)}


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(x, seconds: float):
    """The oracle, as it stands, on whole sequences of the workload until
    `seconds` of wall time: first one thread, then one thread per usable host
    core (at most 16), each taking whole sequences (the oracle's C calls
    release the GIL).  `value` is the all-cores rate."""
    import threading
    import oracle
    f = x.f64()
    B, P = x.wl.B, x.wl.P
    oracle.select(f["logits"][:1], f["hidden"][:1], f["A"], f["Bt"], f["W"], f["prev"][:1], x.wl.K)

    def run(nthreads, budget):
        counts = [0] * nthreads
        t0 = time.perf_counter()

        def work(i):
            b = i
            while time.perf_counter() - t0 < budget:
                oracle.select(f["logits"], f["hidden"], f["A"], f["Bt"], f["W"], f["prev"], x.wl.K,
                              seqs=[b % B])
                counts[i] += 1
                b += nthreads
        ts = [threading.Thread(target=work, args=(i,)) for i in range(nthreads)]
        for t in ts:
            t.start()
        for t in ts:
            t.join()
        el = time.perf_counter() - t0
        return sum(counts), el

    threads = max(1, min(16, len(os.sched_getaffinity(0))))
    n1, e1 = run(1, seconds / 3)
    nt, et = run(threads, 2 * seconds / 3)
    return {"value": nt * P / et, "unit": "positions/s", "cores": threads, "kind": "oracle",
            "cpu_model": cpu_model(), "usable_cores": len(os.sched_getaffinity(0)),
            "single_thread": {"value": n1 * P / e1, "unit": "positions/s", "cores": 1,
                              "sample": "%d whole sequences, %.1f s" % (n1, e1)},
            "sample": "%d whole sequences (P=%d, V=%d) of the same workload on %d threads, %.1f s"
                      % (nt, P, x.wl.V, threads, et)}


def time_project(wl, steps: int, warmup: int, rotate_mb: float):
    """dflash2_project (the gate projection H = W_H h) alone at the workload's
    shape, input copies rotated beyond the Infinity Cache; HIP events per
    call.  Reports TFLOP/s against the bf16 matrix-core peak."""
    import torch
    import numpy as np
    import draft_selection_topk16_amd as df2
    from draft_selection_topk16_amd import synth
    x = synth.make_inputs(wl)

    def dev(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()

    one = (dev(x.hidden), dev(x.W))
    per = sum(t.nbytes for t in one)
    nsets = max(1, int(math.ceil(rotate_mb * 1e6 / per)))
    sets = [one] + [tuple(t.clone() for t in one) for _ in range(nsets - 1)]
    for i in range(warmup):
        df2.project(*sets[i % nsets])
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    for i in range(steps):
        ev[i][0].record(stream)
        df2.project(*sets[(warmup + i) % nsets])
        ev[i][1].record(stream)
    torch.cuda.synchronize()
    us = statistics.fmean(a.elapsed_time(b) for a, b in ev) * 1e3
    M = wl.B * wl.P
    flops = 2.0 * M * wl.d * wl.r
    ab = 2 * (M * wl.d + wl.r * wl.d) + 4 * M * wl.r
    del sets
    torch.cuda.empty_cache()
    return {"workload": "%s gate projection: M=%d d=%d r=%d bf16, fp32 accumulation" % (wl.name, M, wl.d, wl.r),
            "us_per_call": us, "flops": flops, "tflops": flops / (us * 1e-6) / 1e12,
            "mfma_peak_tflops": MFMA_BF16_PEAK_TFLOPS,
            "mfma_frac": flops / (us * 1e-6) / 1e12 / MFMA_BF16_PEAK_TFLOPS,
            "algorithmic_bytes": ab, "hbm_frac": ab / (us * 1e-6) / 1e9 / HBM_PEAK_GBS}


def time_philox(n: int, steps: int, warmup: int):
    """dflash2_philox_uniforms alone: n uniforms per call, the offset advanced
    every call as a serving loop does; HIP events around each call on the
    launch stream.  Reports µs per call and the GB/s of uniforms written."""
    import torch
    import draft_selection_topk16_amd as df2
    out = torch.empty((n,), dtype=torch.float32, device="cuda")
    for i in range(warmup):
        df2.philox_uniforms(0xD1F1A5, i, n, out=out)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    for i in range(steps):
        ev[i][0].record(stream)
        df2.philox_uniforms(0xD1F1A5, warmup + i, n, out=out)
        ev[i][1].record(stream)
    torch.cuda.synchronize()
    us = statistics.fmean(a.elapsed_time(b) for a, b in ev) * 1e3
    return {"n": n, "us_per_call": us, "write_gb_per_s": 4.0 * n / (us * 1e-6) / 1e9}


def lmhead_algorithmic_bytes(M: int, V: int, d: int, K: int) -> int:
    """Bytes the fused LM head must move: the weight once, the hidden states,
    and the candidate outputs (index and value)."""
    return 2 * V * d + 2 * M * d + 8 * M * K


def time_lmhead(name: str, steps: int, warmup: int, cpu_rows: int = 2):
    """dflash2_lmhead_topk on the LM-head inputs of workload `name` (hidden
    states [B*P, d] and W_lm [V, d], bf16); HIP events around each call on
    the launch stream.  The weight (>= 0.78 GB) is far beyond the Infinity
    Cache, so it streams from HBM on every call without rotation."""
    import torch
    import numpy as np
    import oracle
    import draft_selection_topk16_amd as df2
    from draft_selection_topk16_amd import synth
    wl = synth.WORKLOADS[name]
    if wl.dtype != "bf16":
        wl = wl.with_(dtype="bf16")
    li = synth.make_lmhead_inputs(wl)

    def dev(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()

    X, W = dev(li.X), dev(li.W_lm)
    M, V, d, K = wl.rows, wl.V, wl.d, wl.K
    for _ in range(warmup):
        df2.lmhead_topk(X, W, K)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    for i in range(steps):
        ev[i][0].record(stream)
        df2.lmhead_topk(X, W, K)
        ev[i][1].record(stream)
    torch.cuda.synchronize()
    times = [a.elapsed_time(b) * 1e3 for a, b in ev]
    us = statistics.fmean(times)
    ab = lmhead_algorithmic_bytes(M, V, d, K)
    flops = 2.0 * M * V * d
    achieved = ab / (us * 1e-6) / 1e9
    # the oracle on a few rows (float64 dot products and a full sort per row)
    X32, W32 = li.f32()
    rows = np.arange(min(cpu_rows, M))
    t0 = time.time()
    oracle.lmhead_topk(X32, W32, K, rows=rows)
    et = time.time() - t0
    del X, W
    torch.cuda.empty_cache()
    return {"workload": "%s LM head + top-%d: M=B*P=%d V=%d d=%d bf16, fp32 accumulation"
                        % (name, K, M, V, d),
            "us_per_call": us, "us_min": min(times), "positions_per_s": M / (us * 1e-6),
            "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": achieved / HBM_PEAK_GBS, "traffic": traffic_for(name, "lmhead"),
                         "kernel": "k_lmhead + k_lmhead_merge (one dflash2_lmhead_topk call)",
                         "algorithmic_bytes_per_launch": ab},
            "tflops": flops / (us * 1e-6) / 1e12, "mfma_peak_tflops": MFMA_BF16_PEAK_TFLOPS,
            "mfma_frac": flops / (us * 1e-6) / 1e12 / MFMA_BF16_PEAK_TFLOPS,
            "cpu_oracle": {"value": len(rows) / et, "unit": "rows/s", "cores": 1, "kind": "oracle",
                           "sample": "%d rows of the same workload, %.1f s" % (len(rows), et)}}


def copy_calibration(mb: float, reps: int):
    """A plain device-to-device copy of known size, for scaling counters."""
    import torch
    n = int(mb * 1e6) // 4
    a = torch.ones(n, dtype=torch.float32, device="cuda")
    b = torch.empty_like(a)
    for _ in range(reps):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_read": a.nbytes, "copy_bytes_written": b.nbytes, "reps": reps}))


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=1000)
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--workload", default="t27b_b32")
    ap.add_argument("--b1-workload", default="qwen3_4b_b1")
    ap.add_argument("--rotate-mb", type=float, default=600.0)
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-b1", action="store_true")
    ap.add_argument("--no-greedy", action="store_true")
    ap.add_argument("--no-conv", action="store_true")
    ap.add_argument("--no-extra", action="store_true", help="skip the batch-8 and stress lines")
    ap.add_argument("--no-project", action="store_true")
    ap.add_argument("--no-lmhead", action="store_true")
    ap.add_argument("--lmhead-steps", type=int, default=20)
    ap.add_argument("--only", choices=["project", "lmhead", "philox"], default=None,
                    help="time one stage alone (for counter runs) and print its JSON object")
    ap.add_argument("--copy-calibration-mb", type=float, default=0.0)
    args = ap.parse_args()

    if args.gpus != 1:
        print("bench.py measures one GPU only: the selector runs per sequence with no "
              "cross-GPU exchange, and the library has no multi-GPU path (--gpus %d refused)"
              % args.gpus, file=sys.stderr)
        sys.exit(2)

    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    torch.cuda.set_device(0)
    if args.copy_calibration_mb > 0:
        copy_calibration(args.copy_calibration_mb, args.steps)
        return

    from draft_selection_topk16_amd import synth
    import draft_selection_topk16_amd as df2
    df2.load()

    wl = synth.WORKLOADS[args.workload]
    if args.only == "project":
        print(json.dumps(time_project(wl, args.steps, args.warmup, args.rotate_mb)), flush=True)
        return
    if args.only == "philox":
        print(json.dumps(time_philox(wl.B * wl.P, args.steps, args.warmup)), flush=True)
        return
    if args.only == "lmhead":
        print(json.dumps(time_lmhead(wl.name, args.steps, args.warmup, cpu_rows=1)), flush=True)
        return
    log("timing %s: %d warmup + %d steps" % (wl.name, args.warmup, args.steps))
    walks = ("viterbi",) if args.no_greedy else ("viterbi", "greedy", "sample", "sample_dev")
    x, allres, paths = time_workload(wl, args.steps, args.warmup, args.rotate_mb, walks)
    res = allres["viterbi"]
    pos_per_s = wl.B * wl.P / (res["ms_per_step"] * 1e-3)
    abytes = algorithmic_bytes(wl)
    achieved = abytes / (res["kernel_ms_avg"] * 1e-3) / 1e9
    log("  %.2f us/step wall, %.2f us/launch (events), %.0f GB/s algorithmic"
        % (res["ms_per_step"] * 1e3, res["kernel_ms_avg"] * 1e3, achieved))

    out = {
        "metric": METRIC,
        "value": pos_per_s,
        "unit": "positions/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": res["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "%s: B=%d P=%d V=%d d=%d K=%d r=%d %s logits/hidden/tables, "
                               "fp32 accumulation" % (wl.name, wl.B, wl.P, wl.V, wl.d, wl.K, wl.r, wl.dtype),
                   "B": wl.B, "P": wl.P, "V": wl.V, "d": wl.d, "K": wl.K, "r": wl.r,
                   "parallelism": "single-gpu"},
        "us_per_cycle": res["ms_per_step"] * 1e3,
        "hbm_frac": achieved / HBM_PEAK_GBS,
        "timing": res,
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": traffic_for(wl.name),
                     "kernel": "k_scanm + k_pairs_walk (one dflash2_select call: the scan with the row merges, then pairs and walks)",
                     "algorithmic_bytes_per_launch": abytes},
    }
    if not args.no_greedy:
        g = allres["greedy"]
        out["greedy"] = {"walk": "greedy (best successor of the token just chosen)",
                         "workload": wl.name,
                         "us_per_cycle": g["ms_per_step"] * 1e3,
                         "kernel_us_avg": g["kernel_ms_avg"] * 1e3,
                         "positions_per_s": wl.B * wl.P / (g["ms_per_step"] * 1e-3),
                         "paths_differ_from_viterbi": _differ(paths),
                         "timing": g}
        sm = allres["sample"]
        out["sample"] = {"walk": "sampling (softmax of the step's scores, temperature 1)",
                         "workload": wl.name,
                         "us_per_cycle": sm["ms_per_step"] * 1e3,
                         "kernel_us_avg": sm["kernel_ms_avg"] * 1e3,
                         "positions_per_s": wl.B * wl.P / (sm["ms_per_step"] * 1e-3),
                         "timing": sm}
        sd = allres["sample_dev"]
        out["sample"]["with_device_uniforms"] = {
            "cycle": "dflash2_philox_uniforms_next, then the sampling select, per step",
            "us_per_cycle": sd["ms_per_step"] * 1e3,
            "kernel_us_avg": sd["kernel_ms_avg"] * 1e3,
            "positions_per_s": wl.B * wl.P / (sd["ms_per_step"] * 1e-3)}
        log("timing the device uniforms (Philox4x64-10)")
        out["sample"]["philox_uniforms"] = {
            "generator": "Philox4x64-10, one block per four uniforms (dflash2_philox_uniforms)",
            "per_cycle": time_philox(wl.B * wl.P, 200, 20),
            "bulk": time_philox(1 << 26, 20, 3)}
    r1 = None
    if not args.no_b1:
        wl1 = synth.WORKLOADS[args.b1_workload]
        log("timing %s" % wl1.name)
        _, allr1, _ = time_workload(wl1, args.steps, args.warmup, args.rotate_mb, walks, graph=True)
        r1 = allr1["viterbi"]
        ab1 = algorithmic_bytes(wl1)
        out["b1"] = {"workload": "%s: B=%d P=%d V=%d d=%d K=%d" % (wl1.name, wl1.B, wl1.P, wl1.V, wl1.d, wl1.K),
                     "us_per_cycle": r1["ms_per_step"] * 1e3,
                     "kernel_us_avg": r1["kernel_ms_avg"] * 1e3,
                     "positions_per_s": wl1.B * wl1.P / (r1["ms_per_step"] * 1e-3),
                     "hbm_frac": ab1 / (r1["kernel_ms_avg"] * 1e-3) / 1e9 / HBM_PEAK_GBS,
                     "timing": r1,
                     "graph": allr1["graph"]}
        if not args.no_greedy:
            g1 = allr1["greedy"]
            out["greedy"]["b1"] = {"workload": wl1.name,
                                   "us_per_cycle": g1["ms_per_step"] * 1e3,
                                   "kernel_us_avg": g1["kernel_ms_avg"] * 1e3}
            s1 = allr1["sample"]
            out["sample"]["b1"] = {"workload": wl1.name,
                                   "us_per_cycle": s1["ms_per_step"] * 1e3,
                                   "kernel_us_avg": s1["kernel_ms_avg"] * 1e3,
                                   "with_device_uniforms_us_per_cycle":
                                       allr1["sample_dev"]["ms_per_step"] * 1e3}
    if not args.no_greedy:
        wlp = wl.with_(pair_scale=8.0)
        log("greedy vs Viterbi on the pair-dominant variant of %s" % wl.name)
        _, _, pp = time_workload(wlp, 3, 1, 0.0, ("viterbi", "greedy"))
        out["greedy"]["pair_dominant"] = {"workload": "%s with A and B scaled by 8" % wl.name,
                                          "paths_differ_from_viterbi": _differ(pp)}
    if not args.no_extra:
        for key, name, steps in (("c2", "t27b_b8", args.steps), ("stress", "stress_b256", max(20, args.steps // 10))):
            wlx = synth.WORKLOADS[name]
            log("timing %s" % name)
            _, rx, _ = time_workload(wlx, steps, max(5, args.warmup // 10), args.rotate_mb, ("viterbi",))
            r = rx["viterbi"]
            abx = algorithmic_bytes(wlx)
            out[key] = {"workload": "%s: B=%d P=%d V=%d d=%d K=%d r=%d %s" % (
                            name, wlx.B, wlx.P, wlx.V, wlx.d, wlx.K, wlx.r, wlx.dtype),
                        "us_per_cycle": r["ms_per_step"] * 1e3, "kernel_us_avg": r["kernel_ms_avg"] * 1e3,
                        "positions_per_s": wlx.B * wlx.P / (r["ms_per_step"] * 1e-3),
                        "algorithmic_bytes": abx,
                        "hbm_frac": abx / (r["kernel_ms_avg"] * 1e-3) / 1e9 / HBM_PEAK_GBS,
                        "timing": r}
    if not args.no_project:
        log("timing the gate projection alone at %s" % wl.name)
        out["project"] = time_project(wl, args.steps, args.warmup, args.rotate_mb)
    if not args.no_lmhead:
        out["lmhead"] = {}
        for key, name in (("b32", args.workload), ("b1", args.b1_workload)):
            log("timing the LM head fused with top-K at %s" % name)
            out["lmhead"][key] = time_lmhead(name, args.lmhead_steps, 3)
    if not args.no_conv:
        out["conv"] = {}
        for name in synth.CONV_WORKLOADS:
            log("timing %s" % name)
            out["conv"][name] = time_conv(name, args.steps, args.warmup, args.rotate_mb)
    if not args.no_cpu_baseline:
        log("timing the CPU oracle for %.0f s" % args.cpu_seconds)
        out["cpu_baseline"] = cpu_baseline(x, args.cpu_seconds)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
