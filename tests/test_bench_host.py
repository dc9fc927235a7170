"""Host-side logic of bench.py (CPU only): the byte counts the roofline is
priced on, the guard that keeps committed counter runs from being reported
for changed kernels, and the refusal of more than one GPU."""
import json
import os
import subprocess
import sys

import numpy as np

import bench
from draft_selection_topk16_amd import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_algorithmic_bytes_match_the_arrays_a_cycle_reads():
    # logits, hidden and W_H are read once: their byte sizes come from the
    # generated arrays; the gathers are one A or B row per (position,
    # candidate) pair plus prev_tok's row, counted here by enumeration
    for wl in (synth.WORKLOADS["tiny_f32"], synth.WORKLOADS["tiny_f32"].with_(dtype="bf16", B=3, V=4099)):
        x = synth.make_inputs(wl)
        esz = x.logits.dtype.itemsize
        gathers = set()
        for b in range(wl.B):
            gathers.add((b, "A", -1, 0))                     # prev_tok's row
            for t in range(wl.P):
                for k in range(wl.K):
                    gathers.add((b, "B", t, k))              # candidate rows
                    if t + 1 < wl.P:
                        gathers.add((b, "A", t, k))          # predecessor rows
        outputs = wl.B * wl.P * 4 + wl.B * 4                 # path ids, scores
        expect = x.logits.nbytes + x.hidden.nbytes + x.W.nbytes + len(gathers) * wl.r * esz + outputs
        assert bench.algorithmic_bytes(wl) == expect


def test_lmhead_bytes_match_the_arrays_it_reads():
    wl = synth.WORKLOADS["tiny_f32"].with_(dtype="bf16", V=5000, d=256)
    li = synth.make_lmhead_inputs(wl)
    expect = li.W_lm.nbytes + li.X.nbytes + wl.rows * wl.K * (4 + 4)
    assert bench.lmhead_algorithmic_bytes(wl.rows, wl.V, wl.d, wl.K) == expect


def test_traffic_is_reported_only_for_unchanged_kernels(tmp_path, monkeypatch):
    table = {"t27b_b32": {"kernel_source_sha": "aaaa", "hbm_bytes_per_launch": 123},
             "lmhead/t27b_b32": {"kernel_source_sha": "bbbb", "hbm_bytes_per_launch": 456}}
    (tmp_path / "traffic.json").write_text(json.dumps(table))
    monkeypatch.setattr(bench, "PROFILES", str(tmp_path))
    monkeypatch.setattr(bench, "kernel_source_hash", lambda family="select": {"select": "aaaa", "lmhead": "bbbb"}[family])
    assert bench.traffic_for("t27b_b32") == 123
    assert bench.traffic_for("t27b_b32", "lmhead") == 456
    assert bench.traffic_for("qwen3_4b_b1") is None
    monkeypatch.setattr(bench, "kernel_source_hash", lambda family="select": "cccc")
    assert bench.traffic_for("t27b_b32") is None
    assert bench.traffic_for("t27b_b32", "lmhead") is None


def test_kernel_source_hash_ignores_the_host_side(tmp_path, monkeypatch):
    src = tmp_path / "draft_selection_topk16_amd" / "csrc"
    src.mkdir(parents=True)
    for f in bench.KERNEL_SOURCES:
        (src / f).write_text("// %s\n" % f)
    (src / "dflash2.hip").write_text("device code\n// Host side.\nhost code\n")
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    h0 = bench.kernel_source_hash("select")
    (src / "dflash2.hip").write_text("device code\n// Host side.\nother host code\n")
    assert bench.kernel_source_hash("select") == h0
    (src / "dflash2.hip").write_text("changed device code\n// Host side.\nhost code\n")
    assert bench.kernel_source_hash("select") != h0


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120, cwd=ROOT)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_kernel_source_hash_ignores_comments_and_layout(tmp_path, monkeypatch):
    src = tmp_path / "draft_selection_topk16_amd" / "csrc"
    src.mkdir(parents=True)
    (src / "common.hpp").write_text("int f(int x) { return x + 1; }\n")
    (src / "lmhead.hpp").write_text('const char* s = "a // b";\n')
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    h0 = bench.kernel_source_hash("lmhead")
    (src / "common.hpp").write_text("// the successor\nint f(int x)  {\n  return x + 1;  /* one more */ }\n")
    assert bench.kernel_source_hash("lmhead") == h0
    (src / "lmhead.hpp").write_text('const char* s = "a // c";\n')      # inside a string: code
    assert bench.kernel_source_hash("lmhead") != h0
    (src / "lmhead.hpp").write_text('const char* s = "a // b";\n')
    (src / "common.hpp").write_text("int f(int x) { return x + 2; }\n")
    assert bench.kernel_source_hash("lmhead") != h0
