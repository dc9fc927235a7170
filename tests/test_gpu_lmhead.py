"""GPU parity of the drafter's LM head fused with top-K (dflash2_lmhead_topk)
against the oracle (oracle.lmhead_topk: float64 dot products and a full sort).

"DFlash 2: Keep Drafting Parallel", section "A Lightweight Path Selector":
the selector works on the drafter's own logits, U_t(v) = <W_lm[v], h_t>.

Acceptance rule.  bf16 x bf16 products are exact in fp32; the kernel sums
them in fp32 (matrix cores), so a logit differs from the exact one by a few
units in the last place of its scale s(v) = sum_k |W_lm[v][k] h[k]|.
  * Integer inputs (|logit| < 2^24): every sum is exact, so indices and
    values must equal the oracle's bit for bit, ties included.
  * Real inputs: each returned value must lie within TOL_LM * s(v) of the
    exact logit of its own token (TOL_LM = 2^-16: the root-sum-square of
    the d + d/32 fp32 roundings, d * 2^-24 at worst per rounding, is below
    2^-17.5 of s at d = 5120; the rigorous worst case, d * 2^-23, is checked
    too), the list must be ordered by its own values (ties to the lower
    token), and it may differ from the exact top-K only by near-ties: for a
    kept token t and a dropped token u, U(t) >= U(u) - TOL_LM (s(t) + s(u)).
    Rows that differ from the oracle are counted and printed.
"""
from __future__ import annotations

import concurrent.futures
import functools
import os

import numpy as np
import pytest
import torch

import oracle
from draft_selection_topk16_amd import synth
import draft_selection_topk16_amd as df2
from gpu_util import dev_tensor, say

pytestmark = pytest.mark.gpu

TOL_LM = 2.0 ** -16
THREADS = min(16, os.cpu_count() or 1)


def oracle_rows(X32, W32, K, rows):
    """oracle.lmhead_topk on `rows`, split over a host thread pool."""
    rows = np.asarray(rows, dtype=np.int64)
    if len(rows) < 2 or THREADS < 2:
        return oracle.lmhead_topk(X32, W32, K, rows=rows)
    parts = np.array_split(rows, min(THREADS, len(rows)))
    with concurrent.futures.ThreadPoolExecutor(len(parts)) as ex:
        res = list(ex.map(lambda r: oracle.lmhead_topk(X32, W32, K, rows=r), parts))
    return tuple(np.concatenate([r[i] for r in res]) for i in range(3))


def gpu_lmhead(Xb, Wb, K):
    X = dev_tensor(Xb, "bf16")
    W = dev_tensor(Wb, "bf16")
    idx, val = df2.lmhead_topk(X, W, K)
    torch.cuda.synchronize()
    assert df2.device_error() == 0
    return idx.cpu().numpy(), val.cpu().numpy()


def check_exact(gi, gv, X32, W32, K, rows, label):
    oi, ov, _ = oracle_rows(X32, W32, K, rows)
    assert np.array_equal(gi[rows], oi), label + ": indices differ from the oracle"
    assert np.array_equal(gv[rows].astype(np.float64), ov), label + ": values differ"
    say("%s: %d rows bit-exact" % (label, len(rows)))


def check_rule(gi, gv, X32, W32, K, rows, label, E=None):
    """The acceptance rule above on the sampled rows; returns the count of rows
    equal to the oracle's top-K."""
    E = K if E is None else E
    Kx = min(K + E, W32.shape[0])
    oi, ov, osig = oracle_rows(X32, W32, Kx, rows)
    d = X32.shape[1]
    m_rep = np.repeat(np.asarray(rows, dtype=np.int64), K)
    dot, s = oracle.lmhead_dot(X32, W32, m_rep, gi[rows].ravel())
    dot = dot.reshape(len(rows), K)
    s = s.reshape(len(rows), K)
    g = gv[rows].astype(np.float64)
    err = np.abs(g - dot)
    worst = float((err / s).max())
    assert np.all(err <= d * 2.0 ** -23 * s), label + ": beyond the worst-case fp32 bound"
    assert np.all(err <= TOL_LM * s), label + ": value error %.3g of scale > 2^-16" % worst
    exact_rows = 0
    for n, m in enumerate(rows):
        gi_m = gi[m]
        # ordered by the GPU's own values, ties to the lower token
        for j in range(K - 1):
            assert gv[m, j] > gv[m, j + 1] or (gv[m, j] == gv[m, j + 1] and gi_m[j] < gi_m[j + 1]), \
                "%s row %d: list not ordered at rank %d" % (label, m, j)
        assert len(set(gi_m.tolist())) == K, "%s row %d: repeated token" % (label, m)
        if np.array_equal(gi_m, oi[n, :K]):
            exact_rows += 1
            continue
        # near-ties only: every kept token is among the oracle's top K + E
        # (so every token beyond that list is below it), and no kept token
        # is below a dropped one of that list by more than the rounding
        kept = {int(t): (dot[n, j], s[n, j]) for j, t in enumerate(gi_m)}
        ext = set(int(t) for t in oi[n])
        assert set(kept) <= ext, "%s row %d: kept token outside the oracle's top %d" % (label, m, Kx)
        for j in range(Kx):
            u = int(oi[n, j])
            if u in kept:
                continue
            for t, (ut, st) in kept.items():
                assert ut >= ov[n, j] - TOL_LM * (st + osig[n, j]), \
                    "%s row %d: kept %d (%.9g) below dropped %d (%.9g) beyond rounding" % (
                        label, m, t, ut, u, ov[n, j])
    say("%s: %d/%d sampled rows equal to the oracle's top-%d, worst value error %.3g of scale"
        % (label, exact_rows, len(rows), K, worst))
    return exact_rows


# ------------------------------------------------------------ integer inputs
INT_CASES = [
    # M, V, d, K: ragged V, one and several M tiles, every list width
    (7, 5003, 128, 16),
    (1, 17, 64, 16),
    (5, 100, 64, 1),
    (3, 40, 64, 40),
    (224, 32000, 256, 16),
    (300, 20011, 192, 32),
    (33, 4099, 64, 64),
    (130, 9000, 128, 64),
    (16, 70000, 512, 16),
]


@pytest.mark.parametrize("M,V,d,K", INT_CASES, ids=lambda v: str(v))
def test_integer_inputs_bit_exact(M, V, d, K):
    rng = np.random.default_rng(M * 1000 + V + d + K)
    X32 = rng.integers(-3, 4, size=(M, d)).astype(np.float32)
    W32 = rng.integers(-3, 4, size=(V, d)).astype(np.float32)
    gi, gv = gpu_lmhead(synth.f32_to_bf16_bits(X32), synth.f32_to_bf16_bits(W32), K)
    check_exact(gi, gv, X32, W32, K, np.arange(M), "int M=%d V=%d d=%d K=%d" % (M, V, d, K))


def test_constant_logits_keep_lowest_tokens():
    # every logit equal: the K lowest token ids in every row, across ranges
    M, V, d, K = 9, 3000, 64, 16
    X32 = np.ones((M, d), dtype=np.float32)
    W32 = np.full((V, d), 0.5, dtype=np.float32)
    gi, gv = gpu_lmhead(synth.f32_to_bf16_bits(X32), synth.f32_to_bf16_bits(W32), K)
    assert np.array_equal(gi, np.tile(np.arange(K, dtype=np.int32), (M, 1)))
    assert np.all(gv == 32.0)


def test_signed_zero_logits_tie_by_index():
    M, V, d, K = 2, 300, 64, 8
    X32 = np.ones((M, d), dtype=np.float32)
    W32 = np.full((V, d), -1.0, dtype=np.float32)
    W32[[5, 77, 200]] = 0.0
    W32[[3, 150]] = -0.0
    gi, gv = gpu_lmhead(synth.f32_to_bf16_bits(X32), synth.f32_to_bf16_bits(W32), K)
    assert gi[0, :5].tolist() == [3, 5, 77, 150, 200]
    assert np.all(np.signbit(gv[:, :5]) == False)  # noqa: E712  (a -0 logit is returned as +0)


# ------------------------------------------------------- synthetic workloads
@functools.lru_cache(maxsize=1)
def lm_inputs(name):
    wl = synth.WORKLOADS[name]
    if wl.dtype != "bf16":
        wl = wl.with_(dtype="bf16")
    li = synth.make_lmhead_inputs(wl)
    X32, W32 = li.f32()
    return wl, li, X32, W32


WORKLOAD_ROWS = {
    # rows the oracle checks: all of them where it takes seconds
    "tiny_f32": None, "qwen3_4b_b1": None, "t27b_b8": None,
    "t27b_b32": np.arange(0, 224, 7),
    "stress_b256": np.arange(0, 3840, 240),
}


@pytest.mark.parametrize("name", list(WORKLOAD_ROWS))
def test_workloads(name):
    wl, li, X32, W32 = lm_inputs(name)
    say("lmhead %s: M=%d V=%d d=%d K=%d" % (name, wl.rows, wl.V, wl.d, wl.K))
    gi, gv = gpu_lmhead(li.X, li.W_lm, wl.K)
    rows = WORKLOAD_ROWS[name]
    rows = np.arange(wl.rows) if rows is None else rows
    check_rule(gi, gv, X32, W32, wl.K, rows, "lmhead " + name)
    # every row, not only the sampled ones: distinct tokens in range, ordered
    assert np.all((gi >= 0) & (gi < wl.V))
    for m in range(wl.rows):
        assert len(set(gi[m].tolist())) == wl.K
        assert np.all(np.diff(gv[m]) <= 0)


@pytest.mark.parametrize("ranges", [1, 3, 37, 256])
def test_plan_invariance_over_vocabulary_ranges(ranges):
    wl, li, _, _ = lm_inputs("t27b_b8")
    ref_i, ref_v = gpu_lmhead(li.X, li.W_lm, wl.K)
    with df2.plan(lm_ranges=ranges):
        gi, gv = gpu_lmhead(li.X, li.W_lm, wl.K)
    assert np.array_equal(gi, ref_i) and np.array_equal(gv, ref_v)


def test_matches_topk_of_its_own_logits_on_integer_inputs():
    # with exact sums, the fused path equals dflash2_topk run on the logits
    # written out (fp32), element for element
    rng = np.random.default_rng(5)
    M, V, d, K = 40, 12000, 320, 16
    X32 = rng.integers(-2, 3, size=(M, d)).astype(np.float32)
    W32 = rng.integers(-2, 3, size=(V, d)).astype(np.float32)
    gi, gv = gpu_lmhead(synth.f32_to_bf16_bits(X32), synth.f32_to_bf16_bits(W32), K)
    L = torch.from_numpy(X32.astype(np.float64) @ W32.astype(np.float64).T).float().cuda()
    ti, tv = df2.topk(L, K)
    assert np.array_equal(gi, ti.cpu().numpy()) and np.array_equal(gv, tv.cpu().numpy())


def test_repeat_calls_identical():
    wl, li, _, _ = lm_inputs("t27b_b8")
    a = gpu_lmhead(li.X, li.W_lm, wl.K)
    b = gpu_lmhead(li.X, li.W_lm, wl.K)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])
