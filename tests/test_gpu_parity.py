"""GPU parity: the HIP path (through the C ABI) against the CPU oracle.

Every case prints its name before touching the GPU.  Workloads follow the
five seeded workloads of draft_selection_topk16_amd.synth, each checked in
full: every top-K row of the stress workload (3840 rows of 262144 logits)
by the defining property of the top-K (vectorised numpy) and sampled rows
against the oracle's full sort; every one of its 256 sequences against the
oracle, run in a host thread pool (the oracle's C calls release the GIL).
"""
import os

import numpy as np
import pytest
import torch

import oracle
import draft_selection_topk16_amd as df2
from draft_selection_topk16_amd import synth
from gpu_util import (TOL, TOL_SAMPLE, check_greedy, check_sample, check_scores, check_select,
                      dev_tensor, run_oracle, say, to_device)

pytestmark = pytest.mark.gpu

ORACLE_THREADS = max(1, min(16, os.cpu_count() or 1))


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    df2.load()
    yield
    torch.cuda.synchronize()


_cache = {}


def inputs(name, **kw):
    key = (name, tuple(sorted(kw.items())))
    if key not in _cache:
        wl = synth.WORKLOADS[name].with_(**kw) if kw else synth.WORKLOADS[name]
        _cache.clear()      # keep at most one (possibly large) input set alive
        _cache[key] = synth.make_inputs(wl)
    return _cache[key]


_stress = {}


def stress_oracle(x):
    """The oracle on all sequences of the stress workload, with the sampling
    walk at temperature 1 on the uniforms the sampling test draws (cached:
    select, greedy, sample, pair-score and projection tests share it)."""
    key = (x.wl.B, x.wl.P, x.wl.V, x.wl.K, x.wl.d)
    if _stress.get("key") != key:
        _stress.clear()
        _stress["key"] = key
        say("  running the oracle on all %d stress sequences (%d threads)" % (x.wl.B, ORACLE_THREADS))
        u = f32_uniforms(uniforms(x.wl.B, x.wl.P, 99))
        _stress["o"] = run_oracle(x, u=u.astype(np.float64), tau=1.0, threads=ORACLE_THREADS)
        _stress["u"] = u
    return _stress["o"]


def topk_property_violations(x_np, dtype, K, idx, val, row_chunk=128):
    """Rows whose GPU top-K is not THE top-K by definition: its K indices are
    distinct, their values are the row's values at those indices, the list
    is ordered by (value desc, index asc), and no unselected element has a
    larger value, or an equal value at a lower index, than the K-th."""
    bad = []
    rows, V = x_np.shape
    for r0 in range(0, rows, row_chunk):
        xv = synth.to_f64(x_np[r0:r0 + row_chunk], dtype).astype(np.float64)
        xv = np.where(xv == 0.0, 0.0, xv)          # -0 and +0 are one value
        ii = idx[r0:r0 + row_chunk].astype(np.int64)
        vv = val[r0:r0 + row_chunk].astype(np.float64)
        n = xv.shape[0]
        ok = np.all((ii >= 0) & (ii < V), axis=1)
        ii = np.clip(ii, 0, V - 1)
        got = np.take_along_axis(xv, ii, axis=1)
        ok &= np.all(got == vv, axis=1)
        ok &= np.all(np.sort(ii, axis=1)[:, 1:] != np.sort(ii, axis=1)[:, :-1], axis=1)
        order_ok = (vv[:, :-1] > vv[:, 1:]) | ((vv[:, :-1] == vv[:, 1:]) & (ii[:, :-1] < ii[:, 1:]))
        ok &= np.all(order_ok, axis=1)
        sel = np.zeros_like(xv, dtype=bool)
        np.put_along_axis(sel, ii, True, axis=1)
        kv, ki = vv[:, -1:], ii[:, -1:]
        cols = np.arange(V)[None, :]
        beats = ((xv > kv) | ((xv == kv) & (cols < ki))) & ~sel
        ok &= ~np.any(beats, axis=1)
        bad += [r0 + i for i in np.nonzero(~ok)[0]]
    return bad


def gpu_topk(x_np, dtype, K):
    t = dev_tensor(x_np, dtype)
    idx, val = df2.topk(t, K)
    torch.cuda.synchronize()
    return idx.cpu().numpy(), val.cpu().numpy()


# --------------------------------------------------------------------- top-K
@pytest.mark.parametrize("name", ["tiny_f32", "qwen3_4b_b1", "t27b_b8", "t27b_b32", "stress_b256"])
def test_topk_workloads(name):
    x = inputs(name)
    K, V = x.wl.K, x.wl.V
    say("topk %s K=%d V=%d rows=%d" % (name, K, V, x.wl.rows))
    flat = x.logits.reshape(-1, V)
    idx, val = gpu_topk(flat, x.wl.dtype, K)
    bad = topk_property_violations(flat, x.wl.dtype, K, idx, val)
    assert not bad, "%s: %d of %d rows are not the top-K (first: %s)" % (name, len(bad), flat.shape[0], bad[:5])
    rows = np.arange(flat.shape[0])
    if name == "stress_b256":
        rows = np.unique(np.concatenate([np.arange(0, flat.shape[0], 61), [flat.shape[0] - 1]]))
    oi, ov = oracle.topk(synth.to_f64(flat[rows], x.wl.dtype), K)
    assert np.array_equal(idx[rows], oi)
    assert np.array_equal(val[rows].astype(np.float64), ov)
    say("  %d rows top-K by definition, %d rows equal to the oracle's full sort" % (flat.shape[0], len(rows)))


def _tie_rows(kind, V, rng):
    if kind == "constant":
        return np.full((3, V), 1.25, dtype=np.float32)
    if kind == "signed_zero":
        x = np.where(rng.random((3, V)) < 0.5, -0.0, 0.0).astype(np.float32)
        x[:, ::97] = -1.0
        return x
    if kind == "flat_normal":
        return rng.standard_normal((4, V)).astype(np.float32)
    if kind == "two_levels":
        return (rng.random((3, V)) < 0.002).astype(np.float32)
    if kind == "all_negative":
        return (-np.abs(rng.standard_normal((3, V))) - 3.0).astype(np.float32)
    if kind == "neg_inf_mix":
        x = rng.standard_normal((3, V)).astype(np.float32)
        x[:, ::3] = -np.inf
        x[0, :] = -np.inf
        x[0, 5] = np.inf
        return x
    if kind == "ascending":
        return np.tile(np.arange(V, dtype=np.float32) / V, (2, 1))
    raise ValueError(kind)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("kind", ["constant", "signed_zero", "flat_normal", "two_levels",
                                  "all_negative", "neg_inf_mix", "ascending"])
@pytest.mark.parametrize("V,K", [(151936, 16), (40000, 32), (1001, 64), (37, 5), (16, 16), (20000, 1)])
def test_topk_ties_and_edges(dtype, kind, V, K):
    say("topk ties %s %s V=%d K=%d" % (dtype, kind, V, K))
    rng = np.random.default_rng(V * 7 + K)
    x32 = _tie_rows(kind, V, rng)
    x = synth.f32_to_bf16_bits(x32) if dtype == "bf16" else x32
    idx, val = gpu_topk(x, dtype, K)
    oi, ov = oracle.topk(synth.to_f64(x, dtype), K)
    assert np.array_equal(idx, oi)
    assert np.array_equal(val.astype(np.float64), ov)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_topk_unaligned_rows(dtype):
    """Row starts that are not 16-byte aligned take the element-wise loads."""
    V, K, rows = 30001, 16, 5
    say("topk unaligned %s" % dtype)
    rng = np.random.default_rng(3)
    flat32 = rng.standard_normal(rows * V + 1).astype(np.float32)
    flat = synth.f32_to_bf16_bits(flat32) if dtype == "bf16" else flat32
    t = dev_tensor(flat, dtype)[1:].reshape(rows, V)
    assert t.data_ptr() % 16 != 0
    idx, val = df2.topk(t, K)
    oi, ov = oracle.topk(synth.to_f64(flat[1:].reshape(rows, V), dtype), K)
    assert np.array_equal(idx.cpu().numpy(), oi)
    assert np.array_equal(val.cpu().numpy().astype(np.float64), ov)


# ---------------------------------------------------------------- projection
@pytest.mark.parametrize("name", ["tiny_f32", "qwen3_4b_b1", "t27b_b8", "t27b_b32", "stress_b256"])
def test_project_workloads(name):
    x = inputs(name)
    say("project %s M=%d d=%d" % (name, x.wl.rows, x.wl.d))
    t = to_device(x)
    H = df2.project(t["hidden"], t["W"]).cpu().numpy().astype(np.float64)
    f = x.f64()
    Hr = oracle.project(f["hidden"], f["W"])
    scale = np.abs(f["hidden"]) @ np.abs(f["W"]).T       # sum_m |W h|
    rel = np.abs(H - Hr) / scale
    say("  worst rel err %.3g" % rel.max())
    assert rel.max() <= TOL[x.wl.dtype]


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("M,d,r", [(1, 32, 64), (17, 96, 128), (64, 64, 64), (300, 512, 256), (3840, 256, 256),
                                   (17, 96, 320), (40, 256, 512)])
def test_project_shapes(dtype, M, d, r):
    say("project shape %s M=%d d=%d r=%d" % (dtype, M, d, r))
    rng = np.random.default_rng(M + d + r)
    h32 = rng.standard_normal((M, d)).astype(np.float32)
    w32 = (rng.standard_normal((r, d)) / 8).astype(np.float32)
    h = synth.f32_to_bf16_bits(h32) if dtype == "bf16" else h32
    w = synth.f32_to_bf16_bits(w32) if dtype == "bf16" else w32
    H = df2.project(dev_tensor(h, dtype), dev_tensor(w, dtype)).cpu().numpy().astype(np.float64)
    hf, wf = synth.to_f64(h, dtype), synth.to_f64(w, dtype)
    rel = np.abs(H - oracle.project(hf, wf)) / (np.abs(hf) @ np.abs(wf).T)
    assert rel.max() <= TOL[dtype]


# ------------------------------------------------------------- pair scores
@pytest.mark.parametrize("name,kw", [("tiny_f32", {}), ("qwen3_4b_b1", {}),
                                     ("t27b_b8", {"pair_scale": 8.0}),
                                     ("stress_b256", {"B": 3, "V": 20000, "d": 256}),
                                     ("tiny_f32", {"r": 320, "V": 4000}),
                                     ("qwen3_4b_b1", {"r": 512, "V": 20000})])
def test_pair_scores_stage(name, kw):
    x = inputs(name, **kw)
    say("pair_scores %s %s" % (name, kw))
    o = run_oracle(x)
    dt = x.wl.dtype
    t = to_device(x)
    cand = torch.from_numpy(o["cand"]).cuda()
    cval = torch.from_numpy(o["U"].astype(np.float32)).cuda()
    H32 = o["H"].astype(np.float32)
    S = df2.pair_scores(cand, cval, torch.from_numpy(H32).cuda(), t["A"], t["Bt"], t["prev"])
    S = S.cpu().numpy()
    f = x.f64()
    S_ref, sig = oracle.pair_scores(o["cand"], o["U"], H32.astype(np.float64), f["A"], f["Bt"], f["prev"])
    check_scores(S, S_ref, sig, TOL[dt], "S " + name)


def test_pair_scores_stage_stress_full():
    """The pair-score stage at the stress shape (B=256, P=15, K=32, r=256) on
    the oracle's own candidates and gate rows (as fp32), every sequence."""
    x = inputs("stress_b256")
    say("pair_scores stress, all sequences")
    o = stress_oracle(x)
    t = to_device(x)
    H32 = o["H"].astype(np.float32)
    S = df2.pair_scores(torch.from_numpy(o["cand"]).cuda(), torch.from_numpy(o["U"].astype(np.float32)).cuda(),
                        torch.from_numpy(H32).cuda(), t["A"], t["Bt"], t["prev"]).cpu().numpy()
    f = x.f64()
    S_ref, sig = oracle.pair_scores(o["cand"], o["U"], H32.astype(np.float64), f["A"], f["Bt"], f["prev"])
    check_scores(S, S_ref, sig, TOL["bf16"], "S stress")


# ------------------------------------------------------------------- walk
@pytest.mark.parametrize("K,P", [(16, 7), (32, 15), (5, 3), (1, 4), (64, 2), (16, 64)])
def test_viterbi_stage(K, P):
    say("viterbi K=%d P=%d" % (K, P))
    rng = np.random.default_rng(K * 100 + P)
    B = 9
    S = rng.standard_normal((B, P, K, K)).astype(np.float32)
    S[:, 0, 1:, :] = S[:, 0, :1, :]       # t = 0 rows all equal row 0
    cand = rng.integers(0, 1 << 20, size=(B, P, K)).astype(np.int32)
    path, score = df2.viterbi(torch.from_numpy(S).cuda(), torch.from_numpy(cand).cuda())
    pr, pt, sc = oracle.viterbi(S.astype(np.float64), cand)
    sec = oracle.second_best(S.astype(np.float64), pr)
    path = path.cpu().numpy()
    score = score.cpu().numpy().astype(np.float64)
    for b in range(B):
        if not np.array_equal(path[b], pt[b]):
            assert sc[b] - sec[b] <= 1e-5 * P * 4, (b, sc[b], sec[b])
        assert abs(score[b] - sc[b]) <= 1e-5 * P * 4


@pytest.mark.parametrize("K,P", [(8, 6), (16, 7), (13, 20), (16, 64), (4, 33), (1, 3), (32, 17), (64, 5)])
def test_viterbi_integer_ties_exact(K, P):
    """Small-integer scores are exact in fp32: ties must break exactly like
    the oracle (smaller predecessor rank, smaller final rank).  K <= 16 runs
    four lanes per candidate (K = 13 and 4 leave some quads idle and pad the
    predecessors with -inf;
    P = 20, 33 and 64 span two to four groups of sixteen positions in LDS and
    of the backtrack); K = 32 and 64 one lane per candidate."""
    say("viterbi integer ties K=%d P=%d" % (K, P))
    rng = np.random.default_rng(42 + K * 1000 + P)
    B = 16
    S = rng.integers(-2, 3, size=(B, P, K, K)).astype(np.float32)
    S[:, 0, 1:, :] = S[:, 0, :1, :]
    cand = np.tile(np.arange(K, dtype=np.int32), (B, P, 1)) + 1000
    path, score = df2.viterbi(torch.from_numpy(S).cuda(), torch.from_numpy(cand).cuda())
    _, pt, sc = oracle.viterbi(S.astype(np.float64), cand)
    assert np.array_equal(path.cpu().numpy(), pt)
    assert np.array_equal(score.cpu().numpy().astype(np.float64), sc)


@pytest.mark.parametrize("K,P", [(16, 7), (32, 15), (5, 3), (1, 4), (64, 2), (16, 64), (64, 64),
                                 (3, 17)])
def test_greedy_stage(K, P):
    """Greedy decisions compare the same fp32 scores on both sides, so the
    path must match exactly; the score is an fp32 sum in order of t."""
    say("greedy walk K=%d P=%d" % (K, P))
    rng = np.random.default_rng(K * 100 + P + 7)
    B = 9
    S = rng.standard_normal((B, P, K, K)).astype(np.float32)
    S[:, 0, 1:, :] = S[:, 0, :1, :]
    cand = rng.integers(0, 1 << 20, size=(B, P, K)).astype(np.int32)
    path, score = df2.walk(torch.from_numpy(S).cuda(), torch.from_numpy(cand).cuda(), "greedy")
    pr, pt, sc = oracle.greedy(S.astype(np.float64), cand)
    assert np.array_equal(path.cpu().numpy(), pt)
    score = score.cpu().numpy().astype(np.float64)
    for b in range(B):
        mag = abs(S[b, 0, 0, pr[b, 0]]) + sum(abs(S[b, t, pr[b, t - 1], pr[b, t]]) for t in range(1, P))
        assert abs(score[b] - sc[b]) <= 2.0 ** -23 * P * mag, (b, score[b], sc[b])


def test_greedy_integer_ties_exact():
    """Small integers: many exact ties, all sums exact; the lower rank wins."""
    say("greedy walk integer ties")
    rng = np.random.default_rng(43)
    B, P, K = 16, 9, 8
    S = rng.integers(-2, 3, size=(B, P, K, K)).astype(np.float32)
    S[:, 0, 1:, :] = S[:, 0, :1, :]
    cand = np.tile(np.arange(K, dtype=np.int32), (B, P, 1)) + 1000
    path, score = df2.walk(torch.from_numpy(S).cuda(), torch.from_numpy(cand).cuda(), "greedy")
    _, pt, sc = oracle.greedy(S.astype(np.float64), cand)
    assert np.array_equal(path.cpu().numpy(), pt)
    assert np.array_equal(score.cpu().numpy().astype(np.float64), sc)


def test_walk_viterbi_mode_matches_viterbi_entry():
    say("walk(viterbi) equals viterbi")
    rng = np.random.default_rng(44)
    B, P, K = 5, 11, 16
    S = torch.from_numpy(rng.standard_normal((B, P, K, K)).astype(np.float32)).cuda()
    cand = torch.from_numpy(rng.integers(0, 5000, size=(B, P, K)).astype(np.int32)).cuda()
    p1, s1 = df2.viterbi(S, cand)
    p2, s2 = df2.walk(S, cand, "viterbi")
    assert torch.equal(p1, p2) and torch.equal(s1, s2)


# ------------------------------------------------------------ whole select
def gpu_select(x, walk="viterbi"):
    t = to_device(x)
    path, score = df2.select(t["logits"], t["hidden"], t["A"], t["Bt"], t["W"], t["prev"], x.wl.K,
                             walk=walk)
    torch.cuda.synchronize()
    return path.cpu().numpy(), score.cpu().numpy()


@pytest.mark.parametrize("name", ["tiny_f32", "qwen3_4b_b1", "t27b_b8", "t27b_b32", "stress_b256"])
def test_select_workloads(name):
    x = inputs(name)
    say("select %s B=%d P=%d V=%d K=%d" % (name, x.wl.B, x.wl.P, x.wl.V, x.wl.K))
    path, score = gpu_select(x)
    o = stress_oracle(x) if name == "stress_b256" else run_oracle(x, threads=ORACLE_THREADS)
    check_select(path, score, o, TOL[x.wl.dtype], name)
    assert flags_clear()


@pytest.mark.parametrize("name,kw", [
    ("tiny_f32", {"pair_scale": 8.0, "V": 4000}),
    ("qwen3_4b_b1", {"pair_scale": 8.0}),
    ("t27b_b8", {"pair_scale": 8.0, "V": 30000, "d": 512}),
    ("stress_b256", {"pair_scale": 8.0, "B": 4, "V": 50000, "d": 512}),
])
def test_select_pair_dominant(name, kw):
    """A and B scaled so the pair term outweighs logit gaps: the walk, not
    the top-1 pick, decides the path."""
    x = inputs(name, **kw)
    say("select pair-dominant %s %s" % (name, kw))
    path, score = gpu_select(x)
    o = run_oracle(x)
    top1 = o["cand"][:, :, 0]
    say("  positions where the path leaves top-1: %d of %d" % (int((o["path"] != top1).sum()), top1.size))
    check_select(path, score, o, TOL[x.wl.dtype], name)


@pytest.mark.parametrize("K,launches,B", [(16, 0, 6), (16, 4, 6), (24, 3, 6), (24, 4, 6), (32, 4, 6),
                                          (5, 4, 6), (16, 0, 2), (13, 0, 1), (5, 0, 2), (16, 3, 2)])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_select_integer_exact(dtype, K, launches, B):
    """Small-integer inputs keep every step exact on both sides (bf16 hi/lo
    split included): paths and scores must match bit for bit, also with the
    walks in a launch of their own (K = 24 and 32 there walk two lanes per
    candidate) and with a gate of one m-block (B <= 2: H from the tile
    sums)."""
    say("select integer-exact %s K=%d launches=%d B=%d" % (dtype, K, launches, B))
    rng = np.random.default_rng(7 + K + 100 * B)
    P, V, d, r = 7, 3000, 64, 64
    wl = synth.Workload("int", 0, B=B, P=P, V=V, d=d, K=K, r=r, dtype=dtype)
    logits = rng.integers(-6, 7, size=(B, P, V)).astype(np.float32)
    x = synth.make_inputs(wl, seed=123, logits_override=logits)
    for k, shape in (("hidden", (B, P, d)), ("A", (V, r)), ("Bt", (V, r)), ("W", (r, d))):
        v = rng.integers(-2, 3, size=shape).astype(np.float32)
        setattr(x, k, synth.f32_to_bf16_bits(v) if dtype == "bf16" else v)
    with df2.plan(launches=launches):
        path, score = gpu_select(x)
    o = run_oracle(x)
    assert np.array_equal(path, o["path"])
    assert np.array_equal(score.astype(np.float64), o["score"])


@pytest.mark.parametrize("B,P,V,K,d", [(1, 1, 5000, 16, 64), (3, 64, 3000, 16, 64),
                                       (2, 5, 64, 64, 64), (2, 4, 300, 1, 64),
                                       (5, 3, 16, 16, 32), (4, 7, 9999, 3, 96),
                                       (33, 7, 2048, 16, 64)])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_select_edge_shapes(B, P, V, K, d, dtype):
    say("select edge %s B=%d P=%d V=%d K=%d d=%d" % (dtype, B, P, V, K, d))
    wl = synth.Workload("edge", 1, B=B, P=P, V=V, d=d, K=K, r=64, dtype=dtype, pair_scale=4.0)
    x = synth.make_inputs(wl, seed=B * 1000 + P * 10 + K)
    path, score = gpu_select(x)
    check_select(path, score, run_oracle(x), TOL[dtype], "edge")


@pytest.mark.parametrize("r", [320, 512])
@pytest.mark.parametrize("launches", [1, 2, 3, 4])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_select_wide_gate(r, launches, dtype):
    """Gate ranks above one value per thread (r > 256, up to the 512 the
    library accepts): the row merge sums a second gate value per thread, the
    pair job loads a second one per position and takes 16 k steps, in the
    fused launch, in both two-launch plans (in the three-stage one the pair
    job takes H from the gate tile sums) and with the walks in a third
    launch."""
    say("select wide gate %s r=%d launches=%d" % (dtype, r, launches))
    wl = synth.Workload("wide", 1, B=3, P=5, V=3000, d=128, K=16, r=r, dtype=dtype, pair_scale=4.0)
    x = synth.make_inputs(wl, seed=r + 7)
    with df2.plan(launches=launches):
        path, score = gpu_select(x)
    check_select(path, score, run_oracle(x), TOL[dtype], "wide gate")


def test_select_empty_batch():
    say("select empty batch")
    dev = "cuda"
    logits = torch.empty((0, 7, 1000), dtype=torch.bfloat16, device=dev)
    hidden = torch.empty((0, 7, 64), dtype=torch.bfloat16, device=dev)
    A = torch.zeros((1000, 64), dtype=torch.bfloat16, device=dev)
    W = torch.zeros((64, 64), dtype=torch.bfloat16, device=dev)
    prev = torch.empty((0,), dtype=torch.int32, device=dev)
    path, score = df2.select(logits, hidden, A, A, W, prev, 16)
    assert path.shape == (0, 7) and score.shape == (0,)


@pytest.mark.parametrize("name", ["t27b_b8", "qwen3_4b_b1", "stress_b256"])
def test_select_same_result_under_any_segment_plan(name):
    """The segment plan (segments per row, chunk width, words per merge) and
    the choice of launches (one fused, scan then tail, the three-stage
    default, or three stages with the walks in a third launch, the default
    beyond one resident wave of rows) change neither the gate sums nor any
    comparison: candidate words are exact, the merge is independent of how a
    row was cut, and every plan sums H in slice order, so path and score are
    bit-identical across plans.  At the stress workload the scan grid and the
    3840-row pair launch are each more than one resident wave."""
    say("select under segment plans %s" % name)
    x = inputs(name)
    t = to_device(x)
    args = (t["logits"], t["hidden"], t["A"], t["Bt"], t["W"], t["prev"], x.wl.K)
    ref = [a.clone() for a in df2.select(*args)]
    torch.cuda.synchronize()
    for knobs in ({"segment_wgs": 64}, {"segment_wgs": 700}, {"chunk_vectors": 1},
                  {"chunk_vectors": 2, "segment_wgs": 300}, {"merge_words": 256},
                  {"launches": 1}, {"launches": 1, "segment_wgs": 300},
                  {"launches": 2}, {"launches": 2, "segment_wgs": 300},
                  {"launches": 3}, {"launches": 3, "segment_wgs": 300}, {"launches": 3, "merge_words": 256},
                  {"launches": 4}, {"launches": 4, "segment_wgs": 300}):
        with df2.plan(**knobs):
            p, s = df2.select(*args)
            torch.cuda.synchronize()
        assert torch.equal(p, ref[0]) and torch.equal(s, ref[1]), knobs


@pytest.mark.parametrize("name", ["t27b_b8", "qwen3_4b_b1"])
def test_select_walk_modes_same_in_every_plan(name):
    """Every walk mode (max-sum, greedy, sampling) returns the same bits in
    all four launch plans, including the one with the walks in a launch of
    their own."""
    say("select walk modes across launch plans %s" % name)
    x = inputs(name)
    t = to_device(x)
    args = (t["logits"], t["hidden"], t["A"], t["Bt"], t["W"], t["prev"], x.wl.K)
    u = torch.from_numpy(np.random.default_rng(5).random((x.wl.B, x.wl.P), dtype=np.float32)).cuda()
    runs = {"viterbi": lambda: df2.select(*args), "greedy": lambda: df2.select(*args, walk="greedy"),
            "sample": lambda: df2.select_sample(*args, u=u)}
    for wname, fn in runs.items():
        ref = None
        for launches in (0, 1, 2, 3, 4):
            with df2.plan(launches=launches):
                out = [o.clone() for o in fn()]
                torch.cuda.synchronize()
            if ref is None:
                ref = out
            assert all(torch.equal(a, b) for a, b in zip(ref, out)), (wname, launches)
    assert flags_clear()


def test_select_deterministic_and_scratch_reuse():
    say("select determinism and scratch reuse")
    big = inputs("t27b_b32")
    tb = to_device(big)
    small = synth.make_inputs(synth.WORKLOADS["tiny_f32"].with_(V=5000))
    ts = to_device(small)
    ref_b = df2.select(tb["logits"], tb["hidden"], tb["A"], tb["Bt"], tb["W"], tb["prev"], 16)
    ref_s = df2.select(ts["logits"], ts["hidden"], ts["A"], ts["Bt"], ts["W"], ts["prev"], 16)
    ref_b = [a.clone() for a in ref_b]
    ref_s = [a.clone() for a in ref_s]
    for i in range(20):
        if i % 2:
            p, s = df2.select(tb["logits"], tb["hidden"], tb["A"], tb["Bt"], tb["W"], tb["prev"], 16)
            assert torch.equal(p, ref_b[0]) and torch.equal(s, ref_b[1])
        else:
            p, s = df2.select(ts["logits"], ts["hidden"], ts["A"], ts["Bt"], ts["W"], ts["prev"], 16)
            assert torch.equal(p, ref_s[0]) and torch.equal(s, ref_s[1])
    o = run_oracle(small)
    check_select(ref_s[0].cpu().numpy(), ref_s[1].cpu().numpy(), o, TOL["f32"], "small after big")


def flags_clear():
    return df2.device_error() == 0


def test_prev_tok_out_of_range_sets_flag():
    say("select prev_tok out of range")
    x = synth.make_inputs(synth.WORKLOADS["tiny_f32"].with_(V=3000, B=2))
    t = to_device(x)
    assert df2.device_error() == 0
    bad = t["prev"].clone()
    bad[1] = 3000
    path, score = df2.select(t["logits"], t["hidden"], t["A"], t["Bt"], t["W"], bad, 16)
    assert df2.device_error() == 1
    assert df2.device_error() == 0          # reading clears the flag
    x.prev = np.array([x.prev[0], 0], dtype=np.int32)   # replaced by token 0
    check_select(path.cpu().numpy(), score.cpu().numpy(), run_oracle(x), TOL["f32"], "bad prev")


@pytest.mark.parametrize("launches", [1, 2])
def test_gate_wait_give_up_then_recovery(launches):
    """A gate wait that gives up, forced from the host (the row merges wait
    for one gate arrival more than will come, for 64 sleeps, so every kernel
    still exits), raises flag bit 2; the calls after it on the stream equal a
    clean run bit for bit: once the flag is reported, the next call clears
    the arrival counters a late gate slice can leave behind."""
    say("select gate give-up and recovery, launches=%d" % launches)
    x = inputs("t27b_b8")
    t = to_device(x)
    args = (t["logits"], t["hidden"], t["A"], t["Bt"], t["W"], t["prev"], 16)
    with df2.plan(launches=launches):
        ref = [a.clone() for a in df2.select(*args)]
        assert flags_clear()
        with df2.plan(gate_giveup=1):
            df2.select(*args)
            torch.cuda.synchronize()
        assert df2.device_error() == 4
        for _ in range(3):
            p, s = df2.select(*args)
            assert torch.equal(p, ref[0]) and torch.equal(s, ref[1])
        assert flags_clear()


def test_gate_giveup_knob_inert_in_three_stage_plan():
    """The three-stage plan has no gate wait (its pair jobs run after the
    whole scan): with the give-up knob set it still returns the clean result
    and raises no flag."""
    say("select three-stage plan with the give-up knob")
    x = inputs("t27b_b8")
    t = to_device(x)
    args = (t["logits"], t["hidden"], t["A"], t["Bt"], t["W"], t["prev"], 16)
    with df2.plan(launches=3):
        ref = [a.clone() for a in df2.select(*args)]
        assert flags_clear()
        with df2.plan(gate_giveup=1):
            p, s = df2.select(*args)
            torch.cuda.synchronize()
        assert flags_clear()
        assert torch.equal(p, ref[0]) and torch.equal(s, ref[1])


def test_stages_compose_to_select():
    """topk -> project -> pair_scores -> viterbi gives the fused result."""
    x = inputs("qwen3_4b_b1")
    say("stages compose")
    t = to_device(x)
    B, P, V = x.wl.B, x.wl.P, x.wl.V
    idx, val = df2.topk(t["logits"], 16)
    H = df2.project(t["hidden"], t["W"])
    S = df2.pair_scores(idx, val, H, t["A"], t["Bt"], t["prev"])
    p1, s1 = df2.viterbi(S, idx)
    p2, s2 = df2.select(t["logits"], t["hidden"], t["A"], t["Bt"], t["W"], t["prev"], 16)
    assert torch.equal(p1, p2)
    assert torch.allclose(s1, s2, rtol=1e-6, atol=1e-6)


# ------------------------------------------------------ whole select, greedy
@pytest.mark.parametrize("name", ["tiny_f32", "qwen3_4b_b1", "t27b_b32", "stress_b256"])
def test_select_greedy_workloads(name):
    x = inputs(name)
    say("select greedy %s B=%d P=%d V=%d K=%d" % (name, x.wl.B, x.wl.P, x.wl.V, x.wl.K))
    path, score = gpu_select(x, "greedy")
    o = stress_oracle(x) if name == "stress_b256" else run_oracle(x, threads=ORACLE_THREADS)
    check_greedy(path, score, o, TOL[x.wl.dtype], name)
    assert flags_clear()


@pytest.mark.parametrize("name,kw", [
    ("tiny_f32", {"pair_scale": 8.0, "V": 4000}),
    ("qwen3_4b_b1", {"pair_scale": 8.0}),
    ("t27b_b8", {"pair_scale": 8.0, "V": 30000, "d": 512}),
])
def test_select_greedy_pair_dominant(name, kw):
    """Pair-dominant inputs: greedy and Viterbi part ways; both walks of the
    GPU follow their oracle, and the share of sequences where the two walks'
    paths differ is reported."""
    x = inputs(name, **kw)
    say("select greedy pair-dominant %s %s" % (name, kw))
    gp, gs = gpu_select(x, "greedy")
    vp, vs = gpu_select(x, "viterbi")
    o = run_oracle(x)
    check_greedy(gp, gs, o, TOL[x.wl.dtype], name + " greedy")
    check_select(vp, vs, o, TOL[x.wl.dtype], name + " viterbi")
    differ = int(np.sum(np.any(o["greedy_path"] != o["path"], axis=1)))
    say("  greedy and Viterbi paths differ in %d of %d sequences (oracle); GPU: %d"
        % (differ, o["path"].shape[0], int(np.sum(np.any(gp != vp, axis=1)))))
    # the best path never scores below the greedy one
    assert np.all(o["score"] >= o["greedy_score"] - 1e-9 * np.maximum(1.0, np.abs(o["score"])))


@pytest.mark.parametrize("B,P,V,K,d", [(1, 1, 5000, 16, 64), (3, 64, 3000, 16, 64),
                                       (2, 5, 64, 64, 64), (2, 4, 300, 1, 64),
                                       (4, 7, 9999, 3, 96), (33, 7, 2048, 16, 64)])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_select_greedy_edge_shapes(B, P, V, K, d, dtype):
    say("select greedy edge %s B=%d P=%d V=%d K=%d d=%d" % (dtype, B, P, V, K, d))
    wl = synth.Workload("edge", 1, B=B, P=P, V=V, d=d, K=K, r=64, dtype=dtype, pair_scale=4.0)
    x = synth.make_inputs(wl, seed=B * 1000 + P * 10 + K + 5)
    path, score = gpu_select(x, "greedy")
    check_greedy(path, score, run_oracle(x), TOL[dtype], "greedy edge")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_select_greedy_integer_exact(dtype):
    """Small-integer inputs keep every step exact: the greedy path and score
    match the oracle bit for bit, ties included."""
    say("select greedy integer-exact %s" % dtype)
    rng = np.random.default_rng(8)
    B, P, V, d, r, K = 6, 9, 3000, 64, 64, 16
    wl = synth.Workload("int", 0, B=B, P=P, V=V, d=d, K=K, r=r, dtype=dtype)
    logits = rng.integers(-6, 7, size=(B, P, V)).astype(np.float32)
    x = synth.make_inputs(wl, seed=124, logits_override=logits)
    for k, shape in (("hidden", (B, P, d)), ("A", (V, r)), ("Bt", (V, r)), ("W", (r, d))):
        v = rng.integers(-2, 3, size=shape).astype(np.float32)
        setattr(x, k, synth.f32_to_bf16_bits(v) if dtype == "bf16" else v)
    path, score = gpu_select(x, "greedy")
    o = run_oracle(x)
    assert np.array_equal(path, o["greedy_path"])
    assert np.array_equal(score.astype(np.float64), o["greedy_score"])


def test_greedy_stages_compose_to_select():
    """topk -> project -> pair_scores -> walk(greedy) gives the fused greedy result."""
    x = inputs("qwen3_4b_b1")
    say("greedy stages compose")
    t = to_device(x)
    idx, val = df2.topk(t["logits"], 16)
    H = df2.project(t["hidden"], t["W"])
    S = df2.pair_scores(idx, val, H, t["A"], t["Bt"], t["prev"])
    p1, s1 = df2.walk(S, idx, "greedy")
    p2, s2 = df2.select(t["logits"], t["hidden"], t["A"], t["Bt"], t["W"], t["prev"], 16,
                        walk="greedy")
    assert torch.equal(p1, p2)
    assert torch.allclose(s1, s2, rtol=1e-6, atol=1e-6)


# ----------------------------------------------------------- sampling walk
def uniforms(B, P, seed):
    return np.random.default_rng(seed).random((B, P))


def f32_uniforms(u):
    """The uniforms as the GPU sees them (fp32), widened back for the oracle."""
    return u.astype(np.float32)


@pytest.mark.parametrize("K,P,tau", [(16, 7, 1.0), (32, 15, 0.7), (5, 3, 2.0), (1, 4, 1.0), (64, 2, 1.0),
                                     (16, 64, 1.0), (64, 64, 1.5), (3, 17, 0.3)])
def test_sample_stage(K, P, tau):
    say("sample walk K=%d P=%d tau=%g" % (K, P, tau))
    rng = np.random.default_rng(K * 100 + P + 11)
    B = 9
    S = (rng.standard_normal((B, P, K, K)) * 2).astype(np.float32)
    S[:, 0, 1:, :] = S[:, 0, :1, :]
    cand = rng.integers(0, 1 << 20, size=(B, P, K)).astype(np.int32)
    u = f32_uniforms(uniforms(B, P, K + P))
    path, q, score = df2.sample_walk(torch.from_numpy(S).cuda(), torch.from_numpy(cand).cuda(),
                                     torch.from_numpy(u).cuda(), tau)
    Sd = S.astype(np.float64)
    pr, pt, qr, sc = oracle.sample(Sd, cand, u.astype(np.float64), tau)
    o = dict(cand=cand, S=Sd, sigma=np.abs(Sd), u=u.astype(np.float64), tau=tau, sample_path=pt)
    mism = check_sample(path.cpu().numpy(), q.cpu().numpy(), score.cpu().numpy(), o, 1e-6, "stage")
    assert mism <= 1


def test_sample_stage_closed_forms():
    """u = 0 draws rank 0 at every step; a huge temperature draws rank
    floor(u K) with probability 1/K; K = 1 draws the only candidate with
    probability 1."""
    say("sample walk closed forms")
    rng = np.random.default_rng(12)
    B, P, K = 6, 9, 8
    S = torch.from_numpy(rng.standard_normal((B, P, K, K)).astype(np.float32)).cuda()
    cand = torch.from_numpy(np.tile(np.arange(K, dtype=np.int32), (B, P, 1)) + 100).cuda()
    path, q, _ = df2.sample_walk(S, cand, torch.zeros((B, P), dtype=torch.float32, device="cuda"), 1.0)
    assert torch.all(path == 100)
    u = (rng.integers(0, K, size=(B, P)) + rng.uniform(0.05, 0.95, size=(B, P))) / K
    path, q, _ = df2.sample_walk(S, cand, torch.from_numpy(u.astype(np.float32)).cuda(), 1e30)
    assert np.array_equal(path.cpu().numpy() - 100, np.floor(u * K).astype(np.int32))
    assert torch.allclose(q, torch.full_like(q, 1.0 / K), rtol=1e-6)
    S1 = S[:, :, :1, :1].contiguous()
    path, q, score = df2.sample_walk(S1, cand[:, :, :1].contiguous(),
                                     torch.from_numpy(rng.random((B, P)).astype(np.float32)).cuda(), 1.0)
    assert torch.all(path == 100) and torch.all(q == 1.0)


def gpu_select_sample(x, u, tau):
    t = to_device(x)
    path, q, score = df2.select_sample(t["logits"], t["hidden"], t["A"], t["Bt"], t["W"], t["prev"],
                                       x.wl.K, torch.from_numpy(u).cuda(), tau)
    torch.cuda.synchronize()
    return path.cpu().numpy(), q.cpu().numpy(), score.cpu().numpy()


def oracle_sample(x, u, tau, seqs=None):
    f = x.f64()
    return oracle.select(f["logits"], f["hidden"], f["A"], f["Bt"], f["W"], f["prev"], x.wl.K,
                         seqs=seqs, u=u.astype(np.float64), tau=tau)


@pytest.mark.parametrize("name,tau", [("tiny_f32", 1.0), ("qwen3_4b_b1", 1.0), ("t27b_b32", 1.0),
                                      ("t27b_b32", 0.5), ("stress_b256", 1.0)])
def test_select_sample_workloads(name, tau):
    x = inputs(name)
    say("select sample %s tau=%g B=%d P=%d V=%d K=%d" % (name, tau, x.wl.B, x.wl.P, x.wl.V, x.wl.K))
    u = f32_uniforms(uniforms(x.wl.B, x.wl.P, 99))
    path, q, score = gpu_select_sample(x, u, tau)
    if name == "stress_b256":
        assert tau == 1.0
        o = stress_oracle(x)
        assert np.array_equal(_stress["u"], u)
    else:
        o = oracle_sample(x, u, tau)
    check_sample(path, q, score, o, TOL_SAMPLE[x.wl.dtype], name)
    assert flags_clear()


@pytest.mark.parametrize("name,kw", [
    ("tiny_f32", {"pair_scale": 8.0, "V": 4000}),
    ("t27b_b8", {"pair_scale": 8.0, "V": 30000, "d": 512}),
])
def test_select_sample_pair_dominant(name, kw):
    x = inputs(name, **kw)
    say("select sample pair-dominant %s %s" % (name, kw))
    u = f32_uniforms(uniforms(x.wl.B, x.wl.P, 7))
    path, q, score = gpu_select_sample(x, u, 1.0)
    check_sample(path, q, score, oracle_sample(x, u, 1.0), TOL_SAMPLE[x.wl.dtype], name)


@pytest.mark.parametrize("B,P,V,K,d", [(1, 1, 5000, 16, 64), (3, 64, 3000, 16, 64),
                                       (2, 5, 64, 64, 64), (2, 4, 300, 1, 64),
                                       (4, 7, 9999, 3, 96), (33, 7, 2048, 16, 64)])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_select_sample_edge_shapes(B, P, V, K, d, dtype):
    say("select sample edge %s B=%d P=%d V=%d K=%d d=%d" % (dtype, B, P, V, K, d))
    wl = synth.Workload("edge", 1, B=B, P=P, V=V, d=d, K=K, r=64, dtype=dtype, pair_scale=4.0)
    x = synth.make_inputs(wl, seed=B * 1000 + P * 10 + K + 9)
    u = f32_uniforms(uniforms(B, P, B + P + K))
    path, q, score = gpu_select_sample(x, u, 1.0)
    check_sample(path, q, score, oracle_sample(x, u, 1.0), TOL_SAMPLE[dtype], "sample edge")


def test_sample_stages_compose_to_select():
    """topk -> project -> pair_scores -> sample_walk gives the fused draw bit for bit."""
    x = inputs("qwen3_4b_b1")
    say("sample stages compose")
    t = to_device(x)
    u = torch.from_numpy(f32_uniforms(uniforms(x.wl.B, x.wl.P, 5))).cuda()
    idx, val = df2.topk(t["logits"], 16)
    H = df2.project(t["hidden"], t["W"])
    S = df2.pair_scores(idx, val, H, t["A"], t["Bt"], t["prev"])
    p1, q1, s1 = df2.sample_walk(S, idx, u, 0.8)
    p2, q2, s2 = df2.select_sample(t["logits"], t["hidden"], t["A"], t["Bt"], t["W"], t["prev"], 16,
                                   u, 0.8)
    assert torch.equal(p1, p2)
    assert torch.allclose(q1, q2, rtol=1e-6, atol=0)
    assert torch.allclose(s1, s2, rtol=1e-6, atol=1e-6)


def test_sample_draw_frequencies_follow_q():
    """Many draws over one score table (one uniform grid per step): the share
    of draws of each candidate at t = 0 follows the oracle's q within 1/N."""
    say("sample draw frequencies")
    rng = np.random.default_rng(31)
    N, P, K = 4096, 2, 16
    S1 = (rng.standard_normal((1, P, K, K)) * 1.5).astype(np.float32)
    S1[:, 0, 1:, :] = S1[:, 0, :1, :]
    S = np.repeat(S1, N, axis=0)
    cand = np.tile(np.arange(K, dtype=np.int32), (N, P, 1))
    u = np.stack([(np.arange(N) + 0.5) / N, rng.random(N)], axis=1).astype(np.float32)
    path, q, _ = df2.sample_walk(torch.from_numpy(S).cuda(), torch.from_numpy(cand).cuda(),
                                 torch.from_numpy(u).cuda(), 1.0)
    counts = np.bincount(path.cpu().numpy()[:, 0], minlength=K)
    row = S1[0, 0, 0].astype(np.float64)
    e = np.exp(row - row.max())
    qr = e / e.sum()
    assert np.all(np.abs(counts - N * qr) <= 2.0), (counts, N * qr)


def test_select_graph_replay():
    """A select call captured in a HIP graph (its stream warmed first, so the
    capture holds no allocation and no memset) gives the eager result on
    every replay, with eager work on another stream between replays."""
    say("select graph replay")
    x = inputs("qwen3_4b_b1")
    t = to_device(x)
    other = to_device(synth.make_inputs(synth.WORKLOADS["tiny_f32"].with_(V=5000)))
    gs = torch.cuda.Stream()
    with torch.cuda.stream(gs):
        call = df2.PreparedSelect(t["logits"], t["hidden"], t["A"], t["Bt"], t["W"], t["prev"], x.wl.K)
        for _ in range(3):
            call()
    gs.synchronize()
    ref = (call.out_path.clone(), call.out_score.clone())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=gs):
        call()
    for i in range(5):
        call.out_path.zero_()
        call.out_score.zero_()
        df2.select(other["logits"], other["hidden"], other["A"], other["Bt"], other["W"], other["prev"], 16)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(call.out_path, ref[0]) and torch.equal(call.out_score, ref[1]), i
    assert flags_clear()
