"""Pins for the CPU oracle: each check compares it with something other than
itself -- brute-force enumeration, closed forms, exact integer arithmetic, an
independent sort, or hand-worked fixtures under tests/golden/.

Method: "DFlash 2: Keep Drafting Parallel", section "A Lightweight Path
Selector": top-16 candidates per position, pair score
S_t(a,b) = U_t(b) + <A(a) * H(h_t), B(b)>, one walk from the last verified
token (read as max-sum Viterbi with backtrack; the literal greedy walk is a
second mode).
"""
import glob
import os

import numpy as np
import pytest

import oracle
from brute import enumerate_paths, greedy_from_ids, sample_from_ids, topk_lexsort
from golden.golden_io import read_fixture

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def rand_case(rng, B, P, V, d, r, K, pair=1.0, integer=False):
    if integer:
        logits = rng.integers(-4, 5, size=(B, P, V)).astype(np.float64)
        hidden = rng.integers(-2, 3, size=(B, P, d)).astype(np.float64)
        W = rng.integers(-2, 3, size=(r, d)).astype(np.float64)
        A = rng.integers(-2, 3, size=(V, r)).astype(np.float64)
        Bt = rng.integers(-2, 3, size=(V, r)).astype(np.float64)
    else:
        logits = rng.standard_normal((B, P, V))
        hidden = rng.standard_normal((B, P, d))
        W = rng.standard_normal((r, d)) / np.sqrt(d)
        A = rng.standard_normal((V, r)) * pair
        Bt = rng.standard_normal((V, r)) * pair
    prev = rng.integers(0, V, size=B).astype(np.int32)
    return dict(logits=logits, hidden=hidden, W=W, A=A, Bt=Bt, prev=prev)


def run_oracle(c, K):
    return oracle.select(c["logits"], c["hidden"], c["A"], c["Bt"], c["W"], c["prev"], K)


# ---------------------------------------------------------------- golden files
@pytest.mark.parametrize("path", sorted(glob.glob(os.path.join(GOLDEN, "*.txt"))),
                         ids=lambda p: os.path.basename(p))
def test_golden_fixture(path):
    fx, exp = read_fixture(path)
    o = oracle.select(fx["logits"], fx["hidden"], fx["A"], fx["Bt"], fx["W"], fx["prev"], fx["K"])
    assert o["cand"].ravel().tolist() == [int(x) for x in exp["cand"]]
    assert np.array_equal(o["U"].ravel(), np.array(exp["U"]))
    assert o["path"].ravel().tolist() == [int(x) for x in exp["path"]]
    assert o["path_rank"].ravel().tolist() == [int(x) for x in exp["path_rank"]]
    assert o["score"][0] == exp["score"][0]
    assert o["second"][0] == exp["second"][0]
    # the brute-force enumeration agrees with the stored (hand-derived) values
    bf = enumerate_paths(fx["logits"], fx["hidden"], fx["A"], fx["Bt"], fx["W"], fx["prev"], fx["K"])
    assert bf[0]["path"].tolist() == [int(x) for x in exp["path"]]
    assert bf[0]["score"] == exp["score"][0]
    assert bf[0]["second"] == exp["second"][0]
    # the greedy walk, where the fixture derives it by hand
    if "greedy_path" in exp:
        assert o["greedy_path"].ravel().tolist() == [int(x) for x in exp["greedy_path"]]
        assert o["greedy_rank"].ravel().tolist() == [int(x) for x in exp["greedy_rank"]]
        assert o["greedy_score"][0] == exp["greedy_score"][0]
        gb = greedy_from_ids(fx["logits"], fx["hidden"], fx["A"], fx["Bt"], fx["W"], fx["prev"],
                             fx["K"])
        assert gb[0]["path"].tolist() == [int(x) for x in exp["greedy_path"]]
        assert gb[0]["score"] == exp["greedy_score"][0]


# ---------------------------------------------------------- brute force: paths
@pytest.mark.parametrize("seed", range(6))
@pytest.mark.parametrize("K,P", [(2, 5), (3, 4), (4, 3), (4, 5), (1, 4), (3, 1)])
def test_viterbi_matches_enumeration_random(seed, K, P):
    rng = np.random.default_rng(1000 * seed + 10 * K + P)
    c = rand_case(rng, B=2, P=P, V=37, d=12, r=8, K=K, pair=1.5)
    o = run_oracle(c, K)
    bf = enumerate_paths(c["logits"], c["hidden"], c["A"], c["Bt"], c["W"], c["prev"], K)
    for b in range(2):
        assert o["path"][b].tolist() == bf[b]["path"].tolist()
        assert o["path_rank"][b].tolist() == bf[b]["ranks"].tolist()
        assert o["score"][b] == pytest.approx(bf[b]["score"], rel=1e-12, abs=1e-12)
        if K == 1:
            assert o["second"][b] == -np.inf
        else:
            assert o["second"][b] == pytest.approx(bf[b]["second"], rel=1e-12, abs=1e-12)


@pytest.mark.parametrize("seed", range(8))
def test_viterbi_matches_enumeration_integer_ties(seed):
    """Small integers make every sum exact and produce many exact ties, so
    the tie rules (smallest predecessor rank, smallest final rank) are
    checked bit for bit against the enumeration's reverse-lexicographic
    choice."""
    rng = np.random.default_rng(77 + seed)
    K, P = 3, 4
    c = rand_case(rng, B=3, P=P, V=9, d=4, r=4, K=K, integer=True)
    o = run_oracle(c, K)
    bf = enumerate_paths(c["logits"], c["hidden"], c["A"], c["Bt"], c["W"], c["prev"], K)
    for b in range(3):
        assert o["path_rank"][b].tolist() == bf[b]["ranks"].tolist()
        assert o["path"][b].tolist() == bf[b]["path"].tolist()
        assert o["score"][b] == bf[b]["score"]
        assert o["second"][b] == bf[b]["second"]


def test_pair_scores_match_enumeration_terms():
    """Every entry of S equals the pair score written from token ids."""
    rng = np.random.default_rng(5)
    K, P = 3, 3
    c = rand_case(rng, B=2, P=P, V=15, d=6, r=5, K=K)
    o = run_oracle(c, K)
    cand, U = topk_lexsort(c["logits"], K)
    H = c["hidden"] @ c["W"].T
    for b in range(2):
        for t in range(P):
            for i in range(K):
                a = c["prev"][b] if t == 0 else cand[b, t - 1, i]
                for j in range(K):
                    want = U[b, t, j] + np.dot(c["A"][a] * H[b, t], c["Bt"][cand[b, t, j]])
                    assert o["S"][b, t, i, j] == pytest.approx(want, rel=1e-13, abs=1e-13)


# ----------------------------------------------------------------- closed forms
@pytest.mark.parametrize("zero", ["A", "Bt", "W"])
def test_zero_pair_term_gives_independent_top1(zero):
    rng = np.random.default_rng(11)
    K, P = 16, 7
    c = rand_case(rng, B=3, P=P, V=500, d=32, r=16, K=K)
    c[zero] = np.zeros_like(c[zero])
    o = run_oracle(c, K)
    top1 = np.argmax(c["logits"], axis=-1)
    assert np.array_equal(o["path"], top1)
    assert np.allclose(o["score"], c["logits"].max(axis=-1).sum(axis=-1), rtol=0, atol=1e-12)


def test_k1_is_top1():
    rng = np.random.default_rng(12)
    c = rand_case(rng, B=2, P=6, V=300, d=16, r=8, K=1, pair=3.0)
    o = run_oracle(c, 1)
    assert np.array_equal(o["path"], np.argmax(c["logits"], axis=-1))
    assert np.all(o["second"] == -np.inf)


def test_p1_is_argmax_of_first_row():
    rng = np.random.default_rng(13)
    K = 8
    c = rand_case(rng, B=4, P=1, V=200, d=16, r=8, K=K, pair=3.0)
    o = run_oracle(c, K)
    cand, U = topk_lexsort(c["logits"], K)
    H = c["hidden"] @ c["W"].T
    for b in range(4):
        s = [U[b, 0, j] + np.dot(c["A"][c["prev"][b]] * H[b, 0], c["Bt"][cand[b, 0, j]])
             for j in range(K)]
        assert o["path"][b, 0] == cand[b, 0, int(np.argmax(s))]


def test_one_hot_tables_integer_closed_form():
    """A[v] = B[v] = e_{v mod r} and H = 1 give S_t(a,b) = U_t(b) + [a = b mod r]."""
    V, r, d, K, P = 40, 8, 4, 5, 4
    rng = np.random.default_rng(14)
    logits = rng.integers(-3, 4, size=(1, P, V)).astype(np.float64)
    A = np.zeros((V, r))
    A[np.arange(V), np.arange(V) % r] = 1.0
    W = np.zeros((r, d))
    W[:, 0] = 1.0
    hidden = np.zeros((1, P, d))
    hidden[..., 0] = 1.0
    prev = np.array([3], dtype=np.int32)
    o = oracle.select(logits, hidden, A, A.copy(), W, prev, K)
    assert np.array_equal(o["H"], np.ones((1, P, r)))
    cand, U = o["cand"], o["U"]
    for t in range(P):
        for i in range(K):
            a = prev[0] if t == 0 else cand[0, t - 1, i]
            for j in range(K):
                want = U[0, t, j] + (1.0 if (a % r) == (cand[0, t, j] % r) else 0.0)
                assert o["S"][0, t, i, j] == want


def test_logit_shift_invariance():
    """Adding c_t to every logit of position t keeps the path and shifts the
    score by sum_t c_t (integer case: exact)."""
    rng = np.random.default_rng(15)
    K, P = 4, 5
    c = rand_case(rng, B=2, P=P, V=30, d=5, r=4, K=K, integer=True)
    o1 = run_oracle(c, K)
    shift = np.array([3.0, -2.0, 7.0, 0.0, -5.0])
    c2 = dict(c)
    c2["logits"] = c["logits"] + shift[None, :, None]
    o2 = run_oracle(c2, K)
    assert np.array_equal(o1["path"], o2["path"])
    assert np.array_equal(o2["score"], o1["score"] + shift.sum())


def test_score_scale_invariance():
    """Scaling logits and the pair term by the same lambda > 0 keeps the path."""
    rng = np.random.default_rng(16)
    K, P = 4, 5
    c = rand_case(rng, B=2, P=P, V=30, d=5, r=4, K=K, integer=True)
    o1 = run_oracle(c, K)
    c2 = dict(c)
    c2["logits"] = c["logits"] * 4.0
    c2["A"] = c["A"] * 4.0   # pair term is linear in A
    o2 = run_oracle(c2, K)
    assert np.array_equal(o1["path"], o2["path"])
    assert np.array_equal(o2["score"], o1["score"] * 4.0)


# -------------------------------------------------------------------- top-K
@pytest.mark.parametrize("K", [1, 5, 16, 32, 64])
def test_topk_matches_lexsort(K):
    rng = np.random.default_rng(17 + K)
    # bf16-like coarse values to create many ties at the boundary
    x = np.round(rng.standard_normal((6, 3000)) * 8) / 8
    idx, val = oracle.topk(x, K)
    idx2, val2 = topk_lexsort(x, K)
    assert np.array_equal(idx, idx2)
    assert np.array_equal(val, val2)


def test_topk_constant_row_is_lowest_indices():
    x = np.full((2, 1000), 1.5)
    idx, val = oracle.topk(x, 16)
    assert np.array_equal(idx, np.tile(np.arange(16), (2, 1)))
    assert np.all(val == 1.5)


def test_topk_distinct_peaks():
    rng = np.random.default_rng(18)
    x = rng.standard_normal((3, 5000))
    peaks = rng.choice(5000, size=16, replace=False)
    x[:, peaks] = 100.0 + np.arange(16)[::-1]
    idx, _ = oracle.topk(x, 16)
    for row in idx:
        assert row.tolist() == peaks.tolist()


def test_topk_count_property():
    """Every unselected value is below the K-th, or equal to it at a higher index."""
    rng = np.random.default_rng(19)
    x = np.round(rng.standard_normal((4, 2000)) * 4) / 4
    K = 16
    idx, val = oracle.topk(x, K)
    for n in range(4):
        sel = set(idx[n].tolist())
        kth_v, kth_i = val[n, -1], idx[n, -1]
        for v in range(2000):
            if v in sel:
                continue
            assert x[n, v] < kth_v or (x[n, v] == kth_v and v > kth_i)


# ---------------------------------------------------------------- projection
def test_project_integer_exact_and_matmul():
    rng = np.random.default_rng(20)
    h = rng.integers(-3, 4, size=(5, 7, 64)).astype(np.float64)
    W = rng.integers(-3, 4, size=(16, 64)).astype(np.float64)
    H = oracle.project(h, W)
    assert np.array_equal(H, np.einsum("btm,qm->btq", h, W))
    hr = rng.standard_normal((3, 40))
    Wr = rng.standard_normal((12, 40))
    assert np.allclose(oracle.project(hr, Wr), hr @ Wr.T, rtol=1e-13, atol=1e-13)


def test_margin_zero_on_exact_tie():
    """Two identical candidates' scores (duplicate logits, zero pair term)
    tie exactly, so the second-best equals the best."""
    V, P, K = 10, 3, 2
    logits = np.zeros((1, P, V))
    logits[0, :, 4] = 2.0
    logits[0, :, 7] = 2.0
    z = np.zeros
    o = oracle.select(logits, z((1, P, 3)), z((V, 2)), z((V, 2)), z((2, 3)),
                      np.array([0], dtype=np.int32), K)
    assert o["path"][0].tolist() == [4, 4, 4]
    assert o["margin"][0] == 0.0


# ------------------------------------------------------------------ greedy walk
@pytest.mark.parametrize("seed", range(6))
@pytest.mark.parametrize("K,P", [(2, 5), (4, 3), (5, 6), (16, 4), (1, 3), (3, 1)])
def test_greedy_matches_step_scores_from_ids(seed, K, P):
    """The oracle's greedy walk (over its S table) against a walk that scores
    each step straight from token ids."""
    rng = np.random.default_rng(3000 * seed + 10 * K + P)
    c = rand_case(rng, B=3, P=P, V=61, d=12, r=8, K=K, pair=1.5)
    o = run_oracle(c, K)
    gb = greedy_from_ids(c["logits"], c["hidden"], c["A"], c["Bt"], c["W"], c["prev"], K)
    for b in range(3):
        assert o["greedy_rank"][b].tolist() == gb[b]["ranks"].tolist()
        assert o["greedy_path"][b].tolist() == gb[b]["path"].tolist()
        assert o["greedy_score"][b] == pytest.approx(gb[b]["score"], rel=1e-12, abs=1e-12)


@pytest.mark.parametrize("seed", range(8))
def test_greedy_integer_ties(seed):
    """Exact integer scores with many ties: the lower rank must win each step."""
    rng = np.random.default_rng(500 + seed)
    K, P = 4, 5
    c = rand_case(rng, B=3, P=P, V=9, d=4, r=4, K=K, integer=True)
    o = run_oracle(c, K)
    gb = greedy_from_ids(c["logits"], c["hidden"], c["A"], c["Bt"], c["W"], c["prev"], K)
    for b in range(3):
        assert o["greedy_rank"][b].tolist() == gb[b]["ranks"].tolist()
        assert o["greedy_score"][b] == gb[b]["score"]


@pytest.mark.parametrize("seed", range(4))
def test_greedy_is_one_of_the_enumerated_paths_and_never_beats_viterbi(seed):
    """Greedy's score is the enumerated score of its own path, and no greater
    than the best path's."""
    rng = np.random.default_rng(40 + seed)
    K, P = 3, 4
    c = rand_case(rng, B=2, P=P, V=23, d=8, r=6, K=K, pair=2.0)
    o = run_oracle(c, K)
    bf = enumerate_paths(c["logits"], c["hidden"], c["A"], c["Bt"], c["W"], c["prev"], K)
    for b in range(2):
        table = {tuple(rk): sc for rk, sc in bf[b]["all"]}
        own = table[tuple(int(x) for x in o["greedy_rank"][b])]
        assert o["greedy_score"][b] == pytest.approx(own, rel=1e-12, abs=1e-12)
        assert o["greedy_score"][b] <= bf[b]["score"] + 1e-12


@pytest.mark.parametrize("zero", ["A", "Bt", "W"])
def test_greedy_zero_pair_term_is_top1(zero):
    """Without the pair term each step is the top-1 candidate, as for Viterbi."""
    rng = np.random.default_rng(21)
    K, P = 16, 7
    c = rand_case(rng, B=3, P=P, V=500, d=32, r=16, K=K)
    c[zero] = np.zeros_like(c[zero])
    o = run_oracle(c, K)
    top1 = np.argmax(c["logits"], axis=-1)
    assert np.array_equal(o["greedy_path"], top1)
    assert np.array_equal(o["greedy_path"], o["path"])
    assert np.allclose(o["greedy_score"], c["logits"].max(axis=-1).sum(axis=-1), rtol=0, atol=1e-12)


def test_greedy_k1_and_p1():
    """K = 1 leaves one path; P = 1 makes greedy and Viterbi the same argmax."""
    rng = np.random.default_rng(22)
    c = rand_case(rng, B=2, P=5, V=300, d=16, r=8, K=1, pair=3.0)
    o = run_oracle(c, 1)
    assert np.array_equal(o["greedy_path"], np.argmax(c["logits"], axis=-1))
    assert np.array_equal(o["greedy_score"], o["score"])
    c = rand_case(rng, B=4, P=1, V=200, d=16, r=8, K=8, pair=3.0)
    o = run_oracle(c, 8)
    assert np.array_equal(o["greedy_path"], o["path"])
    assert np.array_equal(o["greedy_score"], o["score"])


# ---------------------------------------------------------------- sampling walk
def run_sample(c, K, u, tau):
    return oracle.select(c["logits"], c["hidden"], c["A"], c["Bt"], c["W"], c["prev"], K,
                         u=u, tau=tau)


@pytest.mark.parametrize("seed", range(4))
@pytest.mark.parametrize("K,P,tau", [(2, 5, 1.0), (4, 3, 0.5), (5, 6, 2.0), (16, 4, 1.0), (1, 3, 1.0),
                                     (3, 1, 0.7)])
def test_sample_matches_softmax_walk_from_ids(seed, K, P, tau):
    rng = np.random.default_rng(7000 * seed + 10 * K + P)
    c = rand_case(rng, B=3, P=P, V=61, d=12, r=8, K=K, pair=1.5)
    u = rng.random((3, P))
    o = run_sample(c, K, u, tau)
    sb = sample_from_ids(c["logits"], c["hidden"], c["A"], c["Bt"], c["W"], c["prev"], K, u, tau)
    for b in range(3):
        assert o["sample_rank"][b].tolist() == sb[b]["ranks"].tolist()
        assert o["sample_path"][b].tolist() == sb[b]["path"].tolist()
        np.testing.assert_allclose(o["sample_prob"][b], sb[b]["prob"], rtol=1e-12, atol=1e-15)
        assert o["sample_score"][b] == pytest.approx(sb[b]["score"], rel=1e-12, abs=1e-12)


def test_sample_frequencies_on_a_grid_of_uniforms():
    """One position, N evenly spaced uniforms: rank j is drawn by
    N * q_j (+-1) of them, q from numpy's exp of the step scores."""
    rng = np.random.default_rng(17)
    K, N, tau = 6, 5000, 0.8
    c = rand_case(rng, B=1, P=1, V=40, d=8, r=8, K=K, pair=1.0)
    rep = {k: (np.repeat(v, N, axis=0) if k in ("logits", "hidden", "prev") else v) for k, v in c.items()}
    u = ((np.arange(N) + 0.5) / N).reshape(N, 1)
    o = run_sample(rep, K, u, tau)
    cand, U = topk_lexsort(c["logits"], K)
    H = c["hidden"][0, 0] @ c["W"].T
    s = np.array([U[0, 0, j] + np.dot(c["A"][c["prev"][0]] * H, c["Bt"][cand[0, 0, j]]) for j in range(K)])
    e = np.exp((s - s.max()) / tau)
    q = e / e.sum()
    counts = np.bincount(o["sample_rank"][:, 0], minlength=K)
    assert np.all(np.abs(counts - N * q) <= 1.0), (counts, N * q)
    np.testing.assert_allclose(o["sample_prob"][:, 0], q[o["sample_rank"][:, 0]], rtol=1e-12)


def test_sample_zero_uniform_takes_rank0():
    """u = 0 draws the first candidate with positive probability: rank 0."""
    rng = np.random.default_rng(18)
    K, P = 8, 6
    c = rand_case(rng, B=2, P=P, V=100, d=8, r=8, K=K, pair=2.0)
    o = run_sample(c, K, np.zeros((2, P)), 1.0)
    assert np.all(o["sample_rank"] == 0)
    for b in range(2):
        assert o["sample_score"][b] == pytest.approx(sum(o["S"][b, t, 0, 0] for t in range(P)), rel=1e-14)


def test_sample_small_temperature_is_greedy():
    rng = np.random.default_rng(19)
    K, P = 16, 7
    c = rand_case(rng, B=4, P=P, V=300, d=16, r=8, K=K, pair=2.0)
    o = run_sample(c, K, rng.random((4, P)), 1e-9)
    assert np.array_equal(o["sample_rank"], o["greedy_rank"])
    assert np.all(o["sample_prob"] == 1.0)
    np.testing.assert_allclose(o["sample_score"], o["greedy_score"], rtol=1e-14)


def test_sample_large_temperature_is_uniform():
    """tau -> infinity: every candidate has probability 1/K, so u picks
    rank floor(u * K) (uniforms kept away from the k / K boundaries)."""
    rng = np.random.default_rng(20)
    K, P = 5, 6
    c = rand_case(rng, B=4, P=P, V=100, d=8, r=8, K=K, pair=2.0)
    u = (rng.integers(0, K, size=(4, P)) + rng.uniform(0.05, 0.95, size=(4, P))) / K
    o = run_sample(c, K, u, 1e15)
    assert np.array_equal(o["sample_rank"], np.floor(u * K).astype(np.int32))
    np.testing.assert_allclose(o["sample_prob"], 1.0 / K, rtol=1e-9)


def test_sample_hand_lattice():
    """greedy_trap_k2_p2.txt worked by hand at tau = 1 with u = (0.8, 0.5):
    S_0 = (5, 4): q = (1/(1+e^-1), 1/(1+e)); 0.8 > 0.731 -> rank 1 (token 1);
    row 1 of S_1 = (10, 5): q_0 = 1/(1+e^-5) = 0.9933 > 0.5 -> rank 0 (token 2);
    score 4 + 10 = 14."""
    fx, _ = read_fixture(os.path.join(GOLDEN, "greedy_trap_k2_p2.txt"))
    o = oracle.select(fx["logits"], fx["hidden"], fx["A"], fx["Bt"], fx["W"], fx["prev"], fx["K"],
                      u=np.array([[0.8, 0.5]]), tau=1.0)
    assert o["sample_rank"][0].tolist() == [1, 0]
    assert o["sample_path"][0].tolist() == [1, 2]
    assert o["sample_prob"][0][0] == pytest.approx(1.0 / (1.0 + np.e), rel=1e-14)
    assert o["sample_prob"][0][1] == pytest.approx(1.0 / (1.0 + np.exp(-5.0)), rel=1e-14)
    assert o["sample_score"][0] == 14.0


def test_sample_k1_probability_one():
    rng = np.random.default_rng(21)
    c = rand_case(rng, B=2, P=4, V=50, d=8, r=8, K=1)
    o = run_sample(c, 1, rng.random((2, 4)), 1.0)
    assert np.array_equal(o["sample_path"], np.argmax(c["logits"], axis=-1))
    assert np.all(o["sample_prob"] == 1.0)
