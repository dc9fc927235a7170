"""Pins for the oracle's LM head followed by top-K (oracle.lmhead_topk).

The selector starts from the drafter's own logits ("DFlash 2: Keep Drafting
Parallel", section "A Lightweight Path Selector": no extra LM-head pass is
needed), read here as U_t(v) = sum_k W_lm[v][k] h_t[k] followed by the
top-K order of the rest of the path (value descending, equal values to the
lower index).  Each check compares the oracle with something other than
itself: numpy's matmul on integer inputs (exact in float64) with an
independent lexicographic sort, closed forms for one-hot and planted rows,
and the absolute-product scale.
"""
import numpy as np
import pytest

import oracle
from brute import topk_lexsort


def int_case(rng, M, V, d, lo=-3, hi=3):
    X = rng.integers(lo, hi + 1, size=(M, d)).astype(np.float32)
    W = rng.integers(lo, hi + 1, size=(V, d)).astype(np.float32)
    return X, W


@pytest.mark.parametrize("M,V,d,K", [(1, 50, 32, 1), (3, 200, 64, 16), (7, 501, 96, 32),
                                     (5, 64, 64, 64)])
def test_integer_inputs_match_matmul_and_lexsort(M, V, d, K):
    rng = np.random.default_rng(1000 + M * V + d + K)
    X, W = int_case(rng, M, V, d)
    L = np.matmul(X.astype(np.float64), W.astype(np.float64).T)   # exact: small integers
    idx, val, sig = oracle.lmhead_topk(X, W, K)
    ref_idx, ref_val = topk_lexsort(L, K)
    assert np.array_equal(idx, ref_idx)
    assert np.array_equal(val, ref_val)
    # ties are exercised: the integer logits repeat inside the kept range
    if K >= 16:
        assert any(len(set(r.tolist())) < K for r in ref_val)
    # the scale is the sum of absolute products, also exact here
    S = np.matmul(np.abs(X.astype(np.float64)), np.abs(W.astype(np.float64)).T)
    assert np.array_equal(sig, np.take_along_axis(S, ref_idx, axis=1))


def test_one_hot_rows_select_a_column_of_w():
    # X[m] = c_m e_{k_m}: the logits of row m are c_m * W[:, k_m]; V == d makes
    # a transposed weight plausible, and it would select a row of W instead
    rng = np.random.default_rng(7)
    V = d = 96
    W = rng.standard_normal((V, d)).astype(np.float32)
    ks = [0, 5, 95, 40]
    cs = [1.0, -2.0, 0.5, 3.0]
    X = np.zeros((len(ks), d), dtype=np.float32)
    for m, (k, c) in enumerate(zip(ks, cs)):
        X[m, k] = c
    idx, val, _ = oracle.lmhead_topk(X, W, 8)
    for m, (k, c) in enumerate(zip(ks, cs)):
        col = c * W[:, k].astype(np.float64)
        ref_idx, ref_val = topk_lexsort(col, 8)
        assert idx[m].tolist() == ref_idx.tolist()
        assert np.array_equal(val[m], ref_val)


def test_planted_tokens_come_first_in_order():
    # X[m] = sum_j delta_j W[v_j] / |W[v_j]|^2 with well separated deltas puts
    # the planted tokens first, in order of delta (their logits are delta_j
    # plus cross terms of order |W|^-1, far below the spacing)
    rng = np.random.default_rng(11)
    V, d = 3000, 512
    W = rng.standard_normal((V, d)).astype(np.float32)
    planted = [1234, 7, 2999]
    deltas = [30.0, 20.0, 10.0]
    x = np.zeros(d)
    for v, dl in zip(planted, deltas):
        w = W[v].astype(np.float64)
        x += dl * w / np.dot(w, w)
    X = x.astype(np.float32)[None, :]
    idx, val, _ = oracle.lmhead_topk(X, W, 3)
    assert idx[0].tolist() == planted
    assert np.allclose(val[0], deltas, atol=2.0)


def test_constant_logits_give_lowest_indices():
    # every logit equal: the K lowest token ids, in order
    X = np.ones((2, 32), dtype=np.float32)
    W = np.full((40, 32), 0.25, dtype=np.float32)
    idx, val, _ = oracle.lmhead_topk(X, W, 6)
    assert idx.tolist() == [list(range(6))] * 2
    assert np.all(val == 8.0)


def test_signed_zero_logits_tie():
    # W rows of +0 and -0 give logits +0 and -0, which compare equal: order by id
    X = np.ones((1, 32), dtype=np.float32)
    W = np.zeros((6, 32), dtype=np.float32)
    W[1] = -0.0
    W[3] = -0.0
    W[4, :] = -1.0
    idx, val, _ = oracle.lmhead_topk(X, W, 5)
    assert idx[0].tolist() == [0, 1, 2, 3, 5]


def test_rows_subset_follows_given_order():
    rng = np.random.default_rng(3)
    X, W = int_case(rng, 6, 300, 64)
    full = oracle.lmhead_topk(X, W, 4)
    sub = oracle.lmhead_topk(X, W, 4, rows=[5, 0, 3])
    for a, b in zip(full, sub):
        assert np.array_equal(a[[5, 0, 3]], b)


def test_dot_matches_integer_matmul_and_topk_values():
    rng = np.random.default_rng(5)
    X, W = int_case(rng, 4, 120, 64)
    L = np.matmul(X.astype(np.float64), W.astype(np.float64).T)
    S = np.matmul(np.abs(X.astype(np.float64)), np.abs(W.astype(np.float64)).T)
    m = rng.integers(0, 4, size=50)
    v = rng.integers(0, 120, size=50)
    dot, absdot = oracle.lmhead_dot(X, W, m, v)
    assert np.array_equal(dot, L[m, v])
    assert np.array_equal(absdot, S[m, v])
    idx, val, sig = oracle.lmhead_topk(X, W, 8)
    mm = np.repeat(np.arange(4), 8)
    dot2, abs2 = oracle.lmhead_dot(X, W, mm, idx.ravel())
    assert np.array_equal(dot2, val.ravel())
    assert np.array_equal(abs2, sig.ravel())


def test_bad_sizes_raise():
    X = np.zeros((1, 32), dtype=np.float32)
    W = np.zeros((10, 32), dtype=np.float32)
    with pytest.raises(ValueError):
        oracle.lmhead_topk(X, W, 11)
    with pytest.raises(ValueError):
        oracle.lmhead_topk(X, W, 0)
    with pytest.raises(ValueError):
        oracle.lmhead_topk(X, np.zeros((10, 16), dtype=np.float32), 2)
    with pytest.raises(ValueError):
        oracle.lmhead_dot(X, W, [0], [10])
