"""Brute-force reference used to pin the oracle (tiny inputs only).

Written independently of oracle/: a different sort (numpy lexsort), numpy
matmul for the gate, and plain enumeration of every candidate path instead of
dynamic programming.  It scores each path straight from token ids with the
pair-score equation of "DFlash 2: Keep Drafting Parallel", section "A
Lightweight Path Selector": the path b_0 .. b_{P-1} with b_{-1} = prev_tok
scores sum_t U_t(b_t) + <A(b_{t-1}) * H_t, B(b_t)>.

Tie rule among equal best scores: the reverse-lexicographically smallest rank
sequence (compare the last position first), which is what a max-sum pass with
smallest-index tie breaks returns.
"""
from __future__ import annotations

import itertools

import numpy as np


def topk_lexsort(x: np.ndarray, K: int):
    """Top-K of each row by (value desc, index asc) using numpy.lexsort."""
    x = np.asarray(x, dtype=np.float64)
    V = x.shape[-1]
    flat = x.reshape(-1, V)
    idx = np.empty((flat.shape[0], K), dtype=np.int64)
    for n, row in enumerate(flat):
        # lexsort sorts by the last key first: primary key -value, then index.
        # Adding 0.0 maps -0.0 to +0.0 so both compare equal, as IEEE does.
        order = np.lexsort((np.arange(V), -(row + 0.0)))
        idx[n] = order[:K]
    idx = idx.reshape(x.shape[:-1] + (K,))
    val = np.take_along_axis(x, idx, axis=-1)
    return idx, val


def enumerate_paths(logits, hidden, A, Bt, W, prev, K):
    """Return per sequence: best token path, best rank path, best score,
    second-best score, and a list of all (rank_path, score)."""
    logits = np.asarray(logits, dtype=np.float64)
    B, P, _ = logits.shape
    cand, U = topk_lexsort(logits, K)
    H = np.matmul(np.asarray(hidden, dtype=np.float64), np.asarray(W, dtype=np.float64).T)
    A = np.asarray(A, dtype=np.float64)
    Bt = np.asarray(Bt, dtype=np.float64)
    out = []
    for b in range(B):
        scored = []
        for ranks in itertools.product(range(K), repeat=P):
            toks = [int(cand[b, t, ranks[t]]) for t in range(P)]
            s = 0.0
            pred = int(prev[b])
            for t in range(P):
                s += U[b, t, ranks[t]] + float(np.sum(A[pred] * H[b, t] * Bt[toks[t]]))
                pred = toks[t]
            scored.append((ranks, s))
        best = max(s for _, s in scored)
        ties = [rk for rk, s in scored if s == best]
        best_ranks = min(ties, key=lambda rk: tuple(reversed(rk)))
        others = [s for rk, s in scored if rk != best_ranks]
        second = max(others) if others else -np.inf
        out.append(dict(
            ranks=np.array(best_ranks, dtype=np.int64),
            path=np.array([cand[b, t, best_ranks[t]] for t in range(P)], dtype=np.int64),
            score=best, second=second, all=scored, cand=cand[b], U=U[b], H=H[b]))
    return out


def greedy_from_ids(logits, hidden, A, Bt, W, prev, K):
    """Left-to-right greedy walk scored straight from token ids.

    At each position, every candidate is scored with the pair-score equation
    against the token chosen one step earlier (prev_tok before the first
    position); the largest step score wins, the lower rank on ties.  Returns
    per sequence (ranks, tokens, score), the score summed from t = 0."""
    logits = np.asarray(logits, dtype=np.float64)
    B, P, _ = logits.shape
    cand, U = topk_lexsort(logits, K)
    H = np.matmul(np.asarray(hidden, dtype=np.float64), np.asarray(W, dtype=np.float64).T)
    A = np.asarray(A, dtype=np.float64)
    Bt = np.asarray(Bt, dtype=np.float64)
    out = []
    for b in range(B):
        pred = int(prev[b])
        ranks, toks, total = [], [], 0.0
        for t in range(P):
            steps = [U[b, t, j] + float(np.sum(A[pred] * H[b, t] * Bt[int(cand[b, t, j])]))
                     for j in range(K)]
            best = max(steps)
            j = steps.index(best)          # first (lowest-rank) maximiser
            ranks.append(j)
            toks.append(int(cand[b, t, j]))
            total += best
            pred = toks[-1]
        out.append(dict(ranks=np.array(ranks, dtype=np.int64),
                        path=np.array(toks, dtype=np.int64), score=total))
    return out


def sample_from_ids(logits, hidden, A, Bt, W, prev, K, u, tau):
    """Sampling walk scored straight from token ids: at each position the
    step scores of every candidate (pair-score equation against the token
    chosen one step earlier) go through scipy's softmax at temperature tau,
    and u[b, t] picks by inverse CDF (numpy searchsorted on the cumulative
    sum: the first j whose cumulative probability exceeds u)."""
    from scipy.special import softmax
    logits = np.asarray(logits, dtype=np.float64)
    B, P, _ = logits.shape
    cand, U = topk_lexsort(logits, K)
    H = np.matmul(np.asarray(hidden, dtype=np.float64), np.asarray(W, dtype=np.float64).T)
    A = np.asarray(A, dtype=np.float64)
    Bt = np.asarray(Bt, dtype=np.float64)
    out = []
    for b in range(B):
        pred = int(prev[b])
        ranks, toks, probs, total = [], [], [], 0.0
        for t in range(P):
            steps = np.array([U[b, t, j] + float(np.sum(A[pred] * H[b, t] * Bt[int(cand[b, t, j])]))
                              for j in range(K)])
            q = softmax(steps / tau)
            j = int(np.searchsorted(np.cumsum(q), u[b, t], side="right"))
            if j >= K:
                j = int(np.nonzero(q > 0)[0][-1])
            ranks.append(j)
            toks.append(int(cand[b, t, j]))
            probs.append(float(q[j]))
            total += steps[j]
            pred = toks[-1]
        out.append(dict(ranks=np.array(ranks, dtype=np.int64), path=np.array(toks, dtype=np.int64),
                        prob=np.array(probs), score=total))
    return out
