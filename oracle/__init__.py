"""CPU oracle for the DFlash 2 path selector (ctypes wrapper over oracle.c).

TEST INFRASTRUCTURE ONLY: imported by tests/, by __graft_entry__.smoke() and
by bench.py's cpu_baseline leg.  The GPU product path never imports it.

All arithmetic is float64 on inputs widened exactly from their storage type.
The steps follow "DFlash 2: Keep Drafting Parallel", section "A Lightweight
Path Selector" (top-16 candidates, the pair-score equation, one walk from the
last verified token); the walk is read as max-sum Viterbi with backtrack, the
literal greedy walk and the sampling walk are further modes, and H(h_t) is
read as a bias-free linear map d -> r (see the header of oracle.c).  conv2 is
the drafter's two-tap dynamic convolution ("A Lightweight Local
Convolution"); lmhead_topk is the drafter's LM head followed by top-K, the
logits the selector starts from; philox_uniforms are the counter-based
uniforms a sampling walk consumes (Philox4x64-10, Salmon et al., SC 2011).

Every function here is pinned by CPU tests against something other than
itself (brute-force enumeration, closed forms, exact integer cases, an
independent sort, numpy's own Philox and its published known answer); none
is "parity unpinned".
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Dict, Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None


def build(force: bool = True) -> str:
    """Compile oracle.c into liboracle.so with gcc (IEEE semantics, no fast-math)."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-std=c11", "-fPIC", "-shared",
                               "-fno-fast-math", "-ffp-contract=off",
                               _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build(force=True)
        lib = ctypes.CDLL(_LIB_PATH)
        P = ctypes.c_void_p
        I = ctypes.c_int64
        lib.orc_topk.argtypes = [P, I, I, ctypes.c_int32, P, P]
        lib.orc_topk.restype = ctypes.c_int
        lib.orc_project.argtypes = [P, P, I, I, I, P]
        lib.orc_project.restype = None
        lib.orc_pair_scores.argtypes = [P, P, P, P, P, P, I, I, I, I, P, P]
        lib.orc_pair_scores.restype = None
        lib.orc_viterbi.argtypes = [P, P, I, I, I, P, P, P]
        lib.orc_viterbi.restype = ctypes.c_int
        lib.orc_greedy.argtypes = [P, P, I, I, I, P, P, P]
        lib.orc_greedy.restype = None
        lib.orc_sample.argtypes = [P, P, P, I, I, I, ctypes.c_double, P, P, P, P]
        lib.orc_sample.restype = ctypes.c_int
        lib.orc_conv2.argtypes = [P, P, P, P, I, I, I, P, P]
        lib.orc_conv2.restype = None
        lib.orc_philox4x64_10.argtypes = [P, P, P]
        lib.orc_philox4x64_10.restype = None
        lib.orc_philox_uniforms.argtypes = [ctypes.c_uint64, ctypes.c_uint64, I, I, P]
        lib.orc_philox_uniforms.restype = None
        lib.orc_second_best.argtypes = [P, P, I, I, I, P]
        lib.orc_second_best.restype = ctypes.c_int
        lib.orc_lmhead_topk.argtypes = [P, P, I, I, I, ctypes.c_int32, P, P, P]
        lib.orc_lmhead_topk.restype = ctypes.c_int
        lib.orc_lmhead_dot.argtypes = [P, P, I, P, P, I, P, P]
        lib.orc_lmhead_dot.restype = None
        _lib = lib
    return _lib


def _p(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def _f64(a) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=np.float64)


def _i32(a) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=np.int32)


def topk(x: np.ndarray, K: int):
    """Top-K per row of x[..., V]: (idx int32 [..., K], val float64 [..., K])."""
    x = _f64(x)
    V = x.shape[-1]
    rows = x.size // V if V else 0
    idx = np.empty(x.shape[:-1] + (K,), dtype=np.int32)
    val = np.empty(x.shape[:-1] + (K,), dtype=np.float64)
    if rows and _load().orc_topk(_p(x), rows, V, K, _p(idx), _p(val)) != 0:
        raise ValueError("orc_topk: bad K/V or out of memory")
    return idx, val


def project(h: np.ndarray, W: np.ndarray) -> np.ndarray:
    """H[..., q] = sum_m W[q, m] h[..., m]  (W is [r, d])."""
    h = _f64(h)
    W = _f64(W)
    r, d = W.shape
    M = h.size // d
    H = np.empty(h.shape[:-1] + (r,), dtype=np.float64)
    _load().orc_project(_p(h), _p(W), M, d, r, _p(H))
    return H


def _f32(a) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=np.float32)


def lmhead_topk(X, W, K: int, rows=None):
    """LM head then top-K (see orc_lmhead_topk): X [M, d] hidden states,
    W [V, d] LM-head weight, both holding exact fp32 or bf16 values.
    Returns (idx int32 [M', K], val float64 [M', K], sigma float64 [M', K])
    for the rows listed in `rows` (all rows when None), in that order."""
    X = _f32(X)
    W = _f32(W)
    if X.ndim != 2 or W.ndim != 2 or X.shape[1] != W.shape[1]:
        raise ValueError("lmhead_topk: X must be [M, d] and W [V, d]")
    if rows is not None:
        X = _f32(X[np.asarray(rows, dtype=np.int64)])
    M, d = X.shape
    V = W.shape[0]
    idx = np.empty((M, K), dtype=np.int32)
    val = np.empty((M, K), dtype=np.float64)
    sig = np.empty((M, K), dtype=np.float64)
    if M and _load().orc_lmhead_topk(_p(X), _p(W), M, d, V, K, _p(idx), _p(val), _p(sig)) != 0:
        raise ValueError("orc_lmhead_topk: bad K/V/d or out of memory")
    return idx, val, sig


def lmhead_dot(X, W, m, v):
    """Logits W[v_i] . X[m_i] and their scales sum |W[v_i] * X[m_i]| (float64)."""
    X = _f32(X)
    W = _f32(W)
    m = np.ascontiguousarray(m, dtype=np.int64).ravel()
    v = np.ascontiguousarray(v, dtype=np.int64).ravel()
    if m.shape != v.shape:
        raise ValueError("lmhead_dot: m and v differ in length")
    if m.size and (m.min() < 0 or m.max() >= X.shape[0] or v.min() < 0 or v.max() >= W.shape[0]):
        raise ValueError("lmhead_dot: index out of range")
    dot = np.empty(m.size, dtype=np.float64)
    absdot = np.empty(m.size, dtype=np.float64)
    if m.size:
        _load().orc_lmhead_dot(_p(X), _p(W), X.shape[1], _p(m), _p(v), m.size, _p(dot),
                               _p(absdot))
    return dot, absdot


def pair_scores(cand, U, H, A, Bt, prev):
    """S[b, t, i, j] and the tolerance scale sigma, both [B, P, K, K] float64."""
    cand = _i32(cand)
    U = _f64(U)
    H = _f64(H)
    A = _f64(A)
    Bt = _f64(Bt)
    prev = _i32(prev)
    Bn, P, K = cand.shape
    r = H.shape[-1]
    S = np.empty((Bn, P, K, K), dtype=np.float64)
    sig = np.empty((Bn, P, K, K), dtype=np.float64)
    _load().orc_pair_scores(_p(cand), _p(U), _p(H), _p(A), _p(Bt), _p(prev),
                            Bn, P, K, r, _p(S), _p(sig))
    return S, sig


def viterbi(S, cand):
    """(path_rank [B,P] int32, path_tok [B,P] int32, score [B] float64)."""
    S = _f64(S)
    cand = _i32(cand)
    Bn, P, K = cand.shape
    pr = np.empty((Bn, P), dtype=np.int32)
    pt = np.empty((Bn, P), dtype=np.int32)
    sc = np.empty(Bn, dtype=np.float64)
    if _load().orc_viterbi(_p(S), _p(cand), Bn, P, K, _p(pr), _p(pt), _p(sc)) != 0:
        raise MemoryError("orc_viterbi")
    return pr, pt, sc


def greedy(S, cand):
    """Greedy walk: (path_rank [B,P] int32, path_tok [B,P] int32, score [B] float64)."""
    S = _f64(S)
    cand = _i32(cand)
    Bn, P, K = cand.shape
    pr = np.empty((Bn, P), dtype=np.int32)
    pt = np.empty((Bn, P), dtype=np.int32)
    sc = np.empty(Bn, dtype=np.float64)
    _load().orc_greedy(_p(S), _p(cand), Bn, P, K, _p(pr), _p(pt), _p(sc))
    return pr, pt, sc


def sample(S, cand, u, tau: float):
    """Sampling walk with uniforms u [B,P] in [0, 1) at temperature tau:
    (path_rank [B,P] int32, path_tok [B,P] int32, prob [B,P] float64 = the
    chosen candidate's step probability, score [B] float64)."""
    S = _f64(S)
    cand = _i32(cand)
    u = _f64(u)
    Bn, P, K = cand.shape
    if u.shape != (Bn, P):
        raise ValueError("u must be [B, P]")
    if not (tau > 0 and np.isfinite(tau)):
        raise ValueError("tau must be positive and finite")
    pr = np.empty((Bn, P), dtype=np.int32)
    pt = np.empty((Bn, P), dtype=np.int32)
    q = np.empty((Bn, P), dtype=np.float64)
    sc = np.empty(Bn, dtype=np.float64)
    if _load().orc_sample(_p(S), _p(cand), _p(u), Bn, P, K, float(tau), _p(pr), _p(pt), _p(q),
                          _p(sc)) != 0:
        raise MemoryError("orc_sample")
    return pr, pt, q, sc


def conv2(x, x_prev, base, Wc):
    """Two-tap dynamic depthwise convolution (see orc_conv2):
    x [B,P,d], x_prev [B,d], base [2,d], Wc [2,d/16,d] -> (y, sigma) [B,P,d]."""
    x = _f64(x)
    x_prev = _f64(x_prev)
    base = _f64(base)
    Wc = _f64(Wc)
    Bn, P, d = x.shape
    if d % 16 or x_prev.shape != (Bn, d) or base.shape != (2, d) or Wc.shape != (2, d // 16, d):
        raise ValueError("conv2: inconsistent shapes")
    y = np.empty_like(x)
    sig = np.empty_like(x)
    _load().orc_conv2(_p(x), _p(x_prev), _p(base), _p(Wc), Bn, P, d, _p(y), _p(sig))
    return y, sig


def philox4x64_10(ctr, key) -> np.ndarray:
    """One Philox4x64-10 block (see orc_philox4x64_10): 4 counter words and
    2 key words in, 4 words out, all uint64."""
    c = np.ascontiguousarray(np.asarray(ctr, dtype=np.uint64).reshape(4))
    k = np.ascontiguousarray(np.asarray(key, dtype=np.uint64).reshape(2))
    out = np.zeros(4, dtype=np.uint64)
    _load().orc_philox4x64_10(_p(c), _p(k), _p(out))
    return out


def philox_uniforms(seed: int, offset: int, n: int, first: int = 0) -> np.ndarray:
    """Uniforms first .. first+n-1 of the call (seed, offset) as float32 (see
    orc_philox_uniforms: word i mod 4 of the block at counter
    (i // 4, offset, 0, 0) under key (seed, 0), mapped to (x >> 40) * 2^-24)."""
    u = np.zeros(max(int(n), 0), dtype=np.float32)
    if n > 0:
        _load().orc_philox_uniforms(int(seed) & (2**64 - 1), int(offset) & (2**64 - 1),
                                    int(first), int(n), _p(u))
    return u


def path_sigma(sig, path_rank) -> np.ndarray:
    """Sum of the tolerance scale sigma along each rank path (row 0 at t = 0)."""
    Bn, P = path_rank.shape
    out = np.zeros(Bn, dtype=np.float64)
    for b in range(Bn):
        out[b] = sig[b, 0, 0, path_rank[b, 0]] + sum(
            sig[b, t, path_rank[b, t - 1], path_rank[b, t]] for t in range(1, P))
    return out


def second_best(S, path_rank) -> np.ndarray:
    """Second-best path score per sequence (-inf when K == 1)."""
    S = _f64(S)
    path_rank = _i32(path_rank)
    Bn, P = path_rank.shape
    K = S.shape[-1]
    out = np.empty(Bn, dtype=np.float64)
    if _load().orc_second_best(_p(S), _p(path_rank), Bn, P, K, _p(out)) != 0:
        raise MemoryError("orc_second_best")
    return out


def select(logits, hidden, A, Bt, W, prev, K: int,
           seqs: Optional[np.ndarray] = None, u=None, tau: float = 1.0) -> Dict[str, np.ndarray]:
    """The whole selector on float64 inputs; returns every intermediate.

    logits [B,P,V], hidden [B,P,d], A/Bt [V,r], W [r,d], prev [B].
    `seqs` restricts the work to a subset of sequences (sampled checks on
    large workloads); outputs then follow the order of `seqs`.  With
    uniforms u [B,P] the sampling walk at temperature tau is added.
    """
    if seqs is not None:
        seqs = np.asarray(seqs, dtype=np.int64)
        logits = np.asarray(logits)[seqs]
        hidden = np.asarray(hidden)[seqs]
        prev = np.asarray(prev)[seqs]
        if u is not None:
            u = np.asarray(u)[seqs]
    cand, U = topk(logits, K)
    H = project(hidden, W)
    S, sig = pair_scores(cand, U, H, A, Bt, prev)
    pr, pt, sc = viterbi(S, cand)
    sec = second_best(S, pr)
    gr, gt, gs = greedy(S, cand)
    # scale of each path's score: sum of sigma along it (tolerance for scores)
    out = dict(cand=cand, U=U, H=H, S=S, sigma=sig, path_rank=pr, path=pt,
               score=sc, second=sec, margin=sc - sec, sigma_path=path_sigma(sig, pr),
               greedy_rank=gr, greedy_path=gt, greedy_score=gs,
               sigma_greedy=path_sigma(sig, gr))
    if u is not None:
        sr, st, sq, ss = sample(S, cand, u, tau)
        out.update(sample_rank=sr, sample_path=st, sample_prob=sq, sample_score=ss, u=np.asarray(u),
                   tau=tau)
    return out
