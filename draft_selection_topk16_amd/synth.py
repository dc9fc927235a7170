"""Seeded synthetic inputs for the DFlash 2 path selector.

This module only draws random numbers and lays them out; it holds none of the
selector's arithmetic.  Both the HIP path (through the binding) and the CPU
oracle are fed from here, so that every comparison runs on the same bytes.

Workload recipes (value distributions and shapes) follow the five named
workloads of the selector: a tiny fp32 case, a Qwen3-4B-shaped drafter at
batch 1, a 27B-target-shaped drafter at concurrency 8 and 32, and a stress
sweep.  The pages ("DFlash 2: Keep Drafting Parallel", section "A Lightweight
Path Selector") fix the shape of the method: top-16 candidates per draft
position and 256-dimensional token embeddings; a block of 8 holds one verified
token and 7 draft positions (dev.to model-card article, benchmark setup).

Readings of the recipe wording:
  * "N(mu, s)" means standard deviation s; "N(0, 1/sqrt(r))" is std 1/16.
  * Peaked rows: m ~ U{1,2,3} peak tokens drawn uniformly over V, boosted by
    4 + 6/k for k = 1..m (+10, +7, +6).
  * Sequence b draws its logits, peaks and prev_tok from sub-seed
    seed * 1000 + b ("per-sequence seeded").
  * Flat rows are N(0, 1) with no peak; the saturation workload makes exactly
    round(0.2 * B * P) rows flat, chosen by a seeded permutation; the stress
    workload makes 30 % flat and, in a peaked row at t >= 1, reuses the
    previous row's top-peak token with probability 0.25.
  * Hidden states are N(0, 1) (the recipe does not state them).
bf16 tensors are produced by round-to-nearest-even from fp32 and kept as raw
uint16 bit patterns.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Dict, Optional

import numpy as np

__all__ = [
    "Workload", "WORKLOADS", "Inputs", "make_inputs", "f32_to_bf16_bits",
    "bf16_bits_to_f64", "to_f64", "ConvInputs", "CONV_WORKLOADS", "make_conv_inputs",
    "LmHeadInputs", "make_lmhead_inputs", "bf16_bits_to_f32",
]


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    wid: int            # index into WORKLOADS; base seed is 0xDF2000 + wid
    B: int              # sequences
    P: int              # draft positions (block size minus the verified token)
    V: int              # vocabulary
    d: int              # drafter hidden size
    K: int              # candidates kept per position
    r: int = 256        # embedding rank of A, B, H
    dtype: str = "bf16"     # "f32" or "bf16" for logits, hidden, A, B, W_H
    logit_kind: str = "zipf"   # "true_token" | "zipf"
    flat_frac: float = 0.0
    flat_mode: str = "exact"   # "exact": round(frac*rows) rows; "mixed": per-row draw
    dup_prob: float = 0.0
    pair_scale: float = 1.0    # multiplies A and B (test preset: pair-dominant)

    @property
    def rows(self) -> int:
        return self.B * self.P

    def with_(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


WORKLOADS: Dict[str, Workload] = {
    "tiny_f32": Workload("tiny_f32", 0, B=1, P=7, V=32000, d=1024, K=16,
                         dtype="f32", logit_kind="true_token"),
    "qwen3_4b_b1": Workload("qwen3_4b_b1", 1, B=1, P=7, V=151936, d=2560, K=16),
    "t27b_b8": Workload("t27b_b8", 2, B=8, P=7, V=151936, d=5120, K=16),
    "t27b_b32": Workload("t27b_b32", 3, B=32, P=7, V=151936, d=5120, K=16,
                         flat_frac=0.2, flat_mode="exact"),
    "stress_b256": Workload("stress_b256", 4, B=256, P=15, V=262144, d=5120, K=32,
                            flat_frac=0.3, flat_mode="mixed", dup_prob=0.25),
}


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round-to-nearest-even fp32 -> bf16, returned as uint16 bit patterns."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    bias = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((u + bias) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f64(b: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns to float64."""
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def to_f64(a: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "bf16":
        return bf16_bits_to_f64(a)
    return np.asarray(a, dtype=np.float32).astype(np.float64)


@dataclasses.dataclass
class Inputs:
    """Host arrays in storage form: float32 for "f32", uint16 bits for "bf16"."""
    wl: Workload
    logits: np.ndarray    # [B, P, V]
    hidden: np.ndarray    # [B, P, d]
    A: np.ndarray         # [V, r]
    Bt: np.ndarray        # [V, r]
    W: np.ndarray         # [r, d]
    prev: np.ndarray      # [B] int32

    def f64(self):
        dt = self.wl.dtype
        return dict(logits=to_f64(self.logits, dt), hidden=to_f64(self.hidden, dt),
                    A=to_f64(self.A, dt), Bt=to_f64(self.Bt, dt), W=to_f64(self.W, dt),
                    prev=self.prev)


def _store(x: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "bf16":
        return f32_to_bf16_bits(x)
    return np.ascontiguousarray(x, dtype=np.float32)


def make_inputs(wl: Workload, seed: Optional[int] = None,
                logits_override: Optional[np.ndarray] = None) -> Inputs:
    """Draw one full input set for workload `wl`.

    `logits_override` (float32 [B, P, V]) replaces the drawn logits; tests use
    it for hand-built tie patterns.
    """
    base = (0xDF2000 + wl.wid) if seed is None else int(seed)
    g = np.random.Generator(np.random.PCG64(base))
    B, P, V, d, r = wl.B, wl.P, wl.V, wl.d, wl.r
    s = 1.0 / math.sqrt(r)
    A = g.standard_normal((V, r), dtype=np.float32) * np.float32(s * wl.pair_scale)
    Bt = g.standard_normal((V, r), dtype=np.float32) * np.float32(s * wl.pair_scale)
    W = g.standard_normal((r, d), dtype=np.float32) * np.float32(s)
    hidden = g.standard_normal((B, P, d), dtype=np.float32)

    flat = np.zeros(B * P, dtype=bool)
    if wl.flat_frac > 0 and wl.flat_mode == "exact":
        n_flat = int(round(wl.flat_frac * B * P))
        flat[g.permutation(B * P)[:n_flat]] = True
    elif wl.flat_frac > 0:
        flat = g.random(B * P) < wl.flat_frac
    flat = flat.reshape(B, P)

    prev = np.empty(B, dtype=np.int32)
    if logits_override is not None:
        logits = np.ascontiguousarray(logits_override, dtype=np.float32).reshape(B, P, V)
        for b in range(B):
            gb = np.random.Generator(np.random.PCG64(base * 1000 + b))
            prev[b] = gb.integers(0, V)
    else:
        logits = np.empty((B, P, V), dtype=np.float32)
        for b in range(B):
            gb = np.random.Generator(np.random.PCG64(base * 1000 + b))
            prev[b] = gb.integers(0, V)
            if wl.logit_kind == "true_token":
                row = gb.standard_normal((P, V), dtype=np.float32)
                true_tok = gb.integers(0, V, size=P)
                row[np.arange(P), true_tok] += np.float32(6.0)
                logits[b] = row
                continue
            last_top = -1
            for t in range(P):
                if flat[b, t]:
                    logits[b, t] = gb.standard_normal(V, dtype=np.float32)
                    last_top = -1
                    continue
                row = gb.standard_normal(V, dtype=np.float32) * np.float32(2.0)
                m = int(gb.integers(1, 4))
                toks = gb.integers(0, V, size=m)
                if wl.dup_prob > 0 and last_top >= 0 and gb.random() < wl.dup_prob:
                    toks[0] = last_top
                for k in range(m):
                    row[toks[k]] += np.float32(4.0 + 6.0 / (k + 1))
                last_top = int(toks[0])
                logits[b, t] = row
    dt = wl.dtype
    return Inputs(wl=wl, logits=_store(logits, dt), hidden=_store(hidden, dt),
                  A=_store(A, dt), Bt=_store(Bt, dt), W=_store(W, dt), prev=prev)


# ---------------------------------------------------------------------------
# Inputs of the drafter's two-tap convolution ("A Lightweight Local
# Convolution").  The pages give no trained values; the recipe: sublayer
# inputs x and x_prev ~ N(0, 1); base tap 0 ~ 1 + 0.1 N(0, 1) (close to the
# identity), tap 1 ~ 0.1 N(0, 1); correction map W_c ~ 0.1 N(0, 1) / sqrt(d)
# (a small content-dependent correction, as the pages describe it).
# Shapes follow the selector workloads: d = 2560 (Qwen3-4B drafter) and
# d = 5120 (27B-target drafter), P = 7 draft positions.
# ---------------------------------------------------------------------------
@dataclasses.dataclass
class ConvInputs:
    B: int
    P: int
    d: int
    dtype: str
    x: np.ndarray        # [B, P, d]
    x_prev: np.ndarray   # [B, d]
    base: np.ndarray     # [2, d]
    W_c: np.ndarray      # [2, d/16, d]

    def f64(self):
        dt = self.dtype
        return dict(x=to_f64(self.x, dt), x_prev=to_f64(self.x_prev, dt),
                    base=to_f64(self.base, dt), W_c=to_f64(self.W_c, dt))


CONV_WORKLOADS = {
    "conv_qwen3_4b_b1": dict(B=1, P=7, d=2560),
    "conv_t27b_b32": dict(B=32, P=7, d=5120),
}


def make_conv_inputs(B: int, P: int, d: int, dtype: str = "bf16", seed: int = 0xC0) -> ConvInputs:
    g = np.random.Generator(np.random.PCG64(0xDF2C00 + int(seed)))
    x = g.standard_normal((B, P, d), dtype=np.float32)
    x_prev = g.standard_normal((B, d), dtype=np.float32)
    base = np.stack([1.0 + 0.1 * g.standard_normal(d, dtype=np.float32),
                     0.1 * g.standard_normal(d, dtype=np.float32)]).astype(np.float32)
    W_c = (0.1 / math.sqrt(d)) * g.standard_normal((2, d // 16, d), dtype=np.float32)
    return ConvInputs(B, P, d, dtype, _store(x, dtype), _store(x_prev, dtype), _store(base, dtype),
                      _store(W_c.astype(np.float32), dtype))


# ---------------------------------------------------------------------------
# Inputs of the drafter's LM head (the logits the selector starts from).  The
# pages give no trained weights; the recipe reproduces the logit mix of the
# workloads above from a hidden state and a weight matrix:
#   * W_lm [V, d] ~ N(0, 1/d) (std 1/sqrt(d)), so a hidden state z ~ N(0, 1)^d
#     gives logits ~ N(0, 1);
#   * each position's hidden state is s * z with s = 2 for peaked rows and
#     s = 1 for flat rows (the N(0, 2) and N(0, 1) logits of the selector
#     workloads), plus, for a peaked row, delta_k * w / |w|^2 for each of its
#     m ~ U{1,2,3} peak tokens (w = that token's bf16 weight row,
#     delta_k = 4 + 6/k), which lifts that token's logit by delta_k;
#   * flat rows, their fraction and the stress workload's reuse of the
#     previous position's top peak follow the selector workloads.
# Everything is bf16 (the drafter's precision); sequence b draws from
# sub-seed seed * 1000 + b, the weights from the base seed in row blocks.
# ---------------------------------------------------------------------------
def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns to float32."""
    return (np.asarray(b).astype(np.uint32) << np.uint32(16)).view(np.float32)


@dataclasses.dataclass
class LmHeadInputs:
    wl: Workload
    X: np.ndarray        # [B*P, d] bf16 bits, final hidden state per draft position
    W_lm: np.ndarray     # [V, d] bf16 bits, one weight row per token
    peaks: np.ndarray    # [B*P, 3] int32 planted peak tokens, -1 where none
    flat: np.ndarray     # [B*P] bool

    def f32(self):
        """(X, W_lm) widened exactly to float32."""
        return bf16_bits_to_f32(self.X), bf16_bits_to_f32(self.W_lm)


def make_lmhead_inputs(wl: Workload, seed: Optional[int] = None,
                       row_block: int = 8192) -> LmHeadInputs:
    base = (0xDF2100 + wl.wid) if seed is None else int(seed)
    g = np.random.Generator(np.random.PCG64(base))
    B, P, V, d = wl.B, wl.P, wl.V, wl.d
    M = B * P
    W = np.empty((V, d), dtype=np.uint16)
    scale = np.float32(1.0 / math.sqrt(d))
    for r0 in range(0, V, row_block):
        r1 = min(V, r0 + row_block)
        W[r0:r1] = f32_to_bf16_bits(g.standard_normal((r1 - r0, d), dtype=np.float32) * scale)

    flat = np.zeros(M, dtype=bool)
    if wl.flat_frac > 0 and wl.flat_mode == "exact":
        flat[g.permutation(M)[:int(round(wl.flat_frac * M))]] = True
    elif wl.flat_frac > 0:
        flat = g.random(M) < wl.flat_frac

    X = np.empty((M, d), dtype=np.uint16)
    peaks = np.full((M, 3), -1, dtype=np.int32)
    for b in range(B):
        gb = np.random.Generator(np.random.PCG64(base * 1000 + b))
        last_top = -1
        for t in range(P):
            row = b * P + t
            if flat[row]:
                X[row] = f32_to_bf16_bits(gb.standard_normal(d, dtype=np.float32))
                last_top = -1
                continue
            x = 2.0 * gb.standard_normal(d, dtype=np.float32).astype(np.float64)
            m = int(gb.integers(1, 4))
            toks = gb.integers(0, V, size=m)
            if wl.dup_prob > 0 and last_top >= 0 and gb.random() < wl.dup_prob:
                toks[0] = last_top
            for k in range(m):
                w = bf16_bits_to_f64(W[toks[k]])
                x += (4.0 + 6.0 / (k + 1)) * w / np.dot(w, w)
            peaks[row, :m] = toks
            last_top = int(toks[0])
            X[row] = f32_to_bf16_bits(x.astype(np.float32))
    return LmHeadInputs(wl=wl, X=X, W_lm=W, peaks=peaks, flat=flat)
