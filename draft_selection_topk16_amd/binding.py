"""ctypes binding of libdflash2.so (the C ABI in include/dflash2.h).

Argument marshalling only: every step of the selector runs in the HIP
kernels of the library.  PyTorch supplies device memory and the stream.  If
the library has not been built, every call raises; there is no other path.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Tuple

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libdflash2.so")

DF2_F32 = 0
DF2_BF16 = 1

# df2_walk
WALKS = {"viterbi": 0, "greedy": 1}

# df2_plan_knob
PLAN_KNOBS = {"segment_wgs": 0, "chunk_vectors": 1, "merge_words": 2, "gate_slices": 3,
              "conv_slices": 4, "launches": 5, "lm_ranges": 6, "gate_giveup": 7}

EXPORTED = (
    "dflash2_select", "dflash2_select_walk", "dflash2_select_sample", "dflash2_select_noalloc",
    "dflash2_topk", "dflash2_lmhead_topk",
    "dflash2_project", "dflash2_pair_scores", "dflash2_viterbi", "dflash2_walk",
    "dflash2_sample_walk", "dflash2_philox_uniforms", "dflash2_philox_uniforms_next",
    "dflash2_conv2", "dflash2_device_error",
    "dflash2_plan_override",
    "dflash2_release",
    "dflash2_status_string",
    "dflash2_last_error", "dflash2_version",
)


class SelectorError(RuntimeError):
    """A non-OK status returned by the library."""

    def __init__(self, status: int, msg: str):
        super().__init__(msg)
        self.status = status


class Dims(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int32), ("P", ctypes.c_int32), ("V", ctypes.c_int32),
                ("d", ctypes.c_int32), ("r", ctypes.c_int32), ("dtype", ctypes.c_int)]


_lib = None


def load() -> ctypes.CDLL:
    """Load the HIP library; raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(
            "libdflash2.so is not built; run `python -m draft_selection_topk16_amd.build` "
            "(the selector has no fallback path)")
    lib = ctypes.CDLL(LIB_PATH)
    vp, i32, i64, u32p = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.POINTER(ctypes.c_uint32)
    dp = ctypes.POINTER(Dims)
    sig = {
        "dflash2_select": [dp, vp, vp, vp, vp, vp, vp, i32, vp, vp, vp],
        "dflash2_select_walk": [dp, vp, vp, vp, vp, vp, vp, i32, ctypes.c_int, vp, vp, vp],
        "dflash2_select_noalloc": [dp, vp, vp, vp, vp, vp, vp, i32, vp, vp, vp],
        "dflash2_select_sample": [dp, vp, vp, vp, vp, vp, vp, i32, ctypes.c_float, vp, vp, vp, vp,
                                  vp],
        "dflash2_topk": [vp, i64, i32, ctypes.c_int, i32, vp, vp, vp],
        "dflash2_lmhead_topk": [vp, vp, i64, i32, i32, ctypes.c_int, i32, vp, vp, vp],
        "dflash2_project": [vp, vp, i64, i32, i32, ctypes.c_int, vp, vp],
        "dflash2_pair_scores": [dp, vp, vp, vp, vp, vp, vp, i32, vp, vp],
        "dflash2_viterbi": [vp, vp, i32, i32, i32, vp, vp, vp],
        "dflash2_walk": [vp, vp, i32, i32, i32, ctypes.c_int, vp, vp, vp],
        "dflash2_sample_walk": [vp, vp, vp, i32, i32, i32, ctypes.c_float, vp, vp, vp, vp],
        "dflash2_conv2": [vp, vp, vp, vp, i32, i32, i32, ctypes.c_int, vp, vp],
        "dflash2_philox_uniforms": [ctypes.c_uint64, ctypes.c_uint64, ctypes.c_int64, vp, vp],
        "dflash2_philox_uniforms_next": [ctypes.c_uint64, vp, ctypes.c_int64, vp, vp],
        "dflash2_device_error": [vp, u32p],
        "dflash2_plan_override": [ctypes.c_int, i32],
        "dflash2_release": [],
    }
    for name, args in sig.items():
        f = getattr(lib, name)
        f.argtypes = args
        f.restype = ctypes.c_int
    for name in ("dflash2_status_string",):
        getattr(lib, name).argtypes = [ctypes.c_int]
        getattr(lib, name).restype = ctypes.c_char_p
    for name in ("dflash2_last_error", "dflash2_version"):
        getattr(lib, name).argtypes = []
        getattr(lib, name).restype = ctypes.c_char_p
    _lib = lib
    return lib


def _check(status: int) -> None:
    if status != 0:
        lib = load()
        msg = "%s: %s" % (lib.dflash2_status_string(status).decode(),
                          lib.dflash2_last_error().decode())
        raise SelectorError(status, msg)


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return DF2_BF16
    if t.dtype == torch.float32:
        return DF2_F32
    raise TypeError("expected bfloat16 or float32, got %s" % t.dtype)


def _dev(t: torch.Tensor, name: str) -> int:
    if not t.is_cuda:
        raise ValueError("%s must be a GPU tensor" % name)
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    return t.data_ptr()


def _stream(device: torch.device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


def _walk_code(walk: str) -> int:
    if walk not in WALKS:
        raise ValueError("walk must be one of %s" % sorted(WALKS))
    return WALKS[walk]


def _uniforms(u: Optional[torch.Tensor], B: int, P: int) -> torch.Tensor:
    if u is None:
        raise ValueError("the sampling walk needs uniforms u [B, P]")
    if u.dtype != torch.float32 or tuple(u.shape) != (B, P):
        raise ValueError("u must be float32 [B, P]")
    return u


class PreparedSelect:
    """The checked arguments of one dflash2_select_walk (or, for walk="sample",
    dflash2_select_sample) call, for repeated launches with little host
    overhead (the tensors are kept alive and must not be reallocated; refill
    `u` in place between launches to draw again).  Calling it enqueues one
    launch on the stream that was current when it was prepared.
    walk: "viterbi", "greedy" or "sample" (then u [B, P] float32 uniforms and
    the temperature; the draws' probabilities land in self.out_q)."""

    def __init__(self, logits: torch.Tensor, hidden: torch.Tensor, A: torch.Tensor,
                 Bt: torch.Tensor, W: torch.Tensor, prev: torch.Tensor, K: int,
                 out_path: Optional[torch.Tensor] = None,
                 out_score: Optional[torch.Tensor] = None, walk: str = "viterbi",
                 u: Optional[torch.Tensor] = None, temperature: float = 1.0):
        lib = load()
        sample = walk == "sample"
        wcode = 0 if sample else _walk_code(walk)
        B, P, V = logits.shape
        d = hidden.shape[-1]
        r = A.shape[-1]
        dt = _dtype_code(logits)
        for name, t in (("hidden", hidden), ("A", A), ("Bt", Bt), ("W", W)):
            if t.dtype != logits.dtype:
                raise TypeError("%s must have the logits dtype" % name)
        if (hidden.shape != (B, P, d) or A.shape != (V, r) or Bt.shape != (V, r)
                or W.shape != (r, d)):
            raise ValueError("inconsistent shapes")
        if prev.dtype != torch.int32 or prev.shape != (B,):
            raise ValueError("prev must be int32 [B]")
        if out_path is None:
            out_path = torch.empty((B, P), dtype=torch.int32, device=logits.device)
        if out_score is None:
            out_score = torch.empty((B,), dtype=torch.float32, device=logits.device)
        self.out_path, self.out_score = out_path, out_score
        self.out_q = None
        self._keep = (logits, hidden, A, Bt, W, prev)
        self._dims = Dims(B, P, V, d, r, dt)
        head = (ctypes.byref(self._dims), _dev(logits, "logits"), _dev(hidden, "hidden"),
                _dev(A, "A"), _dev(Bt, "Bt"), _dev(W, "W"), _dev(prev, "prev"), int(K))
        if sample:
            u = _uniforms(u, B, P)
            self.out_q = torch.empty((B, P), dtype=torch.float32, device=logits.device)
            self._keep += (u,)
            self._fn = lib.dflash2_select_sample
            self._args = head + (float(temperature), _dev(u, "u"), _dev(out_path, "out_path"),
                                 _dev(self.out_q, "out_q"), _dev(out_score, "out_score"),
                                 _stream(logits.device))
        else:
            self._fn = lib.dflash2_select_walk
            self._args = head + (wcode, _dev(out_path, "out_path"), _dev(out_score, "out_score"),
                                 _stream(logits.device))

    def __call__(self) -> Tuple[torch.Tensor, torch.Tensor]:
        _check(self._fn(*self._args))
        return self.out_path, self.out_score


def select(logits: torch.Tensor, hidden: torch.Tensor, A: torch.Tensor, Bt: torch.Tensor,
           W: torch.Tensor, prev: torch.Tensor, K: int,
           out_path: Optional[torch.Tensor] = None,
           out_score: Optional[torch.Tensor] = None,
           walk: str = "viterbi") -> Tuple[torch.Tensor, torch.Tensor]:
    """Selected path [B, P] int32 and its score [B] float32 (one select call);
    walk: "viterbi" (max-sum with backtrack) or "greedy"."""
    return PreparedSelect(logits, hidden, A, Bt, W, prev, K, out_path, out_score, walk)()


def select_sample(logits: torch.Tensor, hidden: torch.Tensor, A: torch.Tensor, Bt: torch.Tensor,
                  W: torch.Tensor, prev: torch.Tensor, K: int, u: torch.Tensor,
                  temperature: float = 1.0) -> Tuple[torch.Tensor, torch.Tensor, torch.Tensor]:
    """Sampling walk in one select call: (path [B, P] int32, q [B, P] float32 =
    each drawn token's probability, score [B] float32); u [B, P] float32
    uniforms in [0, 1)."""
    call = PreparedSelect(logits, hidden, A, Bt, W, prev, K, walk="sample", u=u,
                          temperature=temperature)
    path, score = call()
    return path, call.out_q, score


def topk(logits: torch.Tensor, K: int) -> Tuple[torch.Tensor, torch.Tensor]:
    """Top-K of each row of logits[..., V]: (idx int32, val float32)."""
    lib = load()
    V = logits.shape[-1]
    rows = logits.numel() // V if V else 0
    idx = torch.empty(logits.shape[:-1] + (K,), dtype=torch.int32, device=logits.device)
    val = torch.empty(logits.shape[:-1] + (K,), dtype=torch.float32, device=logits.device)
    _check(lib.dflash2_topk(_dev(logits, "logits"), rows, V, _dtype_code(logits), int(K),
                            _dev(idx, "idx"), _dev(val, "val"), _stream(logits.device)))
    return idx, val


def lmhead_topk(hidden: torch.Tensor, W_lm: torch.Tensor, K: int) -> Tuple[torch.Tensor, torch.Tensor]:
    """The LM head fused with top-K: for every row of hidden[..., d] (bf16),
    the top K of W_lm [V, d] @ hidden without writing the logits:
    (idx int32 [..., K], val float32 [..., K])."""
    lib = load()
    V, d = W_lm.shape
    if hidden.shape[-1] != d:
        raise ValueError("hidden [..., d] and W_lm [V, d] disagree on d")
    if W_lm.dtype != hidden.dtype:
        raise TypeError("W_lm must have the hidden dtype")
    M = hidden.numel() // d if d else 0
    idx = torch.empty(hidden.shape[:-1] + (K,), dtype=torch.int32, device=hidden.device)
    val = torch.empty(hidden.shape[:-1] + (K,), dtype=torch.float32, device=hidden.device)
    _check(lib.dflash2_lmhead_topk(_dev(hidden, "hidden"), _dev(W_lm, "W_lm"), M, V, d,
                                   _dtype_code(hidden), int(K), _dev(idx, "idx"), _dev(val, "val"),
                                   _stream(hidden.device)))
    return idx, val


def project(hidden: torch.Tensor, W: torch.Tensor) -> torch.Tensor:
    """H[..., q] = sum_m W[q, m] hidden[..., m], float32."""
    lib = load()
    r, d = W.shape
    M = hidden.numel() // d
    if W.dtype != hidden.dtype:
        raise TypeError("W must have the hidden dtype")
    H = torch.empty(hidden.shape[:-1] + (r,), dtype=torch.float32, device=hidden.device)
    _check(lib.dflash2_project(_dev(hidden, "hidden"), _dev(W, "W"), M, d, r,
                               _dtype_code(hidden), _dev(H, "H"), _stream(hidden.device)))
    return H


def pair_scores(cand: torch.Tensor, cval: torch.Tensor, H: torch.Tensor, A: torch.Tensor,
                Bt: torch.Tensor, prev: torch.Tensor) -> torch.Tensor:
    """S [B, P, K, K] float32 from candidates [B, P, K], gates H [B, P, r]."""
    lib = load()
    B, P, K = cand.shape
    V, r = A.shape
    dims = Dims(B, P, V, 32, r, _dtype_code(A))
    S = torch.empty((B, P, K, K), dtype=torch.float32, device=cand.device)
    _check(lib.dflash2_pair_scores(ctypes.byref(dims), _dev(cand, "cand"), _dev(cval, "cval"),
                                   _dev(H, "H"), _dev(A, "A"), _dev(Bt, "Bt"), _dev(prev, "prev"),
                                   int(K), _dev(S, "S"), _stream(cand.device)))
    return S


def viterbi(S: torch.Tensor, cand: torch.Tensor) -> Tuple[torch.Tensor, torch.Tensor]:
    """Walk over S [B, P, K, K]: (path [B, P] int32, score [B] float32)."""
    lib = load()
    B, P, K = cand.shape
    path = torch.empty((B, P), dtype=torch.int32, device=S.device)
    score = torch.empty((B,), dtype=torch.float32, device=S.device)
    _check(lib.dflash2_viterbi(_dev(S, "S"), _dev(cand, "cand"), B, P, K, _dev(path, "path"),
                               _dev(score, "score"), _stream(S.device)))
    return path, score


def walk(S: torch.Tensor, cand: torch.Tensor, mode: str = "viterbi") -> Tuple[torch.Tensor, torch.Tensor]:
    """Walk over S [B, P, K, K] in either mode: (path [B, P] int32, score [B] float32)."""
    lib = load()
    wcode = _walk_code(mode)
    B, P, K = cand.shape
    path = torch.empty((B, P), dtype=torch.int32, device=S.device)
    score = torch.empty((B,), dtype=torch.float32, device=S.device)
    _check(lib.dflash2_walk(_dev(S, "S"), _dev(cand, "cand"), B, P, K, wcode, _dev(path, "path"),
                            _dev(score, "score"), _stream(S.device)))
    return path, score


def sample_walk(S: torch.Tensor, cand: torch.Tensor, u: torch.Tensor,
                temperature: float = 1.0) -> Tuple[torch.Tensor, torch.Tensor, torch.Tensor]:
    """Sampling walk over S [B, P, K, K]: (path, q, score) as select_sample."""
    lib = load()
    B, P, K = cand.shape
    u = _uniforms(u, B, P)
    path = torch.empty((B, P), dtype=torch.int32, device=S.device)
    q = torch.empty((B, P), dtype=torch.float32, device=S.device)
    score = torch.empty((B,), dtype=torch.float32, device=S.device)
    _check(lib.dflash2_sample_walk(_dev(S, "S"), _dev(cand, "cand"), _dev(u, "u"), B, P, K,
                                   float(temperature), _dev(path, "path"), _dev(q, "q"),
                                   _dev(score, "score"), _stream(S.device)))
    return path, q, score


def philox_uniforms(seed: int, offset: int, n: int, device=None,
                    out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """n uniforms in [0, 1) from the device's Philox4x64-10 stream (seed, offset),
    as a float32 tensor on `device` (default: the current CUDA device)."""
    lib = load()
    if out is None:
        dev = torch.device("cuda", torch.cuda.current_device()) if device is None else torch.device(device)
        out = torch.empty((max(int(n), 0),), dtype=torch.float32, device=dev)
    elif out.dtype != torch.float32 or out.numel() < n or not out.is_contiguous():
        raise ValueError("out must be a contiguous float32 tensor of at least n elements")
    _check(lib.dflash2_philox_uniforms(int(seed) & (2**64 - 1), int(offset) & (2**64 - 1), int(n),
                                       _dev(out, "out") if n > 0 else 0, _stream(out.device)))
    return out


def philox_uniforms_next(seed: int, offset: torch.Tensor, out: torch.Tensor) -> torch.Tensor:
    """out.numel() uniforms of the stream (seed, offset[0]) into `out`, then
    offset[0] += 1 on the device (offset: int64 tensor of one element on the
    GPU, read as uint64); safe to capture in a CUDA/HIP graph."""
    lib = load()
    if offset.dtype != torch.int64 or offset.numel() != 1:
        raise ValueError("offset must be an int64 tensor of one element")
    if out.dtype != torch.float32:
        raise ValueError("out must be float32")
    n = out.numel()
    _check(lib.dflash2_philox_uniforms_next(int(seed) & (2**64 - 1), _dev(offset, "offset"), n,
                                            _dev(out, "out"), _stream(out.device)))
    return out


def conv2(x: torch.Tensor, x_prev: torch.Tensor, base: torch.Tensor, W_c: torch.Tensor,
          out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Two-tap dynamic depthwise convolution: x [B, P, d], x_prev [B, d],
    base [2, d], W_c [2, d/16, d] (one dtype) -> y [B, P, d] in that dtype."""
    lib = load()
    B, P, d = x.shape
    dt = _dtype_code(x)
    for name, t in (("x_prev", x_prev), ("base", base), ("W_c", W_c)):
        if t.dtype != x.dtype:
            raise TypeError("%s must have the dtype of x" % name)
    if x_prev.shape != (B, d) or base.shape != (2, d) or W_c.shape != (2, d // 16, d):
        raise ValueError("inconsistent shapes")
    if out is None:
        out = torch.empty_like(x)
    _check(lib.dflash2_conv2(_dev(x, "x"), _dev(x_prev, "x_prev"), _dev(base, "base"),
                             _dev(W_c, "W_c"), B, P, d, dt, _dev(out, "out"), _stream(x.device)))
    return out


def device_error(device: Optional[torch.device] = None) -> int:
    """Waits for the current stream; returns and clears its device input flags."""
    lib = load()
    flags = ctypes.c_uint32(0)
    dev = device if device is not None else torch.device("cuda", torch.cuda.current_device())
    _check(lib.dflash2_device_error(_stream(dev), ctypes.byref(flags)))
    return int(flags.value)


def plan_override(knob: str, value: int) -> None:
    """Pins one launch-plan knob for later calls (0 = automatic); for
    measurement and plan-invariance tests."""
    if knob not in PLAN_KNOBS:
        raise ValueError("knob must be one of %s" % sorted(PLAN_KNOBS))
    _check(load().dflash2_plan_override(PLAN_KNOBS[knob], int(value)))


class plan:
    """Context manager: plan knobs pinned inside, automatic again after."""

    def __init__(self, **knobs):
        self.knobs = knobs

    def __enter__(self):
        for k, v in self.knobs.items():
            plan_override(k, v)
        return self

    def __exit__(self, *exc):
        for k in self.knobs:
            plan_override(k, 0)
        return False


def release() -> None:
    _check(load().dflash2_release())


def version() -> str:
    return load().dflash2_version().decode()
