"""CPU checks of the C ABI: the library builds/loads, exports every entry point
that include/dflash2.h declares, and rejects bad arguments on the host before
any HIP call (so these run without a GPU)."""
import ctypes
import os
import re
import subprocess

import pytest

import draft_selection_topk16_amd as df2
from draft_selection_topk16_amd.binding import Dims, EXPORTED

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "dflash2.h")

DF2_OK, DF2_EINVAL, DF2_EUNSUPPORTED = 0, 1, 2
FAKE = 0x10000      # a 16-byte aligned non-null address; never dereferenced


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(dflash2_\w+)\s*\(", src)))


@pytest.fixture(scope="module")
def lib():
    return df2.load()


def test_header_declarations_match_binding():
    assert declared_functions() == sorted(EXPORTED)


def test_library_exports_every_declared_symbol(lib):
    out = subprocess.run(["nm", "-D", "--defined-only", df2.binding.LIB_PATH],
                         capture_output=True, text=True, check=True).stdout
    syms = set(line.split()[-1] for line in out.splitlines() if line.strip())
    for name in declared_functions():
        assert name in syms, name
        assert hasattr(lib, name)


def test_version_and_status_strings(lib):
    assert re.fullmatch(r"\d+\.\d+\.\d+", df2.version())
    assert lib.dflash2_status_string(0) == b"ok"
    assert lib.dflash2_status_string(1) == b"invalid argument"
    assert lib.dflash2_status_string(99) == b"unknown status"


def _select(lib, dims, K=16, ptrs=None):
    p = ptrs or [FAKE] * 6
    return lib.dflash2_select(ctypes.byref(dims) if dims is not None else None,
                              p[0], p[1], p[2], p[3], p[4], p[5], K, FAKE, FAKE, None)


@pytest.mark.parametrize("dims,K,status,msg", [
    (None, 16, DF2_EINVAL, "dims is NULL"),
    (Dims(1, 7, 32000, 1024, 256, 7), 16, DF2_EINVAL, "dtype"),
    (Dims(-1, 7, 32000, 1024, 256, 1), 16, DF2_EINVAL, "B < 0"),
    (Dims(1, 0, 32000, 1024, 256, 1), 16, DF2_EINVAL, "P must be"),
    (Dims(1, 65, 32000, 1024, 256, 1), 16, DF2_EINVAL, "P must be"),
    (Dims(1, 7, 0, 1024, 256, 1), 16, DF2_EINVAL, "V < 1"),
    (Dims(1, 7, 32000, 1000, 256, 1), 16, DF2_EUNSUPPORTED, "d must be"),
    (Dims(1, 7, 32000, 1024, 200, 1), 16, DF2_EUNSUPPORTED, "r must be"),
    (Dims(1, 7, 32000, 1024, 2048, 1), 16, DF2_EUNSUPPORTED, "r must be"),
    (Dims(1, 7, 32000, 1024, 576, 1), 16, DF2_EUNSUPPORTED, "r must be"),
    (Dims(1, 7, 32000, 1024, 256, 1), 0, DF2_EINVAL, "K must be"),
    (Dims(1, 7, 32000, 1024, 256, 1), 65, DF2_EINVAL, "K must be"),
    (Dims(1, 7, 10, 1024, 256, 1), 11, DF2_EINVAL, "K must be"),
])
def test_select_rejects_bad_sizes(lib, dims, K, status, msg):
    assert _select(lib, dims, K) == status
    assert msg in lib.dflash2_last_error().decode()


def test_select_rejects_null_and_misaligned(lib):
    dims = Dims(2, 7, 32000, 1024, 256, 1)
    for i in range(6):
        p = [FAKE] * 6
        p[i] = None
        assert _select(lib, dims, 16, p) == DF2_EINVAL
        assert "NULL" in lib.dflash2_last_error().decode()
    for i in (1, 2, 3, 4):          # hidden, A, B, W need 16-byte alignment
        p = [FAKE] * 6
        p[i] = FAKE + 8
        assert _select(lib, dims, 16, p) == DF2_EINVAL
        assert "aligned" in lib.dflash2_last_error().decode()
    p = [FAKE] * 6
    p[0] = FAKE + 1                 # bf16 logits need 2-byte alignment
    assert _select(lib, dims, 16, p) == DF2_EINVAL


def test_empty_batch_is_a_noop(lib):
    # B == 0 returns before touching the device (no GPU needed)
    assert _select(lib, Dims(0, 7, 32000, 1024, 256, 1), 16) == DF2_OK
    assert lib.dflash2_topk(FAKE, 0, 100, 1, 16, FAKE, FAKE, None) == DF2_OK
    assert lib.dflash2_project(FAKE, FAKE, 0, 64, 64, 1, FAKE, None) == DF2_OK
    assert lib.dflash2_viterbi(FAKE, FAKE, 0, 3, 4, FAKE, FAKE, None) == DF2_OK
    assert lib.dflash2_walk(FAKE, FAKE, 0, 3, 4, 1, FAKE, FAKE, None) == DF2_OK
    assert lib.dflash2_select_walk(ctypes.byref(Dims(0, 7, 32000, 1024, 256, 1)), FAKE, FAKE,
                                   FAKE, FAKE, FAKE, FAKE, 16, 1, FAKE, FAKE, None) == DF2_OK
    assert lib.dflash2_philox_uniforms(1, 2, 0, None, None) == DF2_OK


def test_philox_uniforms_rejects_bad_arguments(lib):
    # every check runs on the host before a launch (no GPU needed)
    assert lib.dflash2_philox_uniforms(1, 2, -1, FAKE, None) == DF2_EINVAL
    assert b"n < 0" in lib.dflash2_last_error()
    assert lib.dflash2_philox_uniforms(1, 2, 2**31 + 1, FAKE, None) == DF2_EUNSUPPORTED
    assert lib.dflash2_philox_uniforms(1, 2, 16, None, None) == DF2_EINVAL
    assert b"NULL" in lib.dflash2_last_error()
    assert lib.dflash2_philox_uniforms(1, 2, 16, FAKE + 2, None) == DF2_EINVAL
    assert b"aligned" in lib.dflash2_last_error()
    assert lib.dflash2_philox_uniforms_next(1, FAKE, 0, None, None) == DF2_OK
    assert lib.dflash2_philox_uniforms_next(1, FAKE, -1, FAKE, None) == DF2_EINVAL
    assert lib.dflash2_philox_uniforms_next(1, None, 16, FAKE, None) == DF2_EINVAL
    assert b"NULL" in lib.dflash2_last_error()
    assert lib.dflash2_philox_uniforms_next(1, FAKE + 4, 16, FAKE, None) == DF2_EINVAL
    assert b"offset" in lib.dflash2_last_error()
    assert lib.dflash2_philox_uniforms_next(1, FAKE, 16, FAKE + 1, None) == DF2_EINVAL


def test_stage_entry_points_reject_bad_arguments(lib):
    assert lib.dflash2_topk(FAKE, 4, 100, 1, 0, FAKE, FAKE, None) == DF2_EINVAL
    assert lib.dflash2_topk(FAKE, 4, 10, 1, 11, FAKE, FAKE, None) == DF2_EINVAL
    assert lib.dflash2_topk(FAKE, -1, 100, 1, 4, FAKE, FAKE, None) == DF2_EINVAL
    assert lib.dflash2_topk(FAKE, 4, 100, 5, 4, FAKE, FAKE, None) == DF2_EINVAL
    assert lib.dflash2_topk(None, 4, 100, 1, 4, FAKE, FAKE, None) == DF2_EINVAL
    assert lib.dflash2_topk(FAKE + 1, 4, 100, 0, 4, FAKE, FAKE, None) == DF2_EINVAL
    assert lib.dflash2_project(FAKE, FAKE, 4, 48, 64, 1, FAKE, None) == DF2_EUNSUPPORTED
    assert lib.dflash2_project(FAKE, FAKE, 4, 64, 96, 1, FAKE, None) == DF2_EUNSUPPORTED
    assert lib.dflash2_project(FAKE + 4, FAKE, 4, 64, 64, 1, FAKE, None) == DF2_EINVAL
    assert lib.dflash2_viterbi(FAKE, FAKE, 2, 0, 4, FAKE, FAKE, None) == DF2_EINVAL
    assert lib.dflash2_viterbi(FAKE, FAKE, 2, 3, 65, FAKE, FAKE, None) == DF2_EINVAL
    assert lib.dflash2_viterbi(None, FAKE, 2, 3, 4, FAKE, FAKE, None) == DF2_EINVAL
    for mode in (0, 1):
        assert lib.dflash2_walk(FAKE, FAKE, 2, 0, 4, mode, FAKE, FAKE, None) == DF2_EINVAL
        assert lib.dflash2_walk(FAKE, FAKE, 2, 3, 65, mode, FAKE, FAKE, None) == DF2_EINVAL
        assert lib.dflash2_walk(FAKE + 2, FAKE, 2, 3, 4, mode, FAKE, FAKE, None) == DF2_EINVAL
    # an unknown walk mode is refused before anything else is looked at
    assert lib.dflash2_walk(FAKE, FAKE, 2, 3, 4, 2, FAKE, FAKE, None) == DF2_EINVAL
    assert lib.dflash2_walk(FAKE, FAKE, 2, 3, 4, -1, FAKE, FAKE, None) == DF2_EINVAL
    assert b"walk" in lib.dflash2_last_error()
    dsel = Dims(1, 7, 32000, 1024, 256, 1)
    assert lib.dflash2_select_walk(ctypes.byref(dsel), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 16, 2,
                                   FAKE, FAKE, None) == DF2_EINVAL
    assert b"walk" in lib.dflash2_last_error()
    # sampling walk: temperature, uniforms and out_q are checked on the host
    for tau in (0.0, -1.0, float("inf"), float("nan"), 1e-39):
        assert lib.dflash2_sample_walk(FAKE, FAKE, FAKE, 2, 3, 4, tau, FAKE, FAKE, FAKE, None) == DF2_EINVAL
        assert b"temperature" in lib.dflash2_last_error()
        assert lib.dflash2_select_sample(ctypes.byref(dsel), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 16,
                                         tau, FAKE, FAKE, FAKE, FAKE, None) == DF2_EINVAL
    assert lib.dflash2_sample_walk(FAKE, FAKE, None, 2, 3, 4, 1.0, FAKE, FAKE, FAKE, None) == DF2_EINVAL
    assert lib.dflash2_sample_walk(FAKE, FAKE, FAKE, 2, 3, 4, 1.0, FAKE, None, FAKE, None) == DF2_EINVAL
    assert lib.dflash2_sample_walk(FAKE, FAKE, FAKE + 2, 2, 3, 4, 1.0, FAKE, FAKE, FAKE, None) == DF2_EINVAL
    assert lib.dflash2_sample_walk(FAKE, FAKE, FAKE, 2, 0, 4, 1.0, FAKE, FAKE, FAKE, None) == DF2_EINVAL
    assert lib.dflash2_sample_walk(FAKE, FAKE, FAKE, 2, 3, 65, 1.0, FAKE, FAKE, FAKE, None) == DF2_EINVAL
    assert lib.dflash2_sample_walk(FAKE, FAKE, FAKE, 0, 3, 4, 1.0, FAKE, FAKE, FAKE, None) == DF2_OK
    assert lib.dflash2_select_sample(ctypes.byref(dsel), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 16, 1.0,
                                     None, FAKE, FAKE, FAKE, None) == DF2_EINVAL
    assert lib.dflash2_select_sample(ctypes.byref(dsel), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 16, 1.0,
                                     FAKE, FAKE, FAKE + 1, FAKE, None) == DF2_EINVAL
    assert lib.dflash2_select_sample(ctypes.byref(dsel), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 0, 1.0,
                                     FAKE, FAKE, FAKE, FAKE, None) == DF2_EINVAL
    d = Dims(2, 3, 100, 32, 64, 1)
    assert lib.dflash2_pair_scores(ctypes.byref(d), FAKE, FAKE, FAKE + 4, FAKE, FAKE, FAKE, 4,
                                   FAKE, None) == DF2_EINVAL
    assert lib.dflash2_pair_scores(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 101,
                                   FAKE, None) == DF2_EINVAL
    assert lib.dflash2_device_error(None, None) == DF2_EINVAL
    # two-tap convolution
    assert lib.dflash2_conv2(FAKE, FAKE, FAKE, FAKE, 0, 7, 512, 1, FAKE, None) == DF2_OK
    assert lib.dflash2_conv2(FAKE, FAKE, FAKE, FAKE, 2, 7, 500, 1, FAKE, None) == DF2_EUNSUPPORTED
    assert lib.dflash2_conv2(FAKE, FAKE, FAKE, FAKE, 2, 7, 8704, 1, FAKE, None) == DF2_EUNSUPPORTED
    assert lib.dflash2_conv2(FAKE, FAKE, FAKE, FAKE, 2, 0, 512, 1, FAKE, None) == DF2_EINVAL
    assert lib.dflash2_conv2(FAKE, FAKE, FAKE, FAKE, -1, 7, 512, 1, FAKE, None) == DF2_EINVAL
    assert lib.dflash2_conv2(FAKE, FAKE, FAKE, FAKE, 2, 7, 512, 3, FAKE, None) == DF2_EINVAL
    assert lib.dflash2_conv2(FAKE, None, FAKE, FAKE, 2, 7, 512, 1, FAKE, None) == DF2_EINVAL
    assert lib.dflash2_conv2(FAKE, FAKE, FAKE, FAKE + 8, 2, 7, 512, 1, FAKE, None) == DF2_EINVAL


def test_lmhead_topk_rejects_bad_arguments(lib):
    f = lib.dflash2_lmhead_topk
    # M == 0 enqueues nothing
    assert f(FAKE, FAKE, 0, 151936, 5120, 1, 16, FAKE, FAKE, None) == DF2_OK
    # bf16 only, d a multiple of 64 in [64, 32768]
    assert f(FAKE, FAKE, 4, 1000, 128, 0, 16, FAKE, FAKE, None) == DF2_EUNSUPPORTED
    assert b"bf16" in lib.dflash2_last_error()
    assert f(FAKE, FAKE, 4, 1000, 128, 7, 16, FAKE, FAKE, None) == DF2_EINVAL
    for d in (32, 96, 100, 32768 + 64):
        assert f(FAKE, FAKE, 4, 1000, d, 1, 16, FAKE, FAKE, None) == DF2_EUNSUPPORTED
    # K in [1, min(V, 64)]
    for K, V in ((0, 1000), (65, 1000), (11, 10)):
        assert f(FAKE, FAKE, 4, V, 128, 1, K, FAKE, FAKE, None) == DF2_EINVAL
    assert f(FAKE, FAKE, -1, 1000, 128, 1, 16, FAKE, FAKE, None) == DF2_EINVAL
    assert f(FAKE, FAKE, 4, 0, 128, 1, 16, FAKE, FAKE, None) == DF2_EINVAL
    assert f(FAKE, FAKE, 1 << 25, 1000, 128, 1, 16, FAKE, FAKE, None) == DF2_EUNSUPPORTED
    assert f(FAKE, FAKE, 4, (1 << 29) + 1, 128, 1, 16, FAKE, FAKE, None) == DF2_EUNSUPPORTED
    # pointers and alignment
    assert f(None, FAKE, 4, 1000, 128, 1, 16, FAKE, FAKE, None) == DF2_EINVAL
    assert f(FAKE, FAKE, 4, 1000, 128, 1, 16, FAKE, None, None) == DF2_EINVAL
    assert f(FAKE + 8, FAKE, 4, 1000, 128, 1, 16, FAKE, FAKE, None) == DF2_EINVAL
    assert f(FAKE, FAKE + 2, 4, 1000, 128, 1, 16, FAKE, FAKE, None) == DF2_EINVAL
    assert f(FAKE, FAKE, 4, 1000, 128, 1, 16, FAKE + 2, FAKE, None) == DF2_EINVAL
    # its plan knob: vocabulary ranges in [0, 256]
    assert lib.dflash2_plan_override(6, 257) == DF2_EINVAL
    assert lib.dflash2_plan_override(6, 0) == DF2_OK


def test_binding_rejects_unknown_walk_name():
    import torch
    S = torch.zeros(1, 2, 3, 3)
    cand = torch.zeros(1, 2, 3, dtype=torch.int32)
    with pytest.raises(ValueError):
        df2.walk(S, cand, "beam")


def test_binding_raises_without_gpu_tensors():
    import torch
    x = torch.zeros(2, 3, 100, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        df2.topk(x, 4)


def test_select_noalloc_rejects_beyond_its_scratch(lib):
    """A problem whose scratch exceeds the no-allocation entry point's static
    array (48 MiB) is refused on the host, before any device call."""
    dims = Dims(256, 64, 262144, 5120, 512, 1)
    st = lib.dflash2_select_noalloc(ctypes.byref(dims), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 64,
                                    FAKE, FAKE, None)
    assert st == DF2_EUNSUPPORTED
    msg = lib.dflash2_last_error().decode()
    assert "no-allocation" in msg and "50331648" in msg


def test_select_noalloc_checks_arguments_like_select(lib):
    assert lib.dflash2_select_noalloc(None, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 16, FAKE, FAKE,
                                      None) == DF2_EINVAL
    dims = Dims(0, 7, 32000, 1024, 256, 1)
    assert lib.dflash2_select_noalloc(ctypes.byref(dims), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 16,
                                      FAKE, FAKE, None) == DF2_OK


def test_plan_knobs_match_header_and_reject_bad_values(lib):
    import re
    from draft_selection_topk16_amd.binding import PLAN_KNOBS
    text = open(HEADER).read()
    body = text[text.index("typedef enum {\n    DF2_PLAN_SEGMENT_WGS"):]
    body = body[:body.index("} df2_plan_knob;")]
    declared = {m.group(1).lower(): int(m.group(2)) for m in re.finditer(r"DF2_PLAN_(\w+) = (\d+)", body)}
    assert declared == PLAN_KNOBS
    assert lib.dflash2_plan_override(max(PLAN_KNOBS.values()) + 1, 1) == DF2_EINVAL   # unknown knob
    assert lib.dflash2_plan_override(0, -1) == DF2_EINVAL                             # negative
    assert lib.dflash2_plan_override(PLAN_KNOBS["launches"], 5) == DF2_EINVAL
    assert lib.dflash2_plan_override(PLAN_KNOBS["chunk_vectors"], 3) == DF2_EINVAL
    assert lib.dflash2_plan_override(PLAN_KNOBS["gate_giveup"], 2) == DF2_EINVAL
    for k in PLAN_KNOBS.values():
        assert lib.dflash2_plan_override(k, 0) == DF2_OK
