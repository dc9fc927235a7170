"""The entry point that allocates nothing (dflash2_select_noalloc), through
the C ABI, against dflash2_select on the same inputs: the same kernels, so
paths and scores must be bit-identical.  Consecutive calls of different
sizes share the device's static scratch (the second smaller than the first,
the third larger again), so each must clear what the previous one left."""
import ctypes

import numpy as np
import pytest
import torch

import draft_selection_topk16_amd as df2
from draft_selection_topk16_amd import binding, synth
from gpu_util import say, to_device

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    df2.load()
    yield
    torch.cuda.synchronize()


def select_noalloc(t, K):
    lib = df2.load()
    logits = t["logits"]
    B, P, V = logits.shape
    d, r = t["hidden"].shape[-1], t["A"].shape[-1]
    dims = binding.Dims(B, P, V, d, r, binding._dtype_code(logits))
    path = torch.empty((B, P), dtype=torch.int32, device="cuda")
    score = torch.empty((B,), dtype=torch.float32, device="cuda")
    st = lib.dflash2_select_noalloc(ctypes.byref(dims), logits.data_ptr(), t["hidden"].data_ptr(),
                                    t["A"].data_ptr(), t["Bt"].data_ptr(), t["W"].data_ptr(),
                                    t["prev"].data_ptr(), int(K), path.data_ptr(), score.data_ptr(),
                                    torch.cuda.current_stream().cuda_stream)
    assert st == 0, lib.dflash2_last_error().decode()
    return path, score


@pytest.mark.parametrize("order", [("t27b_b8", "tiny_small", "qwen3_4b_b1")])
def test_noalloc_matches_select(order):
    for name in order:
        wl = synth.WORKLOADS["tiny_f32"].with_(V=5000) if name == "tiny_small" else synth.WORKLOADS[name]
        say("select_noalloc %s B=%d P=%d V=%d" % (name, wl.B, wl.P, wl.V))
        x = synth.make_inputs(wl)
        t = to_device(x)
        ref_p, ref_s = df2.select(t["logits"], t["hidden"], t["A"], t["Bt"], t["W"], t["prev"], wl.K)
        ref_p, ref_s = ref_p.clone(), ref_s.clone()
        for rep in range(2):
            p, s = select_noalloc(t, wl.K)
            torch.cuda.synchronize()
            assert torch.equal(p, ref_p), (name, rep)
            assert torch.equal(s, ref_s), (name, rep)
    assert df2.device_error() == 0


@pytest.mark.parametrize("launches", [1, 2, 4])
def test_noalloc_matches_select_in_every_plan(launches):
    """The other launch plans (forced through the plan knob, which both entry
    points read) on the static scratch: one fused launch, scan then tail, and
    the walks in a launch of their own (the automatic plan beyond one
    resident wave of rows), a larger call then a smaller one."""
    with df2.plan(launches=launches):
        for name in ("t27b_b8", "tiny_small"):
            wl = synth.WORKLOADS["tiny_f32"].with_(V=5000) if name == "tiny_small" else synth.WORKLOADS[name]
            say("select_noalloc %s launches=%d" % (name, launches))
            t = to_device(synth.make_inputs(wl))
            ref_p, ref_s = df2.select(t["logits"], t["hidden"], t["A"], t["Bt"], t["W"], t["prev"], wl.K)
            ref_p, ref_s = ref_p.clone(), ref_s.clone()
            p, s = select_noalloc(t, wl.K)
            torch.cuda.synchronize()
            assert torch.equal(p, ref_p), (name, launches)
            assert torch.equal(s, ref_s), (name, launches)
    assert df2.device_error() == 0
