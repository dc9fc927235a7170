"""GPU parity of the drafter's two-tap dynamic convolution (dflash2_conv2)
against the CPU oracle, element by element.

Tolerance: the corrections are fp32 sums of d products (exact for bf16
inputs), so their error is a small multiple of 2^-24 times sum |W_c x|; the
combine adds a few fp32 roundings.  rel = 1e-4 of the magnitude sigma
(|base| + sum |W_c x|) |x| summed over both taps covers d up to 8192 with a
wide margin.  bf16 outputs add the rounding to bf16: at most half a bf16 ulp
(2^-8 relative) of the fp32 value, so |y - y_ref| <= 2^-8 |y_ref| + 2 rel sigma.
"""
import numpy as np
import pytest
import torch

import oracle
import draft_selection_topk16_amd as df2
from draft_selection_topk16_amd import synth
from gpu_util import dev_tensor, say

pytestmark = pytest.mark.gpu

REL = 1e-4


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    df2.load()
    yield
    torch.cuda.synchronize()


def run_case(c: synth.ConvInputs):
    dt = c.dtype
    y = df2.conv2(dev_tensor(c.x, dt), dev_tensor(c.x_prev, dt), dev_tensor(c.base, dt),
                  dev_tensor(c.W_c, dt))
    torch.cuda.synchronize()
    if dt == "bf16":
        return synth.bf16_bits_to_f64(y.view(torch.int16).cpu().numpy().view(np.uint16))
    return y.cpu().numpy().astype(np.float64)


def check(y, c, label):
    f = c.f64()
    ref, sig = oracle.conv2(f["x"], f["x_prev"], f["base"], f["W_c"])
    bound = 2 * REL * sig + (2.0 ** -8 * np.abs(ref) if c.dtype == "bf16" else 0.0)
    err = np.abs(y - ref)
    worst = float(np.max(err / np.maximum(bound, 1e-30)))
    say("  %s: worst error / bound %.3g" % (label, worst))
    assert np.all(err <= bound), (label, worst)


@pytest.mark.parametrize("B,P,d", [(1, 7, 2560), (32, 7, 5120), (3, 1, 512), (5, 9, 1024),
                                   (2, 16, 4096), (33, 7, 512), (1, 3, 8192)])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_conv2_shapes(B, P, d, dtype):
    say("conv2 %s B=%d P=%d d=%d" % (dtype, B, P, d))
    c = synth.make_conv_inputs(B, P, d, dtype, seed=B * 100 + P * 10 + d // 512)
    check(run_case(c), c, "conv2 %s B=%d P=%d d=%d" % (dtype, B, P, d))


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_conv2_integer_exact(dtype):
    """Small integers keep every product and sum exact in fp32 (and the
    results fit bf16 where they stay below 256): bit-exact output."""
    say("conv2 integer exact %s" % dtype)
    rng = np.random.default_rng(5)
    B, P, d = 3, 5, 512
    x = rng.integers(-2, 3, size=(B, P, d)).astype(np.float32)
    xp = rng.integers(-2, 3, size=(B, d)).astype(np.float32)
    base = rng.integers(-2, 3, size=(2, d)).astype(np.float32)
    Wc = (rng.random((2, d // 16, d)) < 0.01).astype(np.float32) * rng.integers(-1, 2, size=(2, d // 16, d))
    st = (lambda a: synth.f32_to_bf16_bits(a)) if dtype == "bf16" else (lambda a: a.astype(np.float32))
    c = synth.ConvInputs(B, P, d, dtype, st(x), st(xp), st(base), st(Wc.astype(np.float32)))
    y = run_case(c)
    f = c.f64()
    ref, _ = oracle.conv2(f["x"], f["x_prev"], f["base"], f["W_c"])
    assert np.max(np.abs(ref)) < 256
    assert np.array_equal(y, ref)


def test_conv2_empty_and_repeat():
    say("conv2 empty batch and repeat")
    x = torch.empty((0, 7, 512), dtype=torch.bfloat16, device="cuda")
    xp = torch.empty((0, 512), dtype=torch.bfloat16, device="cuda")
    base = torch.zeros((2, 512), dtype=torch.bfloat16, device="cuda")
    Wc = torch.zeros((2, 32, 512), dtype=torch.bfloat16, device="cuda")
    assert df2.conv2(x, xp, base, Wc).shape == (0, 7, 512)
    c = synth.make_conv_inputs(4, 7, 1024, "bf16", seed=3)
    a = run_case(c)
    b = run_case(c)
    assert np.array_equal(a, b)
