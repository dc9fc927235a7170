"""GPU parity of the device-side uniforms (dflash2_philox_uniforms) against
the oracle's Philox4x64-10, and the sampling walk fed from them.

The generator follows Salmon, Moraes, Dror and Shaw, "Parallel Random
Numbers: As Easy as 1, 2, 3" (SC 2011); the sampling walk it feeds is the
one of "DFlash 2: Keep Drafting Parallel", section "A Lightweight Path
Selector" (sampling draws from the same scores).  Uniforms are integer work
(24 bits of a 64-bit word, scaled by a power of two), so every comparison is
bit-exact.
"""
import numpy as np
import pytest
import torch

import oracle
import draft_selection_topk16_amd as df2
from draft_selection_topk16_amd import synth
from gpu_util import TOL_SAMPLE, check_sample, say, to_device

pytestmark = pytest.mark.gpu

M64 = 2**64 - 1


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    df2.load()
    yield
    torch.cuda.synchronize()


def bits(a) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)


@pytest.mark.parametrize("seed,offset,n", [
    (0, 0, 1), (1, 0, 3), (5, 7, 4), (123, 9, 5), (0, 0, 255), (3, 1, 1024), (3, 1, 1025),
    (7, 0, 224), (42, 3, 3840), (M64, M64, 1023), (0x9E3779B97F4A7C15, 2**40 + 17, 4097),
    (2024, 9, 1 << 20),
])
def test_uniforms_bit_exact(seed, offset, n):
    say("philox uniforms seed=%d offset=%d n=%d" % (seed, offset, n))
    got = df2.philox_uniforms(seed, offset, n).cpu().numpy()
    want = oracle.philox_uniforms(seed, offset, n)
    assert np.array_equal(bits(got), bits(want))


@pytest.mark.parametrize("shift", [1, 2, 3, 4])
def test_uniforms_unaligned_output_and_no_overrun(shift):
    """Outputs 4- but not 16-byte aligned take the per-word stores; nothing is
    written outside [0, n)."""
    n = 1001
    say("philox uniforms out shifted by %d floats" % shift)
    buf = torch.full((n + 16,), -7.0, dtype=torch.float32, device="cuda")
    out = buf[shift:shift + n]
    df2.philox_uniforms(11, 5, n, out=out)
    got = buf.cpu().numpy()
    assert np.array_equal(bits(got[shift:shift + n]), bits(oracle.philox_uniforms(11, 5, n)))
    assert np.all(got[:shift] == -7.0) and np.all(got[shift + n:] == -7.0)


def test_uniforms_large_sampled():
    """2^26 + 3 uniforms (ragged last block): the first and last 4096 and
    4096 scattered ones against the oracle, one window each."""
    n = (1 << 26) + 3
    say("philox uniforms n=%d sampled" % n)
    buf = torch.full((n + 8,), -7.0, dtype=torch.float32, device="cuda")
    df2.philox_uniforms(77, 2**33 + 1, n, out=buf)
    got = buf.cpu().numpy()
    assert np.all(got[n:] == -7.0)
    assert np.array_equal(bits(got[:4096]), bits(oracle.philox_uniforms(77, 2**33 + 1, 4096)))
    assert np.array_equal(bits(got[n - 4096:n]),
                          bits(oracle.philox_uniforms(77, 2**33 + 1, 4096, first=n - 4096)))
    idx = np.random.default_rng(5).integers(0, n, size=4096)
    for i in idx:
        assert bits(got[i:i + 1])[0] == bits(oracle.philox_uniforms(77, 2**33 + 1, 1, first=int(i)))[0]
    assert got[:n].min() >= 0.0 and got[:n].max() < 1.0


def test_uniforms_zero_is_a_noop():
    out = torch.full((4,), -7.0, dtype=torch.float32, device="cuda")
    df2.philox_uniforms(1, 1, 0, out=out)
    torch.cuda.synchronize()
    assert torch.all(out == -7.0)


@pytest.mark.parametrize("name", ["qwen3_4b_b1", "t27b_b32"])
def test_select_sample_on_device_uniforms(name):
    """One draft-verify cycle as a serving loop runs it: the uniforms drawn
    on the device at (seed, cycle), then the sampling select; the oracle
    draws the same uniforms itself and walks the same lattice."""
    x = synth.make_inputs(synth.WORKLOADS[name])
    B, P, K = x.wl.B, x.wl.P, x.wl.K
    seed, cycle = 0xD1F1A5, 3
    say("select sample on device uniforms %s seed=%d cycle=%d" % (name, seed, cycle))
    u_dev = df2.philox_uniforms(seed, cycle, B * P).view(B, P)
    t = to_device(x)
    path, q, score = df2.select_sample(t["logits"], t["hidden"], t["A"], t["Bt"], t["W"], t["prev"],
                                       K, u_dev, 1.0)
    torch.cuda.synchronize()
    u = oracle.philox_uniforms(seed, cycle, B * P).reshape(B, P)
    assert np.array_equal(bits(u_dev.cpu().numpy()), bits(u))
    f = x.f64()
    o = oracle.select(f["logits"], f["hidden"], f["A"], f["Bt"], f["W"], f["prev"], K,
                      u=u.astype(np.float64), tau=1.0)
    check_sample(path.cpu().numpy(), q.cpu().numpy(), score.cpu().numpy(), o,
                 TOL_SAMPLE[x.wl.dtype], name)
    assert df2.device_error() == 0


@pytest.mark.parametrize("n", [1, 227, 1024, 1025, 3840])
def test_uniforms_next_advances_the_device_offset(n):
    """Eager calls: each uses the offset the device holds, then adds one (in
    the generator's own workgroup up to 1024 uniforms, by a second launch
    beyond)."""
    say("philox uniforms with a device offset, eager, n=%d" % n)
    off = torch.tensor([41], dtype=torch.int64, device="cuda")
    out = torch.empty((n,), dtype=torch.float32, device="cuda")
    for k in range(3):
        df2.philox_uniforms_next(9, off, out)
        torch.cuda.synchronize()
        assert np.array_equal(bits(out.cpu().numpy()), bits(oracle.philox_uniforms(9, 41 + k, n)))
        assert int(off.item()) == 42 + k


@pytest.mark.parametrize("n", [224, 3840])
def test_uniforms_next_in_a_captured_graph(n):
    """One call captured in a graph and replayed four times, with eager GPU
    work between the replays: every replay draws the next offset's
    uniforms, equal to the oracle's, and leaves the offset one further."""
    say("philox uniforms with a device offset, graph replays, n=%d" % n)
    off = torch.tensor([0], dtype=torch.int64, device="cuda")
    out = torch.empty((n,), dtype=torch.float32, device="cuda")
    other = torch.empty((1000,), dtype=torch.float32, device="cuda")
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        df2.philox_uniforms_next(77, off, out)         # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        df2.philox_uniforms_next(77, off, out)
    torch.cuda.synchronize()
    off.fill_(1000)
    torch.cuda.synchronize()
    for i in range(4):
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(bits(out.cpu().numpy()), bits(oracle.philox_uniforms(77, 1000 + i, n))), i
        assert int(off.item()) == 1001 + i
        df2.philox_uniforms(5, i, 1000, out=other)      # eager work between replays
        torch.cuda.synchronize()
        assert np.array_equal(bits(other.cpu().numpy()), bits(oracle.philox_uniforms(5, i, 1000)))
