"""Pins for the oracle's two-tap dynamic depthwise convolution.

Method: "DFlash 2: Keep Drafting Parallel", section "A Lightweight Local
Convolution": y_t = k_{t,0} * x_t + k_{t,1} * x_{t-1}, the first position
reading the last verified token's representation, each coefficient a learned
base plus a correction from the current hidden state shared by 16 channels
(read as corr_t[tap][g] = sum_m Wc[tap][g][m] x_t[m]).  Every check below is a
closed form or a hand-worked case, none a re-typed formula.
"""
import numpy as np
import pytest

import oracle


def rand_conv(rng, B, P, d, integer=False):
    if integer:
        return (rng.integers(-3, 4, size=(B, P, d)).astype(np.float64),
                rng.integers(-3, 4, size=(B, d)).astype(np.float64),
                rng.integers(-2, 3, size=(2, d)).astype(np.float64),
                rng.integers(-1, 2, size=(2, d // 16, d)).astype(np.float64))
    return (rng.standard_normal((B, P, d)), rng.standard_normal((B, d)),
            rng.standard_normal((2, d)), rng.standard_normal((2, d // 16, d)) / np.sqrt(d))


def test_hand_worked_two_positions():
    """d = 16 (one group), P = 2.  x_prev = 1, x_0[c] = c, x_1 = 2; base0 = 1,
    base1 = 0.5; the tap-0 correction reads channel 0 of the current state,
    the tap-1 correction channel 1.
      t = 0: corr = (x_0[0], x_0[1]) = (0, 1): k0 = 1, k1 = 1.5,
             y_0[c] = c + 1.5 * 1
      t = 1: corr = (2, 2): k0 = 3, k1 = 2.5, y_1[c] = 3 * 2 + 2.5 * c"""
    d = 16
    c = np.arange(d, dtype=np.float64)
    x = np.stack([c, np.full(d, 2.0)])[None]
    xp = np.ones((1, d))
    base = np.stack([np.ones(d), np.full(d, 0.5)])
    Wc = np.zeros((2, 1, d))
    Wc[0, 0, 0] = 1.0
    Wc[1, 0, 1] = 1.0
    y, _ = oracle.conv2(x, xp, base, Wc)
    assert np.array_equal(y[0, 0], c + 1.5)
    assert np.array_equal(y[0, 1], 6.0 + 2.5 * c)


def test_zero_correction_is_a_fixed_two_tap_filter():
    rng = np.random.default_rng(1)
    x, xp, base, Wc = rand_conv(rng, 3, 5, 64)
    y, _ = oracle.conv2(x, xp, base, np.zeros_like(Wc))
    prev = np.concatenate([xp[:, None], x[:, :-1]], axis=1)
    assert np.array_equal(y, base[0] * x + base[1] * prev)


def test_identity_and_shift():
    rng = np.random.default_rng(2)
    x, xp, _, Wc = rand_conv(rng, 2, 4, 32)
    d = 32
    y, _ = oracle.conv2(x, xp, np.stack([np.ones(d), np.zeros(d)]), np.zeros_like(Wc))
    assert np.array_equal(y, x)
    y, _ = oracle.conv2(x, xp, np.stack([np.zeros(d), np.ones(d)]), np.zeros_like(Wc))
    assert np.array_equal(y[:, 0], xp)
    assert np.array_equal(y[:, 1:], x[:, :-1])


@pytest.mark.parametrize("tap", [0, 1])
@pytest.mark.parametrize("g,m", [(0, 5), (2, 40), (3, 0)])
def test_correction_is_shared_by_one_group_and_reads_the_current_state(tap, g, m):
    """A one-hot correction row (group g, channel m) with zero base: only the
    16 channels of group g move, by x_t[m] times the tap's input -- x_t for
    tap 0, x_{t-1} for tap 1 -- so the correction reads the current state."""
    rng = np.random.default_rng(10 + 7 * g + m + tap)
    d = 64
    x, xp, _, _ = rand_conv(rng, 2, 3, d)
    Wc = np.zeros((2, d // 16, d))
    Wc[tap, g, m] = 1.0
    y, _ = oracle.conv2(x, xp, np.zeros((2, d)), Wc)
    prev = np.concatenate([xp[:, None], x[:, :-1]], axis=1)
    src = x if tap == 0 else prev
    want = np.zeros_like(x)
    want[..., 16 * g:16 * g + 16] = x[..., m:m + 1] * src[..., 16 * g:16 * g + 16]
    assert np.array_equal(y, want)


def test_linear_in_base_and_sigma_bounds():
    """With the correction fixed, y is linear in the base; |y| <= sigma."""
    rng = np.random.default_rng(3)
    x, xp, base, Wc = rand_conv(rng, 2, 6, 48, integer=True)
    y1, s1 = oracle.conv2(x, xp, base, Wc)
    y2, _ = oracle.conv2(x, xp, 2 * base, Wc)
    y0, _ = oracle.conv2(x, xp, np.zeros_like(base), Wc)
    assert np.array_equal(y2 - y1, y1 - y0)          # integers: exact
    assert np.all(np.abs(y1) <= s1)
    x, xp, base, Wc = rand_conv(rng, 2, 6, 48)
    y, s = oracle.conv2(x, xp, base, Wc)
    assert np.all(np.abs(y) <= s * (1 + 1e-12))


def test_p1_reads_only_the_verified_token():
    rng = np.random.default_rng(4)
    x, xp, base, Wc = rand_conv(rng, 3, 1, 32)
    y, _ = oracle.conv2(x, xp, base, np.zeros_like(Wc))
    assert np.array_equal(y[:, 0], base[0] * x[:, 0] + base[1] * xp)
