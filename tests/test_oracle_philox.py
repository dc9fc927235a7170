"""Pins for the oracle's counter-based uniforms (Philox4x64-10).

The sampling walk ("DFlash 2: Keep Drafting Parallel", section "A Lightweight
Path Selector": sampling draws from the same scores) needs one uniform per
draft position.  The generator is Philox4x64-10 from Salmon, Moraes, Dror and
Shaw, "Parallel Random Numbers: As Easy as 1, 2, 3" (SC 2011).  The oracle's
block function is checked against numpy's own Philox bit generator (an
independent implementation of the same published definition) and against the
published known answer for the all-zero counter and key; the mapping of
blocks to uniforms is checked word by word against numpy's raw output.
"""
import numpy as np
import pytest

import oracle

M64 = 2**64 - 1


def numpy_block(ctr_words, key_words) -> np.ndarray:
    """The block at counter value c from numpy's Philox: numpy advances its
    counter before each block, so it is seeded one below c (mod 2^256)."""
    c = sum(int(w) << (64 * i) for i, w in enumerate(ctr_words))
    # the key goes in as a uint64 array: a list of Python ints would pass
    # through float64 on numpy's side and lose its low bits
    g = np.random.Philox(counter=(c - 1) % 2**256, key=np.array([int(k) for k in key_words], dtype=np.uint64))
    return g.random_raw(4).astype(np.uint64)


def test_known_answer_zero_counter_and_key():
    """Published known answer of Philox4x64-10 for counter 0 and key 0."""
    got = oracle.philox4x64_10([0, 0, 0, 0], [0, 0])
    want = np.array([0x16554D9ECA36314C, 0xDB20FE9D672D0FDC,
                     0xD7E772CEE186176B, 0x7E68B68AEC7BA23B], dtype=np.uint64)
    assert np.array_equal(got, want)


@pytest.mark.parametrize("ctr,key", [
    ([1, 0, 0, 0], [0, 0]),
    ([0, 1, 0, 0], [0, 0]),
    ([0, 0, 1, 0], [0, 0]),
    ([0, 0, 0, 1], [0, 0]),
    ([5, 7, 0, 0], [0x1234, 0x99]),
    ([M64, M64, M64, M64], [M64, M64]),
    ([0x243F6A8885A308D3, 0x13198A2E03707344, 0xA4093822299F31D0, 0x082EFA98EC4E6C89],
     [0x452821E638D01377, 0xBE5466CF34E90C6C]),
])
def test_block_matches_numpy(ctr, key):
    assert np.array_equal(oracle.philox4x64_10(ctr, key), numpy_block(ctr, key))


def test_random_blocks_match_numpy():
    rng = np.random.default_rng(11)
    for _ in range(200):
        ctr = [int(x) for x in rng.integers(0, 2**64, size=4, dtype=np.uint64)]
        key = [int(x) for x in rng.integers(0, 2**64, size=2, dtype=np.uint64)]
        assert np.array_equal(oracle.philox4x64_10(ctr, key), numpy_block(ctr, key))


@pytest.mark.parametrize("seed,offset", [(0, 0), (1, 0), (0, 1), (0x9E3779B97F4A7C15, 12345), (M64, M64)])
def test_uniforms_are_top_24_bits_of_the_blocks(seed, offset):
    """Uniform i is word i mod 4 of the block at counter (i // 4, offset, 0, 0)
    under key (seed, 0), as (x >> 40) / 2^24; checked on 37 uniforms (ten
    blocks, the last one ragged) against numpy's raw words."""
    n = 37
    u = oracle.philox_uniforms(seed, offset, n)
    assert u.dtype == np.float32 and u.shape == (n,)
    for i in range(n):
        w = numpy_block([i // 4, offset, 0, 0], [seed, 0])[i % 4]
        assert int(u[i].astype(np.float64) * 2**24) == int(w) >> 40
        assert u[i].astype(np.float64) * 2**24 == np.floor(u[i].astype(np.float64) * 2**24)


def test_first_index_windows_agree():
    """A window [first, first + n) equals the same slice of the whole run."""
    whole = oracle.philox_uniforms(42, 3, 1001)
    for first, n in [(0, 1), (1, 4), (3, 9), (500, 501), (997, 4)]:
        assert np.array_equal(oracle.philox_uniforms(42, 3, n, first=first), whole[first:first + n])


def test_empty_and_range():
    assert oracle.philox_uniforms(1, 2, 0).shape == (0,)
    u = oracle.philox_uniforms(7, 0, 200_000)
    assert u.min() >= 0.0 and u.max() < 1.0


def test_uniform_distribution():
    """Kolmogorov-Smirnov against U(0, 1), a chi-square over 64 bins, and
    different seeds / offsets giving different streams."""
    from scipy import stats
    u = oracle.philox_uniforms(2024, 9, 200_000).astype(np.float64)
    assert stats.kstest(u, "uniform").pvalue > 1e-4
    counts = np.bincount((u * 64).astype(np.int64), minlength=64)
    assert stats.chisquare(counts).pvalue > 1e-4
    assert not np.array_equal(oracle.philox_uniforms(2024, 9, 64), oracle.philox_uniforms(2025, 9, 64))
    assert not np.array_equal(oracle.philox_uniforms(2024, 9, 64), oracle.philox_uniforms(2024, 10, 64))
    # neighbouring uniforms are uncorrelated
    assert abs(np.corrcoef(u[:-1], u[1:])[0, 1]) < 0.02
