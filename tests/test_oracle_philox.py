"""Pins of the oracle's Philox4x64-10 and uniform mapping (CPU only)."""

import numpy as np
import pytest

from oracle import philox

MASK = (1 << 64) - 1


def numpy_block(counter, key):
    """numpy's Philox increments its 256-bit counter before it generates."""
    c = sum(int(x) << (64 * i) for i, x in enumerate(counter))
    c = (c - 1) % (1 << 256)
    prev = np.array([(c >> (64 * i)) & MASK for i in range(4)], dtype=np.uint64)
    g = np.random.Philox(key=np.array(key, dtype=np.uint64), counter=prev)
    return tuple(int(x) for x in g.random_raw(4))


CASES = [
    ((0, 0, 0, 0), (0, 0)),
    ((1, 0, 0, 0), (0, 0)),
    ((5, 3, 7, 0), (123456789, 0)),
    ((MASK, 1, 1 << 63, 9), (MASK, MASK)),
    ((0x243F6A8885A308D3, 0x13198A2E03707344, 0xA4093822299F31D0, 0x082EFA98EC4E6C89),
     (0x452821E638D01377, 0xBE5466CF34E90C6C)),
]


@pytest.mark.parametrize("counter,key", CASES)
def test_matches_numpy_philox(counter, key):
    assert philox.philox4x64_10(counter, key) == numpy_block(counter, key)


def test_many_random_blocks_match_numpy():
    rng = np.random.default_rng(3)
    for _ in range(200):
        ctr = tuple(int(x) for x in rng.integers(0, 2**63, 4, dtype=np.int64))
        key = tuple(int(x) for x in rng.integers(0, 2**63, 2, dtype=np.int64))
        assert philox.philox4x64_10(ctr, key) == numpy_block(ctr, key)


def test_uniform_is_exact_in_fp32_and_open_interval():
    for w in [0, 1, (1 << 41) - 1, 1 << 41, MASK, MASK - (1 << 41)]:
        u = philox.uniform_from_word(w)
        assert 0.0 < u < 1.0
        assert float(np.float32(u)) == u
        k = u * 2**24
        assert k == int(k) and int(k) % 2 == 1
    assert philox.uniform_from_word(0) == 2.0 ** -24
    assert philox.uniform_from_word(MASK) == 1.0 - 2.0 ** -24


def test_step_uniforms_layout_and_spread():
    u = philox.step_uniforms(seed=7, step=3, C=5, N=4)
    assert u.shape == (5, 8)
    w = philox.philox4x64_10((6, 2, 3, 0), (7, 0))[0]
    assert u[2, 6] == philox.uniform_from_word(w)
    big = philox.step_uniforms(seed=1, step=0, C=400, N=4).ravel()
    # 3200 draws: mean and a coarse histogram of U(0,1)
    assert abs(big.mean() - 0.5) < 4 * np.sqrt(1 / 12 / big.size)
    hist, _ = np.histogram(big, bins=10, range=(0, 1))
    assert hist.min() > 250
