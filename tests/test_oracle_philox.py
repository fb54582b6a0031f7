"""Pins of the oracle's Philox4x64-10 against numpy's independent C version."""
import numpy as np
import pytest

from oracle.philox import (SLOT_NOISE, noise_id, philox4x64_10, philox4x64_10_np, uniform24,
                           uniform24_np)

MASK = (1 << 64) - 1


def _numpy_words(counter, key):
    # numpy.random.Philox increments its 256-bit counter before each block, so
    # the block for counter c comes out of a generator started at c - 1.
    c = (counter[0] | counter[1] << 64 | counter[2] << 128 | counter[3] << 192) - 1
    c %= 1 << 256
    start = [(c >> (64 * i)) & MASK for i in range(4)]
    bg = np.random.Philox(key=np.array(key, dtype=np.uint64),
                          counter=np.array(start, dtype=np.uint64))
    return tuple(int(bg.random_raw()) for _ in range(4))


@pytest.mark.parametrize("trial", range(40))
def test_matches_numpy_philox(trial):
    rng = np.random.default_rng([99, trial])
    counter = [int(v) for v in rng.integers(0, 2**63, size=4, dtype=np.int64)]
    if trial % 4 == 0:
        counter = [trial, 3, 7, 11]          # small counters like the decode step's
    key = [int(v) for v in rng.integers(0, 2**63, size=2, dtype=np.int64)]
    if trial % 5 == 0:
        counter[0] = MASK                     # carry into the next word inside numpy
    assert philox4x64_10(counter, key) == _numpy_words(counter, key)


def test_vectorised_equals_scalar():
    rng = np.random.default_rng(5)
    c = rng.integers(0, 2**63, size=(4, 257), dtype=np.int64).astype(np.uint64)
    c[0, :3] = np.uint64(MASK)
    out = philox4x64_10_np(c[0], c[1], c[2], c[3], 0xDEADBEEFCAFEBABE, 17)
    for i in range(c.shape[1]):
        ref = philox4x64_10([int(c[k, i]) for k in range(4)], [0xDEADBEEFCAFEBABE, 17])
        assert tuple(int(o[i]) for o in out) == ref
    slot, j, b, s = 1, np.arange(16)[:, None], np.arange(8)[None, :], 42
    u = uniform24_np(7, slot, j, b, s)
    for jj in range(16):
        for bb in range(8):
            assert int(u[jj, bb]) == uniform24(7, slot, jj, bb, s)


def test_uniform24_range_and_spread():
    u = uniform24_np(0, 0, np.arange(100000), 3, 9)
    assert u.max() < 2**24
    # a fair 24-bit uniform: mean 2^23 within 5 sigma
    sigma = 2**24 / np.sqrt(12) / np.sqrt(u.size)
    assert abs(u.astype(np.float64).mean() - 2**23) < 5 * sigma


def test_noise_id_is_word0_times_vocab_over_2_64():
    """Uniform-prior noise tokens: floor(w * V / 2^64) of numpy's own word 0."""
    for (j, b, step, V) in [(1, 0, 0, 512), (15, 63, 1234, 151936), (7, 3, 99, 8)]:
        w = _numpy_words([SLOT_NOISE, j, b, step], [5, 0])[0]
        assert noise_id(5, j, b, step, V) == (w * V) >> 64


def test_noise_id_uniform_chi_square():
    from scipy import stats
    V = 64
    ids = [noise_id(0, j, b, s, V) for j in range(1, 16) for b in range(32) for s in range(20)]
    assert min(ids) >= 0 and max(ids) < V
    counts = np.bincount(ids, minlength=V)
    assert stats.chisquare(counts).pvalue > 0.01
