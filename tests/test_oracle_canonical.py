"""Pins of the oracle's canonical sampler arithmetic.

exp_c against fp64 math.exp; categorical draws and accept tests against exact
counting over every value of the 24-bit uniform; the residual against the
textbook normalised max(0, p - q)."""
import math
from fractions import Fraction

import numpy as np
import pytest

from oracle import canonical as cn

TWO24 = 1 << 24


def _fp32_neg_range(lo_bits, hi_bits, stride):
    bits = np.arange(lo_bits, hi_bits + 1, stride, dtype=np.uint64).astype(np.uint32)
    return bits.view(np.float32)


def _ulp_err(x):
    e = cn.exp_c(x).astype(np.float64)
    ref = np.array([math.exp(float(v)) for v in x]) if x.size < 2000 else np.exp(x.astype(np.float64))
    ulp = np.spacing(ref.astype(np.float32)).astype(np.float64)
    return np.abs(e - ref) / ulp


def test_exp_c_zero_is_one():
    assert cn.exp_c(np.float32(0.0)) == np.float32(1.0)
    assert cn.exp_c(np.float32(-0.0)) == np.float32(1.0)


def test_exp_c_strided_sweep_within_2ulp():
    # every 257th fp32 in [-22, -0]: bit patterns 0x80000000 .. bits(-22)
    hi = int(np.float32(-22.0).view(np.uint32))
    x = _fp32_neg_range(0x80000000, hi, 257)
    assert _ulp_err(x).max() <= 2.0


def test_exp_c_against_math_exp_scalar():
    rng = np.random.default_rng(3)
    x = -rng.uniform(0, 22, size=1500).astype(np.float32)
    assert _ulp_err(x).max() <= 2.0


@pytest.mark.slow
def test_exp_c_full_sweep_within_2ulp():
    hi = int(np.float32(-22.0).view(np.uint32))
    worst = 0.0
    for start in range(0x80000000, hi + 1, 1 << 24):
        x = _fp32_neg_range(start, min(hi, start + (1 << 24) - 1), 1)
        worst = max(worst, float(_ulp_err(x).max()))
    assert worst <= 2.0


def test_row_weights_shape_of_target():
    rng = np.random.default_rng(4)
    z = (rng.standard_normal(4096) * 3).astype(np.float32)
    for inv_t in (1.0, 1.0 / 0.7):
        w, s = cn.row_weights(z, np.float32(inv_t))
        assert w.dtype == np.uint64 and w.max() == 2**31
        assert int(w[np.argmax(z)]) == 2**31
        assert s == sum(int(v) for v in w)
        x = (z.astype(np.float64) - z.max()) * inv_t
        soft = np.exp(x) / np.exp(x).sum()
        assert np.max(np.abs(w / s - soft)) < 1e-7
    z2 = np.array([0.0, -22.5, -30.0, -21.9], dtype=np.float32)
    w, _ = cn.row_weights(z2, np.float32(1.0))
    assert w[1] == 0 and w[2] == 0 and w[0] == 2**31


def _lowest_u(pred):
    """Smallest U in [0, 2^24] with pred(U) true (pred monotone false->true)."""
    lo, hi = 0, TWO24
    while lo < hi:
        mid = (lo + hi) // 2
        if pred(mid):
            hi = mid
        else:
            lo = mid + 1
    return lo


def _cat_counts(weights):
    V = len(weights)
    starts = [_lowest_u(lambda u, v=v: cn.categorical(weights, u) >= v) for v in range(V)]
    starts.append(TWO24)
    return [starts[v + 1] - starts[v] for v in range(V)]


@pytest.mark.parametrize("weights", [
    [5, 0, 7, 1, 2**31],
    [2**31, 2**31, 1, 0, 0, 3],
    [1, 2, 3],
    [0, 0, 9],
])
def test_categorical_exact_counts(weights):
    counts = _cat_counts(weights)
    S = sum(weights)
    assert sum(counts) == TWO24
    for w, c in zip(weights, counts):
        if w == 0:
            assert c == 0
        assert abs(Fraction(c, TWO24) - Fraction(w, S)) <= Fraction(1, TWO24)
    # monotone in U, and the numpy fast path agrees with the list path
    arr = np.array(weights, dtype=np.uint64)
    us = np.random.default_rng(1).integers(0, TWO24, 3000)
    idx = [cn.categorical(weights, int(u)) for u in np.sort(us)]
    assert idx == sorted(idx)
    assert idx == [cn.categorical(arr, int(u)) for u in np.sort(us)]


def test_categorical_brute_force_tiny_all_u():
    # small S: every U in [0, 2^24) evaluated through the numpy fast path
    w = np.array([3, 0, 1, 4], dtype=np.uint64)
    u = np.arange(TWO24, dtype=np.uint64)
    t = (u * np.uint64(8)) >> np.uint64(24)
    idx = np.searchsorted(np.cumsum(w), t, side="right")
    counts = np.bincount(idx, minlength=4)
    assert list(counts) == _cat_counts(w.tolist())
    for uu in (0, 1, 2**23, TWO24 - 1, 6291456):
        assert cn.categorical(w, uu) == idx[uu]


@pytest.mark.parametrize("seed", range(6))
def test_accept_probability_is_min_one_ratio(seed):
    rng = np.random.default_rng(seed)
    zq = (rng.standard_normal(64) * 2).astype(np.float32)
    zp = (rng.standard_normal(64) * 2).astype(np.float32)
    wq, sq = cn.row_weights(zq, 1.0)
    wp, sp = cn.row_weights(zp, 1.0)
    for d in range(64):
        if wq[d] == 0:
            continue
        thr = _lowest_u(lambda u: not cn.accept(int(wq[d]), sq, int(wp[d]), sp, u))
        ratio = Fraction(int(wp[d]), sp) / Fraction(int(wq[d]), sq)
        target = min(Fraction(1), ratio)
        assert abs(Fraction(thr, TWO24) - target) <= Fraction(1, TWO24)
        if ratio >= 1:
            assert thr == TWO24          # p >= q: always kept


def test_residual_is_normalised_positive_part():
    rng = np.random.default_rng(8)
    zq = (rng.standard_normal(50) * 2).astype(np.float32)
    zp = (rng.standard_normal(50) * 2).astype(np.float32)
    wq, sq = cn.row_weights(zq, 1.0)
    wp, sp = cn.row_weights(zp, 1.0)
    r = cn.residual_weights(wp, sp, wq, sq)
    diff = [max(Fraction(0), Fraction(int(a), sp) - Fraction(int(b), sq)) for a, b in zip(wp, wq)]
    tot_r, tot_d = sum(r), sum(diff)
    for rv, dv in zip(r, diff):
        assert Fraction(rv, tot_r) == dv / tot_d
    # identical rows leave nothing
    assert sum(cn.residual_weights(wp, sp, wp, sp)) == 0
