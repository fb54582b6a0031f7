"""Integer-weight categorical sampling, the accept test and the residual
distribution (oracle side, test infrastructure).

The pages fix WHAT is sampled: each drafted token is kept with probability
min(1, p(x)/q(x)); on the first rejection one token is drawn from the
normalised positive part of p - q; if every drafted token is kept, one more
token is drawn from the verifier (paperglide reader, "The Psi-Speculative
Sampler"; picx.dev summary, "Psi-Speculative Sampler").  They do not fix the
arithmetic.  This module fixes one, so that the HIP path and the oracle take the
same decision from the same fp32 logits and the same 24-bit uniform U:

* x_v = fp32((z_v - max z) * inv_temp) (two fp32 round-to-nearest-even ops);
* weight W_v = 0 if x_v < -22, else floor(exp_c(x_v) * 2^31), an integer in
  [0, 2^31]; the row maximum always has weight 2^31;
* S = sum of W_v (exact integer; any summation order gives the same value);
* a categorical draw with U returns the smallest v whose running weight sum
  exceeds t = floor(U * S / 2^24), so a zero-weight entry is never chosen;
* the accept test keeps draft token d iff U * Wq[d] * Sp < Wp[d] * Sq * 2^24,
  i.e. U / 2^24 < (Wp[d]/Sp) / (Wq[d]/Sq);
* the residual weights are R_v = max(0, Wp_v * Sq - Wq_v * Sp), proportional
  to max(0, p~ - q~); when they are all zero the draw falls back to p.

exp_c is a canonical exponential on [-22, 0] written from the mathematics:
Cody-Waite reduction by ln 2 split into a 16-bit head and an fp32 tail, a
degree-7 Taylor polynomial in Horner form, and an exact power-of-two scaling,
every operation a separately rounded fp32 op (no fused multiply-add).

Pins (tests/test_oracle_canonical.py): exp_c against fp64 math.exp over a sweep
of every fp32 in [-22, 0] at a stride, plus exp_c(0) = 1; categorical draws
against exhaustive counting over all 2^24 values of U on tiny rows; accept
probabilities against the closed form min(1, p/q); residual against the
textbook max(0, p - q).
"""
import math
from bisect import bisect_right
from itertools import accumulate

import numpy as np

F32 = np.float32
TWO24 = 1 << 24
X_CUTOFF = F32(-22.0)

# fp32 constants, each derived from its mathematical definition.
LOG2E_F = F32(1.0 / math.log(2.0))
LN2_HI = F32(45426.0 / 65536.0)                      # ln 2 to 16 significant bits
LN2_LO = F32(math.log(2.0) - 45426.0 / 65536.0)      # fp32 of the remainder
TAYLOR = [F32(1.0 / math.factorial(k)) for k in range(8)]
TWO31_F = F32(2.0 ** 31)


def exp_c(x):
    """Canonical fp32 exponential for x in [-22, 0] (array or scalar)."""
    x = np.asarray(x, dtype=F32)
    # subnormal inputs underflow harmlessly (n = 0, every r-term vanishes)
    with np.errstate(all="raise", under="ignore"):
        n = np.rint(x * LOG2E_F).astype(F32)
        r = (x - n * LN2_HI) - n * LN2_LO
        p = np.full_like(r, TAYLOR[7])
        for k in range(6, -1, -1):
            p = p * r
            p = p + TAYLOR[k]
        out = np.ldexp(p, n.astype(np.int32))
    return out.astype(F32)


def scaled_logits(z, inv_temp):
    """x = fp32((z - max z) * inv_temp) for one fp32 logit row."""
    z = np.asarray(z, dtype=F32)
    if not np.all(np.isfinite(z)):
        raise ValueError("non-finite logit in a sampled row")
    m = z.max()
    return (z - m) * F32(inv_temp)


def row_weights(z, inv_temp):
    """Integer weights W (uint64 array) and their exact sum S (Python int)."""
    x = scaled_logits(z, inv_temp)
    keep = x >= X_CUTOFF
    e = exp_c(np.where(keep, x, F32(0.0)))
    w = np.floor(e * TWO31_F).astype(np.uint64)
    w[~keep] = 0
    return w, int(w.sum(dtype=np.uint64))


def weight_of(z, inv_temp, v):
    """W_v alone (same arithmetic as ``row_weights`` for one entry)."""
    x = scaled_logits(z, inv_temp)[v]
    if x < X_CUTOFF:
        return 0
    return int(np.floor(exp_c(x) * TWO31_F))


def categorical(weights, u):
    """Smallest index whose running weight sum exceeds floor(u * S / 2^24).

    ``weights`` is any sequence of non-negative integers with S > 0.
    """
    if isinstance(weights, np.ndarray) and weights.dtype == np.uint64:
        # uint64 rows (W_v <= 2^31, V < 2^20): the running sum stays below 2^51
        cum = np.cumsum(weights, dtype=np.uint64)
        s = int(cum[-1])
        if s <= 0:
            raise ValueError("categorical draw over an all-zero weight row")
        t = (int(u) * s) >> 24
        return int(np.searchsorted(cum, np.uint64(t), side="right"))
    cum = list(accumulate(int(w) for w in weights))
    s = cum[-1]
    if s <= 0:
        raise ValueError("categorical draw over an all-zero weight row")
    t = (int(u) * s) >> 24
    return bisect_right(cum, t)


def accept(wq_d, sq, wp_d, sp, u):
    """Keep the draft token iff U * Wq[d] * Sp < Wp[d] * Sq * 2^24."""
    return int(u) * int(wq_d) * int(sp) < int(wp_d) * int(sq) * TWO24


def residual_weights(wp, sp, wq, sq):
    """R_v = max(0, Wp_v * Sq - Wq_v * Sp) as Python ints."""
    sp, sq = int(sp), int(sq)
    return [max(0, int(a) * sq - int(b) * sp) for a, b in zip(wp.tolist(), wq.tolist())]
