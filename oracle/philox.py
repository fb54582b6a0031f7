"""Philox4x64-10 counter-based generator (oracle side, test infrastructure).

Definition: Salmon, Moraes, Dror, Shaw, "Parallel Random Numbers: As Easy as
1, 2, 3" (SC'11), the Philox-4x64 bijection with 10 rounds.  One round maps the
counter (c0, c1, c2, c3) under key (k0, k1) to

    (hi(M1*c2) ^ c1 ^ k0,  lo(M1*c2),  hi(M0*c0) ^ c3 ^ k1,  lo(M0*c0))

and the key is bumped by the Weyl constants (W0, W1) between rounds.

The pages draw the accept test and the resampling "at random" without naming a
generator (paperglide reader, "The Psi-Speculative Sampler").  A counter-based
generator makes every draw a pure function of (seed, slot, position, sequence,
step), so the HIP path and this oracle can take identical decisions without
sharing a table.  Pinned against ``numpy.random.Philox`` (an independent C
implementation of the same 4x64-10 variant) in the tests.

Counter layout used by the decode step: counter = (slot, j, b, step),
key = (seed, 0); the 24-bit uniform is the top 24 bits of output word 0.
"""
import numpy as np

MASK64 = (1 << 64) - 1
PHILOX_M0 = 0xD2E7470EE14C6C93
PHILOX_M1 = 0xCA5A826395121157
PHILOX_W0 = 0x9E3779B97F4A7C15   # golden ratio
PHILOX_W1 = 0xBB67AE8584CAA73B   # sqrt(3) - 1

SLOT_DRAFT = 0     # draft token j+1 is drawn with j
SLOT_ACCEPT = 1    # accept test of draft i uses j = i - 1
SLOT_EXTRA = 2     # residual / bonus token uses j = a
SLOT_NOISE = 3     # uniform-prior noise token of draft row j >= 1
SLOT_PASS = 4      # sample j of intermediate draft pass i uses slot SLOT_PASS + i
SLOT_KEEP = 64     # corrector after draft pass i: keep-or-remask decision of row j
SLOT_RENOISE = 128  # corrector after draft pass i: fresh uniform token of a remasked row j
MAX_PASSES = 60    # draft passes per step (slots SLOT_PASS + i stay below SLOT_KEEP)


def philox4x64_10(counter, key):
    """Return the four 64-bit output words for one counter (Python ints)."""
    c0, c1, c2, c3 = (int(v) & MASK64 for v in counter)
    k0, k1 = (int(v) & MASK64 for v in key)
    for rnd in range(10):
        if rnd:
            k0 = (k0 + PHILOX_W0) & MASK64
            k1 = (k1 + PHILOX_W1) & MASK64
        p0 = PHILOX_M0 * c0
        p1 = PHILOX_M1 * c2
        c0, c1, c2, c3 = ((p1 >> 64) ^ c1 ^ k0, p1 & MASK64,
                          (p0 >> 64) ^ c3 ^ k1, p0 & MASK64)
    return c0, c1, c2, c3


def uniform24(seed, slot, j, b, step):
    """24-bit uniform integer U in [0, 2^24) for one decision."""
    return philox4x64_10((slot, j, b, step), (seed, 0))[0] >> 40


def token_id(seed, slot, j, b, step, vocab):
    """Uniform token floor(w * vocab / 2^64), w = word 0 at counter (slot, j, b, step)."""
    return (philox4x64_10((slot, j, b, step), (seed, 0))[0] * int(vocab)) >> 64


def noise_id(seed, j, b, step, vocab):
    """Uniform noise token of draft row j for a uniform-state prior:
    floor(w * vocab / 2^64), w = word 0 at counter (SLOT_NOISE, j, b, step)."""
    return token_id(seed, SLOT_NOISE, j, b, step, vocab)


# ---- vectorised form (numpy uint64), used for large batches of draws ----

_M32 = np.uint64(0xFFFFFFFF)
_S32 = np.uint64(32)


def _mulhilo(a, b):
    """Full 64x64 -> 128 product of uint64 arrays, as (hi, lo)."""
    a = np.asarray(a, dtype=np.uint64)
    b = np.asarray(b, dtype=np.uint64)
    a_lo, a_hi = a & _M32, a >> _S32
    b_lo, b_hi = b & _M32, b >> _S32
    ll = a_lo * b_lo
    lh = a_lo * b_hi
    hl = a_hi * b_lo
    hh = a_hi * b_hi
    mid = (ll >> _S32) + (lh & _M32) + (hl & _M32)
    hi = hh + (lh >> _S32) + (hl >> _S32) + (mid >> _S32)
    lo = (ll & _M32) | ((mid & _M32) << _S32)
    return hi, lo


def philox4x64_10_np(c0, c1, c2, c3, k0, k1):
    """Vectorised Philox4x64-10 over broadcastable uint64 arrays."""
    with np.errstate(over="ignore"):
        c0, c1, c2, c3 = (np.asarray(v, dtype=np.uint64) for v in (c0, c1, c2, c3))
        c0, c1, c2, c3 = np.broadcast_arrays(c0, c1, c2, c3)
        k0 = np.uint64(int(k0) & MASK64)
        k1 = np.uint64(int(k1) & MASK64)
        w0, w1 = np.uint64(PHILOX_W0), np.uint64(PHILOX_W1)
        m0, m1 = np.uint64(PHILOX_M0), np.uint64(PHILOX_M1)
        for rnd in range(10):
            if rnd:
                k0 = k0 + w0
                k1 = k1 + w1
            hi0, lo0 = _mulhilo(m0, c0)
            hi1, lo1 = _mulhilo(m1, c2)
            c0, c1, c2, c3 = hi1 ^ c1 ^ k0, lo1, hi0 ^ c3 ^ k1, lo0
    return c0, c1, c2, c3


def uniform24_np(seed, slot, j, b, step):
    """Vectorised ``uniform24``; arguments broadcast, result uint64."""
    out0 = philox4x64_10_np(slot, j, b, step, seed, 0)[0]
    return out0 >> np.uint64(40)
