"""Shared helpers of the GPU parity tests (test code, not product code)."""
import math
import os
import sys
import time

import numpy as np
import torch

from oracle import canonical as cn
from oracle.philox import uniform24

LOGIT_ATOL = 2e-2     # bf16 GPU path vs fp64 oracle (stated by the parity target)
LOGIT_RTOL = 1e-2

_T0 = time.time()


def progress(msg):
    """Progress line on stderr and in gpurun_out/progress.log (long GPU tests)."""
    line = "[%7.1fs] %s" % (time.time() - _T0, msg)
    print(line, file=sys.stderr, flush=True)
    out = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "gpurun_out")
    if os.path.isdir(out):
        with open(os.path.join(out, "progress.log"), "a") as f:
            f.write(line + "\n")


def gpu_or_fail():
    """The GPU tests run only where a GPU exists; there, the library must load."""
    import lossless_decoding_uno_amd as U
    assert torch.cuda.is_available(), "GPU test collected on a machine without a GPU"
    U.load_library()
    return U


def assert_logits_close(got, ref, what):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    err = np.abs(got - ref)
    bound = LOGIT_ATOL + LOGIT_RTOL * np.abs(ref)
    bad = err > bound
    assert not bad.any(), "%s: %d / %d logits outside tolerance, worst %.3g at %s" % (
        what, int(bad.sum()), bad.size, float(err.max()), np.unravel_index(np.argmax(err), err.shape))
    return float(err.max())


def u24(seed, slot, j, b, step):
    return uniform24(seed, slot, j, b, step)


def cat_margin(weights, u):
    """Probability-mass distance of draw u from the edges of the chosen interval."""
    w = np.asarray(weights, dtype=object) if not isinstance(weights, np.ndarray) else weights
    cum = np.cumsum(np.array([int(x) for x in w], dtype=object))
    s = int(cum[-1])
    t = (int(u) * s) >> 24
    v = int(np.searchsorted(cum.astype(float), float(t), side="right"))
    # exact recheck with ints
    while v > 0 and int(cum[v - 1]) > t:
        v -= 1
    while int(cum[v]) <= t:
        v += 1
    lo = int(cum[v - 1]) if v > 0 else 0
    hi = int(cum[v])
    return v, min(t - lo, hi - 1 - t) / s


def shift_bound(max_dz, inv_temp, factor=2.0):
    """Bound on the change of a categorical CDF when every logit moves by at most
    max_dz (probabilities change by a factor within exp(+-2 dz/T))."""
    return math.expm1(factor * float(max_dz) * float(inv_temp))


def kv_to_logical(kv, layer, b, n):
    """K [n, Hkv, hd] and V [n, Hkv, hd] of positions 0..n-1 of sequence b (fp64)."""
    ps = kv.page_size
    pages = kv.page_table[b].long().cpu()
    pos = torch.arange(n)
    pg, sl = pages[pos // ps], pos % ps
    k = kv.k_pages[layer].cpu()[pg, :, sl, :]             # [n, Hkv, hd]
    v = kv.v_pages[layer].cpu()[pg, :, :, sl]             # [n, Hkv, hd]
    return k.double().numpy(), v.double().numpy()


def load_kv_logical(kv, b, k_log, v_log):
    """Write logical K/V [L, n, Hkv, hd] (positions 0..n-1) into sequence b's pages."""
    ps = kv.page_size
    n = k_log.shape[1]
    pages = kv.page_table[b].long()
    pos = torch.arange(n, device=kv.k_pages.device)
    pg, sl = pages[pos // ps], pos % ps
    k = k_log.to(kv.k_pages.device, torch.bfloat16)
    v = v_log.to(kv.k_pages.device, torch.bfloat16)
    for li in range(k.shape[0]):
        kv.k_pages[li][pg, :, sl, :] = k[li]
        kv.v_pages[li][pg, :, :, sl] = v[li]
