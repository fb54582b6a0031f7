"""uno_spec_accept_noalloc (the accept step on the library's static per-GPU
scratch, for callers that cannot allocate) against uno_spec_accept with a
caller workspace: accept lengths, committed tokens, extra tokens and device
status flags bit-identical, on two calls in a row, the second smaller (the
scratch keeps the first call's contents), and the size limit enforced on the
host."""
import numpy as np
import pytest
import torch

import synth

from gpu_util import gpu_or_fail, progress

pytestmark = pytest.mark.gpu


def _case(B, K, V, seed, forced=None, nonfinite_row=None):
    zq, zp = synth.sampler_logits(B, K, V, seed)
    if nonfinite_row is not None:
        b, j = nonfinite_row
        zp[b, j, 7] = np.inf
    rng = np.random.default_rng([seed, 3])
    drafts = rng.integers(0, V, size=(B, K)).astype(np.int32)
    return (torch.from_numpy(zq).cuda(), torch.from_numpy(zp).cuda(),
            torch.from_numpy(drafts).cuda(),
            None if forced is None else torch.from_numpy(forced).cuda())


def _run(U, zq, zp, d, forced, noalloc):
    B, K, _ = zq.shape
    step = torch.arange(B, dtype=torch.int64).to(torch.uint64).cuda()
    a = torch.full((B,), -7, dtype=torch.int32, device="cuda")
    c = torch.full((B, K + 1), -7, dtype=torch.int32, device="cuda")
    e = torch.full((B,), -7, dtype=torch.int32, device="cuda")
    st = torch.zeros(B, dtype=torch.int32, device="cuda")
    if noalloc:
        U.spec_accept_noalloc(zq, zp, d, 1.0, 3, step, a, c, e, forced_accept=forced, status=st)
    else:
        ws = U.alloc_workspace(U.spec_accept_workspace_bytes(B, K))
        U.spec_accept(zq, zp, d, 1.0, 3, step, a, c, e, ws, forced_accept=forced, status=st)
    torch.cuda.synchronize()
    return [t.cpu().numpy() for t in (a, c, e, st)]


def test_noalloc_accept_equals_workspace_accept_two_calls():
    U = gpu_or_fail()
    cases = [
        # first call: many rows, one sequence with a non-finite verify row
        dict(B=48, K=16, V=151936, seed=1, nonfinite_row=(5, 3)),
        # second call, smaller, with forced accept lengths 0..K
        dict(B=3, K=5, V=4096, seed=2, forced=np.array([0, 5, 2], dtype=np.int32)),
    ]
    for i, kw in enumerate(cases):
        progress("noalloc accept call %d: B=%d K=%d V=%d" % (i, kw["B"], kw["K"], kw["V"]))
        zq, zp, d, forced = _case(**kw)
        ref = _run(U, zq, zp, d, forced, noalloc=False)
        got = _run(U, zq, zp, d, forced, noalloc=True)
        for r, g, name in zip(ref, got, ("accept_len", "committed", "extra", "status")):
            np.testing.assert_array_equal(g, r, err_msg="call %d %s" % (i, name))
        if "nonfinite_row" in kw:
            assert got[3][kw["nonfinite_row"][0]] == U.DEV_NONFINITE
        assert (got[0] >= 0).all()


def test_noalloc_accept_rejects_shapes_past_its_scratch():
    U = gpu_or_fail()
    zq = torch.zeros((2049, 16, 16), dtype=torch.float32, device="cuda")   # 2*B*K > 65536
    d = torch.zeros((2049, 16), dtype=torch.int32, device="cuda")
    step = torch.zeros(2049, dtype=torch.uint64, device="cuda")
    a = torch.empty(2049, dtype=torch.int32, device="cuda")
    c = torch.empty((2049, 17), dtype=torch.int32, device="cuda")
    with pytest.raises(U.UnoError, match="workspace"):
        U.spec_accept_noalloc(zq, zq, d, 1.0, 0, step, a, c, a)
