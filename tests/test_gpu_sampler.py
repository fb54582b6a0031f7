"""GPU parity of the sampler (uno_draft_sample, uno_spec_accept) with the
oracle: bit-exact tokens, accept lengths and committed tokens on identical
fp32 logits and Philox counters (sampler-only workload: AR logits N(0, 3^2),
draft logits = AR + N(0, 0.5^2) noise)."""
import numpy as np
import pytest
import torch

import synth
from oracle import spec as ospec

from gpu_util import gpu_or_fail, progress

pytestmark = pytest.mark.gpu

SEED = 0


def _steps(B):
    return np.array([3 + 7 * b for b in range(B)], dtype=np.uint64)


def _gpu_draft_sample(U, zq, inv_t, steps, given_max=False, row_max=None):
    z = torch.from_numpy(zq).cuda()
    st = torch.from_numpy(steps.astype(np.uint64)).cuda()
    tok = torch.full(zq.shape[:2], -7, dtype=torch.int32, device="cuda")
    status = torch.zeros(zq.shape[0], dtype=torch.int32, device="cuda")
    if given_max and row_max is None:
        row_max = z.amax(dim=-1).contiguous()
    U.draft_sample(z, inv_t, SEED, st, tok, status, row_max=row_max)
    torch.cuda.synchronize()
    return tok.cpu().numpy(), status.cpu().numpy()


def _oracle_drafts(zq, inv_t, steps, rows=None):
    B, K, _ = zq.shape
    out = np.zeros((B, K), dtype=np.int64)
    for b in (range(B) if rows is None else rows):
        out[b] = ospec.draft_sample(zq[b], inv_t, ospec.PhiloxDraws(SEED, b, int(steps[b])))
    return out


@pytest.mark.parametrize("given_max", [False, True])
@pytest.mark.parametrize("B,K,V", [(3, 5, 1000), (2, 3, 1003), (1, 1, 16), (4, 2, 4096),
                                   (2, 4, 257)])
def test_draft_sample_bit_exact_small(B, K, V, given_max):
    """Two passes per row (maximum, then weights) or one (maximum given)."""
    U = gpu_or_fail()
    zq, _ = synth.sampler_logits(B, K, V, seed=V)
    for inv_t in (1.0, np.float32(1 / 0.7)):
        steps = _steps(B)
        got, status = _gpu_draft_sample(U, zq, inv_t, steps, given_max)
        assert (status == 0).all()
        np.testing.assert_array_equal(got, _oracle_drafts(zq, inv_t, steps))


def test_given_row_max_below_an_entry_is_flagged():
    """A given maximum below one of its row's entries (or a non-finite entry)
    flags the row and skips its draw; the other rows are unaffected."""
    U = gpu_or_fail()
    zq, _ = synth.sampler_logits(2, 3, 512, seed=3)
    rm = torch.from_numpy(zq.max(axis=-1)).cuda()
    rm[1, 1] -= 0.5
    got, status = _gpu_draft_sample(U, zq, 1.0, _steps(2), row_max=rm)
    assert status[0] == 0 and status[1] & U.DEV_NONFINITE
    assert got[1, 1] == -1
    np.testing.assert_array_equal(got[0], _oracle_drafts(zq, 1.0, _steps(2), rows=[0])[0])


def test_draft_sample_flags_nonfinite_rows():
    U = gpu_or_fail()
    zq, _ = synth.sampler_logits(2, 3, 64, seed=1)
    zq[1, 2, 5] = np.nan
    got, status = _gpu_draft_sample(U, zq, 1.0, _steps(2))
    assert status[0] == 0 and status[1] & U.DEV_NONFINITE
    assert got[1, 2] == -1
    np.testing.assert_array_equal(got[0], _oracle_drafts(zq, 1.0, _steps(2), rows=[0])[0])


def _gpu_accept(U, zq, zp, drafts, inv_t, steps, forced=None, given_max=False):
    B, K, V = zq.shape
    dev = "cuda"
    out = dict(a=torch.full((B,), -9, dtype=torch.int32, device=dev),
               c=torch.full((B, K + 1), -9, dtype=torch.int32, device=dev),
               e=torch.full((B,), -9, dtype=torch.int32, device=dev),
               s=torch.zeros(B, dtype=torch.int32, device=dev))
    ws = U.alloc_workspace(U.spec_accept_workspace_bytes(B, K))
    f = None if forced is None else torch.from_numpy(forced.astype(np.int32)).to(dev)
    zq_d, zp_d = torch.from_numpy(zq).to(dev), torch.from_numpy(zp).to(dev)
    mq = zq_d.amax(dim=-1).contiguous() if given_max else None
    mp = zp_d.amax(dim=-1).contiguous() if given_max else None
    U.spec_accept(zq_d, zp_d, torch.from_numpy(drafts.astype(np.int32)).to(dev), inv_t, SEED,
                  torch.from_numpy(steps).to(dev), out["a"], out["c"], out["e"], ws,
                  forced_accept=f, status=out["s"], draft_row_max=mq, verify_row_max=mp)
    torch.cuda.synchronize()
    return {k: v.cpu().numpy() for k, v in out.items()}


def _check_accept(zq, zp, drafts, inv_t, steps, got, rows, forced=None):
    K = zq.shape[1]
    for b in rows:
        a, comm, extra = ospec.spec_accept(zq[b], zp[b], list(drafts[b]), inv_t,
                                           ospec.PhiloxDraws(SEED, b, int(steps[b])),
                                           None if forced is None else int(forced[b]))
        assert got["s"][b] == 0
        assert got["a"][b] == a, (b, got["a"][b], a)
        assert got["e"][b] == extra, (b, got["e"][b], extra)
        np.testing.assert_array_equal(got["c"][b], comm + [-1] * (K + 1 - len(comm)))


@pytest.mark.parametrize("given_max", [False, True])
@pytest.mark.parametrize("B,K,V,sig,noise", [(4, 6, 1000, 3.0, 0.5), (3, 8, 512, 1.0, 2.0),
                                             (2, 1, 64, 3.0, 0.5), (5, 4, 16, 0.5, 3.0)])
def test_spec_accept_bit_exact_small(B, K, V, sig, noise, given_max):
    U = gpu_or_fail()
    zq, zp = synth.sampler_logits(B, K, V, seed=K * V, sigma_p=sig, sigma_noise=noise)
    steps = _steps(B)
    for inv_t in (1.0, np.float32(1 / 0.7)):
        drafts = _oracle_drafts(zq, inv_t, steps)
        got = _gpu_accept(U, zq, zp, drafts, inv_t, steps, given_max=given_max)
        _check_accept(zq, zp, drafts, inv_t, steps, got, range(B))
        forced = synth.forced_accepts(B, K, 1, seed=V)[0]
        got = _gpu_accept(U, zq, zp, drafts, inv_t, steps, forced, given_max=given_max)
        _check_accept(zq, zp, drafts, inv_t, steps, got, range(B), forced)


def test_spec_accept_rejects_bad_forced_length():
    U = gpu_or_fail()
    zq, zp = synth.sampler_logits(2, 3, 64, seed=5)
    steps = _steps(2)
    drafts = _oracle_drafts(zq, 1.0, steps)
    got = _gpu_accept(U, zq, zp, drafts, 1.0, steps, np.array([1, 9]))
    assert got["s"][1] & U.DEV_BAD_ACCEPT and got["s"][0] == 0
    assert (got["c"][1] == -1).all() and got["e"][1] == -1


def test_sampler_only_workload_full_size():
    """Batch 64 x K 16 x vocab 151936: draft sampling and accept, every sequence."""
    U = gpu_or_fail()
    B, K, V = 64, 16, 151936
    zq, zp = synth.sampler_logits(B, K, V, seed=2)
    steps = np.zeros(B, dtype=np.uint64)
    progress("full sampler workload: logits ready")
    got_d, st = _gpu_draft_sample(U, zq, 1.0, steps)
    assert (st == 0).all()
    ref_d = _oracle_drafts(zq, 1.0, steps)
    np.testing.assert_array_equal(got_d, ref_d)
    got_d1, st = _gpu_draft_sample(U, zq, 1.0, steps, given_max=True)
    assert (st == 0).all()
    np.testing.assert_array_equal(got_d1, ref_d)
    progress("full sampler workload: drafts bit-exact (two-pass and one-pass rows)")
    got = _gpu_accept(U, zq, zp, ref_d, 1.0, steps)
    _check_accept(zq, zp, ref_d, 1.0, steps, got, range(B))
    got = _gpu_accept(U, zq, zp, ref_d, 1.0, steps, given_max=True)
    _check_accept(zq, zp, ref_d, 1.0, steps, got, range(B))
    progress("full sampler workload: accept bit-exact, mean a = %.2f" % got["a"].mean())
    forced = synth.forced_accepts(B, K, 1, seed=2)[0]
    got = _gpu_accept(U, zq, zp, ref_d, 1.0, steps, forced)
    _check_accept(zq, zp, ref_d, 1.0, steps, got, range(0, B, 4), forced)
    inv_t = np.float32(1 / 0.7)
    got_d7, _ = _gpu_draft_sample(U, zq, inv_t, steps)
    ref_d7 = _oracle_drafts(zq, inv_t, steps)
    np.testing.assert_array_equal(got_d7, ref_d7)
    got = _gpu_accept(U, zq, zp, ref_d7, inv_t, steps)
    _check_accept(zq, zp, ref_d7, inv_t, steps, got, range(0, B, 4))
    progress("full sampler workload: T = 0.7 bit-exact")
