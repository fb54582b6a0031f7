"""Device-detected faults, forced from the host on the tiny model (every
kernel checks its page and slot indices, so nothing is read or written out of
bounds): a sequence whose block runs past its page table gets
UNO_DEV_CAPACITY, one whose table holds a page id outside the pool gets
UNO_DEV_BAD_PAGE; the other sequence of the batch is untouched (its logits
equal those of a batch that holds it alone) and its status stays clear."""
import numpy as np
import pytest
import torch

import synth

from gpu_util import gpu_or_fail, progress

pytestmark = pytest.mark.gpu

K = 4


def _setup(U, B, cap, n_extra=0):
    cfg = synth.TINY
    model = U.Model(cfg, synth.make_weights(cfg, 0))
    kv = U.PagedKV(cfg, B, cap, extra_pages=n_extra)
    synth.fill_kv_device(kv.k_pages, kv.v_pages, seed=5)
    ws = U.alloc_workspace(U.workspace_bytes(model, B, K, cap))
    return cfg, model, kv, ws


def _draft_verify(U, model, kv, cap, ws, anchors):
    B = len(anchors)
    V = model.cfg["vocab"]
    zq = torch.empty((B, K, V), dtype=torch.float32, device="cuda")
    zp = torch.empty((B, K, V), dtype=torch.float32, device="cuda")
    d = torch.empty((B, K), dtype=torch.int32, device="cuda")
    status = torch.zeros(B, dtype=torch.int32, device="cuda")
    step = torch.zeros(B, dtype=torch.uint64).cuda()
    anchor = torch.tensor(anchors, dtype=torch.int32, device="cuda")
    U.draft_block(model, kv, anchor, K, cap, 1.0, 0, step, zq, d, ws, status)
    U.verify_block(model, kv, d, cap, 1, zp, ws, status)
    torch.cuda.synchronize()
    return zq.cpu().numpy(), zp.cpu().numpy(), d.cpu().numpy(), status.cpu().numpy()


def _alone(U, cfg, model, kv2, cap, ws, kv_len0, anchor):
    """Sequence 0 of kv2 run in a batch of one (same pages, same content)."""
    kv1 = U.PagedKV(cfg, 1, cap)                  # pages 0.. of seq 0 (identity order)
    n = kv1.n_pages
    assert int(kv2.page_table[0].max()) < n
    kv1.k_pages.copy_(kv2.k_pages[:, :n])
    kv1.v_pages.copy_(kv2.v_pages[:, :n])
    kv1.page_table.copy_(kv2.page_table[:1])
    kv1.kv_len.fill_(kv_len0)
    return _draft_verify(U, model, kv1, cap, ws, [anchor])


def test_block_past_the_page_table_sets_capacity_flag():
    U = gpu_or_fail()
    cap = 64
    cfg, model, kv, ws = _setup(U, 2, cap)
    kv.kv_len.copy_(torch.tensor([20, cap - 2], dtype=torch.int32))   # seq 1: slots past 64
    zq, zp, d, st = _draft_verify(U, model, kv, cap, ws, [7, 9])
    assert st[0] == 0
    assert st[1] & U.DEV_CAPACITY
    zq1, zp1, d1, st1 = _alone(U, cfg, model, kv, cap, ws, 20, 7)
    assert st1[0] == 0
    np.testing.assert_allclose(zq[0], zq1[0], rtol=0, atol=1e-5)
    np.testing.assert_allclose(zp[0], zp1[0], rtol=0, atol=1e-5)
    progress("capacity flag: status %s" % st.tolist())


def test_page_outside_the_pool_sets_bad_page_flag():
    U = gpu_or_fail()
    cap = 64
    cfg, model, kv, ws = _setup(U, 2, cap)
    kv.kv_len.copy_(torch.tensor([20, 30], dtype=torch.int32))
    kv.page_table[1, 0] = kv.n_pages + 5          # a context page of seq 1 outside the pool
    zq, zp, d, st = _draft_verify(U, model, kv, cap, ws, [7, 9])
    assert st[0] == 0
    assert st[1] & U.DEV_BAD_PAGE
    assert np.all(np.isfinite(zq[1])) and np.all(np.isfinite(zp[1]))
    zq1, zp1, d1, st1 = _alone(U, cfg, model, kv, cap, ws, 20, 7)
    np.testing.assert_allclose(zq[0], zq1[0], rtol=0, atol=1e-5)
    np.testing.assert_allclose(zp[0], zp1[0], rtol=0, atol=1e-5)
    progress("bad-page flag: status %s" % st.tolist())
