"""GPU parity of the draft and verify passes with the 8B shape's head layout
(head_dim 128, 4 q heads per kv head) on a small model: batches with ragged
contexts, K = 16 (64 query rows per kv head) and K = 32 (128), several key
ranges per row (merge path) and one (direct path), shuffled pages."""
import numpy as np
import pytest
import torch

import synth
from oracle import spec as ospec

from gpu_util import assert_logits_close, gpu_or_fail, load_kv_logical

pytestmark = pytest.mark.gpu


def _sub_kv(U, kv, b):
    sub = U.PagedKV.__new__(U.PagedKV)
    sub.__dict__.update(kv.__dict__)
    sub.page_table = kv.page_table[b:b + 1].contiguous()
    sub.kv_len = kv.kv_len[b:b + 1]
    sub.struct = U.UnoKV(kv.k_pages.data_ptr(), kv.v_pages.data_ptr(), kv.n_pages,
                         sub.page_table.data_ptr(), kv.max_pages, sub.kv_len.data_ptr())
    return sub


@pytest.mark.parametrize("B,K,ctxs", [(5, 16, [300, 511, 700, 64, 1025]),
                                      (3, 32, [129, 400, 900]),
                                      (1, 16, [2500])])
def test_gqa_draft_verify_synthetic_cache(B, K, ctxs):
    U = gpu_or_fail()
    cfg = synth.SMALL_GQA
    wts = synth.make_weights(cfg, 3)
    w64 = synth.to_f64(wts)
    model = U.Model(cfg, wts)
    cap = max(ctxs) + 2 * K + 8
    n_pages = B * ((cap + 15) // 16)
    kv = U.PagedKV(cfg, B, cap, page_order=torch.randperm(
        n_pages, generator=torch.Generator().manual_seed(K + B)))
    seqs = []
    for b, n in enumerate(ctxs):
        k, v = synth.kv_values(cfg, n, seed=11, seq=b)
        load_kv_logical(kv, b, k, v)
        toks = synth.random_tokens(n + 1, cfg["vocab"], 200 + b, (n + 1,))
        s = ospec.Sequence(cfg, toks, capacity=cap)
        for li in range(cfg["n_layers"]):
            s.cache.k[li][:n] = k[li].double().numpy()
            s.cache.v[li][:n] = v[li].double().numpy()
        s.kv_len = n
        seqs.append(s)
    kv.kv_len.copy_(torch.tensor(ctxs, dtype=torch.int32))
    ws = U.alloc_workspace(U.workspace_bytes(model, B, K, cap))
    anchor = torch.tensor([s.tokens[-1] for s in seqs], dtype=torch.int32, device="cuda")
    V = cfg["vocab"]
    zq = torch.empty((B, K, V), dtype=torch.float32, device="cuda")
    d = torch.empty((B, K), dtype=torch.int32, device="cuda")
    status = torch.zeros(B, dtype=torch.int32, device="cuda")
    U.draft_block(model, kv, anchor, K, cap, 1.0, 0, torch.zeros(B, dtype=torch.uint64).cuda(),
                  zq, d, ws, status)
    rows = synth.random_tokens(K, V, 66, (B, K))
    zp = torch.empty((B, K, V), dtype=torch.float32, device="cuda")
    U.verify_block(model, kv, torch.from_numpy(rows).cuda(), cap, 1, zp, ws, status)
    torch.cuda.synchronize()
    assert (status.cpu().numpy() == 0).all()
    zq_c, zp_c = zq.cpu().numpy(), zp.cpu().numpy()
    for b, s in enumerate(seqs):
        assert_logits_close(zq_c[b], ospec.draft_logits(cfg, w64, s, K), "draft seq %d" % b)
        assert_logits_close(zp_c[b], ospec.verify_logits(cfg, w64, s, list(rows[b])),
                            "verify seq %d" % b)


def test_gqa_prefill_chunk_then_step():
    """A 700-token prompt chunk (causal, 2800 query rows per kv head) through
    the verify pass, then one draft pass, against the oracle."""
    U = gpu_or_fail()
    cfg = synth.SMALL_GQA
    wts = synth.make_weights(cfg, 4)
    w64 = synth.to_f64(wts)
    model = U.Model(cfg, wts)
    prompt = synth.random_tokens(701, cfg["vocab"], 9, (701,))
    cap = 800
    kv = U.PagedKV(cfg, 1, cap)
    ws = U.alloc_workspace(U.workspace_bytes(model, 1, 700, cap))
    rows = torch.from_numpy(prompt[:-1].astype(np.int32)).reshape(1, -1).cuda()
    zpre = torch.empty((1, 700, cfg["vocab"]), dtype=torch.float32, device="cuda")
    U.verify_block(model, kv, rows, cap, 0, zpre, ws)
    U.kv_commit(kv, torch.tensor([699], dtype=torch.int32, device="cuda"), 700)
    s = ospec.Sequence(cfg, prompt, capacity=cap)
    n = len(prompt) - 1
    pos = np.arange(n)
    from oracle.model import forward
    ref = forward(cfg, w64, s.cache, prompt[:-1], pos, np.zeros(n), pos)
    s.kv_len = n
    got = zpre.cpu().numpy()[0]
    assert_logits_close(got[::37], ref[::37], "prefill logits (every 37th row)")
    K = 16
    zq = torch.empty((1, K, cfg["vocab"]), dtype=torch.float32, device="cuda")
    d = torch.empty((1, K), dtype=torch.int32, device="cuda")
    U.draft_block(model, kv, torch.tensor([int(prompt[-1])], dtype=torch.int32, device="cuda"),
                  K, cap, 1.0, 0, torch.zeros(1, dtype=torch.uint64).cuda(), zq, d, ws)
    assert_logits_close(zq.cpu().numpy()[0], ospec.draft_logits(cfg, w64, s, K), "draft")
