"""GPU parity of the draft and verify passes, then commit and a second draft
pass, for every KV page size the library takes from 32 to 256 tokens (the
other GPU tests use 16): with the 8B shape's head layout on a small model,
ragged contexts that end inside a page, shuffled pages, K = 16 and K = 32.
A page size of 64 or more holds a whole 64-key chunk of the attention kernel
in one page; 32 splits a chunk over two."""
import numpy as np
import pytest
import torch

import synth
from oracle import spec as ospec

from gpu_util import assert_logits_close, gpu_or_fail, kv_to_logical, load_kv_logical, progress

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("ps,K,ctxs", [(32, 16, [300, 97, 1025]),
                                       (64, 16, [65, 640, 1000]),
                                       (128, 32, [129, 383]),
                                       (256, 16, [700, 31, 257])])
def test_page_size_draft_verify_commit(ps, K, ctxs):
    U = gpu_or_fail()
    cfg = synth.SMALL_GQA
    wts = synth.make_weights(cfg, 5)
    w64 = synth.to_f64(wts)
    model = U.Model(cfg, wts, page_size=ps)
    B = len(ctxs)
    cap = max(ctxs) + 3 * K + 8
    n_pages = B * ((cap + ps - 1) // ps)
    kv = U.PagedKV(cfg, B, cap, page_size=ps, page_order=torch.randperm(
        n_pages, generator=torch.Generator().manual_seed(ps + K)))
    seqs = []
    for b, n in enumerate(ctxs):
        k, v = synth.kv_values(cfg, n, seed=13, seq=b)
        load_kv_logical(kv, b, k, v)
        toks = synth.random_tokens(n + 1, cfg["vocab"], 300 + b, (n + 1,))
        s = ospec.Sequence(cfg, toks, capacity=cap)
        for li in range(cfg["n_layers"]):
            s.cache.k[li][:n] = k[li].double().numpy()
            s.cache.v[li][:n] = v[li].double().numpy()
        s.kv_len = n
        seqs.append(s)
    kv.kv_len.copy_(torch.tensor(ctxs, dtype=torch.int32))
    ws = U.alloc_workspace(U.workspace_bytes(model, B, K, cap))
    V = cfg["vocab"]
    dev = "cuda"
    zq = torch.empty((B, K, V), dtype=torch.float32, device=dev)
    zp = torch.empty((B, K, V), dtype=torch.float32, device=dev)
    d = torch.empty((B, K), dtype=torch.int32, device=dev)
    status = torch.zeros(B, dtype=torch.int32, device=dev)
    steps = torch.zeros(B, dtype=torch.uint64).to(dev)
    anchor = torch.tensor([s.tokens[-1] for s in seqs], dtype=torch.int32, device=dev)
    U.draft_block(model, kv, anchor, K, cap, 1.0, 0, steps, zq, d, ws, status)
    rows = synth.random_tokens(K, V, 77, (B, K))
    U.verify_block(model, kv, torch.from_numpy(rows).to(dev), cap, 1, zp, ws, status)
    torch.cuda.synchronize()
    assert (status.cpu().numpy() == 0).all()
    zq_c, zp_c = zq.cpu().numpy(), zp.cpu().numpy()
    for b, s in enumerate(seqs):
        assert_logits_close(zq_c[b], ospec.draft_logits(cfg, w64, s, K), "ps %d draft %d" % (ps, b))
        assert_logits_close(zp_c[b], ospec.verify_logits(cfg, w64, s, list(rows[b])),
                            "ps %d verify %d" % (ps, b))

    # commit a ragged number of the verify rows (the anchor's and the kept rows'
    # K/V stay where the passes wrote them), then draft again from the new length
    acc = [K // 2, K, 0, 3][:B]
    U.kv_commit(kv, torch.tensor(acc, dtype=torch.int32, device=dev), K, steps)
    torch.cuda.synchronize()
    got_len = kv.kv_len.cpu().numpy()
    for b, s in enumerate(seqs):
        n0 = s.kv_len
        toks = [s.tokens[-1]] + [int(t) for t in rows[b][:acc[b]]]
        ospec.commit(s, acc[b], toks[1:] + [int(synth.random_tokens(1, V, 90 + b, (1,))[0])])
        assert s.kv_len == n0 + 1 + acc[b] == got_len[b]
        # the cached K/V of the new context equal the oracle's (bf16-rounded)
        for li in range(cfg["n_layers"]):
            kg, vg = kv_to_logical(kv, li, b, s.kv_len)
            assert_logits_close(kg, s.cache.k[li][: s.kv_len], "ps %d K layer %d seq %d" % (ps, li, b))
            assert_logits_close(vg, s.cache.v[li][: s.kv_len], "ps %d V layer %d seq %d" % (ps, li, b))
    anchor = torch.tensor([s.tokens[-1] for s in seqs], dtype=torch.int32, device=dev)
    U.draft_block(model, kv, anchor, K, cap, 1.0, 0, steps, zq, d, ws, status)
    torch.cuda.synchronize()
    assert (status.cpu().numpy() == 0).all()
    zq_c = zq.cpu().numpy()
    for b, s in enumerate(seqs):
        assert_logits_close(zq_c[b], ospec.draft_logits(cfg, w64, s, K),
                            "ps %d second draft %d" % (ps, b))
    progress("page size %d, K %d, contexts %s: draft, verify, commit, draft ok" % (ps, K, ctxs))
