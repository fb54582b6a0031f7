"""GPU parity of the draft and verify passes across pass sizes that take
different GEMM plans: 48 rows (skinny kernel), 80 and 128 (one row of 128x128
tiles split along K), 160 and 528 (tiled configurations chosen by the cost
model, split tiles mixed with whole ones; 528 leaves a partial last row tile).
Small model with the 8B shape's head layout, K = 16, ragged contexts, shuffled
pages; every sequence's logits against the oracle."""
import pytest
import torch

import synth
from oracle import spec as ospec

from gpu_util import assert_logits_close, gpu_or_fail, load_kv_logical, progress

pytestmark = pytest.mark.gpu

K = 16


@pytest.mark.parametrize("B", [3, 5, 8, 10, 33])
def test_pass_sizes(B):
    U = gpu_or_fail()
    cfg = synth.SMALL_GQA
    wts = synth.make_weights(cfg, 41)
    w64 = synth.to_f64(wts)
    model = U.Model(cfg, wts)
    ctxs = [20 + (53 * b) % 300 for b in range(B)]
    cap = max(ctxs) + 2 * K + 8
    n_pages = B * ((cap + 15) // 16)
    kv = U.PagedKV(cfg, B, cap, page_order=torch.randperm(
        n_pages, generator=torch.Generator().manual_seed(B)))
    seqs = []
    for b, n in enumerate(ctxs):
        k, v = synth.kv_values(cfg, n, seed=29, seq=b)
        load_kv_logical(kv, b, k, v)
        toks = synth.random_tokens(n + 1, cfg["vocab"], 600 + b, (n + 1,))
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
    anchor = torch.tensor([s.tokens[-1] for s in seqs], dtype=torch.int32, device=dev)
    U.draft_block(model, kv, anchor, K, cap, 1.0, 0, torch.zeros(B, dtype=torch.uint64).to(dev),
                  zq, d, ws, status)
    rows = synth.random_tokens(K, V, 99, (B, K))
    U.verify_block(model, kv, torch.from_numpy(rows).to(dev), cap, 1, zp, ws, status)
    torch.cuda.synchronize()
    assert (status.cpu().numpy() == 0).all()
    zq_c, zp_c = zq.cpu().numpy(), zp.cpu().numpy()
    worst = 0.0
    for b, s in enumerate(seqs):
        worst = max(worst, assert_logits_close(zq_c[b], ospec.draft_logits(cfg, w64, s, K),
                                               "%d rows draft %d" % (B * K, b)))
        worst = max(worst, assert_logits_close(zp_c[b], ospec.verify_logits(cfg, w64, s, list(rows[b])),
                                               "%d rows verify %d" % (B * K, b)))
    progress("%d rows: worst logit error %.2e" % (B * K, worst))
