"""GPU parity of the draft and verify passes where the attention takes its
two-stage form (two LDS stages, two workgroups per CU): 8 kv heads of
head_dim 128 and 4 sequences make 32 (sequence, kv head) groups, and a cache
capacity above 4096 lets each split into 16 key ranges, so the grid reaches
512 workgroups.  Every query-row layout of the kernel is taken: one, two and
four 16-row groups with two waves per group (G*K = 16, 32, 64 rows per kv
head), and eight row groups with one wave each (G = 4, K = 32).  Contexts are
ragged (one sequence is so short that most of its key ranges are empty, which
the merge of the ranges must absorb) and the pages are shuffled.  Logits
against the oracle."""
import pytest
import torch

import synth
from oracle import spec as ospec

from gpu_util import assert_logits_close, gpu_or_fail, load_kv_logical, progress

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("G,K,ps", [(1, 16, 16), (2, 16, 16), (4, 16, 16), (4, 32, 16), (4, 16, 64)])
def test_two_stage_attention(G, K, ps):
    U = gpu_or_fail()
    cfg = dict(synth.SMALL_GQA, n_q_heads=8 * G, n_kv_heads=8, head_dim=128)
    wts = synth.make_weights(cfg, 51)
    w64 = synth.to_f64(wts)
    model = U.Model(cfg, wts, page_size=ps)
    ctxs = [4500, 1000, 3001, 77]
    B = len(ctxs)
    cap = max(ctxs) + 2 * K + 8
    n_pages = B * ((cap + ps - 1) // ps)
    kv = U.PagedKV(cfg, B, cap, page_size=ps, page_order=torch.randperm(
        n_pages, generator=torch.Generator().manual_seed(G * 100 + K)))
    seqs = []
    for b, n in enumerate(ctxs):
        k, v = synth.kv_values(cfg, n, seed=37, seq=b)
        load_kv_logical(kv, b, k, v)
        toks = synth.random_tokens(n + 1, cfg["vocab"], 700 + b, (n + 1,))
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
    rows = synth.random_tokens(K, V, 66, (B, K))
    U.verify_block(model, kv, torch.from_numpy(rows).to(dev), cap, 1, zp, ws, status)
    torch.cuda.synchronize()
    assert (status.cpu().numpy() == 0).all()
    zq_c, zp_c = zq.cpu().numpy(), zp.cpu().numpy()
    worst = 0.0
    for b, s in enumerate(seqs):
        worst = max(worst, assert_logits_close(zq_c[b], ospec.draft_logits(cfg, w64, s, K),
                                               "G %d K %d draft %d" % (G, K, b)))
        worst = max(worst, assert_logits_close(zp_c[b], ospec.verify_logits(cfg, w64, s, list(rows[b])),
                                               "G %d K %d verify %d" % (G, K, b)))
    progress("two-stage attention, G %d, K %d, page %d: worst logit error %.2e" % (G, K, ps, worst))
