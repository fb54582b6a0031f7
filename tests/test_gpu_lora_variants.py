"""GPU parity of the LoRA path beyond the ranks and projection sets the model
tests use (16, 64, 128 on every projection): ranks 32, 48 (not a whole number
of the tiled kernel's 32-wide K slices, so passes of more than 64 rows take the
skinny kernel) and 256 (the largest the library takes), and LoRA on a subset of
the projections (q|k|v, o with down, gate|up), at 32 rows (skinny kernel; the
LoRA A partials are summed by the projection) and 96 rows (tiled kernel).
Draft logits, with the 8B shape's head layout on a small model, against the
oracle holding LoRA factors for the same projections only."""
import pytest
import torch

import synth
from oracle import spec as ospec

from gpu_util import assert_logits_close, gpu_or_fail, load_kv_logical, progress

pytestmark = pytest.mark.gpu

K = 16
ALL = ("q", "k", "v", "o", "gate", "up", "down")
BITS = {p: 1 << i for i, p in enumerate(ALL)}


@pytest.mark.parametrize("rank,projs", [(32, ALL), (48, ALL), (256, ALL),
                                        (64, ("q", "k", "v")), (64, ("o", "down")),
                                        (64, ("gate", "up"))])
@pytest.mark.parametrize("B", [2, 6])
def test_lora_rank_and_projection_set(rank, projs, B):
    U = gpu_or_fail()
    cfg = dict(synth.SMALL_GQA, lora_rank=rank, lora_alpha=2.0 * rank)
    wts = synth.make_weights(cfg, 21)
    w64 = synth.to_f64(wts)
    for lw in w64["layers"]:
        lw["lora_a"] = {p: t for p, t in lw["lora_a"].items() if p in projs}
        lw["lora_b"] = {p: t for p, t in lw["lora_b"].items() if p in projs}
    mask = sum(BITS[p] for p in projs)
    model = U.Model(cfg, wts, lora=True if mask == 0x7F else mask)
    ctxs = [37 + 61 * b for b in range(B)]
    cap = max(ctxs) + 2 * K + 8
    n_pages = B * ((cap + 15) // 16)
    kv = U.PagedKV(cfg, B, cap, page_order=torch.randperm(
        n_pages, generator=torch.Generator().manual_seed(rank + B)))
    seqs = []
    for b, n in enumerate(ctxs):
        k, v = synth.kv_values(cfg, n, seed=17, seq=b)
        load_kv_logical(kv, b, k, v)
        toks = synth.random_tokens(n + 1, cfg["vocab"], 400 + b, (n + 1,))
        s = ospec.Sequence(cfg, toks, capacity=cap)
        for li in range(cfg["n_layers"]):
            s.cache.k[li][:n] = k[li].double().numpy()
            s.cache.v[li][:n] = v[li].double().numpy()
        s.kv_len = n
        seqs.append(s)
    kv.kv_len.copy_(torch.tensor(ctxs, dtype=torch.int32))
    ws = U.alloc_workspace(U.workspace_bytes(model, B, K, cap))
    V = cfg["vocab"]
    zq = torch.empty((B, K, V), dtype=torch.float32, device="cuda")
    d = torch.empty((B, K), dtype=torch.int32, device="cuda")
    status = torch.zeros(B, dtype=torch.int32, device="cuda")
    anchor = torch.tensor([s.tokens[-1] for s in seqs], dtype=torch.int32, device="cuda")
    U.draft_block(model, kv, anchor, K, cap, 1.0, 0, torch.zeros(B, dtype=torch.uint64).cuda(),
                  zq, d, ws, status)
    torch.cuda.synchronize()
    assert (status.cpu().numpy() == 0).all()
    zq_c = zq.cpu().numpy()
    worst = 0.0
    for b, s in enumerate(seqs):
        worst = max(worst, assert_logits_close(zq_c[b], ospec.draft_logits(cfg, w64, s, K),
                                               "rank %d %s draft %d" % (rank, "+".join(projs), b)))
    progress("LoRA rank %d on %s, %d rows: worst draft logit error %.2e"
             % (rank, "+".join(projs), B * K, worst))
