"""End-to-end generation with natural acceptance (chunked prefill, continuous
steps, KV pages handed out on demand) on the tiny model.

At every step the oracle replays the step on the same committed state: the
GPU's draft and verify logits must lie within the logit tolerance of the
oracle's, and the oracle sampler fed the GPU's own fp32 logits and the same
Philox counters must take exactly the GPU's decisions (draft tokens, accept
length, committed tokens)."""
import numpy as np
import pytest
import torch

import synth
from oracle import spec as ospec

from gpu_util import assert_logits_close, gpu_or_fail, progress

pytestmark = pytest.mark.gpu

SEED = 11


@pytest.mark.parametrize("prior", [0, 1])
def test_natural_generation_matches_oracle_step_by_step(prior):
    U = gpu_or_fail()
    from lossless_decoding_uno_amd.generate import Generator
    cfg = dict(synth.TINY, noise_prior=prior)
    wts = synth.make_weights(cfg, 0)
    w64 = synth.to_f64(wts)
    model = U.Model(cfg, wts)
    B, K, P, n_new = 2, 4, 32, 40
    prompts = np.stack([synth.prompt_ids(cfg, P, 5 + b) for b in range(B)])
    max_ctx = P + n_new + 3 * K + 8
    # a pool smaller than B full-length tables: pages come on demand
    g = Generator(model, B, K, max_ctx, n_pages=(max_ctx // 16 + 2) * B - 1, seed=SEED,
                  prefill_chunk=7)
    g.prefill(prompts)
    seqs = []
    for b in range(B):
        s = ospec.Sequence(cfg, list(prompts[b]), capacity=max_ctx)
        ospec.prefill(cfg, w64, s)
        assert s.kv_len == int(g.kv_len[b]) == P - 1
        seqs.append(s)
    worst = 0.0
    while min(len(o) for o in g.out) < n_new:
        a_g = g.step()
        zq, zp = g.zq.cpu().numpy(), g.zp.cpu().numpy()
        d, c = g.d.cpu().numpy(), g.c.cpu().numpy()
        for b in range(B):
            s = seqs[b]
            draws = ospec.PhiloxDraws(SEED, b, s.step)
            zq_o = ospec.draft_logits(cfg, w64, s, K, draws=draws)
            worst = max(worst, assert_logits_close(zq[b], zq_o, "draft b%d step %d" % (b, s.step)))
            drafts = ospec.draft_sample(zq[b], 1.0, draws)
            np.testing.assert_array_equal(d[b], drafts)
            zp_o = ospec.verify_logits(cfg, w64, s, drafts)
            worst = max(worst, assert_logits_close(zp[b], zp_o, "verify b%d step %d" % (b, s.step)))
            a, committed, extra = ospec.spec_accept(zq[b], zp[b], drafts, 1.0, draws)
            assert a == a_g[b] and a >= 1
            np.testing.assert_array_equal(c[b, : a + 1], committed)
            ospec.commit(s, a, committed)
            assert s.kv_len == int(g.kv_len[b])
    st = g.stats()
    assert 1.0 <= st["TPF"] <= (K + 1) / 2.0
    assert g.pool.pages_in_use() <= g.kv.n_pages
    assert int(g.status.abs().sum().item()) == 0
    for b in range(B):
        assert g.out[b] == seqs[b].tokens[P:]
    progress("natural generation (prior %d): %d steps, TPF %.2f, AL %.2f, worst logit err %.2e"
             % (prior, st["steps"], st["TPF"], st["AL"], worst))


def test_tree_generation_matches_oracle_step_by_step():
    """The generator with the tree sampler (top-4 per drafted position, 6
    kept candidates, K = 5) on a vocab-32 tiny model whose LM head is scaled
    by 4 (sharper laws, so walks go deep): chunked prefill, pages on demand;
    every step starts the oracle from the library's committed bf16 K/V;
    every step's tree equals the oracle's tree on the GPU's draft logits,
    every node's verify logits meet the bf16 yardstick against the exact
    oracle's forward (the head's scale makes the logits, and the rounding of
    any bf16 implementation, four times larger), and the walk (accept length,
    committed tokens, path) equals the oracle's on the GPU's logits.
    The outputs equal the oracle's committed tokens."""
    U = gpu_or_fail()
    from lossless_decoding_uno_amd.generate import Generator
    from oracle import canonical as cn
    from oracle import model as om
    from oracle import tree as ot
    from gpu_util import YardstickTally, teacher_force_cache, u24
    cfg = dict(synth.TINY, vocab=32, mask_id=31)
    wts = synth.make_weights(cfg, 2)
    hs = 4.0
    wts["lm_head"] = (wts["lm_head"].float() * hs).to(torch.bfloat16)
    w64 = synth.to_f64(wts)
    model = U.Model(cfg, wts)
    B, K, P, n_new, topk, n_keep = 2, 5, 24, 40, 4, 6
    N = U.tree_rows(K, topk, n_keep)
    prompts = np.stack([synth.prompt_ids(cfg, P, 40 + b) for b in range(B)])
    max_ctx = P + n_new + 2 * K + N + 8
    g = Generator(model, B, K, max_ctx, n_pages=(max_ctx // 16 + 2) * B - 1, seed=SEED,
                  prefill_chunk=9, tree=(topk, n_keep))
    g.prefill(prompts)
    seqs = []
    for b in range(B):
        s = ospec.Sequence(cfg, list(prompts[b]), capacity=max_ctx)
        ospec.prefill(cfg, w64, s)
        seqs.append(s)
    moves = 0
    tally = YardstickTally("tree generation logits")
    while min(len(o) for o in g.out) < n_new:
        a_g = g.step()
        zq, zp = g.zq.cpu().numpy(), g.zp.cpu().numpy()
        c, path_g = g.c.cpu().numpy(), g.tb.path.cpu().numpy()
        for b in range(B):
            s = seqs[b]
            # the step starts from the library's committed bf16 K/V
            teacher_force_cache(s, g.kv, b)
            s_bf = s.copy()
            zq_o = ospec.draft_logits(cfg, w64, s, K)
            tally.add(zq[b], zq_o, ospec.draft_logits(cfg, w64, s_bf, K, act_round=om.bf16_round),
                      "draft b%d step %d" % (b, s.step))
            d1 = cn.categorical(cn.row_weights(zq[b, 0], 1.0)[0], u24(SEED, 0, 0, b, s.step))
            tree = ot.build_tree(zq[b], d1, topk, n_keep)
            np.testing.assert_array_equal(g.tb.tokens[b].cpu().numpy(), tree.tokens)
            np.testing.assert_array_equal(g.tb.parent[b].cpu().numpy(), tree.parent)
            zp_o = ot.tree_verify_logits(cfg, w64, s, tree)
            tally.add(zp[b, : tree.n_nodes], zp_o,
                      ot.tree_verify_logits(cfg, w64, s_bf, tree, act_round=om.bf16_round),
                      "tree verify b%d step %d" % (b, s.step))
            a, committed, extra, path = ot.tree_accept(tree, zp[b], 1.0,
                                                       ospec.PhiloxDraws(SEED, b, s.step))
            assert a == a_g[b] and a >= 1
            np.testing.assert_array_equal(c[b, : a + 1], committed)
            np.testing.assert_array_equal(path_g[b, :a], path)
            moves += sum(1 for dd in range(1, a) if path[dd] != dd)
            ot.tree_commit(s, path, a, committed)
            assert s.kv_len == int(g.kv_len[b])
    st = g.stats()
    assert int(g.status.abs().sum().item()) == 0
    for b in range(B):
        assert g.out[b] == seqs[b].tokens[P:]
    progress("tree generation: %d steps, TPF %.2f, AL %.2f, %d K/V moves, logits: %s"
             % (st["steps"], st["TPF"], st["AL"], moves, tally.finish()))
    assert 2.0 <= st["AL"] <= K + 1


def test_generate_holds_finished_sequences():
    """Batched generation to a fixed length with a page table sized for
    prompt + n_new + two blocks: sequences that are done hold their cache
    length while the rest finish (no sequence outgrows its table), every
    sequence returns exactly n_new tokens, and the statistics count only the
    steps of unfinished sequences."""
    U = gpu_or_fail()
    from lossless_decoding_uno_amd.generate import Generator
    cfg = synth.TINY
    model = U.Model(cfg, synth.make_weights(cfg, 0))
    B, K, P, n_new = 6, 4, 20, 60
    prompts = np.stack([synth.prompt_ids(cfg, P, 70 + b) for b in range(B)])
    max_ctx = P + n_new + 2 * K + 1
    g = Generator(model, B, K, max_ctx, seed=SEED, prefill_chunk=16)
    g.prefill(prompts)
    outs = g.generate(n_new)
    assert [len(o) for o in outs] == [n_new] * B
    assert (g.kv_len <= P - 1 + n_new + K).all()
    assert np.array_equal(g.kv.kv_len.cpu().numpy(), g.kv_len.astype(np.int32))
    per = np.array(g.committed_per_step)
    assert (per >= 0).all() and (per <= K + 1).all()
    assert int(g.status.abs().sum().item()) == 0
    st = g.stats()
    assert 1.0 <= st["AL"] <= K + 1
    progress("generation held: %d steps, AL %.2f, kv_len %s" % (st["steps"], st["AL"],
                                                                 g.kv_len.tolist()))
