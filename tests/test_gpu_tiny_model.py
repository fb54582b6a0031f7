"""GPU parity of the full decode step on the tiny model (2 layers, d_model 256,
4 heads x 64, SwiGLU 1024, vocab 512, LoRA r16 alpha 32, K = 4, T = 1, 64 new
tokens after a 32-token prompt, Philox seed 0), teacher-forced by the oracle.

Every step both sides start from the same committed state.  Draft and verify
logits must agree with the exact oracle's within 2e-2 abs + 1e-2 rel.  The
oracle's sampler is then fed the GPU's own fp32 logits and the same Philox
counters: the GPU's draft tokens, accept length, committed tokens and extra
token must equal its decisions bit for bit, with no allowance.  Both sides
verify the same drafted rows and commit the same decisions, so their caches
hold the same tokens at every step."""
import numpy as np
import pytest
import torch

import synth
from oracle import spec as ospec

from gpu_util import assert_logits_close, gpu_or_fail, kv_to_logical, progress

pytestmark = pytest.mark.gpu

SEED = 0
K = 4
N_NEW = 64


@pytest.fixture(scope="module")
def setup():
    U = gpu_or_fail()
    cfg = synth.TINY
    wts = synth.make_weights(cfg, 0)
    model = U.Model(cfg, wts)
    return U, cfg, wts, synth.to_f64(wts), model


def _prefill_gpu(U, model, kv, prompt, ws, max_ctx):
    rows = torch.from_numpy(np.asarray(prompt[:-1], dtype=np.int32)).reshape(1, -1).cuda()
    U.verify_block(model, kv, rows, max_ctx, 0, None, ws)
    acc = torch.tensor([rows.shape[1] - 1], dtype=torch.int32, device="cuda")
    U.kv_commit(kv, acc, rows.shape[1])


def test_tiny_model_teacher_forced_generation(setup):
    U, cfg, wts, w64, model = setup
    _teacher_forced(U, cfg, w64, model, N_NEW)


def test_tiny_model_uniform_prior_generation(setup):
    """Uniform-state prior: the draft block's noise tokens are uniform Philox
    draws (slot 3) on the GPU and in the oracle alike."""
    U, cfg, wts, w64, _ = setup
    cfg_u = dict(cfg, noise_prior=1)
    _teacher_forced(U, cfg_u, w64, U.Model(cfg_u, wts), 32)


def _teacher_forced(U, cfg, w64, model, n_new):
    prompt = synth.prompt_ids(cfg, 32, 1)
    cap = len(prompt) + n_new + 2 * K + 8
    max_ctx = cap
    kv = U.PagedKV(cfg, 1, cap, page_order=torch.randperm(
        (cap + 15) // 16 + 3, generator=torch.Generator().manual_seed(3)), extra_pages=3)
    ws = U.alloc_workspace(max(U.workspace_bytes(model, 1, K, max_ctx),
                               U.workspace_bytes(model, 1, len(prompt), max_ctx)))
    _prefill_gpu(U, model, kv, prompt, ws, max_ctx)
    seq = ospec.Sequence(cfg, prompt, capacity=cap)
    ospec.prefill(cfg, w64, seq)
    assert int(kv.kv_len.item()) == seq.kv_len == len(prompt) - 1

    # the prefilled cache holds the oracle's K/V (bf16-rounded)
    for li in range(cfg["n_layers"]):
        kg, vg = kv_to_logical(kv, li, 0, seq.kv_len)
        assert_logits_close(kg, seq.cache.k[li][: seq.kv_len], "prefill K layer %d" % li)
        assert_logits_close(vg, seq.cache.v[li][: seq.kv_len], "prefill V layer %d" % li)

    V = cfg["vocab"]
    dev = "cuda"
    zq_g = torch.empty((1, K, V), dtype=torch.float32, device=dev)
    zp_g = torch.empty((1, K, V), dtype=torch.float32, device=dev)
    d_g = torch.empty((1, K), dtype=torch.int32, device=dev)
    a_g = torch.empty(1, dtype=torch.int32, device=dev)
    c_g = torch.empty((1, K + 1), dtype=torch.int32, device=dev)
    e_g = torch.empty(1, dtype=torch.int32, device=dev)
    status = torch.zeros(1, dtype=torch.int32, device=dev)
    step_g = torch.zeros(1, dtype=torch.uint64).to(dev)
    aws = U.alloc_workspace(U.spec_accept_workspace_bytes(1, K))
    qmax = torch.empty((1, K), dtype=torch.float32, device=dev)
    pmax = torch.empty((1, K), dtype=torch.float32, device=dev)
    worst = 0.0
    n_steps_rejected = 0
    while len(seq.tokens) - len(prompt) < n_new:
        st = seq.step
        anchor = torch.tensor([seq.tokens[-1]], dtype=torch.int32, device=dev)
        U.draft_block(model, kv, anchor, K, max_ctx, 1.0, SEED, step_g, zq_g, d_g, ws, status,
                      row_max=qmax)
        draws = ospec.PhiloxDraws(SEED, 0, st)
        zq = ospec.draft_logits(cfg, w64, seq, K, draws=draws)
        zq_gpu = zq_g.cpu().numpy()[0]
        # the LM head's row maxima are the logits' exact maxima
        np.testing.assert_array_equal(qmax.cpu().numpy()[0], zq_gpu.max(axis=-1))
        worst = max(worst, assert_logits_close(zq_gpu, zq, "draft logits step %d" % st))
        # the oracle's sampler on the GPU's logits takes the GPU's draws
        drafts = ospec.draft_sample(zq_gpu, 1.0, draws)
        assert [int(x) for x in d_g.cpu().numpy()[0]] == drafts, st

        U.verify_block(model, kv, d_g, max_ctx, 1, zp_g, ws, status, row_max=pmax)
        zp = ospec.verify_logits(cfg, w64, seq, drafts)
        zp_gpu = zp_g.cpu().numpy()[0]
        worst = max(worst, assert_logits_close(zp_gpu, zp, "verify logits step %d" % st))
        np.testing.assert_array_equal(pmax.cpu().numpy()[0], zp_gpu.max(axis=-1))

        a, committed, extra = ospec.spec_accept(zq_gpu, zp_gpu, drafts, 1.0, draws)
        U.spec_accept(zq_g, zp_g, d_g, 1.0, SEED, step_g, a_g, c_g, e_g, aws, status=status,
                      draft_row_max=qmax, verify_row_max=pmax)
        assert (int(a_g.item()), int(e_g.item())) == (a, extra), st
        np.testing.assert_array_equal(c_g.cpu().numpy()[0],
                                      committed + [-1] * (K + 1 - len(committed)))
        n_steps_rejected += a < K

        U.kv_commit(kv, a_g, K, step_g, status)
        ospec.commit(seq, a, committed)
        assert int(kv.kv_len.item()) == seq.kv_len
        assert int(step_g.item()) == seq.step
    assert int(status.item()) == 0
    progress("tiny model: %d steps (%d with a rejection), worst logit error %.2e; every "
             "decision bit-exact" % (seq.step, n_steps_rejected, worst))


def test_zero_lora_b_reproduces_ar_weights(setup):
    """B = 0 makes the draft pass identical (bit for bit) to the same pass with
    the LoRA path switched off."""
    U, cfg, wts, _, model = setup
    m0 = U.Model(cfg, synth.zero_lora_b(wts))
    m_off = U.Model(cfg, wts, lora=False)
    prompt = synth.prompt_ids(cfg, 20, 4)
    outs = []
    for m in (m0, m_off):
        kv = U.PagedKV(cfg, 1, 64)
        ws = U.alloc_workspace(max(U.workspace_bytes(m, 1, 20, 64), U.workspace_bytes(m, 1, K, 64)))
        _prefill_gpu(U, m, kv, prompt, ws, 64)
        zq = torch.empty((1, K, cfg["vocab"]), dtype=torch.float32, device="cuda")
        d = torch.empty((1, K), dtype=torch.int32, device="cuda")
        U.draft_block(m, kv, torch.tensor([int(prompt[-1])], dtype=torch.int32, device="cuda"), K,
                      64, 1.0, 0, torch.zeros(1, dtype=torch.uint64).cuda(), zq, d, ws)
        torch.cuda.synchronize()
        outs.append(zq.cpu())
    assert torch.equal(outs[0], outs[1])


def test_batched_ragged_draft_verify_matches_oracle(setup):
    """Batch of 3 sequences with different committed lengths and shuffled pages:
    one draft + verify pass, logits of every row against the oracle."""
    U, cfg, wts, w64, model = setup
    lens = [7, 23, 40]
    prompts = [synth.random_tokens(n, cfg["vocab"], 10 + i, (n,)) for i, n in enumerate(lens)]
    cap = max(lens) + 2 * K + 8
    B = len(lens)
    n_pages = B * ((cap + 15) // 16)
    kv = U.PagedKV(cfg, B, cap, page_order=torch.randperm(
        n_pages, generator=torch.Generator().manual_seed(9)))
    ws = U.alloc_workspace(U.workspace_bytes(model, B, max(K, max(lens)), cap))
    seqs = []
    for b, p in enumerate(prompts):
        s = ospec.Sequence(cfg, p, capacity=cap)
        ospec.prefill(cfg, w64, s)
        seqs.append(s)
    # GPU prefill one sequence at a time through a batch-of-one view of the cache
    for b, p in enumerate(prompts):
        sub = U.PagedKV.__new__(U.PagedKV)
        sub.__dict__.update(kv.__dict__)
        sub.page_table = kv.page_table[b:b + 1].contiguous()
        sub.kv_len = kv.kv_len[b:b + 1]
        sub.struct = U.UnoKV(kv.k_pages.data_ptr(), kv.v_pages.data_ptr(), kv.n_pages,
                             sub.page_table.data_ptr(), kv.max_pages, sub.kv_len.data_ptr())
        _prefill_gpu(U, model, sub, p, ws, cap)
    torch.cuda.synchronize()
    assert kv.kv_len.cpu().tolist() == [n - 1 for n in lens]
    anchor = torch.tensor([int(p[-1]) for p in prompts], dtype=torch.int32, device="cuda")
    zq = torch.empty((B, K, cfg["vocab"]), dtype=torch.float32, device="cuda")
    d = torch.empty((B, K), dtype=torch.int32, device="cuda")
    U.draft_block(model, kv, anchor, K, cap, 1.0, 0, torch.zeros(B, dtype=torch.uint64).cuda(), zq, d, ws)
    rows = synth.random_tokens(K, cfg["vocab"], 77, (B, K))
    zp = torch.empty((B, K, cfg["vocab"]), dtype=torch.float32, device="cuda")
    U.verify_block(model, kv, torch.from_numpy(rows).cuda(), cap, 1, zp, ws)
    zq_c, zp_c = zq.cpu().numpy(), zp.cpu().numpy()
    for b, s in enumerate(seqs):
        assert_logits_close(zq_c[b], ospec.draft_logits(cfg, w64, s, K), "draft seq %d" % b)
        assert_logits_close(zp_c[b], ospec.verify_logits(cfg, w64, s, list(rows[b])),
                            "verify seq %d" % b)


def test_kv_commit_ragged_and_rollback(setup):
    U, cfg, _, _, _ = setup
    B = 6
    kv = U.PagedKV(cfg, B, 128)
    kv.kv_len.copy_(torch.tensor([0, 5, 17, 31, 64, 100], dtype=torch.int32))
    step = torch.tensor([0, 1, 2, 3, 4, 5], dtype=torch.uint64).cuda()
    acc = torch.tensor([0, 3, K, 1, -1, K + 1], dtype=torch.int32, device="cuda")
    status = torch.zeros(B, dtype=torch.int32, device="cuda")
    U.kv_commit(kv, acc, K, step, status)
    torch.cuda.synchronize()
    assert kv.kv_len.cpu().tolist() == [1, 9, 22, 33, 64, 100]
    assert step.cpu().tolist() == [1, 2, 3, 4, 4, 5]
    assert status.cpu().tolist() == [0, 0, 0, 0, U.DEV_BAD_ACCEPT, U.DEV_BAD_ACCEPT]


@pytest.mark.parametrize("B,K_blk,prompt_len", [(40, 4, 150), (9, 16, 300)])
def test_many_rows_tiled_gemm_matches_oracle(B, K_blk, prompt_len):
    """Passes of >= 128 rows (the tiled GEMM with fused LoRA, split-K on the
    residual projections, a ragged last row tile) and a long prompt chunk,
    against the oracle on a rank-64 variant of the tiny model."""
    U = gpu_or_fail()
    cfg = synth.TINY_R64
    wts = synth.make_weights(cfg, 2)
    w64 = synth.to_f64(wts)
    model = U.Model(cfg, wts)
    lens = [prompt_len - 3 * b for b in range(B)]
    cap = max(lens) + 2 * K_blk + 8
    n_pages = B * ((cap + 15) // 16)
    kv = U.PagedKV(cfg, B, cap, page_order=torch.randperm(
        n_pages, generator=torch.Generator().manual_seed(B)))
    ws = U.alloc_workspace(max(U.workspace_bytes(model, B, K_blk, cap),
                               U.workspace_bytes(model, 1, max(lens), cap)))
    prompts = [synth.random_tokens(n, cfg["vocab"], 100 + b, (n,)) for b, n in enumerate(lens)]
    for b, p in enumerate(prompts):   # prefill: one long chunk per sequence (>= 128 rows)
        sub = U.PagedKV.__new__(U.PagedKV)
        sub.__dict__.update(kv.__dict__)
        sub.page_table = kv.page_table[b:b + 1].contiguous()
        sub.kv_len = kv.kv_len[b:b + 1]
        sub.struct = U.UnoKV(kv.k_pages.data_ptr(), kv.v_pages.data_ptr(), kv.n_pages,
                             sub.page_table.data_ptr(), kv.max_pages, sub.kv_len.data_ptr())
        _prefill_gpu(U, model, sub, p, ws, cap)
    anchor = torch.tensor([int(p[-1]) for p in prompts], dtype=torch.int32, device="cuda")
    V = cfg["vocab"]
    zq = torch.empty((B, K_blk, V), dtype=torch.float32, device="cuda")
    d = torch.empty((B, K_blk), dtype=torch.int32, device="cuda")
    U.draft_block(model, kv, anchor, K_blk, cap, 1.0, 0, torch.zeros(B, dtype=torch.uint64).cuda(),
                  zq, d, ws)
    rows = synth.random_tokens(K_blk, V, 55, (B, K_blk))
    zp = torch.empty((B, K_blk, V), dtype=torch.float32, device="cuda")
    U.verify_block(model, kv, torch.from_numpy(rows).cuda(), cap, 1, zp, ws)
    zq_c, zp_c = zq.cpu().numpy(), zp.cpu().numpy()
    for b in range(0, B, max(1, B // 6)):
        s = ospec.Sequence(cfg, prompts[b], capacity=cap)
        ospec.prefill(cfg, w64, s)
        assert_logits_close(zq_c[b], ospec.draft_logits(cfg, w64, s, K_blk), "draft seq %d" % b)
        assert_logits_close(zp_c[b], ospec.verify_logits(cfg, w64, s, list(rows[b])),
                            "verify seq %d" % b)


@pytest.mark.parametrize("prior,kappa", [(0, 1.0), (0, 0.5), (1, 0.5), (0, 0.0)])
def test_multi_pass_draft_matches_oracle(setup, prior, kappa):
    """Multi-pass draft with the corrector, pass by pass: three passes, the
    first two sampling with Philox slots 4 and 5, the last with slot 0; between
    passes each drafted row keeps its sample with probability kappa and else
    returns to the prior (mask or a fresh uniform token).  Each pass's logits
    must match the oracle's on the block the oracle's corrector makes from the
    GPU's samples (a differing keep decision changes a row's token and its
    logits), and its tokens must be exactly the oracle sampler's on the GPU's
    own logits; then verification and the accept step as usual."""
    U, cfg, wts, w64, model = setup
    if prior:
        cfg = dict(cfg, noise_prior=1)
        model = U.Model(cfg, wts)
    prompt = synth.prompt_ids(cfg, 24, 9)
    cap = len(prompt) + 4 * (K + 1) + 8
    kv = U.PagedKV(cfg, 1, cap)
    ws = U.alloc_workspace(max(U.workspace_bytes(model, 1, K, cap),
                               U.workspace_bytes(model, 1, len(prompt), cap)))
    _prefill_gpu(U, model, kv, prompt, ws, cap)
    seq = ospec.Sequence(cfg, prompt, capacity=cap)
    ospec.prefill(cfg, w64, seq)
    dev = "cuda"
    V = cfg["vocab"]
    zq_g = torch.empty((1, K, V), dtype=torch.float32, device=dev)
    zp_g = torch.empty((1, K, V), dtype=torch.float32, device=dev)
    d_g = torch.empty((1, K), dtype=torch.int32, device=dev)
    a_g = torch.empty(1, dtype=torch.int32, device=dev)
    c_g = torch.empty((1, K + 1), dtype=torch.int32, device=dev)
    e_g = torch.empty(1, dtype=torch.int32, device=dev)
    status = torch.zeros(1, dtype=torch.int32, device=dev)
    step_g = torch.zeros(1, dtype=torch.uint64).to(dev)
    aws = U.alloc_workspace(U.spec_accept_workspace_bytes(1, K))
    kept = total = 0
    for _ in range(4):
        draws = ospec.PhiloxDraws(SEED, 0, seq.step)
        anchor = torch.tensor([seq.tokens[-1]], dtype=torch.int32, device=dev)
        block = None
        for p, slot in enumerate((4, 5, 0)):
            U.draft_block_from(model, kv, anchor, d_g if p else None, K, cap, 1.0, SEED, step_g,
                               slot, zq_g, d_g, ws, status, kappa=kappa, corr_pass=p - 1 if p else 0)
            zq = ospec.draft_logits(cfg, w64, seq, K, draws=draws, block=block)
            zq_gpu = zq_g.cpu().numpy()[0]
            assert_logits_close(zq_gpu, zq, "pass %d step %d" % (p, seq.step))
            toks = ospec.draft_sample(zq_gpu, 1.0, draws, slot)
            np.testing.assert_array_equal(d_g.cpu().numpy()[0], toks)
            if slot:
                block = ospec.corrected_block(cfg, toks, p, ospec.keep_threshold(kappa), draws)
                kept += sum(int(x == y) for x, y in zip(block, toks[:K - 1]))
                total += K - 1
            else:
                block = toks
        drafts = block
        rows = torch.tensor([drafts], dtype=torch.int32, device=dev)
        U.verify_block(model, kv, rows, cap, 1, zp_g, ws, status)
        zp = ospec.verify_logits(cfg, w64, seq, drafts)
        zp_gpu = zp_g.cpu().numpy()[0]
        assert_logits_close(zp_gpu, zp, "verify step %d" % seq.step)
        a, committed, extra = ospec.spec_accept(zq_gpu, zp_gpu, drafts, 1.0, draws)
        U.spec_accept(zq_g, zp_g, rows, 1.0, SEED, step_g, a_g, c_g, e_g, aws, status=status)
        assert int(a_g.item()) == a
        np.testing.assert_array_equal(c_g.cpu().numpy()[0][: a + 1], committed)
        U.kv_commit(kv, a_g, K, step_g, status)
        ospec.commit(seq, a, committed)
    assert int(status.item()) == 0
    if kappa == 1.0:
        assert kept == total
    elif kappa == 0.0 and prior == 0:
        assert kept == 0
    progress("multi-pass draft prior %d kappa %g: %d of %d rows kept" % (prior, kappa, kept,
                                                                       total))
