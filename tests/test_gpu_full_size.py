"""Full-size parity on the Qwen3-8B shape (d_model 4096, 32/8 heads x 128,
SwiGLU 12288, vocab 151936, LoRA r128 alpha 256), on sampled outputs the
oracle can compute: one draft and one verify pass (K = 16) of a sequence whose
committed context is seeded synthetic K/V.

Every logit of the sampled sequence (2 x 16 x 151936) is compared.

* 8B width, 1 layer, batch 1, context 1023: within 2e-2 abs + 1e-2 rel of the
  oracle in its bf16-activation mode (the same computation with the GEMM
  inputs and the K/V cache entries rounded to bfloat16, which bf16 matrix cores
  and a bf16 cache require).
* 36 layers, batch 1 / context 1023 and batch 64 / context 9216 (the benchmark's
  launch configuration; sequence 37 is recomputed by the oracle): bf16
  activation rounding compounds with depth (about as the square root of the
  number of layers) and a rounding computation is sensitive to any earlier
  difference, so no elementwise bound of that size holds between two
  implementations there.  The criterion is the rounding model's own accuracy:
  the GPU's mean and largest deviation from the exact fp64 oracle may exceed
  those of the bf16-activation oracle by at most 25% (+1e-3 on the mean).

Afterwards the sampler is checked bit-exact on the oracle's fp32 logits."""
import numpy as np
import pytest
import torch

import synth
from oracle import spec as ospec
from oracle.model import bf16_round

from gpu_util import assert_logits_close, gpu_or_fail, load_kv_logical, progress

pytestmark = pytest.mark.gpu

K = 16


@pytest.fixture(scope="module")
def big():
    U = gpu_or_fail()
    cfg = synth.QWEN3_8B
    progress("8B: generating weights on the host")
    wts = synth.make_weights(cfg, seed=0)
    progress("8B: uploading")
    model = U.Model(cfg, wts)
    torch.cuda.synchronize()
    return U, cfg, wts, synth.to_f64_lazy(wts), model


def _check(gpu, bf, exact, elementwise, what):
    gpu = gpu.astype(np.float64)
    d_gpu = np.abs(gpu - exact)
    d_bf = np.abs(bf - exact)
    progress("%s: |GPU - fp64| mean %.4f max %.3f; |bf16 model - fp64| mean %.4f max %.3f; "
             "|GPU - bf16 model| max %.4f" % (what, d_gpu.mean(), d_gpu.max(), d_bf.mean(),
                                             d_bf.max(), np.abs(gpu - bf).max()))
    if elementwise:
        return assert_logits_close(gpu, bf, what + " logits")
    assert d_gpu.mean() <= 1.25 * d_bf.mean() + 1e-3, what + ": mean deviation"
    assert d_gpu.max() <= 1.25 * d_bf.max(), what + ": largest deviation"
    return float(d_gpu.max())


def _run(big, B, ctx, b_check, elementwise=False, K=K, inv_t=1.0):
    U, cfg, wts, w64, model = big
    cap = ctx + 2 * K + 8
    n_pages = B * ((cap + 15) // 16)
    kv = U.PagedKV(cfg, B, cap, page_order=torch.randperm(
        n_pages, generator=torch.Generator().manual_seed(ctx)))
    if B > 1:
        synth.fill_kv_device(kv.k_pages, kv.v_pages, seed=ctx)
    k, v = synth.kv_values(cfg, ctx, seed=21, seq=b_check)
    load_kv_logical(kv, b_check, k, v)
    kv.kv_len.fill_(ctx)
    toks = synth.random_tokens(ctx + 1, cfg["vocab"], 300, (B, ctx + 1))
    seq = ospec.Sequence(cfg, toks[b_check], capacity=cap)
    for li in range(cfg["n_layers"]):
        seq.cache.k[li][:ctx] = k[li].double().numpy()
        seq.cache.v[li][:ctx] = v[li].double().numpy()
    seq.kv_len = ctx
    del k, v
    ws = U.alloc_workspace(U.workspace_bytes(model, B, K, cap))
    V = cfg["vocab"]
    zq = torch.empty((B, K, V), dtype=torch.float32, device="cuda")
    zp = torch.empty((B, K, V), dtype=torch.float32, device="cuda")
    d = torch.empty((B, K), dtype=torch.int32, device="cuda")
    status = torch.zeros(B, dtype=torch.int32, device="cuda")
    anchor = torch.from_numpy(toks[:, -1].copy()).cuda()
    U.draft_block(model, kv, anchor, K, cap, 1.0, 0, torch.zeros(B, dtype=torch.uint64).cuda(),
                  zq, d, ws, status)
    seq_bf = seq.copy()
    progress("8B L%d b%d: GPU draft done; oracle draft passes (fp64, bf16 activations)" % (
        cfg["n_layers"], B))
    zq_ref = ospec.draft_logits(cfg, w64, seq, K)
    zq_bf = ospec.draft_logits(cfg, w64, seq_bf, K, act_round=bf16_round)
    zq_g = zq[b_check].cpu().numpy()
    err_q = _check(zq_g, zq_bf, zq_ref, elementwise, "8B L%d b%d draft" % (cfg["n_layers"], B))
    drafts = ospec.draft_sample(zq_ref.astype(np.float32), 1.0, ospec.PhiloxDraws(0, b_check, 0))
    rows = np.array(d.cpu().numpy(), dtype=np.int32)     # other sequences: any tokens
    rows[b_check] = drafts
    U.verify_block(model, kv, torch.from_numpy(rows).cuda(), cap, 1, zp, ws, status)
    progress("8B L%d b%d: GPU verify done; oracle verify passes" % (cfg["n_layers"], B))
    zp_ref = ospec.verify_logits(cfg, w64, seq, drafts)
    zp_bf = ospec.verify_logits(cfg, w64, seq_bf, drafts, act_round=bf16_round)
    zp_g = zp[b_check].cpu().numpy()
    err_p = _check(zp_g, zp_bf, zp_ref, elementwise, "8B L%d b%d verify" % (cfg["n_layers"], B))
    assert (status.cpu().numpy() == 0).all()
    # sampler, bit-exact on the oracle's own fp32 logits
    zq32, zp32 = zq_ref.astype(np.float32), zp_ref.astype(np.float32)
    a_ref, comm_ref, e_ref = ospec.spec_accept(zq32, zp32, drafts, inv_t,
                                               ospec.PhiloxDraws(0, 0, 0))
    a = torch.empty(1, dtype=torch.int32, device="cuda")
    c = torch.empty((1, K + 1), dtype=torch.int32, device="cuda")
    e = torch.empty(1, dtype=torch.int32, device="cuda")
    U.spec_accept(torch.from_numpy(zq32[None]).cuda(), torch.from_numpy(zp32[None]).cuda(),
                  torch.tensor([drafts], dtype=torch.int32, device="cuda"), inv_t, 0,
                  torch.zeros(1, dtype=torch.uint64).cuda(), a, c, e,
                  U.alloc_workspace(U.spec_accept_workspace_bytes(1, K)))
    assert (int(a.item()), int(e.item())) == (a_ref, e_ref)
    progress("8B L%d b%d ctx %d: max logit error draft %.2e verify %.2e; a = %d" % (
        cfg["n_layers"], B, ctx, err_q, err_p, a_ref))
    del kv, ws, zq, zp
    torch.cuda.empty_cache()


@pytest.fixture(scope="module")
def big1():
    U = gpu_or_fail()
    cfg = dict(synth.QWEN3_8B, n_layers=1)
    wts = synth.make_weights(cfg, seed=0)
    return U, cfg, wts, synth.to_f64_lazy(wts), U.Model(cfg, wts)


def test_8b_width_one_layer_elementwise(big1):
    _run(big1, 1, 1023, 0, elementwise=True)


def test_8b_width_one_layer_batch16_context_32768_k32(big1):
    """Long-context rollout shape (batch 16, context 32768, K = 32) at 8B width,
    one layer, elementwise; the sampler at temperature 0.7."""
    _run(big1, 16, 32768, 5, elementwise=True, K=32, inv_t=float(np.float32(1 / 0.7)))


def test_8b_batch1_context_1k(big):
    _run(big, 1, 1023, 0)


def test_8b_batch64_context_9216(big):
    _run(big, 64, 9216, 37)


@pytest.mark.parametrize("ctx", [1023, 2100])
def test_8b_width_one_layer_tree_sampler(big1, ctx):
    """Tree sampler at 8B width (one layer), batch 2, context 1023 and 2100,
    K = 16, top-2 per drafted position, 8 kept candidates (121 node rows per
    sequence): the tree built from the GPU's draft logits equals the oracle's
    tree on the same fp32 logits; every node's verify logits (121 x 151936)
    agree elementwise with the oracle's bf16-activation forward over the
    tree; the draws and the walk equal the oracle's on the GPU's logits.
    At context 2100 the tree-masked attention has 8 key ranges per (sequence,
    kv head, row group), 512 workgroups, and takes its two-stage form."""
    from oracle import canonical as cn
    from oracle import tree as ot
    U, cfg, wts, w64, model = big1
    B, b_check, topk, n_keep = 2, 1, 2, 8
    N = U.tree_rows(K, topk, n_keep)
    cap = ctx + N + K + 8
    kv = U.PagedKV(cfg, B, cap, page_order=torch.randperm(
        B * ((cap + 15) // 16), generator=torch.Generator().manual_seed(7)))
    synth.fill_kv_device(kv.k_pages, kv.v_pages, seed=8)
    k, v = synth.kv_values(cfg, ctx, seed=22, seq=b_check)
    load_kv_logical(kv, b_check, k, v)
    kv.kv_len.fill_(ctx)
    toks = synth.random_tokens(ctx + 1, cfg["vocab"], 301, (B, ctx + 1))
    seq = ospec.Sequence(cfg, toks[b_check], capacity=cap)
    seq.cache.k[0][:ctx] = k[0].double().numpy()
    seq.cache.v[0][:ctx] = v[0].double().numpy()
    seq.kv_len = ctx
    V = cfg["vocab"]
    ws = U.alloc_workspace(max(U.workspace_bytes(model, B, K, cap),
                               U.workspace_bytes(model, B, N, cap)))
    zq = torch.empty((B, K, V), dtype=torch.float32, device="cuda")
    zp = torch.empty((B, N, V), dtype=torch.float32, device="cuda")
    d = torch.empty((B, K), dtype=torch.int32, device="cuda")
    a = torch.empty(B, dtype=torch.int32, device="cuda")
    c = torch.empty((B, K + 1), dtype=torch.int32, device="cuda")
    e = torch.empty(B, dtype=torch.int32, device="cuda")
    status = torch.zeros(B, dtype=torch.int32, device="cuda")
    step = torch.zeros(B, dtype=torch.uint64).cuda()
    tb = U.TreeBuffers(B, K, topk, n_keep, V)
    anchor = torch.from_numpy(toks[:, -1].copy()).cuda()
    U.draft_block(model, kv, anchor, K, cap, 1.0, 0, step, zq, d, ws, status)
    U.tree_build(zq, d, tb, status)
    U.verify_tree(model, kv, tb, cap, zp, ws, status)
    U.tree_accept(zp, tb, 1.0, 0, step, a, c, e, status)
    torch.cuda.synchronize()
    assert (status.cpu().numpy() == 0).all()
    progress("8B L1 tree: GPU step done; oracle draft and tree verify (bf16 activations)")
    zq_g = zq[b_check].cpu().numpy()
    assert_logits_close(zq_g, ospec.draft_logits(cfg, w64, seq, K, act_round=bf16_round),
                        "8B L1 tree draft logits")
    u_d1 = ospec.PhiloxDraws(0, b_check, 0).u(0, 0)
    d1 = cn.categorical(cn.row_weights(zq_g[0], 1.0)[0], u_d1)
    assert int(d[b_check, 0]) == d1
    tree = ot.build_tree(zq_g, d1, topk, n_keep)
    assert int(tb.n_nodes[b_check]) == tree.n_nodes
    np.testing.assert_array_equal(tb.tokens[b_check].cpu().numpy(), tree.tokens)
    np.testing.assert_array_equal(tb.parent[b_check].cpu().numpy(), tree.parent)
    zp_ref = ot.tree_verify_logits(cfg, w64, seq, tree, act_round=bf16_round)
    zp_g = zp[b_check].cpu().numpy()
    err = assert_logits_close(zp_g[: tree.n_nodes], zp_ref, "8B L1 tree verify logits")
    a_ref, comm_ref, e_ref, path_ref = ot.tree_accept(tree, zp_g, 1.0,
                                                      ospec.PhiloxDraws(0, b_check, 0))
    assert int(a[b_check]) == a_ref and int(e[b_check]) == e_ref
    np.testing.assert_array_equal(tb.path[b_check].cpu().numpy(),
                                  path_ref + [-1] * (K - len(path_ref)))
    progress("8B L1 tree: %d nodes, max verify logit error %.2e, a = %d"
             % (tree.n_nodes, err, a_ref))
    del kv, ws, zq, zp
    torch.cuda.empty_cache()
