"""GPU parity of the tree sampler (uno_tree_build, uno_verify_tree,
uno_tree_accept, uno_tree_commit) against oracle.tree.

* Tree build on seeded fp32 draft logits: continuous rows, and rows quantised
  to a few values so that top-k entries and candidate scores tie.  Node tokens,
  parents, depths, ancestor bits and node counts must equal the oracle's
  exactly for shapes the oracle can enumerate; at the largest shape (K 32,
  topk 8, n_keep 64, vocab 151936) the kept set is checked against an
  independent best-first enumeration and the tree against its invariants.
* Tree steps on small models (LM head scaled up so that walks go deep): the
  tree built on the GPU from its draft logits equals the oracle's tree built
  from the same fp32 logits; each step starts the oracle from the library's
  committed bf16 K/V (teacher forcing); draft and verify logits of every node
  are compared with the exact oracle's forward: within 2e-2 abs + 1e-2 rel where
  the head is not scaled; where it is scaled by s the logits, and the rounding
  error of any bf16 implementation with them, grow s-fold, and the bf16
  yardstick applies instead (tests/gpu_util.py: every logit within 3x the bar,
  and over the whole test no more logits outside the bar than the oracle's
  bf16 mode puts there);
  the per-node draws and the walk (a, committed, extra token, path) equal the
  oracle's on the GPU's verify logits; both sides commit the same path, and
  after every step the library's cache over the newly committed positions
  (the moved K/V) must hold the oracle's K/V.
"""
import heapq

import numpy as np
import pytest
import torch

import synth
from oracle import canonical as cn
from oracle import model as om
from oracle import spec as ospec
from oracle import tree as ot

from gpu_util import (YardstickTally, assert_logits_close, gpu_or_fail, kv_to_logical,
                      progress, teacher_force_cache, u24)

pytestmark = pytest.mark.gpu

SEED = 5


def _anc_bits(tree, N):
    W = (N + 31) // 32
    out = np.zeros((N, W), dtype=np.uint32)
    for n in range(N):
        for m in tree.anc[n]:
            out[n, m >> 5] |= np.uint32(1 << (m & 31))
    return out


def _gpu_tree(U, zq, d1, topk, n_keep):
    B, K, V = zq.shape
    tb = U.TreeBuffers(B, K, topk, n_keep, V)
    dt = torch.zeros((B, K), dtype=torch.int32)
    dt[:, 0] = torch.as_tensor(d1, dtype=torch.int32)
    status = torch.zeros(B, dtype=torch.int32, device="cuda")
    U.tree_build(torch.from_numpy(zq).cuda(), dt.cuda(), tb, status)
    torch.cuda.synchronize()
    assert int(status.abs().sum()) == 0
    return tb


def _check_tree_equal(tb, b, tree):
    N = tb.N
    assert tree.N == N
    assert int(tb.n_nodes[b]) == tree.n_nodes
    np.testing.assert_array_equal(tb.tokens[b].cpu().numpy(), tree.tokens)
    np.testing.assert_array_equal(tb.parent[b].cpu().numpy(), tree.parent)
    np.testing.assert_array_equal(tb.depth[b].cpu().numpy(), tree.depth)
    np.testing.assert_array_equal(tb.anc[b].cpu().numpy(), _anc_bits(tree, N))


def _draft_rows(rng, B, K, V, kind):
    if kind == "ties":
        z = rng.integers(-3, 3, size=(B, K, V)).astype(np.float32) * np.float32(0.5)
        z[z == 0] = np.float32(-0.0) if rng.integers(2) else np.float32(0.0)
        return z
    return (rng.standard_normal((B, K, V)) * 2.0).astype(np.float32)


@pytest.mark.parametrize("K,topk,n_keep,V,kind", [
    (2, 1, 1, 512, "normal"), (3, 2, 4, 512, "ties"), (5, 3, 10, 512, "normal"),
    (5, 3, 10, 512, "ties"), (8, 4, 16, 1024, "normal"), (16, 2, 8, 512, "ties"),
    (16, 2, 64, 151936, "normal"), (6, 8, 64, 4096, "ties"), (11, 4, 64, 2048, "normal")])
def test_tree_build_matches_oracle(K, topk, n_keep, V, kind):
    U = gpu_or_fail()
    progress("tree build K=%d topk=%d n_keep=%d V=%d %s" % (K, topk, n_keep, V, kind))
    rng = np.random.default_rng([K, topk, n_keep, V, len(kind)])
    B = 3
    zq = _draft_rows(rng, B, K, V, kind)
    d1 = rng.integers(0, V, size=B)
    tb = _gpu_tree(U, zq, d1, topk, n_keep)
    for b in range(B):
        _check_tree_equal(tb, b, ot.build_tree(zq[b], int(d1[b]), topk, n_keep))


def _best_first(deltas, n):
    """The n best rank tuples in (score desc, tuple asc) order, by best-first
    search over the tuples (each tuple generated once: successors raise one
    position at or after the last raised one)."""
    P = len(deltas)
    start = (0,) * P
    heap = [(-sum(d[0] for d in deltas), start, 0)]
    out = []
    while heap and len(out) < n:
        negs, r, last = heapq.heappop(heap)
        out.append((-negs, r))
        for i in range(last, P):
            if r[i] + 1 < len(deltas[i]):
                s = list(r)
                s[i] += 1
                sc = -negs - deltas[i][r[i]] + deltas[i][r[i] + 1]
                heapq.heappush(heap, (-sc, tuple(s), i))
    return out


def test_tree_build_largest_shape_properties():
    U = gpu_or_fail()
    K, topk, n_keep, V, B = 32, 8, 64, 151936, 2
    progress("tree build largest shape")
    rng = np.random.default_rng(11)
    zq = _draft_rows(rng, B, K, V, "normal")
    zq[1, :, : V // 2] = np.round(zq[1, :, : V // 2])      # ties in one sequence
    d1 = rng.integers(0, V, size=B)
    tb = _gpu_tree(U, zq, d1, topk, n_keep)
    N = 1 + n_keep * (K - 1)
    for b in range(B):
        tops = [ot.top_k(zq[b, j], topk) for j in range(1, K)]
        deltas = [[ot.score_delta(zq[b, j, t], zq[b, j, tops[j - 1][0]]) for t in tops[j - 1]]
                  for j in range(1, K)]
        best = _best_first(deltas, n_keep)
        toks = tb.tokens[b].cpu().numpy()
        par = tb.parent[b].cpu().numpy()
        dep = tb.depth[b].cpu().numpy()
        anc = tb.anc[b].cpu().numpy()
        nn = int(tb.n_nodes[b])
        assert toks[0] == d1[b] and par[0] == -1 and dep[0] == 0
        for n in range(1, nn):
            assert 0 <= par[n] < n and dep[n] == dep[par[n]] + 1
            want = anc[par[n]].copy()
            want[n >> 5] |= np.uint32(1 << (n & 31))
            np.testing.assert_array_equal(anc[n], want)
        kids = {}
        for n in range(1, nn):
            kids.setdefault(par[n], []).append(n)
        leaves = [n for n in range(nn) if n not in kids]
        assert len(leaves) == n_keep and all(dep[n] == K - 1 for n in leaves)

        def path(n):
            out = []
            while n >= 0:
                out.append(int(toks[n]))
                n = par[n]
            return tuple(out[::-1])

        want_paths = [tuple([int(d1[b])] + [tops[i][r] for i, r in enumerate(rk)])
                      for _, rk in best]
        # leaves in node order follow the candidates' rank order
        assert [path(n) for n in sorted(leaves)] == want_paths
        assert nn == len({p[:d] for p in want_paths for d in range(1, K + 1)})
        for n in range(nn, N):
            assert toks[n] == d1[b] and par[n] == -1 and dep[n] == 0


def _peaky(cfg, seed, head_scale):
    """Synthetic weights with the LM head scaled by a power of two (exact in
    bf16): sharper next-token laws, so that walks go deep into the tree."""
    wts = synth.make_weights(cfg, seed)
    wts["lm_head"] = (wts["lm_head"].float() * head_scale).to(torch.bfloat16)
    return wts


@pytest.mark.parametrize(
    "name,cfg,B,K,topk,n_keep,n_steps,prompt_len,head_scale,inv_t,min_moves", [
        ("tiny-v32", dict(synth.TINY, vocab=32, mask_id=31), 2, 5, 4, 6, 10, 40, 4.0, 1.0, 1),
        ("tiny-v512", synth.TINY, 1, 4, 2, 3, 4, 20, 1.0, 1.0 / 0.7, 0),
        ("gqa-v64", dict(synth.SMALL_GQA, vocab=64, mask_id=63), 2, 8, 2, 8, 6, 150, 4.0, 1.0,
         1)])
def test_tree_steps_match_oracle(name, cfg, B, K, topk, n_keep, n_steps, prompt_len, head_scale,
                                 inv_t, min_moves):
    U = gpu_or_fail()
    progress("tree steps %s" % name)
    wts = _peaky(cfg, 2, head_scale)
    w64 = synth.to_f64(wts)
    model = U.Model(cfg, wts)
    V = cfg["vocab"]
    N = U.tree_rows(K, topk, n_keep)
    prompts = [synth.prompt_ids(cfg, prompt_len, 10 + b) for b in range(B)]
    cap = prompt_len + n_steps * (K + 1) + N + 8
    max_ctx = cap
    kv = U.PagedKV(cfg, B, cap, page_order=torch.randperm(
        B * ((cap + 15) // 16) + 5, generator=torch.Generator().manual_seed(4)), extra_pages=5)
    ws = U.alloc_workspace(max(U.workspace_bytes(model, B, K, max_ctx),
                               U.workspace_bytes(model, B, N, max_ctx),
                               U.workspace_bytes(model, B, prompt_len, max_ctx)))
    dev = "cuda"
    rows = torch.from_numpy(np.asarray([p[:-1] for p in prompts], dtype=np.int32)).to(dev)
    U.verify_block(model, kv, rows, max_ctx, 0, None, ws)
    U.kv_commit(kv, torch.full((B,), prompt_len - 2, dtype=torch.int32, device=dev),
                prompt_len - 1)
    seqs = []
    for b in range(B):
        s = ospec.Sequence(cfg, prompts[b], capacity=cap)
        ospec.prefill(cfg, w64, s)
        seqs.append(s)
    tb = U.TreeBuffers(B, K, topk, n_keep, V)
    zq_g = torch.empty((B, K, V), dtype=torch.float32, device=dev)
    zp_g = torch.empty((B, N, V), dtype=torch.float32, device=dev)
    d_g = torch.empty((B, K), dtype=torch.int32, device=dev)
    a_g = torch.empty(B, dtype=torch.int32, device=dev)
    c_g = torch.empty((B, K + 1), dtype=torch.int32, device=dev)
    e_g = torch.empty(B, dtype=torch.int32, device=dev)
    status = torch.zeros(B, dtype=torch.int32, device=dev)
    step_g = torch.zeros(B, dtype=torch.uint64).to(dev)
    worst, depths, moves = 0.0, [], 0
    tally = YardstickTally("%s logits" % name)

    def compare(got, exact, bf, where):
        if head_scale == 1.0:
            return assert_logits_close(got, exact, "%s %s" % (name, where))
        tally.add(got, exact, bf, where)
        return float(np.abs(got - exact).max())

    for st in range(n_steps):
        anchor = torch.tensor([s.tokens[-1] for s in seqs], dtype=torch.int32, device=dev)
        U.draft_block(model, kv, anchor, K, max_ctx, inv_t, SEED, step_g, zq_g, d_g, ws, status)
        U.tree_build(zq_g, d_g, tb, status)
        U.verify_tree(model, kv, tb, max_ctx, zp_g, ws, status)
        U.tree_accept(zp_g, tb, inv_t, SEED, step_g, a_g, c_g, e_g, status)
        zq_all, zp_all = zq_g.cpu().numpy(), zp_g.cpu().numpy()
        d_all, a_all, c_all = d_g.cpu().numpy(), a_g.cpu().numpy(), c_g.cpu().numpy()
        e_all, path_all, smp = e_g.cpu().numpy(), tb.path.cpu().numpy(), tb.sample.cpu().numpy()
        kv_before = [s.kv_len for s in seqs]
        for b, s in enumerate(seqs):
            teacher_force_cache(s, kv, b)
            s_bf = s.copy() if head_scale != 1.0 else None
            zq = ospec.draft_logits(cfg, w64, s, K)
            zq_bf = (ospec.draft_logits(cfg, w64, s_bf, K, act_round=om.bf16_round)
                     if s_bf is not None else None)
            worst = max(worst, compare(zq_all[b], zq, zq_bf, "draft b%d step %d" % (b, st)))
            w0, _ = cn.row_weights(zq_all[b, 0], inv_t)
            d1 = cn.categorical(w0, u24(SEED, 0, 0, b, st))
            assert d_all[b, 0] == d1
            tree = ot.build_tree(zq_all[b], d1, topk, n_keep)
            _check_tree_equal(tb, b, tree)
            zp = ot.tree_verify_logits(cfg, w64, s, tree)
            zp_bf = (ot.tree_verify_logits(cfg, w64, s_bf, tree, act_round=om.bf16_round)
                     if s_bf is not None else None)
            worst = max(worst, compare(zp_all[b, : tree.n_nodes], zp, zp_bf,
                                       "tree verify b%d step %d" % (b, st)))
            for n in range(tree.n_nodes):
                wn, _ = cn.row_weights(zp_all[b, n], inv_t)
                assert smp[b, n] == cn.categorical(wn, u24(SEED, 2, tree.depth[n] + 1, b, st))
            assert (smp[b, tree.n_nodes:] == -1).all()
            a, committed, extra, path = ot.tree_accept(tree, zp_all[b], inv_t,
                                                       ospec.PhiloxDraws(SEED, b, st))
            assert a_all[b] == a and e_all[b] == extra
            np.testing.assert_array_equal(c_all[b], committed + [-1] * (K + 1 - len(committed)))
            np.testing.assert_array_equal(path_all[b], path + [-1] * (K - len(path)))
            depths.append(a)
            moves += sum(1 for d in range(1, a) if path[d] != d)
            ot.tree_commit(s, path, a, committed)
        U.tree_commit(model, kv, tb, a_g, step_g, status)
        kvl = kv.kv_len.cpu().numpy()
        assert [int(x) for x in kvl] == [s.kv_len for s in seqs]
        assert int(status.abs().sum()) == 0
        # the newly committed positions (moved K/V included) hold the oracle's K/V
        for b, s in enumerate(seqs):
            n0, n1 = kv_before[b], s.kv_len
            for li in range(cfg["n_layers"]):
                kg, vg = kv_to_logical(kv, li, b, n1)
                assert_logits_close(kg[n0:], s.cache.k[li][n0:n1],
                                    "%s K layer %d b%d step %d" % (name, li, b, st))
                assert_logits_close(vg[n0:], s.cache.v[li][n0:n1],
                                    "%s V layer %d b%d step %d" % (name, li, b, st))
    summary = tally.finish() if head_scale != 1.0 else "elementwise within the bar"
    progress("tree steps %s: worst logit error %.2e (%s), accept lengths %s, %d K/V moves"
             % (name, worst, summary, np.bincount(depths).tolist(), moves))
    assert moves >= min_moves, "no walked node left its slot: the K/V moves were not exercised"
