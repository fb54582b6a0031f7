"""Pins of the oracle's tree sampler (oracle/tree.py).

* top-k against rank counting (ties and signed zeros included);
* the integer score of a position against its definition's arithmetic cases;
* the kept candidates are the best by the fp64 joint log-probability of the
  drafted laws at a temperature (independent of the integer score);
* the pages' worked example (tests/golden/tree_example.json): candidate set,
  tree shape and the accept walk;
* full and greedy trees; structural invariants of the node order;
* every node's verify logits equal a plain uncached causal forward over the
  prompt and the node's root path; a one-candidate tree equals the linear
  verify pass; after the commit the cache equals a linear verify of the kept
  path;
* exact enumeration of one tree step (vocab 8): every output sequence has the
  AR model's probability (the walk is lossless), the outputs are prefix-free
  and their probabilities sum to one.
"""
import json
import os
from fractions import Fraction

import numpy as np
import pytest

import synth
from oracle import canonical as cn
from oracle import model as om
from oracle import spec
from oracle import tree as ot
from oracle.philox import SLOT_DRAFT, SLOT_EXTRA
from test_oracle_spec import _Branch, _EnumDraws, _ar_probs

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rank_by_counting(z, v):
    """Entries ordered before v: larger values, and equal values at smaller ids."""
    return int(np.sum(z > z[v]) + np.sum(z[:v] == z[v]))


def test_top_k_matches_rank_counting():
    rng = np.random.default_rng(0)
    for trial in range(24):
        V = int(rng.integers(8, 300))
        if trial % 3 == 0:
            z = rng.integers(-3, 4, size=V).astype(np.float32)          # many ties
        elif trial % 3 == 1:
            z = rng.choice(np.array([0.0, -0.0, 1.5, -2.0], dtype=np.float32), size=V)
        else:
            z = rng.standard_normal(V).astype(np.float32)
        k = int(rng.integers(1, min(V, 9) + 1))
        ranks = [_rank_by_counting(z, v) for v in range(V)]
        want = [ranks.index(r) for r in range(k)]
        assert ot.top_k(z, k) == want


def test_score_delta_cases():
    f = np.float32
    assert ot.score_delta(f(2.0), f(2.0)) == 0
    assert ot.score_delta(f(1.5), f(2.0)) == -(1 << 19)
    # 2^-22 * 2^20 = 0.25 rounds to 0; 3 * 2^-21 * 2^20 = 1.5 rounds to even 2
    assert ot.score_delta(f(1.0) - f(2.0 ** -22), f(1.0)) == 0
    assert ot.score_delta(f(1.0) - f(3 * 2.0 ** -21), f(1.0)) == -2
    # the difference is an fp32 operation: 1e8 - 1 is not representable
    assert ot.score_delta(f(1e8 - 8), f(1e8)) == -8 * (1 << 20)
    assert ot.score_delta(f(-3e38), f(3e38)) == ot.DELTA_FLOOR
    assert ot.score_delta(f(-1.5e6), f(0.0)) == ot.DELTA_FLOOR


def _brute_top(z, k):
    ranks = [_rank_by_counting(z, v) for v in range(len(z))]
    return [ranks.index(r) for r in range(k)]


@pytest.mark.parametrize("inv_t", [1.0, 1.0 / 0.7, 2.5])
def test_kept_candidates_are_best_by_joint_log_probability(inv_t):
    rng = np.random.default_rng(int(inv_t * 100))
    K, V, topk, n_keep = 5, 40, 3, 10
    z = (rng.standard_normal((K, V)) * 2.0).astype(np.float32)
    ranks_list, _, _ = ot.tree_candidates(z, topk, n_keep)
    # fp64 log q_j at the temperature, over the brute-force top-k sets
    lq = []
    for j in range(1, K):
        x = z[j].astype(np.float64) * inv_t
        lse = x.max() + np.log(np.exp(x - x.max()).sum())
        lq.append({v: x[v] - lse for v in _brute_top(z[j], topk)})
    tops = [_brute_top(z[j], topk) for j in range(1, K)]

    def joint(ranks):
        return sum(lq[i][tops[i][r]] for i, r in enumerate(ranks))

    allc = {r: joint(r) for r in np.ndindex(*([topk] * (K - 1)))}
    kept = [tuple(r) for r in ranks_list]
    assert len(set(kept)) == n_keep
    tol = 1e-5 * inv_t
    worst_kept = min(allc[r] for r in kept)
    best_dropped = max(v for r, v in allc.items() if r not in kept)
    assert worst_kept >= best_dropped - tol
    vals = [allc[r] for r in kept]
    assert all(vals[i] >= vals[i + 1] - tol for i in range(len(vals) - 1))


def test_pages_worked_example():
    ex = json.load(open(os.path.join(GOLDEN, "tree_example.json")))
    name = ex["vocab"]
    ids = {t: i for i, t in enumerate(name)}
    zq32 = np.log(np.asarray(ex["draft_probs"], dtype=np.float64)).astype(np.float32)
    assert zq32.shape[0] == ex["block_length"]
    ranks_list, tops, _ = ot.tree_candidates(zq32, ex["topk"], ex["n_keep"])
    cands = [[name[ex["d1"]]] + [name[tops[i][r]] for i, r in enumerate(rk)] for rk in ranks_list]
    assert cands == ex["expected_candidates"]
    tree = ot.build_tree(zq32, ex["d1"], ex["topk"], ex["n_keep"])
    et = ex["expected_tree"]
    assert tree.n_nodes == tree.N == ot.n_rows(ex["block_length"], ex["n_keep"]) == 5
    assert [name[t] for t in tree.tokens] == et["tokens"]
    assert tree.parent == et["parent"] and tree.depth == et["depth"]

    class Scripted:
        def __init__(self, toks):
            self.toks = list(toks)

        def categorical(self, slot, j, w):
            assert slot == SLOT_EXTRA
            return self.toks.pop(0)

    w = ex["walk"]
    zp32 = np.zeros((tree.N, len(name)), dtype=np.float32)
    a, committed, extra, path = ot.tree_accept(tree, zp32, 1.0,
                                               Scripted(ids[t] for t in w["draws"]))
    assert [name[t] for t in committed] == w["expected_committed"]
    assert a == w["expected_accept_len"] and path == w["expected_path"]
    assert name[extra] == w["expected_committed"][-1]


def test_full_tree_and_greedy_chain():
    rng = np.random.default_rng(3)
    K, V = 4, 30
    z = rng.standard_normal((K, V)).astype(np.float32)
    full = ot.build_tree(z, 7, 3, 27)
    assert full.n_nodes == 1 + 3 + 9 + 27
    for u in range(full.n_nodes):
        kids = full.children(u)
        if full.depth[u] < K - 1:
            assert sorted(full.tokens[c] for c in kids) == sorted(_brute_top(z[full.depth[u] + 1], 3))
        else:
            assert kids == []
    chain = ot.build_tree(z, 7, 1, 1)
    assert chain.tokens == [7] + [int(np.argmax(z[j])) for j in range(1, K)]
    assert chain.parent == [-1, 0, 1, 2] and chain.depth == [0, 1, 2, 3]


def test_tree_structure_invariants():
    rng = np.random.default_rng(5)
    K, V, topk, n_keep = 6, 50, 2, 9
    z = rng.standard_normal((K, V)).astype(np.float32)
    t = ot.build_tree(z, 11, topk, n_keep)
    assert t.N == 1 + n_keep * (K - 1)
    for i in range(1, t.n_nodes):
        p = t.parent[i]
        assert 0 <= p < i and t.depth[i] == t.depth[p] + 1
        assert t.anc[i] == t.anc[p] | {i}
    leaves = [i for i in range(t.n_nodes) if not t.children(i)]
    assert len(leaves) == n_keep and all(t.depth[i] == K - 1 for i in leaves)
    ranks_list, tops, _ = ot.tree_candidates(z, topk, n_keep)
    want = {tuple([11] + [tops[i][r] for i, r in enumerate(rk)]) for rk in ranks_list}
    assert {tuple(t.path_tokens(i)) for i in leaves} == want
    # node order: the candidates in rank order, each one's new prefixes by depth
    order = []
    for rk in ranks_list:
        toks = [11] + [tops[i][r] for i, r in enumerate(rk)]
        for d in range(K):
            if toks[: d + 1] not in order:
                order.append(toks[: d + 1])
    assert [t.path_tokens(i) for i in range(t.n_nodes)] == order
    for i in range(t.n_nodes, t.N):          # padding rows
        assert t.tokens[i] == 11 and t.parent[i] == -1 and t.depth[i] == 0 and t.anc[i] == {i}


@pytest.fixture(scope="module")
def tiny():
    cfg = synth.TINY
    return cfg, synth.to_f64(synth.make_weights(cfg, 1))


def _tree_after_draft(cfg, w, prompt, K, topk, n_keep, seed=0):
    seq = spec.Sequence(cfg, prompt, capacity=len(prompt) + 1 + n_keep * K + 4)
    spec.prefill(cfg, w, seq)
    draws = spec.PhiloxDraws(seed, 0, 0)
    zq32 = spec.draft_logits(cfg, w, seq, K, draws=draws).astype(np.float32)
    d1 = draws.categorical(SLOT_DRAFT, 0, cn.row_weights(zq32[0], 1.0)[0])
    return seq, ot.build_tree(zq32, d1, topk, n_keep)


def test_tree_verify_matches_uncached_causal_forward(tiny):
    cfg, w = tiny
    prompt = [5, 300, 17, 42, 99, 3, 250]
    seq, tree = _tree_after_draft(cfg, w, prompt, 4, 2, 3)
    assert tree.n_nodes >= 6          # branching: node index != depth
    zp = ot.tree_verify_logits(cfg, w, seq, tree)
    for i in range(tree.n_nodes):
        ref = om.full_causal_logits(cfg, w, prompt + tree.path_tokens(i))[-1]
        assert np.abs(zp[i] - ref).max() < 1e-9 * max(1.0, np.abs(ref).max()), i


def test_single_candidate_tree_equals_linear_verify(tiny):
    cfg, w = tiny
    prompt = [9, 8, 7, 6, 5]
    seq, tree = _tree_after_draft(cfg, w, prompt, 5, 2, 1)
    assert tree.n_nodes == 5 and tree.depth == list(range(5))
    s2 = seq.copy()
    zt = ot.tree_verify_logits(cfg, w, seq, tree)
    zl = spec.verify_logits(cfg, w, s2, tree.tokens)
    assert np.abs(zt - zl).max() < 1e-12


def test_commit_leaves_the_cache_of_a_linear_verify(tiny):
    cfg, w = tiny
    prompt = [1, 2, 3, 4, 5, 6]
    seq, tree = _tree_after_draft(cfg, w, prompt, 4, 2, 4)
    # walk to the deepest node of the last candidate (a branch off the first)
    leaf = max(i for i in range(tree.n_nodes) if tree.depth[i] == 3)
    path = []
    u = leaf
    while u >= 0:
        path.append(u)
        u = tree.parent[u]
    path = path[::-1]
    assert path != list(range(4))          # the nodes are not already contiguous
    kv0 = seq.kv_len
    ref = seq.copy()
    ot.tree_verify_logits(cfg, w, seq, tree)
    toks = [tree.tokens[i] for i in path]
    ot.tree_commit(seq, path, len(path), toks + [0])
    spec.verify_logits(cfg, w, ref, toks)
    for li in range(cfg["n_layers"]):
        sl = slice(kv0, kv0 + 1 + len(path))
        assert np.abs(seq.cache.k[li][sl] - ref.cache.k[li][sl]).max() < 1e-12
        assert np.abs(seq.cache.v[li][sl] - ref.cache.v[li][sl]).max() < 1e-12
    assert seq.kv_len == kv0 + 1 + len(path)


@pytest.fixture(scope="module")
def toy():
    cfg = synth.VOCAB8
    wts = synth.make_weights(cfg, 3)
    for lw in wts["layers"]:
        for p in lw["lora_b"]:
            lw["lora_b"][p] = lw["lora_b"][p] * 40
    return cfg, synth.to_f64(wts)


def _enumerate_tree_step(cfg, w, seq, K, topk, n_keep, inv_t):
    out = {}
    stack = [([], Fraction(1))]
    while stack:
        path, prob = stack.pop()
        s = seq.copy()
        try:
            r = ot.step(cfg, w, s, K, topk, n_keep, inv_t, _EnumDraws(path))
        except _Branch as br:
            for dec, p in br.dist.items():
                stack.append((path + [dec], prob * p))
            continue
        key = tuple(r["committed"])
        out[key] = out.get(key, Fraction(0)) + prob
    return out


@pytest.mark.parametrize("K,topk,n_keep,inv_t", [(2, 2, 1, 1.0), (2, 3, 3, 1.0), (3, 2, 2, 1.0),
                                                 (3, 2, 4, 1.0), (3, 3, 5, 1.0 / 0.7)])
def test_exact_enumeration_tree_step_lossless(toy, K, topk, n_keep, inv_t):
    cfg, w = toy
    prompt = [1, 5, 2, 6, 0]
    seq = spec.Sequence(cfg, prompt, capacity=len(prompt) + 2 + n_keep * K + 4)
    spec.prefill(cfg, w, seq)
    dist = _enumerate_tree_step(cfg, w, seq, K, topk, n_keep, np.float32(inv_t))
    assert sum(dist.values()) == 1
    outs = list(dist)
    for c in outs:
        assert 2 <= len(c) <= K + 1
        assert not any(c != d and d[: len(c)] == c for d in outs)     # prefix-free
    assert any(len(c) > 2 for c in outs)                              # the tree is used
    worst = 0.0
    for c, pc in dist.items():
        pref, pe = tuple(prompt), 1.0
        for t in c:
            pe *= _ar_probs(cfg, w, pref, float(inv_t))[t]
            pref += (t,)
        worst = max(worst, abs(float(pc) - pe))
    assert worst < 1e-6, worst
