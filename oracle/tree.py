"""Tree sampler of the Psi-Spec step (oracle, test infrastructure).

What the pages say.  Besides the linear sampler (one drafted block per step)
there is a tree sampler, for per-request speed at low batch: from the one draft
pass it takes the top-K tokens at every drafted position, forms the K^(B-1)
sequences they span, ranks them by joint log-probability, keeps the best V,
verifies every kept prefix with the AR model and keeps the longest prefix the
verifier accepts (picx.dev summary, "Psi-Speculative Sampler"; paperglide reader,
"The Psi-Speculative Sampler", the worked example and the step list, and
"Empirical Results", parameters (B, K, V)).  The pages do not spell out the
multi-candidate accept rule.  Naming here: the block length is ``K`` (as in
``oracle.spec``), the pages' top-K is ``topk`` and their V is ``n_keep``.

Readings (each listed in the design notes):

* the first drafted token d_1 comes from the AR row of the draft pass, as in
  the linear sampler (drawn with Philox slot 0, j = 0), and heads every
  candidate; the candidates range over the positions 2..K;
* top-k of a row orders the fp32 logits, larger first, equal values by
  smaller token id;
* the joint log-probability of a candidate differs from the sum over its
  positions of (logit of its token - largest logit of that row) by a term that
  is the same for every candidate, at any temperature; the ranking uses that
  sum, each term rounded to an integer multiple of 2^-20 (``score_delta``),
  so that the ranking is exact integer arithmetic; equal scores are ordered by
  the candidates' top-k rank tuples, lexicographically;
* the kept candidates form a prefix tree.  Node 0 is d_1; the candidates are
  walked in rank order and each new prefix becomes the next node, by depth.
  A tree of n_keep candidates has at most 1 + n_keep * (K - 1) nodes; the
  verify pass always runs that many rows per sequence, the rows past the tree
  repeat d_1 at depth 0 and see only the context and themselves;
* verify: node i sits at position kv_len + 1 + depth(i), its K/V go to cache
  slot kv_len + 1 + i, and it attends to the context (slots <= kv_len, the
  anchor included) and to the slots of its ancestors and itself;
* lossless accept rule (a reading: the pages leave it open): starting at the
  root, draw x ~ p at the current node (the verifier's next-token law there,
  canonical integer sampler, Philox slot 2 with j = depth + 1); if a child of
  the node carries token x, move to it and repeat; otherwise stop.  Every
  emitted token is an exact draw from the AR model given the tokens before
  it, so the output law is the AR law whatever the tree holds; a leaf's draw
  is the bonus token.  a = number of tree nodes on the walk (d_1 included);
  the step commits those a tokens and the last draw x;
* commit: the K/V of the walked nodes move to the contiguous slots
  kv_len + 1 .. kv_len + a - 1 (node 0 already sits at kv_len + 1), then
  kv_len grows by 1 + a as in the linear step.

Pins (tests/test_oracle_tree.py): top-k against rank counting; the kept set
against fp64 joint log-probabilities of q at a temperature; the pages' worked
example shape (tests/golden/tree_example.json); full and greedy trees;
each node's verify logits against a plain uncached causal forward over its
path; exact enumeration of one step's output law against the AR model.
"""
import itertools

import numpy as np

from . import canonical as cn
from .model import forward
from .philox import SLOT_DRAFT, SLOT_EXTRA
from .spec import draft_logits

F32 = np.float32
SCORE_SHIFT = 20              # score unit: 2^-20 of a logit
DELTA_FLOOR = -(1 << 40)      # per-position floor of the integer score
ENUM_LIMIT = 1 << 20          # candidates the plain enumeration will list


def top_k(z32, k):
    """Token ids of the k largest fp32 logits, largest first, ties by id."""
    z = np.asarray(z32, dtype=F32)
    if not np.all(np.isfinite(z)):
        raise ValueError("non-finite logit in a drafted row")
    return [int(v) for v in np.argsort(-z, kind="stable")[:k]]


def score_delta(z_t, z_top):
    """Integer score of one position: rint(fp32(z_t - z_top) * 2^20), floored."""
    with np.errstate(over="ignore"):
        d = F32(F32(z_t) - F32(z_top))
    if d < F32(-(1 << 20)):
        return DELTA_FLOOR
    return int(np.rint(d * F32(1 << SCORE_SHIFT)))


def tree_candidates(zq32, topk, n_keep):
    """The n_keep best of the topk^(K-1) candidates, best first.

    Returns (rank tuples, per-position top-k token lists, per-position deltas);
    rank tuple entry i is the top-k rank of the token at position i + 2."""
    K = zq32.shape[0]
    tops = [top_k(zq32[j], topk) for j in range(1, K)]
    deltas = [[score_delta(zq32[j][t], zq32[j][tops[j - 1][0]]) for t in tops[j - 1]]
              for j in range(1, K)]
    if topk ** (K - 1) > ENUM_LIMIT:
        raise ValueError("too many candidates for the plain enumeration")
    if n_keep > topk ** (K - 1):
        raise ValueError("n_keep exceeds the number of candidates")
    scored = []
    for ranks in itertools.product(range(topk), repeat=K - 1):
        score = sum(deltas[i][r] for i, r in enumerate(ranks))
        scored.append((-score, ranks))
    scored.sort()
    return [ranks for _, ranks in scored[:n_keep]], tops, deltas


class Tree:
    """Prefix tree of the kept candidates plus padding rows (see header)."""

    def __init__(self, tokens, parent, depth, n_nodes, anc, K):
        self.tokens, self.parent, self.depth = tokens, parent, depth
        self.n_nodes, self.anc, self.K = n_nodes, anc, K
        self.N = len(tokens)

    def children(self, u):
        return [c for c in range(self.n_nodes) if self.parent[c] == u]

    def path_tokens(self, i):
        """Tokens from the root to node i."""
        out = []
        while i >= 0:
            out.append(self.tokens[i])
            i = self.parent[i]
        return out[::-1]


def n_rows(K, n_keep):
    """Verify rows per sequence: 1 + n_keep * (K - 1)."""
    return 1 + n_keep * (K - 1)


def build_tree(zq32, d1, topk, n_keep):
    K = zq32.shape[0]
    ranks_list, tops, _ = tree_candidates(zq32, topk, n_keep)
    node_of = {(): 0}
    tokens, parent, depth = [int(d1)], [-1], [0]
    for ranks in ranks_list:
        for dl in range(1, K):
            pre = ranks[:dl]
            if pre in node_of:
                continue
            node_of[pre] = len(tokens)
            tokens.append(tops[dl - 1][ranks[dl - 1]])
            parent.append(node_of[ranks[: dl - 1]])
            depth.append(dl)
    n_nodes = len(tokens)
    anc = []
    for i in range(n_nodes):
        s, u = set(), i
        while u >= 0:
            s.add(u)
            u = parent[u]
        anc.append(s)
    for i in range(n_nodes, n_rows(K, n_keep)):
        tokens.append(int(d1))
        parent.append(-1)
        depth.append(0)
        anc.append({i})
    return Tree(tokens, parent, depth, n_nodes, anc, K)


def tree_verify_logits(cfg, wts, seq, tree, act_round=None):
    """Verify pass over the tree's nodes (AR weights). fp64 [n_nodes, V]."""
    n, kv = tree.n_nodes, seq.kv_len
    ids = tree.tokens[:n]
    pos = kv + 1 + np.asarray(tree.depth[:n])
    slots = kv + 1 + np.arange(n)
    key_sets = [list(range(kv + 1)) + [kv + 1 + a for a in tree.anc[i]] for i in range(n)]
    return forward(cfg, wts, seq.cache, ids, pos, np.zeros(n), None, act_round=act_round,
                   slots=slots, key_sets=key_sets)


def tree_accept(tree, zp32, inv_temp, draws):
    """Walk from the root drawing from p; returns (a, committed, extra, path)."""
    u, path = 0, [0]
    while True:
        w, _ = cn.row_weights(zp32[u], inv_temp)
        x = int(draws.categorical(SLOT_EXTRA, tree.depth[u] + 1, w))
        nxt = [c for c in tree.children(u) if tree.tokens[c] == x]
        if not nxt:
            break
        u = nxt[0]
        path.append(u)
    committed = [tree.tokens[i] for i in path] + [x]
    return len(path), committed, x, path


def tree_commit(seq, path, a, committed):
    """Move the walked nodes' K/V to contiguous slots; append the tokens."""
    kv = seq.kv_len
    src = kv + 1 + np.asarray(path[:a])
    for li in range(len(seq.cache.k)):
        seq.cache.k[li][kv + 1: kv + 1 + a] = seq.cache.k[li][src].copy()
        seq.cache.v[li][kv + 1: kv + 1 + a] = seq.cache.v[li][src].copy()
    seq.kv_len += 1 + int(a)
    seq.tokens.extend(int(t) for t in committed)
    seq.step += 1


def step(cfg, wts, seq, K, topk, n_keep, inv_temp, draws):
    """Draft -> d_1 -> tree -> tree verify -> walk -> commit."""
    zq = draft_logits(cfg, wts, seq, K, draws=draws)
    zq32 = zq.astype(F32)
    d1 = int(draws.categorical(SLOT_DRAFT, 0, cn.row_weights(zq32[0], inv_temp)[0]))
    tree = build_tree(zq32, d1, topk, n_keep)
    zp = tree_verify_logits(cfg, wts, seq, tree)
    zp32 = zp.astype(F32)
    a, committed, extra, path = tree_accept(tree, zp32, inv_temp, draws)
    tree_commit(seq, path, a, committed)
    return dict(zq=zq, zq32=zq32, d1=d1, tree=tree, zp=zp, zp32=zp32, a=a,
                committed=committed, extra=extra, path=path)
