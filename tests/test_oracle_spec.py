"""Losslessness and structure pins of the oracle's decode step.

Exact enumeration (vocab 8, K = 1, 2, 3): the real ``oracle.spec.step`` is
replayed along every path of random decisions; each decision's probability is
counted exactly over the 2^24 values of its uniform (by bisection on the
oracle's own monotone sampler primitives).  The committed tokens, continued by
exact AR sampling, must reproduce the AR model's distribution (computed by a
plain uncached forward) within 1e-6.  A two-step enumeration (K = 1) checks the
cache/commit hand-over between steps.

Prefix-independent rows (vocab 512, K = 8): acceptance at each position equals
sum_v min(p, q) = 1 - TV(p, q) exactly up to the 2^-24 grid, and a 10^6-sample
chi-square of a vectorised replay of the oracle's sampler (cross-checked draw by
draw against ``oracle.spec.spec_accept``) against the first-token-at-position-j
law p_j.
"""
from fractions import Fraction

import numpy as np
import pytest
import scipy.stats

import synth
from oracle import canonical as cn
from oracle import model as om
from oracle import spec
from oracle.philox import (SLOT_ACCEPT, SLOT_DRAFT, SLOT_EXTRA, SLOT_KEEP, SLOT_PASS, noise_id,
                           token_id, uniform24, uniform24_np)

TWO24 = 1 << 24


def _lowest_u(pred):
    lo, hi = 0, TWO24
    while lo < hi:
        mid = (lo + hi) // 2
        if pred(mid):
            hi = mid
        else:
            lo = mid + 1
    return lo


class _Branch(Exception):
    def __init__(self, dist):
        self.dist = dist


class _EnumDraws:
    """Replays a fixed list of decisions; at the first new one, raises its exact
    distribution (decision -> probability over U)."""

    def __init__(self, path):
        self.path = path
        self.i = 0

    def _take(self, dist_fn):
        if self.i < len(self.path):
            d = self.path[self.i]
            self.i += 1
            return d
        raise _Branch(dist_fn())

    def noise(self, j, vocab):
        # uniform-prior noise tokens: a fixed Philox realisation (losslessness
        # must hold for any draft distribution, hence for any noise)
        return noise_id(7, j, 0, 0, vocab)

    def keep(self, i, j, keep_q24):
        # corrector decisions are enumerated with their exact probabilities
        def dist():
            out = {}
            if keep_q24 > 0:
                out[True] = Fraction(int(keep_q24), TWO24)
            if keep_q24 < TWO24:
                out[False] = Fraction(TWO24 - int(keep_q24), TWO24)
            return out
        return self._take(dist)

    def renoise(self, i, j, vocab):
        return token_id(7, SLOT_KEEP + 64 + i, j, 0, 0, vocab)

    def categorical(self, slot, j, weights):
        def dist():
            w = list(weights)
            starts = [_lowest_u(lambda u, v=v: cn.categorical(w, u) >= v) for v in range(len(w))]
            starts.append(TWO24)
            return {v: Fraction(starts[v + 1] - starts[v], TWO24)
                    for v in range(len(w)) if starts[v + 1] > starts[v]}
        return self._take(dist)

    def accept(self, slot, j, wq_d, sq, wp_d, sp):
        def dist():
            thr = _lowest_u(lambda u: not cn.accept(wq_d, sq, wp_d, sp, u))
            out = {}
            if thr > 0:
                out[True] = Fraction(thr, TWO24)
            if thr < TWO24:
                out[False] = Fraction(TWO24 - thr, TWO24)
            return out
        return self._take(dist)


class _FixedPassDraws(_EnumDraws):
    """Enumerates the final pass; the intermediate passes' samples are fixed."""

    def __init__(self, path, fixed):
        super().__init__(path)
        self.fixed = fixed          # {(slot, j): token}

    def categorical(self, slot, j, weights):
        if slot >= SLOT_PASS:
            return self.fixed[(slot, j)]
        return super().categorical(slot, j, weights)


def _enumerate_step(cfg, w, seq, K, inv_t, n_passes=1, fixed=None, kappa=1.0):
    """{committed tuple: probability} of one step from ``seq`` (exact; with
    ``fixed`` the intermediate draft passes' samples are held fixed, and the
    corrector's keep decisions between passes are enumerated)."""
    out = {}
    stack = [([], Fraction(1))]
    while stack:
        path, prob = stack.pop()
        s = seq.copy()
        draws = _EnumDraws(path) if fixed is None else _FixedPassDraws(path, fixed)
        try:
            r = spec.step(cfg, w, s, K, inv_t, draws, n_passes=n_passes, kappa=kappa)
        except _Branch as br:
            for dec, p in br.dist.items():
                stack.append((path + [dec], prob * p))
            continue
        key = tuple(r["committed"])
        out[key] = out.get(key, Fraction(0)) + prob
    return out


def _ar_probs(cfg, w, prefix, inv_t):
    z = om.full_causal_logits(cfg, w, list(prefix))[-1] * inv_t
    p = np.exp(z - z.max())
    return p / p.sum()


@pytest.fixture(scope="module")
def toy():
    cfg = synth.VOCAB8
    wts = synth.make_weights(cfg, 3)
    # larger LoRA B so that q differs visibly from p (more rejections)
    for lw in wts["layers"]:
        for p in lw["lora_b"]:
            lw["lora_b"][p] = lw["lora_b"][p] * 40
    return cfg, synth.to_f64(wts)


def _check_one_step(cfg, w, prompt, K, inv_t, n_passes=1, fixed=None, kappa=1.0):
    seq = spec.Sequence(cfg, prompt, capacity=len(prompt) + 2 * K + 4)
    spec.prefill(cfg, w, seq)
    dist = _enumerate_step(cfg, w, seq, K, inv_t, n_passes, fixed, kappa)
    assert abs(sum(dist.values()) - 1) == 0
    for c in dist:
        assert 2 <= len(c) <= K + 1          # tokens per step within [2, K+1]
    # continue each outcome with exact AR sampling up to K+1 tokens
    m = K + 1
    ar_cache = {}

    def ar(prefix):
        if prefix not in ar_cache:
            ar_cache[prefix] = _ar_probs(cfg, w, prefix, inv_t)
        return ar_cache[prefix]

    got = {}
    for c, pc in dist.items():
        frontier = [(tuple(c), float(pc))]
        while frontier:
            s, ps = frontier.pop()
            if len(s) >= m:
                got[s[:m]] = got.get(s[:m], 0.0) + ps
                continue
            probs = ar(tuple(prompt) + s)
            for v in range(cfg["vocab"]):
                frontier.append((s + (v,), ps * probs[v]))
    worst = 0.0
    for s, pg in got.items():
        pref = tuple(prompt)
        pe = 1.0
        for t in s:
            pe *= ar(pref)[t]
            pref = pref + (t,)
        worst = max(worst, abs(pg - pe))
    assert worst < 1e-6, worst
    return dist


@pytest.mark.parametrize("K", [1, 2, 3])
def test_exact_enumeration_one_step_lossless(toy, K):
    cfg, w = toy
    prompt = [1, 5, 2, 6, 0]
    dist = _check_one_step(cfg, w, prompt, K, 1.0)
    if K >= 2:
        # some rejections happen, so the check covers the residual branch
        assert any(len(c) < K + 1 for c in dist)


@pytest.mark.parametrize("K", [2, 3])
def test_exact_enumeration_uniform_prior(toy, K):
    """Uniform-state prior: the block's noise tokens are uniform Philox draws
    instead of the mask id (paperglide reader, "Lossless Psi-Spec decoding for
    USDMs"); the committed prefix is still exactly p_AR."""
    cfg, w = toy
    cfg = dict(cfg, noise_prior=1)
    noise = [noise_id(7, j, 0, 0, cfg["vocab"]) for j in range(1, K)]
    assert any(t != cfg["mask_id"] for t in noise)
    _check_one_step(cfg, w, [1, 5, 2, 6, 0], K, 1.0)


@pytest.mark.parametrize("fixed", [{(4, 0): 0, (4, 1): 5}, {(4, 0): 6, (4, 1): 6},
                                   {(4, 0): 2, (4, 1): 7, (5, 0): 1, (5, 1): 3}])
def test_exact_enumeration_multi_pass_draft(toy, fixed):
    """Several draft passes, each feeding its samples back into the block.
    Conditional on any outcome of the intermediate passes the final pass is an
    ordinary draft, so the committed prefix must be exactly p_AR for every such
    outcome (enumerated exactly over the final pass and the accept draws)."""
    cfg, w = toy
    n_passes = 1 + max(slot for slot, _ in fixed) - 3
    _check_one_step(cfg, w, [3, 1, 4], 2, 1.0, n_passes, fixed)


@pytest.mark.parametrize("kappa", [0.0, 0.5, 1.0])
@pytest.mark.parametrize("prior", [0, 1])
def test_exact_enumeration_corrector_strength(toy, kappa, prior):
    """Multi-pass drafting with a correction strength kappa between passes
    (each drafted row keeps its sample with probability kappa, else returns
    to the prior; paperglide reader, "Supplementary Details", Psi-samplers):
    the keep decisions are enumerated with their exact probabilities, the
    intermediate samples held fixed; the committed prefix is exactly p_AR for
    kappa 0, 1/2 and 1 and both priors."""
    cfg, w = toy
    cfg = dict(cfg, noise_prior=prior)
    fixed = {(4, 0): 2, (4, 1): 5, (5, 0): 1, (5, 1): 3}
    _check_one_step(cfg, w, [3, 1, 4], 2, 1.0, 3, fixed, kappa)


def test_corrector_limits_and_keep_rate(toy):
    """kappa = 1 is the plain multi-pass draft (every sample kept); kappa = 0
    with the mask prior hands the last pass the all-mask block, so its logits
    equal a one-pass draft's bit for bit; the keep rate is kappa."""
    cfg, w = toy
    seq = spec.Sequence(cfg, [3, 1, 4, 1, 5], capacity=20)
    spec.prefill(cfg, w, seq)
    z1 = spec.draft_logits(cfg, w, seq.copy(), 3, draws=spec.PhiloxDraws(0, 0, 0))
    z_k1, _, _ = spec.draft_passes(cfg, w, seq.copy(), 3, 3, 1.0, spec.PhiloxDraws(0, 0, 0), 1.0)
    block = None
    for i in range(3):        # the corrector-free chain, written out
        z = spec.draft_logits(cfg, w, seq.copy(), 3, block=block)
        d = spec.draft_sample(z.astype(np.float32), 1.0, spec.PhiloxDraws(0, 0, 0),
                              SLOT_DRAFT if i == 2 else SLOT_PASS + i)
        block = d[:2]
    assert np.array_equal(z_k1, z)
    z_k0, _, _ = spec.draft_passes(cfg, w, seq.copy(), 3, 3, 1.0, spec.PhiloxDraws(0, 0, 0), 0.0)
    assert np.array_equal(z_k0, z1)
    thr = spec.keep_threshold(0.3)
    assert thr == round(0.3 * TWO24) and spec.keep_threshold(1.0) == TWO24
    draws = [spec.PhiloxDraws(9, b, 0).keep(i, j, thr) for b in range(400) for i in range(3)
             for j in range(1, 17)]
    n, k = len(draws), sum(draws)
    assert abs(k / n - 0.3) < 4 * (0.3 * 0.7 / n) ** 0.5
    assert draws[0] == (uniform24(9, SLOT_KEEP, 1, 0, 0) < thr)


def test_multi_pass_changes_the_draft(toy):
    """A second pass conditions the draft on the first pass's tokens: its q
    differs from the one-pass q (otherwise the extra passes would be void)."""
    cfg, w = toy
    seq = spec.Sequence(cfg, [3, 1, 4, 1, 5], capacity=20)
    spec.prefill(cfg, w, seq)
    draws = spec.PhiloxDraws(0, 0, 0)
    z1 = spec.draft_logits(cfg, w, seq, 3, draws=draws)
    z2, _, _ = spec.draft_passes(cfg, w, seq, 3, 2, 1.0, draws)
    assert np.array_equal(z1[0], z2[0])             # row 0 is the AR row in every pass
    assert np.abs(z1[1:] - z2[1:]).max() > 1e-6


def test_exact_enumeration_temperature(toy):
    cfg, w = toy
    _check_one_step(cfg, w, [4, 4, 1], 2, np.float32(1.0 / 0.7))


def test_exact_enumeration_two_steps_k1(toy):
    cfg, w = toy
    prompt = [2, 3, 0]
    seq = spec.Sequence(cfg, prompt, capacity=16)
    spec.prefill(cfg, w, seq)
    first = _enumerate_step(cfg, w, seq, 1, 1.0)
    got = {}
    for c1, p1 in first.items():
        # replay the first step along path c1 so that its cache writes and
        # commit are exactly the ones the step makes
        s2 = seq.copy()
        r = spec.step(cfg, w, s2, 1, 1.0, _FixedDraws(c1))
        assert tuple(r["committed"]) == c1
        for c2, p2 in _enumerate_step(cfg, w, s2, 1, 1.0).items():
            key = c1 + c2
            got[key] = got.get(key, 0) + float(p1 * p2)
    worst = 0.0
    for s, pg in got.items():
        pref, pe = tuple(prompt), 1.0
        for t in s:
            pe *= _ar_probs(cfg, w, pref, 1.0)[t]
            pref += (t,)
        worst = max(worst, abs(pg - pe))
    assert abs(sum(got.values()) - 1) < 1e-12 and worst < 1e-6


class _FixedDraws:
    """Forces the decisions that produce a given committed tuple (K = 1)."""

    def __init__(self, committed):
        self.c = committed

    def categorical(self, slot, j, weights):
        return self.c[0] if slot == SLOT_DRAFT else self.c[1]

    def accept(self, *a):
        raise AssertionError("K = 1 has no accept test")


# ---------------- prefix-independent rows: closed forms and chi-square ----------------

def _indep_rows(V=512, K=8, seed=0, sigma=1.0, noise=0.6):
    zq, zp = synth.sampler_logits(1, K, V, seed, sigma_p=sigma, sigma_noise=noise)
    return zq[0], zp[0]


def test_acceptance_rate_is_one_minus_tv():
    zq, zp = _indep_rows()
    K = zq.shape[0]
    for i in range(2, K + 1):
        wq, sq = cn.row_weights(zq[i - 1], 1.0)
        wp, sp = cn.row_weights(zp[i - 2], 1.0)
        # actual draft law (exact counts over U) times exact accept probability
        cum = np.cumsum(wq)
        starts = [0] + [((int(c) << 24) + sq - 1) // sq for c in cum]   # ceil(C * 2^24 / S)
        acc = Fraction(0)
        for d in range(len(wq)):
            cnt = min(starts[d + 1], TWO24) - min(starts[d], TWO24)
            if cnt == 0:
                continue
            thr = _lowest_u(lambda u: not cn.accept(int(wq[d]), sq, int(wp[d]), sp, u))
            acc += Fraction(cnt, TWO24) * Fraction(thr, TWO24)
        beta = sum(min(Fraction(int(a), sp), Fraction(int(b), sq)) for a, b in zip(wp, wq))
        assert abs(float(acc - beta)) < 600 * 2.0 ** -24     # V entries, each off by < 2^-24


def _vectorised_replay(zq, zp, n, seed, inv_t=1.0):
    """The oracle's sampler on prefix-independent rows, vectorised over n
    sequences b = 0..n-1 at step 0.  Returns (drafts [n,K], a [n], extra [n])."""
    K, V = zq.shape
    q = [cn.row_weights(zq[j], inv_t) for j in range(K)]
    p = {1: q[0]}
    for i in range(2, K + 2):
        p[i] = cn.row_weights(zp[i - 2], inv_t)
    b = np.arange(n, dtype=np.uint64)
    drafts = np.zeros((n, K), dtype=np.int64)
    for j in range(K):
        w, s = q[j]
        u = uniform24_np(seed, SLOT_DRAFT, j, b, 0).astype(object)
        t = np.array([(int(x) * s) >> 24 for x in u], dtype=np.uint64)
        drafts[:, j] = np.searchsorted(np.cumsum(w), t, side="right")
    a = np.full(n, K)
    alive = np.ones(n, dtype=bool)
    for i in range(2, K + 1):
        wq, sq = q[i - 1]
        wp, sp = p[i]
        d = drafts[:, i - 1]
        u = uniform24_np(seed, SLOT_ACCEPT, i - 1, b, 0)
        lhs = u.astype(object) * wq[d].astype(object) * sp
        rhs = wp[d].astype(object) * sq * TWO24
        rej = alive & ~(lhs < rhs).astype(bool)
        a[rej] = i - 1
        alive &= ~rej
    extra = np.zeros(n, dtype=np.int64)
    for av in range(1, K + 1):
        sel = np.nonzero(a == av)[0]
        if sel.size == 0:
            continue
        if av < K:
            wp, sp = p[av + 1]
            wq, sq = q[av]
            r = cn.residual_weights(wp, sp, wq, sq)
            if sum(r) == 0:
                r = [int(x) for x in wp]
        else:
            r = [int(x) for x in p[K + 1][0]]
        cum = np.cumsum(np.array(r, dtype=object))
        tot = int(cum[-1])
        u = uniform24_np(seed, SLOT_EXTRA, av, b[sel], 0)
        for k, uu in zip(sel, u):
            t = (int(uu) * tot) >> 24
            extra[k] = int(np.searchsorted(cum, t, side="right"))
    return drafts, a, extra


def test_vectorised_replay_matches_oracle_step_logic():
    zq, zp = _indep_rows(V=256, K=6, seed=4)
    drafts, a, extra = _vectorised_replay(zq, zp, 1500, seed=9)
    for bb in range(1500):
        dr = spec.draft_sample(zq, 1.0, spec.PhiloxDraws(9, bb, 0))
        assert dr == list(drafts[bb])
        aa, comm, ex = spec.spec_accept(zq, zp, dr, 1.0, spec.PhiloxDraws(9, bb, 0))
        assert (aa, ex) == (a[bb], extra[bb])


def test_chi_square_first_token_law_1e6_samples():
    """Position j's committed token, given that the step reaches position j
    without an earlier rejection, follows p_j: the token there is either the
    kept draft or the residual/bonus draw."""
    zq, zp = _indep_rows(V=512, K=8, seed=1)
    n = 1_000_000
    drafts, a, extra = _vectorised_replay(zq, zp, n, seed=0)
    K, V = zq.shape
    for j in (2, 5, 8):
        reached = a >= j - 1                 # positions 1..j-1 kept
        tok = np.where(a[reached] >= j, drafts[reached, j - 1], extra[reached])
        wp, sp = cn.row_weights(zp[j - 2], 1.0)
        exp = wp.astype(np.float64) / sp * tok.size
        obs = np.bincount(tok, minlength=V).astype(np.float64)
        keep = exp > 5
        stat, pval = scipy.stats.chisquare(obs[keep], exp[keep] * obs[keep].sum() / exp[keep].sum())
        assert pval > 0.01, (j, pval)


# ---------------- the tiny model: the second committed token over 10^6 steps ----------------

def _tiny_second_token_replay(cfg, w, prompt, n, seed, inv_t=1.0):
    """One K = 2 step of the tiny model from ``prompt``, replayed for sequences
    b = 0..n-1 at step 0 with the oracle's sampler arithmetic, vectorised.
    The draft rows q_1, q_2 do not depend on the drafted tokens; the verify row
    p_2 depends on d_1 only (causal), so it is computed once per value of d_1.
    Returns (second committed token [n], q_1 weights, {d_1: p_2 weights})."""
    seq = spec.Sequence(cfg, prompt, capacity=len(prompt) + 8)
    spec.prefill(cfg, w, seq)
    zq = spec.draft_logits(cfg, w, seq, 2).astype(np.float32)
    (wq1, sq1), (wq2, sq2) = cn.row_weights(zq[0], inv_t), cn.row_weights(zq[1], inv_t)
    b = np.arange(n, dtype=np.uint64)

    def draw(w_, s_, u):
        t = (u.astype(np.uint64) * np.uint64(s_)) >> np.uint64(24)     # U*S < 2^64
        return np.searchsorted(np.cumsum(w_, dtype=np.uint64), t, side="right")

    d1 = draw(wq1, sq1, uniform24_np(seed, SLOT_DRAFT, 0, b, 0))
    d2 = draw(wq2, sq2, uniform24_np(seed, SLOT_DRAFT, 1, b, 0))
    u_acc = uniform24_np(seed, SLOT_ACCEPT, 1, b, 0)
    u_ext = uniform24_np(seed, SLOT_EXTRA, 1, b, 0)
    p2 = {}
    second = np.empty(n, dtype=np.int64)
    for x1 in np.unique(d1):
        s2 = seq.copy()
        p2[int(x1)] = cn.row_weights(spec.verify_logits(cfg, w, s2, [int(x1), 0])[0]
                                     .astype(np.float32), inv_t)
        wp, sp = p2[int(x1)]
        sel = np.nonzero(d1 == x1)[0]
        dd = d2[sel]
        lhs = u_acc[sel].astype(object) * wq2[dd].astype(object) * sp
        rhs = wp[dd].astype(object) * sq2 * TWO24
        keep = (lhs < rhs).astype(bool)
        second[sel[keep]] = dd[keep]
        rej = sel[~keep]
        if rej.size:
            r = cn.residual_weights(wp, sp, wq2, sq2)
            r = [int(x) for x in wp] if sum(r) == 0 else r
            cum = np.cumsum(np.array(r, dtype=object))
            tot = int(cum[-1])
            for k, uu in zip(rej, u_ext[rej]):
                second[k] = int(np.searchsorted(cum, (int(uu) * tot) >> 24, side="right"))
    return second, d1, (wq1, sq1), p2


@pytest.fixture(scope="module")
def tiny_second():
    cfg = synth.TINY
    w = synth.to_f64(synth.make_weights(cfg, 0))
    prompt = list(synth.prompt_ids(cfg, 32, 1))
    return cfg, w, prompt


def test_tiny_second_token_replay_matches_oracle_steps(tiny_second):
    """The vectorised replay takes the oracle step's own decisions, draw by draw."""
    cfg, w, prompt = tiny_second
    n = 300
    second, d1, _, _ = _tiny_second_token_replay(cfg, w, prompt, n, seed=5)
    seq0 = spec.Sequence(cfg, prompt, capacity=len(prompt) + 8)
    spec.prefill(cfg, w, seq0)
    for b in range(n):
        r = spec.step(cfg, w, seq0.copy(), 2, 1.0, spec.PhiloxDraws(5, b, 0))
        assert r["committed"][0] == d1[b]
        assert r["committed"][1] == second[b], b


def test_tiny_model_second_token_chi_square_1e6(tiny_second):
    """The second token a step commits (the kept draft d_2, else the residual
    draw) follows the AR marginal sum_x1 p(x1) p(x2 | x1) of the tiny model
    (K = 2, 10^6 seeded steps, chi-square at p > 0.01)."""
    cfg, w, prompt = tiny_second
    n = 1_000_000
    second, d1, (wq1, sq1), p2 = _tiny_second_token_replay(cfg, w, prompt, n, seed=0)
    V = cfg["vocab"]
    # the expected law uses every x1 with q_1(x1) > 0, not only the ones drawn
    seq = spec.Sequence(cfg, prompt, capacity=len(prompt) + 8)
    spec.prefill(cfg, w, seq)
    spec.draft_logits(cfg, w, seq, 2)
    exp = np.zeros(V)
    for x1 in np.nonzero(wq1)[0]:
        if int(x1) not in p2:
            p2[int(x1)] = cn.row_weights(spec.verify_logits(cfg, w, seq.copy(), [int(x1), 0])[0]
                                         .astype(np.float32), 1.0)
        wp, sp = p2[int(x1)]
        exp += (int(wq1[x1]) / sq1) * (wp.astype(np.float64) / sp)
    assert abs(exp.sum() - 1) < 1e-9
    obs = np.bincount(second, minlength=V).astype(np.float64)
    keep = exp * n > 5
    stat, pval = scipy.stats.chisquare(obs[keep], exp[keep] * n * obs[keep].sum() / (exp[keep] * n).sum())
    assert pval > 0.01, pval
