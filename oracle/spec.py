"""One Psi-Spec decode step for one sequence (oracle, test infrastructure).

Follows the step the pages lay out (paperglide reader, "The Psi-Speculative
Sampler"; picx.dev summary, "Psi-Speculative Sampler"; paperglide reader,
"Sampler Extensions"):

1. draft: the block is the last committed token (the anchor) followed by
   mask tokens; one pass with AR + LoRA weights gives per-position draft
   distributions q_1..q_K, and each drafted token is sampled independently from
   its own marginal.  Position 1 is computed with the AR weights alone (gate 0),
   so q_1 is the AR next-token distribution and d_1 is always kept;
2. verify: one pass with the AR weights alone over d_1..d_K gives p_2..p_{K+1};
3. accept: d_i (i >= 2) is kept with probability min(1, p_i(d_i)/q_i(d_i)),
   stopping at the first rejection; a counts the kept drafts;
4. extra token: if a < K, one token from normalise(max(0, p_{a+1} - q_{a+1}));
   if a = K, a bonus token from p_{K+1};
5. commit: the kept drafts and the extra token join the sequence; the cache
   keeps the anchor and the kept drafts and the rest is rolled back.

Readings where the pages are silent (each listed in the design notes):
* block = [anchor, mask x (K-1)] at positions n-1 .. n+K-2, so K drafts per
  step and 2 <= tokens per step <= K+1 (the pages' TPF bound counts two
  forward passes per step);
* the prior of the noise positions is the mask token (id vocab-1);
* draft attention: row 0 attends causally (keys <= n-1); mask rows attend to
  every key up to the end of the block (keys <= n+K-2);
* verify attention is causal: row j (position n+j) sees keys <= n+j;
* the anchor's K/V come from the draft pass (its row 0 is the AR row); verify
  runs K rows;
* the same temperature T applies to p and q;
* a forced accept length (throughput tests) overrides a after the natural
  tests ran; a forced a = 0 draws the extra token from p_1 = q_1 (the residual
  of identical rows is empty).

Random draws come from a ``draws`` object with ``categorical(slot, j, W)`` and
``accept(slot, j, Wq_d, Sq, Wp_d, Sp)``; ``PhiloxDraws`` feeds them with the
counter generator, tests may feed them otherwise (exact enumeration).
"""
import numpy as np

from . import canonical as cn
from .model import KVCache, forward
from .philox import (MAX_PASSES, SLOT_ACCEPT, SLOT_DRAFT, SLOT_EXTRA, SLOT_KEEP, SLOT_PASS,
                     SLOT_RENOISE, noise_id, token_id, uniform24)

TWO24 = 1 << 24


class PhiloxDraws:
    """Draws for sequence ``b`` at step ``step`` from Philox4x64-10."""

    def __init__(self, seed, b, step):
        self.seed, self.b, self.step = int(seed), int(b), int(step)

    def u(self, slot, j):
        return uniform24(self.seed, slot, j, self.b, self.step)

    def noise(self, j, vocab):
        return noise_id(self.seed, j, self.b, self.step, vocab)

    def keep(self, i, j, keep_q24):
        """Corrector after draft pass i: row j keeps its token iff U < keep_q24."""
        return uniform24(self.seed, SLOT_KEEP + i, j, self.b, self.step) < int(keep_q24)

    def renoise(self, i, j, vocab):
        """Corrector after draft pass i: a fresh uniform token for row j."""
        return token_id(self.seed, SLOT_RENOISE + i, j, self.b, self.step, vocab)

    def categorical(self, slot, j, weights):
        return cn.categorical(weights, self.u(slot, j))

    def accept(self, slot, j, wq_d, sq, wp_d, sp):
        return cn.accept(wq_d, sq, wp_d, sp, self.u(slot, j))


class Sequence:
    """Decode state of one sequence: tokens t[0..n-1], cache holding 0..n-2."""

    def __init__(self, cfg, tokens, capacity):
        self.cfg = cfg
        self.tokens = [int(t) for t in tokens]
        self.cache = KVCache(cfg, capacity)
        self.kv_len = 0
        self.step = 0

    def copy(self):
        s = Sequence.__new__(Sequence)
        s.cfg = self.cfg
        s.tokens = list(self.tokens)
        s.cache = self.cache.copy()
        s.kv_len = self.kv_len
        s.step = self.step
        return s


def prefill(cfg, wts, seq):
    """Cache every token but the last (which becomes the anchor)."""
    n = len(seq.tokens)
    rows = seq.tokens[: n - 1]
    pos = np.arange(n - 1)
    forward(cfg, wts, seq.cache, rows, pos, np.zeros(n - 1), pos)
    seq.kv_len = n - 1


def draft_logits(cfg, wts, seq, K, act_round=None, draws=None, block=None, taps=None):
    """Draft pass: rows [anchor, noise x (K-1)], gate (0, 1, ..., 1). fp64 [K, V].

    The noisy block is the anchor followed by K-1 tokens from the diffusion
    prior (paperglide reader, "The Psi-Speculative Sampler"): the mask token
    for a masked model, or uniform tokens for a uniform-state model
    ("Supplementary Details"), chosen by cfg["noise_prior"] (0 / 1); uniform
    tokens come from ``draws.noise(j, V)``.  A later pass of a multi-pass draft
    passes ``block``: rows 1..K-1 then hold block[0..K-2]."""
    n0 = seq.kv_len                       # position of the anchor
    if block is not None:
        noise = [int(t) for t in block[: K - 1]]
    elif cfg.get("noise_prior", 0) == 1:
        noise = [draws.noise(j, cfg["vocab"]) for j in range(1, K)]
    else:
        noise = [cfg["mask_id"]] * (K - 1)
    rows = [seq.tokens[-1]] + noise
    pos = n0 + np.arange(K)
    gate = np.array([0.0] + [1.0] * (K - 1))
    lim = np.array([n0] + [n0 + K - 1] * (K - 1))
    return forward(cfg, wts, seq.cache, rows, pos, gate, lim, act_round=act_round, taps=taps)


def draft_sample(zq32, inv_temp, draws, slot=SLOT_DRAFT):
    """d_{j+1} ~ q_{j+1} for each draft row j (fp32 logits [K, V])."""
    return [draws.categorical(slot, j, cn.row_weights(zq32[j], inv_temp)[0])
            for j in range(zq32.shape[0])]


def keep_threshold(kappa):
    """Correction strength kappa in [0, 1] as the 24-bit threshold of the keep
    test U < round(kappa * 2^24) (kappa = 1 always keeps, 0 always remasks)."""
    k = float(kappa)
    if not 0.0 <= k <= 1.0:
        raise ValueError("kappa must lie in [0, 1]")
    return int(round(k * TWO24))


def corrected_block(cfg, drafts, pass_i, keep_q24, draws):
    """The block the draft pass after pass ``pass_i`` reads, from that pass's
    samples d_1..d_K (paperglide reader, "Supplementary Details": a
    Psi-sampler is a predictor-corrector sampler whose correction strength
    kappa_t in [0, 1] interpolates between the reverse posterior, kappa_t = 1
    being ancestral sampling, and the forward noising process, which remasks a
    masked model's tokens and re-draws a uniform-state model's).  Row j >= 1
    keeps d_j with probability kappa = keep_q24 / 2^24 (U < keep_q24, Philox
    slot SLOT_KEEP + pass_i); otherwise it returns to the prior: the mask token,
    or a fresh uniform token (slot SLOT_RENOISE + pass_i)."""
    K = len(drafts)
    out = []
    for j in range(1, K):
        if int(keep_q24) >= TWO24 or draws.keep(pass_i, j, keep_q24):
            out.append(int(drafts[j - 1]))
        elif cfg.get("noise_prior", 0) == 1:
            out.append(draws.renoise(pass_i, j, cfg["vocab"]))
        else:
            out.append(cfg["mask_id"])
    return out


def draft_passes(cfg, wts, seq, K, n_passes, inv_temp, draws, kappa=1.0):
    """Multi-pass draft (paperglide reader, "Supplementary Details": a
    Psi-sampler refines the block over several denoising steps, and sample
    quality grows with the number of steps).  Pass 0 reads the prior's noisy
    block; pass i > 0 reads the block the corrector makes from pass i-1's
    samples (``corrected_block``, correction strength ``kappa``: one value, or
    one per transition).  Intermediate samples use Philox slot SLOT_PASS + i;
    the last pass samples the drafts with SLOT_DRAFT.  Returns (zq fp64, zq
    fp32, drafts) of the last pass: only those enter the accept test, and
    conditional on everything drawn before it the last pass is an ordinary
    draft, so any number of passes and any kappa keep the decode lossless."""
    if not 1 <= n_passes <= MAX_PASSES:
        raise ValueError("1 <= n_passes <= %d" % MAX_PASSES)
    kap = list(kappa) if isinstance(kappa, (list, tuple)) else [kappa] * max(0, n_passes - 1)
    block = None
    for i in range(n_passes):
        zq = draft_logits(cfg, wts, seq, K, draws=draws, block=block)
        zq32 = zq.astype(np.float32)
        last = i == n_passes - 1
        d = draft_sample(zq32, inv_temp, draws, SLOT_DRAFT if last else SLOT_PASS + i)
        block = d if last else corrected_block(cfg, d, i, keep_threshold(kap[i]), draws)
    return zq, zq32, block


def verify_logits(cfg, wts, seq, rows, pos_offset=1, act_round=None, taps=None):
    """Verify pass with AR weights, causal: row j at position kv_len+pos_offset+j."""
    K = len(rows)
    pos = seq.kv_len + pos_offset + np.arange(K)
    return forward(cfg, wts, seq.cache, rows, pos, np.zeros(K), pos, act_round=act_round,
                   taps=taps)


def spec_accept(zq32, zp32, drafts, inv_temp, draws, forced=None):
    """Accept test, first rejection, residual or bonus token.

    zq32: draft logits [K, V] (row j is q_{j+1}); zp32: verify logits [K, V]
    (row j is p_{j+2}).  Returns (a, committed list, extra token).
    """
    K = len(drafts)
    q = [cn.row_weights(zq32[j], inv_temp) for j in range(K)]
    p_cache = {}

    def p_row(i):                       # p_i, 1-based; p_1 is the AR draft row
        if i not in p_cache:
            z = zq32[0] if i == 1 else zp32[i - 2]
            p_cache[i] = q[0] if i == 1 else cn.row_weights(z, inv_temp)
        return p_cache[i]

    a = K
    for i in range(2, K + 1):
        wq, sq = q[i - 1]
        wp, sp = p_row(i)
        d = int(drafts[i - 1])
        if not draws.accept(SLOT_ACCEPT, i - 1, int(wq[d]), sq, int(wp[d]), sp):
            a = i - 1
            break
    if forced is not None:
        a = int(forced)
    if a < K:
        wp, sp = p_row(a + 1)
        wq, sq = q[a]
        res = cn.residual_weights(wp, sp, wq, sq)
        if sum(res) == 0:
            extra = draws.categorical(SLOT_EXTRA, a, wp)
        else:
            extra = draws.categorical(SLOT_EXTRA, a, res)
    else:
        wp, _ = p_row(K + 1)
        extra = draws.categorical(SLOT_EXTRA, K, wp)
    committed = [int(d) for d in drafts[:a]] + [int(extra)]
    return a, committed, int(extra)


def commit(seq, a, committed):
    """Keep the anchor and the a kept drafts in the cache; append the tokens."""
    seq.kv_len += 1 + int(a)
    seq.tokens.extend(int(t) for t in committed)
    seq.step += 1


def step(cfg, wts, seq, K, inv_temp, draws, forced=None, n_passes=1, kappa=1.0):
    """One full draft (n_passes passes, correction strength kappa between
    them) -> sample -> verify -> accept -> commit step.

    Returns a dict with the logits (fp64 and the fp32 copies the sampler saw),
    drafts, a, committed tokens and the extra token.
    """
    zq, zq32, drafts = draft_passes(cfg, wts, seq, K, n_passes, inv_temp, draws, kappa)
    zp = verify_logits(cfg, wts, seq, drafts)
    zp32 = zp.astype(np.float32)
    a, committed, extra = spec_accept(zq32, zp32, drafts, inv_temp, draws, forced)
    commit(seq, a, committed)
    return dict(zq=zq, zp=zp, zq32=zq32, zp32=zp32, drafts=drafts, a=a,
                committed=committed, extra=extra)


def generate(cfg, wts, prompt, K, n_new, inv_temp, seed, b=0):
    """Prefill the prompt, then run steps until n_new tokens, truncated."""
    seq = Sequence(cfg, prompt, capacity=len(prompt) + n_new + 2 * K + 2)
    prefill(cfg, wts, seq)
    trace = []
    while len(seq.tokens) - len(prompt) < n_new:
        trace.append(step(cfg, wts, seq, K, inv_temp, PhiloxDraws(seed, b, seq.step)))
    return seq.tokens[len(prompt): len(prompt) + n_new], trace, seq
