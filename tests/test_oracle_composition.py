"""Pins of the oracle's layer composition against an independent decoder.

The oracle's primitives (RMSNorm, SiLU, attention, RoPE) are pinned against
torch elsewhere; this module pins how they are put together: pre-norm residual
blocks, silu(gate) * up (not silu(up) * gate), the final norm before the LM
head, the norm gains each block uses, q head h reading kv head h // (Hq/Hkv),
and the gated LoRA term on every projection.  The reference here is a decoder
written from ``torch.nn.functional`` calls (``rms_norm``, ``linear``, ``silu``,
``scaled_dot_product_attention``) and a complex-number rotary embedding, run
uncached over the whole block with an explicit mask, in fp64 on the CPU.

Each pin is shown to bite: the oracle module's source is re-executed with one
planted mistake at a time (gate and up swapped, post-norm blocks, no final norm,
interleaved head packing, a dropped residual, the wrong norm gain, the LoRA gate
inverted), and every planted variant must disagree with the reference.
"""
import inspect
import types

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import synth
from oracle import model as om


def _torch_decoder(cfg, wts, ids, pos, gate, key_limit):
    """Logits [R, V] of one uncached pass; row r attends to rows j <= key_limit[r]
    (rows are at positions pos, keys are the rows themselves)."""
    t = lambda a: torch.from_numpy(np.asarray(a, dtype=np.float64))
    R = len(ids)
    D, Hq, Hkv, hd = cfg["d_model"], cfg["n_q_heads"], cfg["n_kv_heads"], cfg["head_dim"]
    s = cfg["lora_alpha"] / cfg["lora_rank"]
    g = t(gate)[:, None]
    h = t(wts["embed"])[torch.as_tensor(ids, dtype=torch.long)]
    half = hd // 2
    freq = cfg["rope_theta"] ** (-torch.arange(half, dtype=torch.float64) * 2.0 / hd)
    rot = torch.polar(torch.ones(R, half, dtype=torch.float64), t(pos)[:, None] * freq)[:, None]

    def rotary(x):                      # [R, H, hd]: channel pairs (i, i + hd/2)
        z = torch.complex(x[..., :half], x[..., half:]) * rot
        return torch.cat([z.real, z.imag], dim=-1)

    allowed = torch.arange(R)[None, :] <= torch.as_tensor(key_limit)[:, None]   # [R, R]
    for lw in wts["layers"]:
        def lin(x, p):
            y = F.linear(x, t(lw[p]))
            if p in lw["lora_a"]:
                y = y + g * s * F.linear(F.linear(x, t(lw["lora_a"][p])), t(lw["lora_b"][p]))
            return y

        x = F.rms_norm(h, (D,), t(lw["attn_norm"]), cfg["rms_eps"])
        q = rotary(lin(x, "q").view(R, Hq, hd)).transpose(0, 1)             # [Hq, R, hd]
        k = rotary(lin(x, "k").view(R, Hkv, hd)).transpose(0, 1)
        v = lin(x, "v").view(R, Hkv, hd).transpose(0, 1)
        k = k.repeat_interleave(Hq // Hkv, dim=0)                           # q head h -> h // G
        v = v.repeat_interleave(Hq // Hkv, dim=0)
        o = F.scaled_dot_product_attention(q, k, v, attn_mask=allowed)
        h = h + lin(o.transpose(0, 1).reshape(R, Hq * hd), "o")
        x = F.rms_norm(h, (D,), t(lw["mlp_norm"]), cfg["rms_eps"])
        h = h + lin(F.silu(lin(x, "gate")) * lin(x, "up"), "down")
    return F.linear(F.rms_norm(h, (D,), t(wts["final_norm"]), cfg["rms_eps"]),
                    t(wts["lm_head"])).numpy()


def _weights(cfg, seed):
    """fp64 weights with distinct, non-unit norm gains (a swapped gain must show)."""
    w = synth.to_f64(synth.make_weights(cfg, seed))
    rng = np.random.default_rng([seed, 99])
    D = cfg["d_model"]
    w["final_norm"] = 1.0 + 0.3 * rng.standard_normal(D)
    for lw in w["layers"]:
        lw["attn_norm"] = 1.0 + 0.3 * rng.standard_normal(D)
        lw["mlp_norm"] = 1.0 + 0.3 * rng.standard_normal(D)
        # LoRA B large enough that the LoRA term moves the logits visibly
        for p in lw["lora_b"]:
            lw["lora_b"][p] = lw["lora_b"][p] * 10
    return w


def _block(cfg, R):
    """A draft-shaped block of R rows at positions 0..R-1: row 0 gate 0 and
    causal, the other rows gated and seeing the whole block; plus a causal,
    ungated variant."""
    ids = synth.prompt_ids(cfg, R, 31)
    pos = np.arange(R)
    draft = (ids, pos, np.array([0.0] + [1.0] * (R - 1)), np.array([0] + [R - 1] * (R - 1)))
    causal = (ids, pos, np.zeros(R), pos)
    return draft, causal


def _oracle(mod, cfg, w, ids, pos, gate, lim):
    cache = mod.KVCache(cfg, len(ids))
    return mod.forward(cfg, w, cache, ids, pos, gate, lim)


SHAPES = {"tiny": synth.TINY, "gqa": synth.SMALL_GQA}


@pytest.fixture(scope="module", params=sorted(SHAPES))
def case(request):
    cfg = SHAPES[request.param]
    w = _weights(cfg, 4)
    blocks = _block(cfg, 9)
    refs = [_torch_decoder(cfg, w, *b) for b in blocks]
    return request.param, cfg, w, blocks, refs


def test_oracle_forward_equals_torch_decoder(case):
    _, cfg, w, blocks, refs = case
    for b, ref in zip(blocks, refs):
        got = _oracle(om, cfg, w, *b)
        np.testing.assert_allclose(got, ref, rtol=1e-9, atol=1e-10)
    # the pin is sensitive: the LoRA term and the gains matter at this scale
    assert np.abs(refs[0] - refs[1]).max() > 1e-3


# (name, source text in oracle/model.py, replacement); the first two plant
# post-norm blocks together
MUTATIONS = {
    "gate_up_swapped": [('silu(lin(x, "gate")) * lin(x, "up")',
                         'silu(lin(x, "up")) * lin(x, "gate")')],
    "post_norm": [('x = rd(rms_norm(h, lw["attn_norm"], eps))', 'x = rd(h)'),
                  ('h = h + lin(o, "o")', 'h = rms_norm(h + lin(o, "o"), lw["attn_norm"], eps)'),
                  ('x = rd(rms_norm(h, lw["mlp_norm"], eps))', 'x = rd(h)'),
                  ('h = h + lin(rd(silu(lin(x, "gate")) * lin(x, "up")), "down")',
                   'h = rms_norm(h + lin(rd(silu(lin(x, "gate")) * lin(x, "up")), "down"), '
                   'lw["mlp_norm"], eps)')],
    "no_final_norm": [('x = rd(rms_norm(h, wts["final_norm"], eps))', 'x = rd(h)')],
    "interleaved_heads": [("for h in range(g * group, (g + 1) * group):",
                           "for h in range(g, Hq, n_kv_heads):")],
    "mlp_residual_dropped": [('h = h + lin(rd(silu(', 'h = 0 * h + lin(rd(silu(')],
    "attn_norm_gain_swapped": [('x = rd(rms_norm(h, lw["attn_norm"], eps))',
                                'x = rd(rms_norm(h, lw["mlp_norm"], eps))')],
    "lora_gate_inverted": [("t = (gate[:, None] * scale) * (x @ a.T)",
                            "t = ((1 - gate[:, None]) * scale) * (x @ a.T)")],
}


def _mutant(edits):
    src = inspect.getsource(om)
    for old, new in edits:
        assert src.count(old) == 1, "mutation anchor not unique: %r" % old
        src = src.replace(old, new)
    mod = types.ModuleType("oracle_model_mutant")
    exec(compile(src, "oracle/model.py (mutated)", "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_planted_composition_mistake_is_caught(case, name):
    shape, cfg, w, blocks, refs = case
    mod = _mutant(MUTATIONS[name])
    worst = max(np.abs(_oracle(mod, cfg, w, *b) - ref).max() for b, ref in zip(blocks, refs))
    if name == "interleaved_heads" and cfg["n_q_heads"] == cfg["n_kv_heads"]:
        assert worst < 1e-9          # without grouping both packings are the same
        return
    assert worst > 1e-4, (shape, name, worst)
