"""Structural pins of the fp64 model oracle (the pages print no logits).

* the LoRA linear equals the dense merged matmul x (W + s B A)^T;
* B = 0 reduces the LoRA linear and the whole draft pass to the AR weights;
* draft row 0 (gate off, causal) equals the AR next-token logits at the anchor;
* the cached block pass equals a full uncached causal recompute;
* attention, RMSNorm, SiLU match independent torch CPU routines and RoPE matches
  its complex-rotation form;
* the 8B shape's LoRA parameter count is the pages' 0.35B.
"""
import json
import os

import numpy as np
import pytest
import torch

import synth
from oracle import model as om
from oracle import spec

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


@pytest.fixture(scope="module")
def tiny():
    cfg = synth.TINY
    return cfg, synth.to_f64(synth.make_weights(cfg, 0))


def test_lora_linear_equals_dense_merge():
    rng = np.random.default_rng(0)
    x = rng.standard_normal((7, 48))
    w = rng.standard_normal((40, 48))
    a = rng.standard_normal((6, 48))
    b = rng.standard_normal((40, 6))
    gate = np.array([0, 1, 1, 0, 1, 1, 1], dtype=np.float64)
    s = 2.0
    y = om.lora_linear(x, w, a, b, s, gate)
    dense_on = x @ (w + s * b @ a).T
    dense_off = x @ w.T
    ref = np.where(gate[:, None] > 0, dense_on, dense_off)
    np.testing.assert_allclose(y, ref, rtol=1e-12, atol=1e-12)
    y0 = om.lora_linear(x, w, a, np.zeros_like(b), s, gate)
    np.testing.assert_array_equal(y0, x @ w.T)


def test_rmsnorm_silu_match_torch():
    rng = np.random.default_rng(1)
    h = rng.standard_normal((5, 64)) * 3
    g = rng.standard_normal(64)
    ref = torch.nn.functional.rms_norm(torch.from_numpy(h), (64,), torch.from_numpy(g), eps=1e-6)
    np.testing.assert_allclose(om.rms_norm(h, g, 1e-6), ref.numpy(), rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(om.silu(h), torch.nn.functional.silu(torch.from_numpy(h)).numpy(),
                               rtol=1e-12, atol=1e-12)


def test_rope_is_complex_rotation():
    rng = np.random.default_rng(2)
    x = rng.standard_normal((6, 3, 16))
    pos = np.array([0, 1, 5, 100, 9000, 32767])
    out = om.rope(x, pos, 10000.0)
    half = 8
    freq = 10000.0 ** (-np.arange(half) / half)
    zc = (x[..., :half] + 1j * x[..., half:]) * np.exp(1j * pos[:, None, None] * freq)
    np.testing.assert_allclose(out[..., :half], zc.real, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(out[..., half:], zc.imag, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(om.rope(x, np.zeros(6, dtype=int), 10000.0), x)


def test_attention_matches_torch_sdpa():
    rng = np.random.default_rng(3)
    R, Hq, Hkv, hd, cap = 5, 8, 2, 16, 23
    q = rng.standard_normal((R, Hq, hd))
    ck = rng.standard_normal((cap, Hkv, hd))
    cv = rng.standard_normal((cap, Hkv, hd))
    lim = np.array([0, 3, 22, 10, 10])
    out = om.attention(q, ck, cv, lim, Hkv)
    group = Hq // Hkv
    kk = torch.from_numpy(np.repeat(ck, group, axis=1)).permute(1, 0, 2)   # [Hq, cap, hd]
    vv = torch.from_numpy(np.repeat(cv, group, axis=1)).permute(1, 0, 2)
    qq = torch.from_numpy(q).permute(1, 0, 2)                              # [Hq, R, hd]
    mask = torch.from_numpy(np.arange(cap)[None, :] <= lim[:, None])       # [R, cap]
    ref = torch.nn.functional.scaled_dot_product_attention(qq, kk, vv, attn_mask=mask)
    np.testing.assert_allclose(out, ref.permute(1, 0, 2).numpy(), rtol=1e-10, atol=1e-12)


def test_draft_row0_is_ar_and_cached_verify_is_full_recompute(tiny):
    cfg, w = tiny
    prompt = synth.prompt_ids(cfg, 12, 5)
    seq = spec.Sequence(cfg, prompt, capacity=64)
    spec.prefill(cfg, w, seq)
    K = 4
    zq = spec.draft_logits(cfg, w, seq, K)
    full = om.full_causal_logits(cfg, w, list(prompt))
    np.testing.assert_allclose(zq[0], full[-1], rtol=1e-9, atol=1e-11)
    drafts = [3, 77, 400, 12]
    zp = spec.verify_logits(cfg, w, seq, drafts)
    full2 = om.full_causal_logits(cfg, w, list(prompt) + drafts)
    n = len(prompt)
    np.testing.assert_allclose(zp, full2[n: n + K], rtol=1e-9, atol=1e-11)
    # the LoRA term really changes the mask rows
    assert np.max(np.abs(zq[1] - full[-1])) > 1e-6


def test_zero_lora_b_draft_is_ar_weights(tiny):
    cfg, w = tiny
    w0 = synth.to_f64(synth.zero_lora_b(synth.make_weights(cfg, 0)))
    prompt = synth.prompt_ids(cfg, 9, 6)
    s1 = spec.Sequence(cfg, prompt, capacity=32)
    spec.prefill(cfg, w0, s1)
    s2 = s1.copy()
    zq = spec.draft_logits(cfg, w0, s1, 4)
    n0 = s2.kv_len
    rows = [s2.tokens[-1]] + [cfg["mask_id"]] * 3
    pos = n0 + np.arange(4)
    lim = np.array([n0] + [n0 + 3] * 3)
    zar = om.forward(cfg, w0, s2.cache, rows, pos, np.ones(4), lim, lora=False)
    np.testing.assert_array_equal(zq, zar)


def test_commit_cache_equals_fresh_prefill(tiny):
    cfg, w = tiny
    prompt = synth.prompt_ids(cfg, 10, 8)
    seq = spec.Sequence(cfg, prompt, capacity=64)
    spec.prefill(cfg, w, seq)
    for _ in range(3):
        spec.step(cfg, w, seq, 4, 1.0, spec.PhiloxDraws(0, 0, seq.step))
    fresh = spec.Sequence(cfg, seq.tokens, capacity=64)
    spec.prefill(cfg, w, fresh)
    assert fresh.kv_len == seq.kv_len == len(seq.tokens) - 1
    for li in range(cfg["n_layers"]):
        np.testing.assert_allclose(seq.cache.k[li][: seq.kv_len], fresh.cache.k[li][: seq.kv_len],
                                   rtol=1e-9, atol=1e-11)
        np.testing.assert_allclose(seq.cache.v[li][: seq.kv_len], fresh.cache.v[li][: seq.kv_len],
                                   rtol=1e-9, atol=1e-11)


def test_lora_param_count_is_pages_figure():
    facts = json.load(open(os.path.join(GOLDEN, "pages_facts.json")))
    cfg = synth.QWEN3_8B
    shp = synth.proj_shapes(cfg)
    n = cfg["n_layers"] * sum(cfg["lora_rank"] * (o + i) for o, i in shp.values())
    assert n == 349_175_808
    assert round(n / 1e9, 2) == facts["extra_params_8b_billions"]
    kv_bytes = cfg["n_layers"] * 2 * cfg["n_kv_heads"] * cfg["head_dim"] * 2
    assert kv_bytes == 147_456


def test_bf16_round_matches_torch_and_identity_mode(tiny):
    rng = np.random.default_rng(12)
    x = np.concatenate([rng.standard_normal(20000) * 10 ** rng.uniform(-6, 6, 20000),
                        [0.0, -0.0, 1.0, 1.00390625, 1.0078125, 3.0e38, -2.5e-38]])
    ref = torch.from_numpy(x.astype(np.float32)).to(torch.bfloat16).to(torch.float64).numpy()
    np.testing.assert_array_equal(om.bf16_round(x), ref)
    # ties go to even: 1 + 2^-8 lies halfway between 1 and 1 + 2^-7
    assert om.bf16_round(np.array([1.0 + 2 ** -8]))[0] == 1.0
    assert om.bf16_round(np.array([1.0 + 3 * 2 ** -8]))[0] == 1.0 + 2 ** -6
    # the rounded mode changes the logits only by rounding-sized amounts
    cfg, w = tiny
    prompt = synth.prompt_ids(cfg, 10, 3)
    s1 = spec.Sequence(cfg, prompt, capacity=32)
    spec.prefill(cfg, w, s1)
    s2 = s1.copy()
    z = spec.draft_logits(cfg, w, s1, 4)
    zr = spec.draft_logits(cfg, w, s2, 4, act_round=om.bf16_round)
    err = np.abs(z - zr).max()
    assert 0 < err < 0.05
