"""Seeded synthetic inputs shared by the tests, the bench and the smoke check.

This module draws random numbers and arranges them into the shapes of the
workloads; it holds none of the decode method's arithmetic.  Both the HIP path
and the CPU oracle consume what it returns; neither is imported here.

Model shapes:
* ``TINY``: 2 layers, d_model 256, 4 heads x 64 (no GQA), SwiGLU 1024,
  vocab 512 (mask id 511), LoRA rank 16 alpha 32, RoPE base 10000.
* ``QWEN3_8B``: 36 layers, d_model 4096, 32 q / 8 kv heads x 128, SwiGLU 12288,
  vocab 151936 (mask id 151935), LoRA rank 128 alpha 256, RoPE base 1e6.

Weights are N(0, 0.02) (LoRA A ~ N(0, 0.02), LoRA B ~ N(0, 0.01)), rounded to
bf16 by round-to-nearest-even; norm gains are 1.  Tensor i of a model is drawn
from ``numpy.random.default_rng([seed, i, chunk])`` so any subset of layers can
be regenerated alone.
"""
import concurrent.futures as _cf
import os

import numpy as np
import torch

TINY = dict(n_layers=2, d_model=256, n_q_heads=4, n_kv_heads=4, head_dim=64,
            d_ffn=1024, vocab=512, mask_id=511, rms_eps=1e-6, rope_theta=10000.0,
            lora_rank=16, lora_alpha=32.0)

QWEN3_8B = dict(n_layers=36, d_model=4096, n_q_heads=32, n_kv_heads=8, head_dim=128,
                d_ffn=12288, vocab=151936, mask_id=151935, rms_eps=1e-6,
                rope_theta=1000000.0, lora_rank=128, lora_alpha=256.0)

# the tiny shape with a LoRA rank that fills whole 64-wide K slices
TINY_R64 = dict(TINY, lora_rank=64, lora_alpha=128.0)

# small model with the 8B shape's head layout (head_dim 128, 4 q heads per kv head)
SMALL_GQA = dict(n_layers=2, d_model=512, n_q_heads=8, n_kv_heads=2, head_dim=128,
                 d_ffn=1024, vocab=1024, mask_id=1023, rms_eps=1e-6, rope_theta=1000000.0,
                 lora_rank=64, lora_alpha=128.0)

# enumeration vocabulary toy: vocab 8 (mask id 7)
VOCAB8 = dict(n_layers=1, d_model=32, n_q_heads=2, n_kv_heads=1, head_dim=16,
              d_ffn=64, vocab=8, mask_id=7, rms_eps=1e-6, rope_theta=10000.0,
              lora_rank=4, lora_alpha=8.0)

PROJ = ("q", "k", "v", "o", "gate", "up", "down")
W_STD = 0.02
LORA_A_STD = 0.02
LORA_B_STD = 0.01

_CHUNK = 1 << 24          # elements per independently seeded chunk


def proj_shapes(cfg):
    """(out, in) of each projection's base weight."""
    D, F = cfg["d_model"], cfg["d_ffn"]
    qd = cfg["n_q_heads"] * cfg["head_dim"]
    kd = cfg["n_kv_heads"] * cfg["head_dim"]
    return {"q": (qd, D), "k": (kd, D), "v": (kd, D), "o": (D, qd),
            "gate": (F, D), "up": (F, D), "down": (D, F)}


def _normal_f32(shape, std, key, threads):
    n = int(np.prod(shape))
    out = np.empty(n, dtype=np.float32)
    starts = list(range(0, n, _CHUNK))

    def fill(ci):
        s = starts[ci]
        e = min(n, s + _CHUNK)
        rng = np.random.default_rng(list(key) + [ci])
        rng.standard_normal(e - s, dtype=np.float32, out=out[s:e])
        out[s:e] *= np.float32(std)

    if threads > 1 and len(starts) > 1:
        with _cf.ThreadPoolExecutor(threads) as ex:
            list(ex.map(fill, range(len(starts))))
    else:
        for ci in range(len(starts)):
            fill(ci)
    return out.reshape(shape)


def normal_bf16(shape, std, key, threads=None):
    """bf16 (RNE) torch CPU tensor of N(0, std^2) draws for a seed key list."""
    threads = threads or min(16, os.cpu_count() or 1)
    return torch.from_numpy(_normal_f32(shape, std, key, threads)).to(torch.bfloat16)


def tensor_index(layer, name):
    """Stable index of a tensor within a model (for the seed key)."""
    names = list(PROJ) + ["lora_a_" + p for p in PROJ] + ["lora_b_" + p for p in PROJ]
    return 16 + layer * 64 + names.index(name)


def make_layer(cfg, seed, layer, lora=True, threads=None):
    """One layer's logical weights as bf16 CPU tensors (+ fp32 norm gains)."""
    shp = proj_shapes(cfg)
    r = cfg["lora_rank"]
    lw = {"attn_norm": torch.ones(cfg["d_model"], dtype=torch.float32),
          "mlp_norm": torch.ones(cfg["d_model"], dtype=torch.float32),
          "lora_a": {}, "lora_b": {}}
    for p in PROJ:
        out_f, in_f = shp[p]
        lw[p] = normal_bf16((out_f, in_f), W_STD, [seed, tensor_index(layer, p)], threads)
        if lora:
            lw["lora_a"][p] = normal_bf16((r, in_f), LORA_A_STD,
                                          [seed, tensor_index(layer, "lora_a_" + p)], threads)
            lw["lora_b"][p] = normal_bf16((out_f, r), LORA_B_STD,
                                          [seed, tensor_index(layer, "lora_b_" + p)], threads)
    return lw


def make_weights(cfg, seed=0, lora=True, layers=None, threads=None):
    """Whole model (or the listed layers) as bf16 CPU tensors in logical layout."""
    V, D = cfg["vocab"], cfg["d_model"]
    idx = range(cfg["n_layers"]) if layers is None else layers
    return {"embed": normal_bf16((V, D), W_STD, [seed, 0], threads),
            "lm_head": normal_bf16((V, D), W_STD, [seed, 1], threads),
            "final_norm": torch.ones(D, dtype=torch.float32),
            "layers": [make_layer(cfg, seed, li, lora, threads) for li in idx]}


def zero_lora_b(wts):
    """Copy of ``wts`` whose LoRA B factors are all zero (B = 0 case)."""
    out = dict(wts)
    out["layers"] = []
    for lw in wts["layers"]:
        n = dict(lw)
        n["lora_b"] = {p: torch.zeros_like(t) for p, t in lw["lora_b"].items()}
        out["layers"].append(n)
    return out


def to_f64(wts):
    """Same weights as fp64 numpy arrays (the oracle's input form)."""
    def cv(t):
        return t.to(torch.float64).numpy()
    out = {k: cv(wts[k]) for k in ("embed", "lm_head", "final_norm")}
    out["layers"] = []
    for lw in wts["layers"]:
        n = {k: cv(v) for k, v in lw.items() if isinstance(v, torch.Tensor)}
        n["lora_a"] = {p: cv(t) for p, t in lw["lora_a"].items()}
        n["lora_b"] = {p: cv(t) for p, t in lw["lora_b"].items()}
        out["layers"].append(n)
    return out


def prompt_ids(cfg, n, seed, batch=None):
    """Uniform token ids in [0, vocab-1) (the mask id is never a prompt token)."""
    rng = np.random.default_rng([seed, 7])
    shape = (n,) if batch is None else (batch, n)
    return rng.integers(0, cfg["vocab"] - 1, size=shape, dtype=np.int64).astype(np.int32)


def sampler_logits(batch, K, vocab, seed, sigma_p=3.0, sigma_noise=0.5):
    """Sampler-only workload: AR logits P ~ N(0, sigma_p^2) [B, K+1, V];
    draft logits Q = P + N(0, sigma_noise^2) on positions 2..K and Q = P on
    position 1.  Returns (draft_logits [B,K,V], verify_logits [B,K,V]) fp32,
    where verify row j holds P at position j+2."""
    rng = np.random.default_rng([seed, 11])
    p = rng.standard_normal((batch, K + 1, vocab), dtype=np.float32)
    p *= np.float32(sigma_p)
    q = p[:, :K].copy()
    if K > 1:
        noise = rng.standard_normal((batch, K - 1, vocab), dtype=np.float32)
        q[:, 1:] += noise * np.float32(sigma_noise)
    return q, np.ascontiguousarray(p[:, 1:])


def forced_accepts(batch, K, n_steps, seed):
    """Forced accept lengths a ~ U{0..K} per sequence per step, int32 [S, B]."""
    rng = np.random.default_rng([seed, 13])
    return rng.integers(0, K + 1, size=(n_steps, batch), dtype=np.int64).astype(np.int32)


def random_tokens(n, vocab, seed, shape):
    rng = np.random.default_rng([seed, n, 17])
    return rng.integers(0, vocab - 1, size=shape, dtype=np.int64).astype(np.int32)


def kv_values(cfg, seq_len, seed, seq=0, std=1.0):
    """Seeded synthetic committed K/V content for one sequence, bf16 CPU tensors
    of logical shape [n_layers, seq_len, n_kv_heads, head_dim] (K, V)."""
    shape = (cfg["n_layers"], seq_len, cfg["n_kv_heads"], cfg["head_dim"])
    k = normal_bf16(shape, std, [seed, 23, seq, 0])
    v = normal_bf16(shape, std, [seed, 23, seq, 1])
    return k, v


def make_weights_device(cfg, seed=0, device="cuda", lora=True):
    """Whole model drawn directly on the GPU (torch's seeded device generator),
    same shapes and distributions as ``make_weights`` but different values;
    for throughput runs, where no oracle reads the weights."""
    dev = torch.device(device)
    gen = torch.Generator(device=dev)

    def draw(shape, std, key):
        gen.manual_seed(int(np.random.SeedSequence(key).generate_state(1, np.uint64)[0] >> 1))
        t = torch.randn(shape, generator=gen, device=dev, dtype=torch.float32)
        return t.mul_(std).to(torch.bfloat16)

    shp = proj_shapes(cfg)
    r = cfg["lora_rank"]
    D = cfg["d_model"]
    out = {"embed": draw((cfg["vocab"], D), W_STD, [seed, 0]),
           "lm_head": draw((cfg["vocab"], D), W_STD, [seed, 1]),
           "final_norm": torch.ones(D, dtype=torch.float32, device=dev), "layers": []}
    for li in range(cfg["n_layers"]):
        lw = {"attn_norm": torch.ones(D, dtype=torch.float32, device=dev),
              "mlp_norm": torch.ones(D, dtype=torch.float32, device=dev),
              "lora_a": {}, "lora_b": {}}
        for p in PROJ:
            o, i = shp[p]
            lw[p] = draw((o, i), W_STD, [seed, tensor_index(li, p)])
            if lora:
                lw["lora_a"][p] = draw((r, i), LORA_A_STD, [seed, tensor_index(li, "lora_a_" + p)])
                lw["lora_b"][p] = draw((o, r), LORA_B_STD, [seed, tensor_index(li, "lora_b_" + p)])
        out["layers"].append(lw)
    return out


def fill_kv_device(k_pages, v_pages, seed, std=1.0):
    """Seeded N(0, std^2) content for every page of a device KV pool."""
    gen = torch.Generator(device=k_pages.device)
    for li in range(k_pages.shape[0]):
        for which, t in ((0, k_pages), (1, v_pages)):
            gen.manual_seed(int(seed) * 1000003 + li * 2 + which)
            t[li].normal_(0.0, std, generator=gen)


class LazyF64Layers:
    """fp64 numpy view of bf16 layer tensors, converted on every access (keeps
    host memory at one layer's worth for the 8B shape)."""

    def __init__(self, layers):
        self._layers = layers

    def __len__(self):
        return len(self._layers)

    def __iter__(self):
        for lw in self._layers:
            yield _LazyLayer(lw)


class _LazyLayer:
    def __init__(self, lw):
        self._lw = lw

    def __getitem__(self, k):
        v = self._lw[k]
        if isinstance(v, dict):
            return _LazyDict(v)
        return v.to(torch.float64).numpy()


class _LazyDict:
    def __init__(self, d):
        self._d = d

    def get(self, k, default=None):
        v = self._d.get(k)
        return default if v is None else v.to(torch.float64).numpy()


def to_f64_lazy(wts):
    """Like ``to_f64`` but layers convert on access (large models)."""
    return {"embed": wts["embed"].to(torch.float64).numpy(),
            "lm_head": wts["lm_head"].to(torch.float64).numpy(),
            "final_norm": wts["final_norm"].to(torch.float64).numpy(),
            "layers": LazyF64Layers(wts["layers"])}
