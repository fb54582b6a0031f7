"""fp64 forward pass of a diffusion-augmented decoder (oracle, test infrastructure).

Follows the pages' description of the architecture: every layer keeps its
autoregressive weights and adds rank-r LoRA "diffusion weights" with scale
alpha/r; drafting runs the AR + LoRA weights and verification runs the AR
weights alone, over one shared KV cache (picx.dev summary, "Methodology /
Architecture: Diffusion-Augmented LLMs" and "Practical Implications";
paperglide reader, "The Uno Framework").  The first position of a drafted block
is computed with the AR weights only, the remaining positions with AR + LoRA
(paperglide reader, "The Psi-Speculative Sampler", "Sampler Extensions"): a
per-row gate g in {0, 1} multiplies the LoRA term.  The LoRA term sits on the
seven linears q, k, v, o, gate, up, down ("small trainable modules ... every
weight matrix", paperglide reader, "Empirical Results").

The decoder body itself (pre-norm, RMSNorm, rotate-half RoPE, grouped-query
attention, SwiGLU MLP, untied LM head, no biases) is the standard one the model
configurations name; the pages call the base model a standard LLM and print no
layer equations.  Readings: RMSNorm epsilon is a config value; attention
scale 1/sqrt(head_dim); RoPE frequencies theta^(-2i/head_dim); q head h reads
kv head floor(h / (n_q_heads / n_kv_heads)).

Everything here is fp64 numpy on logical (unpacked) weight layouts:
  embed [V, D], lm_head [V, D], final_norm [D];
  per layer: attn_norm [D], mlp_norm [D], q [Hq*hd, D], k [Hkv*hd, D],
  v [Hkv*hd, D], o [D, Hq*hd], gate [F, D], up [F, D], down [D, F];
  LoRA: lora_a[p] [r, in_p], lora_b[p] [out_p, r] for p in PROJ.

Precision.  By default every step is fp64 (the exact reference, and the one
the parity tests gate on).  With ``act_round=bf16_round`` the forward models a
plain bfloat16 implementation of the same computation: every operand of every
matrix product that is not a (bf16) weight is rounded to bfloat16
(round-to-nearest-even), and the products themselves are exact.  Those operands
are the normalised inputs of the seven projections and of the LM head, the LoRA
intermediate s*g*(x A^T), the queries and keys (after RoPE) and the values of
the attention products, the softmax weights that multiply the values, the
attention output and the SwiGLU product.  The pages fix no precision; the
configurations name a bf16 model.  This mode is a yardstick, not a target: it
says how far from the exact logits a bf16 implementation of this shape lands,
so a GPU path can be held to "no less accurate than plain bf16".

Parity: logit VALUES are "parity unpinned" against the pages (none are printed).
Structural pins in tests/test_oracle_model.py: LoRA linear == dense
x (W + s B A)^T; B = 0 makes the LoRA linear the plain linear; the cached block
forward equals a full uncached causal recompute; attention, RMSNorm and SiLU
agree with independent torch CPU routines.
"""
import numpy as np

PROJ = ("q", "k", "v", "o", "gate", "up", "down")


def bf16_round(x):
    """Round to the nearest bfloat16 (ties to even) and return fp64.

    bfloat16 keeps the top 16 bits of an IEEE fp32; the fp64 input is first
    rounded to fp32 (RNE), then the low 16 bits are rounded away with ties to
    even.  Inputs are finite."""
    f = np.ascontiguousarray(np.asarray(x, dtype=np.float64).astype(np.float32))
    u = f.view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16 << 16
    return u.astype(np.uint32).view(np.float32).astype(np.float64)


def rms_norm(h, gain, eps):
    """h / sqrt(mean(h^2) + eps) * gain, row-wise."""
    return h / np.sqrt(np.mean(h * h, axis=-1, keepdims=True) + eps) * gain


def silu(x):
    return x / (1.0 + np.exp(-x))


def rope(x, pos, theta):
    """Rotate-half rotary embedding. x [R, H, hd], pos [R] (absolute positions)."""
    hd = x.shape[-1]
    half = hd // 2
    inv_freq = float(theta) ** (-np.arange(half, dtype=np.float64) * 2.0 / hd)
    ang = np.asarray(pos, dtype=np.float64)[:, None] * inv_freq[None, :]
    cos = np.cos(ang)[:, None, :]
    sin = np.sin(ang)[:, None, :]
    x1, x2 = x[..., :half], x[..., half:]
    return np.concatenate([x1 * cos - x2 * sin, x2 * cos + x1 * sin], axis=-1)


def lora_linear(x, w, a, b, scale, gate, act_round=None):
    """y = x W^T + gate_row * scale * (x A^T) B^T; a/b None means no LoRA.

    With ``act_round`` the intermediate gate*scale*(x A^T) is rounded before
    its product with B (the low-rank path's second product)."""
    y = x @ w.T
    if a is not None and b is not None:
        t = (gate[:, None] * scale) * (x @ a.T)
        if act_round is not None:
            t = act_round(t)
        y = y + t @ b.T
    return y


class KVCache:
    """One sequence's cache: per layer K and V [capacity, Hkv, hd], fp64."""

    def __init__(self, cfg, capacity):
        shape = (capacity, cfg["n_kv_heads"], cfg["head_dim"])
        self.k = [np.zeros(shape) for _ in range(cfg["n_layers"])]
        self.v = [np.zeros(shape) for _ in range(cfg["n_layers"])]
        self.capacity = capacity

    def copy(self):
        c = KVCache.__new__(KVCache)
        c.k = [a.copy() for a in self.k]
        c.v = [a.copy() for a in self.v]
        c.capacity = self.capacity
        return c


def attention(q, cache_k, cache_v, key_limit, n_kv_heads, key_sets=None, p_round=None):
    """Per row r and q head h: softmax over keys 0..key_limit[r] of the cache,
    or over the cache slots listed in key_sets[r] when ``key_sets`` is given
    (a token tree's rows see the context and their own ancestors only).
    ``p_round`` rounds the softmax weights before they multiply the values.

    q [R, Hq, hd]; cache_k/v [cap, Hkv, hd]; returns [R, Hq, hd].
    """
    R, Hq, hd = q.shape
    group = Hq // n_kv_heads
    out = np.zeros_like(q)
    scale = 1.0 / np.sqrt(hd)
    if key_sets is None:
        keys = [np.arange(int(key_limit[r]) + 1) for r in range(R)]
    else:
        keys = [np.asarray(sorted(int(k) for k in key_sets[r])) for r in range(R)]
    top = max(int(k.max()) for k in keys) + 1
    for g in range(n_kv_heads):
        kg = np.ascontiguousarray(cache_k[:top, g, :])     # keys of kv head g
        vg = np.ascontiguousarray(cache_v[:top, g, :])
        for r in range(R):
            idx = keys[r]
            for h in range(g * group, (g + 1) * group):
                s = kg[idx] @ q[r, h] * scale
                s = s - s.max()
                p = np.exp(s)
                p = p / p.sum()
                if p_round is not None:
                    p = p_round(p)
                out[r, h] = p @ vg[idx]
    return out


def forward(cfg, wts, cache, ids, pos, gate, key_limit, lora=True, act_round=None,
            slots=None, key_sets=None, taps=None):
    """One pass over a block of rows of ONE sequence.

    Writes the block's K/V (after RoPE) into ``cache`` at ``pos`` before the
    attention of each layer, then attends row r to cache keys 0..key_limit[r].
    Returns fp64 logits [R, V].  ``act_round`` (e.g. ``bf16_round``) selects the
    bf16-activation mode described in the module header.

    A token tree's rows sit at positions (RoPE) that differ from the cache
    slots holding their K/V: ``slots`` then gives the slots, and ``key_sets``
    the slots each row attends to (``key_limit`` is then unused).

    ``taps`` (a list) receives a copy of the residual rows h entering each
    layer, in layer order (the inputs a per-layer comparison starts from).
    """
    rd = act_round if act_round is not None else (lambda v: v)
    ids = np.asarray(ids)
    pos = np.asarray(pos)
    gate = np.asarray(gate, dtype=np.float64)
    Hq, Hkv, hd = cfg["n_q_heads"], cfg["n_kv_heads"], cfg["head_dim"]
    eps = cfg["rms_eps"]
    scale = cfg["lora_alpha"] / cfg["lora_rank"]
    R = len(ids)
    slots = pos if slots is None else np.asarray(slots)
    h = wts["embed"][ids].astype(np.float64)
    for li, lw in enumerate(wts["layers"]):
        if taps is not None:
            taps.append(h.copy())

        def lin(x, p):
            a = lw["lora_a"].get(p) if lora else None
            b = lw["lora_b"].get(p) if lora else None
            return lora_linear(x, lw[p], a, b, scale, gate, act_round)

        x = rd(rms_norm(h, lw["attn_norm"], eps))
        q = lin(x, "q").reshape(R, Hq, hd)
        k = lin(x, "k").reshape(R, Hkv, hd)
        v = rd(lin(x, "v").reshape(R, Hkv, hd))
        q = rd(rope(q, pos, cfg["rope_theta"]))
        k = rd(rope(k, pos, cfg["rope_theta"]))
        cache.k[li][slots] = k
        cache.v[li][slots] = v
        o = rd(attention(q, cache.k[li], cache.v[li], key_limit, Hkv, key_sets, act_round)
               .reshape(R, Hq * hd))
        h = h + lin(o, "o")
        x = rd(rms_norm(h, lw["mlp_norm"], eps))
        h = h + lin(rd(silu(lin(x, "gate")) * lin(x, "up")), "down")
    x = rd(rms_norm(h, wts["final_norm"], eps))
    return x @ wts["lm_head"].T


def full_causal_logits(cfg, wts, tokens):
    """Textbook AR forward over a whole token sequence, no cache reuse, AR weights.

    Row i is the next-token logit vector after tokens[0..i].
    """
    n = len(tokens)
    cache = KVCache(cfg, n)
    pos = np.arange(n)
    return forward(cfg, wts, cache, tokens, pos, np.zeros(n), pos, lora=False)
