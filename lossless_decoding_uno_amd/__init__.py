"""Python binding of libuno, the gfx950 HIP implementation of the Psi-Spec
draft-and-verify decode step (see include/uno.h for the C ABI).

This layer only marshals arguments: torch tensors on the GPU provide device
memory and ``torch.cuda.current_stream()`` provides the stream; every step of
the decode path runs in the library's HIP kernels.  Importing works without a
GPU (the library is a gfx950 code object plus host code); calling an entry
point needs the library to be built and a GPU to be present, and raises
otherwise -- there is no CPU fallback.
"""
import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libuno.so")

PROJ = ("q", "k", "v", "o", "gate", "up", "down")

UNO_OK = 0
STATUS_NAMES = {1: "invalid argument", 2: "unsupported shape", 3: "page table too small",
                4: "workspace too small", 5: "HIP launch failure"}
DEV_CAPACITY, DEV_BAD_TOKEN, DEV_BAD_PAGE, DEV_NONFINITE, DEV_BAD_ACCEPT = 1, 2, 4, 8, 16
DEV_SYNC_TIMEOUT = 32

EXPORTS = ("uno_workspace_bytes", "uno_draft_block", "uno_draft_block_from", "uno_verify_block",
           "uno_draft_sample",
           "uno_spec_accept_workspace_bytes", "uno_spec_accept", "uno_spec_accept_noalloc",
           "uno_kv_commit",
           "uno_tree_rows", "uno_tree_workspace_bytes", "uno_tree_build", "uno_verify_tree",
           "uno_tree_accept", "uno_tree_commit",
           "uno_pack_weight",
           "uno_set_timing_events", "uno_timing_events_used", "uno_status_string",
           "uno_last_hip_error")

TIME_ATTENTION, TIME_GEMM, TIME_LORA_A, TIME_LM_HEAD, TIME_SAMPLER = 1, 2, 3, 4, 5
TIME_GEMM_QKV, TIME_GEMM_O, TIME_GEMM_GATE_UP, TIME_GEMM_DOWN = 6, 7, 8, 9


class UnoConfig(ctypes.Structure):
    _fields_ = [("n_layers", ctypes.c_int32), ("d_model", ctypes.c_int32),
                ("n_q_heads", ctypes.c_int32), ("n_kv_heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("d_ffn", ctypes.c_int32),
                ("vocab", ctypes.c_int32), ("mask_id", ctypes.c_int32),
                ("rms_eps", ctypes.c_float), ("rope_theta", ctypes.c_float),
                ("lora_rank", ctypes.c_int32), ("lora_scale", ctypes.c_float),
                ("lora_mask", ctypes.c_uint32), ("page_size", ctypes.c_int32),
                ("noise_prior", ctypes.c_int32)]


class UnoLayerWeights(ctypes.Structure):
    _fields_ = [("attn_norm", ctypes.c_void_p), ("mlp_norm", ctypes.c_void_p),
                ("wq", ctypes.c_void_p), ("wk", ctypes.c_void_p), ("wv", ctypes.c_void_p),
                ("wo", ctypes.c_void_p), ("wgate", ctypes.c_void_p), ("wup", ctypes.c_void_p),
                ("wdown", ctypes.c_void_p), ("lora_a", ctypes.c_void_p * 7),
                ("lora_b", ctypes.c_void_p * 7)]


class UnoWeights(ctypes.Structure):
    _fields_ = [("embed", ctypes.c_void_p), ("lm_head", ctypes.c_void_p),
                ("final_norm", ctypes.c_void_p), ("layers", ctypes.POINTER(UnoLayerWeights))]


class UnoKV(ctypes.Structure):
    _fields_ = [("k_pages", ctypes.c_void_p), ("v_pages", ctypes.c_void_p),
                ("n_pages", ctypes.c_int64), ("page_table", ctypes.c_void_p),
                ("max_pages_per_seq", ctypes.c_int32), ("kv_len", ctypes.c_void_p)]


_lib = None


def load_library():
    """Load libuno.so; raise if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError("libuno.so is not built (run lossless_decoding_uno_amd.build)")
    lib = ctypes.CDLL(LIB_PATH)
    P, I, U64, F, SZ = ctypes.c_void_p, ctypes.c_int, ctypes.c_uint64, ctypes.c_float, ctypes.c_size_t
    lib.uno_workspace_bytes.restype = SZ
    lib.uno_workspace_bytes.argtypes = [P, I, I, I]
    lib.uno_draft_block.restype = I
    lib.uno_draft_block.argtypes = [P, P, P, P, I, I, I, F, U64, P, P, P, P, P, P, SZ, P]
    lib.uno_draft_block_from.restype = I
    lib.uno_draft_block_from.argtypes = [P, P, P, P, P, I, I, I, F, U64, P, I, ctypes.c_uint32,
                                         I, P, P, P, P, P, SZ, P]
    lib.uno_verify_block.restype = I
    lib.uno_verify_block.argtypes = [P, P, P, P, I, I, I, I, P, P, P, P, SZ, P]
    lib.uno_draft_sample.restype = I
    lib.uno_draft_sample.argtypes = [P, P, I, I, I, F, U64, P, P, P, P]
    lib.uno_spec_accept_workspace_bytes.restype = SZ
    lib.uno_spec_accept_workspace_bytes.argtypes = [I, I]
    lib.uno_spec_accept.restype = I
    lib.uno_spec_accept.argtypes = [P, P, P, P, P, I, I, I, F, U64, P, P, P, P, P, P, P, SZ, P]
    lib.uno_spec_accept_noalloc.restype = I
    lib.uno_spec_accept_noalloc.argtypes = [P, P, P, P, P, I, I, I, F, U64, P, P, P, P, P, P, P]
    lib.uno_kv_commit.restype = I
    lib.uno_kv_commit.argtypes = [P, P, I, I, P, P, P]
    lib.uno_tree_rows.restype = I
    lib.uno_tree_rows.argtypes = [I, I, I]
    lib.uno_tree_workspace_bytes.restype = SZ
    lib.uno_tree_workspace_bytes.argtypes = [I, I, I]
    lib.uno_tree_build.restype = I
    lib.uno_tree_build.argtypes = [P, P, I, I, I, I, I, P, P, P, P, P, P, P, SZ, P]
    lib.uno_verify_tree.restype = I
    lib.uno_verify_tree.argtypes = [P, P, P, P, P, P, I, I, I, P, P, P, SZ, P]
    lib.uno_tree_accept.restype = I
    lib.uno_tree_accept.argtypes = [P, P, P, P, P, I, I, I, I, F, U64, P, P, P, P, P, P, P, P]
    lib.uno_tree_commit.restype = I
    lib.uno_tree_commit.argtypes = [P, P, P, P, I, I, P, P, P]
    lib.uno_pack_weight.restype = I
    lib.uno_pack_weight.argtypes = [P, P, I, I, P]
    lib.uno_status_string.restype = ctypes.c_char_p
    lib.uno_status_string.argtypes = [I]
    lib.uno_last_hip_error.restype = ctypes.c_char_p
    lib.uno_last_hip_error.argtypes = []
    lib.uno_set_timing_events.restype = I
    lib.uno_set_timing_events.argtypes = [I, P, P, I]
    lib.uno_timing_events_used.restype = I
    lib.uno_timing_events_used.argtypes = []
    _lib = lib
    return lib


class UnoError(RuntimeError):
    pass


def _check(rc):
    if rc != UNO_OK:
        lib = load_library()
        msg = lib.uno_status_string(rc).decode()
        if rc == 5:
            msg += ": " + lib.uno_last_hip_error().decode()
        raise UnoError("libuno error %d (%s)" % (rc, msg))


def _ptr(t):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("expected a GPU tensor")
    if not t.is_contiguous():
        raise ValueError("expected a contiguous tensor")
    return ctypes.c_void_p(t.data_ptr())


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _need(t, dtype, shape, name):
    if t.dtype != dtype or tuple(t.shape) != tuple(shape):
        raise ValueError("%s: expected %s %s, got %s %s" % (name, dtype, tuple(shape), t.dtype,
                                                            tuple(t.shape)))


def make_config(cfg, page_size=16, lora=True):
    """uno_config from a shape dict (keys as in the synthetic model shapes).
    ``lora``: True (LoRA on all seven projections), False, or a lora_mask."""
    r = int(cfg["lora_rank"])
    mask = 0x7F if lora is True else (int(lora) if lora else 0)
    return UnoConfig(int(cfg["n_layers"]), int(cfg["d_model"]), int(cfg["n_q_heads"]),
                     int(cfg["n_kv_heads"]), int(cfg["head_dim"]), int(cfg["d_ffn"]),
                     int(cfg["vocab"]), int(cfg["mask_id"]), float(cfg["rms_eps"]),
                     float(cfg["rope_theta"]), r, float(cfg["lora_alpha"]) / r,
                     mask, int(page_size), int(cfg.get("noise_prior", 0)))


def pack_weight(t):
    """Tile-packed device copy of a row-major bf16 [out, in] GPU matrix
    (uno_pack_weight): the layout the library reads weights in."""
    lib = load_library()
    n_out, n_in = t.shape
    out = torch.empty_like(t)
    _check(lib.uno_pack_weight(_ptr(t), _ptr(out), n_out, n_in, _stream()))
    return out


class Model:
    """Device-resident weights of one model and the uno_weights table over them.

    ``weights`` holds torch tensors in the logical layout (bf16 [out, in]
    base weights, bf16 LoRA A [r, in] / B [out, r], fp32 norm gains); they are
    copied to the GPU and the base weights, LoRA A factors and LM head are
    stored tile-packed (uno_pack_weight), the layout include/uno.h prescribes.
    ``packed`` names top-level entries ("lm_head") given already packed on the
    GPU, used as they are."""

    def __init__(self, cfg, weights, page_size=16, lora=True, device="cuda", packed=()):
        """``lora``: True, False, or a lora_mask (bit p: projection PROJ[p])."""
        self.cfg = dict(cfg)
        self.config = make_config(cfg, page_size, lora)
        dev = torch.device(device)

        def up(t, dtype):
            return t.to(device=dev, dtype=dtype).contiguous()

        def upk(t):
            return pack_weight(up(t, torch.bfloat16))

        self.embed = up(weights["embed"], torch.bfloat16)
        self.lm_head = (up(weights["lm_head"], torch.bfloat16) if "lm_head" in packed
                        else upk(weights["lm_head"]))
        self.final_norm = up(weights["final_norm"], torch.float32)
        self.layers = []
        n = len(weights["layers"])
        if n != cfg["n_layers"]:
            raise ValueError("weights hold %d layers, config %d" % (n, cfg["n_layers"]))
        self._table = (UnoLayerWeights * n)()

        def up_pair(a, b, pack):
            # gate and up stored back to back: the library then fuses SwiGLU
            # into the gate|up product (any placement works, this one is faster)
            both = torch.cat([a.to(device=dev, dtype=torch.bfloat16),
                              b.to(device=dev, dtype=torch.bfloat16)])
            if pack:
                both = pack_weight(both)
            return both[: a.shape[0]], both[a.shape[0]:]

        for li, lw in enumerate(weights["layers"]):
            d = {"attn_norm": up(lw["attn_norm"], torch.float32),
                 "mlp_norm": up(lw["mlp_norm"], torch.float32)}
            for p in PROJ:
                if p not in ("gate", "up"):
                    d[p] = upk(lw[p])
            d["gate"], d["up"] = up_pair(lw["gate"], lw["up"], True)
            d["lora_a"] = {p: upk(t) for p, t in lw.get("lora_a", {}).items()}
            d["lora_b"] = {p: up(t, torch.bfloat16) for p, t in lw.get("lora_b", {}).items()
                           if p not in ("gate", "up")}
            lb = lw.get("lora_b", {})
            if "gate" in lb and "up" in lb:
                d["lora_b"]["gate"], d["lora_b"]["up"] = up_pair(lb["gate"], lb["up"], False)
            self.layers.append(d)
            e = self._table[li]
            e.attn_norm, e.mlp_norm = d["attn_norm"].data_ptr(), d["mlp_norm"].data_ptr()
            e.wq, e.wk, e.wv, e.wo = (d[p].data_ptr() for p in ("q", "k", "v", "o"))
            e.wgate, e.wup, e.wdown = (d[p].data_ptr() for p in ("gate", "up", "down"))
            for i, p in enumerate(PROJ):
                e.lora_a[i] = d["lora_a"][p].data_ptr() if p in d["lora_a"] else None
                e.lora_b[i] = d["lora_b"][p].data_ptr() if p in d["lora_b"] else None
        self.weights = UnoWeights(self.embed.data_ptr(), self.lm_head.data_ptr(),
                                  self.final_norm.data_ptr(),
                                  ctypes.cast(self._table, ctypes.POINTER(UnoLayerWeights)))


class PagedKV:
    """A paged KV cache for `batch` sequences of up to `capacity` positions.

    Pages of sequence b are ``page_table[b]``; by default a seeded permutation
    of the pool is used (any assignment of distinct pages works)."""

    def __init__(self, cfg, batch, capacity, page_size=16, device="cuda", page_order=None,
                 extra_pages=0, n_pages=None):
        """``n_pages`` sets the pool size directly (pages then handed out on
        demand, e.g. by ``generate.PagePool``; the table starts at page 0)."""
        self.cfg = cfg
        self.batch = batch
        self.page_size = page_size
        self.max_pages = (capacity + page_size - 1) // page_size
        self.n_pages = batch * self.max_pages + extra_pages if n_pages is None else int(n_pages)
        if n_pages is not None:
            page_order = torch.zeros(batch * self.max_pages, dtype=torch.int64)
        L, H, hd = cfg["n_layers"], cfg["n_kv_heads"], cfg["head_dim"]
        dev = torch.device(device)
        self.k_pages = torch.zeros((L, self.n_pages, H, page_size, hd), dtype=torch.bfloat16,
                                   device=dev)
        self.v_pages = torch.zeros((L, self.n_pages, H, hd, page_size), dtype=torch.bfloat16,
                                   device=dev)
        if page_order is None:
            page_order = torch.arange(self.n_pages, dtype=torch.int64)
        order = torch.as_tensor(page_order, dtype=torch.int64)[: batch * self.max_pages]
        self.page_table = order.reshape(batch, self.max_pages).to(torch.int32).to(dev).contiguous()
        self.kv_len = torch.zeros(batch, dtype=torch.int32, device=dev)
        self.struct = UnoKV(self.k_pages.data_ptr(), self.v_pages.data_ptr(), self.n_pages,
                            self.page_table.data_ptr(), self.max_pages, self.kv_len.data_ptr())


def workspace_bytes(model, batch, K, max_ctx):
    lib = load_library()
    return int(lib.uno_workspace_bytes(ctypes.byref(model.config), batch, K, max_ctx))


def spec_accept_workspace_bytes(batch, K):
    return int(load_library().uno_spec_accept_workspace_bytes(batch, K))


def alloc_workspace(nbytes, device="cuda"):
    return torch.empty(max(int(nbytes), 256), dtype=torch.uint8, device=device)


def _row_max_arg(row_max, B, K):
    if row_max is not None:
        _need(row_max, torch.float32, (B, K), "row_max")
    return _ptr(row_max)


def draft_block(model, kv, anchor, K, max_ctx, inv_temp, seed, step, draft_logits,
                draft_tokens, ws, status=None, row_max=None):
    """uno_draft_block: anchor [B] int32, step [B] uint64 -> draft_logits
    [B, K, V] fp32 and draft_tokens [B, K] int32 (written in place); row_max
    [B, K] fp32 (optional) receives every logits row's maximum."""
    lib = load_library()
    B = anchor.shape[0]
    V = model.cfg["vocab"]
    _need(anchor, torch.int32, (B,), "anchor")
    _need(step, torch.uint64, (B,), "step")
    _need(draft_logits, torch.float32, (B, K, V), "draft_logits")
    _need(draft_tokens, torch.int32, (B, K), "draft_tokens")
    _check(lib.uno_draft_block(ctypes.byref(model.config), ctypes.byref(model.weights),
                               ctypes.byref(kv.struct), _ptr(anchor), B, K, max_ctx,
                               float(inv_temp), int(seed), _ptr(step), _ptr(draft_logits),
                               _ptr(draft_tokens), _row_max_arg(row_max, B, K), _ptr(status),
                               _ptr(ws), ws.numel(), _stream()))


def keep_threshold(kappa):
    """Correction strength kappa in [0, 1] as the 24-bit keep threshold
    round(kappa * 2^24) of uno_draft_block_from."""
    k = float(kappa)
    if not 0.0 <= k <= 1.0:
        raise ValueError("kappa must lie in [0, 1]")
    return int(round(k * (1 << 24)))


def draft_block_from(model, kv, anchor, block, K, max_ctx, inv_temp, seed, step, sample_slot,
                     draft_logits, draft_tokens, ws, status=None, kappa=1.0, corr_pass=0,
                     row_max=None):
    """uno_draft_block_from: one pass of a multi-pass draft; block [B, K] int32
    (rows 1..K-1 are the corrector's output for block[:, :K-1], each kept with
    probability kappa) or None; sample_slot 0 or 4 + pass; corr_pass the index
    of the pass that sampled block."""
    lib = load_library()
    B = anchor.shape[0]
    V = model.cfg["vocab"]
    _need(anchor, torch.int32, (B,), "anchor")
    if block is not None:
        _need(block, torch.int32, (B, K), "block")
    _need(step, torch.uint64, (B,), "step")
    _need(draft_logits, torch.float32, (B, K, V), "draft_logits")
    _need(draft_tokens, torch.int32, (B, K), "draft_tokens")
    _check(lib.uno_draft_block_from(ctypes.byref(model.config), ctypes.byref(model.weights),
                                    ctypes.byref(kv.struct), _ptr(anchor), _ptr(block), B, K,
                                    max_ctx, float(inv_temp), int(seed), _ptr(step),
                                    int(sample_slot), keep_threshold(kappa), int(corr_pass),
                                    _ptr(draft_logits), _ptr(draft_tokens),
                                    _row_max_arg(row_max, B, K), _ptr(status),
                                    _ptr(ws), ws.numel(), _stream()))


def draft_passes(model, kv, anchor, K, max_ctx, inv_temp, seed, step, n_passes, draft_logits,
                 draft_tokens, ws, status=None, kappa=1.0, row_max=None):
    """n_passes draft passes: pass i > 0 reads the corrector's output for the
    tokens pass i-1 sampled (slot 4 + (i-1)), each kept with probability kappa
    (one value, or one per transition); the last pass samples with slot 0 and
    leaves the logits and tokens that verification uses."""
    kap = list(kappa) if isinstance(kappa, (list, tuple)) else [kappa] * max(0, n_passes - 1)
    for i in range(n_passes):
        draft_block_from(model, kv, anchor, draft_tokens if i else None, K, max_ctx, inv_temp,
                         seed, step, 0 if i == n_passes - 1 else 4 + i, draft_logits,
                         draft_tokens, ws, status, kappa=kap[i - 1] if i else 1.0,
                         corr_pass=i - 1 if i else 0, row_max=row_max)


def verify_block(model, kv, rows, max_ctx, pos_offset, verify_logits, ws, status=None,
                 row_max=None):
    """uno_verify_block: rows [B, K] int32 -> verify_logits [B, K, V] fp32 (or None);
    row_max [B, K] fp32 (optional) receives every logits row's maximum."""
    lib = load_library()
    B, K = rows.shape
    _need(rows, torch.int32, (B, K), "rows")
    if verify_logits is not None:
        _need(verify_logits, torch.float32, (B, K, model.cfg["vocab"]), "verify_logits")
    _check(lib.uno_verify_block(ctypes.byref(model.config), ctypes.byref(model.weights),
                                ctypes.byref(kv.struct), _ptr(rows), B, K, max_ctx, pos_offset,
                                _ptr(verify_logits), _row_max_arg(row_max, B, K), _ptr(status),
                                _ptr(ws), ws.numel(), _stream()))


def draft_sample(logits, inv_temp, seed, step, tokens, status=None, row_max=None):
    lib = load_library()
    B, K, V = logits.shape
    _need(logits, torch.float32, (B, K, V), "logits")
    _need(step, torch.uint64, (B,), "step")
    _need(tokens, torch.int32, (B, K), "tokens")
    _check(lib.uno_draft_sample(_ptr(logits), _row_max_arg(row_max, B, K), B, K, V,
                                float(inv_temp), int(seed), _ptr(step), _ptr(tokens),
                                _ptr(status), _stream()))


def spec_accept(draft_logits, verify_logits, draft_tokens, inv_temp, seed, step, accept_len,
                committed, extra_token, ws, forced_accept=None, status=None,
                draft_row_max=None, verify_row_max=None):
    lib = load_library()
    B, K, V = draft_logits.shape
    _need(draft_logits, torch.float32, (B, K, V), "draft_logits")
    _need(verify_logits, torch.float32, (B, K, V), "verify_logits")
    _need(draft_tokens, torch.int32, (B, K), "draft_tokens")
    _need(step, torch.uint64, (B,), "step")
    _need(accept_len, torch.int32, (B,), "accept_len")
    _need(committed, torch.int32, (B, K + 1), "committed")
    _need(extra_token, torch.int32, (B,), "extra_token")
    if forced_accept is not None:
        _need(forced_accept, torch.int32, (B,), "forced_accept")
    _check(lib.uno_spec_accept(_ptr(draft_logits), _ptr(verify_logits),
                               _row_max_arg(draft_row_max, B, K),
                               _row_max_arg(verify_row_max, B, K), _ptr(draft_tokens), B, K,
                               V, float(inv_temp), int(seed), _ptr(step), _ptr(forced_accept),
                               _ptr(accept_len), _ptr(committed), _ptr(extra_token),
                               _ptr(status), _ptr(ws), ws.numel(), _stream()))


def spec_accept_noalloc(draft_logits, verify_logits, draft_tokens, inv_temp, seed, step,
                        accept_len, committed, extra_token, forced_accept=None, status=None,
                        draft_row_max=None, verify_row_max=None):
    """uno_spec_accept_noalloc: as spec_accept, on the library's static scratch
    (no workspace argument)."""
    lib = load_library()
    B, K, V = draft_logits.shape
    _need(draft_logits, torch.float32, (B, K, V), "draft_logits")
    _need(verify_logits, torch.float32, (B, K, V), "verify_logits")
    _need(draft_tokens, torch.int32, (B, K), "draft_tokens")
    _need(step, torch.uint64, (B,), "step")
    _need(accept_len, torch.int32, (B,), "accept_len")
    _need(committed, torch.int32, (B, K + 1), "committed")
    _need(extra_token, torch.int32, (B,), "extra_token")
    if forced_accept is not None:
        _need(forced_accept, torch.int32, (B,), "forced_accept")
    _check(lib.uno_spec_accept_noalloc(_ptr(draft_logits), _ptr(verify_logits),
                                       _row_max_arg(draft_row_max, B, K),
                                       _row_max_arg(verify_row_max, B, K),
                                       _ptr(draft_tokens), B, K, V, float(inv_temp), int(seed),
                                       _ptr(step), _ptr(forced_accept), _ptr(accept_len),
                                       _ptr(committed), _ptr(extra_token), _ptr(status),
                                       _stream()))


def kv_commit(kv, accept_len, K, step=None, status=None):
    lib = load_library()
    B = accept_len.shape[0]
    _need(accept_len, torch.int32, (B,), "accept_len")
    if step is not None:
        _need(step, torch.uint64, (B,), "step")
    _check(lib.uno_kv_commit(ctypes.byref(kv.struct), _ptr(accept_len), B, K, _ptr(step),
                             _ptr(status), _stream()))


# ---------------------------------------------------------------- tree sampler
def tree_rows(K, topk, n_keep):
    """Node rows per sequence (1 + n_keep * (K - 1)); 0 for an unsupported shape."""
    return int(load_library().uno_tree_rows(K, topk, n_keep))


class TreeBuffers:
    """Device buffers of one tree step for B sequences (block length K)."""

    def __init__(self, B, K, topk, n_keep, vocab, device="cuda"):
        N = tree_rows(K, topk, n_keep)
        if not N:
            raise ValueError("unsupported tree shape K=%d topk=%d n_keep=%d" % (K, topk, n_keep))
        self.B, self.K, self.topk, self.n_keep, self.N = B, K, topk, n_keep, N
        W = (N + 31) // 32
        i32 = dict(dtype=torch.int32, device=device)
        self.tokens = torch.empty((B, N), **i32)
        self.parent = torch.empty((B, N), **i32)
        self.depth = torch.empty((B, N), **i32)
        self.anc = torch.empty((B, N, W), dtype=torch.uint32, device=device)
        self.n_nodes = torch.empty(B, **i32)
        self.sample = torch.empty((B, N), **i32)
        self.path = torch.empty((B, K), **i32)
        self.ws = alloc_workspace(load_library().uno_tree_workspace_bytes(B, K, topk), device)


def tree_build(draft_logits, draft_tokens, tb, status=None):
    """uno_tree_build: the best tb.n_keep candidates of the drafted rows and
    their prefix tree, into tb."""
    lib = load_library()
    B, K, V = draft_logits.shape
    _need(draft_logits, torch.float32, (tb.B, tb.K, V), "draft_logits")
    _need(draft_tokens, torch.int32, (B, K), "draft_tokens")
    _check(lib.uno_tree_build(_ptr(draft_logits), _ptr(draft_tokens), B, K, V, tb.topk,
                              tb.n_keep, _ptr(tb.tokens), _ptr(tb.parent), _ptr(tb.depth),
                              _ptr(tb.anc), _ptr(tb.n_nodes), _ptr(status), _ptr(tb.ws),
                              tb.ws.numel(), _stream()))


def verify_tree(model, kv, tb, max_ctx, verify_logits, ws, status=None):
    """uno_verify_tree: verify_logits [B, N, V] fp32 over the node rows of tb."""
    lib = load_library()
    if verify_logits is not None:
        _need(verify_logits, torch.float32, (tb.B, tb.N, model.cfg["vocab"]), "verify_logits")
    _check(lib.uno_verify_tree(ctypes.byref(model.config), ctypes.byref(model.weights),
                               ctypes.byref(kv.struct), _ptr(tb.tokens), _ptr(tb.depth),
                               _ptr(tb.anc), tb.B, tb.N, max_ctx, _ptr(verify_logits),
                               _ptr(status), _ptr(ws), ws.numel(), _stream()))


def tree_accept(verify_logits, tb, inv_temp, seed, step, accept_len, committed, extra_token,
                status=None):
    """uno_tree_accept: per-node draws (tb.sample), the walk, a / committed /
    extra token, and the walked path (tb.path)."""
    lib = load_library()
    B, N, V = verify_logits.shape
    _need(verify_logits, torch.float32, (tb.B, tb.N, V), "verify_logits")
    _need(step, torch.uint64, (B,), "step")
    _need(accept_len, torch.int32, (B,), "accept_len")
    _need(committed, torch.int32, (B, tb.K + 1), "committed")
    _need(extra_token, torch.int32, (B,), "extra_token")
    _check(lib.uno_tree_accept(_ptr(verify_logits), _ptr(tb.tokens), _ptr(tb.parent),
                               _ptr(tb.depth), _ptr(tb.n_nodes), B, tb.K, N, V, float(inv_temp),
                               int(seed), _ptr(step), _ptr(tb.sample), _ptr(accept_len),
                               _ptr(committed), _ptr(extra_token), _ptr(tb.path), _ptr(status),
                               _stream()))


def tree_commit(model, kv, tb, accept_len, step=None, status=None):
    """uno_tree_commit: move the walked path's K/V into place, then advance
    kv_len (and step)."""
    lib = load_library()
    _need(accept_len, torch.int32, (tb.B,), "accept_len")
    if step is not None:
        _need(step, torch.uint64, (tb.B,), "step")
    _check(lib.uno_tree_commit(ctypes.byref(model.config), ctypes.byref(kv.struct),
                               _ptr(tb.path), _ptr(accept_len), tb.B, tb.K, _ptr(step),
                               _ptr(status), _stream()))


class KernelTimer:
    """HIP events that libuno records around every launch of one kernel class
    (uno_set_timing_events), on the stream each launch uses."""

    def __init__(self, kernel_class, n):
        self.lib = load_library()
        self.hip = ctypes.CDLL("libamdhip64.so")
        self.hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                                 ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.n = n
        self.kernel_class = kernel_class
        self.start = (ctypes.c_void_p * n)()
        self.stop = (ctypes.c_void_p * n)()
        for arr in (self.start, self.stop):
            for i in range(n):
                ev = ctypes.c_void_p()
                if self.hip.hipEventCreate(ctypes.byref(ev)) != 0:
                    raise UnoError("hipEventCreate failed")
                arr[i] = ev.value

    def arm(self):
        _check(self.lib.uno_set_timing_events(self.kernel_class, self.start, self.stop, self.n))

    def disarm(self):
        used = self.lib.uno_timing_events_used()
        _check(self.lib.uno_set_timing_events(0, None, None, 0))
        return used

    def durations_ms(self, used):
        """Elapsed ms of the first `used` bracketed launches (stream synchronised)."""
        out = []
        for i in range(used):
            ms = ctypes.c_float()
            if self.hip.hipEventElapsedTime(ctypes.byref(ms), self.start[i], self.stop[i]) != 0:
                raise UnoError("hipEventElapsedTime failed")
            out.append(ms.value)
        return out

    def close(self):
        for arr in (self.start, self.stop):
            for i in range(self.n):
                if arr[i]:
                    self.hip.hipEventDestroy(arr[i])
                    arr[i] = None
