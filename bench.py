"""Throughput of the Psi-Spec draft-and-verify decode step on one MI355X.

Workload (default): Qwen3-8B-shaped random-init bf16 model (36 layers, d_model
4096, 32 q / 8 kv heads x 128, SwiGLU 12288, vocab 151936, LoRA rank 128
alpha 256 on all seven linears), batch 64, per-sequence context 9216 in 16-token
pages with a seeded page permutation, block K = 16, temperature 1.  Each step
is draft block (36 layers, AR + LoRA) -> draft sampling -> verify block (36
layers, AR) -> accept / resample -> KV commit, entirely device resident.  As in
the pages' fixed-length throughput test, each step commits a forced number of
drafts a ~ U{0..16} per sequence (staggered, exercising ragged commit and
rollback); accepted tokens per step = sum_b (a_b + 1).  KV content and weights
are seeded synthetic data.

Prints one JSON line.  `roofline` covers the single kernel that takes the most
time per step (block attention at this workload; the per-class totals come from
an untimed probe step), timed with HIP events that the library records around
each of its launches inside the timed region: achieved = the algorithmic bytes
of those launches (every cached K/V entry the block's rows may see, read once,
plus q in and the output out) / their summed duration.  `traffic` is the HBM
traffic per launch that rocprofv3 counters measured for the same kernel source
(FETCH_SIZE + WRITE_SIZE, scaled by the factor the same counters give for a
plain copy of known size, `--calibrate-copy`), or null when the kernel source
has changed since.  `roofline_gemm` is the MFMA fraction of the projection
GEMMs of both passes (flops / their probe-step time).  `verify_step` is the
verify pass as a whole (36 layers + LM head, timed with torch events around it
in every timed step): its algorithmic HBM bytes (every AR weight once, every
cached K/V entry the rows may see once per layer, the block's own K/V written,
the fp32 logits written) / its summed duration.  `cpu_baseline` times the CPU
oracle on a bounded sample of the same workload.
"""
import hashlib
import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
BF16_PEAK_TFLOPS = 2500.0

# HBM traffic of the attention kernel from rocprofv3 counters (see the
# attention profile summary under profiles/): mean FETCH_SIZE and WRITE_SIZE per
# dispatch, scaled by the copy calibration factor, for the kernel source with
# this digest.
ATTN_TRAFFIC = {"source": "273908c7a7243788", "bytes_per_launch": 2460721323,
                "fetch_kib": 1196956.93, "write_kib": 9216.01, "fetch_factor": 1.99993, "write_factor": 1.0}
ATTN_SOURCES = ["lossless_decoding_uno_amd/csrc/attention.hip",
                "lossless_decoding_uno_amd/csrc/uno_device.h"]


def attn_source_digest():
    h = hashlib.sha256()
    for rel in ATTN_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--batch", type=int, default=64)
    ap.add_argument("--ctx", type=int, default=9216)
    ap.add_argument("--K", type=int, default=16)
    ap.add_argument("--temp", type=float, default=1.0, help="sampling temperature")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-secondary", action="store_true")
    ap.add_argument("--no-long", action="store_true",
                    help="skip the long-context lines (batch 16, context 32768, K 32)")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run a plain 1 GiB device copy three times (counter calibration)")
    ap.add_argument("--generate", type=int, default=0, metavar="N",
                    help="end-to-end mode: prefill a --prompt-token prompt per sequence, then "
                         "generate N tokens with natural acceptance (pages on demand)")
    ap.add_argument("--prompt", type=int, default=1024)
    ap.add_argument("--prior", type=int, default=0, help="draft noise prior: 0 mask, 1 uniform")
    ap.add_argument("--passes", type=int, default=1, help="draft passes per step (generate mode)")
    ap.add_argument("--kappa", type=float, default=1.0,
                    help="corrector strength between draft passes (generate mode)")
    ap.add_argument("--tree", type=str, default="", metavar="TOPK,NKEEP",
                    help="tree-sampler mode: steps of draft -> tree build (top-TOPK per drafted "
                         "position, best NKEEP candidates) -> tree verify -> walk -> commit, "
                         "natural acceptance (prints its own JSON line)")
    return ap.parse_args()


def log(msg):
    print("[bench] " + msg, file=sys.stderr, flush=True)


class Workload:
    """Device state of one (batch, context, K) decode workload."""

    def __init__(self, U, torch, synth, model, cfg, B, ctx, K, n_steps, seed, temp=1.0):
        self.U, self.torch = U, torch
        self.inv_t = float(np.float32(1.0 / temp))
        self.B, self.ctx, self.K = B, ctx, K
        self.cfg = cfg
        dev = "cuda"
        self.capacity = ctx + n_steps * (K + 1) + K + 2
        n_pages_seq = (self.capacity + 15) // 16
        n_pages = B * n_pages_seq
        perm = torch.randperm(n_pages, generator=torch.Generator().manual_seed(seed))
        self.kv = U.PagedKV(cfg, B, self.capacity, page_order=perm)
        synth.fill_kv_device(self.kv.k_pages, self.kv.v_pages, seed)
        self.kv.kv_len.fill_(ctx)
        self.max_ctx = self.capacity
        V = cfg["vocab"]
        self.ws = U.alloc_workspace(U.workspace_bytes(model, B, K, self.max_ctx))
        self.aws = U.alloc_workspace(U.spec_accept_workspace_bytes(B, K))
        self.zq = torch.empty((B, K, V), dtype=torch.float32, device=dev)
        self.zp = torch.empty((B, K, V), dtype=torch.float32, device=dev)
        self.d = torch.empty((B, K), dtype=torch.int32, device=dev)
        # exact row maxima of the draft / verify logits, written by the LM head
        self.qmax = torch.empty((B, K), dtype=torch.float32, device=dev)
        self.pmax = torch.empty((B, K), dtype=torch.float32, device=dev)
        self.a = torch.empty(B, dtype=torch.int32, device=dev)
        self.c = torch.empty((B, K + 1), dtype=torch.int32, device=dev)
        self.e = torch.from_numpy(synth.prompt_ids(cfg, B, seed)).to(dev)   # first anchors
        self.step_ctr = torch.zeros(B, dtype=torch.uint64).to(dev)
        # device-side fault flags of every call; checked after the timed region
        self.status = torch.zeros(B, dtype=torch.int32, device=dev)
        self.forced_host = synth.forced_accepts(B, K, n_steps, seed=2)
        self.forced = torch.from_numpy(self.forced_host).to(dev)
        self.kv_len_host = np.full(B, ctx, dtype=np.int64)
        self.model = model

    def step(self, i, verify_events=None):
        U = self.U
        U.draft_block(self.model, self.kv, self.e, self.K, self.max_ctx, self.inv_t, 0, self.step_ctr,
                      self.zq, self.d, self.ws, self.status, row_max=self.qmax)
        if verify_events is not None:
            verify_events[0].record()
        U.verify_block(self.model, self.kv, self.d, self.max_ctx, 1, self.zp, self.ws, self.status,
                       row_max=self.pmax)
        if verify_events is not None:
            verify_events[1].record()
        U.spec_accept(self.zq, self.zp, self.d, self.inv_t, 0, self.step_ctr, self.a, self.c, self.e,
                      self.aws, forced_accept=self.forced[i], status=self.status,
                      draft_row_max=self.qmax, verify_row_max=self.pmax)
        U.kv_commit(self.kv, self.a, self.K, self.step_ctr, self.status)

    def check_status(self):
        """No call raised a device fault flag (outside any timed region)."""
        st = self.status.cpu().numpy()
        assert (st == 0).all(), "device status flags raised: %s" % np.unique(st).tolist()

    def attn_bytes(self, i):
        """Algorithmic bytes of the two attention launches of one layer at step i:
        every cached K/V entry a row may see (read once), q in, out written."""
        cfg = self.cfg
        per_tok = 2 * cfg["n_kv_heads"] * cfg["head_dim"] * 2
        qo = 2 * self.B * self.K * cfg["n_q_heads"] * cfg["head_dim"] * 2
        kl = self.kv_len_host
        draft = int(np.sum(kl + self.K)) * per_tok + qo
        verify = int(np.sum(kl + 1 + self.K)) * per_tok + qo
        return draft, verify

    def advance_host(self, i):
        self.kv_len_host += self.forced_host[i].astype(np.int64) + 1

    def verify_bytes(self):
        """Algorithmic HBM bytes of the verify pass at the current kv_len: every
        AR weight once (layers + LM head), every cached K/V entry the rows may
        see once per layer, the block's own K/V written, the logits written."""
        cfg = self.cfg
        D, F, V = cfg["d_model"], cfg["d_ffn"], cfg["vocab"]
        qd = cfg["n_q_heads"] * cfg["head_dim"]
        kd = cfg["n_kv_heads"] * cfg["head_dim"]
        per_layer_w = 2 * (D * (qd + 2 * kd) + qd * D + 2 * F * D + F * D)
        weights = cfg["n_layers"] * per_layer_w + 2 * V * D
        per_tok = cfg["n_kv_heads"] * cfg["head_dim"] * 2 * 2          # K and V, one layer
        kv_read = cfg["n_layers"] * int(np.sum(self.kv_len_host + 1 + self.K)) * per_tok
        kv_write = cfg["n_layers"] * self.B * self.K * per_tok
        logits = self.B * self.K * V * 4
        return weights + kv_read + kv_write + logits


def gemm_flops_per_pass(cfg, R, draft):
    D, F = cfg["d_model"], cfg["d_ffn"]
    qd = cfg["n_q_heads"] * cfg["head_dim"]
    kd = cfg["n_kv_heads"] * cfg["head_dim"]
    r = cfg["lora_rank"]
    per_layer = (qd + 2 * kd) * D + D * qd + 2 * F * D + D * F
    if draft:    # LoRA B product fused as r extra K steps on every output column
        per_layer += (qd + 2 * kd + D + 2 * F + D) * r
    return 2.0 * R * per_layer * cfg["n_layers"]


def measured_ceilings(torch):
    """Ceilings measured on this GPU with the probe kernels of libuno_probe.so
    (include/uno_probe.h), beside the vendor peaks: a streaming read of a cold
    4 GiB buffer (16x the last-level cache) with 16-byte loads, plain and
    non-temporal, four or eight in flight per lane; a 1 GiB -> 1 GiB copy
    (bytes read + written); a register-only loop of v_mfma_f32_32x32x16_bf16.
    Each is the best of three runs at its best grid size of a small sweep."""
    import ctypes
    lib = ctypes.CDLL(os.path.join(ROOT, "lossless_decoding_uno_amd", "libuno_probe.so"))
    P, SZ, I = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int
    lib.uno_probe_read.argtypes = [P, SZ, I, I, P, P]
    lib.uno_probe_copy.argtypes = [P, P, SZ, I, P]
    lib.uno_probe_mfma.argtypes = [I, I, P, P]
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    big = torch.empty(1 << 32, dtype=torch.uint8, device="cuda")
    sink = torch.empty(1 << 16, dtype=torch.float32, device="cuda")
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]

    def best_ms(launch, reps=3):
        launch()
        torch.cuda.synchronize()
        best = 1e30
        for _ in range(reps):
            ev[0].record()
            launch()
            ev[1].record()
            torch.cuda.synchronize()
            best = min(best, ev[0].elapsed_time(ev[1]))
        return best

    out = {}
    for nt, key in ((1, "read_nontemporal_GBps"), (0, "read_GBps")):
        rate = 0.0
        for depth in (0, 2):                 # four or eight loads in flight per lane
            for n_wg in (2048, 4096, 8192, 16384):
                ms = best_ms(lambda: lib.uno_probe_read(
                    ctypes.c_void_p(big.data_ptr()), big.numel(), nt | depth, n_wg,
                    ctypes.c_void_p(sink.data_ptr()), stream))
                rate = max(rate, big.numel() / (ms / 1e3) / 1e9)
        out[key] = round(rate, 1)
    half = big.numel() // 2
    rate = 0.0
    for n_wg in (4096, 16384):
        ms = best_ms(lambda: lib.uno_probe_copy(ctypes.c_void_p(big.data_ptr()),
                                                ctypes.c_void_p(big.data_ptr() + half), half // 2,
                                                n_wg, stream))
        rate = max(rate, 2 * (half // 2) / (ms / 1e3) / 1e9)
    out["copy_GBps"] = round(rate, 1)
    del big
    rate, iters = 0.0, 400
    for n_wg in (256, 512, 1024, 2048):
        ms = best_ms(lambda: lib.uno_probe_mfma(iters, n_wg, ctypes.c_void_p(sink.data_ptr()),
                                                stream))
        rate = max(rate, n_wg * 4 * iters * 4 * 32768 / (ms / 1e3) / 1e12)
    out["mfma_bf16_TFLOPs"] = round(rate, 1)
    torch.cuda.empty_cache()
    return out


def library_gemm_reference(torch, cfg, R):
    """ms per step that torch.matmul (hipBLASLt) takes for the same four
    projection shapes (both passes, no LoRA), for comparison."""
    total = 0.0
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    for name in ("gemm_qkv", "gemm_o", "gemm_gate_up", "gemm_down"):
        N, Kd, _ = proj_shape(cfg, name)
        x = torch.randn(R, Kd, device="cuda", dtype=torch.bfloat16)
        w = torch.randn(N, Kd, device="cuda", dtype=torch.bfloat16)
        for _ in range(3):
            torch.matmul(x, w.t())
        torch.cuda.synchronize()
        ev[0].record()
        for _ in range(10):
            torch.matmul(x, w.t())
        ev[1].record()
        torch.cuda.synchronize()
        total += ev[0].elapsed_time(ev[1]) / 10
        del x, w
    torch.cuda.empty_cache()
    return round(total * 2 * cfg["n_layers"], 3)


def run_timed(W, steps, warmup, torch, timer=None):
    for i in range(warmup):
        W.step(i)
        W.advance_host(i)
    torch.cuda.synchronize()
    kv0 = W.kv_len_host.copy()
    if timer is not None:
        timer.arm()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    t0.record()
    attn_bytes = []
    vev, vbytes = [], 0
    for i in range(warmup, warmup + steps):
        db, vb = W.attn_bytes(i)
        attn_bytes += [db] * W.cfg["n_layers"] + [vb] * W.cfg["n_layers"]
        vbytes += W.verify_bytes()
        ev = (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
        vev.append(ev)
        W.step(i, ev)
        W.advance_host(i)
    t1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    used = timer.disarm() if timer is not None else 0
    ms = t0.elapsed_time(t1)
    W.verify_ms = sum(a.elapsed_time(b) for a, b in vev)
    W.verify_bytes_total = vbytes
    tokens = int(np.sum(W.forced_host[warmup:warmup + steps].astype(np.int64) + 1))
    got = W.kv.kv_len.cpu().numpy()
    assert np.array_equal(got, W.kv_len_host), "device kv_len diverged from the forced schedule"
    W.check_status()
    return ms, wall, tokens, used, attn_bytes, kv0


CLASSES = ["attention", "gemm_qkv", "gemm_o", "gemm_gate_up", "gemm_down", "lora_a", "lm_head",
           "sampler"]


def class_ids(U):
    return {"attention": U.TIME_ATTENTION, "gemm_qkv": U.TIME_GEMM_QKV, "gemm_o": U.TIME_GEMM_O,
            "gemm_gate_up": U.TIME_GEMM_GATE_UP, "gemm_down": U.TIME_GEMM_DOWN,
            "lora_a": U.TIME_LORA_A, "lm_head": U.TIME_LM_HEAD, "sampler": U.TIME_SAMPLER}


def probe_classes(U, W, i, torch):
    """Untimed: total ms per kernel launch site over one step (one class per rerun)."""
    totals = {}
    ids = class_ids(U)
    for name in CLASSES:
        timer = U.KernelTimer(ids[name], 400)
        kv_save = W.kv.kv_len.clone()
        step_save = W.step_ctr.clone()
        e_save = W.e.clone()
        torch.cuda.synchronize()
        timer.arm()
        W.step(i)
        used = timer.disarm()
        torch.cuda.synchronize()
        totals[name] = float(sum(timer.durations_ms(used)))
        timer.close()
        W.kv.kv_len.copy_(kv_save)
        W.step_ctr.copy_(step_save)
        W.e.copy_(e_save)
    torch.cuda.synchronize()
    return totals


def proj_shape(cfg, name):
    """(output columns N, reduction length Kd, output bytes per element) of a projection."""
    D, F = cfg["d_model"], cfg["d_ffn"]
    qd = cfg["n_q_heads"] * cfg["head_dim"]
    kd = cfg["n_kv_heads"] * cfg["head_dim"]
    return {"gemm_qkv": (qd + 2 * kd, D, 4), "gemm_o": (D, qd, 8), "gemm_gate_up": (2 * F, D, 4),
            "gemm_down": (D, F, 8), "lm_head": (cfg["vocab"], D, 4)}[name]


def sampler_roofline(cfg, B, K, ms, read_ceiling):
    """The sampler launches of one step (draft sampling, acceptance statistics,
    accept / resample) against HBM: algorithmic bytes = the fp32 draft logits
    read once to sample the drafts, then the draft and verify logits read once
    each to accept / resample (3 * B * K * V * 4), over their probe-step time.
    The row maxima come from the LM head (its class holds the reduction of
    their per-tile partials), so each row is streamed once per kernel."""
    byts = 3.0 * B * K * cfg["vocab"] * 4
    gbs = byts / (ms / 1e3) / 1e9
    return {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(gbs / HBM_PEAK_GBS, 4),
            "frac_of_measured": round(gbs / read_ceiling, 4), "ms_per_step": round(ms, 3),
            "algorithmic_bytes_per_step": int(byts)}


def gemm_launch_work(cfg, name, R, draft):
    """Algorithmic (flops, bytes) of one launch: every weight (and, drafting, LoRA B
    and the LoRA input T) read once, X read once, the output written (and read,
    for the residual adds)."""
    N, Kd, ob = proj_shape(cfg, name)
    r = cfg["lora_rank"] if (draft and name != "lm_head") else 0
    flops = 2.0 * R * N * (Kd + r)
    byts = 2.0 * N * (Kd + r) + 2.0 * R * (Kd + r) + ob * R * N
    return flops, byts
def host_description():
    """The host the CPU baseline ran on: CPU model, logical CPUs, and the
    thread counts of the BLAS numpy calls and of torch."""
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    blas = []
    try:
        import threadpoolctl
        blas = [{"api": p.get("internal_api"), "threads": p.get("num_threads")}
                for p in threadpoolctl.threadpool_info()]
    except Exception:
        pass
    import torch
    return {"cpu_model": model, "logical_cpus": os.cpu_count(),
            "affinity_cpus": len(os.sched_getaffinity(0)),
            "OMP_NUM_THREADS": os.environ.get("OMP_NUM_THREADS"),
            "numpy_blas": blas, "torch_threads": int(torch.get_num_threads())}


def cpu_baseline(K, ctx, forced_mean_tokens):
    """The oracle (fp64 model, exact-integer sampler) on one sequence of the
    workload: a whole step (best of two) with 1 and with 5 layers of the 8B
    shape (full LM head, context `ctx` of synthetic cache), extrapolated
    linearly to 36 layers."""
    import torch
    import synth
    from oracle import spec as ospec
    cfg = synth.QWEN3_8B
    times = {}
    for L in (1, 5):
        c = dict(cfg, n_layers=L)
        w = synth.to_f64(synth.make_weights(c, seed=5))
        prompt = synth.prompt_ids(c, ctx + 1, 3)
        k, v = synth.kv_values(c, ctx, seed=4)
        best = None
        for rep in range(2):
            seq = ospec.Sequence(c, prompt, capacity=ctx + 2 * K + 4)
            for li in range(L):
                seq.cache.k[li][:ctx] = k[li].double().numpy()
                seq.cache.v[li][:ctx] = v[li].double().numpy()
            seq.kv_len = ctx
            t = time.perf_counter()
            ospec.step(c, w, seq, K, 1.0, ospec.PhiloxDraws(0, 0, 0), forced=K // 2)
            dt = time.perf_counter() - t
            best = dt if best is None else min(best, dt)
        times[L] = best
        del w
    per_layer = max((times[5] - times[1]) / 4.0, 1e-9)
    t36 = times[1] + (cfg["n_layers"] - 1) * per_layer
    return {"value": forced_mean_tokens / t36, "unit": "accepted tokens/s",
            "cores": int(torch.get_num_threads()), "kind": "oracle", "host": host_description(),
            "sample": ("one sequence of the workload, one full step (draft+sample+verify+accept+"
                       "commit) at context %d, K=%d, timed with 1 and 5 of the 36 layers "
                       "(%.2f s, %.2f s; best of 2), extrapolated linearly to 36 layers "
                       "(%.2f s/step); %.1f accepted tokens per step (the forced schedule's mean)"
                       % (ctx, K, times[1], times[5], t36, forced_mean_tokens))}


def generate_mode(args, U, synth, torch, cfg):
    """Chunked prefill of random prompts, then continuous Psi-Spec steps with
    natural acceptance until every sequence has args.generate new tokens."""
    from lossless_decoding_uno_amd.generate import Generator
    K = args.K
    log("generating weights on the GPU")
    model = U.Model(cfg, synth.make_weights_device(cfg, seed=0))
    tree = tuple(int(x) for x in args.tree.split(",")) if args.tree else None
    extra = U.tree_rows(K, *tree) if tree else K
    max_ctx = args.prompt + args.generate + 2 * K + extra + 8
    g = Generator(model, args.batch, K, max_ctx, seed=0, prefill_chunk=512, n_passes=args.passes,
                  kappa=args.kappa,
                  tree=tree)
    prompts = synth.prompt_ids(cfg, args.prompt, 1, batch=args.batch)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    g.prefill(prompts)
    torch.cuda.synchronize()
    t_prefill = time.perf_counter() - t0
    log("prefill done in %.2f s; generating %d tokens" % (t_prefill, args.generate))
    t0 = time.perf_counter()
    last = [t0]

    def progress():
        if time.perf_counter() - last[0] > 30:
            last[0] = time.perf_counter()
            log("%d steps, %d tokens" % (g.steps, min(len(o) for o in g.out)))

    outs = g.generate(args.generate, on_step=progress)
    torch.cuda.synchronize()
    t_gen = time.perf_counter() - t0
    st_flags = g.status.cpu().numpy()
    assert (st_flags == 0).all(), "device status flags raised: %s" % np.unique(st_flags).tolist()
    st = g.stats()
    toks = sum(len(o) for o in outs)
    out = {"metric": "generated tokens/s (natural acceptance, end to end)",
           "value": round(toks / t_gen, 1), "unit": "tokens/s", "n_gpus": 1,
           "higher_is_better": True, "dtype": "bf16",
           "data": "synthetic (random-init weights, uniform random prompts)",
           "config": {"workload": "qwen3-8b-shape b%d prompt%d gen%d K%d natural prior%d passes%d "
                                  "kappa%g%s" % (
               args.batch, args.prompt, args.generate, K, args.prior, args.passes, args.kappa,
               " tree topk%d keep%d" % tree if tree else "")},
           "steps": st["steps"], "TPF": round(st["TPF"], 3), "AL": round(st["AL"], 3),
           "ms_per_step": round(1e3 * t_gen / st["steps"], 3),
           "prefill_s": round(t_prefill, 3), "pages_in_use": st["pages_in_use"]}
    print(json.dumps(out), flush=True)


class TreeWorkload:
    """Device state of a tree-sampler workload (batch, context, block K, topk, n_keep)."""

    def __init__(self, U, torch, synth, model, cfg, B, ctx, K, topk, n_keep, n_steps, seed,
                 temp=1.0):
        self.U, self.torch, self.cfg, self.model = U, torch, cfg, model
        self.inv_t = float(np.float32(1.0 / temp))
        self.B, self.ctx, self.K = B, ctx, K
        V = cfg["vocab"]
        dev = "cuda"
        self.tb = U.TreeBuffers(B, K, topk, n_keep, V)
        N = self.tb.N
        self.capacity = ctx + n_steps * (K + 1) + N + 2
        perm = torch.randperm(B * ((self.capacity + 15) // 16),
                              generator=torch.Generator().manual_seed(seed))
        self.kv = U.PagedKV(cfg, B, self.capacity, page_order=perm)
        synth.fill_kv_device(self.kv.k_pages, self.kv.v_pages, seed)
        self.kv.kv_len.fill_(ctx)
        self.max_ctx = self.capacity
        self.ws = U.alloc_workspace(max(U.workspace_bytes(model, B, K, self.max_ctx),
                                        U.workspace_bytes(model, B, N, self.max_ctx)))
        self.zq = torch.empty((B, K, V), dtype=torch.float32, device=dev)
        self.zp = torch.empty((B, N, V), dtype=torch.float32, device=dev)
        self.d = torch.empty((B, K), dtype=torch.int32, device=dev)
        self.a = torch.empty(B, dtype=torch.int32, device=dev)
        self.c = torch.empty((B, K + 1), dtype=torch.int32, device=dev)
        self.e = torch.from_numpy(synth.prompt_ids(cfg, B, seed)).to(dev)
        self.step_ctr = torch.zeros(B, dtype=torch.uint64).to(dev)
        self.status = torch.zeros(B, dtype=torch.int32, device=dev)

    def step(self, i):
        U = self.U
        U.draft_block(self.model, self.kv, self.e, self.K, self.max_ctx, self.inv_t, 0,
                      self.step_ctr, self.zq, self.d, self.ws, self.status)
        U.tree_build(self.zq, self.d, self.tb, self.status)
        U.verify_tree(self.model, self.kv, self.tb, self.max_ctx, self.zp, self.ws, self.status)
        U.tree_accept(self.zp, self.tb, self.inv_t, 0, self.step_ctr, self.a, self.c, self.e,
                      self.status)
        U.tree_commit(self.model, self.kv, self.tb, self.a, self.step_ctr, self.status)


def tree_mode(args, U, synth, torch, cfg):
    """Steps of the tree sampler with natural acceptance; tokens per step are
    read from the growth of kv_len after the timed region (1 + a per
    sequence and step)."""
    topk, n_keep = (int(x) for x in args.tree.split(","))
    K = args.K
    log("generating weights on the GPU")
    model = U.Model(cfg, synth.make_weights_device(cfg, seed=0))
    W = TreeWorkload(U, torch, synth, model, cfg, args.batch, args.ctx, K, topk, n_keep,
                     args.warmup + args.steps + 1, seed=1, temp=args.temp)
    log("tree rows per sequence: %d; probe step" % W.tb.N)
    W.step(0)
    torch.cuda.synchronize()
    classes = probe_classes(U, W, 0, torch)
    log("class ms per step: %s" % json.dumps({k: round(v, 3) for k, v in classes.items()}))
    for i in range(args.warmup):
        W.step(i)
    torch.cuda.synchronize()
    kv0 = W.kv.kv_len.cpu().numpy().astype(np.int64)
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record()
    for i in range(args.steps):
        W.step(args.warmup + i)
    t1.record()
    torch.cuda.synchronize()
    ms = t0.elapsed_time(t1)
    tokens = int(np.sum(W.kv.kv_len.cpu().numpy().astype(np.int64) - kv0))
    st = W.status.cpu().numpy()
    assert (st == 0).all(), "device status flags raised: %s" % np.unique(st).tolist()
    # projection GEMMs of both passes against HBM: every weight read once per pass
    L = cfg["n_layers"]
    gemm_ms = sum(classes[k] for k in ("gemm_qkv", "gemm_o", "gemm_gate_up", "gemm_down"))
    wbytes = 0.0
    for name in ("gemm_qkv", "gemm_o", "gemm_gate_up", "gemm_down"):
        wbytes += L * (gemm_launch_work(cfg, name, args.batch * K, True)[1] +
                       gemm_launch_work(cfg, name, args.batch * W.tb.N, False)[1])
    out = {"metric": "accepted tokens/s/GPU (Qwen3-8B shape, Psi-Spec tree sampler step, "
                     "natural acceptance)",
           "value": round(tokens / (ms / 1e3), 1), "unit": "accepted tokens/s", "n_gpus": 1,
           "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms / args.steps, 3),
           "higher_is_better": True, "dtype": "bf16",
           "data": "synthetic (seeded random-init weights and KV; natural acceptance of a "
                   "random model, so acceptance is near its floor)",
           "config": {"workload": "qwen3-8b-shape b%d ctx%d K%d tree topk%d keep%d T%g natural"
                      % (args.batch, args.ctx, K, topk, n_keep, args.temp),
                      "tree_rows": W.tb.N},
           "AL": round(tokens / (args.steps * args.batch), 3),
           "roofline_gemm": {"bound": "hbm", "achieved": round(wbytes / (gemm_ms / 1e3) / 1e9, 1),
                             "peak": HBM_PEAK_GBS, "unit": "GB/s",
                             "frac": round(wbytes / (gemm_ms / 1e3) / 1e9 / HBM_PEAK_GBS, 4),
                             "kernel": "k_gemm: projections of the draft and tree-verify passes",
                             "ms_per_step": round(gemm_ms, 3)},
           "kernel_class_ms_per_step": {k: round(v, 3) for k, v in classes.items()}}
    print(json.dumps(out), flush=True)


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path (the batch would "
              "shard by sequence with no per-step communication); run with --gpus 1",
              file=sys.stderr)
        sys.exit(2)
    import torch
    if args.calibrate_copy:
        n = 1 << 30
        src = torch.ones(n // 4, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"calibrate_copy_bytes_per_launch": n, "launches": 3}), flush=True)
        return
    import lossless_decoding_uno_amd as U
    import synth
    U.load_library()
    assert torch.cuda.is_available(), "no GPU"
    cfg = dict(synth.QWEN3_8B, noise_prior=args.prior)
    if args.generate:                       # with --tree: end-to-end with the tree sampler
        return generate_mode(args, U, synth, torch, cfg)
    if args.tree:
        return tree_mode(args, U, synth, torch, cfg)
    K = args.K
    log("generating weights on the GPU")
    model = U.Model(cfg, synth.make_weights_device(cfg, seed=0))
    torch.cuda.synchronize()
    n_steps = args.warmup + args.steps + 1
    log("allocating KV for batch %d context %d" % (args.batch, args.ctx))
    W = Workload(U, torch, synth, model, cfg, args.batch, args.ctx, K, n_steps, seed=1,
                 temp=args.temp)
    torch.cuda.synchronize()
    log("probe step (per-kernel-class times)")
    W.step(0)
    torch.cuda.synchronize()
    W.kv.kv_len.fill_(args.ctx)
    W.step_ctr.copy_(torch.zeros(args.batch, dtype=torch.uint64))
    classes = probe_classes(U, W, 0, torch)
    log("class ms per step: %s" % json.dumps({k: round(v, 3) for k, v in classes.items()}))
    dominant = max(CLASSES, key=lambda k: classes[k])
    L = cfg["n_layers"]
    per_step = {"attention": 2 * L, "gemm_qkv": 2 * L, "gemm_o": 2 * L, "gemm_gate_up": 2 * L,
                "gemm_down": 2 * L, "lora_a": 4 * L, "lm_head": 2, "sampler": 2}[dominant]
    timer = U.KernelTimer(class_ids(U)[dominant], per_step * args.steps)
    log("timed region: %d steps after %d warmup (dominant kernel: %s)" % (args.steps, args.warmup,
                                                                        dominant))
    ms, wall, tokens, used, attn_bytes, kv0 = run_timed(W, args.steps, args.warmup, torch, timer)
    durs = np.array(timer.durations_ms(used))
    timer.close()
    ms_step = ms / args.steps
    value = tokens / (ms / 1e3)
    R = args.batch * K
    avg_us = round(float(durs.mean()) * 1e3, 2)
    if dominant == "attention":
        achieved = float(np.sum(attn_bytes[:used])) / (durs.sum() / 1e3) / 1e9
        traffic = None
        if ATTN_TRAFFIC is not None and ATTN_TRAFFIC["source"] == attn_source_digest():
            traffic = ATTN_TRAFFIC["bytes_per_launch"]
        roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic,
                "kernel": "k_attention (block attention, split-KV partials)", "launches": int(used),
                "avg_launch_us": avg_us,
                "algorithmic_bytes_per_launch": round(float(np.mean(attn_bytes[:used])))}
    elif dominant.startswith("gemm") or dominant == "lm_head":
        # launches alternate draft pass (L layers) / verify pass (L layers) per step
        work = [gemm_launch_work(cfg, dominant, R, (k // (per_step // 2)) % 2 == 0)
                for k in range(used)]
        fl = sum(w[0] for w in work)
        by = sum(w[1] for w in work)
        t = durs.sum() / 1e3
        if fl / by > BF16_PEAK_TFLOPS * 1e12 / (HBM_PEAK_GBS * 1e9):
            roof = {"bound": "mfma", "achieved": round(fl / t / 1e12, 1), "peak": BF16_PEAK_TFLOPS,
                    "unit": "TFLOP/s", "frac": round(fl / t / 1e12 / BF16_PEAK_TFLOPS, 4)}
        else:
            roof = {"bound": "hbm", "achieved": round(by / t / 1e9, 1), "peak": HBM_PEAK_GBS,
                    "unit": "GB/s", "frac": round(by / t / 1e9 / HBM_PEAK_GBS, 4)}
        roof.update({"traffic": None, "kernel": "k_gemm (%s)" % dominant, "launches": int(used),
                     "avg_launch_us": avg_us})
    else:
        roof = {"bound": "hbm", "achieved": None, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": None, "traffic": None, "kernel": dominant, "launches": int(used),
                "avg_launch_us": avg_us}
    log("measured ceilings (probe kernels)")
    ceil = measured_ceilings(torch)
    if roof.get("achieved") is not None:
        c = ceil["read_nontemporal_GBps"] if roof["bound"] == "hbm" else ceil["mfma_bf16_TFLOPs"]
        roof["frac_of_measured"] = round(roof["achieved"] / c, 4)
    # MFMA fraction of the projection GEMMs (both passes) from the probe step
    gemm_ms = sum(classes[k] for k in ("gemm_qkv", "gemm_o", "gemm_gate_up", "gemm_down"))
    gfl = gemm_flops_per_pass(cfg, R, True) + gemm_flops_per_pass(cfg, R, False)
    vfl = gemm_flops_per_pass(cfg, R, False)
    roof_gemm = {"bound": "mfma", "achieved": round(gfl / (gemm_ms / 1e3) / 1e12, 1),
                 "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                 "frac": round(gfl / (gemm_ms / 1e3) / 1e12 / BF16_PEAK_TFLOPS, 4),
                 "ms_per_step": round(gemm_ms, 3), "flop_per_step": gfl,
                 "verify_flop_per_step": vfl,
                 "kernel": "k_gemm: q|k|v, o, gate|up, down projections of both passes",
                 "torch_matmul_ms_per_step": library_gemm_reference(torch, cfg, R)}
    roof_gemm["frac_of_measured"] = round(roof_gemm["achieved"] / ceil["mfma_bf16_TFLOPs"], 4)
    out = {"metric": "accepted tokens/s/GPU (Qwen3-8B shape, Psi-Spec draft+verify step)",
           "value": round(value, 1), "unit": "accepted tokens/s", "n_gpus": 1,
           "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_step, 3),
           "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
           "data": "synthetic (seeded random-init weights and KV, forced accept lengths)",
           "config": {"workload": "qwen3-8b-shape b%d ctx%d K%d T%g forced a~U{0..%d}" % (
               args.batch, args.ctx, K, args.temp, K), "global_batch": args.batch,
               "seq_len": args.ctx, "block_K": K, "temperature": args.temp,
               "parallelism": "none (1 GPU)"},
           "roofline": roof,
           "roofline_gemm": roof_gemm,
           "measured_ceilings": ceil,
           "verify_step": {"ms_per_step": round(W.verify_ms / args.steps, 3),
                           "hbm_GBps": round(W.verify_bytes_total / (W.verify_ms / 1e3) / 1e9, 1),
                           "frac_of_8TBps": round(W.verify_bytes_total / (W.verify_ms / 1e3) / 1e9
                                                  / HBM_PEAK_GBS, 4),
                           "frac_of_measured": round(W.verify_bytes_total / (W.verify_ms / 1e3)
                                                     / 1e9 / ceil["read_nontemporal_GBps"], 4),
                           "algorithmic_GB_per_step": round(W.verify_bytes_total / args.steps / 1e9, 3)},
           "sampler": sampler_roofline(cfg, args.batch, K, classes["sampler"],
                                       ceil["read_nontemporal_GBps"]),
           "kernel_class_ms_per_step": {k: round(v, 3) for k, v in classes.items()},
           "forward_passes_per_s": round(2 * args.steps / (ms / 1e3), 2),
           "wall_s_timed": round(wall, 3)}
    del W
    torch.cuda.empty_cache()
    if not args.no_secondary:
        # batch 1 at the two contexts the single-sequence workload is quoted at
        for key, ctx1 in (("secondary", 1024), ("secondary_ctx9216", 9216)):
            log("%s: batch 1, context %d" % (key, ctx1))
            W1 = Workload(U, torch, synth, model, cfg, 1, ctx1, K, 40 + 6, seed=7)
            ms1, _, tok1, _, _, _ = run_timed(W1, 40, 5, torch)
            out[key] = {"workload": "qwen3-8b-shape b1 ctx%d K%d forced" % (ctx1, K),
                        "value": round(tok1 / (ms1 / 1e3), 1), "unit": "accepted tokens/s",
                        "ms_per_step": round(ms1 / 40, 3),
                        "verify_step_hbm_GBps": round(W1.verify_bytes_total /
                                                      (W1.verify_ms / 1e3) / 1e9, 1),
                        "verify_ms_per_step": round(W1.verify_ms / 40, 3)}
            del W1
    if not args.no_long:
        # the long-context rollout shape, at temperature 0.7 and 1.0
        Kl, ctxl, Bl = 32, 32768, 16
        lines = []
        for temp in (0.7, 1.0):
            log("long context: batch %d, context %d, K %d, temperature %g" % (Bl, ctxl, Kl, temp))
            WL = Workload(U, torch, synth, model, cfg, Bl, ctxl, Kl, 8 + 3, seed=9, temp=temp)
            msl, _, tokl, _, abl, _ = run_timed(WL, 8, 2, torch)
            lines.append({"workload": "qwen3-8b-shape b%d ctx%d K%d T%g forced a~U{0..%d}"
                                      % (Bl, ctxl, Kl, temp, Kl),
                          "value": round(tokl / (msl / 1e3), 1), "unit": "accepted tokens/s",
                          "ms_per_step": round(msl / 8, 3),
                          "verify_step_hbm_GBps": round(WL.verify_bytes_total /
                                                        (WL.verify_ms / 1e3) / 1e9, 1),
                          "verify_ms_per_step": round(WL.verify_ms / 8, 3)})
            del WL
            torch.cuda.empty_cache()
        out["long_context"] = lines
    if not args.no_cpu_baseline:
        log("cpu baseline (oracle)")
        out["cpu_baseline"] = cpu_baseline(K, args.ctx, (K + 2) / 2.0)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
