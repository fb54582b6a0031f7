// C ABI of libuno: argument validation, workspace carving and the layer loop of
// the draft and verify passes ("Unlocking Lossless Speedups in LLMs via
// Discrete Diffusion": picx.dev summary, "Methodology"; paperglide reader, "The
// Psi-Speculative Sampler", "Sampler Extensions").  Every kernel runs on the
// caller's stream; nothing here allocates, copies or synchronises.
#include <hip/hip_runtime.h>
#include <math.h>
#include <string.h>

#include <string>

#include "uno_internal.h"

using namespace uno;

namespace {

thread_local std::string g_last_hip_error;

// Measurement hook (uno_set_timing_events): brackets launches of one kernel
// class with caller-owned HIP events on the launching stream.
struct TimingHook {
  int cls = 0;
  hipEvent_t* start = nullptr;
  hipEvent_t* stop = nullptr;
  int n = 0;
  int count = 0;
};
TimingHook g_hook;

// Records events around `launch` when the armed class is `cls` or `cls2`
// (a projection GEMM belongs to UNO_TIME_GEMM and to its own class).
template <class F>
hipError_t timed(int cls, hipStream_t s, F&& launch, int cls2 = -1) {
  const bool on = (g_hook.cls == cls || g_hook.cls == cls2) && g_hook.count < g_hook.n;
  if (on) hipEventRecord(g_hook.start[g_hook.count], s);
  const hipError_t e = launch();
  if (on) hipEventRecord(g_hook.stop[g_hook.count++], s);
  return e;
}

int hip_fail(hipError_t e) {
  g_last_hip_error = hipGetErrorString(e);
  return UNO_ERR_HIP;
}

enum Proj { P_Q = 0, P_K, P_V, P_O, P_GATE, P_UP, P_DOWN };

bool bit(const uno_config& c, int p) { return (c.lora_mask >> p) & 1u; }

int check_config(const uno_config* c) {
  if (!c) return UNO_ERR_INVALID_ARG;
  if (c->n_layers < 1 || c->d_model < 64 || c->n_q_heads < 1 || c->n_kv_heads < 1 ||
      c->d_ffn < 64 || c->vocab < 16 || c->page_size < 16 || c->lora_rank < 0)
    return UNO_ERR_INVALID_ARG;
  if (c->mask_id < 0 || c->mask_id >= c->vocab) return UNO_ERR_INVALID_ARG;
  if (!(c->rms_eps > 0.f) || !(c->rope_theta > 1.f) || !isfinite(c->lora_scale))
    return UNO_ERR_INVALID_ARG;
  if (c->head_dim != 64 && c->head_dim != 128) return UNO_ERR_UNSUPPORTED;
  if (c->n_q_heads % c->n_kv_heads) return UNO_ERR_UNSUPPORTED;
  if (c->d_model % 64 || c->d_ffn % 64 || (c->n_q_heads * c->head_dim) % 64)
    return UNO_ERR_UNSUPPORTED;
  if (c->vocab % 16 || c->vocab > (1 << 20)) return UNO_ERR_UNSUPPORTED;
  if (c->page_size & (c->page_size - 1)) return UNO_ERR_UNSUPPORTED;   // power of two >= 16
  if (c->lora_mask & ~0x7Fu) return UNO_ERR_INVALID_ARG;
  if (c->noise_prior != 0 && c->noise_prior != 1) return UNO_ERR_INVALID_ARG;
  if (c->lora_mask) {
    if (c->lora_rank < 16 || c->lora_rank % 16 || c->lora_rank > 256) return UNO_ERR_UNSUPPORTED;
    const bool q = bit(*c, P_Q), k = bit(*c, P_K), v = bit(*c, P_V);
    if (q != k || k != v) return UNO_ERR_UNSUPPORTED;
    if (bit(*c, P_GATE) != bit(*c, P_UP)) return UNO_ERR_UNSUPPORTED;
  }
  return UNO_OK;
}

int check_kv(const uno_config& c, const uno_kv* kv, int K, int max_extra) {
  if (!kv || !kv->k_pages || !kv->v_pages || !kv->page_table || !kv->kv_len)
    return UNO_ERR_INVALID_ARG;
  if (kv->n_pages < 1 || kv->max_pages_per_seq < 1) return UNO_ERR_INVALID_ARG;
  if ((int64_t)kv->max_pages_per_seq * c.page_size < (int64_t)K + max_extra)
    return UNO_ERR_CAPACITY;
  return UNO_OK;
}

// rank used by the fused kernels: 16 stays 16 (tiny models) else multiple of 32
int lora_rank_eff(const uno_config& c) { return c.lora_mask ? c.lora_rank : 0; }

struct PassWs {
  float* h;          // [R, D]
  uint16_t* xn;      // [R, max(D, F, Hq*hd)]
  float* qkv;        // [R, (Hq+2Hkv)*hd]
  uint16_t* qb;      // [R, Hq*hd]  q (bf16 high part)
  uint16_t* qlo;     // [R, Hq*hd]  q - high part (bf16)
  uint16_t* ao;      // [R, Hq*hd]
  float* gu;         // [R, 2F]
  uint16_t* act;     // [R, F]
  uint16_t* t;       // [R, 3r]
  float2* cs;        // [R, hd/2]
  int2* row_page;    // [R] K/V page and slot of each row
  float* part_o;
  float* part_ml;
  float* gemm_part;      // split-K partial tiles (passes of more than 64 rows)
  size_t gemm_part_floats;
  float* lora_part;      // LoRA-A split-K partials read by the next projection (<= 64 rows)
  float* max_part;       // [R, V/16] LM-head row-maxima partials (per column group)
  float* row_max;        // [R] row maxima of the logits (when the caller passes none)
  uint64_t* chunk_sums;  // [R, 128] exact chunk sums of the draft sampler
  unsigned* sync;        // [4 * n_layers, kLoraSyncWords] LoRA-A -> projection counters (<= 64 rows),
                         // zeroed by the pass's RoPE-table kernel
  size_t total;
};

PassWs carve(const uno_config& c, int B, int K, int max_ctx, void* base) {
  PassWs w;
  const size_t R = (size_t)B * K;
  const size_t D = c.d_model, F = c.d_ffn, QD = (size_t)c.n_q_heads * c.head_dim;
  const size_t QKV = (size_t)(c.n_q_heads + 2 * c.n_kv_heads) * c.head_dim;
  const size_t X = D > F ? (D > QD ? D : QD) : (F > QD ? F : QD);
  const size_t r = (size_t)(lora_rank_eff(c) ? lora_rank_eff(c) : 16);
  const AttnPlan p = attn_plan(c, B, K, max_ctx);
  const size_t parts = (size_t)B * c.n_kv_heads * p.n_qgroups * p.n_wave_splits * 128;
  size_t off = 0;
  char* b = static_cast<char*>(base);
  auto take = [&](size_t bytes) {
    char* ptr = b ? b + off : nullptr;
    off += align_up(bytes, 256);
    return ptr;
  };
  w.h = reinterpret_cast<float*>(take(R * D * 4));
  w.xn = reinterpret_cast<uint16_t*>(take(R * X * 2));
  w.qkv = reinterpret_cast<float*>(take(R * QKV * 4));
  w.qb = reinterpret_cast<uint16_t*>(take(R * QD * 2));
  w.qlo = reinterpret_cast<uint16_t*>(take(R * QD * 2));
  w.ao = reinterpret_cast<uint16_t*>(take(R * QD * 2));
  w.gu = reinterpret_cast<float*>(take(R * 2 * F * 4));
  w.act = reinterpret_cast<uint16_t*>(take(R * F * 2));
  w.t = reinterpret_cast<uint16_t*>(take(R * 3 * r * 2));
  w.cs = reinterpret_cast<float2*>(take(R * (c.head_dim / 2) * sizeof(float2)));
  w.row_page = reinterpret_cast<int2*>(take(R * sizeof(int2)));
  w.part_o = reinterpret_cast<float*>(take(parts * c.head_dim * 4));
  w.part_ml = reinterpret_cast<float*>(take(parts * 2 * 4));
  w.gemm_part_floats = R > 64 ? kGemmPartFloats : kGemmPartFloatsSkinny;
  w.gemm_part = reinterpret_cast<float*>(take(w.gemm_part_floats * 4));
  w.lora_part = R <= 64 ? reinterpret_cast<float*>(take(kLoraPartFloats * 4)) : nullptr;
  w.max_part = reinterpret_cast<float*>(
      take(R * gemm_row_max_parts_bound(c.vocab, (int)R) * 4));
  w.row_max = reinterpret_cast<float*>(take(R * 4));
  w.chunk_sums = reinterpret_cast<uint64_t*>(take(chunk_sums_bytes((int)R)));
  w.sync = R <= 64 ? reinterpret_cast<unsigned*>(take((size_t)4 * c.n_layers * kLoraSyncWords * 4)) : nullptr;
  w.total = off;
  return w;
}

int check_layers(const uno_config& c, const uno_weights* w, bool lora) {
  if (!w || !w->embed || !w->lm_head || !w->final_norm || !w->layers) return UNO_ERR_INVALID_ARG;
  for (int li = 0; li < c.n_layers; ++li) {
    const uno_layer_weights& L = w->layers[li];
    if (!L.attn_norm || !L.mlp_norm || !L.wq || !L.wk || !L.wv || !L.wo || !L.wgate || !L.wup ||
        !L.wdown)
      return UNO_ERR_INVALID_ARG;
    if (lora)
      for (int p = 0; p < 7; ++p)
        if (bit(c, p) && (!L.lora_a[p] || !L.lora_b[p])) return UNO_ERR_INVALID_ARG;
  }
  return UNO_OK;
}

const bf16_raw_t* bp(const void* p) { return static_cast<const bf16_raw_t*>(p); }

// One forward pass of B*K rows (draft when `anchor` != null, verify otherwise).
// A token tree's verify pass passes tree_depth [B*K] (RoPE positions) and
// tree_anc [B*K, (K+31)/32] (attention mask); both null otherwise.
int run_pass(const uno_config& c, const uno_weights* w, const uno_kv* kv, const int32_t* anchor,
             const int32_t* block, const int32_t* rows, int B, int K, int max_ctx, int pos_offset,
             bool lora,
             uint64_t seed, const uint64_t* step, float* logits, float* row_max,
             int32_t* status, void* ws,
             hipStream_t s, const int32_t* tree_depth = nullptr,
             const uint32_t* tree_anc = nullptr, uint32_t keep_q24 = 1u << 24,
             int corr_pass = 0) {
  const PassWs W = carve(c, B, K, max_ctx, ws);
  const int R = B * K;
  const int D = c.d_model, F = c.d_ffn, hd = c.head_dim;
  const int Hq = c.n_q_heads, Hkv = c.n_kv_heads;
  const int QD = Hq * hd, KD = Hkv * hd, QKV = QD + 2 * KD;
  const int r = lora ? lora_rank_eff(c) : 0;
  const bool draft = anchor != nullptr;
  hipError_t e;
#define UNO_TRY(x) do { e = (x); if (e != hipSuccess) return hip_fail(e); } while (0)

  UNO_TRY(launch_embed(c, bp(w->embed), anchor, block, rows, B, K, seed, step, keep_q24, corr_pass,
                       W.h, status, s));
  UNO_TRY(launch_rope_table(c, *kv, B, K, draft ? 0 : pos_offset, tree_depth, W.cs, W.row_page,
                            status, W.sync, W.sync ? 4 * c.n_layers * kLoraSyncWords : 0, s));
  const AttnPlan plan = attn_plan(c, B, K, max_ctx);
  const size_t layer_elems = (size_t)kv->n_pages * Hkv * c.page_size * hd;

  auto scratch_args = [&] {
    GemmArgs g = {};
    g.part = W.gemm_part;
    g.part_floats = W.gemm_part_floats;
    return g;
  };
  // the LoRA-A product T = scale * gate(row) * (X A^T) of a projection
  auto lora_args = [&](const bf16_raw_t* x, int ldx, int Kd, const void* const* a_ptrs, int n_a) {
    GemmArgs g = scratch_args();
    g.x = x; g.M = R; g.Kd = Kd; g.ldx = ldx;
    for (int i = 0; i < n_a; ++i) g.seg[i] = GemmSeg{bp(a_ptrs[i]), r, nullptr, 0};
    g.n_seg = n_a;
    g.epi = EPI_LORA_T; g.out = W.t; g.ldo = n_a * r; g.scale = c.lora_scale; g.rows_per_seq = K;
    return g;
  };
  // a projection after its LoRA-A product (when `ta` is given); at most 64 rows
  // the two run as one launch (the projection sums the product's split-K
  // partials itself), otherwise as two
  int li_cur = 0;
  auto project = [&](const GemmArgs& g0, const GemmArgs* ta0, int cls, bool* normed_out,
                     bool* roped_out, bool* swiglued_out) -> hipError_t {
    if (ta0 && W.sync && W.lora_part) {
      unsigned* ctr = W.sync + (size_t)(4 * li_cur + cls - UNO_TIME_GEMM_QKV) * kLoraSyncWords;
      bool fused = false;
      return timed(UNO_TIME_GEMM, s, [&] {
        return launch_gemm_lora(g0, *ta0, W.lora_part, kLoraPartFloats, ctr, status, s,
                                normed_out, roped_out, swiglued_out, &fused);
      }, cls);
    }
    GemmArgs g = g0;
    if (ta0) {
      GemmArgs ta;
      gemm_lora_pair(g0, *ta0, W.lora_part, kLoraPartFloats, &g, &ta);
      const hipError_t e = timed(UNO_TIME_LORA_A, s, [&] { return launch_gemm(ta, s); });
      if (e != hipSuccess) return e;
    }
    return timed(UNO_TIME_GEMM, s, [&] { return launch_gemm(g, s, normed_out, roped_out,
                                                             swiglued_out); }, cls);
  };

  // set when a residual projection's split-K reduction also wrote the RMSNorm
  // of the updated rows into W.xn (the stand-alone norm is then skipped)
  bool normed = false;
  for (int li = 0; li < c.n_layers; ++li) {
    li_cur = li;
    const uno_layer_weights& L = w->layers[li];
    const bool lq = r && bit(c, P_Q), lo = r && bit(c, P_O), lg = r && bit(c, P_GATE),
               ld = r && bit(c, P_DOWN);
    // ---- attention block
    if (!normed)
      UNO_TRY(launch_rmsnorm(W.h, static_cast<const float*>(L.attn_norm), R, D, c.rms_eps, W.xn, s));
    {
      const void* a3[3] = {L.lora_a[P_Q], L.lora_a[P_K], L.lora_a[P_V]};
      const GemmArgs ta = lq ? lora_args(W.xn, D, D, a3, 3) : GemmArgs{};
      GemmArgs g = scratch_args();
      g.x = W.xn; g.M = R; g.Kd = D; g.ldx = D;
      g.seg[0] = GemmSeg{bp(L.wq), QD, lq ? bp(L.lora_b[P_Q]) : nullptr, 0};
      g.seg[1] = GemmSeg{bp(L.wk), KD, lq ? bp(L.lora_b[P_K]) : nullptr, r};
      g.seg[2] = GemmSeg{bp(L.wv), KD, lq ? bp(L.lora_b[P_V]) : nullptr, 2 * r};
      g.n_seg = 3;
      g.t = lq ? W.t : nullptr; g.ldt = 3 * r; g.rank = r;
      g.epi = EPI_STORE_F32; g.out = W.qkv; g.ldo = QKV;
      // a split product applies RoPE and writes q and the K/V pages in its reduction
      g.rope_fuse = 1;
      g.rope = make_rope_args(c, W.cs, W.row_page, *kv, li, K, W.qb, W.qlo);
      bool roped = false;
      UNO_TRY(project(g, lq ? &ta : nullptr, UNO_TIME_GEMM_QKV, nullptr, &roped, nullptr));
      if (!roped) UNO_TRY(launch_rope_kv_write(W.qkv, g.rope, R, s));
    }
    {
      AttnArgs a = {};
      a.q = W.qb;
      a.q_lo = W.qlo;
      a.k_layer = static_cast<const uint16_t*>(kv->k_pages) + (size_t)li * layer_elems;
      a.v_layer = static_cast<const uint16_t*>(kv->v_pages) + (size_t)li * layer_elems;
      a.page_table = kv->page_table; a.kv_len = kv->kv_len;
      a.max_pages = kv->max_pages_per_seq; a.n_pages = kv->n_pages;
      a.B = B; a.K = K; a.pos_offset = draft ? 0 : pos_offset; a.draft = draft ? 1 : 0;
      a.tree_anc = tree_anc; a.anc_words = (K + 31) / 32;
      a.Hq = Hq; a.Hkv = Hkv; a.hd = hd; a.ps = c.page_size; a.plan = plan;
      a.ps_shift = __builtin_ctz((unsigned)c.page_size);
      a.part_o = W.part_o; a.part_ml = W.part_ml; a.out = W.ao; a.status = status;
      UNO_TRY(timed(UNO_TIME_ATTENTION, s, [&] { return launch_attention(a, s); }));
      UNO_TRY(launch_attn_merge(a, s));
    }
    {
      const void* a1[1] = {L.lora_a[P_O]};
      const GemmArgs ta = lo ? lora_args(W.ao, QD, QD, a1, 1) : GemmArgs{};
      GemmArgs g = scratch_args();
      g.x = W.ao; g.M = R; g.Kd = QD; g.ldx = QD;
      g.seg[0] = GemmSeg{bp(L.wo), D, lo ? bp(L.lora_b[P_O]) : nullptr, 0};
      g.n_seg = 1;
      g.t = lo ? W.t : nullptr; g.ldt = r; g.rank = r;
      g.epi = EPI_ADD_F32; g.out = W.h; g.ldo = D;
      g.norm_gain = static_cast<const float*>(L.mlp_norm); g.norm_out = W.xn; g.norm_eps = c.rms_eps;
      UNO_TRY(project(g, lo ? &ta : nullptr, UNO_TIME_GEMM_O, &normed, nullptr, nullptr));
    }
    // ---- MLP block
    if (!normed)
      UNO_TRY(launch_rmsnorm(W.h, static_cast<const float*>(L.mlp_norm), R, D, c.rms_eps, W.xn, s));
    {
      const void* a2[2] = {L.lora_a[P_GATE], L.lora_a[P_UP]};
      const GemmArgs ta = lg ? lora_args(W.xn, D, D, a2, 2) : GemmArgs{};
      // gate and up rows stored back to back (and their LoRA B factors too):
      // the tiled kernel pairs them and writes silu(gate) * up directly
      const char* wg = static_cast<const char*>(L.wgate);
      const bool adjacent =
          static_cast<const char*>(L.wup) == wg + (size_t)F * D * 2 &&
          (!lg || static_cast<const char*>(L.lora_b[P_UP]) ==
                      static_cast<const char*>(L.lora_b[P_GATE]) + (size_t)F * r * 2);
      GemmArgs g = scratch_args();
      g.x = W.xn; g.M = R; g.Kd = D; g.ldx = D;
      g.t = lg ? W.t : nullptr; g.ldt = 2 * r; g.rank = r;
      g.seg[0] = GemmSeg{bp(L.wgate), F, lg ? bp(L.lora_b[P_GATE]) : nullptr, 0};
      g.n_seg = 1;
      g.epi = EPI_SWIGLU; g.out = W.act; g.ldo = F;
      const bool fused = adjacent && gemm_swiglu_ok(g);
      if (!fused) {
        // two segments; a split product applies SwiGLU in its reduction
        g.seg[1] = GemmSeg{bp(L.wup), F, lg ? bp(L.lora_b[P_UP]) : nullptr, r};
        g.n_seg = 2;
        g.epi = EPI_STORE_F32; g.out = W.gu; g.ldo = 2 * F;
        g.act_out = W.act;
      }
      bool swiglued = false;
      UNO_TRY(project(g, lg ? &ta : nullptr, UNO_TIME_GEMM_GATE_UP, nullptr, nullptr, &swiglued));
      if (!fused && !swiglued) UNO_TRY(launch_silu_mul(W.gu, R, F, W.act, s));
    }
    {
      const void* a1[1] = {L.lora_a[P_DOWN]};
      const GemmArgs ta = ld ? lora_args(W.act, F, F, a1, 1) : GemmArgs{};
      GemmArgs g = scratch_args();
      g.x = W.act; g.M = R; g.Kd = F; g.ldx = F;
      g.seg[0] = GemmSeg{bp(L.wdown), D, ld ? bp(L.lora_b[P_DOWN]) : nullptr, 0};
      g.n_seg = 1;
      g.t = ld ? W.t : nullptr; g.ldt = r; g.rank = r;
      g.epi = EPI_ADD_F32; g.out = W.h; g.ldo = D;
      const void* next_norm = li + 1 < c.n_layers ? w->layers[li + 1].attn_norm
                              : logits             ? w->final_norm
                                                   : nullptr;
      g.norm_gain = static_cast<const float*>(next_norm); g.norm_out = W.xn; g.norm_eps = c.rms_eps;
      UNO_TRY(project(g, ld ? &ta : nullptr, UNO_TIME_GEMM_DOWN, &normed, nullptr, nullptr));
    }
  }
  if (logits) {
    if (!normed)
      UNO_TRY(launch_rmsnorm(W.h, static_cast<const float*>(w->final_norm), R, D, c.rms_eps, W.xn, s));
    GemmArgs g = scratch_args();
    g.x = W.xn; g.M = R; g.Kd = D; g.ldx = D;
    g.seg[0] = GemmSeg{bp(w->lm_head), c.vocab, nullptr, 0};
    g.n_seg = 1;
    g.epi = EPI_STORE_F32; g.out = logits; g.ldo = c.vocab;
    if (row_max) {
      // the LM head also yields every logits row's exact maximum, so that the
      // sampler streams each row once
      g.max_part = W.max_part;
      g.max_part_ld = gemm_row_max_parts(g);
    }
    // a plan with more column groups than carved for: the maxima are taken
    // from the stored rows instead (one row per workgroup)
    const bool from_rows = row_max && g.max_part_ld > gemm_row_max_parts_bound(c.vocab, R);
    if (from_rows) g.max_part = nullptr;
    UNO_TRY(timed(UNO_TIME_LM_HEAD, s, [&] {
      const hipError_t e1 = launch_gemm(g, s);
      if (e1 != hipSuccess || !row_max) return e1;
      if (from_rows) return launch_row_max(logits, c.vocab, c.vocab, R, row_max, s);
      return launch_row_max(W.max_part, g.max_part_ld, g.max_part_ld, R, row_max, s);
    }));
  }
#undef UNO_TRY
  return UNO_OK;
}

}  // namespace

extern "C" {

size_t uno_workspace_bytes(const uno_config* cfg, int batch, int K, int max_ctx) {
  if (check_config(cfg) != UNO_OK || batch < 1 || K < 1) return 0;
  return carve(*cfg, batch, K, max_ctx, nullptr).total;
}

int uno_draft_block_from(const uno_config* cfg, const uno_weights* w, const uno_kv* kv,
                         const int32_t* anchor, const int32_t* block, int batch, int K,
                         int max_ctx, float inv_temp, uint64_t seed, const uint64_t* step,
                         int sample_slot, uint32_t keep_q24, int corr_pass, float* draft_logits,
                         int32_t* draft_tokens, float* row_max, int32_t* status, void* ws,
                         size_t ws_bytes, void* stream) {
  int rc = check_config(cfg);
  if (rc) return rc;
  if (batch < 1 || K < 1 || K > 64 || max_ctx < 1) return UNO_ERR_INVALID_ARG;
  if (!anchor || !step || !draft_logits || !draft_tokens || !ws) return UNO_ERR_INVALID_ARG;
  if (!(inv_temp > 0.f) || !isfinite(inv_temp)) return UNO_ERR_INVALID_ARG;
  if (sample_slot != 0 && (sample_slot < 4 || sample_slot > 63)) return UNO_ERR_INVALID_ARG;
  if (keep_q24 > (1u << 24) || corr_pass < 0 || corr_pass > 59) return UNO_ERR_INVALID_ARG;
  if ((rc = check_kv(*cfg, kv, K, 0))) return rc;
  if ((rc = check_layers(*cfg, w, true))) return rc;
  if (ws_bytes < carve(*cfg, batch, K, max_ctx, nullptr).total) return UNO_ERR_WORKSPACE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const PassWs W = carve(*cfg, batch, K, max_ctx, ws);
  float* rmax = row_max ? row_max : W.row_max;
  rc = run_pass(*cfg, w, kv, anchor, block, nullptr, batch, K, max_ctx, 0, cfg->lora_mask != 0,
                seed, step, draft_logits, rmax, status, ws, s, nullptr, nullptr, keep_q24,
                corr_pass);
  if (rc) return rc;
  const hipError_t e = timed(UNO_TIME_SAMPLER, s, [&] {
    return launch_draft_sample_chunked(draft_logits, rmax, W.chunk_sums, batch, K, cfg->vocab,
                                       inv_temp, seed, sample_slot, step, draft_tokens, status, s);
  });
  return e == hipSuccess ? UNO_OK : hip_fail(e);
}

int uno_draft_block(const uno_config* cfg, const uno_weights* w, const uno_kv* kv,
                    const int32_t* anchor, int batch, int K, int max_ctx, float inv_temp,
                    uint64_t seed, const uint64_t* step, float* draft_logits,
                    int32_t* draft_tokens, float* row_max, int32_t* status, void* ws,
                    size_t ws_bytes, void* stream) {
  return uno_draft_block_from(cfg, w, kv, anchor, nullptr, batch, K, max_ctx, inv_temp, seed,
                              step, 0, 1u << 24, 0, draft_logits, draft_tokens, row_max, status,
                              ws, ws_bytes, stream);
}

int uno_verify_block(const uno_config* cfg, const uno_weights* w, const uno_kv* kv,
                     const int32_t* rows, int batch, int K, int max_ctx, int pos_offset,
                     float* verify_logits, float* row_max, int32_t* status, void* ws,
                     size_t ws_bytes, void* stream) {
  int rc = check_config(cfg);
  if (rc) return rc;
  if (batch < 1 || K < 1 || K > 4096 || max_ctx < 1) return UNO_ERR_INVALID_ARG;
  if (pos_offset < 0 || pos_offset > 1) return UNO_ERR_INVALID_ARG;
  if (!rows || !ws) return UNO_ERR_INVALID_ARG;
  if (row_max && !verify_logits) return UNO_ERR_INVALID_ARG;
  if ((rc = check_kv(*cfg, kv, K, pos_offset))) return rc;
  if ((rc = check_layers(*cfg, w, false))) return rc;
  if (ws_bytes < carve(*cfg, batch, K, max_ctx, nullptr).total) return UNO_ERR_WORKSPACE;
  return run_pass(*cfg, w, kv, nullptr, nullptr, rows, batch, K, max_ctx, pos_offset, false, 0,
                  nullptr, verify_logits, row_max, status, ws, static_cast<hipStream_t>(stream));
}

int uno_draft_sample(const float* logits, const float* row_max, int batch, int K, int vocab,
                     float inv_temp, uint64_t seed, const uint64_t* step, int32_t* tokens,
                     int32_t* status, void* stream) {
  if (!logits || !step || !tokens) return UNO_ERR_INVALID_ARG;
  if (batch < 1 || K < 1 || vocab < 1 || vocab > (1 << 20)) return UNO_ERR_INVALID_ARG;
  if (!(inv_temp > 0.f) || !isfinite(inv_temp)) return UNO_ERR_INVALID_ARG;
  const hipError_t e = launch_draft_sample(logits, row_max, batch, K, vocab, inv_temp, seed, 0,
                                           step, tokens, status,
                                           static_cast<hipStream_t>(stream));
  return e == hipSuccess ? UNO_OK : hip_fail(e);
}

size_t uno_spec_accept_workspace_bytes(int batch, int K) {
  if (batch < 1 || K < 1) return 0;
  return spec_accept_ws_bytes(batch, K);
}

int uno_spec_accept(const float* draft_logits, const float* verify_logits,
                    const float* draft_row_max, const float* verify_row_max,
                    const int32_t* draft_tokens, int batch, int K, int vocab, float inv_temp,
                    uint64_t seed, const uint64_t* step, const int32_t* forced_accept,
                    int32_t* accept_len, int32_t* committed, int32_t* extra_token,
                    int32_t* status, void* ws, size_t ws_bytes, void* stream) {
  if (!draft_logits || !verify_logits || !draft_tokens || !step || !accept_len || !committed ||
      !extra_token || !ws)
    return UNO_ERR_INVALID_ARG;
  if (!draft_row_max != !verify_row_max) return UNO_ERR_INVALID_ARG;
  if (batch < 1 || K < 1 || K > 4096 || vocab < 1 || vocab > (1 << 20))
    return UNO_ERR_INVALID_ARG;
  if (!(inv_temp > 0.f) || !isfinite(inv_temp)) return UNO_ERR_INVALID_ARG;
  if (ws_bytes < spec_accept_ws_bytes(batch, K)) return UNO_ERR_WORKSPACE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const hipError_t e = timed(UNO_TIME_SAMPLER, s, [&] {
    return launch_spec_accept(draft_logits, verify_logits, draft_row_max, verify_row_max,
                              draft_tokens, batch, K, vocab, inv_temp, seed, step, forced_accept,
                              accept_len, committed, extra_token, status, ws, s);
  });
  return e == hipSuccess ? UNO_OK : hip_fail(e);
}

int uno_spec_accept_noalloc(const float* draft_logits, const float* verify_logits,
                            const float* draft_row_max, const float* verify_row_max,
                            const int32_t* draft_tokens, int batch, int K, int vocab,
                            float inv_temp, uint64_t seed, const uint64_t* step,
                            const int32_t* forced_accept, int32_t* accept_len,
                            int32_t* committed, int32_t* extra_token, int32_t* status,
                            void* stream) {
  if (!draft_logits || !verify_logits || !draft_tokens || !step || !accept_len || !committed ||
      !extra_token)
    return UNO_ERR_INVALID_ARG;
  if (!draft_row_max != !verify_row_max) return UNO_ERR_INVALID_ARG;
  if (batch < 1 || K < 1 || K > 4096 || vocab < 1 || vocab > (1 << 20))
    return UNO_ERR_INVALID_ARG;
  if (!(inv_temp > 0.f) || !isfinite(inv_temp)) return UNO_ERR_INVALID_ARG;
  if (2 * (int64_t)batch * K > static_accept_max_rows()) return UNO_ERR_WORKSPACE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const hipError_t e = timed(UNO_TIME_SAMPLER, s, [&] {
    return launch_spec_accept_static(draft_logits, verify_logits, draft_row_max, verify_row_max,
                                     draft_tokens, batch, K, vocab, inv_temp, seed, step,
                                     forced_accept, accept_len, committed, extra_token, status, s);
  });
  return e == hipSuccess ? UNO_OK : hip_fail(e);
}

int uno_kv_commit(const uno_kv* kv, const int32_t* accept_len, int batch, int K, uint64_t* step,
                  int32_t* status, void* stream) {
  if (!kv || !kv->kv_len || !accept_len) return UNO_ERR_INVALID_ARG;
  if (batch < 1 || K < 0) return UNO_ERR_INVALID_ARG;
  const hipError_t e = launch_kv_commit(kv->kv_len, accept_len, batch, K, step, status,
                                        static_cast<hipStream_t>(stream));
  return e == hipSuccess ? UNO_OK : hip_fail(e);
}

// ---------------------------------------------------------------- tree sampler
int uno_tree_rows(int K, int topk, int n_keep) {
  if (K < 2 || K > 32 || topk < 1 || topk > 8 || n_keep < 1 || n_keep > 64) return 0;
  // n_keep <= topk^(K-1)
  long long cands = 1;
  for (int i = 0; i < K - 1 && cands < n_keep; ++i) cands *= topk;
  if (cands < n_keep) return 0;
  return 1 + n_keep * (K - 1);
}

size_t uno_tree_workspace_bytes(int batch, int K, int topk) {
  if (batch < 1 || K < 2 || K > 32 || topk < 1 || topk > 8) return 0;
  return tree_ws_bytes(batch, K, topk);
}

int uno_tree_build(const float* draft_logits, const int32_t* draft_tokens, int batch, int K,
                   int vocab, int topk, int n_keep, int32_t* node_tokens, int32_t* node_parent,
                   int32_t* node_depth, uint32_t* node_anc, int32_t* n_nodes, int32_t* status,
                   void* ws, size_t ws_bytes, void* stream) {
  const int N = uno_tree_rows(K, topk, n_keep);
  if (!N || batch < 1 || vocab < 16 || vocab > (1 << 20)) return UNO_ERR_INVALID_ARG;
  if (!draft_logits || !draft_tokens || !node_tokens || !node_parent || !node_depth ||
      !node_anc || !n_nodes || !ws)
    return UNO_ERR_INVALID_ARG;
  if (ws_bytes < tree_ws_bytes(batch, K, topk)) return UNO_ERR_WORKSPACE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const hipError_t e = timed(UNO_TIME_SAMPLER, s, [&] {
    return launch_tree_build(draft_logits, draft_tokens, batch, K, vocab, topk, n_keep, N,
                             node_tokens, node_parent, node_depth, node_anc, n_nodes, status, ws,
                             s);
  });
  return e == hipSuccess ? UNO_OK : hip_fail(e);
}

int uno_verify_tree(const uno_config* cfg, const uno_weights* w, const uno_kv* kv,
                    const int32_t* node_tokens, const int32_t* node_depth,
                    const uint32_t* node_anc, int batch, int n_rows, int max_ctx,
                    float* verify_logits, int32_t* status, void* ws, size_t ws_bytes,
                    void* stream) {
  int rc = check_config(cfg);
  if (rc) return rc;
  if (batch < 1 || n_rows < 2 || n_rows > 4096 || max_ctx < 1) return UNO_ERR_INVALID_ARG;
  if (!node_tokens || !node_depth || !node_anc || !ws) return UNO_ERR_INVALID_ARG;
  if ((rc = check_kv(*cfg, kv, n_rows, 1))) return rc;
  if ((rc = check_layers(*cfg, w, false))) return rc;
  if (ws_bytes < carve(*cfg, batch, n_rows, max_ctx, nullptr).total) return UNO_ERR_WORKSPACE;
  return run_pass(*cfg, w, kv, nullptr, nullptr, node_tokens, batch, n_rows, max_ctx, 1, false, 0,
                  nullptr, verify_logits, nullptr, status, ws, static_cast<hipStream_t>(stream),
                  node_depth, node_anc);
}

int uno_tree_accept(const float* verify_logits, const int32_t* node_tokens,
                    const int32_t* node_parent, const int32_t* node_depth,
                    const int32_t* n_nodes, int batch, int K, int n_rows, int vocab,
                    float inv_temp, uint64_t seed, const uint64_t* step, int32_t* node_sample,
                    int32_t* accept_len, int32_t* committed, int32_t* extra_token,
                    int32_t* path, int32_t* status, void* stream) {
  if (!verify_logits || !node_tokens || !node_parent || !node_depth || !n_nodes || !step ||
      !node_sample || !accept_len || !committed || !extra_token || !path)
    return UNO_ERR_INVALID_ARG;
  if (batch < 1 || K < 2 || K > 32 || n_rows < K || n_rows > 4096 || vocab < 16 ||
      vocab > (1 << 20))
    return UNO_ERR_INVALID_ARG;
  if (!(inv_temp > 0.f) || !isfinite(inv_temp)) return UNO_ERR_INVALID_ARG;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const hipError_t e = timed(UNO_TIME_SAMPLER, s, [&] {
    hipError_t r = launch_tree_sample(verify_logits, batch, n_rows, vocab, inv_temp, seed, step,
                                      node_depth, n_nodes, node_sample, status, s);
    if (r != hipSuccess) return r;
    return launch_tree_walk(node_tokens, node_parent, n_nodes, node_sample, batch, K, n_rows,
                            accept_len, committed, extra_token, path, status, s);
  });
  return e == hipSuccess ? UNO_OK : hip_fail(e);
}

int uno_tree_commit(const uno_config* cfg, const uno_kv* kv, const int32_t* path,
                    const int32_t* accept_len, int batch, int K, uint64_t* step, int32_t* status,
                    void* stream) {
  int rc = check_config(cfg);
  if (rc) return rc;
  if (!kv || !kv->kv_len || !kv->k_pages || !kv->v_pages || !kv->page_table || !path ||
      !accept_len)
    return UNO_ERR_INVALID_ARG;
  if (batch < 1 || K < 2 || K > 32) return UNO_ERR_INVALID_ARG;
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e = launch_tree_commit(*cfg, *kv, path, accept_len, batch, K, status, s);
  if (e == hipSuccess) e = launch_kv_commit(kv->kv_len, accept_len, batch, K, step, status, s);
  return e == hipSuccess ? UNO_OK : hip_fail(e);
}

int uno_pack_weight(const void* src, void* dst, int n_out, int n_in, void* stream) {
  if (!src || !dst || src == dst || n_out < 16 || n_in < 32 || n_out % 16 || n_in % 32)
    return UNO_ERR_INVALID_ARG;
  const hipError_t e = launch_pack_tiles(static_cast<const uint16_t*>(src),
                                         static_cast<uint16_t*>(dst), n_out, n_in,
                                         static_cast<hipStream_t>(stream));
  return e == hipSuccess ? UNO_OK : hip_fail(e);
}

int uno_set_timing_events(int kernel_class, void* const* start, void* const* stop, int n) {
  if (kernel_class == 0) {
    g_hook = TimingHook();
    return UNO_OK;
  }
  if (kernel_class < 0 || kernel_class > UNO_TIME_GEMM_DOWN || !start || !stop || n < 1)
    return UNO_ERR_INVALID_ARG;
  g_hook.cls = kernel_class;
  g_hook.start = reinterpret_cast<hipEvent_t*>(const_cast<void**>(start));
  g_hook.stop = reinterpret_cast<hipEvent_t*>(const_cast<void**>(stop));
  g_hook.n = n;
  g_hook.count = 0;
  return UNO_OK;
}

int uno_timing_events_used(void) { return g_hook.count; }

const char* uno_status_string(int status) {
  switch (status) {
    case UNO_OK: return "ok";
    case UNO_ERR_INVALID_ARG: return "invalid argument";
    case UNO_ERR_UNSUPPORTED: return "unsupported shape";
    case UNO_ERR_CAPACITY: return "page table too small for the block";
    case UNO_ERR_WORKSPACE: return "workspace too small";
    case UNO_ERR_HIP: return "HIP launch failure";
    default: return "unknown status";
  }
}

const char* uno_last_hip_error(void) { return g_last_hip_error.c_str(); }

}  // extern "C"
