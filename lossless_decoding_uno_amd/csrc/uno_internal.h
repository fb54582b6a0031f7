// Internal launchers of libuno (host side).  Every launcher only enqueues on
// the given stream and returns hipGetLastError().
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "uno.h"

namespace uno {

typedef uint16_t bf16_raw_t;  // bf16 bits in memory

static inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// ---------------------------------------------------------------- sampler
// row_max [B*K] (the exact maximum of each logits row) or null: with it every
// row is streamed once, without it a maximum pass comes first.
hipError_t launch_draft_sample(const float* logits, const float* row_max, int B, int K, int V,
                               float inv_temp, uint64_t seed, int slot, const uint64_t* step,
                               int32_t* tokens, int32_t* status, hipStream_t s);
// Per-node draws of a token tree's verify rows [B, N]: row (b, n) draws from
// its own logits with Philox slot 2, j = node_depth + 1; rows n >= n_nodes[b]
// get -1.
hipError_t launch_tree_sample(const float* logits, int B, int N, int V, float inv_temp,
                              uint64_t seed, const uint64_t* step, const int32_t* node_depth,
                              const int32_t* n_nodes, int32_t* samples, int32_t* status,
                              hipStream_t s);
size_t spec_accept_ws_bytes(int B, int K);
// mq, mp [B*K]: the row maxima of zq and zp (both or neither; null: computed).
// With them and a full workspace (spec_accept_ws_bytes) every row is cut into
// chunks that separate workgroups weigh; otherwise one workgroup per row, and
// ws needs only the per-row statistics (2*B*K floats, then as many uint64).
hipError_t launch_spec_accept(const float* zq, const float* zp, const float* mq, const float* mp,
                              const int32_t* drafts, int B, int K, int V, float inv_temp,
                              uint64_t seed, const uint64_t* step, const int32_t* forced,
                              int32_t* accept_len, int32_t* committed, int32_t* extra_token,
                              int32_t* status, void* ws, hipStream_t s, bool ws_is_full = true);
// Draft sampling with the row maxima given, rows cut into chunks weighed by
// separate workgroups; sums: chunk_sums_bytes(B*K) of workspace.
size_t chunk_sums_bytes(int rows);
hipError_t launch_draft_sample_chunked(const float* logits, const float* row_max,
                                       uint64_t* sums, int B, int K, int V, float inv_temp,
                                       uint64_t seed, int slot, const uint64_t* step,
                                       int32_t* tokens, int32_t* status, hipStream_t s);

// The same on the library's per-device static scratch (no workspace; rows
// 2*B*K at most static_accept_max_rows(); the caller checks).
int static_accept_max_rows();
hipError_t launch_spec_accept_static(const float* zq, const float* zp, const float* mq,
                                     const float* mp, const int32_t* drafts, int B, int K, int V,
                                     float inv_temp, uint64_t seed, const uint64_t* step,
                                     const int32_t* forced, int32_t* accept_len,
                                     int32_t* committed, int32_t* extra_token, int32_t* status,
                                     hipStream_t s);

// ---------------------------------------------------------------- elementwise / small ops
// Block rows: draft (anchor + mask ids) or given rows; gathers embeddings into
// the fp32 residual stream h [R, D]; also writes ids [R].
// Draft rows (anchor != null): rows j >= 1 take the prior's noise (mask_id, or
// uniform tokens from (seed, step) when c.noise_prior == 1); in a later draft
// pass (block given) row j keeps block[b*K + j-1] with probability
// keep_q24 / 2^24 (Philox slot 64 + corr_pass) and otherwise returns to the
// prior (a fresh uniform token: slot 128 + corr_pass).
hipError_t launch_embed(const uno_config& c, const bf16_raw_t* embed, const int32_t* anchor,
                        const int32_t* block, const int32_t* rows, int B, int K, uint64_t seed,
                        const uint64_t* step, uint32_t keep_q24, int corr_pass, float* h,
                        int32_t* status, hipStream_t s);
// RMSNorm of fp32 rows into bf16 rows.
hipError_t launch_rmsnorm(const float* h, const float* gain, int R, int D, float eps,
                          bf16_raw_t* out, hipStream_t s);
// cos/sin table [R, head_dim/2] (fp32, angles evaluated in fp64) for the rows'
// absolute positions kv_len[b] + pos_offset + j, or kv_len[b] + pos_offset +
// depth[r] for the rows of a token tree (depth != null); and each row's K/V
// slot kv_len[b] + pos_offset + j as (page, slot in page) in row_page [R]
// (page -1, flagged in status, outside the table or the pool).  It also
// zeroes the n_zero words at `zero` (the pass's synchronisation counters).
hipError_t launch_rope_table(const uno_config& c, const uno_kv& kv, int B, int K, int pos_offset,
                             const int32_t* depth, float2* cs, int2* row_page, int32_t* status,
                             unsigned* zero, int n_zero, hipStream_t s);
// RoPE on q and k of the fused qkv rows (fp32 [R, (Hq+2Hkv)*hd]); q, scaled
// by log2(e)/sqrt(hd), -> two bf16 planes [R, Hq*hd] (hi and the rounding
// remainder lo), k/v (bf16) -> paged cache at the rows' slots.
struct RopeArgs;
hipError_t launch_rope_kv_write(const float* qkv, const RopeArgs& ra, int R, hipStream_t s);
// act = silu(g) * u, gu fp32 [R, 2F] (gate then up) -> bf16 [R, F]
hipError_t launch_silu_mul(const float* gu, int R, int F, bf16_raw_t* act, hipStream_t s);
hipError_t launch_kv_commit(int32_t* kv_len, const int32_t* accept_len, int B, int K,
                            uint64_t* step, int32_t* status, hipStream_t s);

// ---------------------------------------------------------------- tree sampler
// Workspace of launch_tree_build (top-k tokens and integer score deltas).
size_t tree_ws_bytes(int B, int K, int topk);
// Top-k of the drafted rows 1..K-1 of zq [B, K, V], the best n_keep
// candidates and their prefix tree: node_tokens/parent/depth [B, N],
// node_anc [B, N, (N+31)/32] (ancestor-or-self bits), n_nodes [B].
hipError_t launch_tree_build(const float* zq, const int32_t* draft_tokens, int B, int K, int V,
                             int topk, int n_keep, int N, int32_t* node_tokens,
                             int32_t* node_parent, int32_t* node_depth, uint32_t* node_anc,
                             int32_t* n_nodes, int32_t* status, void* ws, hipStream_t s);
// Walk of the per-node draws: accept_len [B], committed [B, K+1] (-1 padded),
// extra_token [B], path [B, K] (node at each depth, -1 padded).
hipError_t launch_tree_walk(const int32_t* node_tokens, const int32_t* node_parent,
                            const int32_t* n_nodes, const int32_t* samples, int B, int K, int N,
                            int32_t* accept_len, int32_t* committed, int32_t* extra_token,
                            int32_t* path, int32_t* status, hipStream_t s);
// Moves the walked nodes' K/V (every layer) to slots kv_len+1 .. kv_len+a-1;
// kv_len itself is advanced by launch_kv_commit afterwards.
hipError_t launch_tree_commit(const uno_config& c, const uno_kv& kv, const int32_t* path,
                              const int32_t* accept_len, int B, int K, int32_t* status,
                              hipStream_t s);

// RoPE + paged K/V write of q|k|v rows (row r's slot and page in row_page,
// (cos, sin) of its position in cs, both from launch_rope_table).
struct RopeArgs {
  const float2* cs;      // [R, hd/2]
  const int2* row_page;  // [R] (page or -1, slot in page), from launch_rope_table
  int K, Hq, Hkv, hd, ps;
  uint16_t* k_layer;     // this layer's K pages
  uint16_t* v_layer;     // this layer's V pages
  uint16_t* q_out;       // [R, Hq*hd] bf16 high part of q * log2(e)/sqrt(hd)
  uint16_t* q_lo;        // [R, Hq*hd] bf16 remainder
};
RopeArgs make_rope_args(const uno_config& c, const float2* cs, const int2* row_page,
                        const uno_kv& kv, int layer, int K, bf16_raw_t* q_out, bf16_raw_t* q_lo);

// ---------------------------------------------------------------- GEMM
// Tile-packed copy of a row-major bf16 [N, K] matrix (N % 16 == 0, K % 32 == 0):
// element (n, k) goes to ((n/16) * K/32 + k/32) * 512 + ((k%32)/8) * 128 +
// (n%16) * 8 + k%8, the layout every GEMM here reads its weight operand in.
hipError_t launch_pack_tiles(const uint16_t* src, uint16_t* dst, int N, int K, hipStream_t s);
// Y[m, n] = sum_k X[m, k] W[n, k]  (+ LoRA)  for up to 3 column segments.
struct GemmSeg {
  const bf16_raw_t* w;      // [n, K] bf16
  int n;                    // columns of this segment (multiple of 16)
  const bf16_raw_t* lora_b; // [n, r] bf16 or null
  int t_col;                // first column of this segment's LoRA input in T
};
// EPI_SWIGLU (tiled kernel only, gemm_swiglu_ok): gate|up projection with the
// SwiGLU product fused: seg[0].w holds the gate rows [F, Kd] immediately
// followed by the up rows [F, Kd] (seg[0].n = F), seg[0].lora_b likewise
// [2F, r]; T = [T_gate | T_up] (ldt = 2r); out[m, c] = bf16(silu(g) * u) [M, F].
enum GemmEpilogue { EPI_STORE_F32 = 0, EPI_ADD_F32 = 1, EPI_STORE_BF16 = 2, EPI_LORA_T = 3,
                    EPI_SWIGLU = 4 };
struct GemmArgs {
  const bf16_raw_t* x;   // [M, Kd] bf16, row stride ldx
  int M, Kd, ldx;
  GemmSeg seg[3];
  int n_seg;
  const bf16_raw_t* t;   // LoRA input [M, ldt] bf16 (already scaled and gated) or null
  int ldt, rank;
  int epi;
  void* out;             // [M, ldo]
  int ldo;
  // EPI_LORA_T: out[m, n] = bf16(scale * gate(m) * acc); gate(m) = (m % K != 0)
  float scale;
  int rows_per_seq;
  // split-K scratch (workspace) for fp32 partial tiles; null: no split
  float* part;
  size_t part_floats;
  // optional RMSNorm of the updated rows (EPI_ADD_F32 over whole rows only):
  // norm_out[m] = bf16(out[m] * rsqrt(mean(out[m]^2) + norm_eps) * norm_gain);
  // launch_gemm reports through *normed whether it did this
  const float* norm_gain;
  uint16_t* norm_out;
  float norm_eps;
  // optional RoPE + K/V write of a q|k|v product (EPI_STORE_F32, whole heads
  // per segment): when every tile is split along K, the split-K reduction
  // stores through `rope` instead of writing `out`; launch_gemm reports through
  // *roped whether it did
  int rope_fuse;
  RopeArgs rope;
  // skinny kernel (at most 64 rows): at most this many K splits (0: no cap);
  // partials_only: a split product leaves its fp32 partial sums in `part`
  // [splits][M][all columns] for a later launch and runs no reduction
  int max_splits;
  int partials_only;
  // LoRA input as the split-K partials of its LoRA-A product (set by
  // gemm_lora_pair): T = bf16(t_scale * gate(m) * sum over t_splits partials
  // [t_splits][M][ldt]), gate(m) = m % t_rows != 0; null: T is read from `t`
  const float* t_part;
  int t_splits;
  float t_scale;
  int t_rows;
  // optional SwiGLU of a [gate | up] product (EPI_STORE_F32, two segments of
  // equal width F): when the product is split along K, the split-K reduction
  // writes act_out[m, c] = bf16(silu(y[m, c]) * y[m, F + c]) [M, F] instead of
  // `out`; launch_gemm reports through *swiglued whether it did
  uint16_t* act_out;
  // optional per-row maxima of the stored outputs (EPI_STORE_F32): for each
  // of its rows every column group (a workgroup's columns; a tile of the
  // tiled kernel) gets the exact maximum over its columns in
  // max_part[m * max_part_ld + group] (max_part_ld = gemm_row_max_parts(a)
  // groups); the skinny kernel then runs without a K split, the tiled kernel
  // takes the maxima of its split tiles from their reduced rows
  float* max_part;
  int max_part_ld;
  // set by the skinny launcher (callers leave it 0): tile pairing of a fused
  // RoPE or SwiGLU epilogue without a K split
  int pair_tiles;
  // set by launch_gemm_lora (callers leave them 0): a LoRA-A product run in
  // the same launch as its projection stores its partials at the device
  // coherence point and bumps *t_signal per workgroup; the projection waits
  // until *t_wait reaches t_wait_target before its LoRA step (bounded; on
  // timeout UNO_DEV_SYNC_TIMEOUT is OR-ed into *t_timeout)
  unsigned* t_signal;
  const unsigned* t_wait;
  unsigned t_wait_target;
  int* t_timeout;
  // with t_wait: every 128-byte line of the partials was written by one
  // LoRA-A workgroup, so the projection may read them through its L2 (no
  // line of them can be cached there before the wait ends); otherwise it
  // reads them at the device coherence point
  int t_lines_owned;
  // with t_signal and t_tile_ctr (one row tile): each column group of the
  // LoRA-A product counts its finished K splits in t_tile_ctr[group]; the last
  // split to arrive sums the group's partials in split order, gates, scales
  // and rounds them into `out` (bf16 T) and only then bumps *t_signal, once
  // per group; the projection then reads T itself (t_part null)
  unsigned* t_tile_ctr;
  // skinny kernel: column tiles per workgroup (0: the planner's choice)
  int sk_nt;
};
// split-K scratch carved per pass: 128 MB for passes of more than 64 rows
// (tiled kernel), 4 MB for up to 64 (skinny kernel)
constexpr size_t kGemmPartFloats = size_t(32) << 20;
constexpr size_t kGemmPartFloatsSkinny = size_t(1) << 20;
hipError_t launch_gemm(const GemmArgs& a, hipStream_t s, bool* normed = nullptr,
                       bool* roped = nullptr, bool* swiglued = nullptr);
// A projection `a` and the LoRA-A product `ta` (EPI_LORA_T, same rows) that
// feeds its LoRA step, as two launches.  At most 64 rows: `ta` is split along
// K (at most 4 splits) with its partials left in t_part (t_part_floats of
// scratch) and no reduction launch, and `a`'s last K split sums them itself;
// otherwise both are returned unchanged (`ta` writes T, `a` reads it).
void gemm_lora_pair(const GemmArgs& a, const GemmArgs& ta, float* t_part, size_t t_part_floats,
                    GemmArgs* a_out, GemmArgs* ta_out);
// T partial scratch a pass of at most 64 rows carves for gemm_lora_pair
constexpr size_t kLoraPartFloats = size_t(1) << 18;
// counter words of one fused LoRA-A launch: the projection's wait counter and
// one split counter per LoRA-A column group
constexpr int kLoraSyncWords = 64;
// A projection `a` with the LoRA-A product `ta` that feeds it.  At most 64
// rows, when the LoRA-A product splits along K: one launch (the LoRA-A
// workgroups first, then the projection's, which wait for them through
// `counter`, kLoraSyncWords zeroed words of device memory used once), and
// *fused is set.
// Otherwise the two launches of gemm_lora_pair.  `timeout_flag` (may be
// null) receives UNO_DEV_SYNC_TIMEOUT if a wait ran out.
hipError_t launch_gemm_lora(const GemmArgs& a, const GemmArgs& ta, float* t_part,
                            size_t t_part_floats, unsigned* counter, int* timeout_flag,
                            hipStream_t s, bool* normed, bool* roped, bool* swiglued,
                            bool* fused);
// whether launch_gemm can run this EPI_SWIGLU product (the tiled kernel takes it)
bool gemm_swiglu_ok(const GemmArgs& a);
// column groups of a product with max_part set (the row-maxima partials per row)
int gemm_row_max_parts(const GemmArgs& a);
// the row-maxima partials a pass carves room for: M rows of n output columns
// in groups of 16 (at most 64 rows, the skinny kernel) or 128 (the tiled
// kernel's narrowest tile); a plan with more groups computes the maxima from
// the stored rows instead
static inline int gemm_row_max_parts_bound(int n, int M) {
  return M <= 64 ? (n + 15) / 16 : (n + 127) / 128;
}
// row_max[r] = max over parts of max_part[r * ld + part] (rows r < R)
hipError_t launch_row_max(const float* max_part, int ld, int n_parts, int R, float* row_max,
                          hipStream_t s);

// ---------------------------------------------------------------- attention
// Block attention of a pass over the paged cache.  Query rows of sequence b
// and kv head g are ordered qr = j * G + hh (G = Hq / Hkv).  Keys are split
// into n_wave_splits ranges of split_len positions (the last range runs to the
// end of the keys); every wave of the attention kernel owns one range of one
// group of 64 query rows and writes a partial (max, sum, output) that the merge
// kernel combines.
struct AttnPlan {
  int waves;            // row groups per workgroup (16 query rows each)
  int key_halves;       // waves per row group (each takes half of every chunk)
  int n_qgroups;        // groups of 16*waves query rows
  int n_wave_splits;    // key ranges per query group
  int split_len;        // keys per range (multiple of 64; the last runs to the end)
  int stages;           // KV chunks resident in LDS per workgroup (2 or 4)
};
AttnPlan attn_plan(const uno_config& c, int B, int K, int max_ctx);
size_t attn_ws_bytes(const uno_config& c, int B, int K, int max_ctx);
struct AttnArgs {
  const uint16_t* q;          // [R, Hq, hd] bf16, q * log2(e)/sqrt(hd) (high part)
  const uint16_t* q_lo;       // [R, Hq, hd] bf16, remainder of that
  const uint16_t* k_layer;    // this layer's K pages
  const uint16_t* v_layer;    // this layer's V pages (transposed inside a page)
  const int32_t* page_table;
  const int32_t* kv_len;
  int max_pages;
  int64_t n_pages;
  int B, K, pos_offset, draft;
  // token tree (verify): row j also needs bit (key - kv_len - 1) of its
  // ancestor-or-self row tree_anc[(b*K + j)*anc_words ..] for keys past kv_len
  const uint32_t* tree_anc;
  int anc_words;
  int Hq, Hkv, hd, ps, ps_shift;   // page size and its log2
  AttnPlan plan;
  float* part_o;              // [B*Hkv, n_qgroups, n_wave_splits, 64, hd]
  float* part_ml;             // [B*Hkv, n_qgroups, n_wave_splits, 64, 2]
  uint16_t* out;              // [R, Hq*hd] bf16
  int32_t* status;
};
hipError_t launch_attention(const AttnArgs& a, hipStream_t s);   // partials
hipError_t launch_attn_merge(const AttnArgs& a, hipStream_t s);  // combine -> out

}  // namespace uno
