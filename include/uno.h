/*
 * uno.h -- C ABI of the Psi-Spec draft-and-verify decode step on one gfx950 GPU.
 *
 * The method ("Unlocking Lossless Speedups in LLMs via Discrete Diffusion"):
 * a decoder whose every linear carries rank-r LoRA "diffusion weights" drafts a
 * block of tokens in one forward pass with AR + LoRA weights, verifies the
 * block in one forward pass with the AR weights alone over the same KV cache,
 * and keeps the drafted prefix that speculative rejection sampling accepts, plus
 * one residual or bonus token (picx.dev summary, "Methodology" and
 * "Psi-Speculative Sampler"; paperglide reader, "The Uno Framework",
 * "The Psi-Speculative Sampler", "Sampler Extensions").
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - Pointers marked [dev] are device (HBM) pointers; [host] are host pointers.
 *   The caller owns every buffer (weights, KV pages, page table, lengths,
 *   logits, tokens, workspace).  The library allocates and frees nothing.
 *   Mutable global state: the measurement hook of uno_set_timing_events
 *   (process-wide, not thread-safe: set it from one thread with no other call
 *   in flight), the per-thread text of uno_last_hip_error, and the per-GPU
 *   static scratch of uno_spec_accept_noalloc (calls of it that overlap on one
 *   GPU race).  Apart from these, calls on distinct buffers are re-entrant.
 * - Every call validates its host-visible arguments, then enqueues kernels on
 *   `stream` (a hipStream_t; NULL = the default stream) and returns without a
 *   host synchronisation.  No call issues hipMemset/hipMemcpy or allocates, so a
 *   whole step can be captured into a HIP graph.  Outputs are valid once the
 *   stream has reached them.
 * - Return value: UNO_OK, or an error code.  Argument, shape, capacity and
 *   workspace errors are found on the host before anything is enqueued;
 *   UNO_ERR_HIP (a launch failure) can leave the kernels launched before it
 *   enqueued, i.e. a partly run pass whose outputs are undefined.
 *   Conditions only the device can see (a kv_len that would overflow the page
 *   table, a token id outside the vocabulary, a page id outside the pool, a
 *   non-finite logit in a sampled row) are reported per sequence through the
 *   optional `status` array [dev, int32, batch]: the kernels OR bit flags
 *   UNO_DEV_* into it and skip the offending write or draw; the caller clears it.
 * - Shapes: R = batch * K rows per pass; V = vocab.  All matrices are row-major.
 * - Tokens are int32.  Random draws use Philox4x64-10 with key (seed, 0) and
 *   counter (slot, j, b, step[b]); the uniform is the top 24 bits of word 0.
 *   Slots: 0 draft token j+1; 1 accept test of draft j+1; 2 extra token (j = a;
 *   a tree node at depth d draws with j = d + 1); 3 uniform-prior noise of
 *   draft row j; 4 + i samples of intermediate draft pass i; 64 + i the
 *   corrector's keep test of draft row j after pass i, 128 + i its fresh
 *   uniform token for a remasked row.
 */
#ifndef UNO_H
#define UNO_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
  UNO_OK = 0,
  UNO_ERR_INVALID_ARG = 1,  /* null pointer, size out of range, bad stride      */
  UNO_ERR_UNSUPPORTED = 2,  /* shape the kernels do not implement              */
  UNO_ERR_CAPACITY = 3,     /* (host-checkable) page table too small for K     */
  UNO_ERR_WORKSPACE = 4,    /* workspace smaller than uno_*_workspace_bytes()  */
  UNO_ERR_HIP = 5           /* a kernel launch failed (see uno_last_hip_error) */
};

/* Device-side status bits (OR-ed into status[b]). */
enum {
  UNO_DEV_CAPACITY = 1,     /* a K/V slot fell outside the sequence's pages     */
  UNO_DEV_BAD_TOKEN = 2,    /* a token id outside [0, vocab)                    */
  UNO_DEV_BAD_PAGE = 4,     /* a page id outside [0, n_pages)                   */
  UNO_DEV_NONFINITE = 8,    /* a sampled logit row held NaN or Inf              */
  UNO_DEV_BAD_ACCEPT = 16,  /* a forced / given accept length outside [0, K]    */
  UNO_DEV_SYNC_TIMEOUT = 32 /* a projection waited too long for its LoRA-A part  */
};

/* Model shape.  Supported: head_dim 64 or 128; n_q_heads a multiple of
 * n_kv_heads; d_model, d_ffn, n_q_heads*head_dim multiples of 64; page_size a
 * power of two >= 16; lora_rank a multiple of 16 and <= 256; vocab a multiple of
 * 16 and <= 2^20. */
typedef struct uno_config {
  int32_t n_layers, d_model, n_q_heads, n_kv_heads, head_dim, d_ffn, vocab, mask_id;
  float rms_eps;      /* RMSNorm epsilon                                      */
  float rope_theta;   /* rotate-half RoPE base                                */
  int32_t lora_rank;  /* r                                                    */
  float lora_scale;   /* alpha / r                                            */
  uint32_t lora_mask; /* bit p set: LoRA on projection p; p = 0 q, 1 k, 2 v,
                         3 o, 4 gate, 5 up, 6 down.  q,k,v must agree, and
                         gate,up must agree.                                  */
  int32_t page_size;  /* tokens per KV page (16)                              */
  int32_t noise_prior; /* noise tokens of a draft block (paperglide reader,
                          "The Psi-Speculative Sampler": the block is the
                          anchor plus K-1 tokens drawn from the diffusion
                          prior; "Supplementary Details": a masked model's
                          prior is the mask token, a uniform-state model's is
                          uniform over the vocabulary).
                          0: mask_id at every noise position;
                          1: uniform token ids, floor(w * vocab / 2^64) with w
                             word 0 of Philox4x64-10 at counter (3, j, b,
                             step[b]), key (seed, 0), for draft row j >= 1.  */
} uno_config;

/* One layer's weights [dev].  Base weights W [out, in] and LoRA factors A
 * [r, in] are bf16 in the tile-packed layout uno_pack_weight writes (the
 * layout of the matrix cores' weight operand, so that every 16 x 32 fragment
 * is 1 KB of contiguous memory); LoRA factors B [out, r] are bf16 row-major;
 * norm gains are fp32 [d_model].  LoRA pointers of projections whose bit is
 * clear in lora_mask are ignored. */
typedef struct uno_layer_weights {
  const void *attn_norm, *mlp_norm;                    /* fp32 [D]             */
  const void *wq, *wk, *wv, *wo, *wgate, *wup, *wdown; /* bf16                  */
  const void *lora_a[7];                               /* bf16 [r, in_p]        */
  const void *lora_b[7];                               /* bf16 [out_p, r]       */
} uno_layer_weights;

typedef struct uno_weights {
  const void *embed;       /* bf16 [V, D] [dev], row-major                      */
  const void *lm_head;     /* bf16 [V, D] [dev], tile-packed (untied, no LoRA)  */
  const void *final_norm;  /* fp32 [D]    [dev]                                 */
  const uno_layer_weights *layers; /* [host] array of n_layers                  */
} uno_weights;

/* Paged KV cache shared by the draft and the verify pass.
 * k_pages: bf16 [n_layers][n_pages][n_kv_heads][page_size][head_dim]
 * v_pages: bf16 [n_layers][n_pages][n_kv_heads][head_dim][page_size]
 *          (V is stored transposed inside a page: the keys of one page are
 *           contiguous for each channel)
 * Token position t of sequence b lives in page page_table[b*max_pages + t/ps]
 * at slot t % ps.  kv_len[b] counts the committed positions; positions
 * kv_len[b].. are scratch that the next pass overwrites. */
typedef struct uno_kv {
  void *k_pages, *v_pages;       /* [dev]                                     */
  int64_t n_pages;               /* pages per layer in the pool               */
  const int32_t *page_table;     /* [dev] int32 [batch, max_pages_per_seq]    */
  int32_t max_pages_per_seq;
  int32_t *kv_len;               /* [dev] int32 [batch]                       */
} uno_kv;

/* Tile-packed copy of a row-major bf16 matrix (a weight's layout on the
 * device): src [dev] bf16 [n_out, n_in] row-major, dst [dev] bf16 of the same
 * size (distinct buffers); element (n, k) goes to
 *   ((n / 16) * (n_in / 32) + k / 32) * 512 + ((k % 32) / 8) * 128 + (n % 16) * 8 + k % 8.
 * n_out % 16 == 0, n_in % 32 == 0.  Enqueued on `stream`. */
int uno_pack_weight(const void *src, void *dst, int n_out, int n_in, void *stream);

/* Bytes of workspace the two forward passes need for `batch` sequences of up
 * to `K` rows and up to `max_ctx` cached positions (the split of the attention
 * over the context is sized from it). */
size_t uno_workspace_bytes(const uno_config *cfg, int batch, int K, int max_ctx);

/* Draft block (paperglide reader, "The Psi-Speculative Sampler" and "Sampler
 * Extensions"; picx.dev summary, "Architecture").
 * Rows of sequence b: [anchor[b], noise x (K-1)] at positions kv_len[b] ..
 * kv_len[b]+K-1, the noise tokens being mask_id or uniform Philox draws as
 * cfg->noise_prior says.  Row 0 runs with the AR weights and attends causally (keys
 * <= kv_len[b]); rows 1..K-1 add the LoRA term (scale lora_scale) and attend to
 * every key up to kv_len[b]+K-1.  The pass writes the rows' K/V into the cache
 * at those positions (the anchor's entry is final; the mask rows' are scratch)
 * and leaves kv_len unchanged.
 *   anchor        [dev] int32 [batch]
 *   draft_logits  [dev] fp32 [batch, K, V]   q_1..q_K (untempered logits)
 *   draft_tokens  [dev] int32 [batch, K]     d_j+1 ~ q_j+1 at temperature 1/inv_temp
 *   row_max       [dev] fp32 [batch, K] or NULL: receives the exact maximum of
 *                 every draft logits row (the LM head's epilogue finds it, so
 *                 the sampler streams each row once); pass it to
 *                 uno_spec_accept as draft_row_max
 *   step          [dev] uint64 [batch]       Philox step counter per sequence
 *                                            (draft sampling; uniform noise)
 *   status        [dev] int32 [batch] or NULL
 *   ws/ws_bytes   [dev] workspace of uno_workspace_bytes(cfg, batch, K, max_ctx)
 * 1 <= K <= 64, batch >= 1, inv_temp > 0 and finite. */
int uno_draft_block(const uno_config *cfg, const uno_weights *w, const uno_kv *kv,
                    const int32_t *anchor, int batch, int K, int max_ctx,
                    float inv_temp, uint64_t seed, const uint64_t *step,
                    float *draft_logits, int32_t *draft_tokens, float *row_max,
                    int32_t *status, void *ws, size_t ws_bytes, void *stream);

/* One draft pass of a multi-pass draft (paperglide reader, "Supplementary
 * Details": Psi-samplers are predictor-corrector samplers that refine a block
 * over several denoising steps; a correction strength kappa_t in [0, 1]
 * interpolates between ancestral sampling (kappa_t = 1) and the forward
 * noising process, which remasks a masked model's tokens and re-draws a
 * uniform-state model's).  Same as uno_draft_block, except that
 *   block        [dev] int32 [batch, K] or NULL: when given, draft row j in
 *                1..K-1 of sequence b is the corrector's output for the token
 *                block[b*K + j-1] (the token d_j the previous pass sampled): it
 *                is kept iff keep_q24 == 2^24 or U < keep_q24, U the 24-bit
 *                uniform of Philox counter (64 + corr_pass, j, b, step[b]);
 *                otherwise the row returns to the prior: mask_id, or (noise
 *                prior 1) the uniform token floor(w * vocab / 2^64), w word 0
 *                of counter (128 + corr_pass, j, b, step[b]).  block may
 *                alias draft_tokens (it is read before draft_tokens is written);
 *   sample_slot  Philox slot of this pass's draft sampling: 0 for the pass
 *                whose drafts go to verification (as uno_draft_block), 4 + i
 *                for intermediate pass i (4 <= sample_slot <= 63);
 *   keep_q24     round(kappa * 2^24) in [0, 2^24] (ignored without block);
 *   corr_pass    index of the pass whose samples the block holds (0..59).
 * Only the final pass's logits and tokens enter uno_spec_accept; conditional
 * on everything drawn before it that pass is an ordinary draft, so the decode
 * stays lossless for any number of passes and any kappa. */
int uno_draft_block_from(const uno_config *cfg, const uno_weights *w, const uno_kv *kv,
                         const int32_t *anchor, const int32_t *block, int batch, int K,
                         int max_ctx, float inv_temp, uint64_t seed, const uint64_t *step,
                         int sample_slot, uint32_t keep_q24, int corr_pass,
                         float *draft_logits, int32_t *draft_tokens, float *row_max,
                         int32_t *status, void *ws, size_t ws_bytes, void *stream);

/* Verify block (picx.dev summary, "Architecture": verification uses the AR
 * weights only).  Rows of sequence b: rows[b, 0..K-1] at positions
 * kv_len[b] + pos_offset + j, causal (row j sees keys <= its own position),
 * no LoRA.  Writes the rows' K/V into the cache (pending until a commit).
 * pos_offset = 1 after a draft block (the anchor sits at kv_len[b]);
 * pos_offset = 0 for a prompt chunk (prefill, followed by a commit with
 * accept_len = K-1).  verify_logits [dev] fp32 [batch, K, V] may be NULL to
 * skip the LM head.  row_max [dev] fp32 [batch, K] or NULL (and NULL when
 * verify_logits is) receives the exact maximum of every logits row, for
 * uno_spec_accept's verify_row_max.  1 <= K <= 4096. */
int uno_verify_block(const uno_config *cfg, const uno_weights *w, const uno_kv *kv,
                     const int32_t *rows, int batch, int K, int max_ctx, int pos_offset,
                     float *verify_logits, float *row_max, int32_t *status,
                     void *ws, size_t ws_bytes, void *stream);

/* Draft sampling alone (the categorical draw that uno_draft_block ends with):
 * tokens[b, j] = integer-weight categorical draw from logits[b, j, :] at
 * temperature 1/inv_temp with the slot-0 uniform of (j, b, step[b]).
 * logits [dev] fp32 [batch, K, V]; tokens [dev] int32 [batch, K]; row_max
 * [dev] fp32 [batch, K] or NULL: the exact maximum of each row (then each row
 * is streamed once; an entry that is not finite or exceeds its row's given
 * maximum flags UNO_DEV_NONFINITE and the row's token is -1). */
int uno_draft_sample(const float *logits, const float *row_max, int batch, int K, int vocab,
                     float inv_temp, uint64_t seed, const uint64_t *step, int32_t *tokens,
                     int32_t *status, void *stream);

/* Workspace for uno_spec_accept: per-row statistics of both logit sets. */
size_t uno_spec_accept_workspace_bytes(int batch, int K);

/* Lossless accept / resample (picx.dev summary, "Psi-Speculative Sampler";
 * paperglide reader, "The Psi-Speculative Sampler", "Sampler Extensions").
 * Draft row j of sequence b is q_{j+1}; verify row j is p_{j+2}; p_1 = q_1, so
 * d_1 is always kept.  For i = 2..K: keep d_i iff
 *   U * Wq_i[d_i] * Sp_i < Wp_i[d_i] * Sq_i * 2^24
 * (integer weights W = floor(exp_c((z - max z) * inv_temp) * 2^31), zero below
 * -22, S their exact sum), stopping at the first rejection; a = kept drafts.
 * If forced_accept != NULL, a = forced_accept[b] in [0, K] replaces it.
 * a < K: extra token ~ R_v = max(0, Wp_{a+1,v} Sq_{a+1} - Wq_{a+1,v} Sp_{a+1})
 * (p_{a+1} itself if R is all zero); a = K: bonus token ~ p_{K+1}.
 *   draft_logits, verify_logits [dev] fp32 [batch, K, V]
 *   draft_row_max, verify_row_max [dev] fp32 [batch, K], both or neither: the
 *                exact row maxima the passes wrote (row_max of
 *                uno_draft_block / uno_verify_block); with them every logits
 *                row is streamed once, and an entry that is not finite or
 *                exceeds its given maximum flags UNO_DEV_NONFINITE
 *   draft_tokens [dev] int32 [batch, K]
 *   forced_accept [dev] int32 [batch] or NULL
 *   accept_len   [dev] int32 [batch]           a
 *   committed    [dev] int32 [batch, K+1]      d_1..d_a, extra, then -1
 *   extra_token  [dev] int32 [batch]           the new anchor
 *   ws/ws_bytes  [dev] uno_spec_accept_workspace_bytes(batch, K) bytes */
int uno_spec_accept(const float *draft_logits, const float *verify_logits,
                    const float *draft_row_max, const float *verify_row_max,
                    const int32_t *draft_tokens, int batch, int K, int vocab,
                    float inv_temp, uint64_t seed, const uint64_t *step,
                    const int32_t *forced_accept, int32_t *accept_len,
                    int32_t *committed, int32_t *extra_token, int32_t *status,
                    void *ws, size_t ws_bytes, void *stream);

/* uno_spec_accept without a workspace, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc).  Same arguments, results and device status flags as
 * uno_spec_accept, minus ws/ws_bytes: the per-row statistics live in a static
 * scratch array of the library (768 KiB per GPU, held until the process ends)
 * that serves at most 2 * batch * K <= 65536 rows; larger shapes return
 * UNO_ERR_WORKSPACE before anything is enqueued.  The first call on a device
 * looks up that device's copy of the array (a host-side lookup, no
 * allocation).  Every call on one GPU shares its array: calls that overlap on
 * one GPU (two streams, two threads) race and must be ordered by the caller. */
int uno_spec_accept_noalloc(const float *draft_logits, const float *verify_logits,
                            const float *draft_row_max, const float *verify_row_max,
                            const int32_t *draft_tokens, int batch, int K, int vocab,
                            float inv_temp, uint64_t seed, const uint64_t *step,
                            const int32_t *forced_accept, int32_t *accept_len,
                            int32_t *committed, int32_t *extra_token, int32_t *status,
                            void *stream);

/* KV commit / rollback (picx.dev summary, "Practical Implications": one KV
 * cache serves drafting and verification).  kv_len[b] += 1 + accept_len[b]:
 * the anchor and the kept drafts stay, every later position becomes scratch
 * that the next pass overwrites.  step[b] += 1 when step != NULL.  An
 * accept_len outside [0, K] sets UNO_DEV_BAD_ACCEPT and leaves kv_len[b]. */
int uno_kv_commit(const uno_kv *kv, const int32_t *accept_len, int batch, int K,
                  uint64_t *step, int32_t *status, void *stream);

/* ---------------------------------------------------------------- tree sampler
 * The per-request variant of the step (picx.dev summary, "Psi-Speculative
 * Sampler", tree sampler; paperglide reader, "The Psi-Speculative Sampler",
 * worked example and step list; "Empirical Results", parameters (B, K, V)).
 * With the block length K here (the pages' B), topk (their K) and n_keep (their
 * V): one draft pass (uno_draft_block; only its token d_1 of row 0 is used) ->
 * uno_tree_build -> uno_verify_tree -> uno_tree_accept -> uno_tree_commit.
 * The pages leave the arithmetic and the multi-candidate accept rule open; the
 * readings implemented:
 *  - top-k of a drafted row: the k largest fp32 logits, equal values by id;
 *  - candidates: d_1 followed by one top-k token of each drafted row 1..K-1;
 *    score = sum over rows of rint(fp32(z[token] - z[top-1]) * 2^20) (floored
 *    at -2^40) in exact int64, which ranks like the joint log-probability at
 *    any temperature; ties by the rank tuples, lexicographically; the best
 *    n_keep are kept;
 *  - tree: node 0 = d_1; the kept candidates, best first, add their new
 *    prefixes as nodes, by depth.  A sequence always has N = uno_tree_rows()
 *    node rows; rows n >= n_nodes[b] repeat d_1 at depth 0 and are inert;
 *  - walk (lossless): at node u draw x from the verify row of u (integer
 *    sampler, Philox slot 2, j = depth(u) + 1); move to the child holding x,
 *    else stop.  a = nodes walked (d_1 included); the step commits their
 *    tokens and x.  Every token is an exact AR draw, so the output law is the
 *    AR model's. */

/* Node rows per sequence, N = 1 + n_keep * (K - 1); 0 if the shape is out of
 * range (2 <= K <= 32, 1 <= topk <= 8, 1 <= n_keep <= min(64, topk^(K-1))). */
int uno_tree_rows(int K, int topk, int n_keep);

/* Workspace for uno_tree_build (per-row top-k ids and score terms). */
size_t uno_tree_workspace_bytes(int batch, int K, int topk);

/* Tree of one step per sequence from the draft pass's outputs.
 *   draft_logits [dev] fp32 [batch, K, V]; draft_tokens [dev] int32 [batch, K]
 *   (only column 0, d_1, is read)
 *   node_tokens, node_parent, node_depth [dev] int32 [batch, N]
 *   node_anc  [dev] uint32 [batch, N, (N+31)/32]: bit m of row n set iff node m
 *             is n or an ancestor of n
 *   n_nodes   [dev] int32 [batch]
 * A non-finite drafted row sets UNO_DEV_NONFINITE and gives token -1 (the
 * verify pass then flags UNO_DEV_BAD_TOKEN). */
int uno_tree_build(const float *draft_logits, const int32_t *draft_tokens, int batch, int K,
                   int vocab, int topk, int n_keep, int32_t *node_tokens,
                   int32_t *node_parent, int32_t *node_depth, uint32_t *node_anc,
                   int32_t *n_nodes, int32_t *status, void *ws, size_t ws_bytes,
                   void *stream);

/* Tree-masked verify pass (AR weights) over the node rows, n_rows = N.  Node n
 * sits at position kv_len[b] + 1 + depth(n); its K/V go to slot
 * kv_len[b] + 1 + n; it attends to slots <= kv_len[b] (context and anchor) and
 * to the slots of its ancestors and itself.  verify_logits [dev] fp32
 * [batch, N, V] (rows past n_nodes are inert).  ws: uno_workspace_bytes(cfg,
 * batch, N, max_ctx); the page table must cover kv_len + 1 + N slots. */
int uno_verify_tree(const uno_config *cfg, const uno_weights *w, const uno_kv *kv,
                    const int32_t *node_tokens, const int32_t *node_depth,
                    const uint32_t *node_anc, int batch, int n_rows, int max_ctx,
                    float *verify_logits, int32_t *status, void *ws, size_t ws_bytes,
                    void *stream);

/* Accept walk.  node_sample [dev] int32 [batch, N]: the draw of every node
 * (-1 past n_nodes); accept_len [dev] int32 [batch] (a >= 1); committed [dev]
 * int32 [batch, K+1] (the a walked tokens, then x, then -1); extra_token [dev]
 * int32 [batch] (x, the next anchor); path [dev] int32 [batch, K] (node at
 * each depth, then -1).  A non-finite verify row sets UNO_DEV_NONFINITE, a = 0
 * and committed = -1. */
int uno_tree_accept(const float *verify_logits, const int32_t *node_tokens,
                    const int32_t *node_parent, const int32_t *node_depth,
                    const int32_t *n_nodes, int batch, int K, int n_rows, int vocab,
                    float inv_temp, uint64_t seed, const uint64_t *step,
                    int32_t *node_sample, int32_t *accept_len, int32_t *committed,
                    int32_t *extra_token, int32_t *path, int32_t *status, void *stream);

/* Commit of a tree step: the K/V of path[b, d] (every layer) move from slot
 * kv_len + 1 + path[b, d] to kv_len + 1 + d for d = 1..a-1, then kv_len[b] +=
 * 1 + a and step[b] += 1 (as uno_kv_commit). */
int uno_tree_commit(const uno_config *cfg, const uno_kv *kv, const int32_t *path,
                    const int32_t *accept_len, int batch, int K, uint64_t *step,
                    int32_t *status, void *stream);

/* Measurement hook (not part of the decode path; for benchmarks and
 * profilers).  While set, every launch of one kernel class made by the entry
 * points above is bracketed by hipEventRecord(start[i]) / hipEventRecord(stop[i])
 * on the launching stream, i = 0, 1, ... until n pairs are used; later
 * launches are not bracketed.  start/stop are [host] arrays of hipEvent_t
 * owned by the caller and must outlive their use.  kernel_class 0 clears the
 * hook.  The hook is process-wide state: set it from one thread, with no other
 * call of this library in flight.  uno_timing_events_used() returns i. */
enum {
  UNO_TIME_ATTENTION = 1, /* block attention (the split-KV partial kernel)    */
  UNO_TIME_GEMM = 2,      /* the four projections of every layer (q|k|v, o,
                             gate|up, down), LoRA B fused when drafting       */
  UNO_TIME_LORA_A = 3,    /* the LoRA A products (x A^T, gated and scaled)
                             launched on their own (passes of more than 64
                             rows; at most 64 they share their projection's
                             launch and count in its class)                   */
  UNO_TIME_LM_HEAD = 4,   /* the final vocabulary projection                  */
  UNO_TIME_SAMPLER = 5,   /* draft sampling and the accept / resample kernels */
  /* one projection of every layer (also counted in UNO_TIME_GEMM); a launch
   * is the GEMM plus, when K is split, its ordered reduction kernel         */
  UNO_TIME_GEMM_QKV = 6,
  UNO_TIME_GEMM_O = 7,
  UNO_TIME_GEMM_GATE_UP = 8,
  UNO_TIME_GEMM_DOWN = 9
};
int uno_set_timing_events(int kernel_class, void *const *start, void *const *stop, int n);
int uno_timing_events_used(void);

/* Text of a status code, and of the last HIP error a call reported. */
const char *uno_status_string(int status);
const char *uno_last_hip_error(void);

#ifdef __cplusplus
}
#endif
#endif /* UNO_H */
