// Vocabulary-wide sampler of the Psi-Spec step for gfx950: draft sampling,
// per-row statistics, accept tests, first-rejection index and the residual or
// bonus token ("Unlocking Lossless Speedups in LLMs via Discrete Diffusion",
// paperglide reader, "The Psi-Speculative Sampler"; picx.dev summary,
// "Psi-Speculative Sampler").
//
// Arithmetic contract (bit-exact, order free):
//   x_v = fp32((z_v - max z) * inv_temp);  W_v = x_v < -22 ? 0 : floor(expc(x_v) * 2^31)
//   S = exact integer sum of W;  a draw with 24-bit U returns the smallest v whose
//   running sum exceeds floor(U * S / 2^24).
//   keep d iff U * Wq[d] * Sp < Wp[d] * Sq * 2^24 (128-bit integers).
//   residual R_v = max(0, Wp_v * Sq - Wq_v * Sp) (128-bit integers).
// expc is Cody-Waite reduction by ln 2 (16-bit head + fp32 tail), a degree-7
// Taylor polynomial in Horner form and an exact ldexp, each operation a single
// rounded fp32 op: contraction into FMA is switched off in this file.
//
// Layout: logits are fp32 rows of V entries; row (b, j) of a [B, K, V] tensor
// starts at (b*K + j)*V.  Each row is handled by one workgroup of 4 waves (16
// when there are fewer than 512 rows); rows are streamed with 16-byte loads
// when V % 4 == 0.
#include "uno_device.h"
#include "uno_internal.h"

#pragma clang fp contract(off)

namespace uno {

// ------------------------------------------------------------ Philox draws
// (philox_word0: uno_device.h) 24-bit uniform = top 24 bits of word 0.
__device__ __forceinline__ uint32_t uniform24(uint64_t seed, uint64_t slot, uint64_t j,
                                              uint64_t b, uint64_t step) {
  return (uint32_t)(philox_word0(slot, j, b, step, seed, 0) >> 40);
}

// ------------------------------------------------------------ canonical exp
// fp32 constants: 1/ln 2; ln 2 rounded to 16 significant bits (so n * head is
// exact for |n| <= 32); fp32(ln 2 - head); fp32(1/k!) for k = 0..7.
__device__ __forceinline__ float expc(float x) {
  const float kLog2e = 0x1.715476p+0f;
  const float kLn2Hi = 0x1.62e4p-1f;
  const float kLn2Lo = 0x1.7f7d1cp-20f;
  const float n = __builtin_rintf(x * kLog2e);
  const float r = (x - n * kLn2Hi) - n * kLn2Lo;
  float p = 0x1.a01a02p-13f;          // 1/7!
  p = p * r; p = p + 0x1.6c16c2p-10f; // 1/6!
  p = p * r; p = p + 0x1.111112p-7f;  // 1/5!
  p = p * r; p = p + 0x1.555556p-5f;  // 1/4!
  p = p * r; p = p + 0x1.555556p-3f;  // 1/3!
  p = p * r; p = p + 0.5f;            // 1/2!
  p = p * r; p = p + 1.0f;            // 1/1!
  p = p * r; p = p + 1.0f;            // 1/0!
  return __builtin_ldexpf(p, (int)n);
}

__device__ __forceinline__ uint32_t weight_of(float z, float m, float inv_temp) {
  const float x = (z - m) * inv_temp;
  if (!(x >= -22.0f)) return 0u;
  return (uint32_t)(expc(x) * 2147483648.0f);
}

// t = floor(U * S / 2^24) for S < 2^104
__device__ __forceinline__ u128 scaled_target(uint32_t U, u128 S) {
  const u128 p0 = mul_64x64((uint64_t)U, S.lo);
  const uint64_t hi = p0.hi + (uint64_t)U * S.hi;
  return u128_make((p0.lo >> 24) | (hi << 40), hi >> 24);
}

// ------------------------------------------------------------ row access
struct Row {
  const float* p;
  int V;
  bool vec;
  // the four entries e0..e0+3 (entries past V reported as absent)
  __device__ __forceinline__ void load4(int e0, float v[4], bool ok[4]) const {
    if (vec && e0 + 3 < V) {
      const float4 f = *reinterpret_cast<const float4*>(p + e0);
      v[0] = f.x; v[1] = f.y; v[2] = f.z; v[3] = f.w;
      ok[0] = ok[1] = ok[2] = ok[3] = true;
    } else {
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        ok[c] = e0 + c < V;
        v[c] = ok[c] ? p[e0 + c] : 0.0f;
      }
    }
  }
};

constexpr int kTile = UNO_WAVE * 4;  // entries per wave tile

// TH: threads per workgroup (one workgroup per row).
template <int TH>
struct RowShared {
  float red_f[TH / UNO_WAVE];
  int red_i[TH / UNO_WAVE];
  u128 red_u[TH / UNO_WAVE];
  u128 found_before;
  int found_tile;
  int result;
};

// Block-wide max of a row; sets *nonfinite if any entry is NaN/Inf.
// Rows are streamed kUnroll groups of four entries per thread at a time, their
// loads issued together, so that every wave keeps several requests in flight.
constexpr int kUnroll = 4;

template <int TH>
__device__ float block_row_max(const Row& row, RowShared<TH>& sh, bool* nonfinite) {
  float m = -INFINITY;
  int bad = 0;
  for (int e0 = threadIdx.x * 4; e0 < row.V; e0 += TH * 4 * kUnroll) {
    float v[kUnroll][4];
    bool ok[kUnroll][4];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) row.load4(e0 + u * TH * 4, v[u], ok[u]);
#pragma unroll
    for (int u = 0; u < kUnroll; ++u)
#pragma unroll
      for (int c = 0; c < 4; ++c)
        if (ok[u][c]) {
          bad |= !__builtin_isfinite(v[u][c]);
          m = fmaxf(m, v[u][c]);
        }
  }
  m = wave_max(m);
  bad = __any(bad);
  const int w = threadIdx.x / UNO_WAVE;
  if (lane_id() == 0) { sh.red_f[w] = m; sh.red_i[w] = bad; }
  __syncthreads();
  float r = sh.red_f[0];
  int rb = sh.red_i[0];
  for (int i = 1; i < (TH / UNO_WAVE); ++i) { r = fmaxf(r, sh.red_f[i]); rb |= sh.red_i[i]; }
  __syncthreads();
  *nonfinite = rb != 0;
  return r;
}

// Weight functors: four consecutive entries' integer weights.
// (load: the raw entries; weights: their integer weights; get4: both)
struct PlainWeights {  // W of one row
  Row row;
  float m, inv_temp;
  struct Raw {
    float v[4];
    bool ok[4];
  };
  __device__ __forceinline__ void load(int e0, Raw& r) const { row.load4(e0, r.v, r.ok); }
  __device__ __forceinline__ void weights(const Raw& r, u128 w[4]) const {
#pragma unroll
    for (int c = 0; c < 4; ++c) w[c] = u128_make(r.ok[c] ? weight_of(r.v[c], m, inv_temp) : 0u, 0);
  }
  __device__ __forceinline__ void get4(int e0, u128 w[4]) const {
    Raw r;
    load(e0, r);
    weights(r, w);
  }
};

struct ResidualWeights {  // max(0, Wp Sq - Wq Sp) of a row pair
  Row p, q;
  float mp, mq, inv_temp;
  uint64_t sp, sq;
  struct Raw {
    float vp[4], vq[4];
    bool okp[4], okq[4];
  };
  __device__ __forceinline__ void load(int e0, Raw& r) const {
    p.load4(e0, r.vp, r.okp);
    q.load4(e0, r.vq, r.okq);
  }
  __device__ __forceinline__ void weights(const Raw& r, u128 w[4]) const {
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      w[c] = u128_make(0, 0);
      if (r.okp[c]) {
        const u128 a = mul_64x64(weight_of(r.vp[c], mp, inv_temp), sq);
        const u128 b = mul_64x64(weight_of(r.vq[c], mq, inv_temp), sp);
        if (u128_lt(b, a)) w[c] = u128_sub(a, b);
      }
    }
  }
  __device__ __forceinline__ void get4(int e0, u128 w[4]) const {
    Raw r;
    load(e0, r);
    weights(r, w);
  }
};

// Sum of all weights; tile sums (kTile entries each) go to `tiles` (LDS).
template <int TH, class WF>
__device__ u128 block_weight_sum(const WF& wf, int V, u128* tiles, RowShared<TH>& sh) {
  const int w = threadIdx.x / UNO_WAVE, l = lane_id();
  const int n_tiles = (V + kTile - 1) / kTile;
  constexpr int NW = TH / UNO_WAVE;
  u128 acc = u128_make(0, 0);
  for (int t = w; t < n_tiles; t += kUnroll * NW) {
    typename WF::Raw raw[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) wf.load((t + u * NW) * kTile + l * 4, raw[u]);   // past V: no load
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      if (t + u * NW >= n_tiles) break;
      u128 v[4];
      wf.weights(raw[u], v);
      u128 s = u128_add(u128_add(v[0], v[1]), u128_add(v[2], v[3]));
      s = wave_sum_u128(s);
      if (l == 0) tiles[t + u * NW] = s;
      acc = u128_add(acc, s);
    }
  }
  if (l == 0) sh.red_u[w] = acc;
  __syncthreads();
  u128 tot = sh.red_u[0];
  for (int i = 1; i < (TH / UNO_WAVE); ++i) tot = u128_add(tot, sh.red_u[i]);
  __syncthreads();
  return tot;
}

// Smallest entry whose running weight sum exceeds `t` (t < total).  Needs the
// tile sums from block_weight_sum.  Every thread returns the index.
template <int TH, class WF>
__device__ int block_find(const WF& wf, int V, const u128* tiles, u128 t, RowShared<TH>& sh) {
  const int w = threadIdx.x / UNO_WAVE, l = lane_id();
  const int n_tiles = (V + kTile - 1) / kTile;
  if (w == 0) {
    u128 base = u128_make(0, 0);
    int tile = -1;
    u128 before = base;
    for (int t0 = 0; t0 < n_tiles && tile < 0; t0 += UNO_WAVE) {
      const u128 v = (t0 + l < n_tiles) ? tiles[t0 + l] : u128_make(0, 0);
      const u128 incl = u128_add(wave_inclusive_scan_u128(v), base);
      const uint64_t hit = __ballot(u128_lt(t, incl));
      if (hit) {
        const int f = __ffsll((long long)hit) - 1;
        tile = t0 + f;
        before = u128_sub(u128_shfl(incl, f), u128_shfl(v, f));
      } else {
        base = u128_shfl(incl, UNO_WAVE - 1);
      }
    }
    if (l == 0) { sh.found_tile = tile; sh.found_before = before; }
  }
  __syncthreads();
  const int tile = sh.found_tile;
  if (w == 0) {
    int res = -1;
    if (tile >= 0) {
      const int e0 = tile * kTile + l * 4;
      u128 v[4];
      wf.get4(e0, v);
      u128 mine = u128_add(u128_add(v[0], v[1]), u128_add(v[2], v[3]));
      const u128 incl = wave_inclusive_scan_u128(mine);
      u128 run = u128_add(sh.found_before, u128_sub(incl, mine));
      int cand = -1;
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        run = u128_add(run, v[c]);
        if (cand < 0 && u128_lt(t, run)) cand = e0 + c;
      }
      const uint64_t hit = __ballot(cand >= 0);
      if (hit) res = __shfl(cand, __ffsll((long long)hit) - 1, UNO_WAVE);
    }
    if (l == 0) sh.result = res;
  }
  __syncthreads();
  const int r = sh.result;
  __syncthreads();
  return r;
}

__device__ __forceinline__ void flag(int32_t* status, int b, int32_t f) {
  if (status) atomicOr(status + b, f);
}

// ------------------------------------------------------------ kernels
// One workgroup per draft row (b, j): d = categorical(W(row), U(slot, j, b, step[b]));
// slot 0 for the drafts that go to verification, 4 + i for the samples of an
// intermediate draft pass i.  Token-tree rows (row_j != null) draw with
// j = row_j[row] + j_add, and rows at or past n_valid[b] are skipped (-1).
template <int TH>
__global__ void __launch_bounds__(TH)
k_draft_sample(const float* __restrict__ logits, int K, int V, float inv_temp, uint64_t seed,
               int slot, const uint64_t* __restrict__ step, int32_t* __restrict__ tokens,
               int32_t* __restrict__ status, const int32_t* __restrict__ row_j, int j_add,
               const int32_t* __restrict__ n_valid) {
  extern __shared__ u128 tiles[];
  __shared__ RowShared<TH> sh;
  const int row_id = blockIdx.x;
  const int b = row_id / K;
  if (n_valid && row_id % K >= n_valid[b]) {
    if (threadIdx.x == 0) tokens[row_id] = -1;
    return;
  }
  const int j = row_j ? row_j[row_id] + j_add : row_id % K;
  Row row{logits + (size_t)row_id * V, V, (V & 3) == 0};
  bool bad = false;
  const float m = block_row_max(row, sh, &bad);
  if (bad) {
    if (threadIdx.x == 0) { tokens[row_id] = -1; flag(status, b, UNO_DEV_NONFINITE); }
    return;
  }
  PlainWeights wf{row, m, inv_temp};
  const u128 S = block_weight_sum(wf, V, tiles, sh);
  const uint32_t U = uniform24(seed, slot, j, b, step[b]);
  const int v = block_find(wf, V, tiles, scaled_target(U, S), sh);
  if (threadIdx.x == 0) tokens[row_id] = v;
}

// One workgroup per row of the concatenated [draft rows; verify rows]:
// row maximum and exact weight sum (fits 64 bits: V <= 2^20, W <= 2^31).
template <int TH>
__global__ void __launch_bounds__(TH)
k_row_stats(const float* __restrict__ zq, const float* __restrict__ zp, int K, int V,
            int n_rows_each, float inv_temp, float* __restrict__ m_out,
            uint64_t* __restrict__ s_out, int32_t* __restrict__ status) {
  __shared__ RowShared<TH> sh;
  const int r = blockIdx.x;
  const bool is_p = r >= n_rows_each;
  const int rr = is_p ? r - n_rows_each : r;
  Row row{(is_p ? zp : zq) + (size_t)rr * V, V, (V & 3) == 0};
  bool bad = false;
  const float m = block_row_max(row, sh, &bad);
  uint64_t acc = 0;
  if (!bad) {
    for (int e0 = threadIdx.x * 4; e0 < V; e0 += TH * 4 * kUnroll) {
      float v[kUnroll][4];
      bool ok[kUnroll][4];
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) row.load4(e0 + u * TH * 4, v[u], ok[u]);
#pragma unroll
      for (int u = 0; u < kUnroll; ++u)
#pragma unroll
        for (int c = 0; c < 4; ++c)
          if (ok[u][c]) acc += weight_of(v[u][c], m, inv_temp);
    }
  }
  acc = wave_sum_u64(acc);
  const int w = threadIdx.x / UNO_WAVE;
  if (lane_id() == 0) sh.red_u[w] = u128_make(acc, 0);
  __syncthreads();
  if (threadIdx.x == 0) {
    uint64_t tot = 0;
    for (int i = 0; i < (TH / UNO_WAVE); ++i) tot += sh.red_u[i].lo;
    m_out[r] = m;
    s_out[r] = bad ? 0ull : tot;
    if (bad) flag(status, rr / K, UNO_DEV_NONFINITE);
  }
}

// One workgroup per sequence: accept tests, a, extra token, outputs.
template <int TH>
__global__ void __launch_bounds__(TH)
k_spec_accept(const float* __restrict__ zq, const float* __restrict__ zp,
              const int32_t* __restrict__ drafts, int K, int V, float inv_temp,
              uint64_t seed, const uint64_t* __restrict__ step,
              const int32_t* __restrict__ forced, const float* __restrict__ m_all,
              const uint64_t* __restrict__ s_all, int n_rows_each,
              int32_t* __restrict__ accept_len, int32_t* __restrict__ committed,
              int32_t* __restrict__ extra_token, int32_t* __restrict__ status) {
  extern __shared__ u128 tiles[];
  __shared__ RowShared<TH> sh;
  __shared__ int s_a;
  __shared__ int s_err;
  const int b = blockIdx.x;
  const uint64_t st = step[b];
  const float* qrow0 = zq + (size_t)b * K * V;
  const float* prow0 = zp + (size_t)b * K * V;
  const float* mq = m_all + (size_t)b * K;
  const uint64_t* sq = s_all + (size_t)b * K;
  const float* mp = m_all + n_rows_each + (size_t)b * K;
  const uint64_t* sp = s_all + n_rows_each + (size_t)b * K;

  if (threadIdx.x == 0) {
    int err = 0;
    for (int j = 0; j < K; ++j) {
      const int d = drafts[b * K + j];
      if (d < 0 || d >= V) err |= UNO_DEV_BAD_TOKEN;
      if (sq[j] == 0 || sp[j] == 0) err |= UNO_DEV_NONFINITE;
    }
    int a = K;
    if (!err) {
      for (int i = 2; i <= K; ++i) {
        const int d = drafts[b * K + i - 1];
        const uint64_t wq = weight_of(qrow0[(size_t)(i - 1) * V + d], mq[i - 1], inv_temp);
        const uint64_t wp = weight_of(prow0[(size_t)(i - 2) * V + d], mp[i - 2], inv_temp);
        const uint32_t U = uniform24(seed, 1, i - 1, b, st);
        const u128 lhs = mul_64x64((uint64_t)U * wq, sp[i - 2]);
        const u128 r0 = mul_64x64(wp, sq[i - 1]);
        const u128 rhs = u128_make(r0.lo << 24, (r0.hi << 24) | (r0.lo >> 40));
        if (!u128_lt(lhs, rhs)) { a = i - 1; break; }
      }
      if (forced) {
        const int fa = forced[b];
        if (fa < 0 || fa > K) err |= UNO_DEV_BAD_ACCEPT;
        else a = fa;
      }
    }
    s_a = a;
    s_err = err;
    if (err) flag(status, b, err);
  }
  __syncthreads();
  const int a = s_a;
  if (s_err) {
    for (int j = threadIdx.x; j <= K; j += TH) committed[b * (K + 1) + j] = -1;
    if (threadIdx.x == 0) { accept_len[b] = 0; extra_token[b] = -1; }
    return;
  }
  const bool vec = (V & 3) == 0;
  int e;
  if (a < K) {
    // p_{a+1} is draft row 0 when a == 0, else verify row a-1; q_{a+1} is draft row a
    const bool p_from_q = a == 0;
    Row prow{p_from_q ? qrow0 : prow0 + (size_t)(a - 1) * V, V, vec};
    Row qrow{qrow0 + (size_t)a * V, V, vec};
    const float mpp = p_from_q ? mq[0] : mp[a - 1];
    const uint64_t spp = p_from_q ? sq[0] : sp[a - 1];
    ResidualWeights rw{prow, qrow, mpp, mq[a], inv_temp, spp, sq[a]};
    const u128 SR = block_weight_sum(rw, V, tiles, sh);
    const uint32_t U = uniform24(seed, 2, a, b, st);
    if (!u128_is_zero(SR)) {
      e = block_find(rw, V, tiles, scaled_target(U, SR), sh);
    } else {
      PlainWeights pw{prow, mpp, inv_temp};
      block_weight_sum(pw, V, tiles, sh);
      e = block_find(pw, V, tiles, scaled_target(U, u128_make(spp, 0)), sh);
    }
  } else {
    Row prow{prow0 + (size_t)(K - 1) * V, V, vec};
    PlainWeights pw{prow, mp[K - 1], inv_temp};
    block_weight_sum(pw, V, tiles, sh);
    const uint32_t U = uniform24(seed, 2, K, b, st);
    e = block_find(pw, V, tiles, scaled_target(U, u128_make(sp[K - 1], 0)), sh);
  }
  for (int j = threadIdx.x; j <= K; j += TH) {
    int v = -1;
    if (j < a) v = drafts[b * K + j];
    else if (j == a) v = e;
    committed[b * (K + 1) + j] = v;
  }
  if (threadIdx.x == 0) { accept_len[b] = a; extra_token[b] = e; }
}

// ------------------------------------------------------------ launchers
static size_t tile_lds_bytes(int V) { return (size_t)((V + kTile - 1) / kTile) * sizeof(u128); }

// Every row pass runs in 1024-thread workgroups: at most a few rows per CU are
// in flight, so a row's second pass finds it still in the last-level cache.
constexpr int kRowThreads = 1024;

hipError_t launch_draft_sample(const float* logits, int B, int K, int V, float inv_temp,
                               uint64_t seed, int slot, const uint64_t* step, int32_t* tokens,
                               int32_t* status, hipStream_t s) {
  hipLaunchKernelGGL(k_draft_sample<kRowThreads>, dim3(B * K), dim3(kRowThreads),
                     tile_lds_bytes(V), s, logits, K, V, inv_temp, seed, slot, step, tokens,
                     status, nullptr, 0, nullptr);
  return hipGetLastError();
}

hipError_t launch_tree_sample(const float* logits, int B, int N, int V, float inv_temp,
                              uint64_t seed, const uint64_t* step, const int32_t* node_depth,
                              const int32_t* n_nodes, int32_t* samples, int32_t* status,
                              hipStream_t s) {
  hipLaunchKernelGGL(k_draft_sample<kRowThreads>, dim3(B * N), dim3(kRowThreads),
                     tile_lds_bytes(V), s, logits, N, V, inv_temp, seed, 2, step, samples, status,
                     node_depth, 1, n_nodes);
  return hipGetLastError();
}

size_t spec_accept_ws_bytes(int B, int K) {
  const size_t rows = 2 * (size_t)B * K;
  return align_up(rows * sizeof(float), 256) + align_up(rows * sizeof(uint64_t), 256);
}

hipError_t launch_spec_accept(const float* zq, const float* zp, const int32_t* drafts, int B,
                              int K, int V, float inv_temp, uint64_t seed, const uint64_t* step,
                              const int32_t* forced, int32_t* accept_len, int32_t* committed,
                              int32_t* extra_token, int32_t* status, void* ws, hipStream_t s) {
  const int n_each = B * K;
  float* m_all = static_cast<float*>(ws);
  uint64_t* s_all = reinterpret_cast<uint64_t*>(static_cast<char*>(ws) +
                                                align_up(2 * (size_t)n_each * sizeof(float), 256));
  hipLaunchKernelGGL(k_row_stats<kRowThreads>, dim3(2 * n_each), dim3(kRowThreads), 0, s, zq, zp,
                     K, V, n_each, inv_temp, m_all, s_all, status);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_spec_accept<kRowThreads>, dim3(B), dim3(kRowThreads), tile_lds_bytes(V), s,
                     zq, zp, drafts, K, V, inv_temp, seed, step, forced, m_all, s_all, n_each,
                     accept_len, committed, extra_token, status);
  return hipGetLastError();
}

}  // namespace uno
