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
// starts at (b*K + j)*V.  Each row is handled by one 1024-thread workgroup;
// rows are streamed with 16-byte loads when V % 4 == 0.  When the row maxima
// are given (the LM head's epilogue produces them exactly), every row is
// streamed once: the weights are formed in the same pass that checks each
// entry (finite, not above the given maximum); otherwise a maximum pass
// precedes it.
#include "uno_device.h"
#include "uno_internal.h"

#include <mutex>

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

// The same for a plain row whose maximum m is given (the LM head's epilogue
// found it): one pass over the row, which also checks every entry -- a NaN or
// Inf entry, or one above m, sets *bad (the draw is then skipped).
template <int TH>
__device__ u128 block_weight_sum_given_max(const PlainWeights& wf, int V, u128* tiles,
                                           RowShared<TH>& sh, bool* bad_out) {
  const int w = threadIdx.x / UNO_WAVE, l = lane_id();
  const int n_tiles = (V + kTile - 1) / kTile;
  constexpr int NW = TH / UNO_WAVE;
  u128 acc = u128_make(0, 0);
  int bad = 0;
  for (int t = w; t < n_tiles; t += kUnroll * NW) {
    PlainWeights::Raw raw[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) wf.load((t + u * NW) * kTile + l * 4, raw[u]);
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      if (t + u * NW >= n_tiles) break;
#pragma unroll
      for (int c = 0; c < 4; ++c)
        if (raw[u].ok[c]) bad |= !__builtin_isfinite(raw[u].v[c]) || raw[u].v[c] > wf.m;
      u128 v[4];
      wf.weights(raw[u], v);
      u128 s = u128_add(u128_add(v[0], v[1]), u128_add(v[2], v[3]));
      s = wave_sum_u128(s);
      if (l == 0) tiles[t + u * NW] = s;
      acc = u128_add(acc, s);
    }
  }
  bad = __any(bad);
  if (l == 0) { sh.red_u[w] = acc; sh.red_i[w] = bad; }
  __syncthreads();
  u128 tot = sh.red_u[0];
  int rb = sh.red_i[0];
  for (int i = 1; i < (TH / UNO_WAVE); ++i) { tot = u128_add(tot, sh.red_u[i]); rb |= sh.red_i[i]; }
  __syncthreads();
  *bad_out = rb != 0 || !__builtin_isfinite(wf.m);
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
k_draft_sample(const float* __restrict__ logits, const float* __restrict__ row_max, int K, int V,
               float inv_temp, uint64_t seed,
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
  u128 S;
  PlainWeights wf{row, 0.f, inv_temp};
  if (row_max) {
    // one pass: the maximum is given
    wf.m = row_max[row_id];
    S = block_weight_sum_given_max(wf, V, tiles, sh, &bad);
  } else {
    wf.m = block_row_max(row, sh, &bad);
    if (!bad) S = block_weight_sum(wf, V, tiles, sh);
  }
  if (bad) {
    if (threadIdx.x == 0) { tokens[row_id] = -1; flag(status, b, UNO_DEV_NONFINITE); }
    return;
  }
  const uint32_t U = uniform24(seed, slot, j, b, step[b]);
  const int v = block_find(wf, V, tiles, scaled_target(U, S), sh);
  if (threadIdx.x == 0) tokens[row_id] = v;
}

// One workgroup per row of the concatenated [draft rows; verify rows]:
// row maximum and exact weight sum (fits 64 bits: V <= 2^20, W <= 2^31).
template <int TH>
__global__ void __launch_bounds__(TH)
k_row_stats(const float* __restrict__ zq, const float* __restrict__ zp,
            const float* __restrict__ mq_given, const float* __restrict__ mp_given, int K, int V,
            int n_rows_each, float inv_temp, float* __restrict__ m_out,
            uint64_t* __restrict__ s_out, int32_t* __restrict__ status) {
  __shared__ RowShared<TH> sh;
  const int r = blockIdx.x;
  const bool is_p = r >= n_rows_each;
  const int rr = is_p ? r - n_rows_each : r;
  Row row{(is_p ? zp : zq) + (size_t)rr * V, V, (V & 3) == 0};
  const float* given = is_p ? mp_given : mq_given;
  bool bad = false;
  // with the row maximum given, one pass that also checks every entry;
  // otherwise a maximum pass first
  const float m = given ? given[rr] : block_row_max(row, sh, &bad);
  int chk = given ? !__builtin_isfinite(m) : 0;
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
          if (ok[u][c]) {
            if (given) chk |= !__builtin_isfinite(v[u][c]) || v[u][c] > m;
            acc += weight_of(v[u][c], m, inv_temp);
          }
    }
  }
  acc = wave_sum_u64(acc);
  chk = __any(chk);
  const int w = threadIdx.x / UNO_WAVE;
  if (lane_id() == 0) { sh.red_u[w] = u128_make(acc, 0); sh.red_i[w] = chk; }
  __syncthreads();
  if (threadIdx.x == 0) {
    uint64_t tot = 0;
    for (int i = 0; i < (TH / UNO_WAVE); ++i) { tot += sh.red_u[i].lo; bad |= sh.red_i[i] != 0; }
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

// ------------------------------------------------------------ chunked rows
// With the row maxima given, every row is cut into chunks of kChunk entries
// that separate workgroups weigh in parallel (so that even one sequence's few
// rows fill the chip); a second kernel per row (or per sequence) adds the
// exact chunk sums, picks the chunk that holds the draw, and weighs that chunk
// once more to find the entry.  The sums are exact integers, so the draws are
// the same as with one workgroup per row.
constexpr int kChunk = 8192;
constexpr int kChunkThreads = 256;
constexpr int kMaxChunks = 128;               // V <= 2^20
constexpr uint64_t kBadChunk = ~0ull;         // the chunk holds a non-finite entry or one above
                                              // its row's given maximum
__host__ __device__ inline int n_chunks_of(int V) { return (V + kChunk - 1) / kChunk; }

// Plain weights of chunk blockIdx.x of row blockIdx.y (rows 0..n_q-1 are zq's,
// the rest zp's): sums[row * kMaxChunks + chunk] = their exact sum, or kBadChunk.
__global__ void __launch_bounds__(kChunkThreads)
k_chunk_sums(const float* __restrict__ zq, const float* __restrict__ zp, int n_q,
             const float* __restrict__ mq, const float* __restrict__ mp, int V, float inv_temp,
             uint64_t* __restrict__ sums) {
  __shared__ uint64_t red_s[kChunkThreads / UNO_WAVE];
  __shared__ int red_b[kChunkThreads / UNO_WAVE];
  const int row = blockIdx.y, c = blockIdx.x;
  const bool is_p = row >= n_q;
  const int rr = is_p ? row - n_q : row;
  const float m = (is_p ? mp : mq)[rr];
  const int c0 = c * kChunk;
  const int len = V - c0 < kChunk ? V - c0 : kChunk;
  const Row r{(is_p ? zp : zq) + (size_t)rr * V + c0, len, (V & 3) == 0};
  constexpr int U = kChunk / (kChunkThreads * 4);
  float v[U][4];
  bool ok[U][4];
#pragma unroll
  for (int u = 0; u < U; ++u) r.load4((u * kChunkThreads + threadIdx.x) * 4, v[u], ok[u]);
  uint64_t acc = 0;
  int bad = 0;
#pragma unroll
  for (int u = 0; u < U; ++u)
#pragma unroll
    for (int e = 0; e < 4; ++e)
      if (ok[u][e]) {
        bad |= !__builtin_isfinite(v[u][e]) || v[u][e] > m;
        acc += weight_of(v[u][e], m, inv_temp);
      }
  acc = wave_sum_u64(acc);
  bad = __any(bad);
  const int w = threadIdx.x / UNO_WAVE;
  if (lane_id() == 0) { red_s[w] = acc; red_b[w] = bad; }
  __syncthreads();
  if (threadIdx.x == 0) {
    uint64_t tot = 0;
    int b = !__builtin_isfinite(m);
    for (int i = 0; i < kChunkThreads / UNO_WAVE; ++i) { tot += red_s[i]; b |= red_b[i]; }
    sums[(size_t)row * kMaxChunks + c] = b ? kBadChunk : tot;
  }
}

// Residual weights max(0, Wp Sq - Wq Sp) of chunk blockIdx.x of sequence
// blockIdx.y's row pair (p_{a+1}, q_{a+1}) when its accept length a < K:
// rsums[b * kMaxChunks + chunk] (exact, 128-bit).
__global__ void __launch_bounds__(kChunkThreads)
k_resid_chunk_sums(const float* __restrict__ zq, const float* __restrict__ zp,
                   const float* __restrict__ m_all, const uint64_t* __restrict__ s_all,
                   const int32_t* __restrict__ a_ws, const int32_t* __restrict__ err_ws, int K,
                   int V, float inv_temp, int n_each, u128* __restrict__ rsums) {
  __shared__ u128 red[kChunkThreads / UNO_WAVE];
  const int b = blockIdx.y, c = blockIdx.x;
  const int a = a_ws[b];
  if (err_ws[b] || a >= K) return;
  const bool p_from_q = a == 0;      // p_1 is draft row 0
  const size_t prow = p_from_q ? (size_t)b * K : (size_t)b * K + a - 1;
  const size_t qrow = (size_t)b * K + a;
  const int ip = p_from_q ? (int)prow : n_each + (int)prow;
  const int c0 = c * kChunk;
  const int len = V - c0 < kChunk ? V - c0 : kChunk;
  const bool vec = (V & 3) == 0;
  const ResidualWeights rw{Row{(p_from_q ? zq : zp) + prow * V + c0, len, vec},
                           Row{zq + qrow * V + c0, len, vec}, m_all[ip], m_all[qrow], inv_temp,
                           s_all[ip], s_all[qrow]};
  constexpr int U = kChunk / (kChunkThreads * 4);
  u128 acc = u128_make(0, 0);
  ResidualWeights::Raw raw[U];
#pragma unroll
  for (int u = 0; u < U; ++u) rw.load((u * kChunkThreads + threadIdx.x) * 4, raw[u]);
#pragma unroll
  for (int u = 0; u < U; ++u) {
    u128 wv[4];
    rw.weights(raw[u], wv);
    acc = u128_add(acc, u128_add(u128_add(wv[0], wv[1]), u128_add(wv[2], wv[3])));
  }
  acc = wave_sum_u128(acc);
  const int w = threadIdx.x / UNO_WAVE;
  if (lane_id() == 0) red[w] = acc;
  __syncthreads();
  if (threadIdx.x == 0) {
    u128 tot = red[0];
    for (int i = 1; i < kChunkThreads / UNO_WAVE; ++i) tot = u128_add(tot, red[i]);
    rsums[(size_t)b * kMaxChunks + c] = tot;
  }
}

// The entry a draw with target t picks inside a row whose chunk sums are cs
// (nc chunks, total > t): the chunk whose running sum first exceeds t, then the
// entry inside it (weighed again with wf_of(chunk start, chunk length)).
template <class WF, class MakeWF>
__device__ int chunked_find(const u128* cs, int nc, int V, u128 t, const MakeWF& wf_of,
                            u128* tiles, RowShared<kChunkThreads>& sh) {
  __shared__ int s_chunk;
  __shared__ u128 s_before;
  if (threadIdx.x < UNO_WAVE) {
    // wave 0: running sums of the chunk sums, 64 chunks at a time; the first
    // chunk whose running sum exceeds t (the last chunk if none does)
    const int l = lane_id();
    u128 base = u128_make(0, 0);
    int chunk = -1;
    u128 before = base;
    for (int c0 = 0; c0 < nc && chunk < 0; c0 += UNO_WAVE) {
      const u128 v = c0 + l < nc ? cs[c0 + l] : u128_make(0, 0);
      const u128 incl = u128_add(wave_inclusive_scan_u128(v), base);
      const uint64_t hit = __ballot(u128_lt(t, incl) && c0 + l < nc);
      if (hit) {
        const int f = __ffsll((long long)hit) - 1;
        chunk = c0 + f;
        before = u128_sub(u128_shfl(incl, f), u128_shfl(v, f));
      } else {
        base = u128_shfl(incl, UNO_WAVE - 1);
      }
    }
    if (l == 0) {
      s_chunk = chunk < 0 ? nc - 1 : chunk;
      s_before = chunk < 0 ? u128_sub(base, cs[nc - 1]) : before;
    }
  }
  __syncthreads();
  const int c = s_chunk;
  const u128 tt = u128_sub(t, s_before);
  __syncthreads();
  const int c0 = c * kChunk;
  const int len = V - c0 < kChunk ? V - c0 : kChunk;
  const WF wf = wf_of(c0, len);
  block_weight_sum(wf, len, tiles, sh);
  return c0 + block_find(wf, len, tiles, tt, sh);
}

// One workgroup per draft row: the draw from the chunk sums (maximum given).
__global__ void __launch_bounds__(kChunkThreads)
k_draft_find(const float* __restrict__ logits, const float* __restrict__ row_max,
             const uint64_t* __restrict__ sums, int K, int V, float inv_temp, uint64_t seed,
             int slot, const uint64_t* __restrict__ step, int32_t* __restrict__ tokens,
             int32_t* __restrict__ status) {
  __shared__ RowShared<kChunkThreads> sh;
  __shared__ u128 tiles[kChunk / kTile];
  __shared__ u128 cs[kMaxChunks];
  __shared__ int s_bad;
  __shared__ u128 s_tot;
  const int row = blockIdx.x, b = row / K, j = row % K;
  const int nc = n_chunks_of(V);
  if (threadIdx.x == 0) s_bad = 0;
  __syncthreads();
  for (int c = threadIdx.x; c < nc; c += kChunkThreads) {
    const uint64_t x = sums[(size_t)row * kMaxChunks + c];
    cs[c] = u128_make(x == kBadChunk ? 0 : x, 0);
    if (x == kBadChunk) s_bad = 1;
  }
  __syncthreads();
  if (threadIdx.x < UNO_WAVE) {
    u128 tot = u128_make(0, 0);
    for (int c = lane_id(); c < nc; c += UNO_WAVE) tot = u128_add(tot, cs[c]);
    tot = wave_sum_u128(tot);
    if (threadIdx.x == 0) s_tot = tot;
  }
  __syncthreads();
  if (s_bad) {
    if (threadIdx.x == 0) { tokens[row] = -1; flag(status, b, UNO_DEV_NONFINITE); }
    return;
  }
  const float m = row_max[row];
  const float* z = logits + (size_t)row * V;
  const bool vec = (V & 3) == 0;
  const uint32_t U = uniform24(seed, slot, j, b, step[b]);
  const int v = chunked_find<PlainWeights>(
      cs, nc, V, scaled_target(U, s_tot),
      [&](int c0, int len) { return PlainWeights{Row{z + c0, len, vec}, m, inv_temp}; }, tiles, sh);
  if (threadIdx.x == 0) tokens[row] = v;
}

// One small workgroup per sequence: every row's exact weight sum from its
// chunk sums, the accept tests and the first rejection (as k_spec_accept),
// into m_all / s_all / a_ws / err_ws.
__global__ void __launch_bounds__(UNO_WAVE)
k_accept_decide(const float* __restrict__ zq, const float* __restrict__ zp,
                const float* __restrict__ mq, const float* __restrict__ mp,
                const uint64_t* __restrict__ sums, const int32_t* __restrict__ drafts, int K,
                int V, float inv_temp, uint64_t seed, const uint64_t* __restrict__ step,
                const int32_t* __restrict__ forced, int n_each, float* __restrict__ m_all,
                uint64_t* __restrict__ s_all, int32_t* __restrict__ a_ws,
                int32_t* __restrict__ err_ws, int32_t* __restrict__ status) {
  const int b = blockIdx.x;
  const int nc = n_chunks_of(V);
  int bad_rows = 0;
  // lane l sums rows l, l + 64, ... of the sequence's 2K rows
  for (int i = lane_id(); i < 2 * K; i += UNO_WAVE) {
    const bool is_p = i >= K;
    const int row = (is_p ? n_each : 0) + b * K + (is_p ? i - K : i);
    uint64_t S = 0;
    bool bad = false;
    for (int c = 0; c < nc; ++c) {
      const uint64_t x = sums[(size_t)row * kMaxChunks + c];
      bad |= x == kBadChunk;
      S += x;
    }
    m_all[row] = (is_p ? mp : mq)[b * K + (is_p ? i - K : i)];
    s_all[row] = bad ? 0ull : S;
    bad_rows |= bad;
  }
  bad_rows = __any(bad_rows);
  __syncthreads();             // m_all / s_all of the sequence are written
  const uint64_t st = step[b];
  const float* qrow0 = zq + (size_t)b * K * V;
  const float* prow0 = zp + (size_t)b * K * V;
  const float* mq_b = m_all + (size_t)b * K;
  const uint64_t* sq = s_all + (size_t)b * K;
  const float* mp_b = m_all + n_each + (size_t)b * K;
  const uint64_t* sp = s_all + n_each + (size_t)b * K;
  int bad_tok = 0;
  for (int j = lane_id(); j < K; j += UNO_WAVE) {
    const int d = drafts[b * K + j];
    bad_tok |= d < 0 || d >= V;
  }
  bad_tok = __any(bad_tok);
  const int err0 = (bad_rows ? UNO_DEV_NONFINITE : 0) | (bad_tok ? UNO_DEV_BAD_TOKEN : 0);
  // every accept test i = 2..K is independent of the others: lanes take them
  // in parallel, and a is the draft count before the first rejection
  int a = K;
  if (!err0) {
    for (int i0 = 2; i0 <= K; i0 += UNO_WAVE) {
      const int i = i0 + lane_id();
      bool rej = false;
      if (i <= K) {
        const int d = drafts[b * K + i - 1];
        const uint64_t wq = weight_of(qrow0[(size_t)(i - 1) * V + d], mq_b[i - 1], inv_temp);
        const uint64_t wp = weight_of(prow0[(size_t)(i - 2) * V + d], mp_b[i - 2], inv_temp);
        const uint32_t U = uniform24(seed, 1, i - 1, b, st);
        const u128 lhs = mul_64x64((uint64_t)U * wq, sp[i - 2]);
        const u128 r0 = mul_64x64(wp, sq[i - 1]);
        const u128 rhs = u128_make(r0.lo << 24, (r0.hi << 24) | (r0.lo >> 40));
        rej = !u128_lt(lhs, rhs);
      }
      const uint64_t hit = __ballot(rej);
      if (hit) { a = i0 + __ffsll((long long)hit) - 2; break; }
    }
  }
  if (threadIdx.x != 0) return;
  int err = err0;
  if (!err && forced) {
    const int fa = forced[b];
    if (fa < 0 || fa > K) err |= UNO_DEV_BAD_ACCEPT;
    else a = fa;
  }
  a_ws[b] = a;
  err_ws[b] = err;
  if (err) flag(status, b, err);
}

// One workgroup per sequence: the residual (or bonus) draw from the chunk
// sums, and the outputs.
__global__ void __launch_bounds__(kChunkThreads)
k_extra_find(const float* __restrict__ zq, const float* __restrict__ zp,
             const int32_t* __restrict__ drafts, int K, int V, float inv_temp, uint64_t seed,
             const uint64_t* __restrict__ step, const float* __restrict__ m_all,
             const uint64_t* __restrict__ s_all, const uint64_t* __restrict__ sums,
             const u128* __restrict__ rsums, const int32_t* __restrict__ a_ws,
             const int32_t* __restrict__ err_ws, int n_each, int32_t* __restrict__ accept_len,
             int32_t* __restrict__ committed, int32_t* __restrict__ extra_token) {
  __shared__ RowShared<kChunkThreads> sh;
  __shared__ u128 tiles[kChunk / kTile];
  __shared__ u128 cs[kMaxChunks];
  __shared__ u128 s_tot;
  const int b = blockIdx.x;
  const int a = a_ws[b];
  if (err_ws[b]) {
    for (int j = threadIdx.x; j <= K; j += kChunkThreads) committed[b * (K + 1) + j] = -1;
    if (threadIdx.x == 0) { accept_len[b] = 0; extra_token[b] = -1; }
    return;
  }
  const int nc = n_chunks_of(V);
  const bool vec = (V & 3) == 0;
  // p_{a+1}: draft row 0 when a == 0, else verify row a-1 (verify row K-1 for
  // the bonus draw a == K); q_{a+1}: draft row a
  const bool p_from_q = a == 0;
  const size_t prow = p_from_q ? (size_t)b * K : (size_t)b * K + a - 1;
  const int ip = p_from_q ? (int)prow : n_each + (int)prow;
  const float* pz = (p_from_q ? zq : zp) + prow * V;
  bool resid = false;
  if (a < K) {
    for (int c = threadIdx.x; c < nc; c += kChunkThreads) cs[c] = rsums[(size_t)b * kMaxChunks + c];
    __syncthreads();
    if (threadIdx.x < UNO_WAVE) {
      u128 tot = u128_make(0, 0);
      for (int c = lane_id(); c < nc; c += UNO_WAVE) tot = u128_add(tot, cs[c]);
      tot = wave_sum_u128(tot);
      if (threadIdx.x == 0) s_tot = tot;
    }
    __syncthreads();
    resid = !u128_is_zero(s_tot);
  }
  const uint32_t U = uniform24(seed, 2, a, b, step[b]);
  int e;
  if (resid) {
    const size_t qrow = (size_t)b * K + a;
    const float* qz = zq + qrow * V;
    const float mpp = m_all[ip], mqq = m_all[qrow];
    const uint64_t spp = s_all[ip], sqq = s_all[qrow];
    e = chunked_find<ResidualWeights>(
        cs, nc, V, scaled_target(U, s_tot),
        [&](int c0, int len) {
          return ResidualWeights{Row{pz + c0, len, vec}, Row{qz + c0, len, vec}, mpp, mqq,
                                 inv_temp, spp, sqq};
        },
        tiles, sh);
  } else {
    // the bonus draw, or a residual of zero mass: p_{a+1} itself
    __syncthreads();
    for (int c = threadIdx.x; c < nc; c += kChunkThreads)
      cs[c] = u128_make(sums[(size_t)ip * kMaxChunks + c], 0);
    __syncthreads();
    const float mpp = m_all[ip];
    e = chunked_find<PlainWeights>(
        cs, nc, V, scaled_target(U, u128_make(s_all[ip], 0)),
        [&](int c0, int len) { return PlainWeights{Row{pz + c0, len, vec}, mpp, inv_temp}; },
        tiles, sh);
  }
  for (int j = threadIdx.x; j <= K; j += kChunkThreads) {
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

size_t chunk_sums_bytes(int rows) { return (size_t)rows * kMaxChunks * sizeof(uint64_t); }

hipError_t launch_draft_sample_chunked(const float* logits, const float* row_max,
                                       uint64_t* sums, int B, int K, int V, float inv_temp,
                                       uint64_t seed, int slot, const uint64_t* step,
                                       int32_t* tokens, int32_t* status, hipStream_t s) {
  const int R = B * K;
  hipLaunchKernelGGL(k_chunk_sums, dim3(n_chunks_of(V), R), dim3(kChunkThreads), 0, s, logits,
                     logits, R, row_max, row_max, V, inv_temp, sums);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_draft_find, dim3(R), dim3(kChunkThreads), 0, s, logits, row_max, sums, K,
                     V, inv_temp, seed, slot, step, tokens, status);
  return hipGetLastError();
}

hipError_t launch_draft_sample(const float* logits, const float* row_max, int B, int K, int V,
                               float inv_temp, uint64_t seed, int slot, const uint64_t* step,
                               int32_t* tokens, int32_t* status, hipStream_t s) {
  hipLaunchKernelGGL(k_draft_sample<kRowThreads>, dim3(B * K), dim3(kRowThreads),
                     tile_lds_bytes(V), s, logits, row_max, K, V, inv_temp, seed, slot, step,
                     tokens, status, nullptr, 0, nullptr);
  return hipGetLastError();
}

hipError_t launch_tree_sample(const float* logits, int B, int N, int V, float inv_temp,
                              uint64_t seed, const uint64_t* step, const int32_t* node_depth,
                              const int32_t* n_nodes, int32_t* samples, int32_t* status,
                              hipStream_t s) {
  hipLaunchKernelGGL(k_draft_sample<kRowThreads>, dim3(B * N), dim3(kRowThreads),
                     tile_lds_bytes(V), s, logits, nullptr, N, V, inv_temp, seed, 2, step, samples,
                     status, node_depth, 1, n_nodes);
  return hipGetLastError();
}

// Workspace of the accept step: per-row maxima and weight sums (m_all,
// s_all) for both paths, then, for the chunked path (row maxima given), the
// per-sequence decisions, the plain chunk sums of every row and the residual
// chunk sums of every sequence.
struct AcceptWs {
  float* m_all;
  uint64_t* s_all;
  int32_t* a_ws;
  int32_t* err_ws;
  uint64_t* sums;
  u128* rsums;
  size_t total;
};
static AcceptWs carve_accept(int B, int K, void* base) {
  AcceptWs w;
  const size_t rows = 2 * (size_t)B * K;
  size_t off = 0;
  char* p = static_cast<char*>(base);
  auto take = [&](size_t bytes) {
    char* q = p ? p + off : nullptr;
    off += align_up(bytes, 256);
    return q;
  };
  w.m_all = reinterpret_cast<float*>(take(rows * sizeof(float)));
  w.s_all = reinterpret_cast<uint64_t*>(take(rows * sizeof(uint64_t)));
  w.a_ws = reinterpret_cast<int32_t*>(take((size_t)B * sizeof(int32_t)));
  w.err_ws = reinterpret_cast<int32_t*>(take((size_t)B * sizeof(int32_t)));
  w.sums = reinterpret_cast<uint64_t*>(take(rows * kMaxChunks * sizeof(uint64_t)));
  w.rsums = reinterpret_cast<u128*>(take((size_t)B * kMaxChunks * sizeof(u128)));
  w.total = off;
  return w;
}

size_t spec_accept_ws_bytes(int B, int K) { return carve_accept(B, K, nullptr).total; }

hipError_t launch_spec_accept(const float* zq, const float* zp, const float* mq, const float* mp,
                              const int32_t* drafts, int B, int K, int V, float inv_temp,
                              uint64_t seed, const uint64_t* step, const int32_t* forced,
                              int32_t* accept_len, int32_t* committed, int32_t* extra_token,
                              int32_t* status, void* ws, hipStream_t s, bool ws_is_full) {
  const int n_each = B * K;
  float* m_all;
  uint64_t* s_all;
  if (mq && mp && ws_is_full) {
    // chunked rows: plain chunk sums of every row, decisions, residual chunk
    // sums, the extra token
    const AcceptWs w = carve_accept(B, K, ws);
    const int nc = n_chunks_of(V);
    hipLaunchKernelGGL(k_chunk_sums, dim3(nc, 2 * n_each), dim3(kChunkThreads), 0, s, zq, zp,
                       n_each, mq, mp, V, inv_temp, w.sums);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(k_accept_decide, dim3(B), dim3(UNO_WAVE), 0, s, zq, zp, mq, mp, w.sums,
                       drafts, K, V, inv_temp, seed, step, forced, n_each, w.m_all, w.s_all,
                       w.a_ws, w.err_ws, status);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    hipLaunchKernelGGL(k_resid_chunk_sums, dim3(nc, B), dim3(kChunkThreads), 0, s, zq, zp,
                       w.m_all, w.s_all, w.a_ws, w.err_ws, K, V, inv_temp, n_each, w.rsums);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    hipLaunchKernelGGL(k_extra_find, dim3(B), dim3(kChunkThreads), 0, s, zq, zp, drafts, K, V,
                       inv_temp, seed, step, w.m_all, w.s_all, w.sums, w.rsums, w.a_ws, w.err_ws,
                       n_each, accept_len, committed, extra_token);
    return hipGetLastError();
  }
  m_all = static_cast<float*>(ws);
  s_all = reinterpret_cast<uint64_t*>(static_cast<char*>(ws) +
                                      align_up(2 * (size_t)n_each * sizeof(float), 256));
  hipLaunchKernelGGL(k_row_stats<kRowThreads>, dim3(2 * n_each), dim3(kRowThreads), 0, s, zq, zp,
                     mq, mp, K, V, n_each, inv_temp, m_all, s_all, status);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_spec_accept<kRowThreads>, dim3(B), dim3(kRowThreads), tile_lds_bytes(V), s,
                     zq, zp, drafts, K, V, inv_temp, seed, step, forced, m_all, s_all, n_each,
                     accept_len, committed, extra_token, status);
  return hipGetLastError();
}

// ------------------------------------------------------------ no-allocation variant
// The per-row statistics of uno_spec_accept_noalloc live in a file-scope
// device array instead of a caller-supplied workspace: 2*B*K row maxima
// (fp32) and weight sums (uint64) for at most kStaticAcceptRows rows.  Every
// GPU the library runs on holds its own copy until the process ends; the host
// learns each copy's address once per device (hipGetSymbolAddress, with that
// device current) and passes that address to the kernels.  Nothing in it has to
// start at zero: k_row_stats writes every entry k_spec_accept reads.
constexpr int kStaticAcceptRows = 65536;
static __device__ __align__(256) unsigned char scratch[(size_t)kStaticAcceptRows * 12];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};
}  // namespace

int static_accept_max_rows() { return kStaticAcceptRows; }

hipError_t static_accept_scratch(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}

hipError_t launch_spec_accept_static(const float* zq, const float* zp, const float* mq,
                                     const float* mp, const int32_t* drafts, int B, int K, int V,
                                     float inv_temp, uint64_t seed, const uint64_t* step,
                                     const int32_t* forced, int32_t* accept_len,
                                     int32_t* committed, int32_t* extra_token, int32_t* status,
                                     hipStream_t s) {
  void* ws = nullptr;
  const hipError_t e = static_accept_scratch(&ws);
  if (e != hipSuccess) return e;
  // the static scratch holds the per-row statistics only: one workgroup per row
  return launch_spec_accept(zq, zp, mq, mp, drafts, B, K, V, inv_temp, seed, step, forced,
                            accept_len, committed, extra_token, status, ws, s, false);
}

}  // namespace uno
