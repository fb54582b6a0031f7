// Tree sampler of the Psi-Spec step for gfx950: top-k of every drafted
// position, the best n_keep of the candidate sequences they span, their prefix
// tree, the accept walk over the tree's verify rows and the commit that moves
// the kept path's K/V into place ("Unlocking Lossless Speedups in LLMs via
// Discrete Diffusion": picx.dev summary, "Psi-Speculative Sampler", tree
// sampler; paperglide reader, "The Psi-Speculative Sampler", worked example and
// step list).
//
// Definitions (the pages leave the arithmetic and the accept rule open):
//   * top-k of a row: the k largest fp32 logits, equal values by smaller id;
//   * score of a candidate: sum over its positions of
//     rint(fp32(z[token] - z[top-1]) * 2^20) (floored at -2^40), exact int64;
//     the joint log-probability differs from it (up to that rounding and the
//     temperature's positive factor) by a constant; equal scores are ordered
//     by the top-k rank tuples, lexicographically;
//   * tree: node 0 = d_1 (the draft sampler's token of row 0); the kept
//     candidates, best first, each add their new prefixes, by depth; rows past
//     the tree (up to N = 1 + n_keep*(K-1)) repeat d_1 at depth 0 and see only
//     themselves;
//   * walk: at node u draw x ~ p_u (the verify row of u; canonical integer
//     sampler, Philox slot 2, j = depth(u) + 1); move to the child carrying x,
//     else stop.  Every emitted token is an exact draw from the AR model, so
//     the output law is the AR law;
//   * commit: node path[d] (depth d) moves from slot kv_len+1+path[d] to
//     kv_len+1+d, then kv_len += 1 + a.
//
// The best n_keep of topk^(K-1) candidates come from a beam over the positions:
// with exact integer scores, the best n_keep prefixes of length L+1 all extend
// one of the best n_keep prefixes of length L (an extension never overtakes
// the same extension of a better prefix), so keeping n_keep per position and
// ranking the n_keep*topk extensions gives the global best n_keep.
#include "uno_device.h"
#include "uno_internal.h"

namespace uno {

constexpr int kTreeMaxTopk = 8;
constexpr int kTreeMaxKeep = 64;
constexpr int kTreeMaxK = 32;

// ------------------------------------------------------------ top-k rows
// One workgroup per drafted row (b, j), j = 1..K-1: the T largest logits and
// their integer score deltas -> tok/delta [B][K-1][T].
template <int T>
__global__ void __launch_bounds__(256)
k_tree_topk(const float* __restrict__ zq, int K, int V, int32_t* __restrict__ tok,
            long long* __restrict__ delta, int32_t* __restrict__ status) {
  __shared__ float s_val[4];
  __shared__ int s_idx[4];
  __shared__ int s_bad[4];
  __shared__ float s_top[T];
  __shared__ int s_topi[T];
  const int r = blockIdx.x;                 // b * (K-1) + (j-1)
  const int b = r / (K - 1), j = 1 + r % (K - 1);
  const float* row = zq + ((size_t)b * K + j) * V;
  float val[T];
  int idx[T];
#pragma unroll
  for (int q = 0; q < T; ++q) { val[q] = -INFINITY; idx[q] = 0x7fffffff; }
  int bad = 0;
  // sorted insertion; equal values keep the smaller id (each thread sees its
  // ids in increasing order)
  auto insert = [&](float v, int i) {
    if (!(v > val[T - 1])) return;
#pragma unroll
    for (int q = T - 1; q >= 1; --q) {
      if (v > val[q - 1]) { val[q] = val[q - 1]; idx[q] = idx[q - 1]; }
      else if (v > val[q]) { val[q] = v; idx[q] = i; }
    }
    if (v > val[0]) { val[0] = v; idx[0] = i; }
  };
  const bool vec = (V & 3) == 0;
  for (int e0 = threadIdx.x * 4; e0 < V; e0 += 1024) {
    float v[4];
    if (vec) {
      const float4 f = *reinterpret_cast<const float4*>(row + e0);
      v[0] = f.x; v[1] = f.y; v[2] = f.z; v[3] = f.w;
    } else {
#pragma unroll
      for (int c = 0; c < 4; ++c) v[c] = e0 + c < V ? row[e0 + c] : -INFINITY;
    }
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      if (e0 + c >= V) continue;
      bad |= !__builtin_isfinite(v[c]);
      insert(v[c], e0 + c);
    }
  }
  const int w = threadIdx.x / UNO_WAVE;
  bad = __any(bad);
  if (lane_id() == 0) s_bad[w] = bad;
  // T rounds of a block-wide best (larger value, then smaller id); the
  // winning thread pops its list head
  for (int t = 0; t < T; ++t) {
    float bv = val[0];
    int bi = idx[0];
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
      const float ov = __shfl_xor(bv, off, 64);
      const int oi = __shfl_xor(bi, off, 64);
      if (ov > bv || (ov == bv && oi < bi)) { bv = ov; bi = oi; }
    }
    if (lane_id() == 0) { s_val[w] = bv; s_idx[w] = bi; }
    __syncthreads();
    float gv = s_val[0];
    int gi = s_idx[0];
    for (int q = 1; q < 4; ++q)
      if (s_val[q] > gv || (s_val[q] == gv && s_idx[q] < gi)) { gv = s_val[q]; gi = s_idx[q]; }
    if (threadIdx.x == 0) { s_top[t] = gv; s_topi[t] = gi; }
    if (idx[0] == gi) {
#pragma unroll
      for (int q = 0; q < T - 1; ++q) { val[q] = val[q + 1]; idx[q] = idx[q + 1]; }
      val[T - 1] = -INFINITY;
      idx[T - 1] = 0x7fffffff;
    }
    __syncthreads();
  }
  if (threadIdx.x < T) {
    const int t = threadIdx.x;
    const bool any_bad = s_bad[0] | s_bad[1] | s_bad[2] | s_bad[3];
    long long d = 0;
    if (!any_bad) {
      const float df = s_top[t] - s_top[0];
      d = df < -1048576.0f ? -(1ll << 40) : (long long)__builtin_rintf(df * 1048576.0f);
    }
    tok[(size_t)r * T + t] = any_bad ? -1 : s_topi[t];
    delta[(size_t)r * T + t] = d;
    if (any_bad && t == 0 && status) atomicOr(status + b, UNO_DEV_NONFINITE);
  }
}

// ------------------------------------------------------------ tree build
// One workgroup per sequence: beam over the K-1 drafted positions, then the
// prefix tree of the kept candidates.  Outputs (rows n < N of sequence b):
// tokens, parent (-1 at the root and the padding rows), depth, ancestor-or-self
// bit rows anc[n][W] (bit i of word i/32), and n_nodes[b].
__global__ void __launch_bounds__(256)
k_tree_build(const int32_t* __restrict__ draft_tokens, const int32_t* __restrict__ tok,
             const long long* __restrict__ delta, int K, int T, int n_keep, int N, int W,
             int32_t* __restrict__ node_tokens, int32_t* __restrict__ node_parent,
             int32_t* __restrict__ node_depth, uint32_t* __restrict__ node_anc,
             int32_t* __restrict__ n_nodes_out) {
  __shared__ long long s_delta[kTreeMaxK][kTreeMaxTopk];
  __shared__ long long s_score[2][kTreeMaxKeep];
  __shared__ int s_lex[2][kTreeMaxKeep];
  __shared__ unsigned char s_rank[2][kTreeMaxKeep][kTreeMaxK];
  __shared__ int s_np[kTreeMaxKeep], s_nr[kTreeMaxKeep];
  __shared__ long long s_ns[kTreeMaxKeep];
  __shared__ int s_first[kTreeMaxKeep], s_from[kTreeMaxKeep], s_base[kTreeMaxKeep + 1];
  __shared__ int s_node[kTreeMaxKeep][kTreeMaxK];
  const int b = blockIdx.x, tid = threadIdx.x;
  const int P = K - 1;                              // drafted positions
  for (int e = tid; e < P * T; e += 256) s_delta[e / T][e % T] = delta[(size_t)b * P * T + e];
  if (tid == 0) { s_score[0][0] = 0; s_lex[0][0] = 0; }
  __syncthreads();
  int cur = 0, size = 1;
  for (int pos = 0; pos < P; ++pos) {
    const int C = size * T;
    for (int c = tid; c < C; c += 256) {
      const int p = c / T, rr = c % T;
      const long long sc = s_score[cur][p] + s_delta[pos][rr];
      const int lx = s_lex[cur][p];
      int before = 0;
      for (int c2 = 0; c2 < C; ++c2) {
        const int p2 = c2 / T, r2 = c2 % T;
        const long long sc2 = s_score[cur][p2] + s_delta[pos][r2];
        const int lx2 = s_lex[cur][p2];
        before += sc2 > sc || (sc2 == sc && (lx2 < lx || (lx2 == lx && r2 < rr)));
      }
      if (before < n_keep) { s_np[before] = p; s_nr[before] = rr; s_ns[before] = sc; }
    }
    __syncthreads();
    const int nsize = C < n_keep ? C : n_keep;
    const int nxt = cur ^ 1;
    for (int e = tid; e < nsize; e += 256) {
      const int lx = s_lex[cur][s_np[e]], rr = s_nr[e];
      int before = 0;
      for (int e2 = 0; e2 < nsize; ++e2) {
        const int lx2 = s_lex[cur][s_np[e2]], r2 = s_nr[e2];
        before += lx2 < lx || (lx2 == lx && r2 < rr);
      }
      s_lex[nxt][e] = before;
      s_score[nxt][e] = s_ns[e];
      for (int q = 0; q < pos; ++q) s_rank[nxt][e][q] = s_rank[cur][s_np[e]][q];
      s_rank[nxt][e][pos] = (unsigned char)rr;
    }
    __syncthreads();
    cur = nxt;
    size = nsize;
  }
  // prefix tree: candidate c shares depths 1..l with an earlier candidate
  // (l = longest common rank prefix); its nodes at depths l+1..K-1 are new
  const int V = size;
  for (int c = tid; c < V; c += 256) {
    int best = 0, from = -1;
    for (int c2 = 0; c2 < c; ++c2) {
      int l = 0;
      while (l < P && s_rank[cur][c][l] == s_rank[cur][c2][l]) ++l;
      if (l > best) { best = l; from = c2; }
    }
    s_first[c] = best + 1;
    s_from[c] = from;
  }
  __syncthreads();
  if (tid == 0) {
    s_base[0] = 1;
    for (int c = 0; c < V; ++c) s_base[c + 1] = s_base[c] + (K - s_first[c]);
  }
  __syncthreads();
  for (int c = 0; c < V; ++c) {
    for (int d = tid; d < K; d += 256)
      s_node[c][d] = d == 0 ? 0 : d >= s_first[c] ? s_base[c] + d - s_first[c] : s_node[s_from[c]][d];
    __syncthreads();
  }
  const int n_nodes = s_base[V];
  const int d1 = draft_tokens[(size_t)b * K];
  int32_t* ot = node_tokens + (size_t)b * N;
  int32_t* op = node_parent + (size_t)b * N;
  int32_t* od = node_depth + (size_t)b * N;
  uint32_t* oa = node_anc + (size_t)b * N * W;
  // root and padding rows: d_1 at depth 0, ancestor set = itself
  for (int n = tid; n < N; n += 256) {
    if (n > 0 && n < n_nodes) continue;
    ot[n] = d1;
    op[n] = -1;
    od[n] = 0;
    for (int q = 0; q < W; ++q) oa[(size_t)n * W + q] = (n >> 5) == q ? 1u << (n & 31) : 0u;
  }
  // new nodes: one thread per (candidate, depth >= first new depth)
  for (int e = tid; e < V * P; e += 256) {
    const int c = e / P, d = 1 + e % P;
    if (d < s_first[c]) continue;
    const int n = s_node[c][d];
    const int rk = s_rank[cur][c][d - 1];
    ot[n] = tok[((size_t)b * P + (d - 1)) * T + rk];
    op[n] = s_node[c][d - 1];
    od[n] = d;
    uint32_t* row = oa + (size_t)n * W;
    for (int q = 0; q < W; ++q) {
      uint32_t acc = 0;
      for (int d2 = 0; d2 <= d; ++d2) {
        const int m = s_node[c][d2];
        if ((m >> 5) == q) acc |= 1u << (m & 31);
      }
      row[q] = acc;
    }
  }
  if (tid == 0) n_nodes_out[b] = n_nodes;
}

// ------------------------------------------------------------ walk
// One wave per sequence: follow the per-node draws (samples[b][n], drawn from
// the verify row of n) down the tree.
__global__ void __launch_bounds__(64)
k_tree_walk(const int32_t* __restrict__ node_tokens, const int32_t* __restrict__ node_parent,
            const int32_t* __restrict__ n_nodes, const int32_t* __restrict__ samples, int K, int N,
            int32_t* __restrict__ accept_len, int32_t* __restrict__ committed,
            int32_t* __restrict__ extra_token, int32_t* __restrict__ path,
            int32_t* __restrict__ status) {
  const int b = blockIdx.x, l = threadIdx.x;
  const int32_t* tk = node_tokens + (size_t)b * N;
  const int32_t* pa = node_parent + (size_t)b * N;
  const int32_t* sm = samples + (size_t)b * N;
  const int nn = n_nodes[b];
  int u = 0, d = 0, x = -1, err = 0;
  int my_path = l == 0 ? 0 : -1;            // lane d holds the node at depth d
  if (nn < 1 || nn > N) err = UNO_DEV_BAD_TOKEN;
  while (!err) {
    x = sm[u];
    if (x < 0) { err = UNO_DEV_NONFINITE; break; }
    int found = -1;
    for (int base = u + 1; base < nn && found < 0; base += 64) {
      const int n = base + l;
      const bool hit = n < nn && pa[n] == u && tk[n] == x;
      const uint64_t m = __ballot(hit);
      if (m) found = base + __ffsll((long long)m) - 1;
    }
    if (found < 0 || d + 1 >= K) break;
    u = found;
    ++d;
    if (l == d) my_path = u;
  }
  if (err) {
    if (l == 0 && status) atomicOr(status + b, err);
    for (int j = l; j <= K; j += 64) committed[(size_t)b * (K + 1) + j] = -1;
    for (int j = l; j < K; j += 64) path[(size_t)b * K + j] = -1;
    if (l == 0) { accept_len[b] = 0; extra_token[b] = -1; }
    return;
  }
  // K <= 32: lane l writes entry l (lane d holds the node at depth d)
  const int a = d + 1;
  if (l <= K) committed[(size_t)b * (K + 1) + l] = l < a ? tk[my_path] : l == a ? x : -1;
  if (l < K) path[(size_t)b * K + l] = l < a ? my_path : -1;
  if (l == 0) { accept_len[b] = a; extra_token[b] = x; }
}

// ------------------------------------------------------------ commit
// grid (B, layers, Hkv), hd threads: thread t moves channel t of the walked
// nodes' K and V, depth by depth (a node at depth d sits at slot offset >= d,
// so a move never overwrites a source still to be read).
__global__ void k_tree_commit(const int32_t* __restrict__ path, const int32_t* __restrict__ accept_len,
                              const int32_t* __restrict__ kv_len, const int32_t* __restrict__ page_table,
                              int max_pages, int64_t n_pages, int Hkv, int hd, int ps_shift,
                              size_t layer_elems, int K, uint16_t* __restrict__ k_pages,
                              uint16_t* __restrict__ v_pages, int32_t* __restrict__ status) {
  const int b = blockIdx.x, layer = blockIdx.y, g = blockIdx.z, t = threadIdx.x;
  const int a = accept_len[b];
  if (a < 1 || a > K) return;              // rejected by the kv_len update
  const int kvl = kv_len[b];
  const int ps = 1 << ps_shift, pmask = ps - 1;
  uint16_t* kl = k_pages + (size_t)layer * layer_elems;
  uint16_t* vl = v_pages + (size_t)layer * layer_elems;
  const int32_t* pt = page_table + (size_t)b * max_pages;
  for (int d = 1; d < a; ++d) {
    const int node = path[(size_t)b * K + d];
    const int src = kvl + 1 + node, dst = kvl + 1 + d;
    if (node < d || src == dst) continue;
    const int ps_i = src >> ps_shift, pd_i = dst >> ps_shift;
    const int psrc = ps_i < max_pages ? pt[ps_i] : -1;
    const int pdst = pd_i < max_pages ? pt[pd_i] : -1;
    if (psrc < 0 || psrc >= n_pages || pdst < 0 || pdst >= n_pages) {
      if (t == 0 && layer == 0 && g == 0 && status) atomicOr(status + b, UNO_DEV_BAD_PAGE);
      continue;
    }
    const int ss = src & pmask, sd = dst & pmask;
    kl[(((size_t)pdst * Hkv + g) * ps + sd) * hd + t] = kl[(((size_t)psrc * Hkv + g) * ps + ss) * hd + t];
    vl[(((size_t)pdst * Hkv + g) * hd + t) * ps + sd] = vl[(((size_t)psrc * Hkv + g) * hd + t) * ps + ss];
  }
}

// ------------------------------------------------------------ launchers
size_t tree_ws_bytes(int B, int K, int topk) {
  const size_t n = (size_t)B * (K - 1) * topk;
  return align_up(n * sizeof(int32_t), 256) + align_up(n * sizeof(long long), 256);
}

hipError_t launch_tree_build(const float* zq, const int32_t* draft_tokens, int B, int K, int V,
                             int topk, int n_keep, int N, int32_t* node_tokens,
                             int32_t* node_parent, int32_t* node_depth, uint32_t* node_anc,
                             int32_t* n_nodes, int32_t* status, void* ws, hipStream_t s) {
  const size_t n = (size_t)B * (K - 1) * topk;
  int32_t* tok = static_cast<int32_t*>(ws);
  long long* delta = reinterpret_cast<long long*>(static_cast<char*>(ws) +
                                                  align_up(n * sizeof(int32_t), 256));
  const dim3 grid(B * (K - 1));
  switch (topk) {
#define UNO_TOPK_CASE(T) \
    case T: hipLaunchKernelGGL(k_tree_topk<T>, grid, dim3(256), 0, s, zq, K, V, tok, delta, status); break;
    UNO_TOPK_CASE(1) UNO_TOPK_CASE(2) UNO_TOPK_CASE(3) UNO_TOPK_CASE(4)
    UNO_TOPK_CASE(5) UNO_TOPK_CASE(6) UNO_TOPK_CASE(7) UNO_TOPK_CASE(8)
#undef UNO_TOPK_CASE
    default: return hipErrorInvalidValue;
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int W = (N + 31) / 32;
  hipLaunchKernelGGL(k_tree_build, dim3(B), dim3(256), 0, s, draft_tokens, tok, delta, K, topk,
                     n_keep, N, W, node_tokens, node_parent, node_depth, node_anc, n_nodes);
  return hipGetLastError();
}

hipError_t launch_tree_walk(const int32_t* node_tokens, const int32_t* node_parent,
                            const int32_t* n_nodes, const int32_t* samples, int B, int K, int N,
                            int32_t* accept_len, int32_t* committed, int32_t* extra_token,
                            int32_t* path, int32_t* status, hipStream_t s) {
  hipLaunchKernelGGL(k_tree_walk, dim3(B), dim3(64), 0, s, node_tokens, node_parent, n_nodes,
                     samples, K, N, accept_len, committed, extra_token, path, status);
  return hipGetLastError();
}

hipError_t launch_tree_commit(const uno_config& c, const uno_kv& kv, const int32_t* path,
                              const int32_t* accept_len, int B, int K, int32_t* status,
                              hipStream_t s) {
  const size_t layer_elems = (size_t)kv.n_pages * c.n_kv_heads * c.page_size * c.head_dim;
  const int ps_shift = __builtin_ctz((unsigned)c.page_size);
  hipLaunchKernelGGL(k_tree_commit, dim3(B, c.n_layers, c.n_kv_heads), dim3(c.head_dim), 0, s,
                     path, accept_len, kv.kv_len, kv.page_table, kv.max_pages_per_seq, kv.n_pages,
                     c.n_kv_heads, c.head_dim, ps_shift, layer_elems, K,
                     static_cast<uint16_t*>(kv.k_pages), static_cast<uint16_t*>(kv.v_pages),
                     status);
  return hipGetLastError();
}

}  // namespace uno
