// bf16 MFMA GEMMs of the draft / verify passes for gfx950, with the LoRA
// low-rank path fused as extra K-iterations:
//   Y = X W^T + T B^T,  T = scale * gate(row) * (X A^T)
// ("Unlocking Lossless Speedups in LLMs via Discrete Diffusion": the diffusion
// weights are rank-r LoRA factors with scale alpha/r on every linear, active for
// the noisy positions of a drafted block and off for its first position and for
// verification; picx.dev summary, "Architecture"; paperglide reader, "Sampler
// Extensions").
//
// Weights (W of every product: the projections, the LoRA A factors, the LM
// head) are stored tile-packed: the 16-row x 32-column fragment of 16-row tile
// nt and K step s is 1 KB at element ((nt * K/32) + s) * 512, laid out in the
// lane order of the MFMA operand (lane l = 16 * chunk + row holds the 8 values
// of that row and 8-column chunk), so a wave reads each fragment as one
// contiguous 1 KB.  LoRA B factors stay row-major.
//
// Skinny kernel (decode rows, M <= 64 per workgroup): one workgroup owns
// 16..64 columns of W and 16..64 rows of X; its 2 or 4 waves split the K
// dimension (with one row tile, wave w takes blocks of four or eight
// consecutive 32-wide K steps, so each wave reads its fragments in 4-8 KB
// runs), and every weight byte is read from HBM once, with non-temporal loads.
// Each wave issues v_mfma_f32_16x16x32_bf16 (A = 16 rows of X, B = 16 columns
// of W^T); the waves' partial tiles are summed in LDS in a fixed order and the
// epilogue stores, accumulates into the fp32 residual stream, or forms the
// gated, scaled LoRA input T.  q|k|v and [gate | up] products pair the two
// 16-column tiles that RoPE (channels i and i + hd/2) or SwiGLU (gate and up
// column c) combine in one workgroup over the whole K and apply that in the
// epilogue.  The residual products (o, down) split K over workgroups: the
// splits store fp32 partial rows and a second kernel sums them in split order
// (run-to-run identical) and applies the residual add and RMSNorm.
#include "uno_device.h"
#include "uno_internal.h"
#include "rope_store.h"

#include <algorithm>

namespace uno {

union Frag {
  uint4 u;
  bf16x8 v;
};

__device__ __forceinline__ uint4 ldg16(const uint16_t* p) {
  return *reinterpret_cast<const uint4*>(p);
}
typedef __attribute__((ext_vector_type(4))) unsigned int u32x4_w;
// 16-byte load marked non-temporal (weights: each byte is read once per pass)
__device__ __forceinline__ uint4 ldg16_nt(const uint16_t* p) {
  const u32x4_w v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_w*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}

struct SegView {
  const uint16_t* w;
  const uint16_t* lb;
  int t_col;
  int col_base;
  int n0;
  int n;        // columns of the segment
};

__device__ __forceinline__ SegView pick_segment(const GemmArgs& a, int tile) {
  SegView v;
  int base = 0;
  int t0 = a.seg[0].n >> 4, t1 = a.seg[1].n >> 4;
  if (a.n_seg == 1 || tile < t0) {
    v.w = a.seg[0].w; v.lb = a.seg[0].lora_b; v.t_col = a.seg[0].t_col; v.n0 = tile * 16;
    v.n = a.seg[0].n;
  } else if (a.n_seg == 2 || tile < t0 + t1) {
    base = a.seg[0].n;
    v.w = a.seg[1].w; v.lb = a.seg[1].lora_b; v.t_col = a.seg[1].t_col; v.n0 = (tile - t0) * 16;
    v.n = a.seg[1].n;
  } else {
    base = a.seg[0].n + a.seg[1].n;
    v.w = a.seg[2].w; v.lb = a.seg[2].lora_b; v.t_col = a.seg[2].t_col;
    v.n0 = (tile - t0 - t1) * 16;
    v.n = a.seg[2].n;
  }
  v.col_base = base;
  return v;
}

__device__ __forceinline__ void store_out(const GemmArgs& a, int m, int n, float v) {
  const size_t o = (size_t)m * a.ldo + n;
  switch (a.epi) {
    case EPI_STORE_F32: static_cast<float*>(a.out)[o] = v; break;
    case EPI_ADD_F32: static_cast<float*>(a.out)[o] += v; break;
    case EPI_STORE_BF16: static_cast<uint16_t*>(a.out)[o] = f32_to_bf16(v); break;
    default: {
      const float g = (m % a.rows_per_seq) != 0 ? a.scale : 0.f;
      static_cast<uint16_t*>(a.out)[o] = f32_to_bf16(g * v);
    }
  }
}

// Split-K sums p[0] + p[zs] + ... + p[(splits - 1) zs], added in split order
// (run-to-run identical); the loads go out a chunk at a time so that their
// latencies overlap instead of adding up.
__device__ __forceinline__ float sum_splits(const float* p, size_t zs, int splits) {
  float v = p[0];
  for (int z0 = 1; z0 < splits; z0 += 8) {
    float q[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) q[u] = z0 + u < splits ? p[(size_t)(z0 + u) * zs] : 0.f;
#pragma unroll
    for (int u = 0; u < 8; ++u)
      if (z0 + u < splits) v += q[u];
  }
  return v;
}
__device__ __forceinline__ float4 sum_splits4(const float4* p, size_t zs, int splits) {
  float4 v = p[0];
  for (int z0 = 1; z0 < splits; z0 += 4) {
    float4 q[4];
#pragma unroll
    for (int u = 0; u < 4; ++u)
      q[u] = z0 + u < splits ? p[(size_t)(z0 + u) * zs] : make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
    for (int u = 0; u < 4; ++u)
      if (z0 + u < splits) {
        v.x += q[u].x; v.y += q[u].y; v.z += q[u].z; v.w += q[u].w;
      }
  }
  return v;
}
// output columns of all segments together
__host__ __device__ __forceinline__ int skinny_cols(const GemmArgs& a) {
  int n = 0;
  for (int i = 0; i < a.n_seg; ++i) n += a.seg[i].n;
  return n;
}

// Waves per workgroup: a workgroup streams its columns' W over K, split among
// its waves.  Fewer waves per workgroup, each with more K steps, stream faster
// on this chip: at 16 rows the [gate | up] product (201 MB of W) took 56 us
// with 8 waves per workgroup, 41 us with 4 and 39 us with 2.
constexpr int kSkWaves = 4;         // paired and LoRA-A products
constexpr int kSkWavesSplit = 2;    // split-K products and the LM head

// Producer / consumer handshake of a fused LoRA-A product (k_gemm_skinny_lora).
// The producers store their partials with device-scope (write-through)
// stores, wait until every store of the workgroup has completed, and one
// thread bumps the counter; a consumer's first thread polls the counter with
// device-scope loads (bounded: on timeout it flags UNO_DEV_SYNC_TIMEOUT in
// status[0] and goes on), and the partials are then read with device-scope
// loads.  No L2 write-back or invalidation is needed on either side.  When
// each column group's K splits count themselves in a counter of their own,
// the last of them to arrive (it reads the others' partials with
// device-scope loads) writes the group's final bf16 T the same way and alone
// bumps the projection's counter, which then waits for one bump per group.
constexpr unsigned kLoraSpinLimit = 1u << 22;
__device__ __forceinline__ void signal_done(unsigned* counter) {
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (threadIdx.x == 0) __hip_atomic_fetch_add(counter, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void wait_lora_t(const GemmArgs& a) {
  if (threadIdx.x == 0) {
    unsigned it = 0;
    while (__hip_atomic_load(a.t_wait, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) <
           a.t_wait_target) {
      if (++it > kLoraSpinLimit) {
        if (a.t_timeout) atomicOr(a.t_timeout, UNO_DEV_SYNC_TIMEOUT);
        break;
      }
      __builtin_amdgcn_s_sleep(4);
    }
  }
  __syncthreads();
}
__device__ __forceinline__ float ld_coherent(const float* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t ld_coherent_u32(const uint32_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// eight consecutive floats, summed over `splits` partial planes zs apart in
// split order (device-scope loads, all issued before the first add)
__device__ __forceinline__ void sum_splits8_coherent(const float* p, size_t zs, int splits,
                                                     float4* lo, float4* hi) {
  float v[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) v[i] = ld_coherent(p + i);
  for (int z0 = 1; z0 < splits; z0 += 2) {
    float q[2][8];
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int i = 0; i < 8; ++i) q[u][i] = z0 + u < splits ? ld_coherent(p + (size_t)(z0 + u) * zs + i) : 0.f;
#pragma unroll
    for (int u = 0; u < 2; ++u)
      if (z0 + u < splits)
#pragma unroll
        for (int i = 0; i < 8; ++i) v[i] += q[u][i];
  }
  *lo = make_float4(v[0], v[1], v[2], v[3]);
  *hi = make_float4(v[4], v[5], v[6], v[7]);
}

// 16-column tile t of workgroup g: consecutive tiles, or (PAIR) the tile pair
// (p0, p0 + P), p0 = (g / P) * 2P + g % P, P = a.pair_tiles: the partner
// columns of a rotate-half RoPE pair (P = head_dim / 32) or of SwiGLU's gate
// and up (P = d_ffn / 16) land in one workgroup.
template <int NT, bool PAIR>
__device__ __forceinline__ int skinny_tile(const GemmArgs& a, int g, int t) {
  if (!PAIR) return g * NT + t;
  const int P = a.pair_tiles;
  return (g / P) * 2 * P + g % P + t * P;
}

// MT: 16-row tiles of X per workgroup; NT: 16-column tiles of W per
// workgroup (MT * NT <= 4); WV waves split the workgroup's K range, each with
// UN K steps of loads in flight; PAIR: the tile pairs of skinny_tile, with
// the RoPE + K/V write or the SwiGLU product applied in the epilogue (no K
// split across workgroups).  grid = (column groups, row groups, K splits).
template <int MT, int NT, int WV, int UN, bool PAIR>
__device__ __forceinline__ void skinny_body(const GemmArgs& a, const int bx, const int by,
                                            const int zs, const int splits) {
  __shared__ f32x4 red[WV * MT * NT * 64];
  __shared__ float rmax[MT * 16];             // row maxima of this workgroup (max_part)
  if (threadIdx.x < MT * 16) reinterpret_cast<int*>(rmax)[threadIdx.x] = kNegInfBits;
  const int w = threadIdx.x >> 6, l = threadIdx.x & 63;
  const int rr = l & 15, kg = l >> 4;
  SegView svt[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) svt[t] = pick_segment(a, skinny_tile<NT, PAIR>(a, bx, t));
  const SegView& sv = svt[0];
  const int m0 = by * MT * 16;

  // W in the tile-packed layout: the 16 x 32 fragment of 16-row tile nt and
  // K step s is 1 KB at ((nt * Kd/32) + s) * 512 elements, lane l's 8 values
  // at l * 8, so a wave's fragment load is one contiguous 1 KB read (tiles past
  // the segment re-read its last tile)
  const uint16_t* wrow[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    const int c = PAIR ? svt[t].n0 : sv.n0 + t * 16;
    const int nt = (c < svt[t].n ? c : svt[t].n - 16) >> 4;
    wrow[t] = svt[t].w + (size_t)nt * (a.Kd >> 5) * 512 + l * 8;
  }
  const uint16_t* xrow[MT];
  bool xok[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    const int m = m0 + mt * 16 + rr;
    xok[mt] = m < a.M;
    xrow[mt] = a.x + (size_t)(xok[mt] ? m : 0) * a.ldx + kg * 8;
  }
  f32x4 acc[MT][NT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int t = 0; t < NT; ++t) acc[mt][t] = f32x4{0.f, 0.f, 0.f, 0.f};

  // this split's 32-wide K steps.  One row tile (MT = 1): wave w takes blocks
  // of UN consecutive steps (ks0 + UN*w, then every WV-th block), so each of its
  // W rows is read in 256-byte runs; more row tiles: wave w takes the steps
  // ks0 + w, ks0 + w + WV, ... (even split of short ranges over the waves).
  const int n_all = a.Kd >> 5;
  const int ks0 = n_all * zs / splits, ks1 = n_all * (zs + 1) / splits;
  constexpr bool kBlk = MT == 1;
  constexpr int kUS = kBlk ? 1 : WV;          // step distance inside a group
  // Whole groups of UN steps.  Paired products double-buffer them in
  // registers (kPipe below): the loads of the wave's next group are issued
  // before the MFMAs of the current one, so two groups are in flight while the
  // MFMAs run (with one, a wave sits idle for a whole HBM round trip per
  // group).  The accumulation order is the same either way.  Every load of a
  // group is unconditional, so that the compiler can count exactly how many
  // are still in flight: rows past M re-read row 0 (xrow), and their output
  // rows are never stored.
  int s = ks0 + (kBlk ? w * UN : w);
  constexpr int kGrp = UN * WV;               // distance between a wave's groups
  // whole groups of this wave: s + g * kGrp + (UN - 1) * kUS < ks1
  const int span = ks1 - s - (UN - 1) * kUS;
  const int n_grp = span > 0 ? (span + kGrp - 1) / kGrp : 0;
  Frag bw0[UN][NT], ax0[UN][MT], bw1[UN][NT], ax1[UN][MT];
  auto load_grp = [&](int s_, Frag (&bw)[UN][NT], Frag (&ax)[UN][MT]) {
#pragma unroll
    for (int u = 0; u < UN; ++u)
#pragma unroll
      for (int t = 0; t < NT; ++t) bw[u][t].u = ldg16_nt(wrow[t] + (size_t)(s_ + u * kUS) * 512);
#pragma unroll
    for (int u = 0; u < UN; ++u)
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) ax[u][mt].u = ldg16(xrow[mt] + (s_ + u * kUS) * 32);
  };
  auto mma_grp = [&](const Frag (&bw)[UN][NT], const Frag (&ax)[UN][MT]) {
#pragma unroll
    for (int u = 0; u < UN; ++u)
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int t = 0; t < NT; ++t)
          acc[mt][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ax[u][mt].v, bw[u][t].v, acc[mt][t], 0, 0, 0);
  };
  // Paired products only: they stream the whole K in few workgroups.  Split
  // products run many small workgroups per CU, where the second buffer's
  // registers cost more occupancy than it gains, and groups of more than 16
  // fragments (the LM head's eight K steps of four tiles) already keep enough
  // in flight.
  constexpr bool kPipe = PAIR && UN * (NT + MT) <= 16;
  if (!kPipe) {
    for (int g = 0; g < n_grp; ++g, s += kGrp) {
      load_grp(s, bw0, ax0);
      __builtin_amdgcn_sched_barrier(0);
      mma_grp(bw0, ax0);
      __builtin_amdgcn_sched_barrier(0);
    }
  } else if (n_grp > 0) {
    load_grp(s, bw0, ax0);
    int g = 0;
    // (the fences keep each group's loads ahead of the other group's MFMAs:
    // left alone, the scheduler sinks some of them below the MFMAs)
    for (; g + 2 < n_grp; g += 2) {             // groups g (in bw0/ax0) and g + 1
      load_grp(s + kGrp, bw1, ax1);
      __builtin_amdgcn_sched_barrier(0);
      mma_grp(bw0, ax0);
      __builtin_amdgcn_sched_barrier(0);
      load_grp(s + 2 * kGrp, bw0, ax0);
      __builtin_amdgcn_sched_barrier(0);
      mma_grp(bw1, ax1);
      __builtin_amdgcn_sched_barrier(0);
      s += 2 * kGrp;
    }
    if (g + 2 == n_grp) {                       // two left
      load_grp(s + kGrp, bw1, ax1);
      __builtin_amdgcn_sched_barrier(0);
      mma_grp(bw0, ax0);
      mma_grp(bw1, ax1);
      s += 2 * kGrp;
    } else {                                    // one left
      mma_grp(bw0, ax0);
      s += kGrp;
    }
  }
  // the rest: the wave's partial block (blocked), or its remaining steps
  for (; s < ks1; s += kBlk ? 1 : WV) {
    Frag bw[NT], ax[MT];
#pragma unroll
    for (int t = 0; t < NT; ++t) bw[t].u = ldg16_nt(wrow[t] + (size_t)s * 512);
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) ax[mt].u = xok[mt] ? ldg16(xrow[mt] + s * 32) : make_uint4(0, 0, 0, 0);
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int t = 0; t < NT; ++t)
        acc[mt][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ax[mt].v, bw[t].v, acc[mt][t], 0, 0, 0);
  }
  // fused LoRA (last split): T [M, r] (already gated and scaled) times B [n, r]^T.
  // Wave w takes the rank steps w, w + WV, ... (rank <= 256: at most RS each);
  // its B fragments are loaded first, so that their latency overlaps the wait
  // for T when T comes from the same launch.
  if (a.t && sv.lb && zs == splits - 1) {
    constexpr int RS = (8 + WV - 1) / WV;
    // rank 16 fills half of a 32-wide step: lanes past the rank feed zeros
    const int r_steps = (a.rank + 31) >> 5;
    Frag bwp[RS][NT];
#pragma unroll
    for (int q = 0; q < RS; ++q) {
      const int rs = w + q * WV;
      const bool kin = rs < r_steps && rs * 32 + kg * 8 < a.rank;
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        const int n = (PAIR ? svt[t].n0 : sv.n0 + t * 16) + rr;
        const uint16_t* brow =
            svt[t].lb + (size_t)(n < svt[t].n ? n : svt[t].n - 1) * a.rank + kg * 8;
        bwp[q][t].u = kin ? ldg16(brow + rs * 32) : make_uint4(0, 0, 0, 0);
      }
    }
    if (a.t_wait) wait_lora_t(a);
#pragma unroll
    for (int q = 0; q < RS; ++q) {
      const int rs = w + q * WV;
      if (rs >= r_steps) break;
      const bool kin = rs * 32 + kg * 8 < a.rank;
      Frag axt[PAIR ? NT : 1][MT];
#pragma unroll
      for (int tt = 0; tt < (PAIR ? NT : 1); ++tt)
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        Frag* ax = axt[tt];
        const int m = m0 + mt * 16 + rr;
        const size_t to = (size_t)m * a.ldt + svt[tt].t_col + rs * 32 + kg * 8;
        if (!(kin && m < a.M)) {
          ax[mt].u = make_uint4(0, 0, 0, 0);
        } else if (a.t_part) {
          // T from its LoRA-A product's split-K partials, summed in split order
          // and rounded as that product's epilogue rounds it (read from the
          // device coherence point when they come from the same launch and
          // their lines are shared)
          float4 lo, hi;
          if (a.t_wait && !a.t_lines_owned) {
            sum_splits8_coherent(a.t_part + to, (size_t)a.M * a.ldt, a.t_splits, &lo, &hi);
          } else {
            const float4* tp = reinterpret_cast<const float4*>(a.t_part + to);
            const size_t zs4 = (size_t)a.M * a.ldt / 4;
            lo = sum_splits4(tp, zs4, a.t_splits);
            hi = sum_splits4(tp + 1, zs4, a.t_splits);
          }
          const float g = (m % a.t_rows) != 0 ? a.t_scale : 0.f;
          ax[mt].u = make_uint4(pack_bf16x2(g * lo.x, g * lo.y), pack_bf16x2(g * lo.z, g * lo.w),
                                pack_bf16x2(g * hi.x, g * hi.y), pack_bf16x2(g * hi.z, g * hi.w));
        } else if (a.t_wait) {
          // final T written by the same launch: device-scope loads
          const uint32_t* tw = reinterpret_cast<const uint32_t*>(a.t + to);
          ax[mt].u = make_uint4(ld_coherent_u32(tw), ld_coherent_u32(tw + 1),
                                ld_coherent_u32(tw + 2), ld_coherent_u32(tw + 3));
        } else {
          ax[mt].u = ldg16(a.t + to);
        }
      }
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int t = 0; t < NT; ++t)
          acc[mt][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(axt[PAIR ? t : 0][mt].v,
                                                               bwp[q][t].v, acc[mt][t], 0, 0, 0);
    }
  }
  // the waves' partial tiles are summed in a fixed order
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int t = 0; t < NT; ++t) red[((w * MT + mt) * NT + t) * 64 + l] = acc[mt][t];
  __syncthreads();
  const float* redf = reinterpret_cast<const float*>(red);
  constexpr int kTile = MT * NT * 256;   // outputs of this workgroup
  // split K: fp32 partial Y, row-major [split][M][ncols] (ncols = all segments'
  // columns), so that the reductions read whole rows
  if (splits > 1) {
    const int ncols = skinny_cols(a);
    float* part = a.part + (size_t)zs * a.M * ncols;
    for (int e = threadIdx.x; e < kTile; e += WV * 64) {
      const int r = e / (NT * 16), cl = e % (NT * 16);      // row / column in the tile
      const int mt = r >> 4, rr = r & 15, t = cl >> 4, ln = (rr >> 2) * 16 + (cl & 15);
      float v = 0.f;
#pragma unroll
      for (int ww = 0; ww < WV; ++ww)
        v += redf[((((ww * MT + mt) * NT + t) * 64) + ln) * 4 + (rr & 3)];
      // (unpaired tiles of a workgroup share one segment: no dynamic index
      // into svt, which would put it in scratch memory)
      const SegView& st = PAIR ? svt[t] : sv;
      const int m = m0 + r, nl = (PAIR ? st.n0 : sv.n0 + t * 16) + (cl & 15);
      if (m < a.M && nl < st.n) {
        float* dst = part + (size_t)m * ncols + st.col_base + nl;
        if (a.t_signal) __hip_atomic_store(dst, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        else *dst = v;
      }
    }
    if constexpr (!PAIR) if (a.t_signal && a.t_tile_ctr) {
      // the last K split of this column group turns the partials into T
      // (LoRA-A products are unpaired: their tiles share one segment)
      __shared__ unsigned s_last;
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
      if (threadIdx.x == 0)
        s_last = __hip_atomic_fetch_add(a.t_tile_ctr + bx, 1u, __ATOMIC_RELAXED,
                                        __HIP_MEMORY_SCOPE_AGENT) == (unsigned)(splits - 1);
      __syncthreads();
      if (!s_last) return;
      const size_t zstride = (size_t)a.M * ncols;
      for (int e = threadIdx.x * 2; e < kTile; e += WV * 64 * 2) {
        const int r = e / (NT * 16), cl = e % (NT * 16);   // two adjacent columns
        const SegView& st = sv;
        const int m = m0 + r, nl = sv.n0 + cl;
        if (m >= a.M || nl >= st.n) continue;
        // both columns' partials of every split (at most 8) in flight at once
        const uint64_t* src =
            reinterpret_cast<const uint64_t*>(a.part + (size_t)m * ncols + st.col_base + nl);
        uint64_t q[8];
#pragma unroll
        for (int z = 0; z < 8; ++z)
          q[z] = z < splits ? __hip_atomic_load(src + z * (zstride / 2), __ATOMIC_RELAXED,
                                                __HIP_MEMORY_SCOPE_AGENT)
                            : 0ull;
        float v0 = 0.f, v1 = 0.f;
#pragma unroll
        for (int z = 0; z < 8; ++z)
          if (z < splits) {
            v0 += __uint_as_float((uint32_t)q[z]);
            v1 += __uint_as_float((uint32_t)(q[z] >> 32));
          }
        const float g = (m % a.rows_per_seq) != 0 ? a.scale : 0.f;
        __hip_atomic_store(reinterpret_cast<uint32_t*>(static_cast<uint16_t*>(a.out) +
                                                       (size_t)m * a.ldo + st.col_base + nl),
                           pack_bf16x2(g * v0, g * v1), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
      signal_done(a.t_signal);
      return;
    }
    if (a.t_signal) signal_done(a.t_signal);
    return;
  }
  if (PAIR) {
    // tile 0 holds the first channel of each pair, tile 1 its partner
    for (int e = threadIdx.x; e < MT * 256; e += WV * 64) {
      const int mt = e / 256, ln = (e & 255) >> 2, i = e & 3;
      float v0 = 0.f, v1 = 0.f;
#pragma unroll
      for (int ww = 0; ww < WV; ++ww) {
        v0 += redf[((((ww * MT + mt) * NT + 0) * 64) + ln) * 4 + i];
        v1 += redf[((((ww * MT + mt) * NT + 1) * 64) + ln) * 4 + i];
      }
      const int m = m0 + mt * 16 + 4 * (ln >> 4) + i;
      if (m >= a.M) continue;
      const int c0 = svt[0].col_base + svt[0].n0 + (ln & 15);
      if (a.rope_fuse) {
        const RopeArgs& ra = a.rope;
        const int head = c0 / ra.hd, ch = c0 % ra.hd;
        int slot;
        const int page = rope_page(ra, m, &slot);
        if (head < ra.Hq + ra.Hkv) {
          rope_store_pair(ra, m, head, ch, v0, v1, page, slot);
        } else {
          rope_store_v(ra, head - ra.Hq - ra.Hkv, ch, v0, page, slot);
          rope_store_v(ra, head - ra.Hq - ra.Hkv, ch + ra.hd / 2, v1, page, slot);
        }
      } else {
        a.act_out[(size_t)m * svt[0].n + svt[0].n0 + (ln & 15)] =
            f32_to_bf16(v0 / (1.0f + __expf(-v0)) * v1);
      }
    }
    return;
  }
  for (int e = threadIdx.x; e < kTile; e += WV * 64) {
    const int mt = e / (NT * 256), t = (e / 256) % NT, ln = (e & 255) >> 2, i = e & 3;
    float v = 0.f;
#pragma unroll
    for (int ww = 0; ww < WV; ++ww) v += redf[((((ww * MT + mt) * NT + t) * 64) + ln) * 4 + i];
    const int m = m0 + mt * 16 + 4 * (ln >> 4) + i;
    const int nl = sv.n0 + t * 16 + (ln & 15);
    if (m < a.M && nl < sv.n) {
      store_out(a, m, sv.col_base + nl, v);
      if (a.max_part) atomic_max_f32(&rmax[m - m0], v);
    }
  }
  if (a.max_part) {
    __syncthreads();
    const int t = threadIdx.x;
    if (t < MT * 16 && m0 + t < a.M)
      a.max_part[(size_t)(m0 + t) * a.max_part_ld + bx] = rmax[t];
  }
}

// The bodies read their GemmArgs in place in the kernel-argument segment: a
// reference to the by-value parameter itself makes the compiler copy the whole
// struct to scratch memory (and lose the global address space of every
// pointer loaded from it).
__device__ __forceinline__ const GemmArgs& kernarg_gemm(int i) {
  return ((const GemmArgs*)__builtin_amdgcn_kernarg_segment_ptr())[i];
}

template <int MT, int NT, int WV, int UN, bool PAIR>
__global__ void __launch_bounds__(WV * 64) k_gemm_skinny(GemmArgs) {
  skinny_body<MT, NT, WV, UN, PAIR>(kernarg_gemm(0), blockIdx.x, blockIdx.y, blockIdx.z,
                                    gridDim.z);
}

// A projection and the LoRA-A product T = X A^T that feeds its LoRA step in
// one launch: workgroups [0, n_prod) compute T's split-K partials (`ta`,
// stored at the device coherence point, each workgroup then bumps the
// counter), the rest run the projection (`a`), which streams its W first and
// waits for the counter only when it reaches its LoRA step.  Producers come
// first in dispatch order, so they are running or done by the time any
// projection workgroup waits.  grid = n_prod + gx * gy * splits, 1-D.
template <int MT, int NT, int WV, int UN, bool PAIR>
__global__ void __launch_bounds__(WV * 64)
k_gemm_skinny_lora(GemmArgs /*ta*/, GemmArgs /*a*/, int n_prod, int tgx, int tgy, int tsplits,
                   int gx, int gy, int splits) {
  int b = blockIdx.x;
  if (b < n_prod) {
    const int bx = b % tgx, by = (b / tgx) % tgy, bz = b / (tgx * tgy);
    if (kernarg_gemm(1).t_lines_owned)
      skinny_body<MT, 2, WV, 4, false>(kernarg_gemm(0), bx, by, bz, tsplits);
    else
      skinny_body<MT, 1, WV, 4, false>(kernarg_gemm(0), bx, by, bz, tsplits);
    return;
  }
  b -= n_prod;
  const int bx = b % gx, by = (b / gx) % gy, bz = b / (gx * gy);
  skinny_body<MT, NT, WV, UN, PAIR>(kernarg_gemm(1), bx, by, bz, splits);
}

// Sum the skinny kernel's split-K partials in split order and apply the
// epilogue; one thread per output (m, column).
__global__ void __launch_bounds__(256)
k_gemm_skinny_reduce(GemmArgs a, int splits) {
  const int ncols = skinny_cols(a);
  const int g = blockIdx.x * 256 + threadIdx.x;
  if (g >= a.M * ncols) return;
  const float v = sum_splits(a.part + g, (size_t)a.M * ncols, splits);
  store_out(a, g / ncols, g % ncols, v);
}

// Split-K reduction of a q|k|v product fused with RoPE and the K/V write:
// one thread per output (m, column); for q and k the thread holding channel
// i < hd/2 of a head also sums its partner i + hd/2 and stores the rotated
// pair; v channels are stored as they are.
__global__ void __launch_bounds__(256)
k_gemm_skinny_reduce_rope(GemmArgs a, int splits) {
  const int ncols = skinny_cols(a);
  const int g = blockIdx.x * 256 + threadIdx.x;
  if (g >= a.M * ncols) return;
  const int m = g / ncols, col = g % ncols;
  const RopeArgs& ra = a.rope;
  const int hd = ra.hd, half = hd / 2;
  const int head = col / hd, ch = col % hd;
  const bool rot = head < ra.Hq + ra.Hkv;
  if (rot && ch >= half) return;                 // stored by its partner
  const size_t zs = (size_t)a.M * ncols;
  const float x = sum_splits(a.part + g, zs, splits);
  int slot;
  const int page = rope_page(ra, m, &slot);
  if (!rot) {
    rope_store_v(ra, head - ra.Hq - ra.Hkv, ch, x, page, slot);
    return;
  }
  const float xp = sum_splits(a.part + g + half, zs, splits);
  rope_store_pair(ra, m, head, ch, x, xp, page, slot);
}

// Split-K reduction of a [gate | up] product fused with SwiGLU: one thread per
// four adjacent act columns of one row.
__global__ void __launch_bounds__(256)
k_gemm_skinny_reduce_swiglu(GemmArgs a, int splits) {
  const int F = a.seg[0].n, ncols = 2 * F;
  const int g = blockIdx.x * 256 + threadIdx.x;
  if (g >= a.M * (F / 4)) return;
  const int m = g / (F / 4), c = (g % (F / 4)) * 4;
  const float4* pr = reinterpret_cast<const float4*>(a.part + (size_t)m * ncols + c);
  const size_t zs4 = (size_t)a.M * ncols / 4;
  const float4 gv = sum_splits4(pr, zs4, splits);
  const float4 uv = sum_splits4(pr + F / 4, zs4, splits);
  uint2 pk;
  pk.x = pack_bf16x2(gv.x / (1.0f + __expf(-gv.x)) * uv.x, gv.y / (1.0f + __expf(-gv.y)) * uv.y);
  pk.y = pack_bf16x2(gv.z / (1.0f + __expf(-gv.z)) * uv.z, gv.w / (1.0f + __expf(-gv.w)) * uv.w);
  *reinterpret_cast<uint2*>(a.act_out + (size_t)m * F + c) = pk;
}

// Split-K reduction of a residual-add projection over whole rows, fused with
// the RMSNorm that follows it: one workgroup (16 waves) per row m sums each
// column's splits in split order, adds the sum into the residual row (a.out),
// and writes bf16(h * rsqrt(mean(h^2) + eps) * gain) to a.norm_out.  Thread t
// owns the columns 4t..4t+3 (+ 4096); the sum of squares is reduced in a fixed
// order.
constexpr int kRedNormThreads = 1024;
__global__ void __launch_bounds__(kRedNormThreads)
k_gemm_skinny_reduce_norm(GemmArgs a, int splits) {
  constexpr int kStep = kRedNormThreads * 4;
  constexpr int kMaxIt = 2;                    // D <= 8192
  constexpr int kW = kRedNormThreads / UNO_WAVE;
  __shared__ float red[kW];
  const int m = blockIdx.x;
  const int D = a.seg[0].n;
  float* h = static_cast<float*>(a.out) + (size_t)m * a.ldo;
  const float4* pr = reinterpret_cast<const float4*>(a.part + (size_t)m * D);
  const size_t zs4 = (size_t)a.M * D / 4;
  float4 hv[kMaxIt];
  float ss = 0.f;
#pragma unroll
  for (int it = 0; it < kMaxIt; ++it) {
    const int i = threadIdx.x * 4 + it * kStep;
    if (i >= D) break;
    const float4 v = sum_splits4(pr + i / 4, zs4, splits);
    float4 x = *reinterpret_cast<const float4*>(h + i);
    x.x += v.x; x.y += v.y; x.z += v.z; x.w += v.w;
    *reinterpret_cast<float4*>(h + i) = x;
    hv[it] = x;
    ss += (x.x * x.x + x.y * x.y + x.z * x.z + x.w * x.w);
  }
  ss = wave_sum(ss);
  if (lane_id() == 0) red[threadIdx.x / UNO_WAVE] = ss;
  __syncthreads();
  float tot = 0.f;
#pragma unroll
  for (int q = 0; q < kW; ++q) tot += red[q];
  const float inv = 1.0f / sqrtf(tot / (float)D + a.norm_eps);
  uint16_t* o = a.norm_out + (size_t)m * D;
#pragma unroll
  for (int it = 0; it < kMaxIt; ++it) {
    const int i = threadIdx.x * 4 + it * kStep;
    if (i >= D) break;
    const float4 g = *reinterpret_cast<const float4*>(a.norm_gain + i);
    const float4 x = hv[it];
    uint2 pk;
    pk.x = pack_bf16x2(x.x * inv * g.x, x.y * inv * g.y);
    pk.y = pack_bf16x2(x.z * inv * g.z, x.w * inv * g.w);
    *reinterpret_cast<uint2*>(o + i) = pk;
  }
}

struct SkinnyPlan {
  int mt, nt, gx, gy, splits, waves, un;
};

// Column tiles per workgroup: as many as keep >= 128 workgroups (fewer
// re-reads of X); K splits until about 512 workgroups are in flight.  Waves
// and loads in flight per wave as measured best at 16 rows: 2 waves for the
// long streams (split products, the LM head with 8 K steps in flight), 4 for
// the small LoRA-A products.
static SkinnyPlan plan_skinny(const GemmArgs& a) {
  SkinnyPlan p;
  p.waves = a.epi == EPI_LORA_T ? kSkWaves : kSkWavesSplit;
  p.un = a.max_part ? 8 : 4;
  p.mt = a.M <= 16 ? 1 : a.M <= 32 ? 2 : 4;
  p.gy = a.M <= 32 ? 1 : (a.M + 63) / 64;
  int tiles16 = 0;
  for (int i = 0; i < a.n_seg; ++i) tiles16 += (a.seg[i].n + 15) / 16;
  p.nt = 1;
  for (int nt = a.sk_nt ? 1 : 4 / p.mt; nt > 1; nt /= 2) {
    bool ok = true;
    if (a.n_seg > 1)
      for (int i = 0; i < a.n_seg; ++i) ok = ok && a.seg[i].n % (16 * nt) == 0;
    if (ok && (tiles16 + nt - 1) / nt * p.gy >= 128) { p.nt = nt; break; }
  }
  if (a.sk_nt) p.nt = a.sk_nt;
  p.gx = (tiles16 + p.nt - 1) / p.nt;
  const int steps = a.Kd >> 5;
  const size_t tile = (size_t)p.mt * p.nt * 256;
  p.splits = 1;
  const size_t per_split = (size_t)a.M * skinny_cols(a);
  if (a.part && !a.max_part)
    while (p.gx * p.gy * p.splits < 512 && steps / (p.splits * 2) >= p.waves &&
           (size_t)p.splits * 2 * per_split <= a.part_floats &&
           (a.max_splits <= 0 || p.splits * 2 <= a.max_splits))
      p.splits *= 2;
  return p;
}

// the fused reduce + SwiGLU applies to split [gate | up] products
static bool fuse_swiglu(const GemmArgs& a, const SkinnyPlan& p) {
  return p.splits > 1 && a.act_out && a.epi == EPI_STORE_F32 && a.n_seg == 2 &&
         a.seg[0].n == a.seg[1].n && a.seg[0].n % 4 == 0;
}

// the fused reduce + RMSNorm applies to split residual adds over whole rows
static bool fuse_norm(const GemmArgs& a, const SkinnyPlan& p) {
  return p.splits > 1 && a.norm_gain && a.norm_out && a.epi == EPI_ADD_F32 && a.n_seg == 1 &&
         a.seg[0].n == a.ldo && a.ldo % 4 == 0 && a.ldo <= 8192;
}

// the reduction launch that follows a split skinny product
static void launch_sk_reduce(const GemmArgs& a, const SkinnyPlan& p, hipStream_t s);

template <int MT, int NT>
static void launch_sk(const GemmArgs& a, const SkinnyPlan& p, hipStream_t s) {
  const dim3 grid(p.gx, p.gy, p.splits);
  if (p.waves == kSkWaves)
    hipLaunchKernelGGL((k_gemm_skinny<MT, NT, kSkWaves, 4, false>), grid, dim3(kSkWaves * 64), 0, s, a);
  else if (p.un == 8)
    hipLaunchKernelGGL((k_gemm_skinny<MT, NT, kSkWavesSplit, 8, false>), grid,
                       dim3(kSkWavesSplit * 64), 0, s, a);
  else
    hipLaunchKernelGGL((k_gemm_skinny<MT, NT, kSkWavesSplit, 4, false>), grid,
                       dim3(kSkWavesSplit * 64), 0, s, a);
  launch_sk_reduce(a, p, s);
}

static void launch_sk_reduce(const GemmArgs& a, const SkinnyPlan& p, hipStream_t s) {
  if (p.splits == 1 || a.partials_only) return;
  const int n = a.M * skinny_cols(a);
  if (a.rope_fuse)
    hipLaunchKernelGGL(k_gemm_skinny_reduce_rope, dim3((n + 255) / 256), dim3(256), 0, s, a,
                       p.splits);
  else if (fuse_norm(a, p))
    hipLaunchKernelGGL(k_gemm_skinny_reduce_norm, dim3(a.M), dim3(kRedNormThreads), 0, s, a,
                       p.splits);
  else if (fuse_swiglu(a, p))
    hipLaunchKernelGGL(k_gemm_skinny_reduce_swiglu, dim3((a.M * (a.seg[0].n / 4) + 255) / 256),
                       dim3(256), 0, s, a, p.splits);
  else
    hipLaunchKernelGGL(k_gemm_skinny_reduce, dim3((n + 255) / 256), dim3(256), 0, s, a, p.splits);
}

// RoPE and SwiGLU need both columns of a pair (channel i and i + hd/2 of a
// head; gate and up column c): instead of splitting K and pairing them in a
// reduction launch, one workgroup computes both 16-column tiles over the whole
// K and applies the epilogue itself.  Returns the tile distance P of the
// pairs, or 0.
static int skinny_pair_tiles(const GemmArgs& a) {
  if (a.max_part || a.partials_only || a.epi != EPI_STORE_F32 || a.M > 64) return 0;
  if (a.rope_fuse) {
    const int hd = a.rope.hd;
    if (hd % 32) return 0;
    for (int i = 0; i < a.n_seg; ++i)
      if (a.seg[i].n % hd) return 0;
    return hd / 32;
  }
  if (a.act_out && a.n_seg == 2 && a.seg[0].n == a.seg[1].n && a.seg[0].n % 16 == 0)
    return a.seg[0].n / 16;
  return 0;
}

template <int MT>
static void launch_sk_pair(const GemmArgs& a, hipStream_t s) {
  const int gx = skinny_cols(a) / 32, gy = (a.M + MT * 16 - 1) / (MT * 16);
  hipLaunchKernelGGL((k_gemm_skinny<MT, 2, kSkWaves, 4, true>), dim3(gx, gy, 1),
                     dim3(kSkWaves * 64), 0, s, a);
}

hipError_t launch_gemm_skinny(const GemmArgs& a, hipStream_t s, bool* normed, bool* roped,
                              bool* swiglued) {
  if (const int P = skinny_pair_tiles(a)) {
    GemmArgs b = a;
    b.pair_tiles = P;
    if (normed) *normed = false;
    if (roped) *roped = a.rope_fuse != 0;
    if (swiglued) *swiglued = !a.rope_fuse;
    if (a.M <= 16) launch_sk_pair<1>(b, s);
    else if (a.M <= 32) launch_sk_pair<2>(b, s);
    else launch_sk_pair<4>(b, s);
    return hipGetLastError();
  }
  const SkinnyPlan p = plan_skinny(a);
  if (normed) *normed = fuse_norm(a, p);
  if (roped) *roped = a.rope_fuse && p.splits > 1;
  if (swiglued) *swiglued = !a.rope_fuse && !fuse_norm(a, p) && fuse_swiglu(a, p);
  switch (p.mt * 8 + p.nt) {
    case 8 + 4: launch_sk<1, 4>(a, p, s); break;
    case 8 + 2: launch_sk<1, 2>(a, p, s); break;
    case 8 + 1: launch_sk<1, 1>(a, p, s); break;
    case 16 + 2: launch_sk<2, 2>(a, p, s); break;
    case 16 + 1: launch_sk<2, 1>(a, p, s); break;
    default: launch_sk<4, 1>(a, p, s); break;
  }
  return hipGetLastError();
}

// One launch of a projection and its LoRA-A product (k_gemm_skinny_lora):
// MT row tiles, the projection's NT column tiles, WV waves, UN loads in flight.
template <int MT, int NT, int WV, int UN, bool PAIR>
static void launch_sk_lora(const GemmArgs& ta, const SkinnyPlan& tp, const GemmArgs& a, int gx,
                           int gy, int splits, hipStream_t s) {
  const int n_prod = tp.gx * tp.gy * tp.splits;
  hipLaunchKernelGGL((k_gemm_skinny_lora<MT, NT, WV, UN, PAIR>), dim3(n_prod + gx * gy * splits),
                     dim3(WV * 64), 0, s, ta, a, n_prod, tp.gx, tp.gy, tp.splits, gx, gy, splits);
}

hipError_t launch_gemm_lora(const GemmArgs& a, const GemmArgs& ta, float* t_part,
                            size_t t_part_floats, unsigned* counter, int* timeout_flag,
                            hipStream_t s, bool* normed, bool* roped, bool* swiglued,
                            bool* fused) {
  GemmArgs g, t2;
  gemm_lora_pair(a, ta, t_part, t_part_floats, &g, &t2);
  *fused = false;
  if (!counter || !t2.partials_only || a.M > 32) {
    const hipError_t e = launch_gemm(t2, s);
    if (e != hipSuccess) return e;
    return launch_gemm(g, s, normed, roped, swiglued);
  }
  // LoRA-A workgroups of two 16-column tiles: with 32-float aligned rows each
  // 128-byte line of the partials has one writer
  bool owned = g.ldt == skinny_cols(t2);
  for (int i = 0; i < t2.n_seg; ++i) owned = owned && t2.seg[i].n % 32 == 0;
  if (owned) t2.sk_nt = 2;
  // a narrow LoRA-A product (one segment: the o and down projections) has few
  // workgroups; more K splits let it finish before the projection's deep
  // stream reaches its LoRA step (down at 16 rows: 2.16 -> 2.06 ms per step)
  if (skinny_cols(t2) <= 128) t2.max_splits = 8;
  SkinnyPlan tp = plan_skinny(t2);
  g.t_splits = tp.splits;
  t2.t_signal = counter;
  g.t_wait = counter;
  g.t_wait_target = (unsigned)(tp.gx * tp.gy * tp.splits);
  g.t_timeout = timeout_flag;
  g.t_lines_owned = owned && tp.nt == 2;
  const int P = skinny_pair_tiles(g);
  SkinnyPlan p = plan_skinny(g);
  if (tp.nt != (owned ? 2 : 1) || tp.splits < 2 || (!P && p.mt != tp.mt)) {
    const hipError_t e = launch_gemm(t2, s);
    if (e != hipSuccess) return e;
    g.t_wait = nullptr;
    return launch_gemm(g, s, normed, roped, swiglued);
  }
  // one row tile of 32-column groups whose T is the projection's LoRA input:
  // the last K split of each group writes the group's final bf16 T, so that
  // the projection reads 2-byte T once instead of summing fp32 partials
  if (g.t_lines_owned && tp.gy == 1 && tp.gx < kLoraSyncWords && tp.splits <= 8 &&
      t2.out == g.t && t2.ldo == g.ldt) {
    t2.t_tile_ctr = counter + 1;
    g.t_part = nullptr;
    g.t_wait_target = (unsigned)tp.gx;
  }
  *fused = true;
  if (P) {
    g.pair_tiles = P;
    if (normed) *normed = false;
    if (roped) *roped = g.rope_fuse != 0;
    if (swiglued) *swiglued = !g.rope_fuse;
    const int gx = skinny_cols(g) / 32;
    if (g.M <= 16)
      launch_sk_lora<1, 2, kSkWaves, 4, true>(t2, tp, g, gx, 1, 1, s);
    else if (g.M <= 32)
      launch_sk_lora<2, 2, kSkWaves, 4, true>(t2, tp, g, gx, 1, 1, s);
    else
      launch_sk_lora<4, 2, kSkWaves, 4, true>(t2, tp, g, gx, (g.M + 63) / 64, 1, s);
    return hipGetLastError();
  }
  if (normed) *normed = fuse_norm(g, p);
  if (roped) *roped = g.rope_fuse && p.splits > 1;
  if (swiglued) *swiglued = !g.rope_fuse && !fuse_norm(g, p) && fuse_swiglu(g, p);
  // the LoRA-A workgroups run with the projection's wave count
#define UNO_SK_LORA(MT_, NT_)                                                              \
  (p.waves == kSkWaves                                                                     \
       ? launch_sk_lora<MT_, NT_, kSkWaves, 4, false>(t2, tp, g, p.gx, p.gy, p.splits, s)  \
       : p.un == 8 ? launch_sk_lora<MT_, NT_, kSkWavesSplit, 8, false>(t2, tp, g, p.gx,    \
                                                                       p.gy, p.splits, s)  \
                   : launch_sk_lora<MT_, NT_, kSkWavesSplit, 4, false>(t2, tp, g, p.gx,    \
                                                                       p.gy, p.splits, s))
  switch (p.mt * 8 + p.nt) {
    case 8 + 4: UNO_SK_LORA(1, 4); break;
    case 8 + 2: UNO_SK_LORA(1, 2); break;
    case 8 + 1: UNO_SK_LORA(1, 1); break;
    case 16 + 2: UNO_SK_LORA(2, 2); break;
    case 16 + 1: UNO_SK_LORA(2, 1); break;
    default: UNO_SK_LORA(4, 1); break;
  }
#undef UNO_SK_LORA
  launch_sk_reduce(g, p, s);
  return hipGetLastError();
}

void gemm_lora_pair(const GemmArgs& a, const GemmArgs& ta, float* t_part, size_t t_part_floats,
                    GemmArgs* a_out, GemmArgs* ta_out) {
  *a_out = a;
  *ta_out = ta;
  if (!t_part || a.M > 64 || ta.M != a.M || ta.epi != EPI_LORA_T || !a.t ||
      a.ldt != skinny_cols(ta) || a.ldt % 4)
    return;
  GemmArgs t2 = ta;
  t2.part = t_part;
  t2.part_floats = t_part_floats;
  t2.max_splits = 4;
  const SkinnyPlan p = plan_skinny(t2);
  if (p.splits < 2) return;
  t2.partials_only = 1;
  *ta_out = t2;
  a_out->t_part = t_part;
  a_out->t_splits = p.splits;
  a_out->t_scale = ta.scale;
  a_out->t_rows = ta.rows_per_seq;
}

// ============================================================================
// Tiled kernel (many rows: batched decode blocks, prompt chunks).
// Workgroup tile BM x BN (rows of X x columns of W), WM x WN waves, each wave
// (BM/WM) x (BN/WN) as 32 x 32 tiles of v_mfma_f32_32x32x16_bf16.  Both
// operands stream through LDS in 32-wide K slices by direct global -> LDS DMA
// (global_load_lds_dwordx4), S slices resident: S-1 are in flight while the
// MFMAs of one run.  LDS rows are 64 bytes (4 chunks of 16 bytes), the chunk
// index XOR-ed with (row / 4) % 4 so that the 16 lanes served together hit 16
// distinct 16-byte bank groups; the DMA applies the swizzle by choosing which
// source chunk each lane copies.  Each half-slice's fragments are read while
// the MFMAs of the other half issue.  The LoRA product runs as r/32 extra K
// slices with T and B as operands.  Configurations:
//   L  256 x 256, 8 waves, 5 stages (160 KB LDS): one workgroup per CU
//   M  256 x 128, 4 waves, 3 stages (72 KB): two workgroups per CU
//   S  128 x 128, 4 waves, 4 stages (64 KB): two workgroups per CU
// Two resident workgroups cover each other's barrier waits, prologue and
// epilogue.
//
// Split-K: whole rounds of tiles run unsplit; the tiles left over for a last,
// partly filled round (or all tiles, when there are too few for the chip) are
// split over K.  Every split writes its fp32 partial tile to scratch and a
// second kernel sums the splits in order (run-to-run identical) and applies
// the epilogue.
// ============================================================================
namespace big {
constexpr int BK = 32;
template <int BM_, int BN_, int WM_, int WN_, int S_>
struct Cfg {
  static constexpr int BM = BM_, BN = BN_, WM = WM_, WN = WN_, S = S_;
  static constexpr int kWaves = WM * WN, kThreads = kWaves * 64;
  static constexpr int TM = BM / WM, TN = BN / WN;   // wave tile
  static constexpr int TI = TM / 32, TJ = TN / 32;   // MFMA tiles per wave
  static constexpr int kLdsA = BM * BK * 2, kLdsB = BN * BK * 2, kStage = kLdsA + kLdsB;
  static constexpr int kInstr = kStage / 1024;       // 1 KB DMA instructions per slice
  static constexpr int kIW = kInstr / kWaves;        // per wave
  static constexpr int kInstrA = kLdsA / 1024;
  static constexpr int kIA = kInstrA / kWaves;       // A instructions per wave (first)
  static constexpr int kIB = kIW - kIA;              // then B instructions
  static constexpr int kLds = S * kStage;
  static constexpr int kTileFloats = BM * BN;
  static_assert(kInstr % kWaves == 0 && kInstrA % kWaves == 0,
                "DMA instructions of A and of B must split evenly over the waves");
};
using CfgL = Cfg<256, 256, 2, 4, 5>;
using CfgM = Cfg<256, 128, 2, 2, 3>;
using CfgS = Cfg<128, 128, 2, 2, 4>;
__device__ __forceinline__ int swz_f(int row) { return (row >> 2) & 3; }
__device__ __forceinline__ int swz(int row, int chunk) { return row * 64 + ((chunk ^ swz_f(row)) << 4); }

// Work item -> (m tile, split, n tile).  Consecutive workgroups go round-robin
// over the 8 XCDs; each XCD gets a contiguous range of items (m tile fastest,
// then the split, then the n tile) so the workgroups sharing W columns share
// an L2.
struct Item {
  int mt, z, nt;
};
__device__ __forceinline__ Item item_of(int id, int m_tiles, int splits, int nwg) {
  const int xcd = id & 7, q = nwg >> 3, r8 = nwg & 7;
  const int lin = xcd * q + (xcd < r8 ? xcd : r8) + (id >> 3);
  Item it;
  it.mt = lin % m_tiles;
  const int rest = lin / m_tiles;
  it.z = rest % splits;
  it.nt = rest / splits;
  return it;
}
}  // namespace big


// two waves per SIMD in every configuration (at most 256 VGPRs per wave)
template <class C>
__global__ void __launch_bounds__(C::kThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
k_gemm_big(GemmArgs a, int m_tiles, int n_tiles, int splits, int n_full) {
  using namespace big;
  constexpr int TI = C::TI, TJ = C::TJ, IW = C::kIW, S = C::S;
  extern __shared__ __attribute__((aligned(16))) unsigned char lds[];
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63;
  const int wm = w / C::WN, wn = w % C::WN;

  // Tiles [0, n_full) run whole, one workgroup each (XCD-aware order); the
  // remaining tiles are split `splits` ways over K to fill the last round.
  int mt, nt, z, sp;
  if ((int)blockIdx.x < n_full) {
    const Item it = item_of(blockIdx.x, m_tiles, 1, n_full);
    mt = it.mt; nt = it.nt; z = 0; sp = 1;
  } else {
    const int j = blockIdx.x - n_full;
    const int tile = n_full + j / splits;
    mt = tile % m_tiles; nt = tile / m_tiles; z = j % splits; sp = splits;
  }
  const int m0 = mt * C::BM;
  // SwiGLU pairs: tile nt covers act columns [nt*BN/2, (nt+1)*BN/2); its
  // rows 0..BN/2-1 are those gate rows, rows BN/2..BN-1 the same up rows
  const bool pair = a.epi == EPI_SWIGLU;
  constexpr int HALF = C::BN / 2;
  const SegView sv = pick_segment(a, pair ? 0 : nt * (C::BN / 16));
  const int n0 = pair ? nt * HALF : sv.n0;
  const int wrows = pair ? 2 * sv.n : sv.n;        // rows the W / LoRA B resources span

  // K slices of this split (LoRA slices after the last split's base slices)
  const int nk_base = a.Kd / BK;
  const int nk_r = (a.t && sv.lb) ? a.rank / BK : 0;
  const int nk_lora = pair ? 2 * nk_r : nk_r;   // pairs: [T_gate | T_up] against [B_g, 0 | 0, B_u]
  const int kb0 = nk_base * z / sp, kb1 = nk_base * (z + 1) / sp;
  const int nk = (kb1 - kb0) + (z == sp - 1 ? nk_lora : 0);

  // DMA: every wave issues kIA instructions of A rows, then kIB of B rows,
  // each 16 rows x 64 bytes; lane l fills row 16*i + l/4 (i the instruction's
  // index among all A or all B instructions), physical chunk l%4, which holds
  // logical chunk (l%4) ^ swz_f(row).  Rows past M / past the segment re-read
  // a valid row; their results are discarded.  Buffer loads with per-lane byte
  // offsets fixed here and the slice's K offset as the scalar offset; the
  // resources span exactly the operands, so no load leaves them.
  constexpr int IA = C::kIA, IB = C::kIB;
  const int wu = __builtin_amdgcn_readfirstlane(w);
  const i32x4 rs_x = make_rsrc(a.x, (uint32_t)((size_t)a.M * a.ldx * 2));
  const i32x4 rs_w = make_rsrc(sv.w, (uint32_t)((size_t)wrows * a.Kd * 2));
  const i32x4 rs_t = a.t ? make_rsrc(a.t, (uint32_t)((size_t)a.M * a.ldt * 2)) : rs_x;
  const uint32_t lb_bytes = (uint32_t)((size_t)wrows * a.rank * 2);
  const i32x4 rs_lb = sv.lb ? make_rsrc(sv.lb, lb_bytes) : rs_w;
  uint32_t vb[IW], vl[IW];
#pragma unroll
  for (int ii = 0; ii < IW; ++ii) {
    const bool is_a = ii < IA;
    const int row = (is_a ? wu * IA + ii : wu * IB + ii - IA) * 16 + (l >> 2);
    const int ch = (l & 3) ^ swz_f(row);
    if (is_a) {
      const int m = m0 + row < a.M ? m0 + row : 0;
      vb[ii] = (uint32_t)(((size_t)m * a.ldx + ch * 8) * 2);
      vl[ii] = (uint32_t)(((size_t)m * a.ldt + sv.t_col + ch * 8) * 2);
    } else {
      int n;
      if (pair) n = row < HALF ? n0 + row : sv.n + n0 + row - HALF;
      else n = n0 + row < sv.n ? n0 + row : sv.n - 1;
      // tile-packed W: row n's logical chunk ch of a 32-wide K slice sits at
      // byte ((n / 16) * Kd/32 * 1024) + (ch * 16 + n % 16) * 16 of its tile
      vb[ii] = (uint32_t)((size_t)(n >> 4) * (a.Kd >> 5) * 1024 + (ch * 16 + (n & 15)) * 16);
      vl[ii] = (uint32_t)(((size_t)n * a.rank + ch * 8) * 2);
    }
  }
  // SwiGLU pairs, LoRA slices q < nk_r feed T_gate, the rest T_up: the other
  // half's B rows read past the end of their resource, which returns zeros
  const int b_up0 = pair ? (HALF / 16 - wu * IB + IA) : 0x7fffffff;  // first up instruction
  const uint32_t lds0 = lds_addr(lds);
  const uint32_t dst_a = lds0 + wu * IA * 1024, dst_b = lds0 + C::kLdsA + wu * IB * 1024;
  auto issue = [&](int s, int stage) {
    const int kk = kb0 + s;
    const uint32_t so = stage * C::kStage;
    if (kk < kb1) {
      const uint32_t soff = __builtin_amdgcn_readfirstlane(kk * BK * 2);
      const uint32_t soff_w = __builtin_amdgcn_readfirstlane(kk * 1024);   // packed W
#pragma unroll
      for (int ii = 0; ii < IW; ++ii) {
        if (ii < IA) lds_dma16_buf(rs_x, vb[ii], soff, dst_a + so + ii * 1024);
        else lds_dma16_buf(rs_w, vb[ii], soff_w, dst_b + so + (ii - IA) * 1024);
      }
    } else {
      const int q = kk - kb1;
      const uint32_t soff = __builtin_amdgcn_readfirstlane(q * BK * 2);
      // pairs: gate rows take slices q < nk_r, up rows q >= nk_r (at q - nk_r)
      const uint32_t soff_g = __builtin_amdgcn_readfirstlane(q < nk_r ? q * BK * 2 : lb_bytes);
      const uint32_t soff_u =
          __builtin_amdgcn_readfirstlane(q >= nk_r ? (q - nk_r) * BK * 2 : lb_bytes);
#pragma unroll
      for (int ii = 0; ii < IW; ++ii) {
        if (ii < IA) lds_dma16_buf(rs_t, vl[ii], soff, dst_a + so + ii * 1024);
        else if (!pair) lds_dma16_buf(rs_lb, vl[ii], soff, dst_b + so + (ii - IA) * 1024);
        else lds_dma16_buf(rs_lb, vl[ii], ii < b_up0 ? soff_g : soff_u,
                           dst_b + so + (ii - IA) * 1024);
      }
    }
  };
  // slice s has landed once at most `ahead` later slices of this wave are in flight
  auto wait_slice = [&](int ahead) {
    if (S > 3 && ahead >= 3) wait_vmcnt<3 * IW>();
    else if (ahead >= 2) wait_vmcnt<2 * IW>();
    else if (ahead == 1) wait_vmcnt<IW>();
    else wait_vmcnt<0>();
  };

  Frag fa0[TI], fb0[TJ], fa1[TI], fb1[TJ];
  auto read = [&](int stage, int kk, Frag (&fa)[TI], Frag (&fb)[TJ]) {
    const unsigned char* A = lds + stage * C::kStage;
    const unsigned char* B = A + C::kLdsA;
    const int ch = 2 * kk + (l >> 5);
#pragma unroll
    for (int i = 0; i < TI; ++i)
      fa[i].u = *reinterpret_cast<const uint4*>(A + swz(wm * C::TM + i * 32 + (l & 31), ch));
#pragma unroll
    for (int j = 0; j < TJ; ++j)
      fb[j].u = *reinterpret_cast<const uint4*>(B + swz(wn * C::TN + j * 32 + (l & 31), ch));
  };
  f32x16 acc[TI][TJ];
#pragma unroll
  for (int i = 0; i < TI; ++i)
#pragma unroll
    for (int j = 0; j < TJ; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;
  auto mma = [&](const Frag (&fa)[TI], const Frag (&fb)[TJ]) {
#pragma unroll
    for (int i = 0; i < TI; ++i)
#pragma unroll
      for (int j = 0; j < TJ; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[i].v, fb[j].v, acc[i][j], 0, 0, 0);
  };

  if (nk > 0) {
#pragma unroll
    for (int s = 0; s < S; ++s)
      if (s < nk) issue(s, s);
    wait_slice(nk - 1 < S - 1 ? nk - 1 : S - 1);
    __syncthreads();
    // The scheduling fences keep each half-slice's fragment reads ahead of
    // the MFMAs of the other half (left alone, the compiler sinks the reads
    // next to their use and the LDS latency is exposed).
    int st = 0;                       // stage of slice s
    read(st, 0, fa0, fb0);
    int s = 0;
    // steady state: slices s+1 .. s+S-1 are in flight, s+1 must have landed,
    // and slice s+S refills the stage just read
    for (; s < nk - S; ++s) {
      read(st, 1, fa1, fb1);
      __builtin_amdgcn_sched_barrier(0);
      mma(fa0, fb0);
      __builtin_amdgcn_sched_barrier(0);
      wait_vmcnt<(S - 2) * IW>();
      __syncthreads();   // every wave is done with stage st (and has s+1)
      const int nst = st + 1 == S ? 0 : st + 1;
      read(nst, 0, fa0, fb0);
      issue(s + S, st);
      st = nst;
      __builtin_amdgcn_sched_barrier(0);
      mma(fa1, fb1);
      __builtin_amdgcn_sched_barrier(0);
    }
    // tail: nothing left to issue; wait for everything in flight
    for (; s < nk - 1; ++s) {
      read(st, 1, fa1, fb1);
      __builtin_amdgcn_sched_barrier(0);
      mma(fa0, fb0);
      __builtin_amdgcn_sched_barrier(0);
      wait_vmcnt<0>();
      __syncthreads();
      st = st + 1 == S ? 0 : st + 1;
      read(st, 0, fa0, fb0);
      __builtin_amdgcn_sched_barrier(0);
      mma(fa1, fb1);
      __builtin_amdgcn_sched_barrier(0);
    }
    read(st, 1, fa1, fb1);
    mma(fa0, fb0);
    mma(fa1, fb1);
  }

  if (sp > 1) {
    // partial tile, layout [wave][i][j][e/4][lane] of float4
    const int rem = m_tiles * n_tiles - n_full;
    const int tile = nt * m_tiles + mt - n_full;
    float4* dst = reinterpret_cast<float4*>(
        a.part + ((size_t)z * rem + tile) * C::kTileFloats);
#pragma unroll
    for (int i = 0; i < TI; ++i)
#pragma unroll
      for (int j = 0; j < TJ; ++j)
#pragma unroll
        for (int e4 = 0; e4 < 4; ++e4)
          dst[(((w * TI + i) * TJ + j) * 4 + e4) * 64 + l] =
              make_float4(acc[i][j][4 * e4], acc[i][j][4 * e4 + 1], acc[i][j][4 * e4 + 2],
                          acc[i][j][4 * e4 + 3]);
    return;
  }

  if (pair) {
    // the up waves (wn >= WN/2) hand their tile to the gate waves through LDS
    // (same fragment layout), which write bf16(silu(g) * u)
    constexpr int HW = C::WN / 2, NF = TI * TJ * 16;
    __syncthreads();                                   // stages no longer read
    float* xch = reinterpret_cast<float*>(lds);
    const int slot = wm * HW + (wn % HW);
    if (wn >= HW) {
#pragma unroll
      for (int i = 0; i < TI; ++i)
#pragma unroll
        for (int j = 0; j < TJ; ++j)
#pragma unroll
          for (int e = 0; e < 16; ++e) xch[((slot * NF) + (i * TJ + j) * 16 + e) * 64 + l] = acc[i][j][e];
    }
    __syncthreads();
    if (wn < HW) {
      uint16_t* out = static_cast<uint16_t*>(a.out);
#pragma unroll
      for (int j = 0; j < TJ; ++j) {
        const int c = n0 + wn * C::TN + j * 32 + (l & 31);
#pragma unroll
        for (int i = 0; i < TI; ++i)
#pragma unroll
          for (int e = 0; e < 16; ++e) {
            const int m = m0 + wm * C::TM + i * 32 + (e >> 2) * 8 + (l >> 5) * 4 + (e & 3);
            const float g = acc[i][j][e];
            const float u = xch[((slot * NF) + (i * TJ + j) * 16 + e) * 64 + l];
            if (m < a.M) out[(size_t)m * a.ldo + c] = f32_to_bf16(g / (1.0f + __expf(-g)) * u);
          }
      }
    }
    return;
  }

  // epilogue: lane holds rows (e/4)*8 + (l/32)*4 + e%4, column l%32 of each 32x32 tile
#pragma unroll
  for (int j = 0; j < TJ; ++j) {
    const int nl = n0 + wn * C::TN + j * 32 + (l & 31);
    if (nl >= sv.n) continue;
#pragma unroll
    for (int i = 0; i < TI; ++i)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int m = m0 + wm * C::TM + i * 32 + (e >> 2) * 8 + (l >> 5) * 4 + (e & 3);
        if (m < a.M) store_out(a, m, sv.col_base + nl, acc[i][j][e]);
      }
  }
  if (a.max_part) {
    // row maxima over the tile's columns: a lane's columns, then the 32 lanes
    // that share its rows, then the WN waves (LDS), one partial per row
    __syncthreads();                                   // stages no longer read
    float* rmax = reinterpret_cast<float*>(lds);
    for (int t = tid; t < C::BM; t += C::kThreads) reinterpret_cast<int*>(rmax)[t] = kNegInfBits;
    __syncthreads();
#pragma unroll
    for (int i = 0; i < TI; ++i)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        float mx = -INFINITY;
#pragma unroll
        for (int j = 0; j < TJ; ++j)
          if (n0 + wn * C::TN + j * 32 + (l & 31) < sv.n) mx = fmaxf(mx, acc[i][j][e]);
#pragma unroll
        for (int o = 1; o < 32; o <<= 1) mx = fmaxf(mx, __shfl_xor(mx, o, UNO_WAVE));
        if ((l & 31) == 0)
          atomic_max_f32(&rmax[wm * C::TM + i * 32 + (e >> 2) * 8 + (l >> 5) * 4 + (e & 3)], mx);
      }
    __syncthreads();
    for (int t = tid; t < C::BM; t += C::kThreads)
      if (m0 + t < a.M) a.max_part[(size_t)(m0 + t) * a.max_part_ld + nt] = rmax[t];
  }
}

// Sum the split-K partial tiles in split order and apply the epilogue; one
// thread per float4 of a partial tile (4 rows of one column).
template <class C>
__global__ void __launch_bounds__(256)
k_gemm_splitk_reduce(GemmArgs a, int m_tiles, int n_tiles, int splits, int n_full) {
  constexpr int Q = C::kTileFloats / 4;        // float4 per tile
  const int rem = m_tiles * n_tiles - n_full;  // the split tiles n_full, n_full + 1, ...
  const int g = blockIdx.x * 256 + threadIdx.x;
  if (g >= rem * Q) return;
  const int tr = g / Q, q = g % Q;
  const int tile = n_full + tr;
  const int mt = tile % m_tiles, nt = tile / m_tiles;
  const float4* src = reinterpret_cast<const float4*>(a.part);
  const float4 t = sum_splits4(src + (size_t)tr * Q + q, (size_t)rem * Q, splits);
  // q = (((w * TI + i) * TJ + j) * 4 + e4) * 64 + l
  const int l = q & 63;
  int r = q >> 6;
  const int e4 = r & 3;
  r >>= 2;
  const int j = r % C::TJ;
  r /= C::TJ;
  const int i = r % C::TI, w = r / C::TI;
  const int wm = w / C::WN, wn = w % C::WN;
  const SegView sv = pick_segment(a, nt * (C::BN / 16));
  const int nl = sv.n0 + wn * C::TN + j * 32 + (l & 31);
  if (nl >= sv.n) return;
  const int mb = mt * C::BM + wm * C::TM + i * 32 + e4 * 8 + (l >> 5) * 4;
  const float v[4] = {t.x, t.y, t.z, t.w};
#pragma unroll
  for (int c = 0; c < 4; ++c)
    if (mb + c < a.M) store_out(a, mb + c, sv.col_base + nl, v[c]);
}

// Shapes the tiled kernel takes with column tile bn: K and the LoRA rank in
// whole 32-wide slices, 16-byte aligned rows, every segment but a single one
// a whole number of tiles (a single segment may end in a partial tile).
static bool big_ok(const GemmArgs& a, int bn) {
  if (a.Kd % big::BK || a.ldx % 8) return false;
  if (a.t && (a.rank % big::BK || a.ldt % 8)) return false;
  // buffer offsets are 32-bit: every operand under 2 GiB
  const size_t lim = size_t(1) << 31;
  if ((size_t)a.M * a.ldx * 2 >= lim || (a.t && (size_t)a.M * a.ldt * 2 >= lim)) return false;
  if (a.epi == EPI_SWIGLU)   // one segment of F gate rows followed by F up rows
    return a.n_seg == 1 && a.seg[0].n % (bn / 2) == 0 &&
           (size_t)2 * a.seg[0].n * a.Kd * 2 < lim;
  for (int i = 0; i < a.n_seg; ++i)
    if ((size_t)a.seg[i].n * a.Kd * 2 >= lim) return false;
  if (a.n_seg > 1)
    for (int i = 0; i < a.n_seg; ++i)
      if (a.seg[i].n % bn) return false;
  return true;
}

enum BigCfg { CFG_L = 0, CFG_M = 1, CFG_S = 2 };
struct BigPlan {
  int cfg, m_tiles, n_tiles, splits;
  int n_full;          // tiles run whole; the rest are split `splits` ways
  double cost_us;
};
struct CfgInfo {
  int bm, bn, per_cu;   // tile, workgroups resident per CU
  double rate1, rate2;  // sustained bf16 TFLOP/s per CU with 1 / 2 of them resident
};
// Rates measured on MI355X for 1024-row passes of the Qwen3-8B shapes.
static const CfgInfo kCfgInfo[3] = {
    {256, 256, 1, 4.8, 4.8}, {256, 128, 2, 3.6, 4.5}, {128, 128, 2, 1.9, 3.6}};
constexpr double kL2BytesPerUs = 30e6;     // L2 -> CU operand traffic the chip sustains
constexpr double kPartBytesPerUs = 10e6;   // split-K partial tiles, written and read back (mostly in the 256 MB last-level cache)

// Pick the tile configuration and the K split from a cost model: rounds of
// resident workgroups times the time one workgroup's K range takes at the
// CU's sustained rate (bounded below by the L2 operand traffic), plus the
// split-K partial tiles and the reduction launch.
static BigPlan plan_big(const GemmArgs& a) {
  BigPlan best = {-1, 0, 0, 0, 0, 1e30};
  const int pair = a.epi == EPI_SWIGLU ? 2 : 1;
  const int nk = a.Kd / big::BK + (a.t ? pair * a.rank / big::BK : 0);
  // At most 128 rows the product is bound by streaming W (about 2*rows flop
  // per weight byte, below the chip's ridge): one row of 128x128 tiles, split
  // along K until about 256 workgroups stream W (measured best on the
  // 121-row token-tree verify shapes).
  if (a.M <= 128 && big_ok(a, 128)) {
    int n_tiles = 0;
    for (int i = 0; i < a.n_seg; ++i) n_tiles += (pair * a.seg[i].n + 127) / 128;
    int sp = std::max(1, std::min(16, 256 / n_tiles));
    while (sp > 1 && (a.Kd / big::BK / sp < 4 || !a.part ||
                      (size_t)n_tiles * sp * 128 * 128 > a.part_floats))
      --sp;
    return BigPlan{CFG_S, 1, n_tiles, sp, sp == 1 ? n_tiles : 0, 0.0};
  }
  for (int c = 0; c < 3; ++c) {
    const CfgInfo& ci = kCfgInfo[c];
    if (!big_ok(a, ci.bn)) continue;
    const int m_tiles = (a.M + ci.bm - 1) / ci.bm;
    int n_tiles = 0;
    for (int i = 0; i < a.n_seg; ++i) n_tiles += (pair * a.seg[i].n + ci.bn - 1) / ci.bn;
    const int tiles = m_tiles * n_tiles;
    const double slice_flop = 2.0 * ci.bm * ci.bn * big::BK;
    const double slice_bytes = (ci.bm + ci.bn) * big::BK * 2.0;
    const int slots_max = 256 * ci.per_cu;
    for (int sp = 1; sp <= 16; ++sp) {
      if (sp > 1 && a.Kd / big::BK / sp < 4) break;
      // whole rounds of tiles stay unsplit; the remainder is split
      const int n_full = sp == 1 ? tiles : (tiles / slots_max) * slots_max;
      const int rem = tiles - n_full;
      if (sp > 1 && rem == 0) break;
      const size_t part = (size_t)rem * sp * ci.bm * ci.bn;
      if (sp > 1 && (!a.part || part > a.part_floats)) break;
      const int items = n_full + rem * sp;
      const int occ = items > 256 && ci.per_cu > 1 ? 2 : 1;
      const int slots = 256 * occ;
      const double rate = (occ == 2 ? ci.rate2 : ci.rate1) / occ * 1e6;   // flop/us per WG
      const int k_rem = (nk + sp - 1) / sp;
      // rounds of whole tiles, then rounds of split items
      const int r_full = n_full / slots, left = n_full % slots;
      const int r_rem = (left + rem * sp + slots - 1) / slots;
      double cost = (r_full * nk + r_rem * (left ? nk : k_rem)) * slice_flop / rate;
      const double l2 = ((double)n_full * nk + (double)rem * sp * k_rem) * slice_bytes / kL2BytesPerUs;
      if (l2 > cost) cost = l2;
      cost += 2.0;
      if (sp > 1) cost += (double)part * 4 * 2 / kPartBytesPerUs + 3.0;
      if (cost < best.cost_us) best = BigPlan{c, m_tiles, n_tiles, sp, n_full, cost};
    }
  }
  return best;
}

// Split-K reduction of an EPI_SWIGLU product: one thread per float4 (four
// rows of one column) of a gate wave's partial tile; the matching float4 of
// its up partner sits WN/2 waves on.  Splits are summed in order, then
// bf16(silu(g) * u) is stored.
template <class C>
__global__ void __launch_bounds__(256)
k_gemm_splitk_reduce_swiglu(GemmArgs a, int m_tiles, int n_tiles, int splits, int n_full) {
  constexpr int Q = C::kTileFloats / 4, QH = Q / 2, HW = C::WN / 2;
  const int rem = m_tiles * n_tiles - n_full;
  const int g = blockIdx.x * 256 + threadIdx.x;
  if (g >= rem * QH) return;
  const int tr = g / QH;
  int r = g % QH;
  const int l = r & 63;
  r >>= 6;
  const int e4 = r & 3;
  r >>= 2;
  const int j = r % C::TJ;
  r /= C::TJ;
  const int i = r % C::TI;
  r /= C::TI;
  const int wg = r % HW, wm = r / HW;
  const int w = wm * C::WN + wg;
  const int q = (((w * C::TI + i) * C::TJ + j) * 4 + e4) * 64 + l;
  const int qu = ((((w + HW) * C::TI + i) * C::TJ + j) * 4 + e4) * 64 + l;
  const float4* src = reinterpret_cast<const float4*>(a.part);
  const float4 gs = sum_splits4(src + (size_t)tr * Q + q, (size_t)rem * Q, splits);
  const float4 us = sum_splits4(src + (size_t)tr * Q + qu, (size_t)rem * Q, splits);
  const int tile = n_full + tr;
  const int mt = tile % m_tiles, nt = tile / m_tiles;
  const int c = nt * (C::BN / 2) + wg * C::TN + j * 32 + (l & 31);
  const int mb = mt * C::BM + wm * C::TM + i * 32 + e4 * 8 + (l >> 5) * 4;
  const float gv[4] = {gs.x, gs.y, gs.z, gs.w}, uv[4] = {us.x, us.y, us.z, us.w};
  uint16_t* out = static_cast<uint16_t*>(a.out);
#pragma unroll
  for (int k = 0; k < 4; ++k)
    if (mb + k < a.M)
      out[(size_t)(mb + k) * a.ldo + c] = f32_to_bf16(gv[k] / (1.0f + __expf(-gv[k])) * uv[k]);
}

// Split-K reduction of a q|k|v product (every tile split) fused with RoPE and
// the K/V write: one thread per float4 (four rows of one column) of a partial
// tile; for q and k the thread holding channel i < hd/2 of a head also sums the
// float4 of channel i + hd/2 (same tile: segments and tiles hold whole heads).
template <class C>
__global__ void __launch_bounds__(256)
k_gemm_splitk_reduce_rope(GemmArgs a, int m_tiles, int n_tiles, int splits) {
  constexpr int Q = C::kTileFloats / 4;
  const int rem = m_tiles * n_tiles;
  const int g = blockIdx.x * 256 + threadIdx.x;
  if (g >= rem * Q) return;
  const int tr = g / Q, q = g % Q;
  const int mt = tr % m_tiles, nt = tr / m_tiles;
  const int l = q & 63;
  int r = q >> 6;
  const int e4 = r & 3;
  r >>= 2;
  const int j = r % C::TJ;
  r /= C::TJ;
  const int i = r % C::TI, w = r / C::TI;
  const int wm = w / C::WN, wn = w % C::WN;
  const SegView sv = pick_segment(a, nt * (C::BN / 16));
  const int nn = wn * C::TN + j * 32 + (l & 31);        // column in the tile
  const int nl = sv.n0 + nn;
  if (nl >= sv.n) return;
  const RopeArgs& ra = a.rope;
  const int col = sv.col_base + nl, hd = ra.hd, half = hd / 2;
  const int head = col / hd, ch = col % hd;
  const bool rot = head < ra.Hq + ra.Hkv;
  if (rot && ch >= half) return;                       // stored by its partner
  const float4* src = reinterpret_cast<const float4*>(a.part);
  auto sum_at = [&](int qi) { return sum_splits4(src + (size_t)tr * Q + qi, (size_t)rem * Q, splits); };
  const float4 x = sum_at(q);
  float4 xp = x;
  if (rot) {
    const int np = nn + half;
    const int wp = wm * C::WN + np / C::TN, jp = (np % C::TN) / 32;
    xp = sum_at((((wp * C::TI + i) * C::TJ + jp) * 4 + e4) * 64 + l);
  }
  const int mb = mt * C::BM + wm * C::TM + i * 32 + e4 * 8 + (l >> 5) * 4;
  const float xv[4] = {x.x, x.y, x.z, x.w}, pv[4] = {xp.x, xp.y, xp.z, xp.w};
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    const int m = mb + c;
    if (m >= a.M) break;
    int slot;
    const int page = rope_page(ra, m, &slot);
    if (rot) rope_store_pair(ra, m, head, ch, xv[c], pv[c], page, slot);
    else rope_store_v(ra, head - ra.Hq - ra.Hkv, ch, xv[c], page, slot);
  }
}

// Row maxima (max_part) of the split tiles n_full, n_full + 1, ... from their
// stored rows, after the split-K reduction: one wave per row of a tile.
template <class C>
__global__ void __launch_bounds__(256)
k_tile_row_max(GemmArgs a, int m_tiles, int n_full) {
  constexpr int WGS = C::BM / 4;                 // workgroups per tile
  const int tr = blockIdx.x / WGS;
  const int row = (blockIdx.x % WGS) * 4 + (threadIdx.x >> 6);
  const int tile = n_full + tr;
  const int mt = tile % m_tiles, nt = tile / m_tiles;
  const int m = mt * C::BM + row;
  if (m >= a.M) return;
  const SegView sv = pick_segment(a, nt * (C::BN / 16));
  const int n1 = sv.n0 + C::BN < sv.n ? sv.n0 + C::BN : sv.n;
  const float* y = static_cast<const float*>(a.out) + (size_t)m * a.ldo + sv.col_base;
  float mx = -INFINITY;
  for (int c = sv.n0 + (threadIdx.x & 63); c < n1; c += 64) mx = fmaxf(mx, y[c]);
  mx = wave_max(mx);
  if ((threadIdx.x & 63) == 0) a.max_part[(size_t)m * a.max_part_ld + nt] = mx;
}

template <class C>
static hipError_t launch_big_cfg(const GemmArgs& a, const BigPlan& p, hipStream_t s,
                                 bool* roped) {
  const int rem = p.m_tiles * p.n_tiles - p.n_full;
  hipLaunchKernelGGL(k_gemm_big<C>, dim3(p.n_full + rem * p.splits), dim3(C::kThreads), C::kLds,
                     s, a, p.m_tiles, p.n_tiles, p.splits, p.n_full);
  if (a.rope_fuse && p.splits > 1 && p.n_full == 0) {
    if (roped) *roped = true;
    const int n = rem * (C::kTileFloats / 4);
    hipLaunchKernelGGL(k_gemm_splitk_reduce_rope<C>, dim3((n + 255) / 256), dim3(256), 0, s, a,
                       p.m_tiles, p.n_tiles, p.splits);
    return hipGetLastError();
  }
  if (p.splits > 1 && a.epi == EPI_SWIGLU) {
    const int n = rem * (C::kTileFloats / 8);
    hipLaunchKernelGGL(k_gemm_splitk_reduce_swiglu<C>, dim3((n + 255) / 256), dim3(256), 0, s, a,
                       p.m_tiles, p.n_tiles, p.splits, p.n_full);
  } else if (p.splits > 1) {
    const int n = rem * (C::kTileFloats / 4);
    hipLaunchKernelGGL(k_gemm_splitk_reduce<C>, dim3((n + 255) / 256), dim3(256), 0, s, a,
                       p.m_tiles, p.n_tiles, p.splits, p.n_full);
    if (a.max_part && a.epi == EPI_STORE_F32)
      hipLaunchKernelGGL(k_tile_row_max<C>, dim3(rem * (C::BM / 4)), dim3(256), 0, s, a,
                         p.m_tiles, p.n_full);
  }
  return hipGetLastError();
}

static hipError_t launch_big(const GemmArgs& a, const BigPlan& p, hipStream_t s, bool* roped) {
  switch (p.cfg) {
    case CFG_L: return launch_big_cfg<big::CfgL>(a, p, s, roped);
    case CFG_M: return launch_big_cfg<big::CfgM>(a, p, s, roped);
    default: return launch_big_cfg<big::CfgS>(a, p, s, roped);
  }
}

// The tiled kernel for more than 64 rows (one 128-row tile streams W once);
// decode-sized row counts keep the skinny kernel, which streams W once with
// the rows held in registers (past 64 rows it would stream W once per 64).
bool gemm_swiglu_ok(const GemmArgs& a) {
  return a.epi == EPI_SWIGLU && a.M > 64 && plan_big(a).cfg >= 0;
}

// Tile-packed copy of a row-major bf16 matrix [N, K] (N % 16 == 0, K % 32 ==
// 0): one thread per 16 bytes of the output, 8 values of one row.
__global__ void __launch_bounds__(256)
k_pack_tiles(const uint16_t* __restrict__ src, uint16_t* __restrict__ dst, int N, int K) {
  const size_t o = (size_t)blockIdx.x * 256 + threadIdx.x;       // 16-byte unit
  const size_t n_units = (size_t)N * K / 8;
  if (o >= n_units) return;
  const int lane = (int)(o & 63);
  const size_t blk = o >> 6;
  const int ks = (int)(blk % (size_t)(K >> 5));
  const size_t nt = blk / (size_t)(K >> 5);
  const size_t row = nt * 16 + (lane & 15);
  const int k0 = ks * 32 + (lane >> 4) * 8;
  *reinterpret_cast<uint4*>(dst + o * 8) = *reinterpret_cast<const uint4*>(src + row * K + k0);
}

hipError_t launch_pack_tiles(const uint16_t* src, uint16_t* dst, int N, int K, hipStream_t s) {
  const size_t n_units = (size_t)N * K / 8;
  hipLaunchKernelGGL(k_pack_tiles, dim3((unsigned)((n_units + 255) / 256)), dim3(256), 0, s, src,
                     dst, N, K);
  return hipGetLastError();
}

int gemm_row_max_parts(const GemmArgs& a) {
  if (a.M > 64) {
    const BigPlan p = plan_big(a);
    if (p.cfg >= 0) return p.n_tiles;
  }
  return plan_skinny(a).gx;
}

// One workgroup per row: the maximum of its column-group partials.
__global__ void __launch_bounds__(256)
k_row_max(const float* __restrict__ part, int ld, int n_parts, float* __restrict__ out) {
  __shared__ float red[4];
  const int r = blockIdx.x;
  float mx = -INFINITY;
  for (int i = threadIdx.x; i < n_parts; i += 256) mx = fmaxf(mx, part[(size_t)r * ld + i]);
  mx = wave_max(mx);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = mx;
  __syncthreads();
  if (threadIdx.x == 0) out[r] = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
}

hipError_t launch_row_max(const float* max_part, int ld, int n_parts, int R, float* row_max,
                          hipStream_t s) {
  hipLaunchKernelGGL(k_row_max, dim3(R), dim3(256), 0, s, max_part, ld, n_parts, row_max);
  return hipGetLastError();
}

hipError_t launch_gemm(const GemmArgs& a, hipStream_t s, bool* normed, bool* roped,
                       bool* swiglued) {
  if (normed) *normed = false;
  if (roped) *roped = false;
  if (swiglued) *swiglued = false;
  if (a.epi == EPI_SWIGLU && !gemm_swiglu_ok(a)) return hipErrorInvalidValue;
  if (a.M > 64) {
    const BigPlan p = plan_big(a);
    if (p.cfg >= 0) return launch_big(a, p, s, roped);
  }
  return launch_gemm_skinny(a, s, normed, roped, swiglued);
}

}  // namespace uno
