// bf16 MFMA GEMMs of the draft / verify passes for gfx950, with the LoRA
// low-rank path fused as extra K-iterations:
//   Y = X W^T + T B^T,  T = scale * gate(row) * (X A^T)
// ("Unlocking Lossless Speedups in LLMs via Discrete Diffusion": the diffusion
// weights are rank-r LoRA factors with scale alpha/r on every linear, active for
// the noisy positions of a drafted block and off for its first position and for
// verification; picx.dev summary, "Architecture"; paperglide reader, "Sampler
// Extensions").
//
// Skinny kernel (decode rows, M <= 64 per workgroup): one workgroup owns a
// 16-column tile of W and 16..64 rows of X; its 8 waves split the K dimension
// (wave w takes the 32-wide K steps w, w+8, ...), so every weight byte is read
// from HBM once per tile and the 8 waves' loads cover 512 contiguous bytes of
// each of the 16 weight rows at a time.  Each wave issues
// v_mfma_f32_16x16x32_bf16 (A = 16 rows of X, B = 16 columns of W^T); the eight
// partial 16x16 tiles are summed in LDS in a fixed order (run-to-run identical)
// and the epilogue stores, accumulates into the fp32 residual stream, or forms
// the gated, scaled LoRA input T.
#include "uno_device.h"
#include "uno_internal.h"

namespace uno {

union Frag {
  uint4 u;
  bf16x8 v;
};

__device__ __forceinline__ uint4 ldg16(const uint16_t* p) {
  return *reinterpret_cast<const uint4*>(p);
}

struct SegView {
  const uint16_t* w;
  const uint16_t* lb;
  int t_col;
  int col_base;
  int n0;
};

__device__ __forceinline__ SegView pick_segment(const GemmArgs& a, int tile) {
  SegView v;
  int base = 0;
  int t0 = a.seg[0].n >> 4, t1 = a.seg[1].n >> 4;
  if (a.n_seg == 1 || tile < t0) {
    v.w = a.seg[0].w; v.lb = a.seg[0].lora_b; v.t_col = a.seg[0].t_col; v.n0 = tile * 16;
  } else if (a.n_seg == 2 || tile < t0 + t1) {
    base = a.seg[0].n;
    v.w = a.seg[1].w; v.lb = a.seg[1].lora_b; v.t_col = a.seg[1].t_col; v.n0 = (tile - t0) * 16;
  } else {
    base = a.seg[0].n + a.seg[1].n;
    v.w = a.seg[2].w; v.lb = a.seg[2].lora_b; v.t_col = a.seg[2].t_col;
    v.n0 = (tile - t0 - t1) * 16;
  }
  v.col_base = base;
  return v;
}

constexpr int kSkWaves = 8;

template <int MT>
__global__ void __launch_bounds__(kSkWaves * 64)
k_gemm_skinny(GemmArgs a) {
  __shared__ f32x4 red[kSkWaves * MT * 64];
  const int w = threadIdx.x >> 6, l = threadIdx.x & 63;
  const int rr = l & 15, kg = l >> 4;
  const SegView sv = pick_segment(a, blockIdx.x);
  const int m0 = blockIdx.y * MT * 16;

  const uint16_t* wrow = sv.w + (size_t)(sv.n0 + rr) * a.Kd + kg * 8;
  const uint16_t* xrow[MT];
  bool xok[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    const int m = m0 + mt * 16 + rr;
    xok[mt] = m < a.M;
    xrow[mt] = a.x + (size_t)(xok[mt] ? m : 0) * a.ldx + kg * 8;
  }
  f32x4 acc[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) acc[mt] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int n_steps = a.Kd >> 5;
  int s = w;
  // main loop, 4 K-steps in flight per wave
  for (; s + 3 * kSkWaves < n_steps; s += 4 * kSkWaves) {
    Frag bw[4];
    Frag ax[4][MT];
#pragma unroll
    for (int u = 0; u < 4; ++u) bw[u].u = ldg16(wrow + (s + u * kSkWaves) * 32);
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
        ax[u][mt].u = xok[mt] ? ldg16(xrow[mt] + (s + u * kSkWaves) * 32) : make_uint4(0, 0, 0, 0);
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
        acc[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ax[u][mt].v, bw[u].v, acc[mt], 0, 0, 0);
  }
  for (; s < n_steps; s += kSkWaves) {
    Frag bw, ax;
    bw.u = ldg16(wrow + s * 32);
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      ax.u = xok[mt] ? ldg16(xrow[mt] + s * 32) : make_uint4(0, 0, 0, 0);
      acc[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ax.v, bw.v, acc[mt], 0, 0, 0);
    }
  }
  // fused LoRA: T [M, r] (already gated and scaled) times B [n, r]^T
  if (a.t && sv.lb) {
    // rank 16 fills half of a 32-wide step: lanes past the rank feed zeros
    const int r_steps = (a.rank + 31) >> 5;
    const uint16_t* brow = sv.lb + (size_t)(sv.n0 + rr) * a.rank + kg * 8;
    for (int rs = w; rs < r_steps; rs += kSkWaves) {
      const bool kin = rs * 32 + kg * 8 < a.rank;
      Frag bw, ax;
      bw.u = kin ? ldg16(brow + rs * 32) : make_uint4(0, 0, 0, 0);
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        const int m = m0 + mt * 16 + rr;
        ax.u = (kin && m < a.M) ? ldg16(a.t + (size_t)m * a.ldt + sv.t_col + rs * 32 + kg * 8)
                                : make_uint4(0, 0, 0, 0);
        acc[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ax.v, bw.v, acc[mt], 0, 0, 0);
      }
    }
  }
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) red[(w * MT + mt) * 64 + l] = acc[mt];
  __syncthreads();
  const float* redf = reinterpret_cast<const float*>(red);
  for (int e = threadIdx.x; e < MT * 256; e += kSkWaves * 64) {
    const int mt = e >> 8, rem = e & 255, ln = rem >> 2, i = rem & 3;
    float v = 0.f;
#pragma unroll
    for (int ww = 0; ww < kSkWaves; ++ww) v += redf[((ww * MT + mt) * 64 + ln) * 4 + i];
    const int m = m0 + mt * 16 + 4 * (ln >> 4) + i;
    if (m >= a.M) continue;
    const int n = sv.col_base + sv.n0 + (ln & 15);
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
}

hipError_t launch_gemm(const GemmArgs& a, hipStream_t s) {
  int tiles = 0;
  for (int i = 0; i < a.n_seg; ++i) tiles += a.seg[i].n / 16;
  const dim3 block(kSkWaves * 64);
  if (a.M <= 16) {
    hipLaunchKernelGGL(k_gemm_skinny<1>, dim3(tiles, 1), block, 0, s, a);
  } else if (a.M <= 32) {
    hipLaunchKernelGGL(k_gemm_skinny<2>, dim3(tiles, 1), block, 0, s, a);
  } else {
    hipLaunchKernelGGL(k_gemm_skinny<4>, dim3(tiles, (a.M + 63) / 64), block, 0, s, a);
  }
  return hipGetLastError();
}

}  // namespace uno
