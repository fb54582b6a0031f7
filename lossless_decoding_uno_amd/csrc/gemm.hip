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

hipError_t launch_gemm_skinny(const GemmArgs& a, hipStream_t s) {
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


// ============================================================================
// Tiled kernel (many rows: batched decode blocks, prompt chunks).
// Workgroup tile 256 x 128 (rows of X x columns of W), 4 waves in a 2 x 2
// grid, each wave 128 x 64 = 4 x 2 tiles of v_mfma_f32_32x32x16_bf16.  Both
// operands stream through LDS in 64-wide K slices by direct global -> LDS DMA
// (global_load_lds_dwordx4, no staging registers), three slices resident, so
// two slices are in flight while the MFMAs of the third run.  LDS rows are 128
// bytes (8 chunks of 16 bytes) with the chunk index XOR-swizzled by the row,
// applied by choosing which source chunk each DMA lane copies.  The LoRA
// product runs as r/64 extra K slices with T and B as operands.  Tiles are
// ordered so that the workgroups sharing one W tile run on the same XCD (same
// L2).  Split-K (grid.z) accumulates with fp32 atomics into the residual
// stream.
// ============================================================================
namespace big {
constexpr int BM = 256, BN = 128, BK = 64;
constexpr int kThreads = 256;
constexpr int kLdsA = BM * BK * 2;      // bytes per stage
constexpr int kLdsB = BN * BK * 2;
constexpr int kStage = kLdsA + kLdsB;
constexpr int kStages = 3;
constexpr int kInstr = kStage / 1024;   // 1 KB DMA instructions per slice
constexpr int kIW = kInstr / 4;         // per wave
constexpr int kInstrA = kLdsA / 1024;

__device__ __forceinline__ int swz(int row, int chunk) { return (row * 8 + (chunk ^ (row & 7))) * 16; }
}  // namespace big

__global__ void __launch_bounds__(big::kThreads)
k_gemm_tiled(GemmArgs a, int m_tiles, int n_tiles, int splits) {
  using namespace big;
  extern __shared__ __attribute__((aligned(16))) unsigned char lds[];
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63;
  const int wm = w >> 1, wn = w & 1;

  // XCD-aware order: linear id -> (xcd, slot); tiles of one N column stay together
  const int nwg = m_tiles * n_tiles;
  const int id = blockIdx.x;
  const int per_xcd = (nwg + 7) / 8;
  int lin = (id % 8) * per_xcd + id / 8;
  if (nwg % 8 != 0) lin = id;             // keep it simple when the grid is ragged
  const int mt = lin % m_tiles, nt = lin / m_tiles;
  if (nt >= n_tiles) return;
  const int m0 = mt * BM;
  const SegView sv = pick_segment(a, nt * (BN / 16));
  const int n0 = sv.n0;

  // K slices of this split
  const int nk_base = a.Kd / BK;
  const int nk_lora = (a.t && sv.lb) ? a.rank / BK : 0;
  const int z = blockIdx.z;
  const int kb0 = nk_base * z / splits, kb1 = nk_base * (z + 1) / splits;
  const int nk = (kb1 - kb0) + (z == splits - 1 ? nk_lora : 0);

  // DMA lanes: instruction ins copies 8 rows (A rows 0..255, then B rows 0..127);
  // lane l takes row 8*ins' + l/8 and writes physical chunk l%8, which holds
  // logical chunk (l%8) ^ (row%8).  Row pointers exclude the K offset.
  const uint16_t* pbase[kIW];
  const uint16_t* plora[kIW];
#pragma unroll
  for (int ii = 0; ii < kIW; ++ii) {
    const int ins = w * kIW + ii;
    const bool is_a = ins < kInstrA;
    const int row = (is_a ? ins : ins - kInstrA) * 8 + l / 8;
    const int ch = (l % 8) ^ (row & 7);
    if (is_a) {
      const int m = m0 + row < a.M ? m0 + row : 0;   // rows past M: any valid row (discarded)
      pbase[ii] = a.x + (size_t)m * a.ldx + ch * 8;
      plora[ii] = a.t ? a.t + (size_t)m * a.ldt + sv.t_col + ch * 8 : a.x;
    } else {
      pbase[ii] = sv.w + (size_t)(n0 + row) * a.Kd + ch * 8;
      plora[ii] = sv.lb ? sv.lb + (size_t)(n0 + row) * a.rank + ch * 8 : sv.w;
    }
  }
  const uint32_t lds_base = lds_addr(lds) + w * kIW * 1024;
  auto issue = [&](int s) {
    const int kk = kb0 + s;
    const bool lora = kk >= kb1;
    const int koff = (lora ? kk - kb1 : kk) * BK;
    const uint32_t stage = __builtin_amdgcn_readfirstlane(lds_base + (s % kStages) * kStage);
#pragma unroll
    for (int ii = 0; ii < kIW; ++ii)
      lds_dma16((lora ? plora[ii] : pbase[ii]) + koff, stage + ii * 1024);
  };

  f32x16 acc[4][2];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;

#pragma unroll
  for (int s = 0; s < kStages - 1; ++s)
    if (s < nk) issue(s);
  for (int s = 0; s < nk; ++s) {
    if (s + 1 < nk) wait_vmcnt<kIW>();        // slice s landed (s+1 may be in flight)
    else wait_vmcnt<0>();
    __syncthreads();
    if (s + kStages - 1 < nk) issue(s + kStages - 1);   // into the stage read at s-1
    const unsigned char* A = lds + (s % kStages) * kStage;
    const unsigned char* B = A + kLdsA;
#pragma unroll
    for (int kk = 0; kk < BK / 16; ++kk) {
      const int ch = 2 * kk + (l >> 5);
      Frag fa[4], fb[2];
#pragma unroll
      for (int i = 0; i < 4; ++i)
        fa[i].u = *reinterpret_cast<const uint4*>(A + swz(wm * 128 + i * 32 + (l & 31), ch));
#pragma unroll
      for (int j = 0; j < 2; ++j)
        fb[j].u = *reinterpret_cast<const uint4*>(B + swz(wn * 64 + j * 32 + (l & 31), ch));
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[i].v, fb[j].v, acc[i][j], 0, 0, 0);
    }
  }

  // epilogue: lane holds rows (e/4)*8 + (l/32)*4 + e%4, column l%32 of each 32x32 tile
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int m = m0 + wm * 128 + i * 32 + (e >> 2) * 8 + (l >> 5) * 4 + (e & 3);
        if (m >= a.M) continue;
        const int n = sv.col_base + n0 + wn * 64 + j * 32 + (l & 31);
        const size_t o = (size_t)m * a.ldo + n;
        const float v = acc[i][j][e];
        switch (a.epi) {
          case EPI_STORE_F32: static_cast<float*>(a.out)[o] = v; break;
          case EPI_ADD_F32:
            if (splits > 1) atomicAdd(static_cast<float*>(a.out) + o, v);
            else static_cast<float*>(a.out)[o] += v;
            break;
          case EPI_STORE_BF16: static_cast<uint16_t*>(a.out)[o] = f32_to_bf16(v); break;
          default: {
            const float g = (m % a.rows_per_seq) != 0 ? a.scale : 0.f;
            static_cast<uint16_t*>(a.out)[o] = f32_to_bf16(g * v);
          }
        }
      }
}

static bool tiled_ok(const GemmArgs& a) {
  if (a.M < 128 || a.Kd % big::BK) return false;
  for (int i = 0; i < a.n_seg; ++i)
    if (a.seg[i].n % big::BN) return false;
  if (a.t && a.rank % big::BK) return false;
  return true;
}

hipError_t launch_gemm_tiled(const GemmArgs& a, hipStream_t s) {
  int n_tiles = 0;
  for (int i = 0; i < a.n_seg; ++i) n_tiles += a.seg[i].n / big::BN;
  const int m_tiles = (a.M + big::BM - 1) / big::BM;
  int splits = 1;
  if (a.epi == EPI_ADD_F32) {
    const int wgs = m_tiles * n_tiles;
    while (wgs * splits < 256 && splits < 4 && (a.Kd / big::BK) / (splits * 2) >= 8) splits *= 2;
  }
  const size_t lds = (size_t)big::kStages * big::kStage;
  hipLaunchKernelGGL(k_gemm_tiled, dim3(m_tiles * n_tiles, 1, splits), dim3(big::kThreads), lds,
                     s, a, m_tiles, n_tiles, splits);
  return hipGetLastError();
}

// Tiled kernel when the output has enough 256 x 128 tiles to spread over the
// chip; narrow outputs (the LoRA A products, N = r..3r) keep the skinny kernel,
// whose 8-wave K split gives them enough workgroups.
hipError_t launch_gemm(const GemmArgs& a, hipStream_t s) {
  if (tiled_ok(a)) {
    int n_tiles = 0;
    for (int i = 0; i < a.n_seg; ++i) n_tiles += a.seg[i].n / big::BN;
    const int m_tiles = (a.M + big::BM - 1) / big::BM;
    if (m_tiles * n_tiles >= 64) return launch_gemm_tiled(a, s);
  }
  return launch_gemm_skinny(a, s);
}

}  // namespace uno
