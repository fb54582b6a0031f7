// Small per-row kernels of the draft / verify passes for gfx950: block
// assembly + embedding gather, RMSNorm, the rotary table, RoPE + paged KV
// write, SiLU * up, and the KV commit.
//
// Block assembly follows the draft/verify layout of the step ("Unlocking
// Lossless Speedups in LLMs via Discrete Diffusion", paperglide reader, "The
// Psi-Speculative Sampler"): a draft block is the anchor followed by mask
// tokens; a verify block is the drafted tokens.  The KV commit keeps the anchor
// and the kept drafts of the one shared cache (picx.dev summary, "Practical
// Implications").
#include "uno_device.h"
#include "uno_internal.h"
#include "rope_store.h"

namespace uno {

// ------------------------------------------------------------ embedding
// One workgroup per row r = b*K + j.  Draft mode (anchor != null): id =
// anchor[b] for j == 0; the rows j >= 1 are the prior's noise -- mask_id
// (noise_prior 0) or a uniform token floor(w * V / 2^64), w = Philox word 0 at
// counter (3, j, b, step[b]) under key (seed, 0) (noise_prior 1) -- or, in a
// later draft pass (block != null), the corrector's output: block[b*K + j-1]
// kept iff keep_q24 >= 2^24 or the uniform of counter (64 + corr_pass, j, b,
// step[b]) is below keep_q24, else returned to the prior (mask_id, or a fresh
// uniform token from counter (128 + corr_pass, j, b, step[b])).  Verify mode:
// id = rows[r].
__global__ void __launch_bounds__(256)
k_embed(const uint16_t* __restrict__ embed, const int32_t* __restrict__ anchor,
        const int32_t* __restrict__ block, const int32_t* __restrict__ rows, int K, int D, int V,
        int mask_id, int noise_prior,
        uint64_t seed, const uint64_t* __restrict__ step, uint32_t keep_q24, int corr_pass,
        float* __restrict__ h, int32_t* __restrict__ status) {
  const int r = blockIdx.x;
  const int b = r / K, j = r % K;
  const uint64_t st = step ? step[b] : 0;
  int id;
  if (!anchor) {
    id = rows[r];
  } else if (j == 0) {
    id = anchor[b];
  } else {
    bool noise = true;
    uint64_t noise_slot = 3;
    if (block) {
      noise = keep_q24 < (1u << 24) &&
              (uint32_t)(philox_word0(64 + corr_pass, j, b, st, seed, 0) >> 40) >= keep_q24;
      noise_slot = 128 + corr_pass;
    }
    if (!noise) id = block[b * K + j - 1];
    else if (noise_prior == 0) id = mask_id;
    else id = (int)__umul64hi(philox_word0(noise_slot, j, b, st, seed, 0), (uint64_t)V);
  }
  const bool bad = id < 0 || id >= V;
  if (bad) {
    if (threadIdx.x == 0 && status) atomicOr(status + b, UNO_DEV_BAD_TOKEN);
    id = 0;
  }
  const uint16_t* src = embed + (size_t)id * D;
  float* dst = h + (size_t)r * D;
  for (int i = threadIdx.x * 8; i < D; i += 256 * 8) {
    const uint4 u = *reinterpret_cast<const uint4*>(src + i);
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
    float4 lo, hi;
    lo.x = bad ? 0.f : __uint_as_float(w[0] << 16); lo.y = bad ? 0.f : __uint_as_float(w[0] & 0xFFFF0000u);
    lo.z = bad ? 0.f : __uint_as_float(w[1] << 16); lo.w = bad ? 0.f : __uint_as_float(w[1] & 0xFFFF0000u);
    hi.x = bad ? 0.f : __uint_as_float(w[2] << 16); hi.y = bad ? 0.f : __uint_as_float(w[2] & 0xFFFF0000u);
    hi.z = bad ? 0.f : __uint_as_float(w[3] << 16); hi.w = bad ? 0.f : __uint_as_float(w[3] & 0xFFFF0000u);
    *reinterpret_cast<float4*>(dst + i) = lo;
    *reinterpret_cast<float4*>(dst + i + 4) = hi;
  }
}

hipError_t launch_embed(const uno_config& c, const bf16_raw_t* embed, const int32_t* anchor,
                        const int32_t* block, const int32_t* rows, int B, int K, uint64_t seed,
                        const uint64_t* step, uint32_t keep_q24, int corr_pass, float* h,
                        int32_t* status, hipStream_t s) {
  hipLaunchKernelGGL(k_embed, dim3(B * K), dim3(256), 0, s, embed, anchor, block, rows, K,
                     c.d_model, c.vocab, c.mask_id, c.noise_prior, seed, step, keep_q24, corr_pass,
                     h, status);
  return hipGetLastError();
}

// ------------------------------------------------------------ RMSNorm
// out = bf16(h / sqrt(mean(h^2) + eps) * gain); one workgroup per row, the sum
// of squares reduced in a fixed order (run-to-run identical).
__global__ void __launch_bounds__(256)
k_rmsnorm(const float* __restrict__ h, const float* __restrict__ gain, int D, float eps,
          uint16_t* __restrict__ out) {
  // the first kRegs float4 of each thread stay in registers between the two
  // passes, their loads (and the gains') issued together
  constexpr int kRegs = 8;
  __shared__ float red[4];
  const int r = blockIdx.x;
  const float* x = h + (size_t)r * D;
  float4 xv[kRegs], gv[kRegs];
#pragma unroll
  for (int k = 0; k < kRegs; ++k) {
    const int i = threadIdx.x * 4 + k * 256 * 4;
    if (i < D) {
      xv[k] = *reinterpret_cast<const float4*>(x + i);
      gv[k] = *reinterpret_cast<const float4*>(gain + i);
    }
  }
  float ss = 0.f;
#pragma unroll
  for (int k = 0; k < kRegs; ++k) {
    const int i = threadIdx.x * 4 + k * 256 * 4;
    if (i < D) ss += xv[k].x * xv[k].x + xv[k].y * xv[k].y + xv[k].z * xv[k].z + xv[k].w * xv[k].w;
  }
  for (int i = threadIdx.x * 4 + kRegs * 256 * 4; i < D; i += 256 * 4) {
    const float4 v = *reinterpret_cast<const float4*>(x + i);
    ss += v.x * v.x + v.y * v.y + v.z * v.z + v.w * v.w;
  }
  ss = wave_sum(ss);
  if (lane_id() == 0) red[threadIdx.x / UNO_WAVE] = ss;
  __syncthreads();
  const float tot = (red[0] + red[1]) + (red[2] + red[3]);
  const float inv = 1.0f / sqrtf(tot / (float)D + eps);
  uint16_t* o = out + (size_t)r * D;
  auto put = [&](int i, float4 v, float4 g) {
    uint2 pk;
    pk.x = pack_bf16x2(v.x * inv * g.x, v.y * inv * g.y);
    pk.y = pack_bf16x2(v.z * inv * g.z, v.w * inv * g.w);
    *reinterpret_cast<uint2*>(o + i) = pk;
  };
#pragma unroll
  for (int k = 0; k < kRegs; ++k) {
    const int i = threadIdx.x * 4 + k * 256 * 4;
    if (i < D) put(i, xv[k], gv[k]);
  }
  for (int i = threadIdx.x * 4 + kRegs * 256 * 4; i < D; i += 256 * 4)
    put(i, *reinterpret_cast<const float4*>(x + i), *reinterpret_cast<const float4*>(gain + i));
}

hipError_t launch_rmsnorm(const float* h, const float* gain, int R, int D, float eps,
                          bf16_raw_t* out, hipStream_t s) {
  hipLaunchKernelGGL(k_rmsnorm, dim3(R), dim3(256), 0, s, h, gain, D, eps, out);
  return hipGetLastError();
}

// ------------------------------------------------------------ rotary table
// cs[r, i] = (cos, sin)(pos_r * theta^(-2i/hd)), angle in fp64 so that large
// positions keep full fp32 accuracy.  pos_r = kv_len + pos_offset + j, or
// + depth[r] for a token tree's rows (their slot stays kv_len + pos_offset + j).
__global__ void k_rope_table(const int32_t* __restrict__ kv_len, int K, int pos_offset, int half,
                             double log_theta, const int32_t* __restrict__ depth,
                             float2* __restrict__ cs, const int32_t* __restrict__ page_table,
                             int max_pages, int64_t n_pages, int ps, int2* __restrict__ row_page,
                             int32_t* __restrict__ status, unsigned* __restrict__ zero,
                             int n_zero) {
  const int r = blockIdx.x;
  for (int i = r * blockDim.x + threadIdx.x; i < n_zero; i += gridDim.x * blockDim.x) zero[i] = 0u;
  const int b = r / K, j = r % K;
  const double pos = (double)(kv_len[b] + pos_offset + (depth ? depth[r] : j));
  for (int i = threadIdx.x; i < half; i += blockDim.x) {
    const double inv_freq = exp(-log_theta * (2.0 * i) / (2.0 * half));
    double sn, cn;
    sincos(pos * inv_freq, &sn, &cn);
    cs[(size_t)r * half + i] = make_float2((float)cn, (float)sn);
  }
  // the row's K/V slot (kv_len + pos_offset + j) and its page, for every layer
  if (threadIdx.x == 0) {
    const int slot_pos = kv_len[b] + pos_offset + j;
    const int pidx = slot_pos / ps;
    int page = -1;
    if (slot_pos >= 0 && pidx < max_pages) {
      page = page_table[(size_t)b * max_pages + pidx];
      if (page < 0 || page >= n_pages) {
        if (status) atomicOr(status + b, UNO_DEV_BAD_PAGE);
        page = -1;
      }
    } else if (status) {
      atomicOr(status + b, UNO_DEV_CAPACITY);
    }
    row_page[r] = make_int2(page, slot_pos % ps);
  }
}

hipError_t launch_rope_table(const uno_config& c, const uno_kv& kv, int B, int K, int pos_offset,
                             const int32_t* depth, float2* cs, int2* row_page, int32_t* status,
                             unsigned* zero, int n_zero, hipStream_t s) {
  hipLaunchKernelGGL(k_rope_table, dim3(B * K), dim3(64), 0, s, kv.kv_len, K, pos_offset,
                     c.head_dim / 2, log((double)c.rope_theta), depth, cs, kv.page_table,
                     kv.max_pages_per_seq, kv.n_pages, c.page_size, row_page, status, zero,
                     n_zero);
  return hipGetLastError();
}

// ------------------------------------------------------------ RoPE + KV write
// qkv row layout: [q heads | k heads | v heads], each head hd wide, fp32.
// q (rotated, times log2(e)/sqrt(hd)) -> hi + lo bf16 [R, Hq*hd];
// k (rotated) -> K page [slot][hd]; v -> V page transposed [hd][slot]
// (rope_store.h).  A row's work is spread over gridDim.y workgroups (short
// passes have few rows).
__global__ void __launch_bounds__(256)
k_rope_kv_write(const float* __restrict__ qkv, RopeArgs ra) {
  const int r = blockIdx.x;
  const int half = ra.hd / 2;
  const int width = (ra.Hq + 2 * ra.Hkv) * ra.hd;
  const float* row = qkv + (size_t)r * width;
  int slot;
  const int page = rope_page(ra, r, &slot);
  const int t0 = blockIdx.y * blockDim.x + threadIdx.x, tstep = blockDim.x * gridDim.y;
  const int n_pairs = (ra.Hq + ra.Hkv) * half;
  for (int t = t0; t < n_pairs; t += tstep) {
    const int head = t / half, i = t % half;
    rope_store_pair(ra, r, head, i, row[head * ra.hd + i], row[head * ra.hd + i + half], page,
                    slot);
  }
  if (page >= 0)
    for (int t = t0; t < ra.Hkv * ra.hd; t += tstep)
      rope_store_v(ra, t / ra.hd, t % ra.hd, row[(ra.Hq + ra.Hkv) * ra.hd + t], page, slot);
}

RopeArgs make_rope_args(const uno_config& c, const float2* cs, const int2* row_page,
                        const uno_kv& kv, int layer, int K, bf16_raw_t* q_out, bf16_raw_t* q_lo) {
  const size_t layer_elems = (size_t)kv.n_pages * c.n_kv_heads * c.page_size * c.head_dim;
  RopeArgs ra;
  ra.cs = cs;
  ra.row_page = row_page;
  ra.K = K; ra.Hq = c.n_q_heads; ra.Hkv = c.n_kv_heads; ra.hd = c.head_dim; ra.ps = c.page_size;
  ra.k_layer = static_cast<uint16_t*>(kv.k_pages) + (size_t)layer * layer_elems;
  ra.v_layer = static_cast<uint16_t*>(kv.v_pages) + (size_t)layer * layer_elems;
  ra.q_out = q_out; ra.q_lo = q_lo;
  return ra;
}

hipError_t launch_rope_kv_write(const float* qkv, const RopeArgs& ra, int R, hipStream_t s) {
  const int split = R >= 256 ? 1 : R >= 64 ? 2 : 4;
  hipLaunchKernelGGL(k_rope_kv_write, dim3(R, split), dim3(256), 0, s, qkv, ra);
  return hipGetLastError();
}

// ------------------------------------------------------------ SiLU * up
__global__ void __launch_bounds__(256)
k_silu_mul(const float* __restrict__ gu, int F, uint16_t* __restrict__ act) {
  const int r = blockIdx.y;
  const int i = (blockIdx.x * 256 + threadIdx.x) * 4;
  if (i >= F) return;
  const float* g = gu + (size_t)r * 2 * F;
  const float4 gv = *reinterpret_cast<const float4*>(g + i);
  const float4 uv = *reinterpret_cast<const float4*>(g + F + i);
  const float a0 = gv.x / (1.0f + __expf(-gv.x)) * uv.x;
  const float a1 = gv.y / (1.0f + __expf(-gv.y)) * uv.y;
  const float a2 = gv.z / (1.0f + __expf(-gv.z)) * uv.z;
  const float a3 = gv.w / (1.0f + __expf(-gv.w)) * uv.w;
  uint2 pk;
  pk.x = pack_bf16x2(a0, a1);
  pk.y = pack_bf16x2(a2, a3);
  *reinterpret_cast<uint2*>(act + (size_t)r * F + i) = pk;
}

hipError_t launch_silu_mul(const float* gu, int R, int F, bf16_raw_t* act, hipStream_t s) {
  hipLaunchKernelGGL(k_silu_mul, dim3((F / 4 + 255) / 256, R), dim3(256), 0, s, gu, F, act);
  return hipGetLastError();
}

// ------------------------------------------------------------ KV commit
// kv_len[b] += 1 + a (anchor + kept drafts); later slots become scratch.
__global__ void k_kv_commit(int32_t* __restrict__ kv_len, const int32_t* __restrict__ accept_len,
                            int B, int K, uint64_t* __restrict__ step,
                            int32_t* __restrict__ status) {
  const int b = blockIdx.x * blockDim.x + threadIdx.x;
  if (b >= B) return;
  const int a = accept_len[b];
  if (a < 0 || a > K) {
    if (status) atomicOr(status + b, UNO_DEV_BAD_ACCEPT);
    return;
  }
  kv_len[b] += 1 + a;
  if (step) step[b] += 1;
}

hipError_t launch_kv_commit(int32_t* kv_len, const int32_t* accept_len, int B, int K,
                            uint64_t* step, int32_t* status, hipStream_t s) {
  hipLaunchKernelGGL(k_kv_commit, dim3((B + 255) / 256), dim3(256), 0, s, kv_len, accept_len, B,
                     K, step, status);
  return hipGetLastError();
}

}  // namespace uno
