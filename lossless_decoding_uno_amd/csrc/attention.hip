// Block attention of the draft / verify rows over the shared paged KV cache
// for gfx950 ("Unlocking Lossless Speedups in LLMs via Discrete Diffusion":
// drafting and verification read one KV cache, picx.dev summary, "Practical
// Implications"; the first drafted position is computed like an AR step and the
// noisy positions attend to the whole block, paperglide reader, "Sampler
// Extensions").
//
// Masks (per query row j of a sequence whose cache holds kv_len positions):
//   draft : j == 0 sees keys <= kv_len; j >= 1 sees keys <= kv_len + K - 1
//   verify: row j sees keys <= kv_len + pos_offset + j (causal)
//
// Kernel shape.  One wave owns 64 query rows (4 MFMA tiles of 16: GQA heads of
// one kv head times block rows) and one contiguous range of keys, walked 32
// keys per step.  It computes S^T = K Q^T with v_mfma_f32_16x16x32_bf16 (A = 16
// keys x 32 channels read straight from a K page, B = the wave's Q held in
// registers), so each lane ends with 8 consecutive keys of one query row; the
// key-to-MFMA-row order is permuted so that those 8 keys are contiguous, which
// makes P (bf16) the A operand of O += P V with no data exchange.  V pages are
// stored channel-major ([hd][page_size]) so the B operand of P V is one 16-byte
// load of 8 keys of one channel.  Softmax is online (base 2); the partial
// (max, sum, O) of every wave goes to a workspace and a merge kernel combines
// them.  All KV bytes are read once from HBM per pass.
#include "uno_device.h"
#include "uno_internal.h"

namespace uno {

union AFrag {
  uint4 u;
  bf16x8 v;
};

__device__ __forceinline__ int row_limit(int j, int kvl, int K, int pos_offset, int draft) {
  if (draft) return j == 0 ? kvl : kvl + K - 1;
  return kvl + pos_offset + j;
}

template <int HD>
__global__ void __launch_bounds__(256)
k_attention(AttnArgs a) {
  constexpr int DS = HD / 32;  // 32-channel steps of S
  constexpr int NT = HD / 16;  // 16-channel tiles of O
  const int w = threadIdx.x >> 6, l = threadIdx.x & 63;
  const int lr = l & 15, lg = l >> 4;
  const int bg = blockIdx.z, b = bg / a.Hkv, g = bg % a.Hkv;
  const int G = a.Hq / a.Hkv;
  const int QR = G * a.K;
  const int qg = blockIdx.y, qbase = qg * 64;
  const int NWS = a.plan.n_wave_splits;
  const int sigma = blockIdx.x * 4 + w;
  const int kvl = a.kv_len[b];

  // key range of this wave
  const int j_last = min(a.K - 1, (min(qbase + 63, QR - 1)) / G);
  const int kv_end = (a.draft ? (j_last >= 1 ? kvl + a.K : kvl + 1)
                              : kvl + a.pos_offset + j_last + 1);
  const int lo = sigma * a.plan.split_len;
  const int hi = (sigma == NWS - 1) ? kv_end : min(kv_end, lo + a.plan.split_len);

  // Q as the B operand: lane holds Q[q = lr][ch = ds*32 + lg*8 .. +7]
  AFrag qf[4][DS];
  int lim[4];
#pragma unroll
  for (int mt = 0; mt < 4; ++mt) {
    const int qr = qbase + mt * 16 + lr;
    const bool ok = qr < QR;
    const int j = ok ? qr / G : 0, hh = ok ? qr % G : 0;
    lim[mt] = ok ? row_limit(j, kvl, a.K, a.pos_offset, a.draft) : -1;
    const uint16_t* qp = a.q + ((size_t)(b * a.K + j) * a.Hq + g * G + hh) * HD + lg * 8;
#pragma unroll
    for (int ds = 0; ds < DS; ++ds)
      qf[mt][ds].u = ok ? *reinterpret_cast<const uint4*>(qp + ds * 32) : make_uint4(0, 0, 0, 0);
  }

  const float scale_log2 = 1.4426950408889634f / sqrtf((float)HD);
  float m_run[4], l_run[4];
  f32x4 o[4][NT];
#pragma unroll
  for (int mt = 0; mt < 4; ++mt) {
    m_run[mt] = -INFINITY;
    l_run[mt] = 0.f;
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) o[mt][nt] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  const int32_t* pt = a.page_table + (size_t)b * a.max_pages;
  const size_t head_stride = (size_t)a.ps * HD;
  int bad_page = 0;

  for (int k0 = lo; k0 < hi; k0 += 32) {
    // ---- K: MFMA row rho = lr of tile tt is physical key 8*(rho/4) + 4*tt + rho%4
    AFrag kf[2][DS];
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
      const int key = k0 + 8 * (lr >> 2) + 4 * tt + (lr & 3);
      bool ok = key < hi && key / a.ps < a.max_pages;
      int page = ok ? pt[key / a.ps] : 0;
      if (ok && (page < 0 || page >= a.n_pages)) { bad_page = 1; ok = false; }
      const uint16_t* kp = a.k_layer + ((size_t)page * a.Hkv + g) * head_stride +
                           (size_t)(key % a.ps) * HD + lg * 8;
#pragma unroll
      for (int ds = 0; ds < DS; ++ds)
        kf[tt][ds].u = ok ? *reinterpret_cast<const uint4*>(kp + ds * 32) : make_uint4(0, 0, 0, 0);
    }
    // ---- V: lane holds V[keys k0 + 8*lg .. +7][ch = nt*16 + lr]
    AFrag vf[NT];
    {
      const int key = k0 + 8 * lg;
      bool ok = key < hi && key / a.ps < a.max_pages;
      int page = ok ? pt[key / a.ps] : 0;
      if (ok && (page < 0 || page >= a.n_pages)) { bad_page = 1; ok = false; }
      const uint16_t* vp = a.v_layer + ((size_t)page * a.Hkv + g) * head_stride + (key % a.ps);
      const int n_ok = min(8, hi - key);  // keys of this group inside the range
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        uint4 u = ok ? *reinterpret_cast<const uint4*>(vp + (size_t)(nt * 16 + lr) * a.ps)
                     : make_uint4(0, 0, 0, 0);
        if (ok && n_ok < 8) {  // zero channels of keys past the range (may hold garbage)
          uint32_t* e = reinterpret_cast<uint32_t*>(&u);
#pragma unroll
          for (int c = 0; c < 8; ++c)
            if (c >= n_ok) e[c >> 1] &= (c & 1) ? 0x0000FFFFu : 0xFFFF0000u;
        }
        vf[nt].u = u;
      }
    }
    // ---- S^T tiles and online softmax per query row
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      f32x4 s[2];
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) {
        s[tt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ds = 0; ds < DS; ++ds)
          s[tt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[tt][ds].v, qf[mt][ds].v, s[tt], 0, 0, 0);
      }
      float p[8];
      float rmax = -INFINITY;
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        const int key = k0 + 8 * lg + c;
        const float v = s[c >> 2][c & 3] * scale_log2;
        p[c] = (key <= lim[mt] && key < hi) ? v : -INFINITY;
        rmax = fmaxf(rmax, p[c]);
      }
      rmax = fmaxf(rmax, __shfl_xor(rmax, 16, 64));
      rmax = fmaxf(rmax, __shfl_xor(rmax, 32, 64));
      const float m_new = fmaxf(m_run[mt], rmax);
      const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
      const float alpha = exp2f(m_run[mt] - m_use);
      float rsum = 0.f;
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        p[c] = exp2f(p[c] - m_use);
        rsum += p[c];
      }
      rsum += __shfl_xor(rsum, 16, 64);
      rsum += __shfl_xor(rsum, 32, 64);
      l_run[mt] = l_run[mt] * alpha + rsum;
      m_run[mt] = m_new;
      // O rows of this lane are q = 4*lg + i; their alphas live in lanes 4*lg + i
      float al[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) al[i] = __shfl(alpha, 4 * lg + i, 64);
      AFrag pf;
      uint32_t* pe = reinterpret_cast<uint32_t*>(&pf.u);
#pragma unroll
      for (int c = 0; c < 4; ++c) pe[c] = pack_bf16x2(p[2 * c], p[2 * c + 1]);
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
#pragma unroll
        for (int i = 0; i < 4; ++i) o[mt][nt][i] *= al[i];
        o[mt][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pf.v, vf[nt].v, o[mt][nt], 0, 0, 0);
      }
    }
  }
  if (bad_page && a.status) atomicOr(a.status + b, UNO_DEV_BAD_PAGE);

  // ---- partials
  const size_t part = ((size_t)bg * a.plan.n_qgroups + qg) * NWS + sigma;
  float* po = a.part_o + part * 64 * HD;
  float* pml = a.part_ml + part * 64 * 2;
#pragma unroll
  for (int mt = 0; mt < 4; ++mt) {
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        po[(size_t)(mt * 16 + 4 * lg + i) * HD + nt * 16 + lr] = o[mt][nt][i];
    if (lg == 0) {
      pml[(mt * 16 + lr) * 2 + 0] = m_run[mt];
      pml[(mt * 16 + lr) * 2 + 1] = l_run[mt];
    }
  }
}

// One workgroup (hd threads) per query row: combine the wave partials.
template <int HD>
__global__ void __launch_bounds__(HD)
k_attn_merge(AttnArgs a) {
  const int bg = blockIdx.y, b = bg / a.Hkv, g = bg % a.Hkv;
  const int G = a.Hq / a.Hkv;
  const int qr = blockIdx.x;
  const int qg = qr / 64, ql = qr % 64;
  const int NWS = a.plan.n_wave_splits;
  const size_t base = ((size_t)bg * a.plan.n_qgroups + qg) * NWS;
  float M = -INFINITY;
  for (int s = 0; s < NWS; ++s) M = fmaxf(M, a.part_ml[((base + s) * 64 + ql) * 2]);
  float L = 0.f, acc = 0.f;
  const int d = threadIdx.x;
  for (int s = 0; s < NWS; ++s) {
    const float* ml = a.part_ml + ((base + s) * 64 + ql) * 2;
    if (ml[0] == -INFINITY) continue;
    const float f = exp2f(ml[0] - M);
    L += ml[1] * f;
    acc += a.part_o[((base + s) * 64 + ql) * HD + d] * f;
  }
  const int j = qr / G, hh = qr % G;
  a.out[((size_t)(b * a.K + j) * a.Hq + g * G + hh) * HD + d] = f32_to_bf16(acc / L);
}

AttnPlan attn_plan(const uno_config& c, int B, int K, int max_ctx) {
  AttnPlan p;
  const int G = c.n_q_heads / c.n_kv_heads;
  p.n_qgroups = (G * K + 63) / 64;
  const long groups = (long)B * c.n_kv_heads * p.n_qgroups;
  const int ctx = max_ctx > 1 ? max_ctx : 1;
  long nws = (4096 + groups - 1) / groups;
  const long by_len = (ctx + 63) / 64;
  if (nws > by_len) nws = by_len;
  if (nws < 1) nws = 1;
  nws = (nws + 3) / 4 * 4;
  p.n_wave_splits = (int)nws;
  long sl = (ctx + nws - 1) / nws;
  p.split_len = (int)((sl + 31) / 32 * 32);
  return p;
}

size_t attn_ws_bytes(const uno_config& c, int B, int K, int max_ctx) {
  const AttnPlan p = attn_plan(c, B, K, max_ctx);
  const size_t parts = (size_t)B * c.n_kv_heads * p.n_qgroups * p.n_wave_splits * 64;
  return align_up(parts * c.head_dim * sizeof(float), 256) + align_up(parts * 2 * sizeof(float), 256);
}

hipError_t launch_attention(const AttnArgs& a, hipStream_t s) {
  const dim3 grid(a.plan.n_wave_splits / 4, a.plan.n_qgroups, a.B * a.Hkv);
  if (a.hd == 128) hipLaunchKernelGGL(k_attention<128>, grid, dim3(256), 0, s, a);
  else hipLaunchKernelGGL(k_attention<64>, grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_attn_merge(const AttnArgs& a, hipStream_t s) {
  const int G = a.Hq / a.Hkv;
  const dim3 mgrid(G * a.K, a.B * a.Hkv);
  if (a.hd == 128) hipLaunchKernelGGL(k_attn_merge<128>, mgrid, dim3(128), 0, s, a);
  else hipLaunchKernelGGL(k_attn_merge<64>, mgrid, dim3(64), 0, s, a);
  return hipGetLastError();
}

}  // namespace uno
