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
//   tree  : verify rows are the nodes of a token tree (node j at slot
//           kv_len + 1 + j); row j sees keys <= kv_len and the slots of its
//           ancestors and itself (a bit row per node)
//
// Kernel shape.  A workgroup of 4 waves owns up to 64 query rows of one
// (sequence, kv head) -- GQA heads times block rows, wave w the rows
// 16w..16w+15 -- and one range of keys, walked in chunks of 64 keys (four
// 16-token pages).  Each chunk's K and V are copied once from HBM into LDS with
// coalesced 16-byte loads (double buffered: chunk c+1 is in flight while chunk c
// is computed) and read by all four waves.  S^T = K Q^T runs on
// v_mfma_f32_16x16x32_bf16 (A = 16 keys x 32 channels from LDS, B = the wave's
// Q held in registers), so each lane ends with 8 consecutive keys of one query
// row; the key-to-MFMA-row order is permuted so that those 8 keys are
// contiguous, which makes P the A operand of O += P V with no data exchange.
// q and P enter their products as a high and a low bf16 part (two MFMAs each),
// so the only bf16 rounding left in the attention is that of the cached K/V;
// the extra MFMAs fit in the slack of this HBM-bound kernel.  V pages are
// stored channel-major ([hd][page_size]) in HBM and in LDS ([hd][64 keys]), so the B operand of P V is one 16-byte LDS read of 8
// keys of one channel.  Softmax is online (base 2).  With one key range per
// row the kernel writes the normalised output; otherwise each workgroup writes
// a partial (max, sum, O) and a merge kernel combines them.  Every KV byte is
// read from HBM once per pass.
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

// LDS swizzles (XOR on the 16-byte chunk index of a row).  A 16-byte LDS read
// serves 16 lanes per cycle from 64 banks (256 bytes), so the 16 rows one read
// touches must land in distinct bank groups:
//  * K rows (one key, HD*2 bytes): the 16 keys an S tile reads are
//    8a + 4t + b (a, b in 0..3), so the swizzle is b + 4a;
//  * V rows (one channel, 128 bytes, two per bank window): (channel / 2) % 8.
__device__ __forceinline__ int kswz(int key) { return (key & 3) | (((key >> 3) & 3) << 2); }
__device__ __forceinline__ int vswz(int d) { return (d >> 1) & 7; }

constexpr int kMaxPagesLds = 2048; // page ids of one key range cached in LDS
constexpr int kCUs = 256;

// A workgroup of RW x KH waves owns 16*RW query rows of one (sequence, kv
// head) -- row group rg = w % RW the rows 16rg..16rg+15 -- and one range of
// keys, walked in chunks of 64 keys; with KH = 2 the two waves of a row group
// take one half (32 keys) of every chunk each, with their own online softmax,
// and are merged through LDS at the end (twice the waves for the same LDS).
// Chunks stream HBM -> LDS with global_load_lds_dwordx4 (no registers; with
// the non-temporal hint, since each KV byte is read once per pass), ST deep,
// and every wave reads each chunk from LDS.  ST = 4 stages (136 KB of LDS at
// head_dim 128) keep one workgroup per CU three chunks ahead; where the grid
// fills two workgroups per CU, ST = 2 (72 KB) lets two reside and cover each
// other's waits (the 8-wave kernel is then held to 128 VGPRs, 4 waves per
// SIMD).  LDS layouts
// (16-byte chunks XOR-swizzled; the swizzle is applied by choosing which
// source address each lane loads, since lane i of a DMA writes 16*i):
//   K: [64 keys][HD]  row = one key,      chunk index ^ kswz(key) % (HD/8)
//   V: [HD][64 keys]  row = one channel,  key-group index ^ vswz(channel)
// TREE: the rows are a token tree's nodes (ancestor-bit mask past the context).
template <int HD, int RW, int KH, bool TREE, int ST>
__global__ void __launch_bounds__(RW * KH * 64, ST == 2 ? RW * KH / 2 : 1)
k_attention(AttnArgs a) {
  constexpr int kStages = ST;
  constexpr int NW = RW * KH;             // waves per workgroup
  constexpr int NH = 2 / KH;              // 32-key halves of a chunk per wave
  constexpr int DS = HD / 32;             // 32-channel MFMA steps of S
  constexpr int NT = HD / 16;             // 16-channel tiles of O
  constexpr int KROW = HD * 2;            // bytes per key row in LDS
  constexpr int KCH = HD / 8;             // 16-byte chunks per key row
  constexpr int KBYTES = 64 * KROW;       // K bytes per chunk (= V bytes)
  constexpr int STAGE = 2 * KBYTES;
  constexpr int NINSTR = STAGE / 1024;    // 1 KB DMA instructions per chunk
  constexpr int IW = NINSTR / NW;         // per wave
  static_assert(NINSTR % NW == 0, "chunk copy must split evenly over the waves");
  extern __shared__ __attribute__((aligned(16))) unsigned char lds[];
  int* pages = reinterpret_cast<int*>(lds + kStages * STAGE);

  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63;
  const int lr = l & 15, lg = l >> 4;
  const int rg = w % RW, kh = w / RW;     // row group, key half
  const int bg = blockIdx.z, b = bg / a.Hkv, g = bg % a.Hkv;
  const int G = a.Hq / a.Hkv;
  const int QR = G * a.K;
  const int QPW = 16 * RW;                 // query rows per workgroup
  const int qg = blockIdx.y, qbase = qg * QPW;
  const int split = blockIdx.x, n_split = a.plan.n_wave_splits;
  const int kvl = a.kv_len[b];

  const int j_last = min(a.K - 1, min(qbase + QPW - 1, QR - 1) / G);
  const int kv_end = a.draft ? (j_last >= 1 ? kvl + a.K : kvl + 1) : kvl + a.pos_offset + j_last + 1;
  const int lo = split * a.plan.split_len;
  int hi = (split == n_split - 1) ? kv_end : min(kv_end, lo + a.plan.split_len);
  // a range longer than the LDS page cache (only if max_ctx understated the
  // context) is cut short and flagged
  // (the last 64-key chunk may run 63 keys past hi; its pages must be cached too)
  const int hi_cap = (((lo >> a.ps_shift) + kMaxPagesLds) << a.ps_shift) - 128;
  if (hi > hi_cap) {
    if (tid == 0 && a.status) atomicOr(a.status + b, UNO_DEV_CAPACITY);
    hi = hi_cap;
  }
  const int n_chunks = hi > lo ? (hi - lo + 63) / 64 : 0;

  // page ids of [lo, hi) -> LDS (-1 where outside the table or the pool)
  const int psh = a.ps_shift, pmask = (1 << psh) - 1;
  const int p_lo = lo >> psh;
  const int n_pg = n_chunks > 0 ? ((lo + n_chunks * 64 - 1) >> psh) - p_lo + 1 : 0;
  const int32_t* pt = a.page_table + (size_t)b * a.max_pages;
  int bad_page = 0, missing = 0;
  for (int i = tid; i < n_pg && i < kMaxPagesLds; i += NW * 64) {
    const int pi = p_lo + i;
    int page = pi < a.max_pages ? pt[pi] : -1;
    if (page >= a.n_pages) page = -1;
    if (page < 0 && (pi << psh) < hi) bad_page = 1;
    missing |= page < 0;
    pages[i] = page;
  }
  // any page of the range missing (a short table, or the range's last chunk
  // running past the table): chunks must then be checked one by one
  const int any_missing = __syncthreads_or(missing);

  // this wave's 16 query rows: Q as the B operand of S^T = K Q^T
  const int qr = qbase + rg * 16 + lr;
  const bool q_ok = qr < QR;
  const int qj = q_ok ? qr / G : 0, qh = q_ok ? qr % G : 0;
  const int lim = q_ok ? row_limit(qj, kvl, a.K, a.pos_offset, a.draft) : -1;
  // token tree: keys past the context also need this row's ancestor bit
  const uint32_t* anc_row = TREE ? a.tree_anc + ((size_t)b * a.K + qj) * a.anc_words : nullptr;
  AFrag qf[DS], qfl[DS];    // q = high + low bf16 parts (scores keep ~16 bits of q)
  {
    const size_t qo = ((size_t)(b * a.K + qj) * a.Hq + g * G + qh) * HD + lg * 8;
#pragma unroll
    for (int ds = 0; ds < DS; ++ds) {
      qf[ds].u = q_ok ? *reinterpret_cast<const uint4*>(a.q + qo + ds * 32) : make_uint4(0, 0, 0, 0);
      qfl[ds].u = q_ok ? *reinterpret_cast<const uint4*>(a.q_lo + qo + ds * 32) : make_uint4(0, 0, 0, 0);
    }
  }
  // Q and the page list are complete before the first DMA, so that no wait for
  // them is left inside the chunk loop (where it would drain the DMA ring)
  wait_vmcnt<0>();
  __syncthreads();   // page list visible

  const size_t head_stride = (size_t)HD << psh;   // elements of one (page, head) block
  const size_t page_stride = head_stride * a.Hkv;  // elements of one page (all heads)
  // Per lane and DMA instruction, the key it copies (offset in the chunk) and
  // its byte offset from the K or V base inside the page are fixed; per chunk
  // only the page id changes.  Instructions 0..NINSTR/2-1 of a chunk copy K,
  // the rest V (a wave may own instructions of both kinds when the workgroup
  // has one wave).  Both are packed in one register per instruction: the byte
  // offset (< 2^17: at most 256 keys x 128 channels x 2 bytes) in the low 24
  // bits, the key (0..63) above.
  const uint16_t* kbase = a.k_layer + (size_t)g * head_stride;
  const uint16_t* vbase = a.v_layer + (size_t)g * head_stride;
  uint32_t slot[IW];
#pragma unroll
  for (int ii = 0; ii < IW; ++ii) {
    const int ins = w * IW + ii;
    if (ins < NINSTR / 2) {                      // K: 1024/KROW keys per instruction
      const int key = ins * (1024 / KROW) + l / KCH;
      const int ch = (l % KCH) ^ (kswz(key) & (KCH - 1));
      slot[ii] = (uint32_t)(((key & pmask) * HD + ch * 8) * 2) | ((uint32_t)key << 24);
    } else {                                     // V: 8 channels per instruction
      const int d = (ins - NINSTR / 2) * 8 + l / 8;
      const int kg8 = (l % 8) ^ vswz(d);
      slot[ii] = (uint32_t)(((d << psh) + ((kg8 * 8) & pmask)) * 2) | ((uint32_t)(kg8 * 8) << 24);
    }
  }
  const uint32_t page_bytes = (uint32_t)(page_stride * sizeof(uint16_t));
  const uint64_t safe_src = (uint64_t)(uintptr_t)a.k_layer;   // any readable address
  const uint32_t lds_base = lds_addr(lds) + w * IW * 1024;
  // issue the DMA of chunk c into stage c % kStages (this wave's IW instructions)
  auto issue = [&](int c) {
    const int k0 = lo + c * 64;
    const int pb = (k0 >> psh) - p_lo;           // first page of the chunk in the list
    // bytes from a page's start to key k0 (nonzero only for pages > 64 keys)
    const uint32_t in_page = (uint32_t)((k0 & pmask) & ~63);
    // the packed words enter each chunk's address arithmetic through an empty
    // asm statement, so that the compiler cannot hoist IW 64-bit addresses
    // out of the chunk loop (they would not fit the register budget)
    uint32_t sl[IW];
#pragma unroll
    for (int ii = 0; ii < IW; ++ii) {
      sl[ii] = slot[ii];
      asm volatile("" : "+v"(sl[ii]));
    }
    int pgv[IW];
#pragma unroll
    // key (0..63) first, then its page: psh reaches 8, and one 32-bit shift
    // by 24 + psh = 32 would be undefined
    for (int ii = 0; ii < IW; ++ii) pgv[ii] = pages[pb + (int)((sl[ii] >> 24) >> psh)];
    if (any_missing) {
#pragma unroll
      for (int ii = 0; ii < IW; ++ii)
        if (k0 + (int)(sl[ii] >> 24) >= hi) pgv[ii] = -1;
    }
    const uint32_t stage = __builtin_amdgcn_readfirstlane(lds_base + (c % kStages) * STAGE);
#pragma unroll
    for (int ii = 0; ii < IW; ++ii) {
      const bool is_k = w * IW + ii < NINSTR / 2;   // wave-uniform
      const int page = pgv[ii];
      const uint32_t pu = page < 0 ? 0u : (uint32_t)page;
      uint64_t src = (uint64_t)(uintptr_t)(is_k ? kbase : vbase) + (sl[ii] & 0xFFFFFFu) +
                     (uint64_t)pu * page_bytes + (uint64_t)(in_page * (is_k ? HD * 2u : 2u));
      src = page < 0 ? safe_src : src;           // zeroed below when used
      lds_dma16_nt((const void*)(uintptr_t)src, stage + ii * 1024);
    }
  };

  float m_run = -INFINITY, l_run = 0.f;
  // smallest row limit of the workgroup: chunks below it need no masking
  const int lim_min = (a.draft || TREE) ? kvl : kvl + a.pos_offset + min(a.K - 1, qbase / G);
  f32x4 o[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) o[nt] = f32x4{0.f, 0.f, 0.f, 0.f};

#pragma unroll
  for (int c = 0; c < kStages - 1; ++c)
    if (c < n_chunks) issue(c);

  for (int c = 0; c < n_chunks; ++c) {
    const int ahead = min(kStages - 2, n_chunks - 1 - c);   // chunks issued after c
    if (ahead >= 2) wait_vmcnt<2 * IW>();
    else if (ahead == 1) wait_vmcnt<IW>();
    else wait_vmcnt<0>();
    __syncthreads();
    const int k0 = lo + c * 64;
    unsigned char* K_ = lds + (c % kStages) * STAGE;
    unsigned char* V_ = K_ + KBYTES;
    // keys past the range or on a missing page: zero their V (K is masked)
    bool clean = k0 + 64 <= hi;
    if (any_missing)
      for (int pp = 0; pp < (64 >> psh) + 1 && clean; ++pp)
        clean = pages[min((k0 + (pp << psh)) >> psh, (k0 + 63) >> psh) - p_lo] >= 0;
    if (!clean) {
      for (int e = tid; e < HD * 64; e += NW * 64) {
        const int d = e / 64, key = e % 64, kabs = k0 + key;
        const bool ok = kabs < hi && pages[(kabs >> psh) - p_lo] >= 0;
        if (!ok) {
          const int kg8 = key / 8;
          *reinterpret_cast<uint16_t*>(V_ + d * 128 + ((kg8 ^ vswz(d)) << 4) + (key % 8) * 2) = 0;
        }
      }
      __syncthreads();
    }
    if (c + kStages - 1 < n_chunks) issue(c + kStages - 1);

    // S^T tiles of this wave's halves h: MFMA row rho of tile t is key
    // 32*h + 8*(rho/4) + 4*t + rho%4
    f32x4 s4[2 * NH];
#pragma unroll
    for (int hh = 0; hh < NH; ++hh)
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const int h = kh * NH + hh;
        const int key = 32 * h + 8 * (lr >> 2) + 4 * t + (lr & 3);
        f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ds = 0; ds < DS; ++ds) {
          const int ch = ds * 4 + lg;
          AFrag kf;
          kf.u = *reinterpret_cast<const uint4*>(K_ + key * KROW +
                                                 ((ch ^ (kswz(key) & (KCH - 1))) << 4));
          acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf.v, qf[ds].v, acc, 0, 0, 0);
          acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf.v, qfl[ds].v, acc, 0, 0, 0);
        }
        s4[2 * hh + t] = acc;
      }
    // lane holds keys 32h + 8*lg + c (c = 4t + i) of query row lr; scores are
    // already in log2 units (q carries log2(e)/sqrt(hd))
    float p[NH][8];
    float rmax = -INFINITY;
    const bool all_visible = k0 + 63 <= lim_min && k0 + 64 <= hi;   // wave-uniform
#pragma unroll
    for (int hh = 0; hh < NH; ++hh)
#pragma unroll
      for (int cc = 0; cc < 8; ++cc) {
        const float v = s4[2 * hh + (cc >> 2)][cc & 3];
        if (all_visible) {
          p[hh][cc] = v;
        } else {
          const int key = k0 + 32 * (kh * NH + hh) + 8 * lg + cc;
          bool vis = key <= lim && key < hi;
          if (TREE && vis && key > kvl) {
            const int node = key - kvl - 1;        // < K: key <= lim = kvl + 1 + qj
            vis = (anc_row[node >> 5] >> (node & 31)) & 1u;
          }
          p[hh][cc] = vis ? v : -INFINITY;
        }
        rmax = fmaxf(rmax, p[hh][cc]);
      }
    rmax = fmaxf(rmax, __shfl_xor(rmax, 16, 64));
    rmax = fmaxf(rmax, __shfl_xor(rmax, 32, 64));
    // The reference point m_run moves only when a row's maximum exceeds it by
    // more than 8 (in log2 units): weights then stay <= 2^8, and O and l are
    // rescaled by exp2(old - new) only on those rare chunks (softmax is
    // invariant to the reference point).  m_run starts at -inf, so the first
    // chunk with a visible key sets it.
    const bool move = rmax > m_run + 8.0f;
    const float m_new = move ? rmax : m_run;
    const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
    const float alpha = move ? __builtin_amdgcn_exp2f(m_run - m_use) : 1.0f;
    float rsum = 0.f;
#pragma unroll
    for (int hh = 0; hh < NH; ++hh)
#pragma unroll
      for (int cc = 0; cc < 8; ++cc) {
        p[hh][cc] = __builtin_amdgcn_exp2f(p[hh][cc] - m_use);
        rsum += p[hh][cc];
      }
    rsum += __shfl_xor(rsum, 16, 64);
    rsum += __shfl_xor(rsum, 32, 64);
    l_run = l_run * alpha + rsum;
    m_run = m_new;
    if (__any(move)) {
      float al[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) al[i] = __shfl(alpha, 4 * lg + i, 64);
#pragma unroll
      for (int nt = 0; nt < NT; ++nt)
#pragma unroll
        for (int i = 0; i < 4; ++i) o[nt][i] *= al[i];
    }
#pragma unroll
    for (int hh = 0; hh < NH; ++hh) {
      // P = high + low bf16 parts, so the softmax weights keep ~16 bits
      AFrag pf, pfl;
      uint32_t* pe = reinterpret_cast<uint32_t*>(&pf.u);
      uint32_t* pl = reinterpret_cast<uint32_t*>(&pfl.u);
#pragma unroll
      for (int cc = 0; cc < 4; ++cc) {
        const float x0 = p[hh][2 * cc], x1 = p[hh][2 * cc + 1];
        const uint32_t hi = pack_bf16x2(x0, x1);
        pe[cc] = hi;
        pl[cc] = pack_bf16x2(x0 - __uint_as_float(hi << 16), x1 - __uint_as_float(hi & 0xFFFF0000u));
      }
      const int kg8 = 4 * (kh * NH + hh) + lg;
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        const int d = nt * 16 + lr;
        AFrag vf;
        vf.u = *reinterpret_cast<const uint4*>(V_ + d * 128 + ((kg8 ^ vswz(d)) << 4));
        o[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pf.v, vf.v, o[nt], 0, 0, 0);
        o[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pfl.v, vf.v, o[nt], 0, 0, 0);
      }
    }
  }
  if (bad_page && a.status) atomicOr(a.status + b, UNO_DEV_BAD_PAGE);

  if constexpr (KH == 2) {
    // merge the two key halves of each row group: wave kh = 1 hands its
    // (max, sum, O) to wave kh = 0 through LDS (the chunk stages are free now)
    __syncthreads();
    float* mo = reinterpret_cast<float*>(lds);            // [RW][16][HD]
    float* mml = mo + RW * 16 * HD;                       // [RW][16][2]
    if (kh == 1) {
#pragma unroll
      for (int nt = 0; nt < NT; ++nt)
#pragma unroll
        for (int i = 0; i < 4; ++i) mo[(rg * 16 + 4 * lg + i) * HD + nt * 16 + lr] = o[nt][i];
      if (lg == 0) {
        mml[(rg * 16 + lr) * 2 + 0] = m_run;
        mml[(rg * 16 + lr) * 2 + 1] = l_run;
      }
    }
    __syncthreads();
    if (kh == 1) return;
    const float m1 = mml[(rg * 16 + lr) * 2 + 0], l1 = mml[(rg * 16 + lr) * 2 + 1];
    const float M = fmaxf(m_run, m1);
    const float M_use = (M == -INFINITY) ? 0.f : M;
    const float f0 = __builtin_amdgcn_exp2f(m_run - M_use), f1 = __builtin_amdgcn_exp2f(m1 - M_use);
    l_run = l_run * f0 + l1 * f1;
    m_run = M;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float a0 = __shfl(f0, 4 * lg + i, 64), a1 = __shfl(f1, 4 * lg + i, 64);
#pragma unroll
      for (int nt = 0; nt < NT; ++nt)
        o[nt][i] = o[nt][i] * a0 + mo[(rg * 16 + 4 * lg + i) * HD + nt * 16 + lr] * a1;
    }
  }

  // O rows of this lane: q = 4*lg + i of the row group's 16
  if (n_split == 1) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float li = __shfl(l_run, 4 * lg + i, 64);
      const int r = qbase + rg * 16 + 4 * lg + i;
      if (r >= QR) continue;
      const int j = r / G, hh = r % G;
      uint16_t* op = a.out + ((size_t)(b * a.K + j) * a.Hq + g * G + hh) * HD;
      const float inv = li > 0.f ? 1.0f / li : 0.f;
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) op[nt * 16 + lr] = f32_to_bf16(o[nt][i] * inv);
    }
  } else {
    const size_t part = ((size_t)bg * a.plan.n_qgroups + qg) * n_split + split;
    float* po = a.part_o + part * 128 * HD;
    float* pml = a.part_ml + part * 128 * 2;
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
#pragma unroll
      for (int i = 0; i < 4; ++i) po[(size_t)(rg * 16 + 4 * lg + i) * HD + nt * 16 + lr] = o[nt][i];
    if (lg == 0) {
      pml[(rg * 16 + lr) * 2 + 0] = m_run;
      pml[(rg * 16 + lr) * 2 + 1] = l_run;
    }
  }
}

// One workgroup (hd threads) per query row: combine the key-range partials.
template <int HD>
__global__ void __launch_bounds__(HD)
k_attn_merge(AttnArgs a) {
  const int bg = blockIdx.y, b = bg / a.Hkv, g = bg % a.Hkv;
  const int G = a.Hq / a.Hkv;
  const int QPW = 16 * a.plan.waves;      // query rows per workgroup
  const int qr = blockIdx.x;
  const int qg = qr / QPW, ql = qr % QPW;
  const int NS = a.plan.n_wave_splits;
  const size_t base = ((size_t)bg * a.plan.n_qgroups + qg) * NS;
  const int d = threadIdx.x;
  // the partials are combined in split order; their loads go out eight
  // splits at a time so that the latencies overlap
  constexpr int CH = 8;
  float M = -INFINITY, L = 0.f, acc = 0.f;
  float pm[CH], pl[CH], po[CH];
  auto load = [&](int s0, bool with_o) {
#pragma unroll
    for (int u = 0; u < CH; ++u) {
      const bool ok = s0 + u < NS;
      const size_t pr = (base + s0 + u) * 128 + ql;
      pm[u] = ok ? a.part_ml[pr * 2] : -INFINITY;
      pl[u] = ok ? a.part_ml[pr * 2 + 1] : 0.f;
      po[u] = ok && with_o ? a.part_o[pr * HD + d] : 0.f;
    }
  };
  auto accumulate = [&]() {
#pragma unroll
    for (int u = 0; u < CH; ++u) {
      if (pm[u] == -INFINITY) continue;
      const float f = exp2f(pm[u] - M);
      L += pl[u] * f;
      acc += po[u] * f;
    }
  };
  if (NS <= CH) {
    load(0, true);
#pragma unroll
    for (int u = 0; u < CH; ++u) M = fmaxf(M, pm[u]);
    accumulate();
  } else {
    for (int s0 = 0; s0 < NS; s0 += CH) {
      load(s0, false);
#pragma unroll
      for (int u = 0; u < CH; ++u) M = fmaxf(M, pm[u]);
    }
    for (int s0 = 0; s0 < NS; s0 += CH) {
      load(s0, true);
      accumulate();
    }
  }
  const int j = qr / G, hh = qr % G;
  a.out[((size_t)(b * a.K + j) * a.Hq + g * G + hh) * HD + d] = f32_to_bf16(L > 0.f ? acc / L : 0.f);
}

AttnPlan attn_plan(const uno_config& c, int B, int K, int max_ctx) {
  AttnPlan p;
  const int G = c.n_q_heads / c.n_kv_heads;
  const int tiles = (G * K + 15) / 16;
  p.waves = 1;
  while (p.waves < tiles && p.waves < 8) p.waves *= 2;
  p.key_halves = p.waves <= 4 ? 2 : 1;
  p.n_qgroups = (G * K + 16 * p.waves - 1) / (16 * p.waves);
  const long groups = (long)B * c.n_kv_heads * p.n_qgroups;
  const long ctx = max_ctx > 1 ? max_ctx : 1;
  const long by_len = (ctx + 255) / 256;       // at least 4 chunks of 64 keys per range
  const long max_len = (long)(kMaxPagesLds - 2) * c.page_size - 64;
  const long by_lds = (ctx + max_len - 1) / max_len;
  // key ranges for `per_cu` workgroups per CU, within the limits above
  auto splits_for = [&](long per_cu) {
    long ns = (per_cu * kCUs + groups - 1) / groups;
    if (ns > by_len) ns = by_len;
    if (ns < by_lds) ns = by_lds;
    return ns < 1 ? 1L : ns;
  };
  long ns = splits_for(1);                     // one workgroup per CU, 4 stages
  p.stages = 4;
  if (c.head_dim == 128 && groups * splits_for(2) >= 2 * kCUs) {
    ns = splits_for(2);                        // two per CU, 2 stages each
    p.stages = 2;
  }
  p.n_wave_splits = (int)ns;
  const long sl = (ctx + ns - 1) / ns;
  p.split_len = (int)((sl + 63) / 64 * 64);
  return p;
}

size_t attn_ws_bytes(const uno_config& c, int B, int K, int max_ctx) {
  const AttnPlan p = attn_plan(c, B, K, max_ctx);
  const size_t parts = (size_t)B * c.n_kv_heads * p.n_qgroups * p.n_wave_splits * 128;
  return align_up(parts * c.head_dim * sizeof(float), 256) + align_up(parts * 2 * sizeof(float), 256);
}

template <int HD, bool TREE, int ST>
static hipError_t launch_attention_hd(const AttnArgs& a, hipStream_t s) {
  const dim3 grid(a.plan.n_wave_splits, a.plan.n_qgroups, a.B * a.Hkv);
  const size_t lds = (size_t)ST * 2 * 64 * HD * 2 + kMaxPagesLds * sizeof(int);
  const int kh = a.plan.key_halves;
  const dim3 block(64 * a.plan.waves * kh);
  switch (a.plan.waves * 10 + kh) {
    case 12: hipLaunchKernelGGL((k_attention<HD, 1, 2, TREE, ST>), grid, block, lds, s, a); break;
    case 22: hipLaunchKernelGGL((k_attention<HD, 2, 2, TREE, ST>), grid, block, lds, s, a); break;
    case 42: hipLaunchKernelGGL((k_attention<HD, 4, 2, TREE, ST>), grid, block, lds, s, a); break;
    default: hipLaunchKernelGGL((k_attention<HD, 8, 1, TREE, ST>), grid, block, lds, s, a); break;
  }
  return hipGetLastError();
}

hipError_t launch_attention(const AttnArgs& a, hipStream_t s) {
  const bool two = a.plan.stages == 2;   // head_dim 128 only
  if (a.tree_anc) {
    if (a.hd != 128) return launch_attention_hd<64, true, 4>(a, s);
    return two ? launch_attention_hd<128, true, 2>(a, s) : launch_attention_hd<128, true, 4>(a, s);
  }
  if (a.hd != 128) return launch_attention_hd<64, false, 4>(a, s);
  return two ? launch_attention_hd<128, false, 2>(a, s) : launch_attention_hd<128, false, 4>(a, s);
}

hipError_t launch_attn_merge(const AttnArgs& a, hipStream_t s) {
  if (a.plan.n_wave_splits == 1) return hipSuccess;   // the attention kernel wrote `out`
  const int G = a.Hq / a.Hkv;
  const dim3 mgrid(G * a.K, a.B * a.Hkv);
  if (a.hd == 128) hipLaunchKernelGGL(k_attn_merge<128>, mgrid, dim3(128), 0, s, a);
  else hipLaunchKernelGGL(k_attn_merge<64>, mgrid, dim3(64), 0, s, a);
  return hipGetLastError();
}

}  // namespace uno
