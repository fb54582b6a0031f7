// RoPE on q and k and the paged K/V write of one q|k|v row value pair:
// device helpers shared by the stand-alone kernel (elementwise.hip) and the
// q|k|v projection's split-K reduction (gemm.hip), so that both store exactly
// the same way.  Rotate-half RoPE: (x1, x2) at channels (i, i + hd/2) of a
// head -> (x1 cos - x2 sin, x2 cos + x1 sin) with (cos, sin) from the row's
// table; q is scaled by log2(e)/sqrt(hd) (the attention works in base 2) and
// stored as a high and a low bf16 part; k and v (bf16) go to the row's slot of
// the paged cache, K pages [slot][hd], V pages transposed [hd][slot].
#pragma once
#include "uno_device.h"
#include "uno_internal.h"

namespace uno {

// Page of row r's K/V slot (and the slot in it); -1 when outside the
// sequence's table or the pool (flagged when the table was made).
__device__ __forceinline__ int rope_page(const RopeArgs& ra, int r, int* slot) {
  const int2 p = ra.row_page[r];
  *slot = p.y;
  return p.x;
}

// channels (i, i + hd/2) of q or k head `head` (q heads first) of row r
__device__ __forceinline__ void rope_store_pair(const RopeArgs& ra, int r, int head, int i,
                                                float x1, float x2, int page, int slot) {
  const int hd = ra.hd, half = hd / 2;
  const float2 a = ra.cs[(size_t)r * half + i];
  const float y1 = x1 * a.x - x2 * a.y;
  const float y2 = x2 * a.x + x1 * a.y;
  if (head < ra.Hq) {
    const float q_scale = 1.4426950408889634f / sqrtf((float)hd);
    const size_t o = (size_t)r * ra.Hq * hd + head * hd;
    const float z1 = y1 * q_scale, z2 = y2 * q_scale;
    const uint16_t h1 = f32_to_bf16(z1), h2 = f32_to_bf16(z2);
    ra.q_out[o + i] = h1;
    ra.q_out[o + i + half] = h2;
    ra.q_lo[o + i] = f32_to_bf16(z1 - bf16_to_f32(h1));
    ra.q_lo[o + i + half] = f32_to_bf16(z2 - bf16_to_f32(h2));
  } else if (page >= 0) {
    uint16_t* kp = ra.k_layer + (((size_t)page * ra.Hkv + (head - ra.Hq)) * ra.ps + slot) * hd;
    kp[i] = f32_to_bf16(y1);
    kp[i + half] = f32_to_bf16(y2);
  }
}

// channel d of v head g of a row whose slot is (page, slot)
__device__ __forceinline__ void rope_store_v(const RopeArgs& ra, int g, int d, float v, int page,
                                             int slot) {
  if (page >= 0)
    ra.v_layer[(((size_t)page * ra.Hkv + g) * ra.hd + d) * ra.ps + slot] = f32_to_bf16(v);
}

}  // namespace uno
