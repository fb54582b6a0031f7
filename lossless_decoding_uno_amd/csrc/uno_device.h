// Device-side helpers shared by the gfx950 kernels of libuno.
#pragma once
#include <hip/hip_runtime.h>
#include <hip/hip_bf16.h>
#include <stdint.h>

#define UNO_WAVE 64

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(16))) float f32x16;

// ---------------------------------------------------------------- bf16 <-> fp32
__device__ __forceinline__ float bf16_to_f32(uint16_t v) {
  return __uint_as_float(((uint32_t)v) << 16);
}
// round-to-nearest-even conversions; on gfx950 these lower to the hardware
// v_cvt_pk_bf16_f32 (inputs are finite in this library)
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_v;
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  return __builtin_bit_cast(uint16_t, (__bf16)f);
}
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const bf16x2_v v = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, v);
}

// ---------------------------------------------------------------- wave helpers
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, UNO_WAVE));
  return v;
}
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, UNO_WAVE);
  return v;
}
__device__ __forceinline__ uint64_t wave_sum_u64(uint64_t v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, UNO_WAVE);
  return v;
}
__device__ __forceinline__ int lane_id() { return threadIdx.x & (UNO_WAVE - 1); }

// fp32 maximum by integer atomics (LDS or global), exact and order free: a
// non-negative float orders like its bits as int, a negative one inversely to
// its bits as unsigned.  The slot starts at -inf (kNegInfBits).
constexpr int kNegInfBits = (int)0xFF800000u;
__device__ __forceinline__ void atomic_max_f32(float* p, float v) {
  if (__float_as_int(v) >= 0) atomicMax(reinterpret_cast<int*>(p), __float_as_int(v));
  else atomicMin(reinterpret_cast<unsigned int*>(p), __float_as_uint(v));
}

// ---------------------------------------------------------------- 128-bit unsigned
struct u128 {
  uint64_t lo, hi;
};
__device__ __forceinline__ u128 u128_make(uint64_t lo, uint64_t hi) { u128 r; r.lo = lo; r.hi = hi; return r; }
__device__ __forceinline__ u128 mul_64x64(uint64_t a, uint64_t b) {
  return u128_make(a * b, __umul64hi(a, b));
}
__device__ __forceinline__ u128 u128_add(u128 a, u128 b) {
  u128 r;
  r.lo = a.lo + b.lo;
  r.hi = a.hi + b.hi + (r.lo < a.lo ? 1ull : 0ull);
  return r;
}
__device__ __forceinline__ u128 u128_sub(u128 a, u128 b) {  // a >= b
  u128 r;
  r.lo = a.lo - b.lo;
  r.hi = a.hi - b.hi - (a.lo < b.lo ? 1ull : 0ull);
  return r;
}
__device__ __forceinline__ bool u128_lt(u128 a, u128 b) {
  return a.hi < b.hi || (a.hi == b.hi && a.lo < b.lo);
}
__device__ __forceinline__ bool u128_is_zero(u128 a) { return (a.lo | a.hi) == 0; }
__device__ __forceinline__ u128 u128_shfl_xor(u128 v, int o) {
  return u128_make(__shfl_xor(v.lo, o, UNO_WAVE), __shfl_xor(v.hi, o, UNO_WAVE));
}
__device__ __forceinline__ u128 u128_shfl(u128 v, int src) {
  return u128_make(__shfl(v.lo, src, UNO_WAVE), __shfl(v.hi, src, UNO_WAVE));
}
__device__ __forceinline__ u128 u128_shfl_up(u128 v, int d) {
  return u128_make(__shfl_up(v.lo, d, UNO_WAVE), __shfl_up(v.hi, d, UNO_WAVE));
}
__device__ __forceinline__ u128 wave_sum_u128(u128 v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = u128_add(v, u128_shfl_xor(v, o));
  return v;
}
// inclusive prefix sum over the 64 lanes
__device__ __forceinline__ u128 wave_inclusive_scan_u128(u128 v) {
  const int l = lane_id();
#pragma unroll
  for (int d = 1; d < UNO_WAVE; d <<= 1) {
    u128 o = u128_shfl_up(v, d);
    if (l >= d) v = u128_add(v, o);
  }
  return v;
}

// ---------------------------------------------------------------- LDS DMA
// s_waitcnt with only the vector-memory counter constrained (gfx9 encoding:
// vmcnt bits [3:0] and [15:14], expcnt [6:4] and lgkmcnt [11:8] left at max).
// Counts above the 6-bit field wait for more than needed (always safe).
template <int N0>
__device__ __forceinline__ void wait_vmcnt() {
  constexpr int N = N0 < 63 ? N0 : 63;
  static_assert(N >= 0, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

// One 16-byte-per-lane DMA from global memory into LDS: lane i's bytes land at
// lds_dst + 16*i (lds_dst wave-uniform).  Written as inline asm so that the
// compiler does not serialise the ring of in-flight chunks with vmcnt(0)
// waits; completion is awaited explicitly with wait_vmcnt + a barrier.  The
// instruction has no destination register.
__device__ __forceinline__ void lds_dma16(const void* src, uint32_t lds_off) {
  const uint32_t m0v = __builtin_amdgcn_readfirstlane(lds_off);
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off"
               :
               : "s"(m0v), "v"(src)
               : "memory", "m0");
}
// The same with the non-temporal hint, for data read once per launch (the KV
// pages of a pass): on gfx950 a stream of such loads moves ~7.1 TB/s from HBM
// against ~6.3 TB/s without the hint.
__device__ __forceinline__ void lds_dma16_nt(const void* src, uint32_t lds_off) {
  const uint32_t m0v = __builtin_amdgcn_readfirstlane(lds_off);
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off nt"
               :
               : "s"(m0v), "v"(src)
               : "memory", "m0");
}

// 32-bit LDS address of a pointer into __shared__ memory
// Word 0 of Philox4x64-10 (Salmon et al., SC'11: the 4x64 bijection with 10
// rounds) for counter (c0, c1, c2, c3) and key (k0, k1).  One round maps the
// counter to (hi(M1 c2)^c1^k0, lo(M1 c2), hi(M0 c0)^c3^k1, lo(M0 c0)); the key
// is bumped by the Weyl constants (W0, W1) between rounds.  Every random
// decision of the decode step is one counter: (slot, row j, sequence b, step).
__device__ __forceinline__ uint64_t philox_word0(uint64_t c0, uint64_t c1, uint64_t c2,
                                                 uint64_t c3, uint64_t k0, uint64_t k1) {
  const uint64_t M0 = 0xD2E7470EE14C6C93ull, M1 = 0xCA5A826395121157ull;
  const uint64_t W0 = 0x9E3779B97F4A7C15ull, W1 = 0xBB67AE8584CAA73Bull;
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    if (r) { k0 += W0; k1 += W1; }
    const uint64_t lo0 = M0 * c0, hi0 = __umul64hi(M0, c0);
    const uint64_t lo1 = M1 * c2, hi1 = __umul64hi(M1, c2);
    const uint64_t n0 = hi1 ^ c1 ^ k0, n2 = hi0 ^ c3 ^ k1;
    c0 = n0; c1 = lo1; c2 = n2; c3 = lo0;
  }
  return c0;
}

// Buffer resource (raw, stride 0) over `bytes` bytes at `base`; loads past
// the end return zero instead of faulting.
typedef int i32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ i32x4 make_rsrc(const void* p, uint32_t bytes) {
  const uint64_t base = reinterpret_cast<uint64_t>(p);
  i32x4 r;
  r[0] = __builtin_amdgcn_readfirstlane(static_cast<int>(base & 0xffffffffu));
  r[1] = __builtin_amdgcn_readfirstlane(static_cast<int>(base >> 32));
  r[2] = __builtin_amdgcn_readfirstlane(static_cast<int>(bytes));
  r[3] = 0x00020000;
  return r;
}
// 16 bytes per lane from rsrc + voff + soff into LDS at lds_off + 16 * lane
// (buffer_load_dwordx4 with the LDS bit; counted by vmcnt).
__device__ __forceinline__ void lds_dma16_buf(i32x4 rsrc, uint32_t voff, uint32_t soff,
                                              uint32_t lds_off) {
  const uint32_t m0v = __builtin_amdgcn_readfirstlane(lds_off);
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds"
               :: "s"(m0v), "v"(voff), "s"(rsrc), "s"(soff) : "memory", "m0");
}
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

