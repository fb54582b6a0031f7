// Measurement probes (include/uno_probe.h): a streaming read, a copy and a
// register-only MFMA loop, the ceilings the decode kernels are compared with.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "uno_probe.h"

namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(4))) unsigned int u32x4;

constexpr int kThreads = 256;
constexpr int kUnroll = 4;

template <bool NT, int UN>
__global__ void __launch_bounds__(kThreads) k_probe_read(const u32x4* __restrict__ src,
                                                         size_t n16, float* __restrict__ sink) {
  // each lane reads UN 16-byte words per round; rounds stride by the grid
  const size_t lanes = (size_t)gridDim.x * kThreads;
  uint32_t acc = 0;
  for (size_t i = (size_t)blockIdx.x * kThreads + threadIdx.x; i < n16; i += lanes * UN) {
    u32x4 v[UN];
#pragma unroll
    for (int u = 0; u < UN; ++u) {
      const size_t j = i + u * lanes;
      if (j < n16) {
        if (NT) v[u] = __builtin_nontemporal_load(src + j);
        else v[u] = src[j];
      } else {
        v[u] = u32x4{0u, 0u, 0u, 0u};
      }
    }
#pragma unroll
    for (int u = 0; u < UN; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  __shared__ uint32_t red[kThreads / 64];
  for (int o = 32; o > 0; o >>= 1) acc ^= __shfl_xor(acc, o, 64);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = acc;
  __syncthreads();
  if (threadIdx.x == 0) sink[blockIdx.x] = (float)(red[0] ^ red[1] ^ red[2] ^ red[3]);
}

__global__ void __launch_bounds__(kThreads) k_probe_copy(const uint4* __restrict__ src,
                                                         uint4* __restrict__ dst, size_t n16) {
  const size_t lanes = (size_t)gridDim.x * kThreads;
  for (size_t i = (size_t)blockIdx.x * kThreads + threadIdx.x; i < n16; i += lanes * kUnroll) {
    uint4 v[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const size_t j = i + u * lanes;
      v[u] = j < n16 ? src[j] : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const size_t j = i + u * lanes;
      if (j < n16) dst[j] = v[u];
    }
  }
}

__global__ void __launch_bounds__(kThreads) k_probe_mfma(int iters, float* __restrict__ sink) {
  bf16x8 a, b;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    a[e] = (__bf16)(0.001f * (float)((threadIdx.x + e) & 7));
    b[e] = (__bf16)(0.002f * (float)((threadIdx.x * 3 + e) & 7));
  }
  f32x16 c0 = {}, c1 = {}, c2 = {}, c3 = {};
  for (int it = 0; it < iters; ++it) {
    c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c0, 0, 0, 0);
    c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c1, 0, 0, 0);
    c2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c2, 0, 0, 0);
    c3 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c3, 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int e = 0; e < 16; ++e) s += c0[e] + c1[e] + c2[e] + c3[e];
  if (threadIdx.x == 0) sink[blockIdx.x] = s;
}

}  // namespace

extern "C" {

int uno_probe_read(const void* src, size_t bytes, int mode, int n_wg, float* sink,
                   void* stream) {
  if (!src || !sink || n_wg < 1 || bytes == 0 || bytes % (16 * kThreads) || mode < 0 || mode > 3)
    return -1;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const size_t n16 = bytes / 16;
  const u32x4* p = static_cast<const u32x4*>(src);
  switch (mode) {
    case 0: hipLaunchKernelGGL((k_probe_read<false, 4>), dim3(n_wg), dim3(kThreads), 0, s, p, n16, sink); break;
    case 1: hipLaunchKernelGGL((k_probe_read<true, 4>), dim3(n_wg), dim3(kThreads), 0, s, p, n16, sink); break;
    case 2: hipLaunchKernelGGL((k_probe_read<false, 8>), dim3(n_wg), dim3(kThreads), 0, s, p, n16, sink); break;
    default: hipLaunchKernelGGL((k_probe_read<true, 8>), dim3(n_wg), dim3(kThreads), 0, s, p, n16, sink); break;
  }
  return hipGetLastError() == hipSuccess ? 0 : -2;
}

int uno_probe_copy(const void* src, void* dst, size_t bytes, int n_wg, void* stream) {
  if (!src || !dst || n_wg < 1 || bytes == 0 || bytes % (16 * kThreads)) return -1;
  hipLaunchKernelGGL(k_probe_copy, dim3(n_wg), dim3(kThreads), 0, static_cast<hipStream_t>(stream),
                     static_cast<const uint4*>(src), static_cast<uint4*>(dst), bytes / 16);
  return hipGetLastError() == hipSuccess ? 0 : -2;
}

int uno_probe_mfma(int iters, int n_wg, float* sink, void* stream) {
  if (!sink || n_wg < 1 || iters < 1) return -1;
  hipLaunchKernelGGL(k_probe_mfma, dim3(n_wg), dim3(kThreads), 0,
                     static_cast<hipStream_t>(stream), iters, sink);
  return hipGetLastError() == hipSuccess ? 0 : -2;
}

}  // extern "C"
