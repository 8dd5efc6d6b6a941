// Measured peaks of the two pipes the split kernel is priced against on
// gfx950: HBM read bandwidth and the dense MFMA rate.  The roofline fractions
// of the attention kernels are reported against the datasheet peaks and
// against these (a streaming read and a dependency-free MFMA stream are the
// best a kernel can do on this part).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "mla.h"
#include "mla_peaks.h"

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

constexpr int kThreads = 256;
constexpr int kUnroll = 8;   // 16-byte loads in flight per lane

// Buffer resource over [base, base + bytes); loads past the range read zero.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc_of(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, bytes, 0x00020000);
}

// Streaming read into VGPRs: every lane reads 16-byte chunks, grid-stride, and
// XORs them into one word per workgroup (so the loads cannot be dropped).
__global__ __launch_bounds__(kThreads) void read_vgpr_kernel(const u32x4* __restrict__ p, int64_t n16,
                                                             uint32_t* __restrict__ sink) {
  const int64_t stride = (int64_t)gridDim.x * kThreads;
  uint32_t acc = 0;
  int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  for (; i + (kUnroll - 1) * stride < n16; i += kUnroll * stride) {
    u32x4 v[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) v[u] = __builtin_nontemporal_load(p + i + u * stride);
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) acc ^= v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3];
  }
  for (; i < n16; i += stride) {
    const u32x4 v = p[i];
    acc ^= v[0] ^ v[1] ^ v[2] ^ v[3];
  }
  acc ^= __shfl_xor(acc, 1) ^ __shfl_xor(acc, 2);   // keep the value live
  if (threadIdx.x == 0) sink[blockIdx.x] = acc;
}

// Streaming read straight into LDS (16 bytes a lane with buffer_load ... lds,
// the copy path of the split kernels): each wave fills its 1 KiB LDS slot
// again and again; one word of the slot is folded into the sink at the end.
__global__ __launch_bounds__(kThreads) void read_lds_kernel(const uint8_t* __restrict__ p, int64_t bytes,
                                                            uint32_t* __restrict__ sink) {
  __shared__ __attribute__((aligned(16))) uint8_t slot[kThreads / 64][kUnroll][1024];
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // wave-uniform
  const int lane = threadIdx.x & 63;
  const int64_t waves = (int64_t)gridDim.x * (kThreads / 64);
  const int64_t wave_id = (int64_t)blockIdx.x * (kThreads / 64) + w;
  const int64_t chunks = bytes >> 10;   // 1 KiB per wave-wide load
  for (int64_t c0 = wave_id * kUnroll; c0 < chunks; c0 += waves * kUnroll) {
    // one descriptor per group of kUnroll KiB (32-bit range)
    const __amdgpu_buffer_rsrc_t r = rsrc_of(p + (c0 << 10), (uint32_t)(min<int64_t>(kUnroll, chunks - c0) << 10));
#pragma unroll
    for (int u = 0; u < kUnroll; ++u)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)&slot[w][u][0], 16,
                                               (uint32_t)(u * 1024 + 16 * lane), 0, 0, 0);
  }
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (lane == 0) atomicXor(sink + blockIdx.x % 1024, *(const uint32_t*)&slot[w][0][0]);
}

// Dense MFMA stream: CHAINS independent accumulators per wave, so the matrix
// core of a SIMD never waits on a dependency; one wave per SIMD.
template <int CHAINS>
__global__ __launch_bounds__(kThreads) void mfma_fp8_kernel(int iters, float* __restrict__ sink) {
  const int lane = threadIdx.x & 63;
  i32x8 a, b;
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    a[k] = 0x38383838 ^ (lane * 0x01010101 + k);
    b[k] = 0x30303030 ^ (lane * 0x00010001 + 3 * k);
  }
  f32x16 c[CHAINS];
#pragma unroll
  for (int j = 0; j < CHAINS; ++j) c[j] = f32x16{};
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int j = 0; j < CHAINS; ++j)
      c[j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c[j], 0, 0, 0, 127, 0, 127);
  }
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < CHAINS; ++j)
#pragma unroll
    for (int k = 0; k < 16; ++k) s += c[j][k];
  if (s == 12345.678f) sink[blockIdx.x] = s;   // practically never: keeps the MFMAs
}

template <int CHAINS>
__global__ __launch_bounds__(kThreads) void mfma_bf16_kernel(int iters, float* __restrict__ sink) {
  const int lane = threadIdx.x & 63;
  bf16x8 a, b;
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    a[k] = (__bf16)(0.001f * (lane + k));
    b[k] = (__bf16)(0.002f * (lane - k));
  }
  f32x16 c[CHAINS];
#pragma unroll
  for (int j = 0; j < CHAINS; ++j) c[j] = f32x16{};
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int j = 0; j < CHAINS; ++j) c[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c[j], 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < CHAINS; ++j)
#pragma unroll
    for (int k = 0; k < 16; ++k) s += c[j][k];
  if (s == 12345.678f) sink[blockIdx.x] = s;
}

mla_status launched(hipError_t e) { return e == hipSuccess ? MLA_OK : MLA_ERR_HIP; }

}  // namespace

extern "C" {

mla_status mla_peak_hbm_read(const void* buf, int64_t bytes, int32_t mode, uint32_t* sink,
                             int32_t workgroups, void* stream) {
  if (!buf || !sink) return MLA_ERR_NULL_ARG;
  if (bytes < 1024 || (bytes & 1023) || ((uintptr_t)buf & 15)) return MLA_ERR_BAD_SHAPE;
  if (workgroups < 1 || workgroups > 1024) return MLA_ERR_BAD_SHAPE;
  hipStream_t s = (hipStream_t)stream;
  if (mode == MLA_PEAK_READ_VGPR) {
    hipLaunchKernelGGL(read_vgpr_kernel, dim3(workgroups), dim3(kThreads), 0, s, (const u32x4*)buf,
                       bytes / 16, sink);
  } else if (mode == MLA_PEAK_READ_LDS) {
    hipLaunchKernelGGL(read_lds_kernel, dim3(workgroups), dim3(kThreads), 0, s, (const uint8_t*)buf, bytes,
                       sink);
  } else {
    return MLA_ERR_BAD_SHAPE;
  }
  return launched(hipGetLastError());
}

mla_status mla_peak_mfma(int32_t kind, int32_t iters, float* sink, int32_t workgroups, void* stream) {
  if (!sink) return MLA_ERR_NULL_ARG;
  if (iters < 1 || iters > (1 << 24) || workgroups < 1 || workgroups > 1024) return MLA_ERR_BAD_SHAPE;
  hipStream_t s = (hipStream_t)stream;
  if (kind == MLA_PEAK_MFMA_FP8) {
    hipLaunchKernelGGL(mfma_fp8_kernel<4>, dim3(workgroups), dim3(kThreads), 0, s, iters, sink);
  } else if (kind == MLA_PEAK_MFMA_BF16) {
    hipLaunchKernelGGL(mfma_bf16_kernel<4>, dim3(workgroups), dim3(kThreads), 0, s, iters, sink);
  } else {
    return MLA_ERR_BAD_SHAPE;
  }
  return launched(hipGetLastError());
}

}  // extern "C"
