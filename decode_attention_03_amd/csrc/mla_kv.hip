// KV-cache append with FP8 quantisation, and the dynamic per-tensor scale (gfx950).
//
// The step before attention in a decode or verify step writes the compressed
// latents of the Q newest positions into their paged slots, as bf16 or as FP8
// bytes under one per-tensor scale ("Kimi K2.6 + DFlash on 8x MI300X (508
// tok/s)", section "st=2 vs st=8 & FP8 vs BF16": FP8 doubles the cache's
// token capacity, and a dynamically computed scale costs per-slot throughput;
// section "Next": auto-computed scales today, static calibration proposed).
//
// Slot of new token j of sequence b: position t = L_b - Q + j (seq_lens count
// the new tokens), block page_table[b][t / 16], row t % 16.  FP8 byte of a
// bf16 value x: RNE conversion of the float32 quotient x / kv_scale (IEEE
// division), clamped to +-448 first so that large values saturate.
//
// Both are tiny and HBM/latency bound: one thread per 16-byte chunk (8
// values) of a new latent; the scale of up to 2^16 values is one workgroup's
// max, of more a grid-stride max over bf16 magnitudes combined with one
// 32-bit atomic max per workgroup (three launches).
#include "mla_common.hpp"

namespace mla {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kAppendThreads = 256;
constexpr int kChunksPerRow = kLatent / 8;   // 72
constexpr float kE4M3Max = 448.f;

__device__ __forceinline__ float bf16_lo(uint32_t v) { return __uint_as_float(v << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t v) { return __uint_as_float(v & 0xFFFF0000u); }

__device__ __forceinline__ float sat(float v) { return fminf(fmaxf(v, -kE4M3Max), kE4M3Max); }

template <bool FP8>
__global__ __launch_bounds__(kAppendThreads) void append_kernel(AppendArgs a) {
  const int64_t idx = (int64_t)blockIdx.x * kAppendThreads + threadIdx.x;
  const int64_t total = (int64_t)a.batch * a.num_q * kChunksPerRow;
  if (idx >= total) return;
  const int64_t row = idx / kChunksPerRow;          // b * Q + j
  const int c = (int)(idx - row * kChunksPerRow);
  const int b = (int)(row / a.num_q);
  const int j = (int)(row - (int64_t)b * a.num_q);
  const int t = a.seq_lens[b] - a.num_q + j;
  // a slot outside the page table or the pool is a caller error: nothing is
  // written (the debug build also reports it)
  if (t < 0 || t / kPage >= a.max_blocks) {
    if constexpr (kDebug) debug_report(a.debug_flags, t < 0 ? kDbgSeqShort : kDbgSeqLong);
    return;
  }
  const int blk = a.page_table[(int64_t)b * a.max_blocks + t / kPage];
  if (blk < 0 || blk >= a.num_blocks) {
    if constexpr (kDebug) debug_report(a.debug_flags, kDbgPageId);
    return;
  }
  const int64_t slot = (int64_t)blk * kPage + t % kPage;
  const u32x4 v = *(const u32x4*)(a.kv_new + row * kLatent + 8 * c);
  if constexpr (!FP8) {
    *(u32x4*)(a.kv + (slot * kLatent + 8 * c) * 2) = v;
  } else {
    const float s = a.kv_scale;
    u32x2 o;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const uint32_t w0 = v[2 * h], w1 = v[2 * h + 1];
      int p = __builtin_amdgcn_cvt_pk_fp8_f32(sat(bf16_lo(w0) / s), sat(bf16_hi(w0) / s), 0, false);
      p = __builtin_amdgcn_cvt_pk_fp8_f32(sat(bf16_lo(w1) / s), sat(bf16_hi(w1) / s), p, true);
      o[h] = (uint32_t)p;
    }
    *(u32x2*)(a.kv + slot * kLatent + 8 * c) = o;
  }
}

__global__ void scale_init_kernel(uint32_t* slot) { *slot = 0u; }

// max over bf16 magnitudes (bit patterns with the sign cleared: for non-NaN
// values their integer order is their value order)
__global__ __launch_bounds__(kAppendThreads) void amax_kernel(const uint16_t* x, int64_t count,
                                                               uint32_t* slot) {
  __shared__ uint32_t red[kAppendThreads / 64];
  const int64_t stride = (int64_t)gridDim.x * kAppendThreads;
  const int64_t first = (int64_t)blockIdx.x * kAppendThreads + threadIdx.x;
  const bool vec = (((uintptr_t)x) & 15) == 0;
  const int64_t nvec = vec ? count / 8 : 0;
  uint32_t m = 0;
  for (int64_t i = first; i < nvec; i += stride) {
    const u32x4 v = *(const u32x4*)(x + 8 * i);
#pragma unroll
    for (int k = 0; k < 4; ++k) m = max(m, max(v[k] & 0x7FFFu, (v[k] >> 16) & 0x7FFFu));
  }
  for (int64_t i = 8 * nvec + first; i < count; i += stride) m = max(m, (uint32_t)(x[i] & 0x7FFFu));
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) m = max(m, (uint32_t)__shfl_xor((int)m, d));
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
    m = max(max(red[0], red[1]), max(red[2], red[3]));
    atomicMax(slot, m);
  }
}

__device__ __forceinline__ float scale_of(uint32_t m) {
  if (m > 0x7F80u) return __builtin_nanf("");        // a NaN among the values
  if (m == 0u) return 1.f;                           // all zero
  return __uint_as_float(m << 16) / kE4M3Max;        // inf stays inf
}

__global__ void scale_finalize_kernel(uint32_t* slot) { *(float*)slot = scale_of(*slot); }

// Few values (the new latents of one step): one workgroup, one launch.
constexpr int64_t kSmallScaleCount = 1 << 16;
__global__ __launch_bounds__(kAppendThreads) void small_scale_kernel(const uint16_t* x, int64_t count,
                                                                      float* scale) {
  __shared__ uint32_t red[kAppendThreads / 64];
  uint32_t m = 0;
  for (int64_t i = threadIdx.x; i < count; i += kAppendThreads) m = max(m, (uint32_t)(x[i] & 0x7FFFu));
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) m = max(m, (uint32_t)__shfl_xor((int)m, d));
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) *scale = scale_of(max(max(red[0], red[1]), max(red[2], red[3])));
}

}  // namespace

hipError_t launch_append(const AppendArgs& a, bool fp8, hipStream_t stream) {
  const int64_t total = (int64_t)a.batch * a.num_q * kChunksPerRow;
  const dim3 grid((unsigned)((total + kAppendThreads - 1) / kAppendThreads));
  if (fp8)
    hipLaunchKernelGGL(append_kernel<true>, grid, dim3(kAppendThreads), 0, stream, a);
  else
    hipLaunchKernelGGL(append_kernel<false>, grid, dim3(kAppendThreads), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_dynamic_scale(const uint16_t* x, int64_t count, float* scale, hipStream_t stream) {
  if (count <= kSmallScaleCount) {
    hipLaunchKernelGGL(small_scale_kernel, dim3(1), dim3(kAppendThreads), 0, stream, x, count, scale);
    return hipGetLastError();
  }
  uint32_t* slot = (uint32_t*)scale;
  hipLaunchKernelGGL(scale_init_kernel, dim3(1), dim3(1), 0, stream, slot);
  if (count > 0) {
    const int64_t want = (count / 8 + kAppendThreads - 1) / kAppendThreads;
    const unsigned blocks = (unsigned)(want < 1 ? 1 : (want > 1024 ? 1024 : want));
    hipLaunchKernelGGL(amax_kernel, dim3(blocks), dim3(kAppendThreads), 0, stream, x, count, slot);
  }
  hipLaunchKernelGGL(scale_finalize_kernel, dim3(1), dim3(1), 0, stream, slot);
  return hipGetLastError();
}

}  // namespace mla
