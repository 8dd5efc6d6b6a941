// Log-sum-exp merge of split-KV partials (gfx950).
//
// Each partial carries its normaliser, so the pieces of one history can be
// weighted correctly when they are combined ("Inside Kimi K3 optimization",
// sections "1. Cache -- DCP" and "4. MLA"):
//   lse = ln sum_s exp(lse_s),  out = sum_s exp(lse_s - lse) * o_s  -> bf16 (RNE).
//
// HBM-bound streaming.  One 256-thread workgroup per (row, 256-column half):
//   1. the weights exp(lse_s - max) of all S partials are computed once into
//      LDS (block-wide max and sum reductions);
//   2. 64 column chunks (4 floats) x 4 split lanes stream the partial rows
//      with independent 16-byte loads, and the 4 lanes are summed in LDS.
#include <math.h>

#include "mla_common.hpp"

namespace mla {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));

constexpr float kNegInf = -__builtin_inff();
constexpr int kMergeThreads = 256;
constexpr int kSplitLanes = kMergeThreads / 64;   // 4
constexpr int kMaxCoef = 4096;                     // largest split count (the API bound)

__device__ __forceinline__ float block_max(float v, float* red) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v = fmaxf(v, __shfl_xor(v, m));
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  v = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  __syncthreads();
  return v;
}

__device__ __forceinline__ float block_sum(float v, float* red) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  v = (red[0] + red[1]) + (red[2] + red[3]);
  __syncthreads();
  return v;
}

__global__ __launch_bounds__(kMergeThreads) void merge_kernel(MergeArgs a) {
  __shared__ float coef[kMaxCoef];
  __shared__ float red[4];
  __shared__ __attribute__((aligned(16))) f32x4 part[kSplitLanes][64];

  const int64_t row = (int64_t)blockIdx.x >> 1;
  const int half = blockIdx.x & 1;
  const int tid = threadIdx.x;
  const int S = a.num_splits;

  float m = kNegInf;
  for (int s = tid; s < S; s += kMergeThreads) m = fmaxf(m, a.part_lse[(int64_t)s * a.rows + row]);
  m = block_max(m, red);

  float wsum = 0.f;
  for (int s = tid; s < S; s += kMergeThreads) {
    const float ls = a.part_lse[(int64_t)s * a.rows + row];
    const float wgt = (ls == kNegInf) ? 0.f : expf(ls - m);
    coef[s] = wgt;
    wsum += wgt;
  }
  wsum = block_sum(wsum, red);   // its barriers also publish coef[]

  const int chunk = tid & 63;         // 4-float column chunk inside this half
  const int lane_s = tid >> 6;        // split lane
  const int col = half * 256 + 4 * chunk;
  f32x4 acc{0.f, 0.f, 0.f, 0.f};
  if (m != kNegInf) {
    const float* po = a.part_out + row * kValue + col;
#pragma unroll 4
    for (int s = lane_s; s < S; s += kSplitLanes) {
      const float wgt = coef[s];
      if (wgt != 0.f) {   // uniform branch: an empty partial is never read
        const f32x4 v = *(const f32x4*)(po + (int64_t)s * a.rows * kValue);
        acc += wgt * v;
      }
    }
  }
  part[lane_s][chunk] = acc;
  __syncthreads();
  if (lane_s == 0) {
    const f32x4 t = (part[0][chunk] + part[1][chunk]) + (part[2][chunk] + part[3][chunk]);
    const float inv = (wsum > 0.f) ? 1.f / wsum : 0.f;
    bf16x4 ov;
#pragma unroll
    for (int i = 0; i < 4; ++i) ov[i] = (__bf16)(t[i] * inv);
    *(bf16x4*)(a.out + row * kValue + col) = ov;
    if (tid == 0 && half == 0) a.lse[row] = (wsum > 0.f) ? m + logf(wsum) : kNegInf;
  }
}

}  // namespace

hipError_t launch_merge(const MergeArgs& a, hipStream_t stream) {
  hipLaunchKernelGGL(merge_kernel, dim3((unsigned)(a.rows * 2)), dim3(kMergeThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace mla
