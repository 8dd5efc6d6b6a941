// Log-sum-exp merge of split-KV partials (gfx950).
//
// Each partial carries its normaliser, so the pieces of one history can be
// weighted correctly when they are combined ("Inside Kimi K3 optimization",
// sections "1. Cache -- DCP" and "4. MLA"):
//   lse = ln sum_s exp(lse_s),  out = sum_s exp(lse_s - lse) * o_s  -> bf16 (RNE).
//
// HBM-bound: one wave64 per (row, 256-column half); each lane owns 4 columns
// and streams the S partial rows with 16-byte loads.
#include <math.h>

#include "mla_common.hpp"

namespace mla {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));

constexpr float kNegInf = -__builtin_inff();

__global__ __launch_bounds__(64) void merge_kernel(MergeArgs a) {
  const int64_t row = (int64_t)blockIdx.x >> 1;
  const int col = (blockIdx.x & 1) * 256 + threadIdx.x * 4;
  const int S = a.num_splits;
  const float* lse_p = a.part_lse + row;

  float m = kNegInf;
  for (int s = 0; s < S; ++s) m = fmaxf(m, lse_p[(int64_t)s * a.rows]);

  f32x4 acc{0.f, 0.f, 0.f, 0.f};
  float wsum = 0.f;
  if (m != kNegInf) {
    const float* po = a.part_out + row * kValue + col;
#pragma unroll 4
    for (int s = 0; s < S; ++s) {
      const float ls = lse_p[(int64_t)s * a.rows];
      const float wgt = (ls == kNegInf) ? 0.f : expf(ls - m);
      const f32x4 v = *(const f32x4*)(po + (int64_t)s * a.rows * kValue);
      wsum += wgt;
      acc += wgt * v;
    }
  }
  const float inv = (wsum > 0.f) ? 1.f / wsum : 0.f;
  bf16x4 ov;
#pragma unroll
  for (int i = 0; i < 4; ++i) ov[i] = (__bf16)(acc[i] * inv);
  *(bf16x4*)(a.out + row * kValue + col) = ov;
  if (threadIdx.x == 0 && (blockIdx.x & 1) == 0) a.lse[row] = (wsum > 0.f) ? m + logf(wsum) : kNegInf;
}

}  // namespace

hipError_t launch_merge(const MergeArgs& a, hipStream_t stream) {
  hipLaunchKernelGGL(merge_kernel, dim3((unsigned)(a.rows * 2)), dim3(64), 0, stream, a);
  return hipGetLastError();
}

}  // namespace mla
