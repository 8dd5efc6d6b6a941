// Log-sum-exp merge of split-KV partials (gfx950).
//
// Each partial carries its normaliser, so the pieces of one history can be
// weighted correctly when they are combined ("Inside Kimi K3 optimization",
// sections "1. Cache -- DCP" and "4. MLA"):
//   lse = ln sum_s exp(lse_s),  out = sum_s exp(lse_s - lse) * o_s  -> bf16 (RNE).
//
// HBM-bound streaming of S partial rows per output row.  A 256-thread
// workgroup holds one or more row slices; in each, LANES split lanes x
// COLS/4 column chunks (4 floats) stream the partials with up to eight
// independent 8-byte loads (four bf16 partial values) in flight per thread:
//   S <= 8:  1 lane,  whole rows, two rows per workgroup
//   S <= 32: 2 lanes, whole rows, one row per workgroup
//   S > 32:  8 lanes, 128-column quarters, four workgroups per row
// Per row slice, the weights exp(lse_s - max) are computed once into LDS
// (S floats of dynamic LDS per slice), and the lanes are summed in LDS.  The
// first round of partial loads is issued before the lse loads and their
// reductions (it does not depend on the weights), so the two memory
// latencies overlap; with S <= 8 LANES that round is all of them.
#include <math.h>

#include "mla_common.hpp"

namespace mla {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kNegInf = -__builtin_inff();
constexpr int kMergeThreads = 256;
constexpr int kInFlight = 8;   // loads per thread per round

// max / sum over the WPR waves of one row slice (waves w0 .. w0 + WPR - 1)
template <int WPR, bool MAX>
__device__ __forceinline__ float slice_reduce(float v, float* red) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) {
    const float o = __shfl_xor(v, m);
    v = MAX ? fmaxf(v, o) : v + o;
  }
  const int w = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) red[w] = v;
  __syncthreads();
  const int w0 = w / WPR * WPR;
  v = red[w0];
#pragma unroll
  for (int i = 1; i < WPR; ++i) v = MAX ? fmaxf(v, red[w0 + i]) : v + red[w0 + i];
  __syncthreads();
  return v;
}

template <int LANES, int COLS>
__global__ __launch_bounds__(kMergeThreads) void merge_kernel(MergeArgs a) {
  constexpr int kChunks = COLS / 4;
  constexpr int kTPR = LANES * kChunks;        // threads per row slice
  constexpr int kRPW = kMergeThreads / kTPR;   // row slices per workgroup
  constexpr int kSlices = kValue / COLS;       // workgroups per row
  constexpr int kWPR = kTPR / 64;              // waves per row slice
  static_assert(kTPR % 64 == 0 && kRPW * kTPR == kMergeThreads, "merge shape");
  extern __shared__ float coef[];              // [kRPW][S]
  __shared__ float red[kMergeThreads / 64];
  __shared__ __attribute__((aligned(16))) f32x4 part[kMergeThreads];

  const int tid = threadIdx.x;
  const int rs = tid / kTPR;
  const int t = tid % kTPR;
  const int64_t row = ((int64_t)blockIdx.x / kSlices) * kRPW + rs;
  const int slice = (int)(blockIdx.x % kSlices);
  const bool live = row < a.rows;
  const int64_t lrow = live ? row : 0;
  // the row's partials: S of them, partial s at row pbase + s * pstride of
  // part_out / part_lse (with the plan by length, the slots of the row's
  // sequence; every wave of a row slice computes the plan for that sequence)
  int S = a.num_splits;
  int64_t pbase = lrow, pstride = a.rows;
  int cstride = a.num_splits;   // floats of coef per row slice
  if (a.by_length) {
    const int R = a.rows_per_seq;
    const int bq = (int)(lrow / R);
    const SeqSlots ss = balanced_plan(a.seq_lens, a.batch, a.num_splits, a.max_blocks, bq, false);
    S = ss.count;
    pbase = (int64_t)ss.first * R + (lrow - (int64_t)bq * R);
    pstride = R;
    cstride = a.num_splits * a.batch - a.batch + 1;   // the most slots one sequence can own
  }
  float* cf = coef + rs * cstride;

  const int chunk = t % kChunks;
  const int lane_s = t / kChunks;
  const int col = slice * COLS + 4 * chunk;
  const uint16_t* const po = a.part_out + pbase * kValue + col;
  const int64_t stride = pstride * kValue;
  // lse of split t (the first of this thread's), kept for the weights; issued
  // first, so that waiting for it leaves the partial loads below in flight
  // (loads retire from the wait counter in issue order)
  const float ls_t = a.part_lse[pbase + (int64_t)min(t, S - 1) * pstride];
  // first round of partial loads (splits lane_s + LANES u), in flight during
  // the lse reductions.  The loads are unconditional (split index clamped to
  // S - 1, row 0 for a dead slice: the buffer holds all of those partials), so
  // no branch with its own wait sits between them; a split past S, like an
  // empty one, has weight zero below and its value is not used.
  // The partial loads are non-temporal: each partial is read once, and
  // kept out of the L2 it leaves room for the next launch's stream
  // (long-context layer-step -2.5%, same box; timed alone, with the same
  // partials re-read launch after launch, this kernel looks slower so).
  u32x2 v[kInFlight];   // four bf16 each
#pragma unroll
  for (int u = 0; u < kInFlight; ++u)
    v[u] = __builtin_nontemporal_load((const u32x2*)(po + (int64_t)min(lane_s + LANES * u, S - 1) * stride));

  // (selected only here, after the partial loads have been issued)
  const float ls0 = (live && t < S) ? ls_t : kNegInf;
  float m = ls0;
  if (live)
    for (int s = t + kTPR; s < S; s += kTPR) m = fmaxf(m, a.part_lse[pbase + (int64_t)s * pstride]);
  m = slice_reduce<kWPR, true>(m, red);

  float wsum = 0.f;
  if (live)
    for (int s = t; s < S; s += kTPR) {
      const float ls = s == t ? ls0 : a.part_lse[pbase + (int64_t)s * pstride];
      const float wgt = (ls == kNegInf) ? 0.f : expf(ls - m);
      cf[s] = wgt;
      wsum += wgt;
    }
  wsum = slice_reduce<kWPR, false>(wsum, red);   // its barriers also publish coef[]

  f32x4 acc{0.f, 0.f, 0.f, 0.f};
  if (live && m != kNegInf) {
    for (int s0 = lane_s; s0 < S; s0 += LANES * kInFlight) {
      if (s0 != lane_s) {   // later rounds (S > LANES * kInFlight)
#pragma unroll
        for (int u = 0; u < kInFlight; ++u)
          v[u] = __builtin_nontemporal_load((const u32x2*)(po + (int64_t)min(s0 + LANES * u, S - 1) * stride));
      }
#pragma unroll
      for (int u = 0; u < kInFlight; ++u) {
        const int s = s0 + LANES * u;
        const float wgt = s < S ? cf[s] : 0.f;
        // a partial of weight zero (empty split) contributes nothing, whatever it holds
        if (wgt != 0.f) {
          const f32x4 f{__uint_as_float(v[u][0] << 16), __uint_as_float(v[u][0] & 0xFFFF0000u),
                        __uint_as_float(v[u][1] << 16), __uint_as_float(v[u][1] & 0xFFFF0000u)};
          acc += wgt * f;
        }
      }
    }
  }
  if constexpr (LANES > 1) {
    part[tid] = acc;
    __syncthreads();
    if (lane_s == 0) {
#pragma unroll
      for (int l = 1; l < LANES; ++l) acc += part[tid + l * kChunks];
    }
  }
  if (live && lane_s == 0) {
    const float inv = (wsum > 0.f) ? 1.f / wsum : 0.f;
    bf16x4 ov;
#pragma unroll
    for (int i = 0; i < 4; ++i) ov[i] = (__bf16)(acc[i] * inv);
    *(bf16x4*)(a.out + row * kValue + col) = ov;
    if (t == 0 && slice == 0) a.lse[row] = (wsum > 0.f) ? m + logf(wsum) : kNegInf;
  }
}

// Shape by the split count of a row.  With the plan by length the rows of the
// longest sequences, which set the time, hold about twice the average: up to
// 16 on average that moves the shape to two lanes per chunk (bf16 decode of
// 32 sequences of 1,024..8,192 positions, 8 splits:
// 5.7 -> 5.1 us); at 32 the whole-row shape stays the faster one (bf16 verify
// of 32 sequences, 4,096..32,768 positions: 11.9 us
// against 14.2 for quarter rows).
int shape_splits(const MergeArgs& a) {
  return (a.by_length && a.num_splits <= 16) ? 2 * a.num_splits : a.num_splits;
}

template <int LANES, int COLS>
hipError_t launch_shape(const MergeArgs& a, hipStream_t stream) {
  constexpr int kRPW = kMergeThreads / (LANES * COLS / 4);
  const int64_t groups = (a.rows + kRPW - 1) / kRPW;
  const int cstride = a.by_length ? a.num_splits * a.batch - a.batch + 1 : a.num_splits;
  const size_t lds = (size_t)kRPW * cstride * sizeof(float);
  hipLaunchKernelGGL((merge_kernel<LANES, COLS>), dim3((unsigned)(groups * (kValue / COLS))),
                     dim3(kMergeThreads), lds, stream, a);
  return hipGetLastError();
}

}  // namespace

int64_t merge_work_items(const MergeArgs& a) {
  // the grids of launch_shape for the shapes launch_merge picks
  const int s = shape_splits(a);
  if (s <= 8) return (a.rows + 1) / 2 * kMergeThreads;   // two rows per workgroup
  if (s <= 32) return a.rows * kMergeThreads;            // one row per workgroup
  return a.rows * 4 * kMergeThreads;                     // four quarters per row
}

hipError_t launch_merge(const MergeArgs& a, hipStream_t stream) {
  const int s = shape_splits(a);
  if (s <= 8) return launch_shape<1, 512>(a, stream);
  if (s <= 32) return launch_shape<2, 512>(a, stream);
  return launch_shape<8, 128>(a, stream);
}

}  // namespace mla
