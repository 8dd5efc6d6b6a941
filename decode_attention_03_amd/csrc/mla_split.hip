// Split-KV MLA decode / verify kernel for gfx950 (MI355X).
//
// One workgroup = (split s, sequence b).  It walks its page range in tiles of
// 4 pages (64 positions):
//
//   a2  paged gather: each wave loads one 16-position page (contiguous in HBM)
//       with 16-byte coalesced loads into registers, one tile ahead, and
//       writes it to LDS as bf16 rows (positions past seq_len or past the
//       split's pages are written as zeros, so nothing outside the visible
//       history can reach an MFMA);
//   a3  FP8 E4M3FN -> bf16 on that LDS write (v_cvt_scalef32_pk_bf16_fp8 with
//       scale 1: exact); the per-tensor kv_scale is applied later in fp32, to
//       the scores and to the output, never to the bf16 operand ("Inside Kimi
//       K3 optimization", technical note on KDA precision: FP32 accumulation
//       cannot recover inputs rounded earlier);
//   a4  QK^T on MFMA (v_mfma_f32_16x16x32_bf16): wave w computes the scores
//       of its page against every query row.  Rows are query tokens x heads,
//       each token's heads padded to 16 rows with zero queries ("Inside Kimi
//       K3 optimization", section "4. MLA"); the query stays in registers for
//       the whole workgroup;
//   a5  causal mask + online softmax in the log2 domain; row maxima and row
//       sums are reduced across lanes with shuffles and across the four waves
//       through LDS;
//   a6  PV on MFMA: the probabilities (bf16) go through LDS and each wave
//       owns 128 of the 512 value columns; the value operand is the same LDS
//       tile read transposed with ds_read_b64_tr_b16, so every KV byte is read
//       from HBM once and serves both products;
//   a7  epilogue: per-split output normalised by its own sum and its
//       natural-log lse (partial mode), or bf16 out + lse directly when the
//       launch has a single split.
//
// MFMA 16x16x32 bf16 lane layout (lane l, g = l / 16):
//   A[m][k]: m = l % 16, k = 8g .. 8g+7;   B[k][n]: n = l % 16, k = 8g .. 8g+7;
//   D[m][n]: n = l % 16, m = 4g .. 4g+3.
// Scores are computed transposed, S^T[t][r] = K[t][:] . Q[r][:], so that a
// lane owns one query row r = l % 16 of four positions t = 4g + i.  The output
// is accumulated transposed as well, O^T[c][r] += V^T[c][t] P^T[t][r], so a
// lane owns one row and four consecutive value columns.
#include <math.h>

#include "mla_common.hpp"

namespace mla {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

#define LDS_PTR(T, p) ((__attribute__((address_space(3))) T*)(p))

constexpr int kRowB = kLatent * 2 + 16;   // LDS bytes per bf16 latent row (+16 B skew)
constexpr int kPRowB = kTilePos * 2 + 16; // LDS bytes per probability row
constexpr int kKSteps = kLatent / 32;     // 18 MFMA k-steps over the 576 dims
constexpr int kColTiles = kValue / kWaves / 16;  // 8 tiles of 16 value columns per wave
constexpr float kNegInf = -__builtin_inff();
constexpr float kLn2 = 0.69314718055994530942f;

__device__ __forceinline__ float wave_max16(float x) {
  // max over lanes l, l^16, l^32, l^48 (the four position groups of one row)
  x = fmaxf(x, __shfl_xor(x, 16));
  x = fmaxf(x, __shfl_xor(x, 32));
  return x;
}

__device__ __forceinline__ float wave_sum16(float x) {
  x += __shfl_xor(x, 16);
  x += __shfl_xor(x, 32);
  return x;
}

// 16 FP8 E4M3FN codes -> 16 bf16 values (exact), as two 16-byte vectors.
__device__ __forceinline__ void fp8x16_to_bf16(u32x4 raw, u32x4& lo, u32x4& hi) {
  uint32_t o[8];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    bf16x2 a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)raw[k], 1.0f, false);
    bf16x2 b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)raw[k], 1.0f, true);
    o[2 * k] = __builtin_bit_cast(uint32_t, a);
    o[2 * k + 1] = __builtin_bit_cast(uint32_t, b);
  }
  lo = u32x4{o[0], o[1], o[2], o[3]};
  hi = u32x4{o[4], o[5], o[6], o[7]};
}

template <int NQ, bool FP8, bool FINAL>
__global__ __launch_bounds__(kThreads, 1) void split_kernel(SplitArgs a) {
  // Query row tiles kept in LDS instead of registers: with bf16 pages the
  // 72-register staging buffer does not fit beside three register-resident
  // query tiles, so the last tile is read from LDS at each k-step instead.
  constexpr int QL = (!FP8 && NQ == 3) ? 1 : 0;
  constexpr int QR = NQ - QL;
  // 16-byte chunks of one page: 576 B (fp8) or 1152 B (bf16) per position.
  constexpr int kEsz = FP8 ? 1 : 2;
  constexpr int kPageBytes = kPage * kLatent * kEsz;
  constexpr int kChunksPerRow = kLatent * kEsz / 16;   // 36 or 72
  constexpr int kChunks = kPageBytes / 16 / 64;        // per lane: 9 or 18

  __shared__ __attribute__((aligned(16))) uint8_t kv_lds[kTilePos * kRowB];
  __shared__ __attribute__((aligned(16))) uint8_t p_lds[NQ * 16 * kPRowB];
  __shared__ float red_max[kWaves][NQ * 16];
  __shared__ float red_sum[kWaves][NQ * 16];
  __shared__ __attribute__((aligned(16))) uint8_t q_lds[QL > 0 ? QL * 16 * kRowB : 16];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = tid >> 6;
  const int g = lane >> 4;
  const int r16 = lane & 15;
  const int split = blockIdx.x;
  const int b = blockIdx.y;

  const int L = a.seq_lens[b];
  const int P = (L + kPage - 1) / kPage;
  const int p0 = (int)(((int64_t)split * P) / a.num_splits);
  const int p1 = (int)(((int64_t)(split + 1) * P) / a.num_splits);
  const int ntiles = (p1 - p0 + kTilePages - 1) / kTilePages;
  const int32_t* pt_row = a.page_table + (int64_t)b * a.max_blocks;

  // ---- query fragments (B operand of S^T = K Q^T): row n = head r16, k = d.
  bf16x8 qf[QR > 0 ? QR : 1][kKSteps];
#pragma unroll
  for (int j = 0; j < QR; ++j) {
    const bool real = r16 < a.heads;
    const uint16_t* qrow = a.q + (((int64_t)b * a.num_q + j) * a.heads + (real ? r16 : 0)) * kLatent;
#pragma unroll
    for (int ks = 0; ks < kKSteps; ++ks) {
      u32x4 v = real ? *(const u32x4*)(qrow + 32 * ks + 8 * g) : u32x4{0, 0, 0, 0};
      qf[j][ks] = __builtin_bit_cast(bf16x8, v);
    }
  }

  if constexpr (QL > 0) {
    // rows 16 * (j - QR) + h of q_lds hold token j >= QR; pad rows are zero.
    for (int c = tid; c < QL * 16 * (kLatent / 8); c += kThreads) {
      const int row = c / (kLatent / 8);
      const int col = c % (kLatent / 8);
      const int j = QR + row / 16, h = row % 16;
      u32x4 v{0, 0, 0, 0};
      if (h < a.heads) v = *(const u32x4*)(a.q + (((int64_t)b * a.num_q + j) * a.heads + h) * kLatent + 8 * col);
      *(u32x4*)(q_lds + row * kRowB + 16 * col) = v;
    }
  }

  float m_run[NQ], l_run[NQ];
  f32x4 o[NQ][kColTiles];
#pragma unroll
  for (int j = 0; j < NQ; ++j) {
    m_run[j] = kNegInf;
    l_run[j] = 0.f;
#pragma unroll
    for (int ct = 0; ct < kColTiles; ++ct) o[j][ct] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  // ---- a2: page gather into registers (one tile ahead).
  u32x4 stg[kChunks];
  auto load_tile = [&](int it) {
    const int page = p0 + it * kTilePages + w;
    if (page < p1) {
      const int blk = pt_row[page];
      const uint8_t* src = a.kv + (int64_t)blk * kPageBytes;
#pragma unroll
      for (int c = 0; c < kChunks; ++c) stg[c] = *(const u32x4*)(src + (lane + 64 * c) * 16);
    }
  };
  auto store_tile = [&](int it) {
    const int page = p0 + it * kTilePages + w;
    const bool have = page < p1;
    const int valid_rows = have ? min(kPage, L - page * kPage) : 0;
#pragma unroll
    for (int c = 0; c < kChunks; ++c) {
      const int chunk = lane + 64 * c;
      const int row = chunk / kChunksPerRow;
      const int col = chunk % kChunksPerRow;
      const bool ok = row < valid_rows;
      uint8_t* dst = kv_lds + (w * kPage + row) * kRowB;
      if constexpr (FP8) {
        u32x4 lo, hi;
        fp8x16_to_bf16(stg[c], lo, hi);
        const u32x4 z{0, 0, 0, 0};
        *(u32x4*)(dst + col * 32) = ok ? lo : z;
        *(u32x4*)(dst + col * 32 + 16) = ok ? hi : z;
      } else {
        *(u32x4*)(dst + col * 16) = ok ? stg[c] : u32x4{0, 0, 0, 0};
      }
    }
  };

  if (ntiles > 0) load_tile(0);

  for (int it = 0; it < ntiles; ++it) {
    __syncthreads();  // previous tile's readers are done with kv_lds / p_lds / red_sum
    store_tile(it);
    if (it + 1 < ntiles) load_tile(it + 1);
    __syncthreads();  // tile visible to all waves

    // ---- a4: S^T for this wave's page, all query rows.
    f32x4 sacc[NQ];
#pragma unroll
    for (int j = 0; j < NQ; ++j) sacc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
    const uint8_t* krow = kv_lds + (w * kPage + r16) * kRowB + 16 * g;
#pragma unroll
    for (int ks = 0; ks < kKSteps; ++ks) {
      const bf16x8 kf = *(const bf16x8*)(krow + 64 * ks);
#pragma unroll
      for (int j = 0; j < QR; ++j)
        sacc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf, qf[j][ks], sacc[j], 0, 0, 0);
#pragma unroll
      for (int j = QR; j < NQ; ++j) {
        const bf16x8 qv = *(const bf16x8*)(q_lds + ((j - QR) * 16 + r16) * kRowB + 16 * g + 64 * ks);
        sacc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf, qv, sacc[j], 0, 0, 0);
      }
    }

    // ---- a5: mask, scale (log2 domain), tile row maxima.
    const int page = p0 + it * kTilePages + w;
    const int t0 = page * kPage + 4 * g;
    float sv[NQ][4];
#pragma unroll
    for (int j = 0; j < NQ; ++j) {
      const int lim = (page < p1) ? (L - a.num_q + j + 1) : 0;  // visible: t < lim
      float mx = kNegInf;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        sv[j][i] = (t0 + i < lim) ? sacc[j][i] * a.score_scale_log2 : kNegInf;
        mx = fmaxf(mx, sv[j][i]);
      }
      mx = wave_max16(mx);
      if (g == 0) red_max[w][j * 16 + r16] = mx;
    }
    __syncthreads();

    float alpha[NQ];
#pragma unroll
    for (int j = 0; j < NQ; ++j) {
      float mt = red_max[0][j * 16 + r16];
#pragma unroll
      for (int ww = 1; ww < kWaves; ++ww) mt = fmaxf(mt, red_max[ww][j * 16 + r16]);
      const float m_new = fmaxf(m_run[j], mt);
      alpha[j] = (m_new == kNegInf) ? 1.f : __builtin_amdgcn_exp2f(m_run[j] - m_new);
      bf16x4 pb;
      float ps = 0.f;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float p = (sv[j][i] == kNegInf) ? 0.f : __builtin_amdgcn_exp2f(sv[j][i] - m_new);
        pb[i] = (__bf16)p;
        ps += p;  // fp32 weights: lse stays exact to fp32; the bf16 rounding of the
                  // MFMA operand only perturbs the output, unbiased (RNE)
      }
      ps = wave_sum16(ps);
      if (g == 0) red_sum[w][j * 16 + r16] = ps;
      *(bf16x4*)(p_lds + (j * 16 + r16) * kPRowB + (w * kPage + 4 * g) * 2) = pb;
      m_run[j] = m_new;
    }
    __syncthreads();

#pragma unroll
    for (int j = 0; j < NQ; ++j) {
      float ts = 0.f;
#pragma unroll
      for (int ww = 0; ww < kWaves; ++ww) ts += red_sum[ww][j * 16 + r16];
      l_run[j] = l_run[j] * alpha[j] + ts;
#pragma unroll
      for (int ct = 0; ct < kColTiles; ++ct) o[j][ct] *= alpha[j];
    }

    // ---- a6: O^T[c][r] += V^T[c][t] P^T[t][r] over the tile's 64 positions.
#pragma unroll
    for (int kk = 0; kk < kTilePos / 32; ++kk) {
      bf16x8 pf[NQ];
#pragma unroll
      for (int j = 0; j < NQ; ++j)
        pf[j] = *(const bf16x8*)(p_lds + (j * 16 + r16) * kPRowB + (32 * kk + 8 * g) * 2);
      // transposed read: lane s of a 16-lane group loads row (s / 4) and
      // columns 4 * (s % 4) .. +3 of a 4 x 16 block; afterwards lane i holds
      // column i of the four rows.
      const int vrow = 32 * kk + 8 * g + (r16 >> 2);
      const uint8_t* vbase = kv_lds + vrow * kRowB + (w * (kValue / kWaves) + 4 * (lane & 3)) * 2;
#pragma unroll
      for (int ct = 0; ct < kColTiles; ++ct) {
        const i16x4 v0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(LDS_PTR(i16x4, vbase + ct * 32));
        const i16x4 v1 =
            __builtin_amdgcn_ds_read_tr16_b64_v4i16(LDS_PTR(i16x4, vbase + 4 * kRowB + ct * 32));
        const u32x2 u0 = __builtin_bit_cast(u32x2, v0);
        const u32x2 u1 = __builtin_bit_cast(u32x2, v1);
        const bf16x8 vf = __builtin_bit_cast(bf16x8, u32x4{u0[0], u0[1], u1[0], u1[1]});
#pragma unroll
        for (int j = 0; j < NQ; ++j)
          o[j][ct] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf, pf[j], o[j][ct], 0, 0, 0);
      }
    }
  }

  // ---- a7: epilogue (real rows only).
  const int h = r16;
  if (h < a.heads) {
#pragma unroll
    for (int j = 0; j < NQ; ++j) {
      const bool any = l_run[j] > 0.f;
      const float lse_v = any ? (m_run[j] + log2f(l_run[j])) * kLn2 : kNegInf;
      const float sc = any ? a.out_scale / l_run[j] : 0.f;
      const int64_t row = ((int64_t)b * a.num_q + j) * a.heads + h;
      if constexpr (FINAL) {
        uint16_t* dst = a.out + row * kValue + w * (kValue / kWaves) + 4 * g;
#pragma unroll
        for (int ct = 0; ct < kColTiles; ++ct) {
          bf16x4 ov;
#pragma unroll
          for (int i = 0; i < 4; ++i) ov[i] = (__bf16)(o[j][ct][i] * sc);
          *(bf16x4*)(dst + 16 * ct) = ov;
        }
        if (w == 0 && g == 0) a.lse[row] = lse_v;
      } else {
        const int64_t prow = (int64_t)split * a.batch * a.num_q * a.heads + row;
        float* dst = a.part_out + prow * kValue + w * (kValue / kWaves) + 4 * g;
#pragma unroll
        for (int ct = 0; ct < kColTiles; ++ct) *(f32x4*)(dst + 16 * ct) = o[j][ct] * sc;
        if (w == 0 && g == 0) a.part_lse[prow] = lse_v;
      }
    }
  }
}

template <int NQ, bool FP8>
hipError_t launch_nq(const SplitArgs& a, bool final_out, hipStream_t stream) {
  dim3 grid(a.num_splits, a.batch);
  if (final_out)
    hipLaunchKernelGGL((split_kernel<NQ, FP8, true>), grid, dim3(kThreads), 0, stream, a);
  else
    hipLaunchKernelGGL((split_kernel<NQ, FP8, false>), grid, dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

template <bool FP8>
hipError_t launch_dtype(const SplitArgs& a, bool final_out, hipStream_t stream) {
  switch (a.num_q) {
    case 1: return launch_nq<1, FP8>(a, final_out, stream);
    case 2: return launch_nq<2, FP8>(a, final_out, stream);
    case 3: return launch_nq<3, FP8>(a, final_out, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_split(const SplitArgs& a, bool fp8, bool final_out, hipStream_t stream) {
  return fp8 ? launch_dtype<true>(a, final_out, stream) : launch_dtype<false>(a, final_out, stream);
}

}  // namespace mla
