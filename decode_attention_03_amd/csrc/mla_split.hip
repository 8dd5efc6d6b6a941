// Split-KV MLA decode / verify kernel for gfx950 (MI355X).
//
// One workgroup (4 wave64s, one per SIMD) = (split s, sequence b).  It walks
// its page range in tiles of 4 pages (64 positions):
//
//   a2  paged gather: each wave copies one 16-position page (contiguous in
//       HBM) straight into LDS with 16-byte buffer_load_dwordx4 ... lds (no
//       register staging), NBUF - 1 tiles ahead of the tile being computed
//       (three buffers for FP8, two for bf16).  16-byte chunks are XOR-swizzled
//       inside each latent row to spread LDS banks.  Positions past seq_len
//       and pages past the split's range are zeroed in LDS, so nothing outside
//       the visible history can reach an MFMA;
//   a3  FP8 E4M3FN stays FP8 in LDS and is decoded exactly to bf16 right after
//       each LDS read (v_cvt_scalef32_pk_bf16_fp8 with scale 1); the
//       per-tensor kv_scale is applied in fp32 to the scores and to the
//       output, never to the bf16 operand ("Inside Kimi K3 optimization",
//       technical note on KDA precision: FP32 accumulation cannot recover
//       inputs rounded earlier);
//   a4  QK^T on MFMA.  Query rows are (token j, head h) packed as r = j*H + h.
//       With more than 16 rows (speculative verify), rows 0..31 form a 32-row
//       tile computed with v_mfma_f32_32x32x16_bf16 and rows 32..47 a 16-row
//       tile computed with v_mfma_f32_16x16x32_bf16: 36 real rows cost 48
//       padded rows, the 32x32 shape running ~1.6x more flops per cycle than
//       16x16.  Zero query rows stand in for the padding ("Inside Kimi K3
//       optimization", section "4. MLA").  Waves 0/1 own the 32-row tile over
//       the two 32-position halves of the tile, waves 2/3 the 16-row tile; the
//       query fragments stay in registers for the whole workgroup.  With at
//       most 16 rows (decode), every wave owns one page against one 16-row tile;
//   a5  causal mask + online softmax in the log2 domain; row maxima and row
//       sums are reduced across lanes with shuffles and across waves in LDS;
//   a6  PV on MFMA: probabilities (bf16) go through LDS; each wave owns 128 of
//       the 512 value columns for every row; the value operand is the same LDS
//       tile read transposed (ds_read_b64_tr_b8 for FP8, ds_read_b64_tr_b16
//       for bf16), so every KV byte crosses HBM once and serves both products;
//   a7  epilogue: per-split output normalised by its own sum plus its
//       natural-log lse (partial mode), or bf16 out + lse when the launch has a
//       single split.
//
// MFMA lane layouts (lane l):
//   16x16x32: A[m][k] m = l%16, k = 8(l/16)+j;  B[k][n] n = l%16, same k;
//             D[m][n] n = l%16, m = 4(l/16)+i.
//   32x32x16: A[m][k] m = l%32, k = 8(l/32)+j;  B[k][n] n = l%32, same k;
//             D[m][n] n = l%32, m = 8(i/4) + 4(l/32) + i%4, i = 0..15.
// Scores are computed transposed, S^T = K Q^T (a lane owns one query row), and
// so is the output, O^T += V^T P^T (a lane owns one row and 4-column runs).
#include <math.h>

#include <type_traits>

#include "mla_common.hpp"

namespace mla {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef int i32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x8 __attribute__((ext_vector_type(8)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

#define LDS_PTR(T, p) ((__attribute__((address_space(3))) T*)(p))

constexpr int kLayout16 = 0;   // at most 16 query rows: one 16-row tile
constexpr int kLayout48 = 1;   // 17..48 query rows: a 32-row tile + a 16-row tile
constexpr float kNegInf = -__builtin_inff();
constexpr float kLn2 = 0.69314718055994530942f;

// s_waitcnt immediates (gfx9 encoding: vmcnt[3:0] and [15:14], expcnt[6:4], lgkmcnt[11:8]).
constexpr int waitcnt_vm(int n) { return (n & 0xF) | ((n >> 4) << 14) | (0x7 << 4) | (0xF << 8); }
constexpr int kWaitLgkm0 = 0xF | (0x3 << 14) | (0x7 << 4);
// Word 3 of a raw (untyped, stride 0) buffer resource on gfx9-family GPUs.
constexpr int kBufferRsrcWord3 = 0x00020000;

// Workgroup -> (split, sequence, query-row block) over a one-dimensional grid.
// Units u = split + S * sequence in id order, so the splits of one sequence
// (which read the same query rows) start together on all XCDs.  With several
// row blocks, which read the same pages, the row blocks of a unit are kept on
// one XCD back to back: consecutive ids go to the eight XCDs in turn (each
// with its own L2), so XCD x's k-th id takes row block k % Z of its unit
// 8 (k / Z) + x; this is a bijection when the unit count is a multiple of 8,
// else the row block is simply the slowest index.
struct WgCoord {
  int split, b, z;
};
__device__ __forceinline__ WgCoord wg_coord(int num_splits, int batch, int row_blocks) {
  const int id = (int)blockIdx.x;
  const int units = num_splits * batch;
  int u, z;
  if (row_blocks > 1 && (units & 7) == 0) {
    const int k = id >> 3;
    u = ((k / row_blocks) << 3) + (id & 7);
    z = k % row_blocks;
  } else {
    u = id % units;
    z = id / units;
  }
  WgCoord c;
  c.split = u % num_splits;
  c.b = u / num_splits;
  c.z = z;
  return c;
}

// Workgroup barrier for LDS data written with ds_write: drain this wave's LDS
// traffic, then s_barrier.  (No memory fence: the direct-to-LDS loads are
// waited for explicitly with vmcnt, so no blanket vmcnt(0) is wanted here.)
__device__ __forceinline__ void lds_barrier() {
  asm volatile("" ::: "memory");   // compiler-only: no LDS access moves across
  __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

__device__ __forceinline__ float xor_max(float x, int m) { return fmaxf(x, __shfl_xor(x, m)); }
// x combined with the value of lane l ^ 32 (a VALU lane swap, no LDS round trip)
__device__ __forceinline__ float max32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float xor_sum(float x, int m) { return x + __shfl_xor(x, m); }

// 8 FP8 E4M3FN codes (two dwords) -> 8 bf16 (exact).
__device__ __forceinline__ bf16x8 fp8x8_to_bf16(u32x2 raw) {
  const bf16x2 a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)raw[0], 1.0f, false);
  const bf16x2 b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)raw[0], 1.0f, true);
  const bf16x2 c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)raw[1], 1.0f, false);
  const bf16x2 d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)raw[1], 1.0f, true);
  return bf16x8{a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
}

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

__device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

template <bool FP8>
struct KvGeom {
  static constexpr int kEsz = FP8 ? 1 : 2;
  static constexpr int kRowB = kLatent * kEsz;        // bytes per position (HBM and LDS)
  static constexpr int kChunksPerRow = kRowB / 16;    // 36 or 72
  static constexpr int kPageB = kPage * kRowB;        // 9216 or 18432
  static constexpr int kLoadsPerPage = kPageB / 1024; // wave-wide 1 KiB DMA loads: 9 or 18
  static constexpr int kTileB = kTilePages * kPageB;
  static constexpr int kNBuf = FP8 ? 3 : 2;
  // XOR applied to the 16-byte chunk index of a row.  Rows are 144 (FP8) or
  // 288 (bf16) dwords apart, so rows r and r+4 (FP8) or r and r+2 (bf16) start
  // on the same LDS bank; the XOR separates exactly those rows, which makes a
  // 16-lane access to one chunk of 16 consecutive rows conflict-free.
  static __device__ __forceinline__ int swz(int row) { return FP8 ? (row >> 2) & 3 : (row >> 1) & 7; }
  // LDS byte offset (inside a page) of byte `inner` of logical 16-byte chunk x of row `row`.
  static __device__ __forceinline__ int off(int row, int x, int inner) {
    return (row * kChunksPerRow + (x ^ swz(row))) * 16 + inner;
  }
};

// Raw value operand: 8 consecutive positions t0..t0+7 of column (cb + lane % 16),
// from a 16-lane group's transposed LDS read; vop() converts it.  `tile` is
// the LDS tile base, t0 a multiple of 8, cb a multiple of 16, s = lane % 16.
template <bool FP8>
__device__ __forceinline__ typename std::conditional<FP8, u32x2, u32x4>::type load_v8(
    const uint8_t* tile, int t0, int cb, int s) {
  using G = KvGeom<FP8>;
  if constexpr (FP8) {
    // source lane s: position t0 + s/2, byte half s%2 of the 16 columns cb..cb+15
    const int t = t0 + (s >> 1);
    const uint8_t* p = tile + (t >> 4) * G::kPageB + G::off(t & 15, cb >> 4, 8 * (s & 1));
    return __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr8_b64_v2i32(LDS_PTR(i32x2, p)));
  } else {
    // source lane s: position t0 + s/4 (and +4), columns cb + 4(s%4) .. +3
    const int cbyte = 2 * cb + 8 * (s & 3);
    const int t = t0 + (s >> 2);
    const uint8_t* p0 = tile + (t >> 4) * G::kPageB + G::off(t & 15, cbyte >> 4, cbyte & 15);
    const int t4 = t + 4;
    const uint8_t* p1 = tile + (t4 >> 4) * G::kPageB + G::off(t4 & 15, cbyte >> 4, cbyte & 15);
    const u32x2 u0 = __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16(LDS_PTR(i16x4, p0)));
    const u32x2 u1 = __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16(LDS_PTR(i16x4, p1)));
    return u32x4{u0[0], u0[1], u1[0], u1[1]};
  }
}

// Raw key operand: dims d0..d0+7 (d0 a multiple of 8) of position `row` of
// `page`: 8 FP8 bytes or 8 bf16 values, converted by kop() right before use so
// the LDS latency overlaps the previous MFMAs.
template <bool FP8>
struct KRaw {
  using T = typename std::conditional<FP8, u32x2, u32x4>::type;
};
template <bool FP8>
__device__ __forceinline__ typename KRaw<FP8>::T load_k8(const uint8_t* page, int row, int d0) {
  using G = KvGeom<FP8>;
  const int byte = d0 * G::kEsz;
  return *(const typename KRaw<FP8>::T*)(page + G::off(row, byte >> 4, byte & 15));
}
__device__ __forceinline__ bf16x8 kop(u32x2 raw) { return fp8x8_to_bf16(raw); }
__device__ __forceinline__ bf16x8 kop(u32x4 raw) { return as_bf16x8(raw); }

// Software-pipelined operand stream: load(i) issues the LDS read of step i,
// use(i, raw) converts and consumes it.  Steps are grouped GRP at a time; the
// reads of group n+1 are issued before the MFMAs of group n, and a scheduling
// barrier keeps the compiler from hoisting further reads (register pressure).
template <int N, int GRP, typename Raw, typename LoadF, typename UseF>
__device__ __forceinline__ void pipelined(LoadF&& load, UseF&& use) {
  static_assert(N % GRP == 0, "group size must divide the step count");
  Raw cur[GRP], nxt[GRP];
#pragma unroll
  for (int j = 0; j < GRP; ++j) cur[j] = load(j);
#pragma unroll
  for (int gi = 0; gi < N / GRP; ++gi) {
    if (gi + 1 < N / GRP) {
#pragma unroll
      for (int j = 0; j < GRP; ++j) nxt[j] = load((gi + 1) * GRP + j);
    }
#pragma unroll
    for (int j = 0; j < GRP; ++j) use(gi * GRP + j, cur[j]);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int j = 0; j < GRP; ++j) cur[j] = nxt[j];
  }
}

template <int LAYOUT, bool FP8, bool FINAL>
__global__ __launch_bounds__(kThreads, 1) void split_kernel(SplitArgs a) {
#if defined(__HIP_DEVICE_COMPILE__)  // the host pass only needs the launch stub
  using G = KvGeom<FP8>;
  using KR = typename KRaw<FP8>::T;
  constexpr bool L16 = LAYOUT == kLayout16;
  // Tile: 64 positions (4 pages), except 32 (2 pages) for bf16 with 48 rows,
  // where LDS holds three bf16 tiles plus the partial-score exchange.
  constexpr int TP = (!L16 && !FP8) ? 32 : 64;
  constexpr int TPG = TP / kPage;                  // pages per tile
  constexpr int kTileB = TPG * G::kPageB;
  constexpr int kNBuf = L16 ? G::kNBuf : 3;
  constexpr int kWaveLoads = kTileB / kWaves / 1024;   // 1 KiB DMA loads per wave per tile (9 or 18)
  constexpr int RPAD = L16 ? 16 : 48;
  constexpr int kPRB = TP * 2 + 16;                // LDS bytes per probability row
  constexpr int NS32 = TP / 32;                    // 32-position sub-tiles of the 32-row tile
  constexpr int NS16 = TP / 16;                    // 16-position sub-tiles of the 16-row tile
  constexpr int kQRegs = 18;                       // query fragments held per wave
  constexpr int kXFloats = L16 ? 1 : 16 * NS32;    // partial scores exchanged per lane
  // Lazy rescale: a row's reference maximum moves only when a tile maximum
  // exceeds it by more than 2^kSlack (bf16 probabilities up to 2^8 are exact
  // enough and far from overflow), which skips most output rescales.
  constexpr float kSlack = 8.f;

  __shared__ __attribute__((aligned(16))) uint8_t kv_lds[kNBuf * kTileB];
  __shared__ __attribute__((aligned(16))) uint8_t p_lds[RPAD * kPRB];
  __shared__ float red_max[kWaves][RPAD];
  __shared__ float red_sum[kWaves][RPAD];
  __shared__ __attribute__((aligned(16))) float xbuf[L16 ? 4 : kWaves * kXFloats * 64];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int r16 = lane & 15;
  const int g = lane >> 4;       // 16-lane group
  const int r32 = lane & 31;
  const int h = lane >> 5;       // 32-lane half
  const int dh = w & 1;          // layout 48: which half of the 576 dims this wave contracts
  const bool t32 = !L16 && w < 2;  // layout 48: wave works on the 32-row tile
  const int H = a.heads;
  const int R = a.num_q * H;
  const WgCoord wc = wg_coord(a.num_splits, a.batch, (R + RPAD - 1) / RPAD);
  const int split = wc.split;
  const int b = wc.b;

  const int L = a.seq_lens[b];
  const int P = (L + kPage - 1) / kPage;
  const int p0 = (int)(((int64_t)split * P) / a.num_splits);
  const int p1 = (int)(((int64_t)(split + 1) * P) / a.num_splits);
  const int ntiles = (p1 - p0 + TPG - 1) / TPG;
  // read-only page table through the constant address space: uniform
  // indices become scalar loads, which do not count against vmcnt
  const __attribute__((address_space(4))) int32_t* pt_row =
      (const __attribute__((address_space(4))) int32_t*)(a.page_table + (int64_t)b * a.max_blocks);

  // Rows owned by this lane: A = the 32-row tile row (layout 48) or the 16-row
  // tile row (layout 16); B = the 16-row tile row 32 + r16 (layout 48).
  const int rowA = L16 ? r16 : r32;
  const int rowB = 32 + r16;
  // rows rb0 .. rb0 + RPAD - 1 of the Q*H query rows are this workgroup's
  const int rb0 = wc.z * RPAD;
  const int limA = L - a.num_q + (rb0 + rowA) / H + 1;   // visible: position < lim
  const int limB = L - a.num_q + (rb0 + rowB) / H + 1;

  // ---- query fragments (B operand of S^T = K Q^T), kept in registers.
  //      layout 16:             row r16,      dims 32ks + 8g,          ks < 18
  //      layout 48, waves 0/1:  row r32,      dims 288dh + 16ks + 8h,  ks < 18
  //      layout 48, waves 2/3:  row 32 + r16, dims 288dh + 32ks + 8g,  ks < 9
  u32x4 qreg[kQRegs];
  {
    const int qrow = L16 ? r16 : (t32 ? r32 : rowB);
    const bool real = rb0 + qrow < R;
    const uint16_t* qp = a.q + ((int64_t)b * R + (real ? rb0 + qrow : 0)) * kLatent;
#pragma unroll
    for (int ks = 0; ks < kQRegs; ++ks) {
      int d0;
      if (L16) d0 = 32 * ks + 8 * g;
      else d0 = t32 ? 288 * dh + 16 * ks + 8 * h : 288 * dh + 32 * (ks % 9) + 8 * g;
      const bool use = real && (L16 || t32 || ks < 9);
      qreg[ks] = use ? *(const u32x4*)(qp + d0) : u32x4{0, 0, 0, 0};
    }
  }

  float m_runA = kNegInf, l_runA = 0.f, m_runB = kNegInf, l_runB = 0.f;
  constexpr int kN16a = L16 ? 8 : 1;   // layout 16: 8 tiles of 16 columns
  constexpr int kN32 = L16 ? 1 : 4;    // layout 48: 32-row tile, 4 x 32 columns
  constexpr int kN16b = L16 ? 1 : 8;   // layout 48: 16-row tile, 8 x 16 columns
  f32x4 o16a[kN16a];
  f32x16 o32[kN32];
  f32x4 o16b[kN16b];
#pragma unroll
  for (int c = 0; c < kN16a; ++c) o16a[c] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int c = 0; c < kN32; ++c) o32[c] = f32x16{};
#pragma unroll
  for (int c = 0; c < kN16b; ++c) o16b[c] = f32x4{0.f, 0.f, 0.f, 0.f};

  // ---- a2: tile T -> LDS buffer T % NBUF.  Wave w copies 1 KiB DMA loads
  // [w * kWaveLoads, (w+1) * kWaveLoads) of the tile: one page, or half a page
  // for 32-position bf16 tiles.  Lane `lane` of a load fills the LDS slot
  // (row, x ^ (row & swz)) of its page and fetches logical chunk x of that row.
  constexpr int kWavesPerPage = kWaves / TPG;     // 1 or 2
  const int wpage = w / kWavesPerPage;            // tile page this wave copies
  const int wslot0 = (w % kWavesPerPage) * kWaveLoads * 64;  // first 16-byte slot in that page
  auto issue_tile = [&](int T) {
    uint8_t* dst = kv_lds + (T % kNBuf) * kTileB + wpage * G::kPageB + wslot0 * 16;
    const int page = p0 + T * TPG + wpage;
    if (page < p1) {
      // one buffer resource per page: the copy is bounds-checked to the page
      const int blk = __builtin_amdgcn_readfirstlane(pt_row[page]);
      const __amdgpu_buffer_rsrc_t rsrc = __builtin_amdgcn_make_buffer_rsrc(
          (void*)(a.kv + (int64_t)blk * G::kPageB), 0, G::kPageB, kBufferRsrcWord3);
#pragma unroll
      for (int c = 0; c < kWaveLoads; ++c) {
        const uint32_t slot = wslot0 + 64 * c + lane;
        const uint32_t row = slot / G::kChunksPerRow;
        const uint32_t x = (slot - row * G::kChunksPerRow) ^ G::swz(row);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, LDS_PTR(void, dst + 1024 * c), 16,
                                                 row * G::kRowB + x * 16, 0, 0, 0);
      }
    } else {
#pragma unroll
      for (int c = 0; c < kWaveLoads; ++c)
        *(u32x4*)(dst + 1024 * c + 16 * lane) = u32x4{0, 0, 0, 0};
    }
  };
  auto has_page = [&](int T) { return p0 + T * TPG + wpage < p1; };

#pragma unroll
  for (int T = 0; T < kNBuf - 1; ++T)
    if (T < ntiles) issue_tile(T);

  const float c2 = a.score_scale_log2;

  for (int it = 0; it < ntiles; ++it) {
    // Wait for this wave's copy of tile `it`; a later tile may stay in flight.
    if (kNBuf == 3 && it + 1 < ntiles && has_page(it + 1))
      __builtin_amdgcn_s_waitcnt(waitcnt_vm(kWaveLoads));
    else
      __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
    uint8_t* tile = kv_lds + (it % kNBuf) * kTileB;
    {
      // zero the slots past seq_len among the rows this wave copied (last page only)
      const int page = p0 + it * TPG + wpage;
      const int valid = L - page * kPage;
      constexpr int kRowsPerWave = kPage / kWavesPerPage;
      const int row0 = (w % kWavesPerPage) * kRowsPerWave;
      const int z0 = valid > row0 ? valid : row0;
      if (page < p1 && z0 < row0 + kRowsPerWave) {
        uint8_t* pg = tile + wpage * G::kPageB;
        for (int c = lane; c < (row0 + kRowsPerWave - z0) * G::kChunksPerRow; c += 64)
          *(u32x4*)(pg + (z0 * G::kChunksPerRow + c) * 16) = u32x4{0, 0, 0, 0};
      }
    }
    lds_barrier();  // tile `it` visible; every wave is done with tile it - 1
    issue_tile(it + kNBuf - 1);

    const int tpos0 = (p0 + it * TPG) * kPage;      // sequence position of tile slot 0
    const int tlim = (p1 - p0 - it * TPG) * kPage;  // tile slots inside the split

    float alphaA = 1.f, alphaB = 1.f;
    if constexpr (L16) {
      // ---- a4/a5 (<= 16 rows): wave w scores page w of the tile against the 16-row tile.
      float sv[4];
      f32x4 s0 = f32x4{0.f, 0.f, 0.f, 0.f}, s1 = s0;
      const uint8_t* pg = tile + w * G::kPageB;
      pipelined<18, 3, KR>([&](int ks) { return load_k8<FP8>(pg, r16, 32 * ks + 8 * g); },
                           [&](int ks, KR raw) {
                             if (ks & 1) s1 = mfma16(kop(raw), as_bf16x8(qreg[ks]), s1);
                             else s0 = mfma16(kop(raw), as_bf16x8(qreg[ks]), s0);
                           });
      const f32x4 s = s0 + s1;
      float mx = kNegInf;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int tt = 16 * w + 4 * g + i;
        const bool ok = tt < tlim && tpos0 + tt < limA;
        sv[i] = ok ? s[i] * c2 : kNegInf;
        mx = fmaxf(mx, sv[i]);
      }
      mx = xor_max(xor_max(mx, 16), 32);
      if (g == 0) red_max[w][r16] = mx;
      lds_barrier();

      const float mt = fmaxf(fmaxf(red_max[0][r16], red_max[1][r16]), fmaxf(red_max[2][r16], red_max[3][r16]));
      const float mA = (mt > m_runA + kSlack) ? mt : m_runA;   // lazy rescale
      alphaA = (mA == m_runA) ? 1.f : __builtin_amdgcn_exp2f(m_runA - mA);
      m_runA = mA;
      bf16x4 pb;
      float ps = 0.f;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float p = (sv[i] == kNegInf) ? 0.f : __builtin_amdgcn_exp2f(sv[i] - mA);
        pb[i] = (__bf16)p;
        ps += p;
      }
      ps = xor_sum(xor_sum(ps, 16), 32);
      if (g == 0) red_sum[w][r16] = ps;
      *(bf16x4*)(p_lds + r16 * kPRB + (16 * w + 4 * g) * 2) = pb;
      lds_barrier();
      l_runA = l_runA * alphaA + ((red_sum[0][r16] + red_sum[1][r16]) + (red_sum[2][r16] + red_sum[3][r16]));
    } else {
      // ---- a4 (17..48 rows): the wave pair of a row tile splits the 576 dims in
      // halves; partial scores of every tile position are swapped through LDS.
      float* xme = xbuf + w * kXFloats * 64;
      const float* xpeer = xbuf + (w ^ 1) * kXFloats * 64;
      if (t32) {
        f32x16 s[NS32];
#pragma unroll
        for (int sp = 0; sp < NS32; ++sp) s[sp] = f32x16{};
        // step i: k-step i % 18 of sub-tile i / 18
        pipelined<18 * NS32, 3, KR>(
            [&](int i) {
              const int tt = 32 * (i / 18) + r32;
              return load_k8<FP8>(tile + (tt >> 4) * G::kPageB, tt & 15, 288 * dh + 16 * (i % 18) + 8 * h);
            },
            [&](int i, KR raw) { s[i / 18] = mfma32(kop(raw), as_bf16x8(qreg[i % 18]), s[i / 18]); });
#pragma unroll
        for (int sp = 0; sp < NS32; ++sp)
#pragma unroll
          for (int q = 0; q < 4; ++q)
            *(f32x4*)(xme + ((sp * 4 + q) * 64 + lane) * 4) =
                f32x4{s[sp][4 * q], s[sp][4 * q + 1], s[sp][4 * q + 2], s[sp][4 * q + 3]};
        lds_barrier();
        float sv[16 * NS32];
        float mx = kNegInf;
#pragma unroll
        for (int sp = 0; sp < NS32; ++sp)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const f32x4 pv = *(const f32x4*)(xpeer + ((sp * 4 + q) * 64 + lane) * 4);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const int tq = 32 * sp + 8 * q + 4 * h + i;
              const bool ok = tq < tlim && tpos0 + tq < limA;
              const float v = ok ? (s[sp][4 * q + i] + pv[i]) * c2 : kNegInf;
              sv[16 * sp + 4 * q + i] = v;
              mx = fmaxf(mx, v);
            }
          }
        mx = xor_max(mx, 32);
        const float mA = (mx > m_runA + kSlack) ? mx : m_runA;   // lazy rescale
        if (w == 0 && h == 0) red_max[0][r32] = mA;
        // this wave writes the probabilities of its half of the tile positions
        float ps = 0.f;
#pragma unroll
        for (int k = 0; k < 8 * NS32; k += 4) {
          const int base = (NS32 == 2) ? 16 * dh + k : 8 * dh + k;  // sv index of a 4-run
          bf16x4 pb;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const float v = sv[base + i];
            const float p = (v == kNegInf) ? 0.f : __builtin_amdgcn_exp2f(v - mA);
            pb[i] = (__bf16)p;
            ps += p;
          }
          const int sp = base / 16, q = (base % 16) / 4;
          *(bf16x4*)(p_lds + r32 * kPRB + (32 * sp + 8 * q + 4 * h) * 2) = pb;
        }
        ps = xor_sum(ps, 32);
        if (h == 0) red_sum[w][r32] = ps;
      } else {
        f32x4 s[NS16];
#pragma unroll
        for (int sp = 0; sp < NS16; ++sp) s[sp] = f32x4{0.f, 0.f, 0.f, 0.f};
        // step i: k-step i % 9 of sub-tile i / 9
        pipelined<9 * NS16, 3, KR>(
            [&](int i) {
              return load_k8<FP8>(tile + (i / 9) * G::kPageB, r16, 288 * dh + 32 * (i % 9) + 8 * g);
            },
            [&](int i, KR raw) { s[i / 9] = mfma16(kop(raw), as_bf16x8(qreg[i % 9]), s[i / 9]); });
#pragma unroll
        for (int sp = 0; sp < NS16; ++sp) *(f32x4*)(xme + (sp * 64 + lane) * 4) = s[sp];
        lds_barrier();
        float sv[4 * NS16];
        float mx = kNegInf;
#pragma unroll
        for (int sp = 0; sp < NS16; ++sp) {
          const f32x4 pv = *(const f32x4*)(xpeer + (sp * 64 + lane) * 4);
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int tq = 16 * sp + 4 * g + i;
            const bool ok = tq < tlim && tpos0 + tq < limB;
            const float v = ok ? (s[sp][i] + pv[i]) * c2 : kNegInf;
            sv[4 * sp + i] = v;
            mx = fmaxf(mx, v);
          }
        }
        mx = xor_max(xor_max(mx, 16), 32);
        const float mB = (mx > m_runB + kSlack) ? mx : m_runB;   // lazy rescale
        if (w == 2 && g == 0) red_max[2][rowB] = mB;
        float ps = 0.f;
#pragma unroll
        for (int k = 0; k < NS16 / 2; ++k) {
          const int sp = dh * (NS16 / 2) + k;
          bf16x4 pb;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const float v = sv[4 * sp + i];
            const float p = (v == kNegInf) ? 0.f : __builtin_amdgcn_exp2f(v - mB);
            pb[i] = (__bf16)p;
            ps += p;
          }
          *(bf16x4*)(p_lds + rowB * kPRB + (16 * sp + 4 * g) * 2) = pb;
        }
        ps = xor_sum(xor_sum(ps, 16), 32);
        if (g == 0) red_sum[w][rowB] = ps;
      }
      lds_barrier();
      // every wave tracks both row tiles (it holds their outputs for its columns)
      const float mA = red_max[0][r32];
      alphaA = (mA == m_runA) ? 1.f : __builtin_amdgcn_exp2f(m_runA - mA);
      m_runA = mA;
      l_runA = l_runA * alphaA + (red_sum[0][r32] + red_sum[1][r32]);
      const float mB = red_max[2][rowB];
      alphaB = (mB == m_runB) ? 1.f : __builtin_amdgcn_exp2f(m_runB - mB);
      m_runB = mB;
      l_runB = l_runB * alphaB + (red_sum[2][rowB] + red_sum[3][rowB]);
    }

    // ---- output rescale, only when some row's maximum moved.
    if (__any(alphaA != 1.f || alphaB != 1.f)) {
      if constexpr (L16) {
#pragma unroll
        for (int c = 0; c < 8; ++c) o16a[c] *= alphaA;
      } else {
#pragma unroll
        for (int c = 0; c < 4; ++c) o32[c] *= alphaA;
#pragma unroll
        for (int c = 0; c < 8; ++c) o16b[c] *= alphaB;
      }
    }

    // ---- a6: O^T[c][r] += V^T[c][t] P^T[t][r] for this wave's 128 columns.
    const int col0 = 128 * w;
    if constexpr (L16) {
      bf16x8 pf[2];
#pragma unroll
      for (int kk = 0; kk < 2; ++kk)
        pf[kk] = as_bf16x8(*(const u32x4*)(p_lds + r16 * kPRB + (32 * kk + 8 * g) * 2));
      // step i: k-step i/8 (32 positions), column tile i%8
      pipelined<16, 4, KR>(
          [&](int i) { return load_v8<FP8>(tile, 32 * (i >> 3) + 8 * g, col0 + 16 * (i & 7), r16); },
          [&](int i, KR raw) { o16a[i & 7] = mfma16(kop(raw), pf[i >> 3], o16a[i & 7]); });
    } else {
      constexpr int K32 = TP / 16;   // 16-position k-steps of the 32-row tile
      constexpr int K16 = TP / 32;   // 32-position k-steps of the 16-row tile
      bf16x8 pf32[K32], pf16[K16];
#pragma unroll
      for (int kk = 0; kk < K32; ++kk)
        pf32[kk] = as_bf16x8(*(const u32x4*)(p_lds + r32 * kPRB + (16 * kk + 8 * h) * 2));
#pragma unroll
      for (int kk = 0; kk < K16; ++kk)
        pf16[kk] = as_bf16x8(*(const u32x4*)(p_lds + rowB * kPRB + (32 * kk + 8 * g) * 2));
      // steps [0, 4*K32): 32-row tile, k-step i/4 (16 positions), column tile i%4 (32 columns);
      // then 8*K16 steps: 16-row tile, k-step j/8 (32 positions), column tile j%8.
      pipelined<4 * K32 + 8 * K16, 4, KR>(
          [&](int i) {
            if (i < 4 * K32)
              return load_v8<FP8>(tile, 16 * (i >> 2) + 8 * h, col0 + 32 * (i & 3) + 16 * (g & 1), r16);
            const int j = i - 4 * K32;
            return load_v8<FP8>(tile, 32 * (j >> 3) + 8 * g, col0 + 16 * (j & 7), r16);
          },
          [&](int i, KR raw) {
            if (i < 4 * K32) {
              o32[i & 3] = mfma32(kop(raw), pf32[i >> 2], o32[i & 3]);
            } else {
              const int j = i - 4 * K32;
              o16b[j & 7] = mfma16(kop(raw), pf16[j >> 3], o16b[j & 7]);
            }
          });
    }
  }

  // ---- a7: epilogue.  Each wave's rows x 128 columns go through LDS (the KV
  // buffers: every copy has landed, and the barrier below ends every wave's
  // last reads of them), so that a store instruction writes four whole
  // 256-byte row segments instead of 16 or 32 rows with 16-32 bytes each.
  lds_barrier();
  {
    constexpr int kSRow = 256 + 16;   // staged row stride (bytes), skewed against bank conflicts
    static_assert(kWaves * RPAD * kSRow <= kNBuf * kTileB, "epilogue staging fits the KV buffers");
    uint8_t* const stage = kv_lds + w * RPAD * kSRow;
    auto put4 = [&](int r, int c, f32x4 v, float sc) {
      bf16x4 ov;
#pragma unroll
      for (int i = 0; i < 4; ++i) ov[i] = (__bf16)(v[i] * sc);
      *(bf16x4*)(stage + r * kSRow + 2 * c) = ov;
    };
    const float scA = l_runA > 0.f ? a.out_scale / l_runA : 0.f;
    if constexpr (L16) {
#pragma unroll
      for (int ct = 0; ct < 8; ++ct) put4(r16, 16 * ct + 4 * g, o16a[ct], scA);
    } else {
#pragma unroll
      for (int ct = 0; ct < 4; ++ct)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const f32x4 v{o32[ct][4 * q], o32[ct][4 * q + 1], o32[ct][4 * q + 2], o32[ct][4 * q + 3]};
          put4(r32, 32 * ct + 8 * q + 4 * h, v, scA);
        }
      const float scB = l_runB > 0.f ? a.out_scale / l_runB : 0.f;
#pragma unroll
      for (int ct = 0; ct < 8; ++ct) put4(rowB, 16 * ct + 4 * g, o16b[ct], scB);
    }
    // each wave reads back only its own rows (LDS is in order within a wave)
    uint16_t* const dst = FINAL ? a.out : a.part_out;
    const int64_t row0 = FINAL ? (int64_t)b * R : ((int64_t)split * a.batch + b) * R;
    const int cc = 8 * (lane & 15);
#pragma unroll
    for (int j = 0; j < RPAD / 4; ++j) {
      const int r = 4 * j + (lane >> 4);
      const u32x4 v = *(const u32x4*)(stage + r * kSRow + 2 * cc);
      if (rb0 + r < R) *(u32x4*)(dst + (row0 + rb0 + r) * kValue + 128 * w + cc) = v;
    }
  }
  auto store_lse = [&](int r, float m_run, float l_run) {
    const float v = (l_run > 0.f) ? (m_run + log2f(l_run)) * kLn2 : kNegInf;
    const int64_t lrow = ((FINAL ? 0 : (int64_t)split * a.batch) + b) * R + rb0 + r;
    if constexpr (FINAL) a.lse[lrow] = v;
    else a.part_lse[lrow] = v;
  };
  if (w == 0) {
    if constexpr (L16) {
      if (g == 0 && rb0 + r16 < R) store_lse(r16, m_runA, l_runA);
    } else {
      if (h == 0 && rb0 + r32 < R) store_lse(r32, m_runA, l_runA);
      if (g == 0 && rb0 + rowB < R) store_lse(rowB, m_runB, l_runB);
    }
  }
#endif  // __HIP_DEVICE_COMPILE__
}

// ---------------------------------------------------------------------------
// FP8 KV with 33..64 query rows (speculative verify): the FP8 latents are fed
// to the 32x32x64 FP8 MFMA as stored, with no decode.  The bf16 side of each
// product is written as a sum of two FP8 terms:
//   query:         q * 2^e = q1 + q2, e chosen per row so max|q * 2^e| is in
//                  [64, 128); q has 8 significant bits and the residual of the
//                  first RNE rounding fits the second term, so q1 + q2 equals
//                  q * 2^e up to 2^-10 absolute, i.e. 2^-16 of the row maximum;
//   probabilities: p * 2^8 = p1 + p2, accurate to 2^-8 relative (bf16 gives
//                  2^-9), while the softmax denominator keeps the fp32 p.
// Each product therefore takes two FP8 MFMAs, which cost what one bf16 MFMA of
// the same shape costs, and no VALU conversion touches the KV stream.
// Rows are two 32-row tiles (r = j*H + h); wave w owns row tile w/2 and the
// 32-position half w%2 of every 64-position tile; PV is column-split as above.
// ---------------------------------------------------------------------------
__device__ __forceinline__ f32x16 mfma_f8(i32x8 a, i32x8 b, f32x16 c) {
  // formats 0/0 = FP8 E4M3 for both operands; E8M0 scales 127 = 1.0
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
}

__device__ __forceinline__ float bf16_lo(uint32_t v) { return __uint_as_float(v << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t v) { return __uint_as_float(v & 0xFFFF0000u); }
__device__ __forceinline__ float pow2f(int e) { return __uint_as_float((uint32_t)(e + 127) << 23); }

// four fp32 values -> (RNE FP8 of each, RNE FP8 of each residual), packed 4 per dword
__device__ __forceinline__ void split4_fp8(float v0, float v1, float v2, float v3, int& hi, int& lo) {
  hi = __builtin_amdgcn_cvt_pk_fp8_f32(v0, v1, 0, false);
  hi = __builtin_amdgcn_cvt_pk_fp8_f32(v2, v3, hi, true);
  const f32x2 b01 = __builtin_amdgcn_cvt_pk_f32_fp8(hi, false);
  const f32x2 b23 = __builtin_amdgcn_cvt_pk_f32_fp8(hi, true);
  lo = __builtin_amdgcn_cvt_pk_fp8_f32(v0 - b01[0], v1 - b01[1], 0, false);
  lo = __builtin_amdgcn_cvt_pk_fp8_f32(v2 - b23[0], v3 - b23[1], lo, true);
}

// Byte offset, from a lane's value base, of the 8 positions 8e..8e+7 (e < 4)
// of column tile ct of the FP8 PV step (see the PV comment below).
constexpr int pv_voff(int ct, int e) {
  return (e >> 1) * KvGeom<true>::kPageB + 8 * (e & 1) * KvGeom<true>::kRowB +
         16 * (4 * (ct >> 1) + 2 * ((ct ^ e) & 1));
}

// LDS reads of the FP8 kernel's key, value and probability operands are
// issued from inline assembly, which waits for its own reads before it ends:
// the compiler would otherwise treat these reads as possibly aliasing the
// in-flight direct-to-LDS copies of later tiles and wait for all of them
// (vmcnt(0)), which defeats the copy pipeline.  The copies of the tile being
// read were waited for explicitly before the barrier that published it.

// Key operand of one k-step: 16 bytes at each of two lane addresses (chunks
// 4ks + 2h and 4ks + 2h + 1 of the lane's position row).
template <int OFF>
__device__ __forceinline__ i32x8 read_k_f8(uint32_t a0, uint32_t a1) {
  u32x4 v0, v1;
  asm volatile(
      "ds_read_b128 %0, %2 offset:%4\n\t"
      "ds_read_b128 %1, %3 offset:%4\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(v0), "=&v"(v1)
      : "v"(a0), "v"(a1), "i"(OFF));
  return __builtin_bit_cast(i32x8, u32x8{v0[0], v0[1], v0[2], v0[3], v1[0], v1[1], v1[2], v1[3]});
}

// Value offsets of column tiles 0 and 1 (read_v128_f8 checks tiles 2 and 3).
static_assert(pv_voff(0, 0) == 0 && pv_voff(0, 1) == 4640 && pv_voff(0, 2) == 9216 &&
              pv_voff(0, 3) == 13856 && pv_voff(1, 0) == 32 && pv_voff(1, 1) == 4608 &&
              pv_voff(1, 2) == 9248 && pv_voff(1, 3) == 13824, "offsets in read_v128_f8");

// Key operands of two consecutive k-steps (offsets OFF and OFF + 64).
template <int OFF>
__device__ __forceinline__ void read_k2_f8(uint32_t a0, uint32_t a1, i32x8& k0, i32x8& k1) {
  u32x4 v0, v1, v2, v3;
  asm volatile(
      "ds_read_b128 %0, %4 offset:%6\n\t"
      "ds_read_b128 %1, %5 offset:%6\n\t"
      "ds_read_b128 %2, %4 offset:%7\n\t"
      "ds_read_b128 %3, %5 offset:%7\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(v0), "=&v"(v1), "=&v"(v2), "=&v"(v3)
      : "v"(a0), "v"(a1), "i"(OFF), "i"(OFF + 64));
  k0 = __builtin_bit_cast(i32x8, u32x8{v0[0], v0[1], v0[2], v0[3], v1[0], v1[1], v1[2], v1[3]});
  k1 = __builtin_bit_cast(i32x8, u32x8{v2[0], v2[1], v2[2], v2[3], v3[0], v3[1], v3[2], v3[3]});
}

constexpr int kF8Waves = 8;
constexpr int kF8Threads = kF8Waves * 64;

// LDS reads of the start of an MFMA phase, one round trip: the group's four
// tile maxima and four row sums of row r32 (red_max / red_sum rows are 128
// bytes apart) and its two probability terms (as read_p32_f8).
__device__ __forceinline__ void read_phase_f8(uint32_t maddr, uint32_t saddr, uint32_t paddr,
                                              float (&rm)[4], float (&rs)[4], i32x8 (&pf)[2]) {
  u32x4 p0, p1, p2, p3;
  asm volatile(
      "ds_read_b32 %0, %12\n\t"
      "ds_read_b32 %1, %12 offset:128\n\t"
      "ds_read_b32 %2, %12 offset:256\n\t"
      "ds_read_b32 %3, %12 offset:384\n\t"
      "ds_read_b32 %4, %13\n\t"
      "ds_read_b32 %5, %13 offset:128\n\t"
      "ds_read_b32 %6, %13 offset:256\n\t"
      "ds_read_b32 %7, %13 offset:384\n\t"
      "ds_read_b128 %8, %14\n\t"
      "ds_read_b128 %9, %14 offset:16\n\t"
      "ds_read_b128 %10, %14 offset:2560\n\t"
      "ds_read_b128 %11, %14 offset:2576\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(rm[0]), "=&v"(rm[1]), "=&v"(rm[2]), "=&v"(rm[3]), "=&v"(rs[0]), "=&v"(rs[1]),
        "=&v"(rs[2]), "=&v"(rs[3]), "=&v"(p0), "=&v"(p1), "=&v"(p2), "=&v"(p3)
      : "v"(maddr), "v"(saddr), "v"(paddr));
  pf[0] = __builtin_bit_cast(i32x8, u32x8{p0[0], p0[1], p0[2], p0[3], p1[0], p1[1], p1[2], p1[3]});
  pf[1] = __builtin_bit_cast(i32x8, u32x8{p2[0], p2[1], p2[2], p2[3], p3[0], p3[1], p3[2], p3[3]});
}

// Value operand of one PV step: column tiles 0..3 (128 columns) x positions
// 32h + 0..31, sixteen transposed reads at the offsets pv_voff(ct, e).
static_assert(pv_voff(2, 0) == 64 && pv_voff(2, 1) == 4704 && pv_voff(2, 2) == 9280 &&
              pv_voff(2, 3) == 13920 && pv_voff(3, 0) == 96 && pv_voff(3, 1) == 4672 &&
              pv_voff(3, 2) == 9312 && pv_voff(3, 3) == 13888, "offsets in read_v128_f8");
__device__ __forceinline__ void read_v128_f8(uint32_t vaddr, u32x2 (&v)[16]) {
  asm volatile(
      "ds_read_b64_tr_b8 %0, %16\n\t"
      "ds_read_b64_tr_b8 %1, %16 offset:4640\n\t"
      "ds_read_b64_tr_b8 %2, %16 offset:9216\n\t"
      "ds_read_b64_tr_b8 %3, %16 offset:13856\n\t"
      "ds_read_b64_tr_b8 %4, %16 offset:32\n\t"
      "ds_read_b64_tr_b8 %5, %16 offset:4608\n\t"
      "ds_read_b64_tr_b8 %6, %16 offset:9248\n\t"
      "ds_read_b64_tr_b8 %7, %16 offset:13824\n\t"
      "ds_read_b64_tr_b8 %8, %16 offset:64\n\t"
      "ds_read_b64_tr_b8 %9, %16 offset:4704\n\t"
      "ds_read_b64_tr_b8 %10, %16 offset:9280\n\t"
      "ds_read_b64_tr_b8 %11, %16 offset:13920\n\t"
      "ds_read_b64_tr_b8 %12, %16 offset:96\n\t"
      "ds_read_b64_tr_b8 %13, %16 offset:4672\n\t"
      "ds_read_b64_tr_b8 %14, %16 offset:9312\n\t"
      "ds_read_b64_tr_b8 %15, %16 offset:13888\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(v[0]), "=&v"(v[1]), "=&v"(v[2]), "=&v"(v[3]), "=&v"(v[4]), "=&v"(v[5]), "=&v"(v[6]),
        "=&v"(v[7]), "=&v"(v[8]), "=&v"(v[9]), "=&v"(v[10]), "=&v"(v[11]), "=&v"(v[12]),
        "=&v"(v[13]), "=&v"(v[14]), "=&v"(v[15])
      : "v"(vaddr));
}

// The two probability terms (32 bytes each) of one lane's row, 2560 bytes apart.
__device__ __forceinline__ void read_p32_f8(uint32_t paddr, i32x8 (&pf)[2]) {
  u32x4 a0, a1, b0, b1;
  asm volatile(
      "ds_read_b128 %0, %4\n\t"
      "ds_read_b128 %1, %4 offset:16\n\t"
      "ds_read_b128 %2, %4 offset:2560\n\t"
      "ds_read_b128 %3, %4 offset:2576\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(a0), "=&v"(a1), "=&v"(b0), "=&v"(b1)
      : "v"(paddr));
  pf[0] = __builtin_bit_cast(i32x8, u32x8{a0[0], a0[1], a0[2], a0[3], a1[0], a1[1], a1[2], a1[3]});
  pf[1] = __builtin_bit_cast(i32x8, u32x8{b0[0], b0[1], b0[2], b0[3], b1[0], b1[1], b1[2], b1[3]});
}

// A lane's query fragments from the block staged in LDS (see the prologue of
// split_kernel_f8x64): a[c] is the address of chunk pair c at the lane's
// first k-step, and k-step ks lies 128 ks bytes further.  NKS = 5 or 4 steps.
template <int NKS>
__device__ __forceinline__ void read_q_f8(const uint32_t (&a)[4], u32x4 (&v)[5][4]) {
  static_assert(NKS == 4 || NKS == 5, "four or five k-steps");
  if constexpr (NKS == 5) {
    asm volatile(
        "ds_read_b128 %0, %20\n\t"
        "ds_read_b128 %1, %21\n\t"
        "ds_read_b128 %2, %22\n\t"
        "ds_read_b128 %3, %23\n\t"
        "ds_read_b128 %4, %20 offset:128\n\t"
        "ds_read_b128 %5, %21 offset:128\n\t"
        "ds_read_b128 %6, %22 offset:128\n\t"
        "ds_read_b128 %7, %23 offset:128\n\t"
        "ds_read_b128 %8, %20 offset:256\n\t"
        "ds_read_b128 %9, %21 offset:256\n\t"
        "ds_read_b128 %10, %22 offset:256\n\t"
        "ds_read_b128 %11, %23 offset:256\n\t"
        "ds_read_b128 %12, %20 offset:384\n\t"
        "ds_read_b128 %13, %21 offset:384\n\t"
        "ds_read_b128 %14, %22 offset:384\n\t"
        "ds_read_b128 %15, %23 offset:384\n\t"
        "ds_read_b128 %16, %20 offset:512\n\t"
        "ds_read_b128 %17, %21 offset:512\n\t"
        "ds_read_b128 %18, %22 offset:512\n\t"
        "ds_read_b128 %19, %23 offset:512\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(v[0][0]), "=&v"(v[0][1]), "=&v"(v[0][2]), "=&v"(v[0][3]), "=&v"(v[1][0]),
          "=&v"(v[1][1]), "=&v"(v[1][2]), "=&v"(v[1][3]), "=&v"(v[2][0]), "=&v"(v[2][1]),
          "=&v"(v[2][2]), "=&v"(v[2][3]), "=&v"(v[3][0]), "=&v"(v[3][1]), "=&v"(v[3][2]),
          "=&v"(v[3][3]), "=&v"(v[4][0]), "=&v"(v[4][1]), "=&v"(v[4][2]), "=&v"(v[4][3])
        : "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3]));
  } else {
    asm volatile(
        "ds_read_b128 %0, %16\n\t"
        "ds_read_b128 %1, %17\n\t"
        "ds_read_b128 %2, %18\n\t"
        "ds_read_b128 %3, %19\n\t"
        "ds_read_b128 %4, %16 offset:128\n\t"
        "ds_read_b128 %5, %17 offset:128\n\t"
        "ds_read_b128 %6, %18 offset:128\n\t"
        "ds_read_b128 %7, %19 offset:128\n\t"
        "ds_read_b128 %8, %16 offset:256\n\t"
        "ds_read_b128 %9, %17 offset:256\n\t"
        "ds_read_b128 %10, %18 offset:256\n\t"
        "ds_read_b128 %11, %19 offset:256\n\t"
        "ds_read_b128 %12, %16 offset:384\n\t"
        "ds_read_b128 %13, %17 offset:384\n\t"
        "ds_read_b128 %14, %18 offset:384\n\t"
        "ds_read_b128 %15, %19 offset:384\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(v[0][0]), "=&v"(v[0][1]), "=&v"(v[0][2]), "=&v"(v[0][3]), "=&v"(v[1][0]),
          "=&v"(v[1][1]), "=&v"(v[1][2]), "=&v"(v[1][3]), "=&v"(v[2][0]), "=&v"(v[2][1]),
          "=&v"(v[2][2]), "=&v"(v[2][3]), "=&v"(v[3][0]), "=&v"(v[3][1]), "=&v"(v[3][2]),
          "=&v"(v[3][3])
        : "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3]));
    v[4][0] = v[4][1] = v[4][2] = v[4][3] = u32x4{0u, 0u, 0u, 0u};
  }
}

// Eight waves in two groups of four; group g owns query rows 32g..32g+31 and
// waves 4g..4g+3, and SIMD k runs wave k of group 0 and wave k of group 1.
// Within a group, wave v = w & 3:
//   QK:  position half sp = v & 1 of the 64-position tile and dimension half
//        dh = v >> 1 (k-steps 0..4 or 5..8 of 64 dims): 80 registers of query
//        fragments.  Partners v and v ^ 2 add their partial scores through
//        LDS; the dh = 1 wave reads its key rows rotated by 16 positions, so
//        both keep accumulator elements 0..7 (positions 16dh + 0..15 of the
//        half) and send elements 8..15.
//   PV:  output columns 128v..128v+127 for the group's 32 rows.
// The groups run one phase apart (each phase ends with a workgroup barrier):
//   phase E(i): group 0: PV(i-1), QK(i)   | group 1: softmax(i-1)
//   phase O(i): group 0: softmax(i)       | group 1: PV(i-1), QK(i)
// so on every SIMD one wave issues MFMAs while the other does the softmax
// arithmetic.  QK(i) also reads the tile's value fragments into registers,
// so a tile is only read in E(i) and O(i): buffer (i + 2) % 3 can be refilled
// at the start of E(i), two tiles ahead.
// Probabilities use a per-row reference maximum that moves only when a tile
// maximum exceeds it by more than 2^kSlack; the check runs at the start of
// the phase after each softmax, on data every wave reads, so the rare
// recomputation (and its barriers) is taken by all waves together.
template <bool FINAL>
__global__ __launch_bounds__(kF8Threads, 1) void split_kernel_f8x64(SplitArgs a) {
#if defined(__HIP_DEVICE_COMPILE__)  // the host pass only needs the launch stub
  using G = KvGeom<true>;
  constexpr int kNBuf = 3;
  constexpr int kTileB = kTilePages * G::kPageB;          // 36,864
  constexpr int kWaveLoads = G::kPageB / 1024;            // 9 wave-wide 1 KiB copies per page
  constexpr int kPRB = kTilePos + 16;                     // bytes per FP8 probability row (+skew)
  constexpr int kPTerm = 32 * kPRB;                       // 2560: second probability term
  constexpr float kSlack = 4.f;                           // p * 2^kPShift <= 256
  constexpr float kPShift = 4.f;
  static_assert(kPTerm == 2560, "read_p32_f8 assumes 2560 bytes between the terms");

  __shared__ __attribute__((aligned(16))) uint8_t kv_lds[kNBuf * kTileB];
  __shared__ __attribute__((aligned(16))) uint8_t p_lds[2][2 * kPTerm];   // [group][term][row][position]
  __shared__ __attribute__((aligned(16))) f32x4 xbuf[kF8Waves][2][64];    // partial scores for the partner
  // tile maxima and row sums of each wave's rows, in one array so that the
  // two addresses of a row differ by a constant
  __shared__ float red[2][kF8Waves][32];
  float (&red_max)[kF8Waves][32] = red[0];
  float (&red_sum)[kF8Waves][32] = red[1];
  __shared__ float qmax[kF8Waves][32];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int r32 = lane & 31;
  const int h = lane >> 5;
  const int g16 = lane >> 4;
  const int grp = w >> 2;
  const int v4 = w & 3;
  const int sp = v4 & 1;
  const int dh = v4 >> 1;
  const int ks0 = dh ? 5 : 0;
  const int nks = dh ? 4 : 5;
  const int H = a.heads;
  const int R = a.num_q * H;
  const WgCoord wc = wg_coord(a.num_splits, a.batch, (R + 63) / 64);
  const int split = wc.split;
  const int b = wc.b;
  // rows 64 * wc.z .. + 63 of the Q*H query rows are this workgroup's
  const int myrow = 64 * wc.z + 32 * grp + r32;

  // seq_lens[b] is requested first (a scalar load, waited for below), then
  // the query block's loads go out: they need only the workgroup's
  // coordinates (see the query conversion below for the layout).
  const int L = a.seq_lens[b];
  uint8_t* const qlds = kv_lds + kTileB;
  {
    const int nrows = min(64, R - 64 * wc.z);
    const __amdgpu_buffer_rsrc_t qrsrc = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(a.q + ((int64_t)b * R + 64 * wc.z) * kLatent), 0, nrows * 2 * kLatent, kBufferRsrcWord3);
#pragma unroll
    for (int i = 0; i < 9; ++i) {
      const int slot = 64 * (w + 8 * i) + lane;   // 16-byte LDS slot of this lane
      const int r = slot / 72, x = slot - 72 * (slot / 72);
      const uint32_t src = 16u * (uint32_t)(72 * r + (x ^ (r & 7)));
      __builtin_amdgcn_raw_ptr_buffer_load_lds(qrsrc, LDS_PTR(void, qlds + 1024 * (w + 8 * i)), 16, src, 0, 0, 0);
    }
  }
  __builtin_amdgcn_sched_barrier(0);
  const int P = (L + kPage - 1) / kPage;
  // page range [floor(split P / S), floor((split + 1) P / S)) in 32-bit
  // arithmetic: floor(s P / S) = s floor(P / S) + floor(s (P mod S) / S)
  const int S = a.num_splits;
  const int pq = P / S, pr = P - pq * S;
  const int p0 = split * pq + (split * pr) / S;
  const int p1 = (split + 1) * pq + ((split + 1) * pr) / S;
  const int ntiles = (p1 - p0 + kTilePages - 1) / kTilePages;

  // ---- a2: copies.  Tile T goes to LDS buffer T % 3; wave w copies page
  // w % 4 (nine wave-wide one-KiB loads from one buffer descriptor).  Tiles 0
  // and 1 are copied in the prologue: tile 0 by waves 0..3 as soon as its
  // page-table entries are known, tile 1 by waves 4..7 once every wave has
  // read the query staged in buffers 1 and 2;
  // tile T >= 2 is copied by group 1 at E(T - 2), while it runs its softmax,
  // so the copy issue never sits on the MFMA-role path and two tiles are in
  // flight.  A page outside the split, or the positions past seq_len in the
  // last page, lie outside the buffer range and are written to LDS as zeros by
  // the copy itself.
  // Page-table entry of page v4 of tile T (entries past the sequence are
  // clamped to its last page and not used).
  const int32_t* pt_b = a.page_table + (int64_t)b * a.max_blocks;
  const int plast = max(P - 1, 0);
  auto pt_load = [&](int T) -> int {
    return pt_b[min(p0 + T * kTilePages + v4, plast)];
  };
  auto issue_tile = [&](int T, int ptv) {
    const int gp = p0 + T * kTilePages + v4;
    const int blk = __builtin_amdgcn_readfirstlane(ptv);
    const int bytes = gp < p1 ? min(kPage, L - gp * kPage) * G::kRowB : 0;
    const __amdgpu_buffer_rsrc_t rsrc = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(a.kv + (int64_t)(gp < p1 ? blk : 0) * G::kPageB), 0, bytes, kBufferRsrcWord3);
    uint8_t* dst = kv_lds + (T % kNBuf) * kTileB + v4 * G::kPageB;
    // LDS slot s = 64c + lane of the page holds source chunk
    // 36 row + (x ^ swz(row)) with row = s / 36, x = s % 36.  As 36 is a
    // multiple of 4 the XOR only touches the two low bits, so the source chunk
    // is s ^ swz(s / 36) = s ^ (s / 144), and s / 144 = d0 + (lane >= t) with
    // d0 = 64c / 144 and t = 144 (d0 + 1) - 64c known per load: one or three
    // VALU operations per load instead of a division.
    static_assert(G::kChunksPerRow == 36, "FP8 page rows of 36 chunks");
    const uint32_t vb = 16u * (uint32_t)lane;
#pragma unroll
    for (int c = 0; c < kWaveLoads; ++c) {
      constexpr int kRowsPerSwz = 4 * G::kChunksPerRow;   // 144 slots per swizzle value
      const int d0 = (64 * c) / kRowsPerSwz;
      const int t = kRowsPerSwz * (d0 + 1) - 64 * c;
      const uint32_t d = (uint32_t)d0 + ((t < 64 && lane >= t) ? 1u : 0u);
      const uint32_t voff = (vb + 1024u * (uint32_t)c) ^ (d << 4);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, LDS_PTR(void, dst + 1024 * c), 16, voff, 0, 0, 0);
    }
  };

  // ---- query: q * 2^e = q1 + q2 (FP8), dims 64(ks0 + ks) + 32h + j of row `myrow`.
  // The workgroup's 64 query rows (1,152 bytes each) are staged once in KV
  // buffers 1 and 2 (exactly 73,728 bytes) by direct-to-LDS loads, 16 bytes a
  // lane: read by every wave straight from memory, the same rows would be
  // requested twice per workgroup at kernel start, when every workgroup's
  // first loads queue up.  Rows past Q*H lie outside the buffer range and
  // arrive as zeros.  Chunk j of row r sits at chunk (j & ~7) | ((j ^ r) & 7)
  // of its LDS row, so the 16 rows one ds_read_b128 phase reads fall in
  // distinct bank groups (two-way at most).
  i32x8 q1[5], q2[5];
  float q_unscale;
  int ptA, ptB;   // group 1: page-table entries of the next two tiles to copy
  {
    const int pt0 = pt_load(grp);
    ptA = pt_load(2);
    ptB = pt_load(3);
    // tile 0's copies go out as soon as its page-table entries are known
    // (group 0; buffer 0 is not part of the staged query)
    if (grp == 0) {
      issue_tile(0, pt0);
      __builtin_amdgcn_s_waitcnt(waitcnt_vm(kWaveLoads));   // this wave's query loads
    } else {
      __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
    }
    lds_barrier();   // every wave's query loads have landed
    u32x4 qv[5][4];
    {
      const int lr = 32 * grp + r32;   // row within the block
      const uint32_t rb = (uint32_t)(uintptr_t)LDS_PTR(uint8_t, qlds + lr * (2 * kLatent) + 128 * ks0);
      uint32_t qa[4];
#pragma unroll
      for (int c = 0; c < 4; ++c) qa[c] = rb + 16u * (uint32_t)((4 * h + c) ^ (lr & 7));
      if (dh) read_q_f8<4>(qa, qv);
      else read_q_f8<5>(qa, qv);
    }
    float mx = 0.f;
#pragma unroll
    for (int ks = 0; ks < 5; ++ks)
#pragma unroll
      for (int c = 0; c < 4; ++c)
#pragma unroll
        for (int k = 0; k < 4; ++k)
          mx = fmaxf(mx, fmaxf(fabsf(bf16_lo(qv[ks][c][k])), fabsf(bf16_hi(qv[ks][c][k]))));
    mx = max32(mx);                                 // the two lanes holding this row
    if (h == 0) qmax[w][r32] = mx;
    lds_barrier();   // also: every wave has read the staged query
    if (grp == 1) {
      issue_tile(1, pt0);
      __builtin_amdgcn_sched_barrier(0);
    }
    mx = fmaxf(qmax[w][r32], qmax[w ^ 2][r32]);     // the other half of the dims
    int e = 0;
    if (mx > 0.f) {
      const int ex = (int)((__float_as_uint(mx) >> 23) & 0xFF) - 126;  // mx = m * 2^ex, m in [0.5, 1)
      e = min(max(7 - ex, -100), 100);
    }
    const float sc = pow2f(e);
    q_unscale = pow2f(-e);
#pragma unroll
    for (int ks = 0; ks < 5; ++ks) {
      if (ks >= nks) break;   // dh = 1 has four steps
      i32x8 hi8, lo8;
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const u32x4 v = qv[ks][c];
        int hh, ll;
        split4_fp8(bf16_lo(v[0]) * sc, bf16_hi(v[0]) * sc, bf16_lo(v[1]) * sc, bf16_hi(v[1]) * sc, hh, ll);
        hi8[2 * c] = hh;
        lo8[2 * c] = ll;
        split4_fp8(bf16_lo(v[2]) * sc, bf16_hi(v[2]) * sc, bf16_lo(v[3]) * sc, bf16_hi(v[3]) * sc, hh, ll);
        hi8[2 * c + 1] = hh;
        lo8[2 * c + 1] = ll;
      }
      q1[ks] = hi8;
      q2[ks] = lo8;
    }
  }
  // scale of this lane's scores (row `myrow`) into the log2 domain
  const float cs = a.score_scale_log2 * q_unscale;

  // Reference maxima of rows r32 of group 0 and group 1 (every wave tracks
  // both, from the same LDS data), the row sum of this wave's row, and the
  // output of this wave's 128 columns x the group's 32 rows.
  float mref0 = kNegInf, mref1 = kNegInf;
  float l_run = 0.f;
  f32x16 o[4];
#pragma unroll
  for (int c = 0; c < 4; ++c) o[c] = f32x16{};
  i32x8 vfr[4];     // value fragments of the group's next PV
  float x[8];       // scores of this wave's last softmax (kept for a recomputation)
#pragma unroll
  for (int k = 0; k < 8; ++k) x[k] = kNegInf;

  const int prow = r32 & 15;
  const int kpage = 2 * sp + ((r32 >> 4) ^ dh);
  const int sl = lane & 15;
  const int vbase = 2 * h * G::kPageB + (sl >> 1) * G::kRowB + 16 * (8 * v4 + ((g16 ^ (sl >> 3)) & 1)) + 8 * (sl & 1);
  const int pbase = r32 * kPRB + 32 * sp + 16 * dh + 4 * h;
  uint8_t* const pg_lds = p_lds[grp];

  // An opaque copy of the lane index, taken where a lane-dependent address or
  // bound is needed inside the loop: derived from it there (one or two VALU
  // operations), the value does not hold a register of its own across the
  // loop, where nearly every register is taken.
  auto lane_now = [&]() -> int {
    int l = lane;
    asm volatile("" : "+v"(l));
    return l;
  };
  // Causal limit of the lane's row (visible: position < lim), needed on edge
  // tiles only and recomputed there (with an opaque divisor, so that the
  // division's reciprocal is not kept either).
  auto lim_now = [&]() -> int {
    int hd = H;
    asm volatile("" : "+s"(hd));
    return L - a.num_q + (64 * wc.z + 32 * grp + (lane_now() & 31)) / hd + 1;
  };

  // ---- a4: partial S^T over this wave's k-steps, then the value fragments.
  // Key addresses of tile T for this wave (lane's row, chunk pair 2h, 2h + 1).
  auto kaddr = [&](int T, uint32_t& kb0, uint32_t& kb1) {
    const uint8_t* tile = kv_lds + (T % kNBuf) * kTileB;
    kb0 = (uint32_t)(uintptr_t)LDS_PTR(const uint8_t, tile + kpage * G::kPageB + G::off(prow, 2 * h, 0) + 64 * ks0);
    kb1 = (uint32_t)(uintptr_t)LDS_PTR(const uint8_t, tile + kpage * G::kPageB + G::off(prow, 2 * h + 1, 0) + 64 * ks0);
  };
  // The value operand for the PV of this tile is read after the last key
  // operands, while the last score MFMAs drain (the tile is not read after
  // this phase).  Column tile ct, positions 32h + 8e .. +7: source lane sl of
  // a 16-lane group reads position 32h + 8e + sl/2, i.e. page 2h + e/2, row
  // 8(e%2) + sl/2, byte half sl%2 of chunk 8v + 2ct + (g16%2), XOR-swizzled by
  // (row/4)%4 = sl/8 + 2(e%2); vbase is the lane part of that address and
  // pv_voff(ct, e) the rest.
  auto qk = [&](int T) {
    uint32_t kb0, kb1;
    kaddr(T, kb0, kb1);
    const uint32_t vaddr = (uint32_t)(uintptr_t)LDS_PTR(const uint8_t, kv_lds + (T % kNBuf) * kTileB + vbase);
    f32x16 s = f32x16{};
    u32x2 vr[16];
    i32x8 ka, kb;
    read_k2_f8<0>(kb0, kb1, ka, kb);
    s = mfma_f8(ka, q1[0], s);
    s = mfma_f8(ka, q2[0], s);
    s = mfma_f8(kb, q1[1], s);
    s = mfma_f8(kb, q2[1], s);
    __builtin_amdgcn_sched_barrier(0);
    read_k2_f8<128>(kb0, kb1, ka, kb);
    s = mfma_f8(ka, q1[2], s);
    s = mfma_f8(ka, q2[2], s);
    s = mfma_f8(kb, q1[3], s);
    s = mfma_f8(kb, q2[3], s);
    __builtin_amdgcn_sched_barrier(0);
    if (!dh) {
      ka = read_k_f8<256>(kb0, kb1);
      s = mfma_f8(ka, q1[4], s);
      s = mfma_f8(ka, q2[4], s);
    }
    __builtin_amdgcn_sched_barrier(0);
    read_v128_f8(vaddr, vr);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int ct = 0; ct < 4; ++ct)
      vfr[ct] = __builtin_bit_cast(i32x8, u32x8{vr[4 * ct][0], vr[4 * ct][1], vr[4 * ct + 1][0],
                                                vr[4 * ct + 1][1], vr[4 * ct + 2][0], vr[4 * ct + 2][1],
                                                vr[4 * ct + 3][0], vr[4 * ct + 3][1]});
    // elements 8..15 belong to the partner wave; elements 0..7 stay for softmax
    {
      const int ln = lane_now();
      xbuf[w][0][ln] = f32x4{s[8], s[9], s[10], s[11]};
      xbuf[w][1][ln] = f32x4{s[12], s[13], s[14], s[15]};
    }
#pragma unroll
    for (int k = 0; k < 8; ++k) x[k] = s[k];
  };

  // probabilities p * 2^kPShift against the reference maximum, as two FP8 terms
  auto probs = [&](float m) {
    const float c0 = kPShift - (m == kNegInf ? 0.f : m);
    float ps = 0.f;
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      float p4[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        p4[i] = __builtin_amdgcn_exp2f(x[4 * q + i] + c0);
        ps += p4[i];
      }
      int hi, lo;
      split4_fp8(p4[0], p4[1], p4[2], p4[3], hi, lo);
      *(int*)(pg_lds + pbase + 8 * q) = hi;
      *(int*)(pg_lds + kPTerm + pbase + 8 * q) = lo;
    }
    ps = sum32(ps);
    if (h == 0) red_sum[w][r32] = ps;
  };

  // ---- a5: partner's partial scores added, scale to log2 units, mask (edge
  // tiles only), tile maxima, probabilities.  Element k of x is position
  // 32sp + 16dh + 8(k/4) + 4h + k%4 of the tile.
  auto softmax = [&](int T) {
    {
      const int ln = lane_now();
      const f32x4 u0 = xbuf[w ^ 2][0][ln];
      const f32x4 u1 = xbuf[w ^ 2][1][ln];
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        x[k] += u0[k];
        x[4 + k] += u1[k];
      }
    }
    const int tpos0 = (p0 + T * kTilePages) * kPage;
    const int tlim = (p1 - p0 - T * kTilePages) * kPage;
    float mx = kNegInf;
    if (tlim >= kTilePos && tpos0 + kTilePos <= L - a.num_q + 1) {   // every row sees the whole tile
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        x[k] *= cs;
        mx = fmaxf(mx, x[k]);
      }
    } else {
      // position tq = 32 sp + 16 dh + 4 h + (8 (k / 4) + k % 4) is visible
      // when it is below both tlim and lim - tpos0
      const int kvis = min(tlim, lim_now() - tpos0) - (32 * sp + 16 * dh + 4 * (lane_now() >> 5));
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        x[k] = 8 * (k >> 2) + (k & 3) < kvis ? x[k] * cs : kNegInf;
        mx = fmaxf(mx, x[k]);
      }
    }
    mx = max32(mx);
    if (h == 0) red_max[w][r32] = mx;
    probs(grp ? mref1 : mref0);
  };

  // Start of the phase after group gx's softmax: move gx's reference maxima
  // where a tile maximum passed them by more than 2^kSlack, and in that (rare,
  // workgroup-uniform) case let gx recompute its probabilities.  This is the
  // other group's side (gx != grp): it only tracks gx's maxima and joins the
  // two barriers.
  auto check = [&](int gx) {
    const float nm = fmaxf(fmaxf(red_max[4 * gx][r32], red_max[4 * gx + 1][r32]),
                           fmaxf(red_max[4 * gx + 2][r32], red_max[4 * gx + 3][r32]));
    const float mo = gx ? mref1 : mref0;
    const bool ov = nm > mo + kSlack;
    if (__any(ov)) {
      const float mn = ov ? nm : mo;
      if (gx) mref1 = mn;
      else mref0 = mn;
      lds_barrier();   // every wave has read the maxima (and the first sums)
      lds_barrier();   // gx has recomputed its probabilities
    }
  };

  // The same check run by the group that ran that softmax (gx = grp), on the
  // maxima and sums read with its phase's other LDS data; after a
  // recomputation the probability terms pf are read again.
  const uint32_t p_addr = (uint32_t)(uintptr_t)LDS_PTR(const uint8_t, pg_lds + r32 * kPRB + 32 * h);
  auto check_own = [&](const float (&rm)[4], const float (&rs)[4], i32x8 (&pf)[2]) -> float {
    const float nm = fmaxf(fmaxf(rm[0], rm[1]), fmaxf(rm[2], rm[3]));
    float sm = (rs[0] + rs[1]) + (rs[2] + rs[3]);
    const float mo = grp ? mref1 : mref0;
    const bool ov = nm > mo + kSlack;
    if (__any(ov)) {
      const float mn = ov ? nm : mo;
      const float alpha = ov ? __builtin_amdgcn_exp2f(mo - mn) : 1.f;
      l_run *= alpha;
      o[0] *= alpha;
      o[1] *= alpha;
      o[2] *= alpha;
      o[3] *= alpha;
      if (grp) mref1 = mn;
      else mref0 = mn;
      lds_barrier();
      probs(mn);
      lds_barrier();
      sm = (red_sum[4 * grp][r32] + red_sum[4 * grp + 1][r32]) +
           (red_sum[4 * grp + 2][r32] + red_sum[4 * grp + 3][r32]);
      read_p32_f8(p_addr, pf);
    }
    return sm;
  };

  // ---- a6: O^T[c][r] += V^T[c][t] (p1 + p2)^T[t][r], columns 128v .. 128v + 127.
  auto pv = [&](float row_sum, const i32x8 (&pf)[2]) {
    l_run += row_sum;
    // written out: a rolled loop here makes the compiler rotate the four
    // accumulators through one register window with moves
    o[0] = mfma_f8(vfr[0], pf[0], o[0]);
    o[1] = mfma_f8(vfr[1], pf[0], o[1]);
    o[2] = mfma_f8(vfr[2], pf[0], o[2]);
    o[3] = mfma_f8(vfr[3], pf[0], o[3]);
    o[0] = mfma_f8(vfr[0], pf[1], o[0]);
    o[1] = mfma_f8(vfr[1], pf[1], o[1]);
    o[2] = mfma_f8(vfr[2], pf[1], o[2]);
    o[3] = mfma_f8(vfr[3], pf[1], o[3]);
  };

  // Half-steps hs = 0, 1, ...: E(i) = 2i, O(i) = 2i + 1.  Group g's own step
  // count is hs - g: even -> MFMA role (PV of tile T - 1, QK of tile T,
  // T = (hs - g) / 2), odd -> softmax of tile T = (hs - g - 1) / 2.  At each
  // half-step the group that ran its softmax in the previous one (g = hs % 2)
  // is checked first.
  // Tile 0 (group 0's prologue copies) has landed before the loop; tile 1
  // (group 1's) only before E(1).
  if (grp == 0) __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
  for (int hs = 0; hs <= 2 * ntiles + 1; ++hs) {
    const bool copier = grp == 1 && (hs & 1) == 0;
    // Group 1's vector-memory order: copies(1), PT(4), copies(2), PT(5),
    // copies(3) ...  Before E(T), T >= 1, copies(T) must have landed while
    // PT(T + 3) and copies(T + 1) may still be in flight.
    if (copier && hs >= 2) __builtin_amdgcn_s_waitcnt(waitcnt_vm(kWaveLoads + 1));
    lds_barrier();
    if (copier) {
      const int it = hs >> 1;
      const int cur = (it & 1) ? ptB : ptA;
      const int nxt = pt_load(it + 4);
      asm volatile("" ::: "memory");   // keep PT(it + 4) ahead of the copies
      issue_tile(it + 2, cur);
      // use the new entry only after the copies are issued: waiting for it
      // then leaves them in flight
      __builtin_amdgcn_sched_barrier(0);
      if (it & 1) ptB = nxt;
      else ptA = nxt;
    }
    const int st = hs - grp;
    if (st >= 0 && (st & 1) == 0) {
      // MFMA role (grp == hs % 2): one LDS round trip for the check and the
      // PV's probabilities (stale data where unused)
      const int T = st >> 1;
      // the MFMA role is the phase's critical path: its instructions go first
      // on the SIMD it shares with a softmax-role wave
      __builtin_amdgcn_s_setprio(2);
      float rm[4], rs[4];
      i32x8 pf[2];
      read_phase_f8((uint32_t)(uintptr_t)LDS_PTR(const float, &red_max[4 * grp][r32]),
                    (uint32_t)(uintptr_t)LDS_PTR(const float, &red_sum[4 * grp][r32]), p_addr, rm, rs,
                    pf);
      const float row_sum = hs >= 2 ? check_own(rm, rs, pf) : 0.f;
      if (T >= 1) pv(row_sum, pf);
      if (T < ntiles) qk(T);
      __builtin_amdgcn_s_setprio(0);
    } else {
      if (hs >= 2) check(hs & 1);
      if (st >= 1) {
        const int T = (st - 1) >> 1;
        if (T < ntiles) softmax(T);
      }
    }
  }

  // No copy may still be writing this workgroup's LDS when it ends, and the
  // epilogue reuses the KV buffers: every wave's copies have landed.
  __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
  lds_barrier();

  // ---- a7: epilogue.  O and l both carry the 2^kPShift factor.  Each wave's
  // 32 rows x 128 columns go through LDS (the free KV buffers) so that a store
  // instruction writes four whole 256-byte row segments; stored straight from
  // the accumulators, each instruction would touch 32 rows with 16 bytes each.
  {
    constexpr int kSRow = 256 + 16;   // staged row stride (bytes), skewed against bank conflicts
    static_assert(kF8Waves * 32 * kSRow <= kNBuf * kTileB, "epilogue staging fits the KV buffers");
    uint8_t* const stage = kv_lds + w * 32 * kSRow;
    const float sc = l_run > 0.f ? a.out_scale / l_run : 0.f;
#pragma unroll
    for (int ct = 0; ct < 4; ++ct)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        bf16x4 ov;
#pragma unroll
        for (int i = 0; i < 4; ++i) ov[i] = (__bf16)(o[ct][4 * q + i] * sc);
        *(bf16x4*)(stage + r32 * kSRow + 2 * (32 * ct + 8 * q + 4 * h)) = ov;
      }
    // each wave reads back only its own rows (LDS is in order within a wave)
    uint16_t* const dst = FINAL ? a.out : a.part_out;
    const int64_t row0 = FINAL ? (int64_t)b * R : ((int64_t)split * a.batch + b) * R;
    const int cc = 8 * (lane & 15);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int r = 4 * j + (lane >> 4);
      const int grow = 64 * wc.z + 32 * grp + r;
      const u32x4 v = *(const u32x4*)(stage + r * kSRow + 2 * cc);
      if (grow < R) *(u32x4*)(dst + (row0 + grow) * kValue + 128 * v4 + cc) = v;
    }
  }
  if (myrow < R && v4 == 0 && h == 0) {
    const float lv = (l_run > 0.f) ? ((grp ? mref1 : mref0) - kPShift + log2f(l_run)) * kLn2 : kNegInf;
    if constexpr (FINAL) a.lse[(int64_t)b * R + myrow] = lv;
    else a.part_lse[((int64_t)split * a.batch + b) * R + myrow] = lv;
  }
#endif  // __HIP_DEVICE_COMPILE__
}

template <int LAYOUT, bool FP8>
hipError_t launch_layout(const SplitArgs& a, bool final_out, hipStream_t stream) {
  const int rows = a.num_q * a.heads;
  const int rpad = LAYOUT == kLayout16 ? 16 : 48;
  const dim3 grid((unsigned)(a.num_splits * a.batch * ((rows + rpad - 1) / rpad)));
  if (final_out)
    hipLaunchKernelGGL((split_kernel<LAYOUT, FP8, true>), grid, dim3(kThreads), 0, stream, a);
  else
    hipLaunchKernelGGL((split_kernel<LAYOUT, FP8, false>), grid, dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

template <bool FP8>
hipError_t launch_dtype(const SplitArgs& a, bool final_out, hipStream_t stream) {
  const int rows = a.num_q * a.heads;
  if (FP8 && rows > 32) {
    const dim3 grid((unsigned)(a.num_splits * a.batch * ((rows + 63) / 64)));
    if (final_out)
      hipLaunchKernelGGL(split_kernel_f8x64<true>, grid, dim3(kF8Threads), 0, stream, a);
    else
      hipLaunchKernelGGL(split_kernel_f8x64<false>, grid, dim3(kF8Threads), 0, stream, a);
    return hipGetLastError();
  }
  if (rows <= 16) return launch_layout<kLayout16, FP8>(a, final_out, stream);
  return launch_layout<kLayout48, FP8>(a, final_out, stream);
}

}  // namespace

int64_t split_work_items(const SplitArgs& a, bool fp8) {
  // the grids of launch_dtype / launch_layout
  const int64_t rows = (int64_t)a.num_q * a.heads;
  const int64_t units = (int64_t)a.num_splits * a.batch;
  if (fp8 && rows > 32) return units * ((rows + 63) / 64) * kF8Threads;
  const int64_t rpad = rows <= 16 ? 16 : 48;
  return units * ((rows + rpad - 1) / rpad) * kThreads;
}

hipError_t launch_split(const SplitArgs& a, bool fp8, bool final_out, hipStream_t stream) {
  return fp8 ? launch_dtype<true>(a, final_out, stream) : launch_dtype<false>(a, final_out, stream);
}

}  // namespace mla
