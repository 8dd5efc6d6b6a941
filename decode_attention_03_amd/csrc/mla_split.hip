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
typedef short s16x2 __attribute__((ext_vector_type(2)));
typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));

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
  int nsplit;     // splits of sequence b
  int64_t slot;   // partial slot: rows slot * R .. of part_out / part_lse
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
  c.nsplit = num_splits;
  c.slot = 0;
  return c;
}

// The workgroup's split: with S splits per sequence, unit u = split + S b of
// wg_coord and slot split * B + b; with the plan by length, unit u is slot u,
// which balanced_plan maps to its sequence and its index among that
// sequence's splits.
__device__ __forceinline__ WgCoord split_coord(const SplitArgs& a, int row_blocks) {
  WgCoord c = wg_coord(a.num_splits, a.batch, row_blocks);
  c.slot = (int64_t)c.split * a.batch + c.b;
  if (a.by_length) {
    const int u = c.split + a.num_splits * c.b;
    const SeqSlots ss = balanced_plan(a.seq_lens, a.batch, a.num_splits, a.max_blocks, u, true);
    c.b = ss.b;
    c.split = u - ss.first;
    c.nsplit = ss.count;
    c.slot = u;
  }
  return c;
}

// Buffer resource (four SGPRs: base, stride 0, byte range, flags) of `bytes`
// bytes at `base`; loads past the range read as zero.
__device__ __forceinline__ u32x4 buffer_rsrc(const void* base, uint32_t bytes) {
  const uint64_t a = (uint64_t)(uintptr_t)base;
  return u32x4{(uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)a),
               (uint32_t)__builtin_amdgcn_readfirstlane((int)((uint32_t)(a >> 32) & 0xFFFFu)),
               (uint32_t)__builtin_amdgcn_readfirstlane((int)bytes), (uint32_t)kBufferRsrcWord3};
}

// Wave-wide direct-to-LDS copy: lane i's 16 bytes at byte offset `voffset`
// of the buffer go to LDS address lds_addr + 16 i (buffer_load_dwordx4 ...
// lds, LDS base in M0, which is saved and restored around it).  Issued from
// inline assembly so that the compiler does not see an asynchronous LDS
// write: it would otherwise wait for every copy in flight (vmcnt(0)) before
// the next LDS read of any buffer, which takes away the prefetch.  Every
// wait for these copies is an explicit s_waitcnt vmcnt; the asm has no
// register outputs besides the saved M0.
__device__ __forceinline__ void copy16_to_lds(u32x4 rsrc, uint32_t voffset, uint32_t lds_addr) {
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %3\n\t"
      "s_nop 0\n\t"
      "buffer_load_dwordx4 %1, %2, 0 offen lds\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(voffset), "s"(rsrc), "s"(lds_addr));
}
// The same with the non-temporal bit, for pages that one launch reads
// exactly once (a single row block per split): the page stream then does
// not push out of the L2 what is shared between workgroups (the query rows
// of a sequence).  Same-box timing: bf16 decode of 32 sequences (generic
// kernel) 41.9 -> 38.2 us per layer-step, bf16 verify of 32 sequences
// (eight-wave kernel, one row block) 169.9 -> 167.2 us, packed FP8 kernel:
// long-context split kernel -1.3%, FP8 verify of 64 sequences -1%.  Kernels
// whose row blocks share pages (several per split) keep cached loads.
__device__ __forceinline__ void copy16_to_lds_nt(u32x4 rsrc, uint32_t voffset, uint32_t lds_addr) {
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %3\n\t"
      "s_nop 0\n\t"
      "buffer_load_dwordx4 %1, %2, 0 offen nt lds\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(voffset), "s"(rsrc), "s"(lds_addr));
}
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)LDS_PTR(const uint8_t, p);
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

// x combined with the value of lane l ^ 32 (a VALU lane swap, no LDS round trip)
__device__ __forceinline__ float max32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
// x combined with the value of lane l ^ 16 (a VALU row swap); both lanes of
// a pair add in the same order
__device__ __forceinline__ float max16(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum16(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Maximum / sum over each aligned group of eight lanes, with DPP moves
// (quad permutations for lane ^ 1 and lane ^ 2, then the mirror inside each
// half-row of eight lanes): three VALU steps, no LDS round trip.  Every lane of
// a group ends with the same value (each step combines two equal-order pairs).
template <int CTRL>
__device__ __forceinline__ float dpp_f(float x) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), CTRL, 0xF, 0xF, false));
}
constexpr int kDppXor1 = 0xB1;          // quad_perm [1, 0, 3, 2]
constexpr int kDppXor2 = 0x4E;          // quad_perm [2, 3, 0, 1]
constexpr int kDppHalfMirror = 0x141;   // lane i <- lane 7 - i within each group of eight
__device__ __forceinline__ float max8(float x) {
  x = fmaxf(x, dpp_f<kDppXor1>(x));
  x = fmaxf(x, dpp_f<kDppXor2>(x));
  return fmaxf(x, dpp_f<kDppHalfMirror>(x));
}
__device__ __forceinline__ float sum8(float x) {
  x = x + dpp_f<kDppXor1>(x);
  x = x + dpp_f<kDppXor2>(x);
  return x + dpp_f<kDppHalfMirror>(x);
}

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
  // bf16 KV with at most 16 rows (decode): 32-position tiles in a ring of
  // four, so three tiles (110,592 bytes) are in flight while one is
  // computed; each wave contracts half the dims of one page of the tile.
  constexpr bool kHalf = L16 && !FP8;
  // Tile: 64 positions (4 pages), except 32 (2 pages) for bf16 with 48 rows,
  // where LDS holds three bf16 tiles plus the partial-score exchange, and for
  // bf16 with at most 16 rows (kHalf).
  constexpr int TP = (!FP8 && (!L16 || kHalf)) ? 32 : 64;
  constexpr int TPG = TP / kPage;                  // pages per tile
  constexpr int kTileB = TPG * G::kPageB;
  constexpr int kNBuf = kHalf ? 4 : (L16 ? G::kNBuf : 3);
  constexpr int kWaveLoads = kTileB / kWaves / 1024;   // 1 KiB DMA loads per wave per tile (9 or 18)
  constexpr int RPAD = L16 ? 16 : 48;
  constexpr int kPRB = TP * 2 + 16;                // LDS bytes per probability row
  constexpr int NS32 = TP / 32;                    // 32-position sub-tiles of the 32-row tile
  constexpr int NS16 = TP / 16;                    // 16-position sub-tiles of the 16-row tile
  constexpr int kQRegs = kHalf ? 9 : 18;           // query fragments held per wave
  // partial scores exchanged per lane
  constexpr int kXFloats = kHalf ? 4 : (L16 ? 1 : 16 * NS32);
  // Lazy rescale: a row's reference maximum moves only when a tile maximum
  // exceeds it by more than 2^kSlack (bf16 probabilities up to 2^8 are exact
  // enough and far from overflow), which skips most output rescales.
  constexpr float kSlack = 8.f;

  __shared__ __attribute__((aligned(16))) uint8_t kv_lds[kNBuf * kTileB];
  // probabilities: one copy per wave with kHalf (each wave computes the whole
  // tile's softmax for its own PV), else one shared copy
  __shared__ __attribute__((aligned(16))) uint8_t p_lds[(kHalf ? kWaves : 1) * RPAD * kPRB];
  __shared__ float red_max[kWaves][RPAD];
  __shared__ float red_sum[kWaves][RPAD];
  __shared__ __attribute__((aligned(16))) float xbuf[(L16 && !kHalf) ? 4 : kWaves * kXFloats * 64];

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
  const WgCoord wc = split_coord(a, (R + RPAD - 1) / RPAD);
  const int split = wc.split;
  const int b = wc.b;

  const int L = kDebug ? debug_seq_len(a.seq_lens[b], a.num_q, a.max_blocks, a.debug_flags) : a.seq_lens[b];
  const int P = (L + kPage - 1) / kPage;
  const int p0 = (int)(((int64_t)split * P) / wc.nsplit);
  const int p1 = (int)(((int64_t)(split + 1) * P) / wc.nsplit);
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
      if (L16) d0 = (kHalf ? 288 * (w >> 1) : 0) + 32 * ks + 8 * g;
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
      int blk = __builtin_amdgcn_readfirstlane(pt_row[page]);
      if constexpr (kDebug) blk = debug_page_id(blk, a.num_blocks, a.debug_flags);
      const u32x4 rsrc = buffer_rsrc(a.kv + (int64_t)blk * G::kPageB, G::kPageB);
      // issued from inline assembly (copy16_to_lds): seen by the compiler as
      // LDS writes, these copies would make it wait for all of them (the
      // next tile's included) before the LDS reads of the current tile; the
      // waits for them are the explicit vmcnt waits at the top of the loop
#pragma unroll
      for (int c = 0; c < kWaveLoads; ++c) {
        const uint32_t slot = wslot0 + 64 * c + lane;
        const uint32_t row = slot / G::kChunksPerRow;
        const uint32_t x = (slot - row * G::kChunksPerRow) ^ G::swz(row);
        copy16_to_lds_nt(rsrc, row * G::kRowB + x * 16, lds_addr(dst + 1024 * c));
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
  // The query loads are waited for here, once, together with the first
  // tiles' copies: at their first use inside the loop the compiler's wait
  // (vmcnt(0), it does not count the copies) would come back in every
  // iteration and hold each one up until the next tile had landed.
#pragma unroll
  for (int ks = 0; ks < kQRegs; ++ks) asm volatile("" ::"v"(qreg[ks]));

  const float c2 = a.score_scale_log2;

  for (int it = 0; it < ntiles; ++it) {
    // Wait for this wave's copy of tile `it`; later tiles may stay in flight
    // (a wave copies nothing for a tile past its last page).
    if constexpr (kNBuf == 4) {
      if (has_page(it + 2)) __builtin_amdgcn_s_waitcnt(waitcnt_vm(2 * kWaveLoads));
      else if (has_page(it + 1)) __builtin_amdgcn_s_waitcnt(waitcnt_vm(kWaveLoads));
      else __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
    } else {
      if (kNBuf == 3 && it + 1 < ntiles && has_page(it + 1))
        __builtin_amdgcn_s_waitcnt(waitcnt_vm(kWaveLoads));
      else
        __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
    }
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
    if constexpr (kHalf) {
      // ---- a4/a5 (bf16, <= 16 rows): wave w contracts page w % 2 of the tile
      // over dims 288 (w / 2) .. + 287 against the 16-row tile; after one
      // exchange of the four partial tiles every wave holds the scores of
      // all 32 positions (its lane r16 + 16 g: positions 4g + i of each
      // page) and runs the tile's softmax itself, in the same order as the
      // others, so all four keep the same running maximum and sum, and writes
      // the probabilities to its own copy for its PV.
      {
        f32x4 s0 = f32x4{0.f, 0.f, 0.f, 0.f}, s1 = s0;
        const uint8_t* pg = tile + (w & 1) * G::kPageB;
        pipelined<9, 3, KR>([&](int ks) { return load_k8<FP8>(pg, r16, 288 * (w >> 1) + 32 * ks + 8 * g); },
                            [&](int ks, KR raw) {
                              if (ks & 1) s1 = mfma16(kop(raw), as_bf16x8(qreg[ks]), s1);
                              else s0 = mfma16(kop(raw), as_bf16x8(qreg[ks]), s0);
                            });
        *(f32x4*)(xbuf + (w * 64 + lane) * 4) = s0 + s1;
      }
      lds_barrier();
      float sv[8];
      float mx = kNegInf;
#pragma unroll
      for (int pp = 0; pp < 2; ++pp) {
        // page pp: dims 0..287 from wave pp, dims 288..575 from wave pp + 2
        const f32x4 lo = *(const f32x4*)(xbuf + (pp * 64 + lane) * 4);
        const f32x4 hi = *(const f32x4*)(xbuf + ((pp + 2) * 64 + lane) * 4);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int tt = 16 * pp + 4 * g + i;
          const bool ok = tt < tlim && tpos0 + tt < limA;
          sv[4 * pp + i] = ok ? (lo[i] + hi[i]) * c2 : kNegInf;
          mx = fmaxf(mx, sv[4 * pp + i]);
        }
      }
      mx = max32(max16(mx));
      const float mA = (mx > m_runA + kSlack) ? mx : m_runA;   // lazy rescale
      alphaA = (mA == m_runA) ? 1.f : __builtin_amdgcn_exp2f(m_runA - mA);
      m_runA = mA;
      uint8_t* const pme = p_lds + w * RPAD * kPRB;
      float ps = 0.f;
#pragma unroll
      for (int pp = 0; pp < 2; ++pp) {
        bf16x4 pb;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float v = sv[4 * pp + i];
          const float pr = (v == kNegInf) ? 0.f : __builtin_amdgcn_exp2f(v - mA);
          pb[i] = (__bf16)pr;
          ps += pr;
        }
        *(bf16x4*)(pme + r16 * kPRB + (16 * pp + 4 * g) * 2) = pb;
      }
      ps = sum32(sum16(ps));
      l_runA = l_runA * alphaA + ps;
    } else if constexpr (L16) {
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
      mx = max32(max16(mx));
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
      ps = sum32(sum16(ps));
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
        mx = max32(mx);
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
        ps = sum32(ps);
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
        mx = max32(max16(mx));
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
        ps = sum32(sum16(ps));
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
    if constexpr (kHalf) {
      // one 32-position k-step: probabilities 8g .. 8g + 7 of row r16 from
      // this wave's own copy (written above by this wave: LDS is in order)
      const bf16x8 pf = as_bf16x8(*(const u32x4*)(p_lds + w * RPAD * kPRB + r16 * kPRB + 16 * g));
      pipelined<8, 4, KR>([&](int i) { return load_v8<FP8>(tile, 8 * g, col0 + 16 * i, r16); },
                          [&](int i, KR raw) { o16a[i] = mfma16(kop(raw), pf, o16a[i]); });
    } else if constexpr (L16) {
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
  __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
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
    const int64_t row0 = FINAL ? (int64_t)b * R : wc.slot * R;
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
    const int64_t lrow = (FINAL ? (int64_t)b : wc.slot) * R + rb0 + r;
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
// to the 32x32x64 FP8 MFMA as stored, with no decode.  The other operand of
// each product is written as a sum of two FP8 terms:
//   query:         q * 2^e = q1 + q2, e chosen per row so max|q * 2^e| is in
//                  [64, 128); q has 8 significant bits and the residual of the
//                  first RNE rounding fits the second term, so q1 + q2 equals
//                  q * 2^e up to 2^-10 absolute, i.e. 2^-16 of the row maximum;
//   probabilities: per (row, 32-position block) x = 2^(s - f + 7) in [0, 256)
//                  against the block's own floor maximum f, x ~ p1 + p2 with
//                  |x - (p1 + p2)| <= max(2^-8 x, 2^-10), and the block's
//                  magnitude restored by the MFMA's E8M0 scale on that operand
//                  (see split_kernel_f8x64 for the bound on the output); the
//                  softmax denominator adds the fp32 x.
// Each product therefore takes two FP8 MFMAs, which cost what one bf16 MFMA of
// the same shape costs, and no VALU conversion touches the KV stream.
// Rows are two 32-row tiles (r = j*H + h); wave w owns row tile w/2 and the
// 32-position half w%2 of every 64-position tile; PV is column-split as above.
// ---------------------------------------------------------------------------
__device__ __forceinline__ f32x16 mfma_f8(i32x8 a, i32x8 b, f32x16 c) {
  // formats 0/0 = FP8 E4M3 for both operands; E8M0 scales 127 = 1.0
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
}
// The same with E8M0 scale code e (2^(e - 127)) on operand B, one code per
// lane: for B = P^T, lane l's code scales positions 32(l / 32) .. +31 of row l % 32.
__device__ __forceinline__ f32x16 mfma_f8s(i32x8 a, i32x8 b, f32x16 c, int e) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 127, 0, e);
}

__device__ __forceinline__ float bf16_lo(uint32_t v) { return __uint_as_float(v << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t v) { return __uint_as_float(v & 0xFFFF0000u); }
__device__ __forceinline__ float pow2f(int e) { return __uint_as_float((uint32_t)(e + 127) << 23); }

// Four bf16 query values (two dwords) q -> hi = RNE FP8 of q / isc and lo =
// RNE FP8 of (q - hi * isc) / isc, packed 4 per dword (isc a power of two).
// The scaled conversions divide by isc on the way to FP8 and multiply by it
// on the way back, exactly, so hi and lo are those of q * 2^e with isc = 2^-e.
__device__ __forceinline__ void split4_bf16_fp8(uint32_t d0, uint32_t d1, float isc, int& hi, int& lo) {
  const s16x2 z = {0, 0};
  s16x2 h = __builtin_amdgcn_cvt_scalef32_pk_fp8_bf16(z, __builtin_bit_cast(bf16x2, d0), isc, false);
  h = __builtin_amdgcn_cvt_scalef32_pk_fp8_bf16(h, __builtin_bit_cast(bf16x2, d1), isc, true);
  hi = __builtin_bit_cast(int, h);
  const f32x2 b01 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(hi, isc, false);
  const f32x2 b23 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(hi, isc, true);
  s16x2 l = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(z, __uint_as_float(d0 << 16) - b01[0],
                                                     __uint_as_float(d0 & 0xFFFF0000u) - b01[1], isc, false);
  l = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(l, __uint_as_float(d1 << 16) - b23[0],
                                               __uint_as_float(d1 & 0xFFFF0000u) - b23[1], isc, true);
  lo = __builtin_bit_cast(int, l);
}

// four fp32 values -> (RNE FP8 of each, RNE FP8 of each residual), packed 4 per dword
__device__ __forceinline__ void split4_fp8(float v0, float v1, float v2, float v3, int& hi, int& lo) {
  hi = __builtin_amdgcn_cvt_pk_fp8_f32(v0, v1, 0, false);
  hi = __builtin_amdgcn_cvt_pk_fp8_f32(v2, v3, hi, true);
  const f32x2 b01 = __builtin_amdgcn_cvt_pk_f32_fp8(hi, false);
  const f32x2 b23 = __builtin_amdgcn_cvt_pk_f32_fp8(hi, true);
  lo = __builtin_amdgcn_cvt_pk_fp8_f32(v0 - b01[0], v1 - b01[1], 0, false);
  lo = __builtin_amdgcn_cvt_pk_fp8_f32(v2 - b23[0], v3 - b23[1], lo, true);
}

// Byte offset, from a lane's value base, of the 8 positions
// 32(e/2) + 8(e%2) .. +7 (e < 4, relative to the lane half's first position)
// of column tile ct of the FP8 PV step (see the PV comment below).
constexpr int pv_voff(int ct, int e) {
  return (e >> 1) * 2 * KvGeom<true>::kPageB + 8 * (e & 1) * KvGeom<true>::kRowB +
         16 * (4 * (ct >> 1) + 2 * ((ct ^ e) & 1));
}

// The FP8 kernel issues its tile and query copies with copy16_to_lds, which
// the compiler does not see as LDS writes, so its key, value and probability
// reads are ordinary LDS loads that the compiler schedules between the
// MFMAs (with the copies visible it would wait for all of them before each
// read).  The copies of the tile being read were waited for explicitly
// before the barrier that published it.

// Value offsets of column tiles 0 and 1 (tiles 2 and 3 below).
static_assert(pv_voff(0, 0) == 0 && pv_voff(0, 1) == 4640 && pv_voff(0, 2) == 18432 &&
              pv_voff(0, 3) == 23072 && pv_voff(1, 0) == 32 && pv_voff(1, 1) == 4608 &&
              pv_voff(1, 2) == 18464 && pv_voff(1, 3) == 23040, "value offsets");

constexpr int kF8Waves = 8;
constexpr int kF8Threads = kF8Waves * 64;

// Value operand of one PV step: column tiles 0..3 (128 columns) x positions
// 16h + 0..15 and 32 + 16h + 0..15, sixteen transposed reads at the offsets
// pv_voff(ct, e).
static_assert(pv_voff(2, 0) == 64 && pv_voff(2, 1) == 4704 && pv_voff(2, 2) == 18496 &&
              pv_voff(2, 3) == 23136 && pv_voff(3, 0) == 96 && pv_voff(3, 1) == 4672 &&
              pv_voff(3, 2) == 18528 && pv_voff(3, 3) == 23104, "value offsets");

// Eight waves in two groups of four; group g owns query rows 32g..32g+31 and
// waves 4g..4g+3, and SIMD k runs wave k of group 0 and wave k of group 1.
// (Group 1 of a block of at most 48 rows is packed: its at most 16 rows
// carry both FP8 terms in one 32-row operand, see pk in the kernel.)
// Within a group, wave v = w & 3:
//   QK:  position half sp = v & 1 of the 64-position tile (a 32-position
//        block) and dimension half dh = v >> 1 (k-steps 0..4 or 5..8 of 64
//        dims): 80 registers of query fragments.  Partners v and v ^ 2 add
//        their partial scores through LDS by rows: wave dh takes rows
//        16dh..16dh+15 of its block and hands the partner the other 16, so
//        that all 32 scores of a (row, block) end up in one wave.
//   PV:  output columns 128v..128v+127 for the group's 32 rows.
// The groups run one phase apart (each phase ends with a workgroup barrier):
//   phase E(i): group 0: PV(i-1), QK(i)   | group 1: softmax(i-1)
//   phase O(i): group 0: softmax(i)       | group 1: PV(i-1), QK(i)
// so on every SIMD one wave issues MFMAs while the other does the softmax
// arithmetic.  QK(i) also reads the tile's value fragments into registers,
// so a tile is only read in E(i) and O(i): buffer (i + 2) % 3 can be refilled
// at the start of E(i), two tiles ahead.
//
// Probabilities enter the FP8 PV product as two E4M3 terms per value, scaled
// per (row, 32-position block).  E4M3 spans only about 18 binades, while a
// long history can hold most of its probability mass far below its maximum
// (tens of thousands of positions ten nats down carry more mass than the top
// one), so one scale per row would round that mass away, and FP32
// accumulation cannot bring back what the operand lost ("Inside Kimi K3
// optimization", technical note "KDA precision & on-chip memory").  Each
// block is therefore stored against its own maximum bm (log2 units): with
// f = floor(bm), x = 2^(s - f + 7) lies in [0, 256) with the block's largest
// value in [128, 256), x ~ hi + lo (hi = E4M3(x), lo = E4M3(x - hi)), and the
// MFMA's E8M0 block scale for operand B, 2^(f - 7 - m), restores the
// magnitude against the row's integer reference maximum m.  Per value
// |x - (hi + lo)| <= max(2^-8 x, 2^-10), so each block's weights are off by
// at most 2^-8 of its mass plus 2^-12 of its largest value: relative error
// <= 2^-8 + 2^-12 on the whole weight vector of a row, however wide the
// spread of the scores, hence |dout| <= (2^-8 + 2^-12) max|v|.  The row sum
// (and so lse) adds the fp32 x: a sum of the stored terms would carry their
// 2^-8 error into lse, up to 4e-3 in a row dominated by one position.  The
// reference m only sets the exponent range of the fp32 accumulators: it
// moves (by an exact power of two applied to O and l) when a tile maximum
// passes it by more than 2^kSlack, and nothing is ever recomputed.
template <bool FINAL, bool PACK>
__global__ __launch_bounds__(kF8Threads, 1) void split_kernel_f8x64(SplitArgs a) {
#if defined(__HIP_DEVICE_COMPILE__)  // the host pass only needs the launch stub
  using G = KvGeom<true>;
  constexpr int kNBuf = 3;
  constexpr int kTileB = kTilePages * G::kPageB;          // 36,864
  constexpr int kWaveLoads = G::kPageB / 1024;            // 9 wave-wide 1 KiB copies per page
  constexpr int kPRB = kTilePos + 16;                     // bytes per FP8 probability row (+skew)
  constexpr int kPTerm = 32 * kPRB;                       // 2560: second probability term
  // the reference maximum moves when a tile maximum passes it by more than
  // this (log2 units): stored weights stay below 2^(kSlack + 1), far from
  // fp32 overflow, and E8M0 block scales below 2^(kSlack - 7)
  constexpr float kSlack = 16.f;
  // floor of the maximum of a block with no visible position (its weights are 0)
  constexpr float kEmptyBlock = -1.0e30f;
  

  __shared__ __attribute__((aligned(16))) uint8_t kv_lds[kNBuf * kTileB];
  __shared__ __attribute__((aligned(16))) uint8_t p_lds[2][2 * kPTerm];   // [group][term][row][position]
  // partial scores after the QK exchange (see the MFMA phase): [wave][set][half][lane]
  __shared__ __attribute__((aligned(16))) f32x4 xbuf[kF8Waves][2][2][64];
  // per group and row: {f of block 0, f of block 1, fp32 weight sum of block 0, of block 1}
  __shared__ __attribute__((aligned(16))) f32x4 blk[2][32];
  __shared__ float qsc[64];   // 2^-e of each query row of the block

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int r32 = lane & 31;
  const int h = lane >> 5;
  const int grp = w >> 2;
  const int v4 = w & 3;
  const int sp = v4 & 1;
  const int dh = v4 >> 1;
  const int ks0 = dh ? 5 : 0;
  const int H = a.heads;
  const int R = a.num_q * H;
  const WgCoord wc = split_coord(a, (R + 63) / 64);
  const int split = wc.split;
  const int b = wc.b;
  // rows 64 * wc.z .. + 63 of the Q*H query rows are this workgroup's
  const int myrow = 64 * wc.z + 32 * grp + r32;
  // Packed group (PACK: launched for 33..48 query rows, one row block):
  // group 1 then has at most 16 real rows, so the two FP8 terms of its
  // operands share one 32-row MFMA operand instead of taking an MFMA each:
  // MFMA row n < 16 carries the first term of the group's row n, row n + 16
  // its second term.  Its score products and its output then come out as two
  // halves, added back per row (the scores in the softmax, the output in the
  // epilogue), and the group issues half the MFMAs of an unpacked one.  The
  // copies are placed differently too (see copies below).  Other row counts run
  // the kernel without any of it: carrying the packed code, the unpacked
  // blocks of the DCP8 shape ran 2.4% slower (more scalar registers, a
  // longer kernel).
  const bool pk = PACK && grp == 1;

  // seq_lens[b] is requested first (a scalar load, waited for below), then
  // the query block's loads go out: they need only the workgroup's
  // coordinates (see the query conversion below for the layout).
  const int L = kDebug ? debug_seq_len(a.seq_lens[b], a.num_q, a.max_blocks, a.debug_flags) : a.seq_lens[b];
  uint8_t* const qlds = kv_lds + kTileB;
  {
    const int nrows = min(64, R - 64 * wc.z);
    const u32x4 qrsrc = buffer_rsrc(a.q + ((int64_t)b * R + 64 * wc.z) * kLatent, nrows * 2 * kLatent);
#pragma unroll
    for (int i = 0; i < 9; ++i) {
      const int slot = 64 * (w + 8 * i) + lane;   // 16-byte LDS slot of this lane
      const int r = slot / 72, x = slot - 72 * (slot / 72);
      const uint32_t src = 16u * (uint32_t)(72 * r + (x ^ (r & 7)));
      copy16_to_lds(qrsrc, src, lds_addr(qlds + 1024 * (w + 8 * i)));
    }
  }
  __builtin_amdgcn_sched_barrier(0);
  const int P = (L + kPage - 1) / kPage;
  // page range [floor(split P / S), floor((split + 1) P / S)) in 32-bit
  // arithmetic: floor(s P / S) = s floor(P / S) + floor(s (P mod S) / S)
  const int S = wc.nsplit;
  const int pq = P / S, pr = P - pq * S;
  const int p0 = split * pq + (split * pr) / S;
  const int p1 = (split + 1) * pq + ((split + 1) * pr) / S;
  const int ntiles = (p1 - p0 + kTilePages - 1) / kTilePages;

  // An opaque copy of the lane index, taken where a lane-dependent address or
  // bound is needed inside the loop: derived from it there (one or two VALU
  // operations), the value does not hold a register of its own across the
  // loop, where nearly every register is taken.
  auto lane_now = [&]() -> int {
    int l = lane;
    asm volatile("" : "+v"(l));
    return l;
  };
  // ---- a2: copies.  Tile T goes to LDS buffer T % 3; wave w copies page
  // w % 4 (wave-wide one-KiB loads from one buffer descriptor).  Tiles 0
  // and 1 are copied in the prologue, whole pages: tile 0 by waves 0..3 as
  // soon as its page-table entries are known, tile 1 by waves 4..7 once every
  // wave has read the query staged in buffers 1 and 2.  Each tile T >= 2 is
  // copied by both groups while they run their softmax, two tiles ahead:
  // group 1 loads 0..kLoads1-1 of each page at E(T - 2), group 0 the rest at
  // O(T - 2), so the copy issue never sits on the MFMA-role path and is shared
  // between the two softmax phases.  In a packed workgroup (see pk below) the
  // two group-1 waves with no softmax rows (dh = 1) copy whole pages v4 and
  // v4 ^ 2 at E(T - 2) and no other wave copies: no softmax wave waits on a
  // copy issue (FP8 verify of 64 sequences, 3 x 12 rows: split kernel -4%;
  // long context, 4 x 35,500 positions: -1.6%, against the shared
  // copies, same-box timing).  A page outside the split, or the
  // positions past seq_len in the last page, lie outside the buffer range and
  // are written to LDS as zeros by the copy itself.
  // Page-table entry of page pg (v4 unless given) of tile T (entries past the sequence are
  // clamped to its last page and not used), read through the constant
  // address space: the index is wave-uniform, so this is a scalar load,
  // which does not count against vmcnt.
  constexpr int kLoads1 = 5;   // group 1's share of a page's nine loads
  const __attribute__((address_space(4))) int32_t* pt_b =
      (const __attribute__((address_space(4))) int32_t*)(a.page_table + (int64_t)b * a.max_blocks);
  const int plast = max(P - 1, 0);
  auto pt_load_pg = [&](int T, int pg) -> int {
    return pt_b[min(p0 + T * kTilePages + pg, plast)];
  };
  auto pt_load = [&](int T) -> int { return pt_load_pg(T, v4); };
  // loads C0 .. C1 - 1 (compile-time range) of page pg of tile T
  auto issue_page = [&](int T, int pg, int ptv, auto C0, auto C1) {
    constexpr int c0 = decltype(C0)::value, c1 = decltype(C1)::value;
    const int gp = p0 + T * kTilePages + pg;
    int blk = __builtin_amdgcn_readfirstlane(ptv);
    if constexpr (kDebug) blk = gp < p1 ? debug_page_id(blk, a.num_blocks, a.debug_flags) : 0;
    const int bytes = gp < p1 ? min(kPage, L - gp * kPage) * G::kRowB : 0;
    const u32x4 rsrc = buffer_rsrc(a.kv + (int64_t)(gp < p1 ? blk : 0) * G::kPageB, bytes);
    uint8_t* dst = kv_lds + (T % kNBuf) * kTileB + pg * G::kPageB;
    // LDS slot s = 64c + lane of the page holds source chunk
    // 36 row + (x ^ swz(row)) with row = s / 36, x = s % 36.  As 36 is a
    // multiple of 4 the XOR only touches the two low bits, so the source chunk
    // is s ^ swz(s / 36) = s ^ (s / 144), and s / 144 = d0 + (lane >= t) with
    // d0 = 64c / 144 and t = 144 (d0 + 1) - 64c known per load: one or three
    // VALU operations per load instead of a division.
    static_assert(G::kChunksPerRow == 36, "FP8 page rows of 36 chunks");
    // derived from an opaque copy of the lane index: hoisted out of the loop,
    // the offsets would hold registers (or spill) between copies
    const int ln = lane_now();
    const uint32_t vb = 16u * (uint32_t)ln;
#pragma unroll
    for (int c = c0; c < c1; ++c) {
      constexpr int kRowsPerSwz = 4 * G::kChunksPerRow;   // 144 slots per swizzle value
      const int d0 = (64 * c) / kRowsPerSwz;
      const int t = kRowsPerSwz * (d0 + 1) - 64 * c;
      const uint32_t d = (uint32_t)d0 + ((t < 64 && ln >= t) ? 1u : 0u);
      const uint32_t voff = (vb + 1024u * (uint32_t)c) ^ (d << 4);
      if constexpr (PACK) copy16_to_lds_nt(rsrc, voff, lds_addr(dst + 1024 * c));
      else copy16_to_lds(rsrc, voff, lds_addr(dst + 1024 * c));
    }
  };
  auto issue_part = [&](int T, int ptv, auto C0, auto C1) { issue_page(T, v4, ptv, C0, C1); };
  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, kLoads1>;
  using I9 = std::integral_constant<int, kWaveLoads>;

  // ---- query: q * 2^e = q1 + q2 (FP8), dims 64(ks0 + ks) + 32h + j of row `myrow`.
  // The workgroup's 64 query rows (1,152 bytes each) are staged once in KV
  // buffers 1 and 2 (exactly 73,728 bytes) by direct-to-LDS loads, 16 bytes a
  // lane: read by every wave straight from memory, the same rows would be
  // requested twice per workgroup at kernel start, when every workgroup's
  // first loads queue up.  Rows past Q*H lie outside the buffer range and
  // arrive as zeros.  Chunk j of row r sits at chunk (j & ~7) | ((j ^ r) & 7)
  // of its LDS row, so the 16 rows one ds_read_b128 phase reads fall in
  // distinct bank groups (two-way at most).
  // Each row is converted once per workgroup, in place: wave w takes rows
  // 8w .. 8w + 7, eight lanes a row and nine 16-byte chunks a lane (chunks
  // l % 8 + 8i), finds the row's exponent e with the other seven lanes of
  // the row, and writes the two FP8 terms over the row's own 1,152 bytes:
  // term t at byte 576 t of the row, its 16-byte chunk x at chunk
  // x ^ ((r / 2) % 4) (rows 1,152 bytes apart fall on two bank offsets; the
  // XOR, inside each group of four chunks, spreads 16 rows over 8 of them).
  // A wave writes only the rows it has itself read, so no barrier sits
  // between the reads and the writes.  Waves whose rows are all padding only
  // write zeros.
  i32x8 q1[5], q2[5];
  int ptA, ptB;   // page-table entries of page v4 of the next two tiles to copy
  const int pt0 = pt_load(grp);   // page v4 of the group's first tile
  {
    ptA = pt_load(2);
    ptB = pt_load(3);
    // The probability terms and block data read by each group's first PV
    // are zeros (that PV adds nothing; published by the barrier below).
    for (int i = tid; i < (int)(sizeof(p_lds) / 16); i += kF8Threads) ((u32x4*)p_lds)[i] = u32x4{};
    if (tid < 64) blk[tid >> 5][tid & 31] = f32x4{kEmptyBlock, kEmptyBlock, 0.f, 0.f};
    // tile 0's copies go out as soon as its page-table entries are known
    // (group 0; buffer 0 is not part of the staged query)
    if (grp == 0) {
      issue_part(0, pt0, I0{}, I9{});
      __builtin_amdgcn_s_waitcnt(waitcnt_vm(kWaveLoads));   // this wave's query loads
    } else {
      __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
    }
    lds_barrier();   // every wave's query loads have landed
    {
      const int crow = 8 * w + (lane >> 3);          // the lane's row within the block
      uint8_t* const rowp = qlds + crow * (2 * kLatent);
      const int sw = (crow >> 1) & 3;
      u32x2 th[9], tl[9];                            // terms of the lane's nine chunks
      float isc = 1.f;
      if (8 * w < min(64, R - 64 * wc.z)) {
        u32x4 c[9];
#pragma unroll
        for (int i = 0; i < 9; ++i) c[i] = *(const u32x4*)(rowp + 16 * (8 * i + ((lane ^ crow) & 7)));
        // largest magnitude of the row: the magnitude bits of bf16 values
        // order as integers, two per dword (packed 16-bit maximum)
        u16x2 mk = {0, 0};
#pragma unroll
        for (int i = 0; i < 9; ++i)
#pragma unroll
          for (int k = 0; k < 4; ++k)
            mk = __builtin_elementwise_max(mk, __builtin_bit_cast(u16x2, c[i][k] & 0x7FFF7FFFu));
        float mx = __uint_as_float((uint32_t)max(mk[0], mk[1]) << 16);
        mx = max8(mx);   // the row's eight lanes
        int e = 0;
        if (mx > 0.f) {
          const int ex = (int)((__float_as_uint(mx) >> 23) & 0xFF) - 126;  // mx = m * 2^ex, m in [0.5, 1)
          e = min(max(7 - ex, -100), 100);
        }
        isc = pow2f(-e);
#pragma unroll
        for (int i = 0; i < 9; ++i) {
          int h0, l0, h1, l1;
          split4_bf16_fp8(c[i][0], c[i][1], isc, h0, l0);
          split4_bf16_fp8(c[i][2], c[i][3], isc, h1, l1);
          th[i] = u32x2{(uint32_t)h0, (uint32_t)h1};
          tl[i] = u32x2{(uint32_t)l0, (uint32_t)l1};
        }
      } else {
#pragma unroll
        for (int i = 0; i < 9; ++i) th[i] = tl[i] = u32x2{0u, 0u};
      }
      // bf16 chunk j = l % 8 + 8i holds dims 8j .. 8j + 7: bytes 8(j % 2) of
      // FP8 chunk j / 2 = 4i + (l % 8) / 2 of each term
#pragma unroll
      for (int i = 0; i < 9; ++i) {
        uint8_t* const p = rowp + 16 * (4 * i + (((lane & 7) >> 1) ^ sw)) + 8 * (lane & 1);
        *(u32x2*)p = th[i];
        *(u32x2*)(p + kLatent) = tl[i];
      }
      if ((lane & 7) == 0) qsc[crow] = isc;
    }
    lds_barrier();   // every row's terms and scale are in place
    {
      // the lane's fragment row (packed: first term of row r32 for lanes of
      // rows 0..15, second term of row r32 - 16 for the others)
      const int lr = pk ? 32 + (r32 & 15) : 32 * grp + r32;
      const uint8_t* const fb = qlds + lr * (2 * kLatent) + 64 * ks0 + (pk && r32 >= 16 ? kLatent : 0);
      const int sw = (lr >> 1) & 3;
      const int o0 = 16 * ((2 * h) ^ sw), o1 = 16 * ((2 * h + 1) ^ sw);
      auto frag = [&](int off) -> i32x8 {
        const u32x4 x0 = *(const u32x4*)(fb + off + o0);
        const u32x4 x1 = *(const u32x4*)(fb + off + o1);
        return __builtin_bit_cast(i32x8, u32x8{x0[0], x0[1], x0[2], x0[3], x1[0], x1[1], x1[2], x1[3]});
      };
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        q1[ks] = frag(64 * ks);
        q2[ks] = pk ? i32x8{} : frag(64 * ks + kLatent);   // (packed: not used)
      }
      // dh = 1 has four k-steps: its fifth query terms are zeros
      q1[4] = dh ? i32x8{} : frag(256);
      q2[4] = (dh || pk) ? i32x8{} : frag(256 + kLatent);
    }
  }
  // scale into the log2 domain of the scores this lane handles in the
  // softmax: row 16dh + l % 16 of the group
  const float cs = a.score_scale_log2 * qsc[32 * grp + 16 * dh + (lane & 15)];
  lds_barrier();   // every wave has read its query terms
  if (grp == 1) {
    issue_part(1, pt0, I0{}, I9{});
    __builtin_amdgcn_sched_barrier(0);
  }

  // Integer reference maximum of row r32 of this wave's group (log2 units),
  // the row sum and the output of this wave's 128 columns x the group's 32
  // rows, all relative to 2^mref.
  float mref = kNegInf;
  float l_run = 0.f;
  f32x16 o[4];
#pragma unroll
  for (int c = 0; c < 4; ++c) o[c] = f32x16{};
  i32x8 vfr[4];     // value fragments of the group's next PV (zeros before the first)
#pragma unroll
  for (int c = 0; c < 4; ++c) vfr[c] = i32x8{};

  uint8_t* const pg_lds = p_lds[grp];

  // Row (within the group) of the lane's scores in the softmax: 16dh + l % 16.
  auto srow_now = [&]() -> int { return (lane_now() & 15) + 16 * dh; };
  // Causal limit of that row (visible: position < lim), needed on edge tiles
  // only and recomputed there (with an opaque divisor, so that the division's
  // reciprocal is not kept either).
  auto lim_now = [&]() -> int {
    int hd = H;
    asm volatile("" : "+s"(hd));
    return L - a.num_q + (64 * wc.z + 32 * grp + srow_now()) / hd + 1;
  };
  // Lane-dependent LDS offsets, likewise derived where they are used.
  // Value operand base (see qk below).
  auto vbase_now = [&]() -> int {
    const int ln = lane_now();
    const int s16 = ln & 15;
    return (ln >> 5) * G::kPageB + (s16 >> 1) * G::kRowB +
           16 * (8 * v4 + (((ln >> 4) ^ (s16 >> 3)) & 1)) + 8 * (s16 & 1);
  };
  // First position (within the block) of the lane's softmax scores: they
  // are 16u + 8(k/4) + 4h + k%4, k < 8, with u = 1 for the lanes that hold
  // elements 8..15 of their row (lanes of rows 16..31, see qk).
  auto spos_now = [&]() -> int {
    const int ln = lane_now();
    return 16 * ((ln >> 4) & 1) + 4 * (ln >> 5);
  };

  // ---- a4: partial S^T over this wave's k-steps.
  // Key operand of k-step ks (relative to the wave's first, ks0) of tile T:
  // 16 bytes at each of chunks 2h and 2h + 1 of the k-step's 64 dims of the
  // lane's position row (XOR-swizzled within the row's 4-chunk groups).
  auto kptr = [&](int T) -> const uint8_t* {
    const int ln = lane_now();
    const int prow = ln & 15;
    const int kpage = 2 * sp + ((ln >> 4) & 1);
    return kv_lds + (T % kNBuf) * kTileB + kpage * G::kPageB + G::off(prow, 2 * (ln >> 5), 0) + 64 * ks0;
  };
  // distance from chunk 2h to chunk 2h + 1 after the swizzle: +16 or -16 bytes
  auto kpair = [&]() -> int {
    const int ln = lane_now();
    return ((ln & 15) >> 2) & 1 ? -16 : 16;
  };
  auto kop = [&](const uint8_t* kp, int d1, int ks) -> i32x8 {
    const u32x4 x0 = *(const u32x4*)(kp + 64 * ks);
    const u32x4 x1 = *(const u32x4*)(kp + 64 * ks + d1);
    return __builtin_bit_cast(i32x8, u32x8{x0[0], x0[1], x0[2], x0[3], x1[0], x1[1], x1[2], x1[3]});
  };
  // Value operand of the PV (read for the next phase once this phase's PV
  // has used the registers; the tile is not read after this phase).  The PV
  // product's K index runs over the tile's 64 positions so that each
  // 32-index block of its E8M0 scales (bytes 0..15 of both lane halves, then
  // bytes 16..31 of both) is one position block of the softmax: lane half h,
  // byte j holds position 32(j/16) + 16h + j%16.  Column tile ct, bytes
  // 8e .. 8e+7: source lane sl of a 16-lane group reads position
  // 32(e/2) + 16h + 8(e%2) + sl/2, i.e. page h + 2(e/2), row 8(e%2) + sl/2,
  // byte half sl%2 of chunk 8v + 2ct + (g16%2), XOR-swizzled by
  // (row/4)%4 = sl/8 + 2(e%2); vbase is the lane part of that address and
  // pv_voff(ct, e) the rest.
  auto vread = [&](const uint8_t* vp, int ct) -> i32x8 {
    u32x2 vr[4];
#pragma unroll
    for (int e = 0; e < 4; ++e)
      vr[e] = __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr8_b64_v2i32(LDS_PTR(i32x2, vp + pv_voff(ct, e))));
    return __builtin_bit_cast(i32x8, u32x8{vr[0][0], vr[0][1], vr[1][0], vr[1][1], vr[2][0], vr[2][1], vr[3][0], vr[3][1]});
  };
  // Partial scores to the softmax.  Rows 16dh..16dh+15 are finished by this
  // wave, the other 16 by the partner (wave w ^ 2, the other dimension
  // half), 8 scores per lane either way.  Lane l (row l % 32, position half
  // h) holds elements 0..15 of its row.  One lane swap between lanes l and
  // l ^ 16 per element pair (k, k + 8) gives set 0 (the lanes of rows 0..15
  // with their elements 0..7, the lanes of rows 16..31 with elements 8..15 of
  // row (l % 32) - 16: rows 0..15) and set 1 (rows 16..31 likewise); both
  // sets go to LDS, and the softmax of wave w adds set dh of wave w and of
  // its partner.
  auto send_scores = [&](const f32x16& s) {
    uint32_t r0[8], r1[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(s[k]), __float_as_uint(s[k + 8]),
                                                      false, false);
      r0[k] = r[0];
      r1[k] = r[1];
    }
    const int ln = lane_now();
    xbuf[w][0][0][ln] = __builtin_bit_cast(f32x4, u32x4{r0[0], r0[1], r0[2], r0[3]});
    xbuf[w][0][1][ln] = __builtin_bit_cast(f32x4, u32x4{r0[4], r0[5], r0[6], r0[7]});
    xbuf[w][1][0][ln] = __builtin_bit_cast(f32x4, u32x4{r1[0], r1[1], r1[2], r1[3]});
    xbuf[w][1][1][ln] = __builtin_bit_cast(f32x4, u32x4{r1[4], r1[5], r1[6], r1[7]});
  };

  // ---- a5: partner's partial scores added, scale to log2 units, mask (edge
  // tiles only), block maximum, probabilities as two FP8 terms against it.
  // Element k of x is position spos + 8(k/4) + k%4 of block sp of row
  // 16dh + l % 16; lanes l, l ^ 16, l ^ 32 and l ^ 48 together hold the
  // row's whole block.
  auto softmax = [&](int T) {
    float x[8];
    {
      const int ln = lane_now();
      const f32x4 a0 = xbuf[w][dh][0][ln];
      const f32x4 a1 = xbuf[w][dh][1][ln];
      const f32x4 u0 = xbuf[w ^ 2][dh][0][ln];
      const f32x4 u1 = xbuf[w ^ 2][dh][1][ln];
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        x[k] = a0[k] + u0[k];
        x[4 + k] = a1[k] + u1[k];
      }
      if (pk) {
        // packed group (only its dh = 0 waves run the softmax): set 1 holds
        // the second query term's products of the same rows, lane for lane
        const f32x4 b0 = xbuf[w][1][0][ln];
        const f32x4 b1 = xbuf[w][1][1][ln];
        const f32x4 t0 = xbuf[w ^ 2][1][0][ln];
        const f32x4 t1 = xbuf[w ^ 2][1][1][ln];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          x[k] += b0[k] + t0[k];
          x[4 + k] += b1[k] + t1[k];
        }
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
      // position tq = 32 sp + spos + (8 (k / 4) + k % 4) is visible when it
      // is below both tlim and lim - tpos0
      const int kvis = min(tlim, lim_now() - tpos0) - (32 * sp + spos_now());
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        x[k] = 8 * (k >> 2) + (k & 3) < kvis ? x[k] * cs : kNegInf;
        mx = fmaxf(mx, x[k]);
      }
    }
    mx = max16(max32(mx));                            // the block's maximum
    const float f = mx == kNegInf ? kEmptyBlock : floorf(mx);
    const float c0 = 7.f - f;
    float ws = 0.f;
    int hi[2], lo[2];
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      float p4[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) p4[i] = __builtin_amdgcn_exp2f(x[4 * q + i] + c0);
      ws += (p4[0] + p4[1]) + (p4[2] + p4[3]);
      split4_fp8(p4[0], p4[1], p4[2], p4[3], hi[q], lo[q]);
    }
    ws = sum16(sum32(ws));
    {
      const int row = srow_now();
      const int pos = spos_now();
      uint8_t* const pp = pg_lds + row * kPRB + 32 * sp + pos;
      *(int*)pp = hi[0];
      *(int*)(pp + 8) = hi[1];
      *(int*)(pp + kPTerm) = lo[0];
      *(int*)(pp + kPTerm + 8) = lo[1];
      if (pos == 0) {   // one lane per row: u = 0, h = 0
        float* const bp = (float*)&blk[grp][row];
        bp[sp] = f;
        bp[2 + sp] = ws;
      }
    }
  };

  // Reference maximum of the lane's row, checked in each MFMA phase: it
  // moves to the tile maximum when that passes it by more than 2^kSlack (O
  // and l are rescaled by the exact power of two), then the E8M0 codes of the
  // two blocks against it, 127 + f - 7 - mref (at least 0: a block more than
  // 2^120 below the reference weighs at most 2^-119 of it), and the row sum
  // of the tile under the same codes.  Returns the code of the lane's own
  // block (the B operand's scale of its PV lane).  `s` is the score
  // accumulator of the MFMAs issued before the check: named in the (rarely
  // taken) rescale branch so that the compiler keeps those MFMAs ahead of the
  // branch instead of moving them to the join, where they would wait for it.
  auto rebase = [&](const f32x4 bk, const f32x16& s) -> int {
    const float tm = fmaxf(bk[0], bk[1]);
    const bool mv = tm > mref + kSlack;
    const float mn = mv ? tm : mref;
    // nothing to rescale while no weight has been added (then O is exactly
    // zero): the first tiles, whose maxima always move the reference, skip it
    if (__any(mv && l_run > 0.f)) {
      const float alpha = mv ? __builtin_amdgcn_exp2f(mref - mn) : 1.f;   // integer argument
      l_run *= alpha;
      o[0] *= alpha;
      o[1] *= alpha;
      o[2] *= alpha;
      o[3] *= alpha;
      asm volatile("" ::"v"(s));
    }
    mref = mn;
    const int e0 = (int)fminf(fmaxf(120.f + bk[0] - mn, 0.f), 254.f);
    const int e1 = (int)fminf(fmaxf(120.f + bk[1] - mn, 0.f), 254.f);
    l_run += ldexpf(bk[2], e0 - 127) + ldexpf(bk[3], e1 - 127);
    return h ? e1 : e0;
  };

  // Half-steps hs = 0, 1, ...: E(i) = 2i, O(i) = 2i + 1.  Group 0 runs
  // MFMA(T) (QK of tile T, PV of tile T - 1) at hs = 2T and softmax(T) at
  // 2T + 1; group 1 one half-step later, after an idle first one.  Each
  // group's loop holds one MFMA phase and one softmax phase; the partial
  // scores pass from QK to the softmax through LDS.  Both groups start
  // 2 ntiles + 2 half-steps, each with one workgroup barrier.  Tile 0 (group
  // 0's prologue copies) has landed before the loop; tile 1 (group 1's) only
  // before E(1).
  // Start of a half-step: the copy waits and the workgroup barrier.  A
  // group's vector-memory order is its share of tiles 2, 3, 4 ... (group 1:
  // tile 1 whole before them): before E(T), T >= 1, its share of tile T must
  // have landed while that of tile T + 1 may still be in flight.
  // In a packed workgroup the copying waves (group 1, dh = 1) have tile
  // T + 1's 18 loads in flight at most, group 1's other waves only their
  // share of tile 1, and group 0 no copy in the loop.
  auto begin = [&](int hs, auto PKc) {
    if ((hs & 1) == 0 && hs >= 2) {
      if constexpr (decltype(PKc)::value) {   // group 1, packed
        if (dh) __builtin_amdgcn_s_waitcnt(waitcnt_vm(2 * kWaveLoads));
        else __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
      } else if (grp) {
        __builtin_amdgcn_s_waitcnt(waitcnt_vm(kLoads1));
      } else if constexpr (!PACK) {
        __builtin_amdgcn_s_waitcnt(waitcnt_vm(kWaveLoads - kLoads1));
      }
    }
    lds_barrier();
  };
  // End of a half-step: group 1 copies at even half-steps (hs = 0 and its
  // softmax phases), group 0 at odd ones (its softmax phases), after the
  // softmax work (issued first, a copy that stalls on a full memory queue
  // would hold the softmax up).  The page-table entries are scalar loads,
  // requested two tiles ahead (the copying waves of a packed workgroup read
  // their second page's entry when they issue: they have no other work then).
  auto copies = [&](int hs, auto PKc) {
    const int it = hs >> 1;
    auto next_entries = [&]() {
      const int nxt = pt_load(it + 4);
      if (it & 1) ptB = nxt;
      else ptA = nxt;
    };
    if constexpr (decltype(PKc)::value) {   // group 1, packed: its dh = 1 waves copy everything
      if ((hs & 1) == 0 && dh) {
        const int cur = (it & 1) ? ptB : ptA;
        const int cur2 = pt_load_pg(it + 2, v4 ^ 2);
        issue_page(it + 2, v4, cur, I0{}, I9{});
        issue_page(it + 2, v4 ^ 2, cur2, I0{}, I9{});
        next_entries();
      }
    } else if ((hs & 1) == 1 - grp && !(PACK && grp == 0)) {
      const int cur = (it & 1) ? ptB : ptA;
      if (grp) issue_part(it + 2, cur, I0{}, I1{});
      else issue_part(it + 2, cur, I1{}, I9{});
      next_entries();
    }
  };
  // MFMA role, the phase's critical path (its instructions go first on the
  // SIMD it shares with a softmax-role wave).  The block data, the PV's
  // probability terms and the first two key operands are requested at the
  // start; the score MFMAs run first (they need only the keys), the
  // reference maximum is checked while they run, then the PV MFMAs of the
  // previous tile, column tile by column tile, each followed by the value
  // reads of this tile into the registers it has just consumed, with the
  // score exchange between them.  PV and QK run in every MFMA phase: at T = 0
  // the probability terms, block data and value fragments are zeros (PV adds
  // nothing), and past the last tile QK reads a stale buffer and its results
  // are never used.
  // ---- a6: O^T[c][r] += V^T[c][t] (p1 + p2)^T[t][r], columns 128v .. 128v + 127,
  // with the block's E8M0 scale on operand B.
  // Packed (PK): one MFMA per k-step and per column tile, the operand rows
  // carrying both terms (MFMA row n: row n % 16 of the group, term n / 16);
  // the block data of MFMA row n are those of row n % 16.
  auto mfma_phase = [&](int T, auto PKc) {
    constexpr bool PK = decltype(PKc)::value;
    __builtin_amdgcn_s_setprio(2);
    const int ln = lane_now();
    const int row = PK ? (ln & 15) : (ln & 31);
    const f32x4 bk = blk[grp][row];
    const uint8_t* kp = kptr(T);
    const int d1 = kpair();
    i32x8 ka = kop(kp, d1, 0);
    i32x8 kb = kop(kp, d1, 1);
    i32x8 pf[2];
    {
      const uint8_t* pp = pg_lds + row * kPRB + 16 * (ln >> 5) + (PK && (ln & 16) ? kPTerm : 0);
      const u32x4 a0 = *(const u32x4*)pp;
      const u32x4 a1 = *(const u32x4*)(pp + 32);
      pf[0] = __builtin_bit_cast(i32x8, u32x8{a0[0], a0[1], a0[2], a0[3], a1[0], a1[1], a1[2], a1[3]});
      if constexpr (!PK) {
        const u32x4 b0 = *(const u32x4*)(pp + kPTerm);
        const u32x4 b1 = *(const u32x4*)(pp + kPTerm + 32);
        pf[1] = __builtin_bit_cast(i32x8, u32x8{b0[0], b0[1], b0[2], b0[3], b1[0], b1[1], b1[2], b1[3]});
      }
    }
    // one k-step (both query terms unless packed) and one column tile of PV
    auto qk = [&](const i32x8& k, int ks, f32x16 acc) -> f32x16 {
      acc = mfma_f8(k, q1[ks], acc);
      if constexpr (!PK) acc = mfma_f8(k, q2[ks], acc);
      return acc;
    };
    auto pv = [&](int c, int e) {
      o[c] = mfma_f8s(vfr[c], pf[0], o[c], e);
      if constexpr (!PK) o[c] = mfma_f8s(vfr[c], pf[1], o[c], e);
    };
    constexpr int kT = PK ? 1 : 2;   // MFMAs per k-step and per column tile
    f32x16 s = f32x16{};
    s = qk(ka, 0, s);
    const int e = rebase(bk, s);
    ka = kop(kp, d1, 2);
    s = qk(kb, 1, s);
    kb = kop(kp, d1, 3);
    s = qk(ka, 2, s);
    // the dh = 1 waves have four k-steps: their fifth reuses the fourth's
    // keys against zero query terms (no branch, so the phase is one block;
    // the dh = 0 waves on the other SIMDs run five steps anyway)
    ka = kop(kp, d1, dh ? 3 : 4);
    s = qk(kb, 3, s);
    s = qk(ka, 4, s);
    const uint8_t* vp = kv_lds + (T % kNBuf) * kTileB + vbase_now();
    // written out: a rolled loop here makes the compiler rotate the four
    // accumulators through one register window with moves
    pv(0, e);
    vfr[0] = vread(vp, 0);
    pv(1, e);
    vfr[1] = vread(vp, 1);
    send_scores(s);
    pv(2, e);
    vfr[2] = vread(vp, 2);
    pv(3, e);
    vfr[3] = vread(vp, 3);
    // Order after the rescale check: each k-step's key reads two MFMAs ahead
    // of their use, then the PV pairs with each column tile's value reads after it
    // and the score exchange's LDS writes in the middle.
    __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);        // keys, step 2
    __builtin_amdgcn_sched_group_barrier(0x008, kT, 0);       // QK, step 1
    __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);        // keys, step 3
    __builtin_amdgcn_sched_group_barrier(0x008, kT, 0);       // QK, step 2
    __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);        // keys, step 4
    __builtin_amdgcn_sched_group_barrier(0x008, 2 * kT, 0);   // QK, steps 3 and 4
    __builtin_amdgcn_sched_group_barrier(0x008, kT, 0);       // PV, column tile 0
    __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);        // values 0
    __builtin_amdgcn_sched_group_barrier(0x008, kT, 0);       // PV 1
    __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);        // values 1
    __builtin_amdgcn_sched_group_barrier(0x200, 4, 0);        // scores to LDS
    __builtin_amdgcn_sched_group_barrier(0x008, kT, 0);       // PV 2
    __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);        // values 2
    __builtin_amdgcn_sched_group_barrier(0x008, kT, 0);       // PV 3
    __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);        // values 3
    __builtin_amdgcn_s_setprio(0);
  };
  if (grp == 0) __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
  // A group whose 32 rows all lie past Q*H (group 1 of the last row block
  // when Q*H is an odd multiple of 32) does no matrix or softmax work: its
  // waves only take part in the barriers and issue their share of the copies.
  const bool live = 64 * wc.z + 32 * grp < R;
  // The packed and unpacked groups run separate copies of the loop (one
  // loop holding both MFMA phases would need more registers than a wave has).
  auto run = [&](auto PKc) {
    for (int hs = 0; hs <= 2 * ntiles + 1; ++hs) {
      begin(hs, PKc);
      const int st = hs - grp;
      if (live && st >= 0 && (st & 1) == 0) {
        mfma_phase(st >> 1, PKc);
      } else if (live && st >= 1 && !(decltype(PKc)::value && dh)) {   // (packed: dh = 1 has no rows)
        const int T = (st - 1) >> 1;
        if (T < ntiles) softmax(T);
      }
      copies(hs, PKc);
    }
  };
  if constexpr (PACK) {
    if (pk) run(std::true_type{});
    else run(std::false_type{});
  } else {
    run(std::false_type{});
  }

  // No copy may still be writing this workgroup's LDS when it ends, and the
  // epilogue reuses the KV buffers: every wave's copies have landed.
  __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
  lds_barrier();

  // ---- a7: epilogue.  O and l are relative to 2^mref.  Each wave's
  // 32 rows x 128 columns go through LDS (the free KV buffers) so that a store
  // instruction writes four whole 256-byte row segments; stored straight from
  // the accumulators, each instruction would touch 32 rows with 16 bytes each.
  {
    constexpr int kSRow = 256 + 16;   // staged row stride (bytes), skewed against bank conflicts
    static_assert(kF8Waves * 32 * kSRow <= kNBuf * kTileB, "epilogue staging fits the KV buffers");
    uint8_t* const stage = kv_lds + w * 32 * kSRow;
    const float sc = l_run > 0.f ? a.out_scale / l_run : 0.f;
    if (pk) {
      // packed: output row n % 16 is the sum of MFMA rows n and n ^ 16 (the
      // two probability terms), held by lanes l and l ^ 16; both lanes of a
      // pair add in the same order, and only rows 0..15 are stored
#pragma unroll
      for (int ct = 0; ct < 4; ++ct)
#pragma unroll
        for (int k = 0; k < 16; ++k) o[ct][k] = sum16(o[ct][k]);
    }
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
    const int64_t row0 = FINAL ? (int64_t)b * R : wc.slot * R;
    const int cc = 8 * (lane & 15);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int r = 4 * j + (lane >> 4);
      const int grow = 64 * wc.z + 32 * grp + r;
      const u32x4 v = *(const u32x4*)(stage + r * kSRow + 2 * cc);
      if (grow < R) {
        u32x4* const gp = (u32x4*)(dst + (row0 + grow) * kValue + 128 * v4 + cc);
        // partials of the packed form go out non-temporally: the merge reads
        // each once, from other XCDs (long context, 4 x 35,500 positions:
        // layer-step -1.1%, same box; the DCP8 shape's 75 MB of partials ran
        // slower so, and its unpacked form stores them as usual)
        if constexpr (PACK && !FINAL) __builtin_nontemporal_store(v, gp);
        else *gp = v;
      }
    }
  }
  if (myrow < R && v4 == 0 && h == 0) {
    const float lv = (l_run > 0.f) ? (mref + log2f(l_run)) * kLn2 : kNegInf;
    if constexpr (FINAL) a.lse[(int64_t)b * R + myrow] = lv;
    else a.part_lse[wc.slot * R + myrow] = lv;
  }
#endif  // __HIP_DEVICE_COMPILE__
}

// ---------------------------------------------------------------------------
// bf16 KV with more than 32 query rows (speculative verify): the schedule of
// split_kernel_f8x64 on bf16 operands.  Eight waves in two groups of four;
// group g owns query rows 32g .. 32g + 31 of the 64-row block (r = j*H + h),
// SIMD k runs wave k of each group, and the groups run one phase apart, so on
// every SIMD one wave issues MFMAs while the other runs the softmax:
//   phase E(i): group 0: PV(i-1), QK(i)   | group 1: softmax(i-1)
//   phase O(i): group 0: softmax(i)       | group 1: PV(i-1), QK(i)
// A tile is 32 positions (two pages, 36,864 bytes), three tiles in a ring.
// Within a group, wave v = w & 3:
//   QK:      S^T = K Q^T over the dimension quarter 144v .. 144v + 143 of the
//            tile's 32 positions: nine v_mfma_f32_32x32x16_bf16 against query
//            fragments held in 36 registers; the four partial tiles go to LDS;
//   softmax: rows 8v .. 8v + 7 of the group, eight lanes a row and four
//            positions a lane: the four partials added, the row's running
//            maximum (lazy, as in split_kernel) and sum kept by those lanes,
//            the probabilities (bf16) and the row's rescale factor for the
//            output written to LDS;
//   PV:      output columns 128v .. 128v + 127 of the group's 32 rows; the
//            value operand is read transposed from the tile in the MFMA phase
//            that scores it and held in registers until the next one, so a
//            tile is read only in E(i) and O(i) and buffer (i + 2) % 3 can be
//            refilled from the start of E(i).
// The KV bytes reach the bf16 MFMAs as stored; every KV byte crosses HBM once.
template <bool FINAL>
__global__ __launch_bounds__(kF8Threads, 1) void split_kernel_b16x64(SplitArgs a) {
#if defined(__HIP_DEVICE_COMPILE__)  // the host pass only needs the launch stub
  using G = KvGeom<false>;
  constexpr int kNBuf = 3;
  constexpr int kTP = 32;                                // positions per tile
  constexpr int kTPages = kTP / kPage;                   // 2
  constexpr int kTileB = kTPages * G::kPageB;            // 36,864
  constexpr int kRangeLoads = G::kPageB / 1024 / 2;      // 9: a wave's half of a page
  constexpr int kPRB = kTP * 2 + 16;                     // bytes per bf16 probability row (+skew)
  // one wave's partial-score tile in LDS: 64 lanes x 64 bytes, lanes 32..63
  // 128 bytes further (see send_scores)
  constexpr int kXB = 64 * 64 + 128;
  // the reference maximum moves when a tile maximum passes it by more than
  // 2^kSlack (bf16 probabilities up to 2^8, far from overflow)
  constexpr float kSlack = 8.f;

  __shared__ __attribute__((aligned(16))) uint8_t kv_lds[kNBuf * kTileB];
  __shared__ __attribute__((aligned(16))) uint8_t p_lds[2][32 * kPRB];   // [group][row][position]
  __shared__ __attribute__((aligned(16))) uint8_t xbuf[2][4][kXB];       // [group][wave][...]
  __shared__ float alpha_lds[2][32];                                     // output rescale per row
  __shared__ float rowstat[2][32][2];                                    // final maximum and sum per row

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int r32 = lane & 31;
  const int h = lane >> 5;
  const int grp = w >> 2;
  const int v4 = w & 3;
  const int H = a.heads;
  const int R = a.num_q * H;
  const WgCoord wc = split_coord(a, (R + 63) / 64);
  const int split = wc.split;
  const int b = wc.b;
  const int myrow = 64 * wc.z + 32 * grp + r32;

  // seq_lens[b] first (a scalar load), then the query block's loads: the
  // workgroup's 64 query rows (1,152 bytes each) are staged once in KV
  // buffers 1 and 2 by direct-to-LDS loads, chunk j of row r at chunk
  // (j & ~7) | ((j ^ r) & 7) of its LDS row; rows past Q*H lie outside the
  // buffer range and arrive as zeros.
  const int L = kDebug ? debug_seq_len(a.seq_lens[b], a.num_q, a.max_blocks, a.debug_flags) : a.seq_lens[b];
  uint8_t* const qlds = kv_lds + kTileB;
  {
    const int nrows = min(64, R - 64 * wc.z);
    const u32x4 qrsrc = buffer_rsrc(a.q + ((int64_t)b * R + 64 * wc.z) * kLatent, nrows * 2 * kLatent);
#pragma unroll
    for (int i = 0; i < 9; ++i) {
      const int slot = 64 * (w + 8 * i) + lane;   // 16-byte LDS slot of this lane
      const int r = slot / 72, x = slot - 72 * (slot / 72);
      const uint32_t src = 16u * (uint32_t)(72 * r + (x ^ (r & 7)));
      copy16_to_lds(qrsrc, src, lds_addr(qlds + 1024 * (w + 8 * i)));
    }
  }
  __builtin_amdgcn_sched_barrier(0);
  const int P = (L + kPage - 1) / kPage;
  const int S = wc.nsplit;
  const int pq = P / S, pr = P - pq * S;
  const int p0 = split * pq + (split * pr) / S;
  const int p1 = (split + 1) * pq + ((split + 1) * pr) / S;
  const int ntiles = (p1 - p0 + kTPages - 1) / kTPages;

  // opaque copy of the lane index (see split_kernel_f8x64)
  auto lane_now = [&]() -> int {
    int l = lane;
    asm volatile("" : "+v"(l));
    return l;
  };

  // ---- a2: copies.  Tile T goes to LDS buffer T % 3.  Wave (g, v) copies
  // half v % 2 of page v / 2 of the tile (loads 9 (v % 2) .. + 8 of the
  // page's eighteen one-KiB loads): tile 0 whole by group 0 in the prologue,
  // tile 1 whole by group 1 once the staged query has been read, each tile
  // T >= 2 shared by both groups during their softmax phases two tiles
  // ahead (group 1 the first kLoads1 loads of each range at E(T - 2), group
  // 0 the rest at O(T - 2)).  Pages outside the split and positions past
  // seq_len lie outside the buffer range: the copy writes zeros.
  constexpr int kLoads1 = 5;
  const int cpage = v4 >> 1;
  const int chalf = v4 & 1;
  const __attribute__((address_space(4))) int32_t* pt_b =
      (const __attribute__((address_space(4))) int32_t*)(a.page_table + (int64_t)b * a.max_blocks);
  const int plast = max(P - 1, 0);
  auto pt_load = [&](int T) -> int { return pt_b[min(p0 + T * kTPages + cpage, plast)]; };
  auto issue_part = [&](int T, int ptv, auto C0, auto C1) {
    constexpr int c0 = decltype(C0)::value, c1 = decltype(C1)::value;
    const int gp = p0 + T * kTPages + cpage;
    int blk = __builtin_amdgcn_readfirstlane(ptv);
    if constexpr (kDebug) blk = gp < p1 ? debug_page_id(blk, a.num_blocks, a.debug_flags) : 0;
    const int bytes = gp < p1 ? min(kPage, L - gp * kPage) * G::kRowB : 0;
    const u32x4 rsrc = buffer_rsrc(a.kv + (int64_t)(gp < p1 ? blk : 0) * G::kPageB, bytes);
    uint8_t* dst = kv_lds + (T % kNBuf) * kTileB + cpage * G::kPageB;
    // LDS slot s = 64c + lane of the page holds source chunk
    // 72 row + (x ^ swz(row)) with row = s / 72, x = s % 72; as 72 is a
    // multiple of 8 that is s ^ swz(s / 72) = s ^ (s / 144) (s < 1152), and
    // s / 144 = d0 + (lane >= t) with d0 = 64c / 144, t = 144 (d0 + 1) - 64c.
    static_assert(G::kChunksPerRow == 72, "bf16 page rows of 72 chunks");
    const int ln = lane_now();
    const uint32_t vb = 16u * (uint32_t)ln;
#pragma unroll
    for (int c = c0; c < c1; ++c) {
      const int base = 64 * (kRangeLoads * chalf + c);   // first slot of the load (wave-uniform)
      const int d0 = base / 144;
      const int t = 144 * (d0 + 1) - base;
      const uint32_t d = (uint32_t)d0 + ((t < 64 && ln >= t) ? 1u : 0u);
      const uint32_t voff = (vb + 16u * (uint32_t)base) ^ (d << 4);
      if (R <= 64) copy16_to_lds_nt(rsrc, voff, lds_addr(dst + 16 * base));
      else copy16_to_lds(rsrc, voff, lds_addr(dst + 16 * base));
    }
  };
  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, kLoads1>;
  using I9 = std::integral_constant<int, kRangeLoads>;

  // ---- query fragments (B operand of S^T = K Q^T): row 32g + l % 32, dims
  // 144v + 16ks + 8h .. + 7 (bf16 chunk 18v + 2ks + h), ks < 9.
  u32x4 qf[9];
  int ptA, ptB;   // page-table entries of the next two tiles this wave copies
  const int pt0 = pt_load(grp);
  {
    ptA = pt_load(2);
    ptB = pt_load(3);
    // probabilities read by each group's first PV are zeros and its rescale
    // factors ones (that PV adds nothing; published by the barrier below)
    for (int i = tid; i < (int)(sizeof(p_lds) / 16); i += kF8Threads) ((u32x4*)p_lds)[i] = u32x4{};
    if (tid < 64) alpha_lds[tid >> 5][tid & 31] = 1.f;
    if (grp == 0) {
      issue_part(0, pt0, I0{}, I9{});
      __builtin_amdgcn_s_waitcnt(waitcnt_vm(kRangeLoads));   // this wave's query loads
    } else {
      __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
    }
    lds_barrier();   // every wave's query loads have landed
    const int lr = 32 * grp + r32;
    const uint8_t* const qrow = qlds + lr * (2 * kLatent);
#pragma unroll
    for (int ks = 0; ks < 9; ++ks) {
      const int j = 18 * v4 + 2 * ks + h;
      qf[ks] = *(const u32x4*)(qrow + 16 * ((j & ~7) | ((j ^ lr) & 7)));
    }
  }
  lds_barrier();   // every wave has read the staged query
  if (grp == 1) {
    issue_part(1, pt0, I0{}, I9{});
    __builtin_amdgcn_sched_barrier(0);
  }

  const float c2 = a.score_scale_log2;
  float m_run = kNegInf, l_run = 0.f;   // softmax rows 8v + l / 8 (all eight lanes of a row hold them)
  f32x16 o[4];
  u32x4 vfr[8];   // value fragments of the group's next PV: column tile i / 2, k-step i % 2
#pragma unroll
  for (int c = 0; c < 4; ++c) o[c] = f32x16{};
#pragma unroll
  for (int c = 0; c < 8; ++c) vfr[c] = u32x4{0u, 0u, 0u, 0u};
  uint8_t* const pg = p_lds[grp];

  // Partial scores to LDS.  Lane l holds row l % 32 and positions
  // 8(i / 4) + 4h + i % 4 of the tile (32x32 MFMA output layout); 16-byte
  // chunk q (elements 4q .. 4q + 3) goes to byte 64 l + 128 h + 16 (q ^ ((l / 4) % 4))
  // of the wave's tile, which spreads both the writes and the softmax's
  // reads (eight rows, both halves, four chunks) over distinct bank groups.
  auto send_scores = [&](const f32x16& s) {
    const int ln = lane_now();
    uint8_t* const xp = xbuf[grp][v4] + 64 * ln + 128 * (ln >> 5);
    const int sw = (ln >> 2) & 3;
#pragma unroll
    for (int q = 0; q < 4; ++q)
      *(f32x4*)(xp + 16 * (q ^ sw)) = f32x4{s[4 * q], s[4 * q + 1], s[4 * q + 2], s[4 * q + 3]};
  };

  // ---- a5: softmax of tile T for rows 8v .. 8v + 7 of the group.  Lane
  // l = 8k + 4u + c takes row 8v + k, positions 8c + 4u .. + 3: element
  // chunk c of source lane 8v + k + 32u of each of the group's four waves.
  auto softmax = [&](int T) {
    __builtin_amdgcn_s_setprio(2);
    const int ln = lane_now();
    const int k = ln >> 3, u = (ln >> 2) & 1, c = ln & 3;
    const int sl = 8 * v4 + k + 32 * u;
    const int xoff = 64 * sl + 128 * u + 16 * (c ^ ((sl >> 2) & 3));
    float x[4];
    {
      const f32x4 a0 = *(const f32x4*)(xbuf[grp][0] + xoff);
      const f32x4 a1 = *(const f32x4*)(xbuf[grp][1] + xoff);
      const f32x4 a2 = *(const f32x4*)(xbuf[grp][2] + xoff);
      const f32x4 a3 = *(const f32x4*)(xbuf[grp][3] + xoff);
#pragma unroll
      for (int j = 0; j < 4; ++j) x[j] = (a0[j] + a1[j]) + (a2[j] + a3[j]);
    }
    const int row = 8 * v4 + k;
    const int pos0 = 8 * c + 4 * u;
    const int tpos0 = (p0 + T * kTPages) * kPage;
    const int tlim = (p1 - p0 - T * kTPages) * kPage;
    float mx = kNegInf;
    if (tlim >= kTP && tpos0 + kTP <= L - a.num_q + 1) {   // every row sees the whole tile
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        x[j] *= c2;
        mx = fmaxf(mx, x[j]);
      }
    } else {
      const int lim = L - a.num_q + (64 * wc.z + 32 * grp + row) / H + 1;
      const int kvis = min(tlim, lim - tpos0) - pos0;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        x[j] = j < kvis ? x[j] * c2 : kNegInf;
        mx = fmaxf(mx, x[j]);
      }
    }
    mx = max8(mx);   // the row's eight lanes
    const float mn = (mx > m_run + kSlack) ? mx : m_run;   // lazy rescale
    const float al = (mn == m_run) ? 1.f : __builtin_amdgcn_exp2f(m_run - mn);
    m_run = mn;
    bf16x4 pb;
    float ps = 0.f;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float p = (x[j] == kNegInf) ? 0.f : __builtin_amdgcn_exp2f(x[j] - mn);
      pb[j] = (__bf16)p;
      ps += p;
    }
    ps = sum8(ps);
    l_run = l_run * al + ps;
    *(bf16x4*)(pg + row * kPRB + 2 * pos0) = pb;
    if ((ln & 7) == 0) alpha_lds[grp][row] = al;
  };

  // ---- MFMA phase T: QK(T) and PV(T - 1), then the value fragments of tile T.
  // a4 key operand of k-step ks: position l % 32 of the tile (page
  // (l / 16) % 2, row l % 16), dims 144v + 16ks + 8h .. + 7.
  // a6 O^T[c][r] += V^T[c][t] P^T[t][r], columns 128v + 32ct + l % 32, k-step
  // kk = positions 16kk + 8h .. + 7 (value operand: two transposed reads).
  auto mfma_phase = [&](int T) {
    const int ln = lane_now();
    const int row = ln & 31;
    const float al = alpha_lds[grp][row];
    const uint8_t* const tile = kv_lds + (T % kNBuf) * kTileB;
    const uint8_t* const kp = tile + ((ln >> 4) & 1) * G::kPageB;
    auto kop8 = [&](int ks) -> bf16x8 {
      return as_bf16x8(load_k8<false>(kp, ln & 15, 144 * v4 + 16 * ks + 8 * (ln >> 5)));
    };
    const uint8_t* const pp = pg + row * kPRB + 16 * (ln >> 5);
    const bf16x8 pf0 = as_bf16x8(*(const u32x4*)pp);
    const bf16x8 pf1 = as_bf16x8(*(const u32x4*)(pp + 32));
    // all nine key operands requested up front: the score MFMAs then wait
    // only for the first, not for an LDS round trip each
    bf16x8 kr[9];
#pragma unroll
    for (int ks = 0; ks < 9; ++ks) kr[ks] = kop8(ks);
    __builtin_amdgcn_sched_barrier(0);
    f32x16 s = f32x16{};
#pragma unroll
    for (int ks = 0; ks < 9; ++ks) s = mfma32(kr[ks], as_bf16x8(qf[ks]), s);
    if (__any(al != 1.f)) {
#pragma unroll
      for (int c = 0; c < 4; ++c) o[c] *= al;
    }
    const int r16 = ln & 15;
    const int cb = 128 * v4 + 16 * ((ln >> 4) & 1);
    const int t0 = 8 * (ln >> 5);
#pragma unroll
    for (int ct = 0; ct < 4; ++ct) {
      o[ct] = mfma32(as_bf16x8(vfr[2 * ct]), pf0, o[ct]);
      o[ct] = mfma32(as_bf16x8(vfr[2 * ct + 1]), pf1, o[ct]);
      vfr[2 * ct] = load_v8<false>(tile, t0, cb + 32 * ct, r16);
      vfr[2 * ct + 1] = load_v8<false>(tile, 16 + t0, cb + 32 * ct, r16);
      if (ct == 1) send_scores(s);
    }
  };

  // Half-steps hs = 0, 1, ...: E(i) = 2i, O(i) = 2i + 1, as in
  // split_kernel_f8x64: copy waits and barrier at the start of each, copy
  // issue at the end.  Here the softmax role is the longer one: it runs at
  // raised priority (with its copies), the MFMA role at the normal one.
  auto begin = [&](int hs) {
    if ((hs & 1) == 0 && hs >= 2) {
      if (grp) __builtin_amdgcn_s_waitcnt(waitcnt_vm(kLoads1));
      else __builtin_amdgcn_s_waitcnt(waitcnt_vm(kRangeLoads - kLoads1));
    }
    lds_barrier();
  };
  auto copies = [&](int hs) {
    if ((hs & 1) == 1 - grp) {
      const int it = hs >> 1;
      const int cur = (it & 1) ? ptB : ptA;
      const int nxt = pt_load(it + 4);
      if (grp) issue_part(it + 2, cur, I0{}, I1{});
      else issue_part(it + 2, cur, I1{}, I9{});
      if (it & 1) ptB = nxt;
      else ptA = nxt;
    }
  };
  if (grp == 0) __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
  // a group whose 32 rows all lie past Q*H only takes part in the barriers
  // and the copies
  const bool live = 64 * wc.z + 32 * grp < R;
  // A wave whose eight softmax rows all lie past Q*H skips the softmax (the
  // probabilities of those rows stay zero and their rescale factors one, as
  // set in the prologue; rows that are never stored).  Bf16 verify B=32 (36
  // rows, group 1's waves 1..3): layer-step 173.5 -> 170.0 us, same-box
  // timing.  Handing those waves the copies as well was slower (180-185 us):
  // this kernel's copies want the raised priority of the softmax role.
  const bool srows = 64 * wc.z + 32 * grp + 8 * v4 < R;
  for (int hs = 0; hs <= 2 * ntiles + 1; ++hs) {
    begin(hs);
    const int st = hs - grp;
    if (live && st >= 0 && (st & 1) == 0) {
      mfma_phase(st >> 1);
    } else if (srows && st >= 1) {
      const int T = (st - 1) >> 1;
      if (T < ntiles) softmax(T);
    }
    copies(hs);
    __builtin_amdgcn_s_setprio(0);
  }

  // every copy has landed (the epilogue reuses the KV buffers); the softmax
  // lanes publish each row's maximum and sum
  __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
  {
    const int ln = lane_now();
    if (live && (ln & 7) == 0) {
      rowstat[grp][8 * v4 + (ln >> 3)][0] = m_run;
      rowstat[grp][8 * v4 + (ln >> 3)][1] = l_run;
    }
  }
  lds_barrier();
  const float m_fin = rowstat[grp][r32][0];
  const float l_fin = rowstat[grp][r32][1];

  // ---- a7: epilogue, staged through the free KV buffers as in split_kernel_f8x64.
  {
    constexpr int kSRow = 256 + 16;
    static_assert(kF8Waves * 32 * kSRow <= kNBuf * kTileB, "epilogue staging fits the KV buffers");
    uint8_t* const stage = kv_lds + w * 32 * kSRow;
    const float sc = l_fin > 0.f ? a.out_scale / l_fin : 0.f;
#pragma unroll
    for (int ct = 0; ct < 4; ++ct)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        bf16x4 ov;
#pragma unroll
        for (int i = 0; i < 4; ++i) ov[i] = (__bf16)(o[ct][4 * q + i] * sc);
        *(bf16x4*)(stage + r32 * kSRow + 2 * (32 * ct + 8 * q + 4 * h)) = ov;
      }
    uint16_t* const dst = FINAL ? a.out : a.part_out;
    const int64_t row0 = FINAL ? (int64_t)b * R : wc.slot * R;
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
    const float lv = (l_fin > 0.f) ? (m_fin + log2f(l_fin)) * kLn2 : kNegInf;
    if constexpr (FINAL) a.lse[(int64_t)b * R + myrow] = lv;
    else a.part_lse[wc.slot * R + myrow] = lv;
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
  if (rows > 32) {
    const dim3 grid((unsigned)(a.num_splits * a.batch * ((rows + 63) / 64)));
    if constexpr (FP8) {
      if (rows <= 48) {   // one row block whose group 1 is packed
        if (final_out)
          hipLaunchKernelGGL((split_kernel_f8x64<true, true>), grid, dim3(kF8Threads), 0, stream, a);
        else
          hipLaunchKernelGGL((split_kernel_f8x64<false, true>), grid, dim3(kF8Threads), 0, stream, a);
      } else {
        if (final_out)
          hipLaunchKernelGGL((split_kernel_f8x64<true, false>), grid, dim3(kF8Threads), 0, stream, a);
        else
          hipLaunchKernelGGL((split_kernel_f8x64<false, false>), grid, dim3(kF8Threads), 0, stream, a);
      }
    } else {
      if (final_out)
        hipLaunchKernelGGL(split_kernel_b16x64<true>, grid, dim3(kF8Threads), 0, stream, a);
      else
        hipLaunchKernelGGL(split_kernel_b16x64<false>, grid, dim3(kF8Threads), 0, stream, a);
    }
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
  if (rows > 32) return units * ((rows + 63) / 64) * kF8Threads;
  const int64_t rpad = rows <= 16 ? 16 : 48;
  return units * ((rows + rpad - 1) / rpad) * kThreads;
}

hipError_t launch_split(const SplitArgs& a, bool fp8, bool final_out, hipStream_t stream) {
  return fp8 ? launch_dtype<true>(a, final_out, stream) : launch_dtype<false>(a, final_out, stream);
}

}  // namespace mla
