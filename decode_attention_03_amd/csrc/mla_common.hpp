// Shared definitions of the gfx950 MLA kernels (device side) and their host launchers.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mla {

// Geometry fixed by the method: one 576-wide latent per cached position
// (512 latent + 64 rope dims), value vector = first 512 dims, pages of 16
// positions ("Inside Kimi K3 optimization", section "1. Cache -- DCP";
// "Kimi K2.6 + DFlash on 8x MI300X", section "Technical numbers").
constexpr int kLatent = 576;
constexpr int kValue = 512;
constexpr int kPage = 16;

// Workgroup shape of the split kernel: four wave64s, one KV page per wave per
// tile, so a tile is 4 pages = 64 positions.
constexpr int kWaves = 4;
constexpr int kThreads = kWaves * 64;
constexpr int kTilePages = kWaves;
constexpr int kTilePos = kTilePages * kPage;

// Largest query-token count per launch and largest head count per token.
constexpr int kMaxQ = 8;
constexpr int kMaxHeads = 128;
constexpr int kMaxSplits = 256;

struct SplitArgs {
  const uint16_t* q;          // bf16 [B][Q][H][576]
  const uint8_t* kv;          // bf16 or fp8 [NB][16][576]
  const int32_t* page_table;  // [B][max_blocks]
  const int32_t* seq_lens;    // [B]
  uint16_t* part_out;         // bf16 [S][B][Q][H][512]  (partial mode)
  float* part_lse;            // fp32 [S][B][Q][H]
  uint16_t* out;              // bf16 [B][Q][H][512]     (final mode, S == 1)
  float* lse;                 // fp32 [B][Q][H]
  int32_t batch;
  int32_t num_q;
  int32_t heads;
  int32_t max_blocks;
  int32_t num_splits;
  float score_scale_log2;     // softmax_scale * kv_scale * log2(e)
  float out_scale;            // kv_scale (value vectors are used undecoded-scale in the MFMA)
  int32_t num_blocks;         // pool blocks (checked by the debug build only)
  uint32_t* debug_flags;      // debug build: contract violations found (kDbg* bits)
  int32_t by_length;          // split plan by length (balanced_plan), else S per sequence
};

struct MergeArgs {
  const uint16_t* part_out;   // bf16 [S][rows][512], or [S * batch slots][R][512] by length
  const float* part_lse;      // [S][rows], or [S * batch slots][R]
  uint16_t* out;              // bf16 [rows][512]
  float* lse;                 // [rows]
  int64_t rows;
  int32_t num_splits;
  // split plan by length: the partials of row b * R + r are the slots of
  // sequence b (balanced_plan over seq_lens), R = rows per sequence
  int32_t by_length;
  int32_t batch;
  int32_t rows_per_seq;
  int32_t max_blocks;
  const int32_t* seq_lens;
};

// Split plan by length.  The G = S * B split slots of a launch are shared
// among the B sequences in proportion to their pages, at least one each:
// sequence b owns slots [C(b - 1), C(b)) with
//   C(b) = b + 1 + floor((G - B) * (P_0 + ... + P_b) / (P_0 + ... + P_{B-1})),
// C(-1) = 0, P_i = ceil(seq_lens[i] / 16) clamped into [1, max_blocks], so a
// long sequence gets many splits and a short one few, and every split slot
// covers about the same number of pages.  Computed by one wave (B <= 64, one
// sequence per lane: a lane-prefix sum and a ballot); every workgroup of the
// split and merge launches computes the same plan from seq_lens.  Returns,
// for the sequence found by `find` (a slot w when by_slot, else a sequence
// index), its first slot and slot count.
constexpr int kMaxBatchByLength = 64;

struct SeqSlots {
  int b, first, count;
};
__device__ __forceinline__ SeqSlots balanced_plan(const int32_t* seq_lens, int B, int S, int max_blocks,
                                                  int find, bool by_slot) {
  const int lane = (int)(threadIdx.x & 63);
  int P = 0;
  if (lane < B) P = min(max((seq_lens[lane] + kPage - 1) / kPage, 1), max(max_blocks, 1));
  int pref = P;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int t = __shfl_up(pref, d);
    if (lane >= d) pref += t;
  }
  const int ptot = __shfl(pref, 63);
  const int G = S * B;
  int C = G + 1;   // lanes past the batch: past every slot
  if (lane < B) C = lane + 1 + (int)(((int64_t)(G - B) * pref) / max(ptot, 1));
  int b;
  if (by_slot) b = __builtin_ctzll(__ballot(C > find));
  else b = find;
  b = __builtin_amdgcn_readfirstlane(b);
  const int hi = __shfl(C, b);
  const int lo = __shfl(C, max(b - 1, 0));
  SeqSlots r;
  r.b = b;
  r.first = __builtin_amdgcn_readfirstlane(b > 0 ? lo : 0);
  r.count = __builtin_amdgcn_readfirstlane(hi) - r.first;
  return r;
}

struct AppendArgs {
  const uint16_t* kv_new;     // bf16 [B][Q][576]
  uint8_t* kv;                // bf16 or fp8 [NB][16][576]
  const int32_t* page_table;  // [B][max_blocks]
  const int32_t* seq_lens;    // [B]
  int32_t batch;
  int32_t num_q;
  int32_t max_blocks;
  int32_t num_blocks;
  float kv_scale;             // fp8 only
  uint32_t* debug_flags;      // debug build: contract violations found (kDbg* bits)
};

// Debug build (compiled with MLA_DEBUG=1, as libmla_hip_debug.so): the
// kernels check the caller contract of the C ABI on the device before any
// read that depends on it, replace a violating value by one inside its range
// (so every kernel still runs to its end and touches only caller memory) and
// report the violation in a flag word (kDbg* bits).  The release build trusts
// the contract and compiles none of this.
#ifndef MLA_DEBUG
#define MLA_DEBUG 0
#endif
constexpr bool kDebug = MLA_DEBUG != 0;
constexpr uint32_t kDbgPageId = 1u;     // a page_table entry read is outside [0, num_blocks)
constexpr uint32_t kDbgSeqShort = 2u;   // seq_lens[b] < num_q_tokens
constexpr uint32_t kDbgSeqLong = 4u;    // seq_lens[b] > 16 * max_blocks_per_seq

// Vector-memory atomic OR of the lane's bits into the flag word.
__device__ __forceinline__ void debug_report(uint32_t* flags, uint32_t bits) {
  if (bits) atomicOr(flags, bits);
}
// seq_lens[b] clamped into [num_q, 16 * max_blocks]
__device__ __forceinline__ int debug_seq_len(int L, int num_q, int max_blocks, uint32_t* flags) {
  uint32_t bits = 0;
  if (L < num_q) {
    bits |= kDbgSeqShort;
    L = num_q;
  }
  if (L > kPage * max_blocks) {
    bits |= kDbgSeqLong;
    L = kPage * max_blocks;
  }
  debug_report(flags, bits);
  return L;
}
// a page-table entry clamped into [0, num_blocks)
__device__ __forceinline__ int debug_page_id(int blk, int num_blocks, uint32_t* flags) {
  if (blk >= 0 && blk < num_blocks) return blk;
  debug_report(flags, kDbgPageId);
  return blk < 0 ? 0 : num_blocks - 1;
}

// Host launchers (defined next to their kernels).  Return hipSuccess or the
// launch error.
hipError_t launch_split(const SplitArgs& a, bool fp8, bool final_out, hipStream_t stream);
hipError_t launch_merge(const MergeArgs& a, hipStream_t stream);
// Work-items (workgroups x threads) the split and merge launches would have:
// a dispatch packet holds the grid size in 32 bits, so the host rejects a
// launch above kMaxWorkItems before making it.
constexpr int64_t kMaxWorkItems = 0xFFFFFFFFll;
int64_t split_work_items(const SplitArgs& a, bool fp8);
int64_t merge_work_items(const MergeArgs& a);
hipError_t launch_append(const AppendArgs& a, bool fp8, hipStream_t stream);
hipError_t launch_dynamic_scale(const uint16_t* x, int64_t count, float* scale, hipStream_t stream);

}  // namespace mla
