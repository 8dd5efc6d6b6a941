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
};

struct MergeArgs {
  const uint16_t* part_out;   // bf16 [S][rows][512]
  const float* part_lse;      // [S][rows]
  uint16_t* out;              // bf16 [rows][512]
  float* lse;                 // [rows]
  int64_t rows;
  int32_t num_splits;
};

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
