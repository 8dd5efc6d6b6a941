/*
 * mla.h -- C ABI of the MI355X (gfx950) MLA decode / speculative-verify library.
 *
 * What is computed
 * ----------------
 * Multi-head Latent Attention over a paged, compressed KV cache.  Every cached
 * position is one 576-wide latent (512 latent + 64 rope dims) shared by all
 * query heads of the rank ("Inside Kimi K3 optimization", section
 * "1. Cache -- DCP": 576 FP8 bytes per position; tensor parallelism splits
 * heads, not the cache).  Each head dots its 576-wide query with the latent;
 * the value vector is the first 512 dims of the same latent.  For sequence b,
 * query token j (of Q) and head h:
 *
 *     s_t   = softmax_scale * kv_scale * <q[b,j,h,:], latent_t>     (t visible)
 *     lse   = ln sum_t exp(s_t)
 *     out[c] = sum_t exp(s_t - lse) * kv_scale * latent_t[c],   c < 512
 *
 * where latent_t is the stored value (bf16, or the decoded FP8 E4M3FN code),
 * and kv_scale is the per-tensor FP8 scale (1 for bf16).
 *
 * Causal rule for speculative verify ("Inside Kimi K3 optimization",
 * section "1. Cache -- DCP": multi-token verify): seq_lens[b] counts every
 * cached position including the Q new tokens, and token j sees positions
 * 0 .. seq_lens[b] - Q + j.  Q = 1 is plain decode.
 *
 * Split-KV ("Inside Kimi K3 optimization", section "4. MLA": the history is
 * divided into pieces processed by parallel workgroups and the pieces are
 * combined): sequence b has P_b = ceil(seq_lens[b] / 16) pages; split s of S
 * covers pages [floor(s * P_b / S), floor((s + 1) * P_b / S)).  Each split
 * produces a partial output normalised by its own softmax sum and its
 * natural-log log-sum-exp (the "normalisation information" partial answers
 * carry, section "1. Cache -- DCP"); mla_merge combines them.  A split with
 * no visible position has lse = -inf and output 0.
 *
 * Head padding ("Inside Kimi K3 optimization", section "4. MLA"; "Kimi K3 on
 * AMD MI355X", section "What had to be fixed"): the Q*H query rows (token-major,
 * r = j*H + h) are processed in blocks of 16, 48 or 64 rows, the last block
 * padded inside the kernel with zero queries; pad rows are never read from or
 * written to caller memory.
 *
 * Layouts (all row-major, contiguous, caller-owned device memory)
 * --------------------------------------------------------------
 *   q          bf16  [batch][num_q_tokens][num_heads][576]
 *   kv_cache   bf16 or uint8 (FP8 E4M3FN codes) [num_blocks][16][576]
 *              (block size 16: "Kimi K2.6 + DFlash on 8x MI300X",
 *              section "Technical numbers")
 *   page_table int32 [batch][max_blocks_per_seq]; entry p of row b is the
 *              pool block holding positions 16p .. 16p+15 of sequence b; only
 *              entries p < ceil(seq_lens[b] / 16) are read
 *   seq_lens   int32 [batch]
 *   out        bf16  [batch][num_q_tokens][num_heads][512]
 *   lse        fp32  [batch][num_q_tokens][num_heads]   (natural log)
 *   part_out   bf16  [S][batch][num_q_tokens][num_heads][512]
 *   part_lse   fp32  [S][batch][num_q_tokens][num_heads]
 *
 * Conventions
 * -----------
 * - Every call is asynchronous on `stream` (a hipStream_t, NULL = default
 *   stream); the library never allocates, frees or synchronises, and keeps no
 *   state besides a per-thread last HIP error code.
 * - Host-side validation runs before any HIP call; a failing call returns a
 *   status and launches nothing.  After a launch, a HIP error maps to
 *   MLA_ERR_HIP (the code is kept by mla_last_hip_error()).
 * - A dispatch holds its grid size in 32 bits: a call whose split or merge
 *   launch would exceed 2^32 - 1 work-items returns MLA_ERR_UNSUPPORTED (for
 *   example S = 256 with 65,535 sequences of 1,024 query rows; the split
 *   launch has 256 threads per workgroup and query-row block, 512 for FP8
 *   with more than 32 rows, the merge 128, 256 or 1,024 threads per row for
 *   S <= 8, <= 32 or more).
 * - Caller contract, not checked on the device by the release library:
 *   num_q_tokens <= seq_lens[b] <= 16 * max_blocks_per_seq and
 *   0 <= page_table[b][p] < num_blocks for the pages read (paged addressing in
 *   blocks of 16: "Kimi K2.6 + DFlash on 8x MI300X", section "Technical
 *   numbers").  The debug build of the library (libmla_hip_debug.so, compiled
 *   with MLA_DEBUG=1) checks it on the device: see mla_debug_flags.
 *   kv_cache and page_table are only read.
 * - Concurrent calls on different streams are safe when their outputs and
 *   workspaces do not overlap.
 */
#ifndef MLA_H
#define MLA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MLA_OK = 0,
  MLA_ERR_NULL_ARG = 1,     /* a required pointer is NULL */
  MLA_ERR_BAD_SHAPE = 2,    /* a size is out of range */
  MLA_ERR_BAD_DTYPE = 3,    /* kv_dtype is not an mla_kv_dtype */
  MLA_ERR_BAD_SCALE = 4,    /* softmax_scale not finite, or kv_scale not finite and > 0 */
  MLA_ERR_UNSUPPORTED = 5,  /* valid request this library does not implement */
  MLA_ERR_WORKSPACE = 6,    /* workspace NULL or smaller than mla_workspace_size() */
  MLA_ERR_HIP = 7,          /* the HIP runtime reported an error */
  MLA_ERR_SCRATCH_LIMIT = 8 /* mla_verify_static: partials larger than its static scratch */
} mla_status;

/* Size of the static device array behind mla_verify_static (96 MiB per GPU). */
#define MLA_STATIC_SCRATCH_BYTES ((size_t)96 << 20)

typedef enum {
  MLA_KV_BF16 = 0,          /* bf16 latents, 1152 bytes per position */
  MLA_KV_FP8_E4M3 = 1       /* OCP FP8 E4M3FN codes, 576 bytes per position, per-tensor kv_scale */
} mla_kv_dtype;

typedef struct {
  int32_t batch;              /* B >= 1 */
  int32_t num_q_tokens;       /* Q: 1 for mla_decode; 1..8 for mla_verify */
  int32_t num_heads;          /* H: 1..128 (12 per TP8 rank, 96 for DCP8-shaped attention) */
  int32_t num_blocks;         /* pool blocks in kv_cache, >= 1 */
  int32_t max_blocks_per_seq; /* page_table row stride, >= 1 */
  int32_t max_seq_len_hint;   /* largest seq_len the caller expects; 0 = 16 * max_blocks_per_seq.
                                 Only steers the automatic split count. */
  int32_t kv_dtype;           /* mla_kv_dtype */
  int32_t num_splits;         /* 0 = library chooses; 1..256 = exactly this many splits */
  int32_t split_policy;       /* mla_split_policy: how the S * batch split slots are spread */
} mla_params;

/* How mla_decode / mla_verify / mla_verify_static spread the S * batch split
 * slots of a call (S = mla_num_splits) over the sequences.  Results are the
 * same up to rounding order either way; only the work per workgroup differs.
 *   MLA_SPLIT_PER_SEQUENCE: every sequence gets S splits (S is chosen from the
 *     longest expected sequence), so with unequal lengths the splits of long
 *     sequences hold many more pages than those of short ones;
 *   MLA_SPLIT_BY_LENGTH: sequence b gets C(b) - C(b - 1) slots with
 *     C(b) = b + 1 + floor((S*B - B) * (P_0 + ... + P_b) / (P_0 + ... + P_{B-1})),
 *     P_i = ceil(seq_lens[i] / 16) clamped into [1, max_blocks_per_seq] --
 *     at least one each, the rest in proportion to its pages -- so every
 *     workgroup gets about the same number of pages (the history "divided into
 *     pieces processed by parallel workgroups", "Inside Kimi K3 optimization",
 *     section "4. MLA").  The kernels compute the plan on the device from
 *     seq_lens.  Used for 2 <= batch <= 64 and S > 1 when the merge's weight
 *     table fits (S * batch - batch + 1 <= 12,288); otherwise the call uses
 *     MLA_SPLIT_PER_SEQUENCE.  mla_split, whose partial layout is per
 *     sequence, returns MLA_ERR_UNSUPPORTED for it. */
typedef enum {
  MLA_SPLIT_PER_SEQUENCE = 0,
  MLA_SPLIT_BY_LENGTH = 1
} mla_split_policy;

/* Split count the library uses for these parameters (>= 1), or 0 if the
 * parameters are invalid.  Depends only on host-side values: with num_splits
 * = 0 it is max(ceil(pages / M), F), at least 1 and at most 256, with the
 * fill F = min(ceil(256 / U), pages / 2) and an F above 128 reduced to
 * max(128, min(F, pages / 16)), for pages = ceil(hint / 16), M = 128 pages
 * per split for FP8 (64 for bf16: about 1.1 MiB of cache either way) and U = B times the
 * number of query-row blocks (blocks of 64 rows for FP8 with more than 32 rows
 * Q*H, else 48, or 16 for at most 16 rows); when U * S falls between one and
 * two rounds of 256 workgroups, S = 256 / U (one full round). */
int32_t mla_num_splits(const mla_params* p);

/* Bytes of workspace mla_decode / mla_verify need: the partials of all splits
 * (0 when the split count is 1).  Returns 0 for invalid parameters. */
size_t mla_workspace_size(const mla_params* p);

/* Single-token decode (p->num_q_tokens must be 1).  Writes out and lse.
 * workspace: device memory of at least mla_workspace_size(p) bytes (may be
 * NULL when that is 0); its contents are scratch. */
mla_status mla_decode(const mla_params* p, const void* q, const void* kv_cache,
                      const int32_t* page_table, const int32_t* seq_lens,
                      float softmax_scale, float kv_scale, void* out, float* lse,
                      void* workspace, size_t workspace_bytes, void* stream);

/* Speculative verify: Q query tokens per sequence with the causal rule above
 * (Q = 1 is allowed and equals mla_decode). */
mla_status mla_verify(const mla_params* p, const void* q, const void* kv_cache,
                      const int32_t* page_table, const int32_t* seq_lens,
                      float softmax_scale, float kv_scale, void* out, float* lse,
                      void* workspace, size_t workspace_bytes, void* stream);

/* mla_verify without a workspace argument, for callers that cannot allocate
 * device memory: code under HIP graph capture, tight serving loops and
 * harnesses that forbid allocation.  It allocates nothing.  The split
 * partials go to a static device array of MLA_STATIC_SCRATCH_BYTES bytes
 * that the library holds on every GPU it runs on until the process ends
 * (its address is looked up once per GPU, on the first call there; the
 * GPU is the device of `stream`, the current device for the NULL stream).
 * A call whose partials (mla_workspace_size(p) bytes) exceed the array
 * returns MLA_ERR_SCRATCH_LIMIT and launches nothing (for example B = 64
 * sequences of up to 65,536 FP8 positions with Q = 3 and 12 heads need
 * 75.8 MB at 32 splits and fit).  Every call on one GPU shares that GPU's
 * array, and the array keeps the last call's contents (the partials are
 * fully rewritten by each call, nothing needs to start at zero): calls that
 * overlap in time on one GPU -- on different streams or from different host
 * threads -- race on it and give undefined results; serialise them.  Same
 * arguments (minus the workspace), results and other errors as mla_verify. */
mla_status mla_verify_static(const mla_params* p, const void* q, const void* kv_cache,
                             const int32_t* page_table, const int32_t* seq_lens,
                             float softmax_scale, float kv_scale, void* out, float* lse,
                             void* stream);

/* Split-KV partials only: S = mla_num_splits(p) partial outputs (bf16, RNE of
 * the fp32 result, normalised by their own sums, already multiplied by
 * kv_scale) and their fp32 natural-log normalisers, in the part_out /
 * part_lse layouts above.  Partial rows are bf16 because they are written
 * and read once per step at every split boundary; their rounding (relative
 * 2^-9 per element) stays far below the bf16 rounding of the merged output
 * combined with the FP8 cache quantisation. */
mla_status mla_split(const mla_params* p, const void* q, const void* kv_cache,
                     const int32_t* page_table, const int32_t* seq_lens,
                     float softmax_scale, float kv_scale, void* part_out, float* part_lse,
                     void* stream);

/* Log-sum-exp merge of S partials ("normalisation information" lets shards be
 * weighted correctly, "Inside Kimi K3 optimization", section "1. Cache -- DCP"):
 *     lse[r] = ln sum_s exp(part_lse[s][r])        (-inf partials weigh 0)
 *     out[r][c] = bf16_rne( sum_s exp(part_lse[s][r] - lse[r]) * part_out[s][r][c] )
 * part_out bf16 [num_splits][rows][512], part_lse fp32 [num_splits][rows],
 * out bf16 [rows][512], lse fp32 [rows].  All partials -inf: out 0, lse -inf.
 * 1 <= num_splits <= 4096, 1 <= rows <= 2^28; otherwise MLA_ERR_BAD_SHAPE
 * (and MLA_ERR_UNSUPPORTED above 2^32 - 1 work-items, see above).  A
 * partial of weight zero (part_lse = -inf) is never used, whatever part_out
 * holds for it. */
mla_status mla_merge(const void* part_out, const float* part_lse, int32_t num_splits,
                     int64_t rows, void* out, float* lse, void* stream);

/* KV-cache append: write the latents of the Q newest positions of every
 * sequence into their cache slots, the step before attention in a decode or
 * verify step.  An FP8 cache stores one byte per value under a per-tensor
 * scale ("Kimi K2.6 + DFlash on 8x MI300X (508 tok/s)", section "st=2 vs
 * st=8 & FP8 vs BF16": FP8 doubles the cache's token capacity; section
 * "Next": auto-computed scales today, static calibration proposed).
 *   kv_new  bf16 [batch][num_q_tokens][576], 16-byte aligned
 *   kv_cache bf16 or FP8 E4M3FN bytes [num_blocks][16][576], 16-byte aligned
 * New token j of sequence b goes to position t = seq_lens[b] - Q + j (seq_lens
 * count the new tokens, as in mla_verify): block page_table[b][t / 16], row
 * t % 16.  bf16 cache: the bits are copied.  FP8 cache: each value x becomes
 * the E4M3FN code nearest to the float32 quotient x / kv_scale (IEEE
 * division; ties to even; |x / kv_scale| >= 448 saturates to +-448); inputs
 * must be finite.  Uses p->batch, num_q_tokens (1..8), num_blocks,
 * max_blocks_per_seq and kv_dtype; the other fields are ignored.  A slot
 * with t < 0, t / 16 >= max_blocks_per_seq or a page-table entry outside
 * [0, num_blocks) is a caller error and is skipped (nothing is written).
 * Errors: NULL_ARG, BAD_SHAPE (ranges, alignment), BAD_DTYPE, BAD_SCALE
 * (FP8 with kv_scale not finite and positive), HIP. */
mla_status mla_kv_append(const mla_params* p, const void* kv_new, void* kv_cache,
                         const int32_t* page_table, const int32_t* seq_lens, float kv_scale,
                         void* stream);

/* Dynamic per-tensor FP8 scale of `count` bf16 values x (the auto-computed
 * scale of the same page, section "Next"): writes, to the device float
 * *scale (4-byte aligned), fp32(max|x| / 448) -- 1.0 when every value is
 * zero or count == 0, +inf when the largest magnitude is inf, NaN when a
 * value is NaN.  The maximum is exact (taken over bf16 magnitudes); the
 * division is IEEE float32.  One kernel on `stream` for count <= 65536; above
 * that three small kernels, and *scale doubles as their accumulator, so it
 * must not be read by other work until they end.
 * Errors: NULL_ARG, BAD_SHAPE (count < 0 or > 2^40, misaligned scale), HIP. */
mla_status mla_kv_dynamic_scale(const void* x, int64_t count, float* scale, void* stream);

/* Static description of a status code. */
const char* mla_status_string(int32_t status);

/* HIP error code (hipError_t value) behind the last MLA_ERR_HIP on this thread. */
int32_t mla_last_hip_error(void);

/* Contract violations reported by the debug build (bits of the flag word). */
#define MLA_DEBUG_PAGE_ID 1u    /* a page_table entry read is outside [0, num_blocks) */
#define MLA_DEBUG_SEQ_SHORT 2u  /* seq_lens[b] < num_q_tokens */
#define MLA_DEBUG_SEQ_LONG 4u   /* seq_lens[b] > 16 * max_blocks_per_seq */

/* 1 if this library is the debug build, else 0.  In the debug build every
 * kernel of mla_decode, mla_verify, mla_verify_static, mla_split and
 * mla_kv_append checks the caller contract above on the device, before any
 * read that depends on it: a seq_lens[b] outside [num_q_tokens,
 * 16 * max_blocks_per_seq] is clamped into that range and a page-table entry
 * outside [0, num_blocks) is clamped to the nearest block (mla_kv_append
 * writes nothing for such a slot), so every kernel runs to its end and
 * touches only the caller's buffers; the violation is ORed into a flag word
 * of the device (one per GPU, kept until read).  Results of a call with a
 * violation are not meaningful. */
int32_t mla_debug_build(void);

/* Debug build: *flags = the current device's flag word (MLA_DEBUG_* bits
 * ORed by every call since it was last cleared), cleared when `clear` is
 * nonzero.  Synchronous: waits for the device's outstanding work (unlike
 * every other entry point).  Release build: *flags = 0, no HIP call.
 * Errors: NULL_ARG, HIP. */
mla_status mla_debug_flags(uint32_t* flags, int32_t clear);

#ifdef __cplusplus
}
#endif

#endif /* MLA_H */
