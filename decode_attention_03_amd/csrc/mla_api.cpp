// C ABI of the MLA library: host validation, split planning, launches.
// Declarations and the full contract are in include/mla.h.
#include <hip/hip_runtime_api.h>
#include <math.h>
#include <stddef.h>
#include <stdint.h>

#include <algorithm>
#include <mutex>

#include "mla.h"
#include "mla_common.hpp"

namespace {

thread_local int32_t g_last_hip_error = 0;

// Automatic split count.  One split workgroup occupies a CU (its LDS).  A
// split of the longest sequence gets about 1.1 MiB of cache (128 FP8 or 64
// bf16 pages): less and the fixed cost per workgroup (query preparation,
// first tiles, epilogue) dominates, more and a batch of unequal lengths
// balances poorly over the rounds of workgroups.  A batch that would not fill
// one round of 256 workgroups is split further, while each split keeps at
// least 2 pages; a count that lands between one and two rounds is cut back
// to one full round.  (Measured on the workloads: bf16 decode of 32
// sequences up to 8192 positions runs best at 8 splits, bf16 and FP8 verify
// of 32 / 64 sequences up to 32768 / 65536 positions at 32, four long
// sequences at 64.  Small batches are latency-bound and gain most from the
// fill: one 2048-position bf16 sequence runs in 9.9 us at 64 splits against
// 20.8 us at 4, two of 1024 positions with Q = 3 in 13.4 us at 32 against
// 42.5 us at 2, one of 256 positions in 9.3 us at 8 against 11.1 us at 1.
// Beyond 128 splits the merge of the extra partials costs more than the
// added parallelism gains unless each split keeps 16 pages: one FP8
// sequence of 8192 positions runs in 18.2 us at 128 splits and 22.9 us at
// 256, one of 32768 in 24.2 and 24.8 us.)
constexpr int kComputeUnits = 256;
constexpr int64_t kSplitBytes = 128 * 16 * 576;   // 1,179,648 bytes of cache per split
constexpr int kMinPagesPerSplit = 2;
constexpr int kWideSplits = 128;        // fill beyond this many splits ...
constexpr int kMinPagesWide = 16;       // ... only while each keeps this many pages

mla_status check_params(const mla_params* p, int max_q) {
  if (!p) return MLA_ERR_NULL_ARG;
  if (p->batch < 1 || p->batch > 65535) return MLA_ERR_BAD_SHAPE;
  if (p->num_q_tokens < 1 || p->num_q_tokens > max_q) return MLA_ERR_BAD_SHAPE;
  if (p->num_heads < 1) return MLA_ERR_BAD_SHAPE;
  if (p->num_heads > mla::kMaxHeads) return MLA_ERR_UNSUPPORTED;
  if (p->num_blocks < 1 || p->max_blocks_per_seq < 1) return MLA_ERR_BAD_SHAPE;
  if (p->max_seq_len_hint < 0) return MLA_ERR_BAD_SHAPE;
  if (p->num_splits < 0 || p->num_splits > mla::kMaxSplits) return MLA_ERR_BAD_SHAPE;
  if (p->kv_dtype != MLA_KV_BF16 && p->kv_dtype != MLA_KV_FP8_E4M3) return MLA_ERR_BAD_DTYPE;
  if (p->split_policy != MLA_SPLIT_PER_SEQUENCE && p->split_policy != MLA_SPLIT_BY_LENGTH)
    return MLA_ERR_BAD_SHAPE;
  return MLA_OK;
}

// Whether a call with S splits uses the plan by length (see include/mla.h):
// the kernels compute it with one wave (a batch of at most 64), and the
// merge keeps a weight table of up to S * B - B + 1 floats per row in LDS.
constexpr int64_t kMaxByLengthSlots = 12288;
bool uses_by_length(const mla_params* p, int32_t S) {
  const int64_t B = p->batch;
  return p->split_policy == MLA_SPLIT_BY_LENGTH && B >= 2 && B <= mla::kMaxBatchByLength && S > 1 &&
         (int64_t)S * B - B + 1 <= kMaxByLengthSlots;
}

int32_t choose_splits(const mla_params* p) {
  if (p->num_splits > 0) return p->num_splits;
  int64_t max_len = p->max_seq_len_hint > 0 ? p->max_seq_len_hint
                                            : (int64_t)p->max_blocks_per_seq * mla::kPage;
  const int64_t pages = (max_len + mla::kPage - 1) / mla::kPage;
  const int64_t page_bytes = (int64_t)mla::kPage * mla::kLatent * (p->kv_dtype == MLA_KV_FP8_E4M3 ? 1 : 2);
  const int64_t pages_per_split = kSplitBytes / page_bytes;   // 128 FP8 or 64 bf16 pages
  // query rows are processed in blocks (64 rows above 32, else 48 or 16),
  // each a workgroup of its own over the same split
  const int64_t rows = (int64_t)p->num_q_tokens * p->num_heads;
  const int64_t rblock = rows > 32 ? 64 : (rows <= 16 ? 16 : 48);
  const int64_t units = (int64_t)p->batch * ((rows + rblock - 1) / rblock);
  int64_t s = (pages + pages_per_split - 1) / pages_per_split;
  int64_t fill = (kComputeUnits + units - 1) / units;
  const int64_t fill_cap = pages / kMinPagesPerSplit;
  if (fill > fill_cap) fill = fill_cap;
  if (fill > kWideSplits) fill = std::max<int64_t>(kWideSplits, std::min<int64_t>(fill, pages / kMinPagesWide));
  if (s < fill) s = fill;
  // between one and two rounds of workgroups: use exactly one full round
  // rather than leave most CUs idle during a short second one
  const int64_t wg = s * units;
  if (wg > kComputeUnits && wg < 2 * kComputeUnits) s = kComputeUnits / units;
  if (s > mla::kMaxSplits) s = mla::kMaxSplits;
  if (s < 1) s = 1;
  return (int32_t)s;
}

size_t rows_of(const mla_params* p) {
  return (size_t)p->batch * (size_t)p->num_q_tokens * (size_t)p->num_heads;
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

size_t partial_bytes(const mla_params* p, int32_t S) {
  const size_t rows = rows_of(p) * (size_t)S;
  return align256(rows * mla::kValue * sizeof(uint16_t)) + align256(rows * sizeof(float));
}

mla_status check_scales(float softmax_scale, float kv_scale, int32_t kv_dtype) {
  if (!isfinite(softmax_scale)) return MLA_ERR_BAD_SCALE;
  if (kv_dtype == MLA_KV_FP8_E4M3 && !(isfinite(kv_scale) && kv_scale > 0.f)) return MLA_ERR_BAD_SCALE;
  return MLA_OK;
}

mla::SplitArgs make_args(const mla_params* p, const void* q, const void* kv, const int32_t* pt,
                         const int32_t* sl, float softmax_scale, float kv_scale, int32_t S) {
  mla::SplitArgs a{};
  a.q = (const uint16_t*)q;
  a.kv = (const uint8_t*)kv;
  a.page_table = pt;
  a.seq_lens = sl;
  a.batch = p->batch;
  a.num_q = p->num_q_tokens;
  a.heads = p->num_heads;
  a.max_blocks = p->max_blocks_per_seq;
  a.num_blocks = p->num_blocks;
  a.num_splits = S;
  const float ks = p->kv_dtype == MLA_KV_FP8_E4M3 ? kv_scale : 1.0f;
  a.score_scale_log2 = (float)((double)softmax_scale * (double)ks * 1.4426950408889634);
  a.out_scale = ks;
  return a;
}

// Both launches of a call (split, and merge when S > 1) within the 32-bit
// grid size of a dispatch.
bool launches_fit(const mla::SplitArgs& a, const mla_params* p, int32_t S) {
  if (mla::split_work_items(a, p->kv_dtype == MLA_KV_FP8_E4M3) > mla::kMaxWorkItems) return false;
  if (S == 1) return true;
  mla::MergeArgs m{};
  m.rows = (int64_t)rows_of(p);
  m.num_splits = S;
  m.by_length = a.by_length;
  return mla::merge_work_items(m) <= mla::kMaxWorkItems;
}

mla_status hip_status(hipError_t e) {
  if (e == hipSuccess) return MLA_OK;
  g_last_hip_error = (int32_t)e;
  return MLA_ERR_HIP;
}

}  // namespace

// Partials of mla_verify_static: one array per GPU the library runs on, held
// until the process ends.  Host code never uses this name as an address (on
// the host it is only a stand-in for the symbol); static_scratch() looks up
// each device's copy with hipGetSymbolAddress.
static __device__ __align__(256) uint8_t scratch[MLA_STATIC_SCRATCH_BYTES];

static_assert(mla::kDbgPageId == MLA_DEBUG_PAGE_ID && mla::kDbgSeqShort == MLA_DEBUG_SEQ_SHORT &&
                  mla::kDbgSeqLong == MLA_DEBUG_SEQ_LONG,
              "debug flag bits of the kernels and the C ABI");

// Contract violations found by the kernels of the debug build (kDbg* bits of
// mla_common.hpp), one word per GPU; read and cleared by mla_debug_flags.
static __device__ uint32_t debug_flags_word;

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_symbol_mutex;
void* g_scratch_ptr[kMaxDevices] = {};
void* g_debug_ptr[kMaxDevices] = {};

// Device address of a library symbol (`sym` is its host-side handle) on the
// device of `stream`, looked up once per device with that device current.
mla_status symbol_address(hipStream_t stream, const void* sym, void* (&cache)[kMaxDevices], void** ptr) {
  int cur = 0, dev = 0;
  hipError_t e = hipGetDevice(&cur);
  if (e != hipSuccess) return hip_status(e);
  dev = cur;
  if (stream) {
    e = hipStreamGetDevice(stream, &dev);
    if (e != hipSuccess) return hip_status(e);
  }
  if (dev < 0 || dev >= kMaxDevices) return MLA_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_symbol_mutex);
  if (!cache[dev]) {
    if (dev != cur && (e = hipSetDevice(dev)) != hipSuccess) return hip_status(e);
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, sym);
    if (dev != cur) {
      const hipError_t e2 = hipSetDevice(cur);
      if (e == hipSuccess) e = e2;
    }
    if (e != hipSuccess) return hip_status(e);
    cache[dev] = p;
  }
  *ptr = cache[dev];
  return MLA_OK;
}

// Device address of the static partials array on the device of `stream`.
mla_status static_scratch(hipStream_t stream, void** ptr) {
  return symbol_address(stream, HIP_SYMBOL(scratch), g_scratch_ptr, ptr);
}

// Debug build: the flag word of the device of `stream` (release: none).
mla_status debug_flags_ptr(hipStream_t stream, uint32_t** ptr) {
  *ptr = nullptr;
  if constexpr (!mla::kDebug) return MLA_OK;
  void* p = nullptr;
  const mla_status st = symbol_address(stream, (const void*)&debug_flags_word, g_debug_ptr, &p);
  *ptr = (uint32_t*)p;
  return st;
}

// One attention call: split launch (+ merge when S > 1).  With static_ws the
// partials go to the static array instead of the caller's workspace.
mla_status attend(const mla_params* p, int max_q, const void* q, const void* kv,
                  const int32_t* pt, const int32_t* sl, float softmax_scale, float kv_scale,
                  void* out, float* lse, void* ws, size_t ws_bytes, void* stream,
                  bool static_ws = false) {
  mla_status st = check_params(p, max_q);
  if (st != MLA_OK) return st;
  if (!q || !kv || !pt || !sl || !out || !lse) return MLA_ERR_NULL_ARG;
  st = check_scales(softmax_scale, kv_scale, p->kv_dtype);
  if (st != MLA_OK) return st;
  const int32_t S = choose_splits(p);
  hipStream_t s = (hipStream_t)stream;
  mla::SplitArgs a = make_args(p, q, kv, pt, sl, softmax_scale, kv_scale, S);
  a.by_length = uses_by_length(p, S) ? 1 : 0;
  if (!launches_fit(a, p, S)) return MLA_ERR_UNSUPPORTED;
  st = debug_flags_ptr(s, &a.debug_flags);
  if (st != MLA_OK) return st;
  if (S == 1) {
    a.out = (uint16_t*)out;
    a.lse = lse;
    return hip_status(mla::launch_split(a, p->kv_dtype == MLA_KV_FP8_E4M3, true, s));
  }
  const size_t need = partial_bytes(p, S);
  if (static_ws) {
    if (need > MLA_STATIC_SCRATCH_BYTES) return MLA_ERR_SCRATCH_LIMIT;
    st = static_scratch(s, &ws);
    if (st != MLA_OK) return st;
  } else if (!ws || ws_bytes < need) {
    return MLA_ERR_WORKSPACE;
  }
  const size_t rows = rows_of(p) * (size_t)S;
  a.part_out = (uint16_t*)ws;
  a.part_lse = (float*)((char*)ws + align256(rows * mla::kValue * sizeof(uint16_t)));
  st = hip_status(mla::launch_split(a, p->kv_dtype == MLA_KV_FP8_E4M3, false, s));
  if (st != MLA_OK) return st;
  mla::MergeArgs m{};
  m.part_out = a.part_out;
  m.part_lse = a.part_lse;
  m.out = (uint16_t*)out;
  m.lse = lse;
  m.rows = (int64_t)rows_of(p);
  m.num_splits = S;
  m.by_length = a.by_length;
  m.batch = p->batch;
  m.rows_per_seq = p->num_q_tokens * p->num_heads;
  m.max_blocks = p->max_blocks_per_seq;
  m.seq_lens = sl;
  return hip_status(mla::launch_merge(m, s));
}

}  // namespace

extern "C" {

int32_t mla_num_splits(const mla_params* p) {
  if (check_params(p, mla::kMaxQ) != MLA_OK) return 0;
  return choose_splits(p);
}

size_t mla_workspace_size(const mla_params* p) {
  if (check_params(p, mla::kMaxQ) != MLA_OK) return 0;
  const int32_t S = choose_splits(p);
  return S == 1 ? 0 : partial_bytes(p, S);
}

mla_status mla_decode(const mla_params* p, const void* q, const void* kv_cache,
                      const int32_t* page_table, const int32_t* seq_lens, float softmax_scale,
                      float kv_scale, void* out, float* lse, void* workspace,
                      size_t workspace_bytes, void* stream) {
  return attend(p, 1, q, kv_cache, page_table, seq_lens, softmax_scale, kv_scale, out, lse,
                workspace, workspace_bytes, stream);
}

mla_status mla_verify(const mla_params* p, const void* q, const void* kv_cache,
                      const int32_t* page_table, const int32_t* seq_lens, float softmax_scale,
                      float kv_scale, void* out, float* lse, void* workspace,
                      size_t workspace_bytes, void* stream) {
  return attend(p, mla::kMaxQ, q, kv_cache, page_table, seq_lens, softmax_scale, kv_scale, out,
                lse, workspace, workspace_bytes, stream);
}

mla_status mla_verify_static(const mla_params* p, const void* q, const void* kv_cache,
                             const int32_t* page_table, const int32_t* seq_lens, float softmax_scale,
                             float kv_scale, void* out, float* lse, void* stream) {
  return attend(p, mla::kMaxQ, q, kv_cache, page_table, seq_lens, softmax_scale, kv_scale, out,
                lse, nullptr, 0, stream, true);
}

mla_status mla_split(const mla_params* p, const void* q, const void* kv_cache,
                     const int32_t* page_table, const int32_t* seq_lens, float softmax_scale,
                     float kv_scale, void* part_out, float* part_lse, void* stream) {
  mla_status st = check_params(p, mla::kMaxQ);
  if (st != MLA_OK) return st;
  if (p->split_policy != MLA_SPLIT_PER_SEQUENCE) return MLA_ERR_UNSUPPORTED;   // partials per sequence
  if (!q || !kv_cache || !page_table || !seq_lens || !part_out || !part_lse) return MLA_ERR_NULL_ARG;
  st = check_scales(softmax_scale, kv_scale, p->kv_dtype);
  if (st != MLA_OK) return st;
  const int32_t S = choose_splits(p);
  mla::SplitArgs a = make_args(p, q, kv_cache, page_table, seq_lens, softmax_scale, kv_scale, S);
  if (mla::split_work_items(a, p->kv_dtype == MLA_KV_FP8_E4M3) > mla::kMaxWorkItems)
    return MLA_ERR_UNSUPPORTED;
  st = debug_flags_ptr((hipStream_t)stream, &a.debug_flags);
  if (st != MLA_OK) return st;
  a.part_out = (uint16_t*)part_out;
  a.part_lse = part_lse;
  return hip_status(mla::launch_split(a, p->kv_dtype == MLA_KV_FP8_E4M3, false, (hipStream_t)stream));
}

mla_status mla_merge(const void* part_out, const float* part_lse, int32_t num_splits, int64_t rows,
                     void* out, float* lse, void* stream) {
  if (!part_out || !part_lse || !out || !lse) return MLA_ERR_NULL_ARG;
  if (num_splits < 1 || num_splits > 4096) return MLA_ERR_BAD_SHAPE;
  if (rows < 1 || rows > ((int64_t)1 << 28)) return MLA_ERR_BAD_SHAPE;
  mla::MergeArgs m{};
  m.part_out = (const uint16_t*)part_out;
  m.part_lse = part_lse;
  m.out = (uint16_t*)out;
  m.lse = lse;
  m.rows = rows;
  m.num_splits = num_splits;
  if (mla::merge_work_items(m) > mla::kMaxWorkItems) return MLA_ERR_UNSUPPORTED;
  return hip_status(mla::launch_merge(m, (hipStream_t)stream));
}

mla_status mla_kv_append(const mla_params* p, const void* kv_new, void* kv_cache,
                         const int32_t* page_table, const int32_t* seq_lens, float kv_scale,
                         void* stream) {
  if (!p) return MLA_ERR_NULL_ARG;
  if (p->batch < 1 || p->batch > 65535) return MLA_ERR_BAD_SHAPE;
  if (p->num_q_tokens < 1 || p->num_q_tokens > mla::kMaxQ) return MLA_ERR_BAD_SHAPE;
  if (p->num_blocks < 1 || p->max_blocks_per_seq < 1) return MLA_ERR_BAD_SHAPE;
  if (p->kv_dtype != MLA_KV_BF16 && p->kv_dtype != MLA_KV_FP8_E4M3) return MLA_ERR_BAD_DTYPE;
  if (!kv_new || !kv_cache || !page_table || !seq_lens) return MLA_ERR_NULL_ARG;
  if (((uintptr_t)kv_new | (uintptr_t)kv_cache) & 15) return MLA_ERR_BAD_SHAPE;   // 16-byte rows
  const bool fp8 = p->kv_dtype == MLA_KV_FP8_E4M3;
  if (fp8 && !(isfinite(kv_scale) && kv_scale > 0.f)) return MLA_ERR_BAD_SCALE;
  mla::AppendArgs a{};
  a.kv_new = (const uint16_t*)kv_new;
  a.kv = (uint8_t*)kv_cache;
  a.page_table = page_table;
  a.seq_lens = seq_lens;
  a.batch = p->batch;
  a.num_q = p->num_q_tokens;
  a.max_blocks = p->max_blocks_per_seq;
  a.num_blocks = p->num_blocks;
  a.kv_scale = fp8 ? kv_scale : 1.f;
  const mla_status st = debug_flags_ptr((hipStream_t)stream, &a.debug_flags);
  if (st != MLA_OK) return st;
  return hip_status(mla::launch_append(a, fp8, (hipStream_t)stream));
}

mla_status mla_kv_dynamic_scale(const void* x, int64_t count, float* scale, void* stream) {
  if (!x || !scale) return MLA_ERR_NULL_ARG;
  if (count < 0 || count > ((int64_t)1 << 40)) return MLA_ERR_BAD_SHAPE;
  if ((uintptr_t)scale & 3) return MLA_ERR_BAD_SHAPE;
  return hip_status(mla::launch_dynamic_scale((const uint16_t*)x, count, scale, (hipStream_t)stream));
}

const char* mla_status_string(int32_t status) {
  switch (status) {
    case MLA_OK: return "ok";
    case MLA_ERR_NULL_ARG: return "a required pointer is NULL";
    case MLA_ERR_BAD_SHAPE: return "a size is out of range";
    case MLA_ERR_BAD_DTYPE: return "unknown kv_dtype";
    case MLA_ERR_BAD_SCALE: return "softmax_scale not finite, or kv_scale not finite and positive";
    case MLA_ERR_UNSUPPORTED: return "request not supported by this library";
    case MLA_ERR_WORKSPACE: return "workspace missing or smaller than mla_workspace_size()";
    case MLA_ERR_HIP: return "HIP runtime error (see mla_last_hip_error)";
    case MLA_ERR_SCRATCH_LIMIT:
      return "partials exceed the static scratch of mla_verify_static (MLA_STATIC_SCRATCH_BYTES)";
    default: return "unknown status";
  }
}

int32_t mla_last_hip_error(void) { return g_last_hip_error; }

int32_t mla_debug_build(void) { return mla::kDebug ? 1 : 0; }

mla_status mla_debug_flags(uint32_t* flags, int32_t clear) {
  if (!flags) return MLA_ERR_NULL_ARG;
  *flags = 0;
  if constexpr (!mla::kDebug) return MLA_OK;
  hipError_t e = hipMemcpyFromSymbol(flags, HIP_SYMBOL(debug_flags_word), sizeof(uint32_t));
  if (e != hipSuccess) return hip_status(e);
  if (clear) {
    const uint32_t zero = 0;
    e = hipMemcpyToSymbol(HIP_SYMBOL(debug_flags_word), &zero, sizeof(uint32_t));
    if (e != hipSuccess) return hip_status(e);
  }
  return MLA_OK;
}

}  // extern "C"
