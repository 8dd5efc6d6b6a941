"""ctypes binding of libmla_hip.so (argument marshalling only).

Every function here checks tensor placement, dtype and contiguity, allocates
missing outputs/workspace with torch on the query's device, and calls the C
entry point of the same name on the current HIP stream.  All arithmetic runs
in the HIP kernels; if the library is missing, loading fails loudly.
"""

import ctypes
import os

import torch

from .build import DEBUG_LIB_PATH, LIB_PATH

MLA_KV_BF16 = 0
MLA_KV_FP8_E4M3 = 1
# mla_split_policy
SPLIT_PER_SEQUENCE = 0
SPLIT_BY_LENGTH = 1
LATENT_DIM = 576
VALUE_DIM = 512

_STATUS_NAMES = {
    0: "MLA_OK", 1: "MLA_ERR_NULL_ARG", 2: "MLA_ERR_BAD_SHAPE", 3: "MLA_ERR_BAD_DTYPE",
    4: "MLA_ERR_BAD_SCALE", 5: "MLA_ERR_UNSUPPORTED", 6: "MLA_ERR_WORKSPACE", 7: "MLA_ERR_HIP",
    8: "MLA_ERR_SCRATCH_LIMIT",
}
STATIC_SCRATCH_BYTES = 96 << 20   # MLA_STATIC_SCRATCH_BYTES

# Every symbol include/mla.h declares.
EXPORTS = ("mla_num_splits", "mla_workspace_size", "mla_decode", "mla_verify", "mla_verify_static",
           "mla_split", "mla_merge", "mla_kv_append", "mla_kv_dynamic_scale", "mla_status_string",
           "mla_last_hip_error", "mla_debug_build", "mla_debug_flags")
# Every symbol include/mla_peaks.h declares (measured-peak microbenchmarks).
PEAK_EXPORTS = ("mla_peak_hbm_read", "mla_peak_mfma")
PEAK_READ_VGPR, PEAK_READ_LDS = 0, 1
PEAK_MFMA_FP8, PEAK_MFMA_BF16 = 0, 1
# Contract violations reported by the debug build (MLA_DEBUG_* of include/mla.h).
DEBUG_PAGE_ID, DEBUG_SEQ_SHORT, DEBUG_SEQ_LONG = 1, 2, 4


class MLAError(RuntimeError):
    def __init__(self, status, message):
        super().__init__(f"{_STATUS_NAMES.get(status, status)}: {message}")
        self.status = status


class Params(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int32),
        ("num_q_tokens", ctypes.c_int32),
        ("num_heads", ctypes.c_int32),
        ("num_blocks", ctypes.c_int32),
        ("max_blocks_per_seq", ctypes.c_int32),
        ("max_seq_len_hint", ctypes.c_int32),
        ("kv_dtype", ctypes.c_int32),
        ("num_splits", ctypes.c_int32),
        ("split_policy", ctypes.c_int32),
    ]


_LIB = None


def _configure(lib):
    vp, i32, f32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_float, ctypes.c_size_t
    pp = ctypes.POINTER(Params)
    lib.mla_num_splits.argtypes = [pp]
    lib.mla_num_splits.restype = i32
    lib.mla_workspace_size.argtypes = [pp]
    lib.mla_workspace_size.restype = sz
    for name in ("mla_decode", "mla_verify"):
        fn = getattr(lib, name)
        fn.argtypes = [pp, vp, vp, vp, vp, f32, f32, vp, vp, vp, sz, vp]
        fn.restype = i32
    lib.mla_verify_static.argtypes = [pp, vp, vp, vp, vp, f32, f32, vp, vp, vp]
    lib.mla_verify_static.restype = i32
    lib.mla_split.argtypes = [pp, vp, vp, vp, vp, f32, f32, vp, vp, vp]
    lib.mla_split.restype = i32
    lib.mla_merge.argtypes = [vp, vp, i32, ctypes.c_int64, vp, vp, vp]
    lib.mla_merge.restype = i32
    lib.mla_kv_append.argtypes = [pp, vp, vp, vp, vp, f32, vp]
    lib.mla_kv_append.restype = i32
    lib.mla_kv_dynamic_scale.argtypes = [vp, ctypes.c_int64, vp, vp]
    lib.mla_kv_dynamic_scale.restype = i32
    lib.mla_status_string.argtypes = [i32]
    lib.mla_status_string.restype = ctypes.c_char_p
    lib.mla_last_hip_error.argtypes = []
    lib.mla_last_hip_error.restype = i32
    lib.mla_debug_build.argtypes = []
    lib.mla_debug_build.restype = i32
    lib.mla_debug_flags.argtypes = [ctypes.POINTER(ctypes.c_uint32), i32]
    lib.mla_debug_flags.restype = i32
    lib.mla_peak_hbm_read.argtypes = [vp, ctypes.c_int64, i32, vp, i32, vp]
    lib.mla_peak_hbm_read.restype = i32
    lib.mla_peak_mfma.argtypes = [i32, i32, vp, i32, vp]
    lib.mla_peak_mfma.restype = i32
    return lib


def _open(path):
    if not os.path.exists(path):
        raise RuntimeError(f"HIP library {path} is missing; build it with "
                           "`python -m decode_attention_03_amd.build`")
    return _configure(ctypes.CDLL(path))


def load(path=None):
    """Load the HIP library (once).  Raises if it has not been built."""
    global _LIB
    if _LIB is not None:
        return _LIB
    _LIB = _open(path or LIB_PATH)
    return _LIB


def load_debug():
    """A handle of the debug build (libmla_hip_debug.so, built with MLA_DEBUG=1),
    separate from the one load() returns; raises if it has not been built."""
    return _open(DEBUG_LIB_PATH)


def debug_flags(lib, clear=True):
    """The MLA_DEBUG_* bits the debug library `lib` has reported on the current
    device (synchronous), cleared afterwards unless clear=False."""
    v = ctypes.c_uint32(0)
    _check_lib(lib, lib.mla_debug_flags(ctypes.byref(v), 1 if clear else 0))
    return int(v.value)


def _check_lib(lib, status):
    if status != 0:
        msg = lib.mla_status_string(status).decode()
        if status == 7:
            msg += f" (hipError {lib.mla_last_hip_error()})"
        raise MLAError(status, msg)


def _check(status):
    _check_lib(load(), status)


def _kv_dtype(kv_cache):
    if kv_cache.dtype == torch.bfloat16:
        return MLA_KV_BF16
    if kv_cache.dtype in (torch.uint8, torch.float8_e4m3fn):
        return MLA_KV_FP8_E4M3
    raise MLAError(3, f"kv_cache dtype {kv_cache.dtype} is neither bfloat16 nor FP8 E4M3FN bytes")


def make_params(q, kv_cache, page_table, num_splits=0, max_seq_len_hint=0,
                split_policy=SPLIT_PER_SEQUENCE):
    return Params(batch=q.shape[0], num_q_tokens=q.shape[1], num_heads=q.shape[2],
                  num_blocks=kv_cache.shape[0], max_blocks_per_seq=page_table.shape[1],
                  max_seq_len_hint=int(max_seq_len_hint), kv_dtype=_kv_dtype(kv_cache),
                  num_splits=int(num_splits), split_policy=int(split_policy))


def _check_inputs(q, kv_cache, page_table, seq_lens):
    dev = q.device
    if dev.type != "cuda":
        raise MLAError(2, "q must be a GPU tensor")
    for name, t in (("kv_cache", kv_cache), ("page_table", page_table), ("seq_lens", seq_lens)):
        if t.device != dev:
            raise MLAError(2, f"{name} is on {t.device}, q on {dev}")
    if q.dtype != torch.bfloat16 or q.dim() != 4 or q.shape[3] != LATENT_DIM or not q.is_contiguous():
        raise MLAError(2, "q must be contiguous bf16 [B, Q, H, 576]")
    if kv_cache.dim() != 3 or kv_cache.shape[1:] != (16, LATENT_DIM) or not kv_cache.is_contiguous():
        raise MLAError(2, "kv_cache must be contiguous [num_blocks, 16, 576]")
    if page_table.dtype != torch.int32 or page_table.dim() != 2 or not page_table.is_contiguous() \
            or page_table.shape[0] != q.shape[0]:
        raise MLAError(2, "page_table must be contiguous int32 [B, max_blocks_per_seq]")
    if seq_lens.dtype != torch.int32 or seq_lens.shape != (q.shape[0],) or not seq_lens.is_contiguous():
        raise MLAError(2, "seq_lens must be contiguous int32 [B]")


def _check_out(name, t, dtype, shape, dev):
    """A caller-supplied output: contiguous, of the kernel's dtype and shape, on dev."""
    if t.dtype != dtype or tuple(t.shape) != tuple(shape) or not t.is_contiguous() \
            or t.device != dev:
        raise MLAError(2, f"{name} must be a contiguous {dtype} tensor of shape {tuple(shape)} "
                          f"on {dev} (got {t.dtype} {tuple(t.shape)} on {t.device})")


def _stream(dev):
    return ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)


def num_splits(q, kv_cache, page_table, num_splits=0, max_seq_len_hint=0):
    p = make_params(q, kv_cache, page_table, num_splits, max_seq_len_hint)
    return int(load().mla_num_splits(ctypes.byref(p)))


def workspace_size(q, kv_cache, page_table, num_splits=0, max_seq_len_hint=0):
    p = make_params(q, kv_cache, page_table, num_splits, max_seq_len_hint)
    return int(load().mla_workspace_size(ctypes.byref(p)))


def _attend(entry, q, kv_cache, page_table, seq_lens, softmax_scale, kv_scale, num_splits,
            max_seq_len_hint, out, lse, workspace, split_policy):
    lib = load()
    _check_inputs(q, kv_cache, page_table, seq_lens)
    p = make_params(q, kv_cache, page_table, num_splits, max_seq_len_hint, split_policy)
    B, Q, H, _ = q.shape
    if out is None:
        out = torch.empty((B, Q, H, VALUE_DIM), dtype=torch.bfloat16, device=q.device)
    if lse is None:
        lse = torch.empty((B, Q, H), dtype=torch.float32, device=q.device)
    _check_out("out", out, torch.bfloat16, (B, Q, H, VALUE_DIM), q.device)
    _check_out("lse", lse, torch.float32, (B, Q, H), q.device)
    need = int(lib.mla_workspace_size(ctypes.byref(p)))
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    if workspace is not None and (workspace.device != q.device or not workspace.is_contiguous()):
        raise MLAError(6, f"workspace must be contiguous on {q.device}")
    ws_ptr = workspace.data_ptr() if workspace is not None else None
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(getattr(lib, entry)(ctypes.byref(p), q.data_ptr(), kv_cache.data_ptr(),
                               page_table.data_ptr(), seq_lens.data_ptr(), float(softmax_scale),
                               float(kv_scale), out.data_ptr(), lse.data_ptr(), ws_ptr, ws_bytes,
                               _stream(q.device)))
    return out, lse


def decode(q, kv_cache, page_table, seq_lens, softmax_scale, kv_scale=1.0, num_splits=0,
           max_seq_len_hint=0, out=None, lse=None, workspace=None,
           split_policy=SPLIT_PER_SEQUENCE):
    """mla_decode: Q = 1.  Returns (out bf16 [B,1,H,512], lse fp32 [B,1,H])."""
    return _attend("mla_decode", q, kv_cache, page_table, seq_lens, softmax_scale, kv_scale,
                   num_splits, max_seq_len_hint, out, lse, workspace, split_policy)


def verify(q, kv_cache, page_table, seq_lens, softmax_scale, kv_scale=1.0, num_splits=0,
           max_seq_len_hint=0, out=None, lse=None, workspace=None,
           split_policy=SPLIT_PER_SEQUENCE):
    """mla_verify: Q query tokens with the causal rule.  Returns (out, lse)."""
    return _attend("mla_verify", q, kv_cache, page_table, seq_lens, softmax_scale, kv_scale,
                   num_splits, max_seq_len_hint, out, lse, workspace, split_policy)


def verify_static(q, kv_cache, page_table, seq_lens, softmax_scale, kv_scale=1.0, num_splits=0,
                  max_seq_len_hint=0, out=None, lse=None, split_policy=SPLIT_PER_SEQUENCE):
    """mla_verify_static: as verify, with the split partials in the library's static
    per-GPU array instead of a workspace (the C call allocates nothing).  Calls
    that overlap in time on one GPU race on that array."""
    lib = load()
    _check_inputs(q, kv_cache, page_table, seq_lens)
    p = make_params(q, kv_cache, page_table, num_splits, max_seq_len_hint, split_policy)
    B, Q, H, _ = q.shape
    if out is None:
        out = torch.empty((B, Q, H, VALUE_DIM), dtype=torch.bfloat16, device=q.device)
    if lse is None:
        lse = torch.empty((B, Q, H), dtype=torch.float32, device=q.device)
    _check_out("out", out, torch.bfloat16, (B, Q, H, VALUE_DIM), q.device)
    _check_out("lse", lse, torch.float32, (B, Q, H), q.device)
    _check(lib.mla_verify_static(ctypes.byref(p), q.data_ptr(), kv_cache.data_ptr(),
                                 page_table.data_ptr(), seq_lens.data_ptr(), float(softmax_scale),
                                 float(kv_scale), out.data_ptr(), lse.data_ptr(),
                                 _stream(q.device)))
    return out, lse


def split(q, kv_cache, page_table, seq_lens, softmax_scale, kv_scale=1.0, num_splits=0,
          max_seq_len_hint=0, part_out=None, part_lse=None):
    """mla_split: returns (part_out bf16 [S,B,Q,H,512], part_lse fp32 [S,B,Q,H])."""
    lib = load()
    _check_inputs(q, kv_cache, page_table, seq_lens)
    p = make_params(q, kv_cache, page_table, num_splits, max_seq_len_hint)
    S = int(lib.mla_num_splits(ctypes.byref(p)))
    if S < 1:
        raise MLAError(2, "invalid parameters")
    B, Q, H, _ = q.shape
    if part_out is None:
        part_out = torch.empty((S, B, Q, H, VALUE_DIM), dtype=torch.bfloat16, device=q.device)
    if part_lse is None:
        part_lse = torch.empty((S, B, Q, H), dtype=torch.float32, device=q.device)
    if part_out.dtype != torch.bfloat16 or part_lse.dtype != torch.float32 \
            or not part_out.is_contiguous() or not part_lse.is_contiguous() \
            or part_out.device != q.device or part_lse.device != q.device:
        raise MLAError(2, "partials must be contiguous on q's device "
                          "(part_out bfloat16, part_lse float32)")
    if part_out.numel() < S * B * Q * H * VALUE_DIM or part_lse.numel() < S * B * Q * H:
        raise MLAError(2, "part_out / part_lse too small")
    _check(lib.mla_split(ctypes.byref(p), q.data_ptr(), kv_cache.data_ptr(), page_table.data_ptr(),
                         seq_lens.data_ptr(), float(softmax_scale), float(kv_scale),
                         part_out.data_ptr(), part_lse.data_ptr(), _stream(q.device)))
    return part_out, part_lse


def merge(part_out, part_lse, out=None, lse=None):
    """mla_merge over axis 0: part_out bf16 [S, ..., 512], part_lse fp32 [S, ...]."""
    lib = load()
    S = part_out.shape[0]
    lead = tuple(part_out.shape[1:-1])
    if part_out.shape[-1] != VALUE_DIM or tuple(part_lse.shape) != (S,) + lead:
        raise MLAError(2, "part_out must be [S, ..., 512] and part_lse [S, ...]")
    if part_out.dtype != torch.bfloat16 or part_lse.dtype != torch.float32 \
            or not part_out.is_contiguous() or not part_lse.is_contiguous():
        raise MLAError(2, "partials must be contiguous (part_out bfloat16, part_lse float32)")
    dev = part_out.device
    if dev.type != "cuda" or part_lse.device != dev:
        raise MLAError(2, "part_out and part_lse must be on the same GPU")
    rows = 1
    for d in lead:
        rows *= int(d)
    if out is None:
        out = torch.empty(lead + (VALUE_DIM,), dtype=torch.bfloat16, device=dev)
    if lse is None:
        lse = torch.empty(lead, dtype=torch.float32, device=dev)
    _check_out("out", out, torch.bfloat16, lead + (VALUE_DIM,), dev)
    _check_out("lse", lse, torch.float32, lead, dev)
    _check(lib.mla_merge(part_out.data_ptr(), part_lse.data_ptr(), S, rows, out.data_ptr(),
                         lse.data_ptr(), _stream(part_out.device)))
    return out, lse


def kv_append(kv_new, kv_cache, page_table, seq_lens, kv_scale=1.0):
    """mla_kv_append: kv_new bf16 [B, Q, 576] into kv_cache (bf16 or FP8 bytes) in place."""
    lib = load()
    dev = kv_new.device
    if dev.type != "cuda":
        raise MLAError(2, "kv_new must be a GPU tensor")
    for name, t in (("kv_cache", kv_cache), ("page_table", page_table), ("seq_lens", seq_lens)):
        if t.device != dev:
            raise MLAError(2, f"{name} is on {t.device}, kv_new on {dev}")
    if kv_new.dtype != torch.bfloat16 or kv_new.dim() != 3 or kv_new.shape[2] != LATENT_DIM \
            or not kv_new.is_contiguous():
        raise MLAError(2, "kv_new must be contiguous bf16 [B, Q, 576]")
    if kv_cache.dim() != 3 or kv_cache.shape[1:] != (16, LATENT_DIM) or not kv_cache.is_contiguous():
        raise MLAError(2, "kv_cache must be contiguous [num_blocks, 16, 576]")
    B, Q = kv_new.shape[0], kv_new.shape[1]
    if page_table.dtype != torch.int32 or page_table.dim() != 2 or page_table.shape[0] != B \
            or not page_table.is_contiguous():
        raise MLAError(2, "page_table must be contiguous int32 [B, max_blocks_per_seq]")
    if seq_lens.dtype != torch.int32 or seq_lens.shape != (B,) or not seq_lens.is_contiguous():
        raise MLAError(2, "seq_lens must be contiguous int32 [B]")
    p = Params(batch=B, num_q_tokens=Q, num_heads=1, num_blocks=kv_cache.shape[0],
               max_blocks_per_seq=page_table.shape[1], max_seq_len_hint=0,
               kv_dtype=_kv_dtype(kv_cache), num_splits=0)
    _check(lib.mla_kv_append(ctypes.byref(p), kv_new.data_ptr(), kv_cache.data_ptr(),
                             page_table.data_ptr(), seq_lens.data_ptr(), float(kv_scale),
                             _stream(dev)))
    return kv_cache


def kv_dynamic_scale(x, scale=None):
    """mla_kv_dynamic_scale over every value of the bf16 tensor x -> float32 [1] on x's device."""
    lib = load()
    if x.device.type != "cuda" or x.dtype != torch.bfloat16 or not x.is_contiguous():
        raise MLAError(2, "x must be a contiguous bf16 GPU tensor")
    if scale is None:
        scale = torch.empty((1,), dtype=torch.float32, device=x.device)
    if scale.dtype != torch.float32 or scale.device != x.device or scale.numel() < 1:
        raise MLAError(2, "scale must be a float32 tensor on x's device")
    _check(lib.mla_kv_dynamic_scale(x.data_ptr(), x.numel(), scale.data_ptr(), _stream(x.device)))
    return scale


def peak_hbm_read(buf, mode, sink, workgroups):
    """One streaming read of the uint8 device tensor `buf` (mla_peak_hbm_read)
    on the current stream; `sink` is a uint32 device tensor of >= workgroups."""
    assert buf.is_cuda and buf.dtype == torch.uint8 and buf.is_contiguous()
    assert sink.is_cuda and sink.dtype == torch.int32 and sink.numel() >= workgroups
    lib = load()
    _check(lib.mla_peak_hbm_read(buf.data_ptr(), buf.numel(), mode, sink.data_ptr(), workgroups,
                                 _stream(buf.device)))


def peak_mfma(kind, iters, sink, workgroups):
    """One dense MFMA stream (mla_peak_mfma) on the current stream; `sink` is a
    float32 device tensor of >= workgroups."""
    assert sink.is_cuda and sink.dtype == torch.float32 and sink.numel() >= workgroups
    lib = load()
    _check(lib.mla_peak_mfma(kind, iters, sink.data_ptr(), workgroups, _stream(sink.device)))
