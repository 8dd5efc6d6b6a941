"""MI355X-native MLA decode / speculative-verify attention over a paged latent KV cache.

The compute path is the HIP library ``libmla_hip.so`` (gfx950 kernels behind
the C ABI in ``include/mla.h``); this package only marshals torch tensors to
it.  There is no CPU fallback: if the library is missing, calls fail.
"""

from ._lib import (
    EXPORTS,
    MLAError,
    MLA_KV_BF16,
    MLA_KV_FP8_E4M3,
    SPLIT_BY_LENGTH,
    SPLIT_PER_SEQUENCE,
    Params,
    decode,
    kv_append,
    kv_dynamic_scale,
    load,
    make_params,
    merge,
    num_splits,
    split,
    verify,
    verify_static,
    workspace_size,
    STATIC_SCRATCH_BYTES,
)
from .build import LIB_PATH

__all__ = [
    "EXPORTS", "MLAError", "MLA_KV_BF16", "MLA_KV_FP8_E4M3", "SPLIT_BY_LENGTH",
    "SPLIT_PER_SEQUENCE", "Params", "decode", "kv_append",
    "kv_dynamic_scale", "load",
    "make_params", "merge", "num_splits", "split", "verify", "verify_static", "workspace_size",
    "STATIC_SCRATCH_BYTES", "LIB_PATH",
]
