"""Float64 CPU oracle for MLA decode / speculative-verify attention over a paged latent KV cache.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path imports this package:
only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import, call or execute anything here.  It shares no code,
header, table or helper with the HIP path in ``decode_attention_03_amd``.

Sources (web pages; cited by title and section):

* "Inside Kimi K3 optimization: the bottlenecks and decisions that make
  inference faster" (AMD engineering blog, Korean translation), sections
  "1. Cache -- DCP: sharing history across GPUs" and "4. MLA: faster
  long-context decoding with AMD AITER assembly".
* "Kimi K3 on AMD MI355X: better price per token than NVIDIA B300",
  section "What had to be fixed".
* "Kimi K2.6 + DFlash on 8x MI300X (508 tok/s)", section "Technical numbers".

Contents:

* :mod:`oracle.formats` -- exact bit-level decoding of bf16 and OCP FP8 E4M3FN.
* :mod:`oracle.mla`     -- NumPy float64 reference (gather, attend, causal
  verify, partials over position ranges, log-sum-exp merge).
* :mod:`oracle.brute`   -- pure-Python loops with ``math.fsum`` for tiny
  inputs; an independent second implementation used to pin :mod:`oracle.mla`.

Pins (tests/test_oracle_*.py, ``-m "not gpu"``): brute force, closed forms
(single position, tied scores, q = 0, dominant key, verify with L = Q),
split + merge = unsplit, causal verify = truncated decodes, head padding,
page-table permutation invariance, the FP8 table against
``torch.float8_e4m3fn`` and the OCP formula's special values, and
``torch.nn.functional.scaled_dot_product_attention`` in float64.  No function
here is "parity unpinned".
"""

from .formats import bf16_bits_to_f64, e4m3fn_table, decode_kv
from .mla import (
    gather_sequence,
    attend,
    mla_reference,
    mla_partials,
    merge,
)
from .brute import brute_force_mla

__all__ = [
    "bf16_bits_to_f64",
    "e4m3fn_table",
    "decode_kv",
    "gather_sequence",
    "attend",
    "mla_reference",
    "mla_partials",
    "merge",
    "brute_force_mla",
]
