"""KV-cache append with FP8 quantisation (oracle; test infrastructure only).

The step just before attention in a decode or verify step: the compressed
latents of the Q newest positions of each sequence are written into their
paged cache slots, as bf16 or as FP8 bytes under one per-tensor scale
("Kimi K2.6 + DFlash on 8x MI300X (508 tok/s)", section "st=2 vs st=8 &
FP8 vs BF16": an FP8 KV cache doubles the token capacity, and computing the
scale dynamically costs per-slot throughput; section "Next": the scale is
auto-computed today, and a static calibrated scale is the proposed fix).

Readings taken here (the pages give no formula):

* Slot of new token j of sequence b: position t = L_b - Q + j, where L_b
  counts the Q new tokens (the same reading as the causal verify rule), i.e.
  block page_table[b, t // 16], row t % 16.
* Quantised byte of a bf16 value x under scale s: the E4M3FN code nearest to
  the float32 quotient fp32(x / s), ties to the code with an even mantissa,
  magnitudes beyond 448 saturated to 448.  The quotient is taken in float32
  because that is the precision in which the byte is decided on the GPU.
* Dynamic per-tensor scale of a set of bf16 values: fp32(max|x| / 448), or 1
  when every value is zero (the reading of an "auto-computed" scale).

Everything here is written from the E4M3FN definition (see
:mod:`oracle.formats`): the candidate values are that format's finite
values, found by search, not by a conversion routine.
"""

import numpy as np

from .formats import bf16_bits_to_f64, e4m3fn_table

PAGE = 16
LATENT = 576
E4M3_MAX = 448.0

# non-negative finite E4M3FN values in code order 0x00 .. 0x7E (increasing)
_POS_VALUES = e4m3fn_table()[:0x7F]
assert np.all(np.diff(_POS_VALUES) > 0)


def e4m3fn_quantize(v):
    """float32 values -> E4M3FN codes (uint8): nearest, ties to even, saturating.

    For |v| between two consecutive non-negative values a < b (codes c, c+1),
    the nearer one is taken; at the exact midpoint, the one whose code is even
    (its mantissa's last bit is 0).  |v| >= 448 gives code 0x7E (448).  The
    sign bit is the sign of v (so -0.0 and negative values that round to
    zero give 0x80).  Inputs must be finite.
    """
    v = np.asarray(v, dtype=np.float32)
    mag = np.abs(v).astype(np.float64)          # exact
    if not np.all(np.isfinite(mag)):
        raise ValueError("e4m3fn_quantize needs finite inputs")
    mag = np.minimum(mag, E4M3_MAX)
    hi = np.searchsorted(_POS_VALUES, mag, side="left")   # first value >= mag
    hi = np.minimum(hi, 0x7E)
    lo = np.maximum(hi - 1, 0)
    dlo = mag - _POS_VALUES[lo]
    dhi = _POS_VALUES[hi] - mag
    pick_hi = (dhi < dlo) | ((dhi == dlo) & (hi % 2 == 0))
    code = np.where(pick_hi, hi, lo)
    code = np.where(mag == _POS_VALUES[hi], hi, code)     # exact values
    sign = np.signbit(v).astype(np.int64) << 7
    return (code | sign).astype(np.uint8)


def quantize_bf16(x_bits, kv_scale):
    """bf16 bit patterns -> E4M3FN codes of fp32(x / kv_scale)."""
    x = bf16_bits_to_f64(x_bits).astype(np.float32)       # exact
    q = x / np.float32(kv_scale)                          # IEEE float32 division
    return e4m3fn_quantize(q)


def dynamic_scale(x_bits):
    """Per-tensor scale of bf16 values: fp32(max|x| / 448), 1.0 if all are zero."""
    x = np.abs(bf16_bits_to_f64(np.asarray(x_bits).reshape(-1)))
    amax = np.float32(x.max()) if x.size else np.float32(0.0)
    if amax == 0:
        return np.float32(1.0)
    return np.float32(amax) / np.float32(E4M3_MAX)


def append_slots(seq_lens, num_q):
    """[(b, j, t)] for every new token: position t = L_b - Q + j."""
    out = []
    for b, L in enumerate(np.asarray(seq_lens).tolist()):
        for j in range(num_q):
            out.append((b, j, int(L) - num_q + j))
    return out


def kv_append(kv_cache, page_table, seq_lens, kv_new_bits, kv_dtype, kv_scale=1.0):
    """Return a copy of the cache with the new latents written into their slots.

    kv_cache    : uint16 bf16 bits [blocks][16][576] or uint8 FP8 codes
    page_table  : int32 [B][max_blocks]
    seq_lens    : int32 [B], each >= Q (they count the new tokens)
    kv_new_bits : uint16 bf16 bits [B][Q][576]
    """
    out = np.array(kv_cache, copy=True)
    new = np.asarray(kv_new_bits, dtype=np.uint16)
    num_q = new.shape[1]
    for b, j, t in append_slots(seq_lens, num_q):
        blk = int(page_table[b][t // PAGE])
        row = new[b, j]
        if kv_dtype == "bf16":
            out[blk, t % PAGE] = row
        elif kv_dtype == "fp8":
            out[blk, t % PAGE] = quantize_bf16(row, kv_scale)
        else:
            raise ValueError(f"unknown kv_dtype {kv_dtype!r}")
    return out
