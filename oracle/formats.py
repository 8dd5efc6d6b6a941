"""Exact decoding of the stored number formats (oracle; test infrastructure only).

The latent KV cache holds either bf16 values or FP8 bytes with one per-tensor
float32 scale ("Inside Kimi K3 optimization", section "1. Cache -- DCP":
576 FP8 bytes per cached position; "Kimi K2.6 + DFlash on 8x MI300X",
sections "Technical numbers" and "Next": FP8 KV cache with an auto-computed
per-tensor scale).  The pages do not name the FP8 variant; the reading taken
here is OCP E4M3FN (bias 7, subnormals, no infinities, NaN = S.1111.111),
the variant gfx950 implements natively.

Both decoders are exact: every bf16 and every finite E4M3FN value is a
float64 value.
"""

import math

import numpy as np


def bf16_bits_to_f64(bits):
    """bf16 bit patterns (uint16 array) -> float64.

    A bf16 value is by definition the binary32 value whose upper 16 bits are
    the pattern and whose lower 16 bits are zero.
    """
    b = np.asarray(bits).astype(np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def e4m3fn_value(code):
    """Value of one OCP E4M3FN byte, from the format's definition.

    sign s = bit 7, exponent e = bits 6..3 (bias 7), mantissa m = bits 2..0:
      e >= 1: (-1)^s * 2^(e-7) * (1 + m/8)
      e == 0: (-1)^s * 2^(-6) * (m/8)          (subnormal; m = 0 is +-0)
      e == 15 and m == 7: NaN                   (the format has no infinity)
    """
    code = int(code) & 0xFF
    s = (code >> 7) & 1
    e = (code >> 3) & 0xF
    m = code & 0x7
    if e == 0xF and m == 0x7:
        return math.nan
    sign = -1.0 if s else 1.0
    if e == 0:
        return sign * math.ldexp(m / 8.0, -6)
    return sign * math.ldexp(1.0 + m / 8.0, e - 7)


def e4m3fn_table():
    """256-entry float64 table: code -> value (NaN for 0x7F and 0xFF)."""
    return np.array([e4m3fn_value(c) for c in range(256)], dtype=np.float64)


_E4M3FN = e4m3fn_table()


def decode_kv(raw, kv_dtype, kv_scale=1.0):
    """Stored KV -> float64 values.

    raw      : uint16 bf16 bit patterns (kv_dtype "bf16") or uint8 FP8 codes
               (kv_dtype "fp8"), any shape.
    kv_scale : float32 per-tensor scale; the dequantised value of a byte is
               decode(byte) * kv_scale.  Ignored for bf16.
    """
    if kv_dtype == "bf16":
        return bf16_bits_to_f64(raw)
    if kv_dtype == "fp8":
        return _E4M3FN[np.asarray(raw, dtype=np.uint8)] * np.float64(np.float32(kv_scale))
    raise ValueError(f"unknown kv_dtype {kv_dtype!r}")
