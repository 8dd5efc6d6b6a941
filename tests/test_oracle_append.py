"""Pins of the KV-append oracle (oracle.append) to facts outside itself:
the E4M3FN definition (every finite code round-trips, midpoints go to the
even code, saturation at 448), torch's own float32 -> float8_e4m3fn
conversion (an independent round-to-nearest-even implementation), closed
forms of the dynamic scale, and hand-placed slots of the append."""

import math

import numpy as np
import pytest
import torch

from oracle import append as oa
from oracle.formats import e4m3fn_value, e4m3fn_table

FINITE_CODES = [c for c in range(256) if c not in (0x7F, 0xFF)]


def _bf16_bits(x):
    return torch.tensor(np.asarray(x, dtype=np.float32)).to(torch.bfloat16).view(torch.int16) \
        .numpy().view(np.uint16)


def test_every_finite_code_round_trips():
    vals = np.array([e4m3fn_value(c) for c in FINITE_CODES], dtype=np.float32)
    got = oa.e4m3fn_quantize(vals)
    assert got.tolist() == FINITE_CODES


def test_midpoints_go_to_even_code_and_neighbours_to_nearest():
    t = e4m3fn_table()
    for c in range(0x7E):
        a, b = np.float32(t[c]), np.float32(t[c + 1])
        mid = np.float32((t[c] + t[c + 1]) / 2)      # exact: at most 5 significant bits
        assert float(mid) == (t[c] + t[c + 1]) / 2
        even = c if c % 2 == 0 else c + 1
        assert oa.e4m3fn_quantize([mid])[0] == even, c
        assert oa.e4m3fn_quantize([np.nextafter(mid, a)])[0] == c, c
        assert oa.e4m3fn_quantize([np.nextafter(mid, b)])[0] == c + 1, c
        # negative side mirrors with the sign bit
        assert oa.e4m3fn_quantize([-mid])[0] == (even | 0x80), c


def test_saturation_and_signed_zero():
    q = oa.e4m3fn_quantize(np.array([448, 449, 464, 480, 1e30, -448, -500, -3e38], np.float32))
    assert q.tolist() == [0x7E, 0x7E, 0x7E, 0x7E, 0x7E, 0xFE, 0xFE, 0xFE]
    q = oa.e4m3fn_quantize(np.array([0.0, -0.0, 2.0 ** -11, -(2.0 ** -11), 2.0 ** -10,
                                     2.0 ** -10 * 1.0001], np.float32))
    # 2^-10 is the midpoint between 0 and the smallest subnormal 2^-9: ties to code 0
    assert q.tolist() == [0x00, 0x80, 0x00, 0x80, 0x00, 0x01]
    with pytest.raises(ValueError):
        oa.e4m3fn_quantize([float("nan")])


def test_matches_torch_conversion_in_range():
    rng = np.random.default_rng(11)
    v = np.concatenate([
        rng.normal(size=20000) * 40,
        rng.normal(size=20000) * 0.01,
        rng.uniform(-448, 448, size=20000),
        # every bf16 value in [-448, 448]: exact ties included
        _all_bf16_in_range(),
    ]).astype(np.float32)
    v = v[np.abs(v) <= 448]
    ref = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = oa.e4m3fn_quantize(v)
    bad = np.nonzero(got != ref)[0]
    assert bad.size == 0, (v[bad[:5]], got[bad[:5]], ref[bad[:5]])


def _all_bf16_in_range():
    bits = np.arange(0, 1 << 16, dtype=np.uint32)
    vals = (bits << 16).astype(np.uint32).view(np.float32)
    return vals[np.isfinite(vals) & (np.abs(vals) <= 448)]


def test_quantize_bf16_divides_in_float32():
    # x / s rounds in float32 before the FP8 decision: 3 / 7 * 7 is not 3 in float32,
    # and the quotient is what gets quantised
    x = _bf16_bits([3.0, -1.5, 100.0, 0.0])
    s = np.float32(0.0375)
    want = oa.e4m3fn_quantize(np.array([3.0, -1.5, 100.0, 0.0], np.float32) / s)
    assert oa.quantize_bf16(x, s).tolist() == want.tolist()
    # s = 1: the codes of values that are exactly representable are those values' codes
    vals = np.array([e4m3fn_value(c) for c in FINITE_CODES], dtype=np.float32)
    assert oa.quantize_bf16(_bf16_bits(vals), 1.0).tolist() == FINITE_CODES


def test_dynamic_scale_closed_forms():
    assert oa.dynamic_scale(_bf16_bits([0.0, -3.5, 2.0])) == np.float32(3.5 / 448)
    assert oa.dynamic_scale(_bf16_bits([0.0, -0.0])) == np.float32(1.0)
    assert oa.dynamic_scale(np.zeros(0, np.uint16)) == np.float32(1.0)
    assert oa.dynamic_scale(_bf16_bits([448.0, 1.0])) == np.float32(1.0)
    rng = np.random.default_rng(5)
    x = rng.normal(size=(33, 576)) * 0.5
    bits = _bf16_bits(x)
    amax = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).float().abs().max().item()
    assert oa.dynamic_scale(bits) == np.float32(np.float64(amax) / 448.0)
    # the scale maps the largest magnitude onto 448 (or just below, by rounding)
    s = oa.dynamic_scale(bits)
    assert abs(np.float32(amax) / s - 448) <= 448 * 2 ** -23 * 2


def test_append_hand_placed_slots():
    # two sequences: L = 20 and L = 3 with Q = 3 -> positions 17..19 and 0..2
    nb = 5
    cache = np.zeros((nb, 16, 576), np.uint16)
    pt = np.array([[3, 1], [4, -1]], np.int32)
    new = np.zeros((2, 3, 576), np.uint16)
    for b in range(2):
        for j in range(3):
            new[b, j] = _bf16_bits(np.full(576, 10 * b + j + 1.0))
    out = oa.kv_append(cache, pt, np.array([20, 3], np.int32), new, "bf16")
    # sequence 0: positions 17, 18, 19 -> page 1 -> block 1, rows 1, 2, 3
    for j, row in enumerate((1, 2, 3)):
        assert (out[1, row] == new[0, j]).all()
    # sequence 1: positions 0, 1, 2 -> page 0 -> block 4, rows 0, 1, 2
    for j in range(3):
        assert (out[4, j] == new[1, j]).all()
    changed = np.argwhere((out != cache).any(axis=2))
    assert sorted(map(tuple, changed.tolist())) == [(1, 1), (1, 2), (1, 3), (4, 0), (4, 1), (4, 2)]


def test_append_fp8_matches_slotwise_definition():
    rng = np.random.default_rng(8)
    nb, B, Q = 9, 3, 2
    cache = rng.integers(0, 0x7E, size=(nb, 16, 576), dtype=np.uint8)
    pt = np.array([[5, 2, 7], [0, -1, -1], [8, 1, -1]], np.int32)
    lens = np.array([48, 2, 17], np.int32)
    new = _bf16_bits(rng.normal(size=(B, Q, 576)) * 0.3)
    s = np.float32(0.3 * 4 / 448)
    out = oa.kv_append(cache, pt, lens, new, "fp8", s)
    expect = cache.copy()
    for b in range(B):
        for j in range(Q):
            t = int(lens[b]) - Q + j
            blk = pt[b, t // 16]
            x = torch.from_numpy(new[b, j].view(np.int16)).view(torch.bfloat16).float().numpy()
            expect[blk, t % 16] = torch.from_numpy((x / s).clip(-448, 448)).to(
                torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert (out == expect).all()
