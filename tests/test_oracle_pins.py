"""Pins of the float64 oracle against facts other than itself (CPU only).

Each ``pin_*`` function raises AssertionError when the oracle disagrees with
the fact it pins; the tests call them directly, and ``test_planted_mistakes``
re-runs them against deliberately broken copies of the oracle (on the CPU) to
show that every plausible slip -- a dropped term, a wrong sign or index, a
transposed operand -- fails at least one pin.

Facts used:
* the OCP FP8 E4M3FN definition (special values) and torch's float8_e4m3fn
  and bfloat16 decoders (library routines);
* a pure-Python brute force (oracle.brute) written with its own decoding,
  gather and loops;
* torch.nn.functional.scaled_dot_product_attention in float64 (library
  routine) with torch.logsumexp;
* closed forms: one visible position returns its value vector; tied scores
  or q = 0 return the mean value vector with lse = s + ln n; a dominant key
  returns its value; verify with seq_len = Q lets token 0 see only
  position 0;
* invariants the pages state: partials with normalisers merge to the
  unsplit answer; padding heads with zero queries leaves the real heads
  unchanged; the page table only addresses storage.
"""

import math

import numpy as np
import pytest
import torch

import oracle
import oracle.mla as om
from workloads import make_inputs, compact_for_oracle, SOFTMAX_SCALE

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")


def _tiny(seq_lens, num_q, heads, kv_dtype, seed, **kw):
    inp = make_inputs(seq_lens, num_q, heads, kv_dtype, seed, device="cpu", **kw)
    return inp, compact_for_oracle(inp)


def _ref(d, **kw):
    return oracle.mla_reference(d["q_bits"], d["kv_raw"], d["page_table"], d["seq_lens"],
                                d["softmax_scale"], d["kv_dtype"], d["kv_scale"], **kw)


# --------------------------------------------------------------------------- formats

def pin_e4m3fn_special_values():
    t = oracle.e4m3fn_table()
    expect = {0x00: 0.0, 0x01: 2.0 ** -9, 0x07: 7 * 2.0 ** -9, 0x08: 2.0 ** -6, 0x38: 1.0,
              0x39: 1.125, 0x40: 2.0, 0x7E: 448.0, 0xFE: -448.0, 0xB8: -1.0, 0x81: -(2.0 ** -9),
              0x77: 240.0, 0x30: 0.5}
    for code, v in expect.items():
        assert t[code] == v, (hex(code), t[code], v)
    assert math.copysign(1.0, t[0x80]) == -1.0 and t[0x80] == 0.0
    assert np.isnan(t[0x7F]) and np.isnan(t[0xFF])
    assert np.isnan(t).sum() == 2


def pin_e4m3fn_vs_torch():
    t = oracle.e4m3fn_table()
    ref = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    assert np.array_equal(np.isnan(t), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(t[ok], ref[ok])


def pin_bf16_vs_torch():
    rng = np.random.default_rng(0)
    bits = rng.integers(0, 1 << 16, size=20000, dtype=np.uint32).astype(np.uint16)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    got = oracle.bf16_bits_to_f64(bits)
    ok = ~np.isnan(ref)
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    assert np.array_equal(got[ok], ref[ok])


def test_e4m3fn_special_values():
    pin_e4m3fn_special_values()


def test_e4m3fn_vs_torch():
    pin_e4m3fn_vs_torch()


def test_bf16_vs_torch():
    pin_bf16_vs_torch()


# --------------------------------------------------------------------------- brute force

BRUTE_CASES = [
    # (seq_lens, Q, H, kv_dtype, seed)
    ([1, 17], 1, 4, "bf16", 11),
    ([23, 40], 3, 3, "bf16", 12),
    ([5, 33], 2, 2, "fp8", 13),
    ([3, 16], 3, 4, "fp8", 14),
]


def pin_brute(case):
    lens, nq, nh, dt, seed = case
    _, d = _tiny(lens, nq, nh, dt, seed)
    out, lse = _ref(d)
    bo, bl = oracle.brute_force_mla(d["q_bits"].tolist(), d["kv_raw"].tolist(),
                                    d["page_table"].tolist(), d["seq_lens"].tolist(),
                                    d["softmax_scale"], dt, d["kv_scale"])
    bo, bl = np.array(bo), np.array(bl)
    np.testing.assert_allclose(lse, bl, rtol=1e-12, atol=0)
    np.testing.assert_allclose(out, bo, rtol=1e-10, atol=1e-13 * np.abs(bo).max())


@pytest.mark.parametrize("case", BRUTE_CASES)
def test_brute_force(case):
    pin_brute(case)


# --------------------------------------------------------------------------- library routine

def pin_sdpa(kv_dtype, seed):
    lens, nq, nh = [37, 70, 129], 3, 5
    _, d = _tiny(lens, nq, nh, kv_dtype, seed)
    out, lse = _ref(d)
    q = torch.from_numpy(oracle.bf16_bits_to_f64(d["q_bits"]))
    for b, L in enumerate(d["seq_lens"]):
        x = torch.from_numpy(om.gather_sequence(d["kv_raw"], d["page_table"][b], L, kv_dtype,
                                                d["kv_scale"]))
        k = x[None, None].expand(1, nh, -1, -1)                    # [1, H, L, 576]
        v = x[:, :512][None, None].expand(1, nh, -1, -1)
        qq = q[b].permute(1, 0, 2)[None]                           # [1, H, Q, 576]
        mask = torch.arange(L)[None, :] <= (L - nq + torch.arange(nq))[:, None]   # [Q, L]
        o = torch.nn.functional.scaled_dot_product_attention(
            qq, k, v, attn_mask=mask, scale=float(d["softmax_scale"]))
        sc = float(d["softmax_scale"]) * (qq @ k.transpose(-1, -2))
        ls = torch.logsumexp(sc.masked_fill(~mask, -math.inf), dim=-1)   # [1, H, Q]
        np.testing.assert_allclose(out[b], o[0].permute(1, 0, 2).numpy(), rtol=1e-9,
                                   atol=1e-12)
        np.testing.assert_allclose(lse[b], ls[0].T.numpy(), rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("kv_dtype,seed", [("bf16", 21), ("fp8", 22)])
def test_sdpa_float64(kv_dtype, seed):
    pin_sdpa(kv_dtype, seed)


# --------------------------------------------------------------------------- closed forms

def pin_single_position():
    """One visible position: out = its value vector exactly, lse = its score."""
    inp, d = _tiny([1, 1], 1, 6, "bf16", 31)
    out, lse = _ref(d)
    q = oracle.bf16_bits_to_f64(d["q_bits"])
    for b in range(2):
        x = oracle.bf16_bits_to_f64(d["kv_raw"][d["page_table"][b, 0], 0])
        assert np.array_equal(out[b, 0], np.broadcast_to(x[:512], out[b, 0].shape))
        s0 = [float(d["softmax_scale"]) * math.fsum(q[b, 0, h] * x) for h in range(6)]
        np.testing.assert_allclose(lse[b, 0], s0, rtol=1e-14, atol=1e-14)


def pin_q_zero():
    """q = 0: every score is 0, out = mean of value vectors, lse = ln n."""
    inp, d = _tiny([45, 19], 1, 2, "fp8", 32)
    d["q_bits"] = np.zeros_like(d["q_bits"])
    out, lse = _ref(d)
    for b, L in enumerate(d["seq_lens"]):
        x = om.gather_sequence(d["kv_raw"], d["page_table"][b], L, "fp8", d["kv_scale"])
        np.testing.assert_allclose(out[b, 0], np.broadcast_to(x[:, :512].mean(0), (2, 512)),
                                   rtol=1e-12, atol=1e-15)
        np.testing.assert_allclose(lse[b, 0], math.log(L), rtol=1e-14)


def pin_tied_scores():
    """q zero on the 512 latent dims and every position sharing the same 64 rope
    dims: all scores equal s, so out = mean of the (different) value vectors and
    lse = s + ln n."""
    inp, d = _tiny([50], 1, 3, "bf16", 33)
    kv = d["kv_raw"].copy()
    kv[:, :, 512:] = kv[0, 0, 512:]
    qb = d["q_bits"].copy()
    qb[..., :512] = 0
    d.update(kv_raw=kv, q_bits=qb)
    out, lse = _ref(d)
    x = om.gather_sequence(kv, d["page_table"][0], 50, "bf16")
    q = oracle.bf16_bits_to_f64(qb)[0, 0]
    for h in range(3):
        s = float(d["softmax_scale"]) * math.fsum(q[h] * x[0])
        np.testing.assert_allclose(lse[0, 0, h], s + math.log(50), rtol=1e-13)
        np.testing.assert_allclose(out[0, 0, h], x[:, :512].mean(0), rtol=1e-12, atol=1e-15)


def pin_dominant_key():
    """q = alpha * latent_0 with large alpha: out -> value_0, lse -> s_0."""
    inp, d = _tiny([30], 1, 1, "bf16", 34)
    x = om.gather_sequence(d["kv_raw"], d["page_table"][0], 30, "bf16")
    qf = (torch.from_numpy(x[0]).float() * 4.0).to(torch.bfloat16)
    d["q_bits"] = qf.view(torch.int16).numpy().view(np.uint16).reshape(1, 1, 1, 576)
    out, lse = _ref(d)
    q = oracle.bf16_bits_to_f64(d["q_bits"])[0, 0, 0]
    s = float(d["softmax_scale"]) * (x @ q)
    gap = s[0] - np.max(s[1:])
    assert gap > 20
    bound = 30 * math.exp(-gap) * (1 + np.abs(x).max())
    assert np.abs(out[0, 0, 0] - x[0, :512]).max() <= bound
    assert abs(lse[0, 0, 0] - s[0]) <= 30 * math.exp(-gap)


def pin_verify_seq_eq_q():
    """seq_len = Q: token j sees exactly j + 1 positions; token 0 returns value_0."""
    inp, d = _tiny([3, 3], 3, 4, "fp8", 35)
    out, lse = _ref(d)
    for b in range(2):
        x = om.gather_sequence(d["kv_raw"], d["page_table"][b], 3, "fp8", d["kv_scale"])
        assert np.array_equal(out[b, 0], np.broadcast_to(x[0, :512], (4, 512)))
        q = oracle.bf16_bits_to_f64(d["q_bits"])[b]
        for j in range(3):
            s = float(d["softmax_scale"]) * (x[: j + 1] @ q[j].T)      # [j+1, H]
            m = s.max(0)
            np.testing.assert_allclose(lse[b, j], m + np.log(np.exp(s - m).sum(0)), rtol=1e-13)


def test_single_position():
    pin_single_position()


def test_q_zero():
    pin_q_zero()


def test_tied_scores():
    pin_tied_scores()


def test_dominant_key():
    pin_dominant_key()


def test_verify_seq_eq_q():
    pin_verify_seq_eq_q()


def test_seq_shorter_than_q_rejected():
    """seq_len < Q is outside the causal rule (the Q new tokens belong to the
    sequence): the oracle refuses it instead of wrapping a negative count."""
    assert om._visible(8, 8, 0) == 1
    with pytest.raises(ValueError):
        om._visible(5, 8, 0)
    with pytest.raises(ValueError):
        om._visible(7, 8, 7)


# --------------------------------------------------------------------------- invariants

def _ranges_equal(L, s):
    cuts = np.linspace(0, L, s + 1).astype(int)
    return [(int(cuts[i]), int(cuts[i + 1])) for i in range(s)]


def pin_split_merge():
    """Partials carrying their normalisers merge to the unsplit answer, for even,
    uneven and empty splits; merging one partial is the identity."""
    lens = [97, 300, 4]
    inp, d = _tiny(lens, 3, 2, "bf16", 41)
    out, lse = _ref(d)
    for s in (1, 2, 3, 8, 16):
        ranges = [_ranges_equal(L, s) for L in lens]
        po, pl = oracle.mla_partials(d["q_bits"], d["kv_raw"], d["page_table"], d["seq_lens"],
                                     d["softmax_scale"], ranges, "bf16")
        mo, ml = oracle.merge(po, pl)
        np.testing.assert_allclose(mo, out, rtol=1e-11, atol=1e-14)
        np.testing.assert_allclose(ml, lse, rtol=1e-13)
        if s == 1:
            assert np.array_equal(mo, po[0]) and np.array_equal(ml, pl[0])
    uneven = [[(0, 0), (0, 5), (5, 5), (5, 60), (60, L), (L, L)] for L in lens]
    uneven[2] = [(0, 0), (0, 1), (1, 1), (1, 3), (3, 4), (4, 4)]
    po, pl = oracle.mla_partials(d["q_bits"], d["kv_raw"], d["page_table"], d["seq_lens"],
                                 d["softmax_scale"], uneven, "bf16")
    assert np.isneginf(pl[0]).all() and (po[0] == 0).all()
    mo, ml = oracle.merge(po, pl)
    np.testing.assert_allclose(mo, out, rtol=1e-11, atol=1e-14)
    np.testing.assert_allclose(ml, lse, rtol=1e-13)
    eo, el = oracle.merge(np.zeros((3, 2, 512)), np.full((3, 2), -np.inf))
    assert (eo == 0).all() and np.isneginf(el).all()


def pin_head_padding():
    """12 real heads vs the same 12 plus 4 zero-query heads: real rows identical."""
    inp, d = _tiny([40, 77], 3, 12, "fp8", 42)
    out, lse = _ref(d)
    q16 = np.zeros(d["q_bits"].shape[:2] + (16, 576), dtype=np.uint16)
    q16[:, :, :12] = d["q_bits"]
    o16, l16 = oracle.mla_reference(q16, d["kv_raw"], d["page_table"], d["seq_lens"],
                                    d["softmax_scale"], "fp8", d["kv_scale"])
    # BLAS may block a 16-row product differently from a 12-row one: equal to rounding.
    np.testing.assert_allclose(o16[:, :, :12], out, rtol=1e-13, atol=1e-16)
    np.testing.assert_allclose(l16[:, :, :12], lse, rtol=1e-14)


def pin_page_table_is_storage_only():
    """The same latents stored at permuted pool blocks, with spare poisoned
    blocks and poisoned tail slots, give the same answer as an identity table."""
    lens = [33, 64, 7]
    a, da = _tiny(lens, 2, 3, "bf16", 43, identity_pages=True)
    oa, la = _ref(da)
    nb = da["kv_raw"].shape[0]
    perm = np.random.default_rng(5).permutation(nb + 3)     # 3 spare blocks
    pool = np.full((nb + 3, 16, 576), 0x7FC0, dtype=np.uint16)  # bf16 NaN everywhere
    pool[perm[:nb]] = da["kv_raw"]
    pt = np.where(da["page_table"] >= 0, perm[np.maximum(da["page_table"], 0)], -1)
    for b, L in enumerate(lens):                            # poison slots past L
        p = -(-L // 16)
        pool[pt[b, p - 1], L - (p - 1) * 16:] = 0x7FC0
    db = dict(da, kv_raw=pool, page_table=pt)
    ob, lb = _ref(db)
    np.testing.assert_array_equal(oa, ob)
    np.testing.assert_array_equal(la, lb)
    assert np.isfinite(ob).all()


def pin_causal_against_truncation():
    """Verify token j equals a Q = 1 decode over the first L - Q + j + 1 positions
    (speculative decoding is lossless: verifying Q tokens equals Q decodes)."""
    lens = [29, 64]
    inp, d = _tiny(lens, 3, 2, "fp8", 44)
    out, lse = _ref(d)
    for j in range(3):
        dj = dict(d)
        dj["q_bits"] = d["q_bits"][:, j:j + 1]
        dj["seq_lens"] = np.array([L - 3 + j + 1 for L in lens])
        oj, lj = _ref(dj)
        np.testing.assert_allclose(oj[:, 0], out[:, j], rtol=1e-13, atol=1e-16)
        np.testing.assert_allclose(lj[:, 0], lse[:, j], rtol=1e-14)


def test_split_merge():
    pin_split_merge()


def test_head_padding():
    pin_head_padding()


def test_page_table_is_storage_only():
    pin_page_table_is_storage_only()


def test_causal_against_truncation():
    pin_causal_against_truncation()


# --------------------------------------------------------------------------- planted mistakes

ALL_PINS = [
    pin_e4m3fn_special_values, pin_e4m3fn_vs_torch, pin_bf16_vs_torch,
    lambda: [pin_brute(c) for c in BRUTE_CASES],
    lambda: (pin_sdpa("bf16", 21), pin_sdpa("fp8", 22)),
    pin_single_position, pin_q_zero, pin_tied_scores, pin_dominant_key, pin_verify_seq_eq_q,
    pin_split_merge, pin_head_padding, pin_page_table_is_storage_only,
]


def _attend_v_tail(q_rows, latents, softmax_scale):          # value = last 512 dims
    o, lse = _ORIG_ATTEND(q_rows, latents, softmax_scale)
    if latents.shape[0]:
        s = softmax_scale * (q_rows @ latents.T)
        o = np.exp(s - lse[:, None]) @ latents[:, 64:]
    return o, lse


def _attend_no_scale(q_rows, latents, softmax_scale):        # dropped softmax scale
    return _ORIG_ATTEND(q_rows, latents, 1.0)


def _attend_lse_log2(q_rows, latents, softmax_scale):        # lse in base 2
    o, lse = _ORIG_ATTEND(q_rows, latents, softmax_scale)
    return o, lse / math.log(2.0)


def _attend_no_max_sub(q_rows, latents, softmax_scale):      # lse missing the max term
    o, lse = _ORIG_ATTEND(q_rows, latents, softmax_scale)
    if latents.shape[0]:
        s = softmax_scale * (q_rows @ latents.T)
        lse = lse - s.max(axis=1)
    return o, lse


def _attend_transposed(q_rows, latents, softmax_scale):      # scores summed over the wrong axis
    if latents.shape[0] == 0:
        return _ORIG_ATTEND(q_rows, latents, softmax_scale)
    s = softmax_scale * (q_rows @ latents.T)
    m = s.max(axis=0, keepdims=True)
    p = np.exp(s - m) / np.exp(s - m).sum(axis=0, keepdims=True)
    lse = (m[0] + np.log(np.exp(s - m).sum(axis=0)))[: q_rows.shape[0]]
    if lse.shape[0] < q_rows.shape[0]:
        lse = np.resize(lse, q_rows.shape[0])
    return p @ latents[:, :512], lse


def _visible_off_by_one(seq_len, num_q, j):
    return int(seq_len) - int(num_q) + int(j)


def _visible_reversed(seq_len, num_q, j):
    return int(seq_len) - int(j)


def _merge_wrong_sign(part_out, part_lse):
    o, lse = _ORIG_MERGE(part_out, -np.asarray(part_lse))
    return o, -lse


def _decode_kv_no_scale(raw, kv_dtype, kv_scale=1.0):
    return _ORIG_DECODE(raw, kv_dtype, 1.0)


def _decode_kv_fp8_bias8(raw, kv_dtype, kv_scale=1.0):     # E4M3 exponent bias 8, not 7
    x = _ORIG_DECODE(raw, kv_dtype, kv_scale)
    return x * 0.5 if kv_dtype == "fp8" else x


def _partials_inclusive_end(q_bits, kv_raw, page_table, seq_lens, softmax_scale, ranges,
                            kv_dtype="bf16", kv_scale=1.0, batch_indices=None):
    # each split also takes the first position of the next: [lo, hi]
    wide = [[(lo, hi + 1) for lo, hi in r] for r in ranges]
    return _ORIG_PARTIALS(q_bits, kv_raw, page_table, seq_lens, softmax_scale, wide, kv_dtype,
                          kv_scale, batch_indices)


def _gather_slot_swap(kv_raw, page_table_row, seq_len, kv_dtype, kv_scale=1.0):
    n_pages = -(-int(seq_len) // 16)
    if n_pages == 0:
        return _ORIG_GATHER(kv_raw, page_table_row, seq_len, kv_dtype, kv_scale)
    blocks = np.asarray(page_table_row[:n_pages], dtype=np.int64)
    raw = np.asarray(kv_raw)[blocks][:, ::-1]              # slots reversed inside each page
    x = om.decode_kv(raw, kv_dtype, kv_scale).reshape(n_pages * 16, 576)
    return x[: int(seq_len)]


_ORIG_ATTEND = om.attend
_ORIG_MERGE = om.merge
_ORIG_DECODE = om.decode_kv
_ORIG_GATHER = om.gather_sequence
_ORIG_PARTIALS = om.mla_partials

MUTANTS = [
    ("attend", _attend_v_tail), ("attend", _attend_no_scale), ("attend", _attend_lse_log2),
    ("attend", _attend_no_max_sub), ("attend", _attend_transposed),
    ("_visible", _visible_off_by_one), ("_visible", _visible_reversed),
    ("merge", _merge_wrong_sign), ("decode_kv", _decode_kv_no_scale),
    ("decode_kv", _decode_kv_fp8_bias8), ("gather_sequence", _gather_slot_swap),
    ("mla_partials", _partials_inclusive_end),
]


@pytest.mark.parametrize("name,fn", MUTANTS, ids=[f.__name__ for _, f in MUTANTS])
def test_planted_mistakes(monkeypatch, name, fn):
    """Each planted slip in a copy of the oracle is caught by at least one pin."""
    monkeypatch.setattr(om, name, fn)
    if name in ("merge", "attend", "gather_sequence", "mla_partials"):
        monkeypatch.setattr(oracle, name, fn)
    caught = 0
    for pin in ALL_PINS:
        try:
            pin()
        except (AssertionError, ValueError, IndexError):
            caught += 1
            break
    assert caught, f"no pin caught the planted mistake {fn.__name__}"
