"""CPU model of how the FP8 split kernel carries softmax probabilities into the
FP8 PV product, checked against float64 attention (no GPU).

The FP8 kernel feeds the stored E4M3 latents to the FP8 matrix cores as they
are, so the probabilities of the PV product must be FP8 too; each is carried
as two E4M3 terms, p ~ hi + lo with lo the E4M3 rounding of the residual of
hi.  E4M3 spans only about 18 binades (smallest subnormal 2^-9, largest
finite 448), while a softmax over tens of thousands of positions can hold
most of its mass in positions far below its maximum: a flat body of n
positions d nats below one dominant key holds n e^-d of the mass, which for
n = 35,500 and d = 10 is 1.6 times the key's own.  FP32 accumulation after
the product cannot restore inputs that were already rounded away ("Inside
Kimi K3 optimization", technical note "KDA precision & on-chip memory").

Two representations are modelled, with torch's round-to-nearest-even
float8_e4m3fn conversion standing in for the hardware conversion:

* relative to the row's running reference maximum (values p * 2^4 <= 256):
  every p below about 2^-14 of the reference is lost from the numerator,
  while the row sum keeps it in fp32;
* per 32-position block of a row: the block's own maximum bm (log2 units)
  gives the integer f = floor(bm), the block is stored as x = 2^(s - f + 7)
  in [0, 256) with the largest x in [128, 256), and the E8M0 block scale
  2^(f - 7 - m) of the product restores the magnitude against the row's
  integer reference m; the row sum adds the fp32 values.  Per value
  |x - (hi + lo)| <= max(2^-8 x, 2^-10), so a block's total weight is off by
  at most 2^-8 of its mass plus 32 * 2^-10 <= 2^-12 of its largest value:
  a relative bound of 2^-8 + 2^-12 on the whole weight vector, whatever the
  spread of the scores, and |dout| <= (2^-8 + 2^-12) max|v|.  A row sum of
  the stored terms would carry their 2^-8 error into lse, up to 4e-3 nats
  in a row dominated by one position; the fp32 sum keeps lse exact to fp32.

The tests show the first representation missing the output tolerance on
such inputs and the second staying inside the bound.
"""

import numpy as np
import torch

OUT_REL_TOL = 1e-2
LOG2E = 1.4426950408889634


def _e4m3(x):
    """Round float32 values to E4M3FN (RNE) and return them as float64."""
    return torch.from_numpy(np.asarray(x, dtype=np.float32)).to(torch.float8_e4m3fn) \
        .to(torch.float64).numpy()


def _two_terms(x):
    x = np.asarray(x, dtype=np.float32)
    hi = _e4m3(x)
    lo = _e4m3((x.astype(np.float64) - hi).astype(np.float32))
    return hi, lo


def _exact(s_nat, v):
    w = np.exp(s_nat - s_nat.max())
    return (w[:, None] * v).sum(0) / w.sum(), w


def model_reference_max(s_nat, v, tile=64, slack=4.0, shift=4.0):
    """Probabilities p * 2^shift against a lazily moved per-row reference
    maximum, two E4M3 terms in the numerator, fp32 p in the row sum."""
    s = s_nat * LOG2E
    m = -np.inf
    num = np.zeros(v.shape[1])
    den = 0.0
    for t0 in range(0, len(s), tile):
        st = s[t0:t0 + tile]
        mt = st.max()
        if mt > m + slack:
            if np.isfinite(m):
                a = 2.0 ** (m - mt)
                num *= a
                den *= a
            m = mt
        x = np.exp2(st - m + shift).astype(np.float32)
        hi, lo = _two_terms(x)
        num += ((hi + lo)[:, None] * v[t0:t0 + tile]).sum(0)
        den += float(x.astype(np.float64).sum())
    return num / den


def model_block_scale(s_nat, v, tile=64, block=32, slack=16):
    """Per-(row, 32-position block) E8M0 scale: each block stored against its
    own maximum, integer reference maximum, row sum from the same terms."""
    s = s_nat * LOG2E
    m = None
    num = np.zeros(v.shape[1])
    den = 0.0
    weights = np.zeros(len(s))
    for t0 in range(0, len(s), tile):
        st = s[t0:t0 + tile]
        blocks = [(b0, st[b0:b0 + block]) for b0 in range(0, len(st), block)]
        fb = [int(np.floor(np.float32(bs.max()))) for _, bs in blocks]
        mt = max(fb)
        if m is None or mt > m + slack:
            if m is not None:
                num *= 2.0 ** (m - mt)
                den *= 2.0 ** (m - mt)
            m = mt
        for (b0, bs), f in zip(blocks, fb):
            x = np.exp2(np.float32(bs) - np.float32(f) + np.float32(7.0)).astype(np.float32)
            assert x.max() < 256.0 and x.max() >= 128.0
            hi, lo = _two_terms(x)
            code = max(0, 120 + f - m)           # E8M0 exponent code of the block
            w = (hi + lo) * 2.0 ** (code - 127)
            weights[t0 + b0:t0 + b0 + len(bs)] = w * 2.0 ** m
            num += (w[:, None] * v[t0 + b0:t0 + b0 + len(bs)]).sum(0)
            # the row sum takes the fp32 values (lse stays exact to fp32)
            den += float(np.float32(x.sum(dtype=np.float32))) * 2.0 ** (code - 127)
    lse = (m + np.log2(den)) / LOG2E
    return num / den, weights, lse


def _dominant_key_case(n, gap_nat, body_std, tied, key_pos, seed):
    rng = np.random.default_rng(seed)
    s = rng.normal(0.0, body_std, size=n) if not tied else np.zeros(n)
    s[key_pos] = gap_nat
    v = rng.normal(0.3, 0.5, size=(n, 64))
    return s, v


CASES = [
    # (positions, gap in nats, body std, tied body, key position)
    (35500, 10.0, 0.3, False, 5),
    (35500, 10.0, 0.3, False, 35000),
    (35500, 14.0, 0.0, True, 5),
    (4438, 9.0, 0.3, False, 100),
    (2048, 8.0, 0.5, False, 3),
    (65536, 12.0, 1.0, False, 40000),
]


def test_reference_max_representation_misses_the_tolerance():
    """The representation against the row's reference maximum drops the
    body's mass from the numerator: far outside the tolerance."""
    worst = 0.0
    for i, (n, gap, std, tied, kp) in enumerate(CASES[:3]):
        s, v = _dominant_key_case(n, gap, std, tied, kp, seed=i)
        ref, _ = _exact(s, v)
        got = model_reference_max(s, v)
        worst = max(worst, np.abs(got - ref).max() / np.abs(ref).max())
    assert worst > 5 * OUT_REL_TOL, worst


def test_block_scale_representation_within_bound():
    """Per-block E8M0 scales: the total weight perturbation stays within
    2^-8 + 2^-12 of the mass, the output within that bound times max|v|
    (and the tolerance), lse within fp32 rounding."""
    bound = 2.0 ** -8 + 2.0 ** -12
    for i, (n, gap, std, tied, kp) in enumerate(CASES):
        s, v = _dominant_key_case(n, gap, std, tied, kp, seed=i)
        ref, _ = _exact(s, v)
        got, wq, lse = model_block_scale(s, v)
        lse_ref = s.max() + np.log(np.exp(s - s.max()).sum())
        assert abs(lse - lse_ref) <= 1e-5, (CASES[i], lse - lse_ref)
        # the model's weights stand for e^s (the block scale restores the
        # magnitude): their total perturbation against the exact weights
        w = np.exp(s)
        rel = np.abs(wq - w).sum() / w.sum()
        assert rel <= bound, (CASES[i], rel)
        err = np.abs(got - ref).max()
        assert err <= bound * np.abs(v).max(), (CASES[i], err)
        assert err / np.abs(ref).max() <= OUT_REL_TOL / 4, (CASES[i], err)


def test_block_scale_per_value_bound():
    """|x - (hi + lo)| <= max(2^-8 x, 2^-10) for x in [0, 256), the bound the
    block-scale argument rests on (swept over 2^-40 .. 256)."""
    x = np.float32(2.0) ** np.linspace(-40.0, 8.0, 200001, dtype=np.float32)
    x = x[x < 256.0]
    hi, lo = _two_terms(x)
    err = np.abs(x.astype(np.float64) - (hi + lo))
    assert (err <= np.maximum(2.0 ** -8 * x, 2.0 ** -10)).all()
