"""GPU parity: the HIP path (through the C ABI) against the float64 oracle on the
same seeded inputs, at the tolerance stated in parity_util.

Small cases span several 64-position tiles with ragged tails, empty splits,
1-3 query tokens, bf16 and FP8 KV, padded and unpadded head counts; the
named workloads run at their full sizes in the launch configuration the
bench uses, with the oracle evaluated on all sequences or a seeded sample.
"""

import numpy as np
import pytest
import torch

import oracle
import workloads
from workloads import make_inputs, make_config, make_c5_layer
from parity_util import (compare, oracle_out, oracle_partials, run_verify, split_page_ranges)

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)


SMALL_CASES = [
    # (seq_lens, Q, H, kv_dtype, num_splits)
    ([256], 1, 12, "bf16", 1),
    ([1, 15, 16, 17, 64, 65, 200], 1, 12, "bf16", 0),
    ([3, 63, 64, 65, 129, 300], 3, 12, "bf16", 0),
    ([3, 63, 64, 65, 129, 300], 3, 12, "fp8", 0),
    ([100, 1000], 2, 12, "fp8", 3),
    ([517, 33], 3, 16, "bf16", 7),
    ([517, 33], 1, 5, "fp8", 2),
    ([2000], 3, 12, "fp8", 16),
    ([4, 5, 6], 3, 12, "bf16", 1),
    ([777], 2, 1, "bf16", 5),
]


@pytest.mark.parametrize("case", SMALL_CASES, ids=[f"{c[3]}-Q{c[1]}-H{c[2]}-S{c[4]}-{len(c[0])}seq"
                                                    for c in SMALL_CASES])
def test_small_cases(gpu_lib, case):
    lens, nq, nh, dt, S = case
    _say(f"small case {case}")
    inp = make_inputs(lens, nq, nh, dt, seed=sum(lens) + nq, device="cuda", spare_blocks=2,
                      poison=True)
    out, lse = run_verify(gpu_lib, inp, num_splits=S)
    ro, rl, _ = oracle_out(inp)
    compare(out, lse, ro, rl, str(case))


# Query rows beyond one block: row blocks of 64 (FP8, more than 32 rows), 48
# or 16 (generic kernel), including a partial last block and single-split
# (direct bf16 output) launches over several row blocks.
WIDE_CASES = [
    # (seq_lens, Q, H, kv_dtype, num_splits)
    ([300, 1500], 3, 96, "fp8", 0),
    ([300, 1500], 3, 96, "bf16", 0),
    ([65, 700], 8, 12, "fp8", 3),
    ([65, 700], 8, 12, "bf16", 3),
    ([129, 40], 5, 16, "fp8", 2),
    ([257], 1, 128, "bf16", 1),
    ([257], 1, 128, "fp8", 2),
    ([100], 1, 20, "fp8", 0),
    ([8, 9], 8, 3, "bf16", 0),
    ([33], 7, 16, "fp8", 1),
    # split x sequence units a multiple of 8 with several row blocks: the row
    # blocks of a unit are placed on one XCD back to back
    ([300, 1500], 3, 96, "fp8", 4),
    ([300, 1500], 3, 96, "bf16", 4),
    ([257], 1, 128, "fp8", 8),
]


@pytest.mark.parametrize("case", WIDE_CASES, ids=[f"{c[3]}-Q{c[1]}-H{c[2]}-S{c[4]}-{len(c[0])}seq"
                                                   for c in WIDE_CASES])
def test_wide_row_blocks(gpu_lib, case):
    lens, nq, nh, dt, S = case
    _say(f"wide case {case}")
    inp = make_inputs(lens, nq, nh, dt, seed=7 * sum(lens) + nq + nh, device="cuda",
                      spare_blocks=2, poison=True)
    out, lse = run_verify(gpu_lib, inp, num_splits=S)
    ro, rl, _ = oracle_out(inp)
    compare(out, lse, ro, rl, str(case))


# FP8 blocks of 33..48 query rows: the eight-wave kernel's second wave group
# holds 1..16 real rows and the rest padding, at both ends of that range and
# with every causal token count.  These launch the packed kernel (the group's
# two FP8 terms in one 32-row operand, its copies issued by its two waves
# without softmax rows); 49 rows is the first count past it (unpacked, a
# second row block holding one row).
PARTIAL_GROUP_CASES = [
    # (seq_lens, Q, H, kv_dtype, num_splits)
    ([3, 63, 64, 65, 129, 300], 3, 16, "fp8", 0),   # 48 rows
    ([700, 17], 3, 11, "fp8", 3),                   # 33 rows
    ([2000, 8], 8, 5, "fp8", 0),                    # 40 rows, eight causal tokens (the
                                                    # first sees one position)
    ([4, 16, 100], 4, 12, "fp8", 1),                # 48 rows, direct bf16 output
    ([1300, 250], 1, 48, "fp8", 5),                 # 48 rows of one token
    ([500, 1200], 7, 7, "fp8", 0),                  # 49 rows: unpacked
]


@pytest.mark.parametrize("case", PARTIAL_GROUP_CASES, ids=[f"{c[3]}-Q{c[1]}-H{c[2]}-S{c[4]}-{len(c[0])}seq"
                                                     for c in PARTIAL_GROUP_CASES])
def test_partial_second_group(gpu_lib, case):
    lens, nq, nh, dt, S = case
    _say(f"partial second group {case}")
    inp = make_inputs(lens, nq, nh, dt, seed=5 * sum(lens) + nq + nh, device="cuda",
                      spare_blocks=2, poison=True)
    out, lse = run_verify(gpu_lib, inp, num_splits=S)
    ro, rl, _ = oracle_out(inp)
    compare(out, lse, ro, rl, str(case))


def _random_cases(n, seed):
    # seeded shapes across the kernel choices: query rows Q*H on both sides of
    # 16, 32, 48 and 64 (layouts and row blocks), Q = 1..8, both KV types,
    # automatic and forced split counts, ragged lengths >= Q
    rng = np.random.default_rng(seed)
    heads = [1, 2, 3, 5, 6, 8, 11, 12, 16, 17, 20, 24, 32, 33, 48, 64, 96, 128]
    out = []
    for _ in range(n):
        nq = int(rng.integers(1, 9))
        nh = int(rng.choice(heads))
        nb = int(rng.integers(1, 4))
        lens = [int(x) for x in rng.integers(nq, 2200, size=nb)]
        dt = str(rng.choice(["bf16", "fp8"]))
        S = int(rng.choice([0, 0, 1, 2, 5, 16]))
        out.append((lens, nq, nh, dt, S))
    return out


RANDOM_CASES = _random_cases(24, 2024)


@pytest.mark.parametrize("case", RANDOM_CASES, ids=[f"{i}-{c[3]}-Q{c[1]}-H{c[2]}-S{c[4]}"
                                                    for i, c in enumerate(RANDOM_CASES)])
def test_random_shapes(gpu_lib, case):
    lens, nq, nh, dt, S = case
    _say(f"random case {case}")
    inp = make_inputs(lens, nq, nh, dt, seed=11 * sum(lens) + nq + nh, device="cuda",
                      spare_blocks=1, poison=True)
    out, lse = run_verify(gpu_lib, inp, num_splits=S)
    ro, rl, _ = oracle_out(inp)
    compare(out, lse, ro, rl, str(case))


@pytest.mark.parametrize("dt,nq,S", [("bf16", 1, 0), ("fp8", 3, 2)])
def test_max_batch_sampled(gpu_lib, dt, nq, S):
    """The largest batch the boundary accepts: 65,535 sequences of Q..40
    positions, so grid and row indexing run at their limits (with S = 2 the
    merge covers 2.4 M rows).  The oracle checks a seeded sample with both ends."""
    B = 65535
    _say(f"max batch {dt} Q={nq} S={S}")
    lens = np.random.default_rng(65535).integers(nq, 41, size=B)
    inp = make_inputs(lens, nq, 12, dt, seed=65535 + nq, device="cuda")
    out, lse = run_verify(gpu_lib, inp, num_splits=S)
    pick = np.random.default_rng(7).choice(B, size=7, replace=False).tolist()
    idx = sorted({0, 1, B // 2, B - 2, B - 1} | set(pick))
    ro, rl, _ = oracle_out(inp, idx)
    compare(out[idx], lse[idx], ro, rl, f"B={B} {dt} Q={nq} S={S}")


@pytest.mark.parametrize("dt", ["bf16", "fp8"])
def test_max_splits(gpu_lib, dt):
    """The largest split count (256): about one page per split of the long
    sequence, and almost every split of the short ones empty."""
    _say(f"max splits {dt}")
    inp = make_inputs([5000, 40, 3], 3, 12, dt, seed=256, device="cuda", spare_blocks=2,
                      poison=True)
    out, lse = run_verify(gpu_lib, inp, num_splits=256)
    ro, rl, _ = oracle_out(inp)
    compare(out, lse, ro, rl, f"S=256 {dt}")


@pytest.mark.parametrize("alpha", [0.02, 0.3, 4.0])
def test_fp8_growing_scores(gpu_lib, alpha):
    """Queries aligned with one late key, so the running maximum of those rows
    jumps far above the early tiles' (by a few units up to hundreds in log2
    units): the reference maximum moves, the probability scale follows it,
    and for the largest jumps the accumulators are rebased.  The lse bound is
    the absolute 1e-3 while |lse| stays in the workloads' range (ln n + 0.4);
    with alpha = 4 it reaches about 415, where the float32 score sums alone
    are good to about 1e-5 relative, so there the bound scales as
    1e-3 * max(1, |lse| / 100), the stated reading of the tolerance."""
    _say(f"growing scores alpha={alpha}")
    inp = make_inputs([1000, 3000], 3, 12, "fp8", seed=41, device="cuda")
    kv = inp.kv.view(torch.float8_e4m3fn).float() * inp.kv_scale
    q = inp.q.clone()
    pt = inp.page_table.cpu().numpy()
    for b, L in enumerate(inp.seq_lens.cpu().numpy().tolist()):
        t = L - 40                                  # a late position, visible to every token
        lat = kv[int(pt[b, t // 16]), t % 16]
        for j in range(3):
            for hh in range(0, 12, 3):              # every third head follows the key
                q[b, j, hh] = (alpha * (1 + hh) * lat).to(torch.bfloat16)
    inp.q = q
    ro, rl, _ = oracle_out(inp)
    lse_tol = 1e-3 * max(1.0, float(np.abs(rl).max()) / 100.0)
    for S in (0, 1, 3):
        out, lse = run_verify(gpu_lib, inp, num_splits=S)
        dout, dlse = compare(out, lse, ro, rl, f"alpha={alpha} S={S}", lse_tol=lse_tol)
        _say(f"  alpha={alpha} S={S}: max|lse| = {np.abs(rl).max():.1f}, bound {lse_tol:.2e}, "
             f"max|dout|/max|ref| = {dout:.3e}, max|dlse| = {dlse:.3e}")


def _dominant_key_inputs(lens, gap_nat, body_std, tied, key_pos, seed):
    """FP8 verify inputs whose scores (from the 64 rope dims only) put one key
    gap_nat nats above a body of near-equal scores (std body_std nats, or
    exactly tied), with value vectors of mean +0.3.  The body's total
    probability mass is then comparable to the key's, and far below it per
    position: the case where a probability format of narrow range loses mass.
    Head h scales the query, so the rows span 0.5x .. 1.5x the gap."""
    inp = make_inputs(lens, 3, 12, "fp8", seed=seed, device="cpu")
    g = torch.Generator().manual_seed(seed)
    nb = inp.kv.shape[0]
    lat = torch.randn((nb, 16, 576), generator=g) * 0.5
    lat[:, :, :512] += 0.3
    u = torch.ones(64) / 8.0                        # unit vector over the rope dims
    sc = float(inp.softmax_scale)
    beta = max(body_std, 0.3) / (sc * 0.5)          # body score std = body_std nats
    c = gap_nat / (sc * beta)                       # the key's rope part, along u
    pt = inp.page_table.numpy()
    for b, L in enumerate(lens):
        if tied:
            for p in range(-(-L // 16)):
                lat[int(pt[b, p]), :, 512:] = 0.02 * u
        t = key_pos if key_pos >= 0 else L + key_pos
        lat[int(pt[b, t // 16]), t % 16, 512:] = c * u
    amax = float(lat.abs().max())
    kv_scale = float(np.float32(amax / 448.0))
    inp.kv = (lat / kv_scale).clamp(-448.0, 448.0).to(torch.float8_e4m3fn).view(torch.uint8)
    inp.kv_scale = kv_scale
    q = torch.zeros((len(lens), 3, 12, 576))
    for hh in range(12):
        q[:, :, hh, 512:] = beta * (0.5 + hh / 11.0) * u
    inp.q = q.to(torch.bfloat16)
    return workloads.MLAInputs(q=inp.q.cuda(), kv=inp.kv.cuda(), page_table=inp.page_table.cuda(),
                               seq_lens=inp.seq_lens.cuda(), kv_dtype="fp8", kv_scale=kv_scale,
                               softmax_scale=inp.softmax_scale, meta={})


DOMINANT_KEY_CASES = [
    # (seq_lens, gap in nats, body std in nats, tied body, key position (<0: from the end))
    ([35500], 10.0, 0.3, False, 5),
    ([35500], 10.0, 0.3, False, -40),
    ([35500, 3000], 14.0, 0.0, True, 5),
    ([35500], 7.0, 1.0, False, 20000),
]


@pytest.mark.parametrize("case", DOMINANT_KEY_CASES,
                         ids=[f"L{c[0][0]}-gap{c[1]:g}-std{c[2]:g}-{'tied' if c[3] else 'rand'}-key{c[4]}"
                              for c in DOMINANT_KEY_CASES])
def test_fp8_dominant_key_over_flat_body(gpu_lib, case):
    """One key several nats above tens of thousands of near-equal scores:
    most of the probability mass sits far below the maximum.  Every split
    count (one split over the whole history, the 8 chunks of the long-context
    workload, the automatic count) must match the oracle."""
    lens, gap, std, tied, kp = case
    _say(f"dominant key {case}")
    inp = _dominant_key_inputs(lens, gap, std, tied, kp, seed=31 + int(gap))
    ro, rl, _ = oracle_out(inp)
    for S in (1, 8, 0):
        out, lse = run_verify(gpu_lib, inp, num_splits=S)
        dout, dlse = compare(out, lse, ro, rl, f"{case} S={S}")
        _say(f"  S={S}: max|dout|/max|ref| = {dout:.3e}, max|dlse| = {dlse:.3e}")


def test_fp8_dominant_key_long_sequence_c4_splits(gpu_lib):
    """The same structure over 65,536 positions at the split count of the
    B = 64 FP8 verify workload (32)."""
    _say("dominant key, 65,536 positions, S = 32")
    inp = _dominant_key_inputs([65536], 12.0, 1.0, False, 40000, seed=65)
    ro, rl, _ = oracle_out(inp)
    out, lse = run_verify(gpu_lib, inp, num_splits=32)
    dout, dlse = compare(out, lse, ro, rl, "65536 S=32")
    _say(f"  max|dout|/max|ref| = {dout:.3e}, max|dlse| = {dlse:.3e}")


def test_c6_dcp8_shaped(gpu_lib):
    """The DCP8-shaped workload (96 heads over an eighth of the history), every
    sequence checked."""
    _say("config c6")
    inp = make_config("c6", device="cuda")
    out, lse = run_verify(gpu_lib, inp, max_seq_len_hint=8192)
    ro, rl, _ = oracle_out(inp)
    dout, dlse = compare(out, lse, ro, rl, "c6")
    _say(f"  c6: max|dout|/max|ref| = {dout:.3e}, max|dlse| = {dlse:.3e}")


def test_decode_entry_point(gpu_lib):
    inp = make_inputs([50, 900, 2049], 1, 12, "fp8", seed=5, device="cuda")
    out, lse = gpu_lib.decode(inp.q, inp.kv, inp.page_table, inp.seq_lens, inp.softmax_scale,
                              inp.kv_scale)
    torch.cuda.synchronize()
    ro, rl, _ = oracle_out(inp)
    compare(out, lse, ro, rl, "decode")


def test_c1_tiny(gpu_lib):
    _say("config c1")
    inp = make_config("c1", device="cuda")
    for S in (0, 1, 2, 4):
        out, lse = run_verify(gpu_lib, inp, num_splits=S)
        ro, rl, _ = oracle_out(inp)
        compare(out, lse, ro, rl, f"c1 S={S}")


def test_c2_batched_decode(gpu_lib):
    _say("config c2")
    inp = make_config("c2", device="cuda")
    out, lse = run_verify(gpu_lib, inp, max_seq_len_hint=8192)
    ro, rl, _ = oracle_out(inp)
    compare(out, lse, ro, rl, "c2")


def test_c3_spec_verify(gpu_lib):
    _say("config c3")
    inp = make_config("c3", device="cuda")
    out, lse = run_verify(gpu_lib, inp, max_seq_len_hint=32768)
    ro, rl, _ = oracle_out(inp)
    compare(out, lse, ro, rl, "c3")


def test_c4_fp8_verify(gpu_lib):
    """B = 64 FP8 verify over up to 65,536 positions, every sequence checked."""
    _say("config c4")
    inp = make_config("c4", device="cuda")
    out, lse = run_verify(gpu_lib, inp, max_seq_len_hint=65536)
    ro, rl, _ = oracle_out(inp)
    dout, dlse = compare(out, lse, ro, rl, "c4")
    _say(f"  c4: max|dout|/max|ref| = {dout:.3e}, max|dlse| = {dlse:.3e}")


def test_c5_long_context_all_layers(gpu_lib):
    """All 24 layer caches of the long-context workload at the benchmark's
    split count (64, a multiple of the 8 chunks per sequence); the tolerance
    is per layer."""
    worst = (0.0, 0.0)
    for layer in range(24):
        _say(f"config c5 layer {layer}")
        inp = make_c5_layer(layer, device="cuda")
        out, lse = run_verify(gpu_lib, inp, num_splits=64)
        ro, rl, _ = oracle_out(inp)
        dout, dlse = compare(out, lse, ro, rl, f"c5 layer {layer}")
        worst = (max(worst[0], dout), max(worst[1], dlse))
        del inp
    _say(f"  c5 worst layer: max|dout|/max|ref| = {worst[0]:.3e}, max|dlse| = {worst[1]:.3e}")


def test_c5b_long_context_layer(gpu_lib):
    """One layer of the other reading of the long-context sizes: 4 sequences of
    142,000 positions each, at the split count the library picks for it."""
    _say("config c5b layer 0")
    inp = make_c5_layer(0, device="cuda", name="c5b")
    out, lse = run_verify(gpu_lib, inp, max_seq_len_hint=142000)
    ro, rl, _ = oracle_out(inp)
    dout, dlse = compare(out, lse, ro, rl, "c5b layer 0")
    _say(f"  c5b: max|dout|/max|ref| = {dout:.3e}, max|dlse| = {dlse:.3e}")


def test_split_partials_match_oracle(gpu_lib):
    """mla_split partials (each split's own normalised output and lse) against the
    oracle's partials over the same page ranges, including empty splits."""
    lens = [3, 40, 64, 300, 1000]
    inp = make_inputs(lens, 3, 12, "fp8", seed=77, device="cuda")
    S = 9
    po, pl = gpu_lib.split(inp.q, inp.kv, inp.page_table, inp.seq_lens, inp.softmax_scale,
                           inp.kv_scale, num_splits=S)
    torch.cuda.synchronize()
    ro, rl = oracle_partials(inp, S)
    for s in range(S):
        for b in range(len(lens)):
            lo, hi = split_page_ranges(lens[b], S)[s]
            if not np.isfinite(rl[s, b]).any():
                assert torch.isneginf(pl[s, b]).all() and (po[s, b] == 0).all()
                continue
            fin = np.isfinite(rl[s, b])
            got_l = pl[s, b].cpu().numpy()
            assert np.array_equal(np.isfinite(got_l), fin)
            assert np.abs(got_l[fin] - rl[s, b][fin]).max() <= 1e-3
            got_o = po[s, b].float().cpu().numpy()   # bf16 partials
            assert np.abs(got_o - ro[s, b]).max() <= 1e-2 * np.abs(ro[s, b]).max() + 1e-30


# S = 300 and 1000 exceed the 256 threads of a row slice, so each thread
# reduces several normalisers and streams several rounds of partials
@pytest.mark.parametrize("S", [1, 8, 13, 64, 129, 300, 1000])
def test_merge_matches_oracle(gpu_lib, S):
    rng = np.random.default_rng(3 + S)
    rows = 300 if S <= 300 else 64
    # bf16 partial rows (the split kernel's output type); the oracle merges the
    # same bf16 values, widened exactly
    po_bf = torch.from_numpy(rng.normal(size=(S, rows, 512)).astype(np.float32)).bfloat16()
    pl = (rng.normal(size=(S, rows)) * 3).astype(np.float32)
    pl[rng.random(size=(S, rows)) < 0.2] = -np.inf
    pl[:, 7] = -np.inf          # a row with every partial empty
    empty = torch.from_numpy(np.isneginf(pl))
    po_bf[empty] = 0.0
    po = po_bf.float().numpy()
    # partials of weight zero must not be read into the result: poison them
    po_dev = po_bf.clone()
    po_dev[empty] = float("nan")
    out, lse = gpu_lib.merge(po_dev.cuda(), torch.from_numpy(pl).cuda())
    torch.cuda.synchronize()
    ro, rl = oracle.merge(po.astype(np.float64), pl.astype(np.float64))
    fin = np.isfinite(rl)
    assert np.isneginf(lse.cpu().numpy()[~fin]).all()
    assert (out.float().cpu().numpy()[~fin] == 0).all()
    compare(out[fin], lse[fin], ro[fin], rl[fin], "merge")


@pytest.mark.parametrize("dt,nq,S", [("fp8", 3, 5), ("bf16", 1, 1)])
def test_graph_replay_matches_eager(gpu_lib, dt, nq, S):
    """bench.py times the path as a replayed HIP graph: every replay, with
    eager work and synchronisations between replays, reproduces the eager
    result bit for bit (split + merge with S = 5; one direct launch with S = 1)."""
    _say(f"graph replay {dt} Q={nq} S={S}")
    lens = [300, 1500, 40]
    inp = make_inputs(lens, nq, 12, dt, seed=21 + nq, device="cuda")
    hint = max(lens)
    ws = torch.empty(max(256, gpu_lib.workspace_size(inp.q, inp.kv, inp.page_table, S, hint)),
                     dtype=torch.uint8, device="cuda")
    out = torch.empty((len(lens), nq, 12, 512), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((len(lens), nq, 12), dtype=torch.float32, device="cuda")

    def call():
        gpu_lib.verify(inp.q, inp.kv, inp.page_table, inp.seq_lens, inp.softmax_scale,
                       inp.kv_scale, num_splits=S, max_seq_len_hint=hint, out=out, lse=lse,
                       workspace=ws)

    call()
    torch.cuda.synchronize()
    out_e, lse_e = out.clone(), lse.clone()
    st = torch.cuda.Stream()
    st.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(st):
        call()
    torch.cuda.current_stream().wait_stream(st)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=st):
        call()
    for i in range(4):
        out.zero_()
        lse.zero_()
        ws.fill_(0xFF)   # stale workspace contents must not matter
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, out_e) and torch.equal(lse, lse_e), f"replay {i}"


# The split plan by length (MLA_SPLIT_BY_LENGTH): the S * B split slots spread
# over the sequences in proportion to their pages.  Very unequal lengths,
# sequences shorter than a page, both kernels, several row blocks, the
# largest batch the plan takes (64) and one past it (per-sequence plan used).
BY_LENGTH_CASES = [
    # (seq_lens, Q, H, kv_dtype, num_splits)
    ([16, 40000, 33, 5000], 3, 12, "fp8", 0),
    ([16, 40000, 33, 5000], 3, 12, "fp8", 64),
    ([1, 15, 16, 17, 64, 65, 200, 3000], 1, 12, "bf16", 0),
    ([3, 300, 1029, 7000], 3, 96, "fp8", 4),
    ([100, 8000], 8, 12, "bf16", 6),
    ([5, 9000, 700], 3, 12, "bf16", 9),
    ([2000, 30], 1, 12, "fp8", 16),
]


@pytest.mark.parametrize("case", BY_LENGTH_CASES, ids=[f"{c[3]}-Q{c[1]}-H{c[2]}-S{c[4]}-{len(c[0])}seq"
                                                       for c in BY_LENGTH_CASES])
def test_split_by_length(gpu_lib, case):
    """The plan by length gives the oracle's result (with NaN-poisoned spare
    blocks and page tails), within tolerance of the per-sequence plan."""
    lens, nq, nh, dt, S = case
    _say(f"split by length {case}")
    inp = make_inputs(lens, nq, nh, dt, seed=11 * sum(lens) + nq + nh, device="cuda",
                      spare_blocks=2, poison=True)
    out, lse = run_verify(gpu_lib, inp, num_splits=S, split_policy=gpu_lib.SPLIT_BY_LENGTH)
    ro, rl, _ = oracle_out(inp)
    compare(out, lse, ro, rl, f"by length {case}")
    out_p, lse_p = run_verify(gpu_lib, inp, num_splits=S)
    compare(out, lse, out_p.float().cpu().numpy().astype(np.float64),
            lse_p.cpu().numpy().astype(np.float64), "by length vs per sequence")


@pytest.mark.parametrize("batch", [64, 65])
def test_split_by_length_batch_limit(gpu_lib, batch):
    """64 sequences of random lengths use the plan by length; 65 fall back to
    the per-sequence plan (bit for bit the per-sequence call)."""
    rng = np.random.default_rng(batch)
    lens = [int(x) for x in rng.integers(3, 6000, size=batch)]
    _say(f"split by length, {batch} sequences")
    inp = make_inputs(lens, 3, 12, "fp8", seed=batch, device="cuda")
    out, lse = run_verify(gpu_lib, inp, split_policy=gpu_lib.SPLIT_BY_LENGTH)
    out_p, lse_p = run_verify(gpu_lib, inp)
    if batch > 64:
        assert torch.equal(out, out_p) and torch.equal(lse, lse_p)
    ro, rl, _ = oracle_out(inp)
    compare(out, lse, ro, rl, f"{batch} sequences by length")


@pytest.mark.parametrize("S", [192, 193])
def test_split_by_length_slot_limit(gpu_lib, S):
    """64 sequences with S = 192 splits give 12,288 slots: the longest run of
    one sequence (12,225 slots) is the most the merge's weight table takes,
    and the plan by length is used; at S = 193 it is past that and the call
    uses the per-sequence plan (bit for bit)."""
    rng = np.random.default_rng(S)
    lens = [int(x) for x in rng.integers(3, 400, size=64)]
    lens[7] = 20000
    _say(f"split by length at the slot limit, S = {S}")
    inp = make_inputs(lens, 3, 12, "fp8", seed=S, device="cuda")
    out, lse = run_verify(gpu_lib, inp, num_splits=S, split_policy=gpu_lib.SPLIT_BY_LENGTH)
    out_p, lse_p = run_verify(gpu_lib, inp, num_splits=S)
    if S > 192:
        assert torch.equal(out, out_p) and torch.equal(lse, lse_p)
    ro, rl, _ = oracle_out(inp)
    compare(out, lse, ro, rl, f"S={S} by length")


def test_split_by_length_equal_lengths_bitwise(gpu_lib):
    """With equal lengths the plan by length is the per-sequence plan: the
    same bits."""
    inp = make_inputs([3000] * 4, 3, 12, "fp8", seed=41, device="cuda")
    out, lse = run_verify(gpu_lib, inp, num_splits=16, split_policy=gpu_lib.SPLIT_BY_LENGTH)
    out_p, lse_p = run_verify(gpu_lib, inp, num_splits=16)
    assert torch.equal(out, out_p) and torch.equal(lse, lse_p)


@pytest.mark.parametrize("cfg", ["c2", "c3", "c4", "c6"])
def test_workload_split_by_length(gpu_lib, cfg):
    """The ragged workloads at full size with the plan by length: every
    sequence against the oracle."""
    _say(f"workload {cfg} by length")
    inp = make_config(cfg, device="cuda")
    hint = workloads.CONFIGS[cfg]["seq_hi"]
    out, lse = run_verify(gpu_lib, inp, max_seq_len_hint=hint, split_policy=gpu_lib.SPLIT_BY_LENGTH)
    ro, rl, _ = oracle_out(inp)
    compare(out, lse, ro, rl, f"{cfg} by length")


def test_split_then_merge_equals_verify(gpu_lib):
    """mla_split followed by mla_merge on the same S is the verify call's own
    two launches: bitwise the same output and lse."""
    lens = [700, 2100, 65]
    inp = make_inputs(lens, 3, 12, "fp8", seed=23, device="cuda")
    S = 7
    out_v, lse_v = run_verify(gpu_lib, inp, num_splits=S)
    po, pl = gpu_lib.split(inp.q, inp.kv, inp.page_table, inp.seq_lens, inp.softmax_scale,
                           inp.kv_scale, num_splits=S)
    out_m, lse_m = gpu_lib.merge(po, pl)
    torch.cuda.synchronize()
    assert torch.equal(out_m, out_v) and torch.equal(lse_m, lse_v)


def test_concurrent_streams(gpu_lib):
    """Calls on two streams at once, with their own outputs and workspaces,
    give what they give one after the other (the library keeps no state
    between calls)."""
    a = make_inputs([900, 3000], 3, 12, "fp8", seed=24, device="cuda")
    b = make_inputs([1200, 64, 5000], 1, 12, "bf16", seed=25, device="cuda")
    ref_a = run_verify(gpu_lib, a, num_splits=6)
    ref_b = run_verify(gpu_lib, b, num_splits=3)
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    s1.wait_stream(torch.cuda.current_stream())
    s2.wait_stream(torch.cuda.current_stream())
    res = {}
    for rep in range(3):
        with torch.cuda.stream(s1):
            res["a"] = gpu_lib.verify(a.q, a.kv, a.page_table, a.seq_lens, a.softmax_scale,
                                      a.kv_scale, num_splits=6)
        with torch.cuda.stream(s2):
            res["b"] = gpu_lib.verify(b.q, b.kv, b.page_table, b.seq_lens, b.softmax_scale,
                                      b.kv_scale, num_splits=3)
        torch.cuda.synchronize()
        for key, ref in (("a", ref_a), ("b", ref_b)):
            assert torch.equal(res[key][0], ref[0]) and torch.equal(res[key][1], ref[1]), (key, rep)


def test_deterministic_and_inputs_untouched(gpu_lib):
    inp = make_inputs([300, 1234, 17], 3, 12, "fp8", seed=9, device="cuda")
    kv0, pt0, q0 = inp.kv.clone(), inp.page_table.clone(), inp.q.clone()
    o1, l1 = run_verify(gpu_lib, inp, num_splits=5)
    o2, l2 = run_verify(gpu_lib, inp, num_splits=5)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    assert torch.equal(inp.kv, kv0) and torch.equal(inp.page_table, pt0) and torch.equal(inp.q, q0)


def test_page_table_permutation_bitwise(gpu_lib):
    """Same latents at permuted pool blocks (with poisoned spares and tails):
    bitwise-equal outputs."""
    lens = [70, 333, 1000]
    a = make_inputs(lens, 3, 12, "bf16", seed=10, device="cuda", identity_pages=True)
    nb = a.kv.shape[0]
    perm = torch.from_numpy(np.random.default_rng(1).permutation(nb + 5)).cuda()
    pool = torch.full((nb + 5, 16, 576), float("nan"), dtype=torch.bfloat16, device="cuda")
    pool[perm[:nb]] = a.kv
    pt = torch.where(a.page_table >= 0, perm[a.page_table.clamp(min=0).long()].int(),
                     a.page_table)
    for b, L in enumerate(lens):
        p = -(-L // 16)
        pool[pt[b, p - 1].long(), L - (p - 1) * 16:] = float("nan")
    oa, la = run_verify(gpu_lib, a, num_splits=4)
    ob, lb = gpu_lib.verify(a.q, pool, pt.contiguous(), a.seq_lens, a.softmax_scale, 1.0,
                            num_splits=4)
    torch.cuda.synchronize()
    assert torch.equal(oa, ob) and torch.equal(la, lb)


def test_head_padding(gpu_lib):
    """12 heads vs the same 12 + 4 zero-query heads.  Rows are packed
    token-major, so padding moves a head to another row of the MFMA tiles, but
    every row is computed from its own query alone: a head that stays in the
    same kind of 32-row group agrees bit for bit.  The FP8 kernel packs a
    group of at most 16 real rows (group 1 of a 33..48-row block) with the two
    FP8 terms of each operand in the two halves of one MFMA operand, so there
    the two terms' products are summed in separate fp32 accumulators and added
    at the end, where an unpacked group accumulates them in one: token 2's
    heads 0..7 (rows 24..31 of 36, unpacked; rows 32..39 of 48, packed) agree
    to within one bf16 unit in the last place and 1e-6 relative in lse.  Both
    match the oracle."""
    inp = make_inputs([100, 900], 3, 12, "fp8", seed=11, device="cuda")
    o12, l12 = run_verify(gpu_lib, inp, num_splits=3)
    q16 = torch.zeros((2, 3, 16, 576), dtype=torch.bfloat16, device="cuda")
    q16[:, :, :12] = inp.q
    o16, l16 = gpu_lib.verify(q16, inp.kv, inp.page_table, inp.seq_lens, inp.softmax_scale,
                              inp.kv_scale, num_splits=3)
    torch.cuda.synchronize()
    a, b = o16[:, :, :12], o12
    same = torch.ones((3, 12), dtype=torch.bool, device="cuda")
    same[2, :8] = False          # token 2, heads 0..7: unpacked at H = 12, packed at H = 16
    assert torch.equal(a[:, same], b[:, same]) and torch.equal(l16[:, :, :12][:, same], l12[:, same])
    ai = a[:, ~same].contiguous().view(torch.int16).int()
    bi = b[:, ~same].contiguous().view(torch.int16).int()
    ulps = (ai - bi).abs()
    # equal signs: bit patterns of bf16 values of one sign order as integers
    assert bool(((ai < 0) == (bi < 0)).all()) and int(ulps.max()) <= 1, int(ulps.max())
    la, lb = l16[:, :, :12][:, ~same], l12[:, ~same]
    assert float(((la - lb).abs() / lb.abs().clamp_min(1e-30)).max()) <= 1e-6
    ro, rl, _ = oracle_out(inp)
    compare(o16[:, :, :12].contiguous(), l16[:, :, :12].contiguous(), ro, rl, "H=16 padded")
    compare(o12, l12, ro, rl, "H=12")


@pytest.mark.parametrize("dt,nq,S", [("fp8", 3, 4), ("fp8", 3, 1), ("bf16", 3, 4)])
@pytest.mark.parametrize("neg_scale", [False, True])
def test_query_row_magnitudes(gpu_lib, dt, nq, S, neg_scale):
    """Query rows of very different magnitudes in one row block.  The FP8
    kernel takes each row's exponent from its largest |q| (compared on the
    bf16 magnitude bits) and writes the row as two FP8 terms; the rows here
    are scaled by 2^-110 (past the exponent clamp), 2^-40, 2^-8, 1 and 4, one
    is all zero, one holds bf16 subnormals only, one has its largest values in
    the rope dims, one is negative throughout and one mixes 2^-20 and 2^10
    elements.  A negative softmax scale reverses the order of the scores.
    Every row matches the oracle on both KV types."""
    _say(f"query magnitudes {dt} Q={nq} S={S} negative scale={neg_scale}")
    inp = make_inputs([300, 1100], nq, 12, dt, seed=31 + nq + S, device="cuda")
    q = inp.q.float()
    scales = [2.0 ** -110, 2.0 ** -40, 2.0 ** -8, 1.0, 4.0, 0.0]
    for h, sc in enumerate(scales):
        q[:, :, h] *= sc
    q[:, :, 6] = torch.sign(q[:, :, 6]) * 2.0 ** -130 * (1 + torch.rand_like(q[:, :, 6]))
    q[:, :, 7, 512:] *= 16.0
    q[:, :, 8] = -q[:, :, 8].abs()
    mix = torch.full_like(q[:, :, 9], 2.0 ** -20)
    mix[..., ::37] = 2.0 ** 10 / 64
    q[:, :, 9] = mix * torch.sign(q[:, :, 9])
    inp.q = q.to(torch.bfloat16).contiguous()
    assert (inp.q[:, :, 6] != 0).any() and (inp.q[:, :, 6].float().abs() < 2.0 ** -126).all()
    if neg_scale:
        inp.softmax_scale = -inp.softmax_scale
    out, lse = run_verify(gpu_lib, inp, num_splits=S)
    ro, rl, _ = oracle_out(inp)
    compare(out, lse, ro, rl, f"{dt} S={S} neg={neg_scale}")


def test_verify_equals_truncated_decodes(gpu_lib):
    """Speculative verify is lossless: token j of a Q = 3 verify equals a decode
    over the first L - 3 + j + 1 positions (within tolerance of the oracle)."""
    lens = [200, 1500]
    inp = make_inputs(lens, 3, 12, "fp8", seed=12, device="cuda")
    ov, lv = run_verify(gpu_lib, inp)
    for j in range(3):
        sl = (inp.seq_lens - 3 + j + 1).int().contiguous()
        od, ld = gpu_lib.decode(inp.q[:, j:j + 1].contiguous(), inp.kv, inp.page_table, sl,
                                inp.softmax_scale, inp.kv_scale)
        torch.cuda.synchronize()
        ref = ov[:, j:j + 1].float().cpu().numpy().astype(np.float64)
        compare(od, ld, ref, lv[:, j:j + 1].cpu().numpy().astype(np.float64), f"token {j}")


def test_split_count_invariance(gpu_lib):
    inp = make_inputs([1500, 64, 4097], 3, 12, "bf16", seed=13, device="cuda")
    ro, rl, _ = oracle_out(inp)
    for S in (1, 2, 8, 31, 64):
        out, lse = run_verify(gpu_lib, inp, num_splits=S)
        compare(out, lse, ro, rl, f"S={S}")


def test_fp8_scale_not_rounded_into_operand(gpu_lib):
    """kv_scale must stay out of the bf16 operand: with a scale whose products with
    E4M3 values are not bf16-representable, the result still matches the oracle,
    which uses decode(byte) * kv_scale exactly."""
    inp = make_inputs([333], 3, 12, "fp8", seed=14, device="cuda")
    inp.kv_scale = float(np.float32(0.0370000008))
    out, lse = run_verify(gpu_lib, inp)
    ro, rl, _ = oracle_out(inp)
    compare(out, lse, ro, rl, "odd kv_scale")


def test_errors_raise(gpu_lib):
    inp = make_inputs([100], 1, 12, "bf16", seed=15, device="cuda")
    with pytest.raises(gpu_lib.MLAError):
        gpu_lib.verify(inp.q, inp.kv, inp.page_table, inp.seq_lens, float("nan"), 1.0)
    q3 = torch.zeros((1, 3, 12, 576), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(gpu_lib.MLAError):
        gpu_lib.decode(q3, inp.kv, inp.page_table, inp.seq_lens, inp.softmax_scale, 1.0)
    ws = torch.empty(16, dtype=torch.uint8, device="cuda")
    with pytest.raises(gpu_lib.MLAError):
        gpu_lib.verify(inp.q, inp.kv, inp.page_table, inp.seq_lens, inp.softmax_scale, 1.0,
                       num_splits=4, workspace=ws)
    # caller-supplied outputs of the wrong dtype, shape or device
    for kw in (dict(out=torch.empty((1, 1, 12, 512), dtype=torch.float32, device="cuda")),
               dict(out=torch.empty((1, 1, 12, 256), dtype=torch.bfloat16, device="cuda")),
               dict(out=torch.empty((1, 1, 12, 512), dtype=torch.bfloat16)),
               dict(lse=torch.empty((1, 1, 12), dtype=torch.bfloat16, device="cuda")),
               dict(lse=torch.empty((1, 1, 6), dtype=torch.float32, device="cuda"))):
        with pytest.raises(gpu_lib.MLAError):
            gpu_lib.verify(inp.q, inp.kv, inp.page_table, inp.seq_lens, inp.softmax_scale, 1.0,
                           **kw)
    po = torch.zeros((2, 1, 1, 12, 512), dtype=torch.bfloat16, device="cuda")
    pl = torch.zeros((2, 1, 1, 12), dtype=torch.float32, device="cuda")
    with pytest.raises(gpu_lib.MLAError):
        gpu_lib.merge(po, pl, out=torch.empty((1, 1, 12, 512), dtype=torch.float32, device="cuda"))
    with pytest.raises(gpu_lib.MLAError):
        gpu_lib.merge(po, pl.cpu())
