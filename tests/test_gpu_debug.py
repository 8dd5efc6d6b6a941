"""The debug build of the library (libmla_hip_debug.so, compiled with
MLA_DEBUG=1) on the GPU: it checks the caller contract of include/mla.h on the
device ("Kimi K2.6 + DFlash on 8x MI300X", section "Technical numbers": paged
KV in blocks of 16).  Out-of-range page ids and sequence lengths are passed to
the debug library only: it clamps them before any read, every kernel runs to
its end, and the violation shows up in the flag word.  On valid inputs it
reports nothing and computes what the release library computes, bit for bit.
"""

import contextlib

import numpy as np
import pytest
import torch

import decode_attention_03_amd as mla
from decode_attention_03_amd import _lib
from workloads import make_inputs

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


@pytest.fixture(scope="module")
def debug_lib():
    mla.load()
    return _lib.load_debug()


@contextlib.contextmanager
def using(lib):
    """Route the binding's calls to `lib` for the duration."""
    saved = _lib._LIB
    _lib._LIB = lib
    try:
        yield
    finally:
        _lib._LIB = saved


def _run(lib, inp, num_splits):
    with using(lib):
        out, lse = mla.verify(inp.q, inp.kv, inp.page_table, inp.seq_lens, inp.softmax_scale,
                              inp.kv_scale, num_splits=num_splits)
        torch.cuda.synchronize()
    return out, lse


# (kv dtype, query tokens, heads): the FP8 eight-wave kernel packed (36 rows)
# and unpacked (80 rows, two row blocks), the generic kernel with FP8 and with
# bf16 KV (12 rows), the bf16 eight-wave kernel (36 rows)
SHAPES = [("fp8", 3, 12), ("fp8", 5, 16), ("fp8", 1, 12), ("bf16", 1, 12), ("bf16", 3, 12)]


@pytest.mark.parametrize("dtype,Q,H", SHAPES)
@pytest.mark.parametrize("num_splits", [1, 3])
def test_debug_build_matches_release_on_valid_inputs(debug_lib, dtype, Q, H, num_splits):
    print(f"[debug build] valid inputs {dtype} Q={Q} H={H} S={num_splits}", flush=True)
    inp = make_inputs([70, 333, 1100], Q, H, dtype, seed=91, device=DEV)
    _lib.debug_flags(debug_lib)   # start clean
    ro, rl = _run(mla.load(), inp, num_splits)
    do, dl = _run(debug_lib, inp, num_splits)
    assert _lib.debug_flags(debug_lib) == 0
    assert torch.equal(ro.view(torch.int16), do.view(torch.int16))
    assert torch.equal(rl, dl)


@pytest.mark.parametrize("dtype,Q,H", SHAPES)
@pytest.mark.parametrize("case", ["page_too_large", "page_negative", "seq_too_long", "seq_too_short"])
def test_debug_build_reports_contract_violations(debug_lib, dtype, Q, H, case):
    print(f"[debug build] {case} {dtype} Q={Q} H={H}", flush=True)
    inp = make_inputs([70, 333, 1100], Q, H, dtype, seed=92, device=DEV)
    pt = inp.page_table.clone()
    sl = inp.seq_lens.clone()
    nb = inp.num_blocks
    if case == "page_too_large":
        pt[1, 5] = nb + 7           # a page the call reads (sequence 1 has 21 pages)
        expect = _lib.DEBUG_PAGE_ID
    elif case == "page_negative":
        pt[2, 0] = -3
        expect = _lib.DEBUG_PAGE_ID
    elif case == "seq_too_long":
        # clamped to 16 * max_blocks, the sequence also reads the unused
        # entries (-1) of its page-table row: both violations are reported
        sl[0] = 16 * inp.max_blocks_per_seq + 40
        expect = _lib.DEBUG_SEQ_LONG | _lib.DEBUG_PAGE_ID
    else:
        sl[1] = Q - 1 if Q > 1 else 0
        expect = _lib.DEBUG_SEQ_SHORT
    bad = type(inp)(q=inp.q, kv=inp.kv, page_table=pt, seq_lens=sl, kv_dtype=inp.kv_dtype,
                    kv_scale=inp.kv_scale, softmax_scale=inp.softmax_scale)
    _lib.debug_flags(debug_lib)
    for S in (1, 4):
        out, lse = _run(debug_lib, bad, S)
        assert torch.isfinite(out.float()).all()
        flags = _lib.debug_flags(debug_lib)
        assert flags == expect, (case, S, flags)
    # the sequences the violation does not touch are computed as usual
    ok = [b for b in range(3) if not ((case == "page_too_large" and b == 1) or
                                      (case == "page_negative" and b == 2) or
                                      (case == "seq_too_long" and b == 0) or
                                      (case == "seq_too_short" and b == 1))]
    ro, rl = _run(mla.load(), inp, 4)
    out, lse = _run(debug_lib, bad, 4)
    _lib.debug_flags(debug_lib)
    assert torch.equal(ro[ok].view(torch.int16), out[ok].view(torch.int16))


@pytest.mark.parametrize("dtype", ["fp8", "bf16"])
def test_debug_build_append_reports_bad_slots(debug_lib, dtype):
    print(f"[debug build] append {dtype}", flush=True)
    inp = make_inputs([40, 97], 3, 12, dtype, seed=93, device=DEV)
    g = torch.Generator(device="cpu").manual_seed(5)
    new = (torch.randn((2, 3, 576), generator=g) * 0.5).to(torch.bfloat16).to(DEV)
    pt = inp.page_table.clone()
    # the blocks of sequence 1's new tokens (positions 94, 95, 96: pages 5 and 6)
    pt[1, 5] = inp.num_blocks + 2
    pt[1, 6] = -1
    kv_ref = inp.kv.clone()
    kv_dbg = inp.kv.clone()
    _lib.debug_flags(debug_lib)
    with using(mla.load()):   # release build: valid slots only (sequence 0)
        ok_pt = inp.page_table.clone()
        mla.kv_append(new[:1], kv_ref, ok_pt[:1].contiguous(), inp.seq_lens[:1].contiguous(),
                      kv_scale=inp.kv_scale)
    with using(debug_lib):
        mla.kv_append(new, kv_dbg, pt, inp.seq_lens, kv_scale=inp.kv_scale)
    torch.cuda.synchronize()
    assert _lib.debug_flags(debug_lib) == _lib.DEBUG_PAGE_ID
    # sequence 0 written as by the release build; nothing written for sequence 1
    # (its slots' block is out of range, and its other blocks are untouched)
    assert torch.equal(kv_ref.view(torch.uint8), kv_dbg.view(torch.uint8))
