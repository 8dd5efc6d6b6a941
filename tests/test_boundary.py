"""The C-ABI library on the CPU: it loads, exports every symbol include/mla.h
declares, and its host-side validation rejects bad arguments before any HIP
call (so these run without a GPU).  No compute call is made here."""

import ctypes
import os
import re

import pytest

import decode_attention_03_amd as mla
from decode_attention_03_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mla.h")

OK, NULL, SHAPE, DTYPE, SCALE, UNSUPPORTED, WS, HIP = range(8)


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(mla_[a-z_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    return mla.load()


def params(**kw):
    d = dict(batch=4, num_q_tokens=3, num_heads=12, num_blocks=8876, max_blocks_per_seq=2219,
             max_seq_len_hint=35500, kv_dtype=1, num_splits=0)
    d.update(kw)
    return _lib.Params(**d)


def test_exports_every_declared_symbol(lib):
    names = _declared()
    assert set(names) == set(_lib.EXPORTS), names
    for n in names:
        assert hasattr(lib, n), n


def test_exports_every_peak_symbol(lib):
    """include/mla_peaks.h (measured-peak microbenchmarks) is exported too, and
    its host-side validation rejects bad arguments before any launch."""
    text = re.sub(r"/\*.*?\*/", "", open(os.path.join(ROOT, "include", "mla_peaks.h")).read(), flags=re.S)
    names = sorted(set(re.findall(r"\b(mla_[a-z_]+)\s*\(", text)))
    assert set(names) == set(_lib.PEAK_EXPORTS), names
    for n in names:
        assert hasattr(lib, n), n
    assert lib.mla_peak_hbm_read(None, 1 << 20, 0, None, 64, None) == NULL
    fake = ctypes.c_void_p(1 << 40)   # never dereferenced: rejected first
    assert lib.mla_peak_hbm_read(fake, 1000, 0, fake, 64, None) == SHAPE
    assert lib.mla_peak_hbm_read(fake, 1 << 20, 2, fake, 64, None) == SHAPE
    assert lib.mla_peak_hbm_read(fake, 1 << 20, 0, fake, 0, None) == SHAPE
    assert lib.mla_peak_mfma(0, 0, fake, 64, None) == SHAPE
    assert lib.mla_peak_mfma(2, 10, fake, 64, None) == SHAPE
    assert lib.mla_peak_mfma(0, 10, None, 64, None) == NULL


def test_missing_library_fails_loudly(tmp_path):
    saved = _lib._LIB
    _lib._LIB = None
    try:
        with pytest.raises(RuntimeError):
            _lib.load(str(tmp_path / "nope.so"))
    finally:
        _lib._LIB = saved


def test_status_strings(lib):
    for s in range(9):
        assert lib.mla_status_string(s) != b"unknown status"
    assert lib.mla_status_string(99) == b"unknown status"


def test_split_planning(lib):
    # long-context layer, FP8: 4 sequences x 2219 pages -> ceil(2219 / 128) = 18,
    # but one round of 256 workgroups needs 64 (<= 2219 / 32): 64
    assert lib.mla_num_splits(ctypes.byref(params())) == 64
    # 4 x 142,000 positions (8875 pages) -> 70 -> 280 workgroups, between one
    # and two rounds -> one full round: 64
    assert lib.mla_num_splits(ctypes.byref(params(max_seq_len_hint=142000))) == 64
    assert lib.mla_num_splits(ctypes.byref(params(num_splits=8))) == 8
    # 64 FP8 sequences up to 4096 pages -> 32 (2048 workgroups)
    assert lib.mla_num_splits(ctypes.byref(params(batch=64, max_seq_len_hint=65536))) == 32
    # 32 bf16 sequences up to 2048 pages -> 2048 / 64 = 32
    assert lib.mla_num_splits(ctypes.byref(params(batch=32, max_seq_len_hint=32768,
                                                  kv_dtype=0))) == 32
    # 32 bf16 decode sequences (Q = 1) up to 512 pages -> 8 (one round)
    assert lib.mla_num_splits(ctypes.byref(params(batch=32, num_q_tokens=1,
                                                  max_seq_len_hint=8192, kv_dtype=0))) == 8
    # 32 FP8 sequences up to 512 pages -> 4, but one round needs 8 (<= 256): 8
    assert lib.mla_num_splits(ctypes.byref(params(batch=32, max_seq_len_hint=8192))) == 8
    # one sequence of 16 pages: a round would need 256 splits, 2 pages each
    # allow 8
    assert lib.mla_num_splits(ctypes.byref(params(batch=1, max_seq_len_hint=256,
                                                  max_blocks_per_seq=16))) == 8
    # 2 bf16 sequences (Q = 3) of 64 pages: 64 / 2 = 32
    assert lib.mla_num_splits(ctypes.byref(params(batch=2, max_seq_len_hint=1024,
                                                  kv_dtype=0))) == 32
    # one FP8 sequence of 512 pages: a round would need 256 splits of 2 pages;
    # past 128 each split must keep 16 pages -> 128
    assert lib.mla_num_splits(ctypes.byref(params(batch=1, max_seq_len_hint=8192))) == 128
    # 8875 pages: 256 splits keep 34 pages each
    assert lib.mla_num_splits(ctypes.byref(params(batch=1, max_seq_len_hint=142000))) == 256
    # two pages: one split
    assert lib.mla_num_splits(ctypes.byref(params(batch=1, max_seq_len_hint=20))) == 1
    assert lib.mla_num_splits(ctypes.byref(params(batch=1, max_seq_len_hint=48))) == 1
    assert lib.mla_num_splits(ctypes.byref(params(num_heads=129))) == 0
    # 96 heads x 3 tokens = 288 FP8 rows -> 5 row blocks of 64: 4 x 5 = 20 units;
    # max(18, min(13, 69)) = 18 -> 360 workgroups -> one round: 12
    assert lib.mla_num_splits(ctypes.byref(params(num_heads=96))) == 12
    # DCP8 shape: 64 sequences x 5 row blocks up to 512 pages -> 4 (1280 workgroups)
    assert lib.mla_num_splits(ctypes.byref(params(batch=64, num_heads=96,
                                                  max_seq_len_hint=8192))) == 4
    S = 8
    rows = 4 * 3 * 12
    expect = ((S * rows * 512 * 2 + 255) // 256) * 256 + ((S * rows * 4 + 255) // 256) * 256
    assert lib.mla_workspace_size(ctypes.byref(params(num_splits=S))) == expect
    assert lib.mla_workspace_size(ctypes.byref(params(num_splits=1))) == 0


FAKE = ctypes.c_void_p(0x1000)  # never dereferenced: every call below fails validation


def _verify(lib, p, ss=0.07, ks=0.03, ws=None, wsb=0, entry="mla_verify", nulls=()):
    ptrs = [FAKE] * 6
    for i in nulls:
        ptrs[i] = None
    q, kv, pt, sl, out, lse = ptrs
    return getattr(lib, entry)(ctypes.byref(p) if p is not None else None, q, kv, pt, sl, ss, ks,
                               out, lse, ws, wsb, None)


@pytest.mark.parametrize("entry", ["mla_verify", "mla_decode"])
def test_validation_errors(lib, entry):
    q1 = 1 if entry == "mla_decode" else 3
    assert _verify(lib, None, entry=entry) == NULL
    for i in range(6):
        assert _verify(lib, params(num_q_tokens=q1), entry=entry, nulls=(i,)) == NULL
    for bad in (dict(batch=0), dict(num_q_tokens=0), dict(num_q_tokens=9), dict(num_heads=0),
                dict(num_blocks=0), dict(max_blocks_per_seq=0), dict(max_seq_len_hint=-1),
                dict(num_splits=-1), dict(num_splits=257)):
        d = dict(num_q_tokens=q1)
        d.update(bad)
        assert _verify(lib, params(**d), entry=entry) == SHAPE, bad
    assert _verify(lib, params(num_q_tokens=q1, num_heads=129), entry=entry) == UNSUPPORTED
    assert _verify(lib, params(num_q_tokens=q1, kv_dtype=2), entry=entry) == DTYPE
    assert _verify(lib, params(num_q_tokens=q1), ss=float("nan"), entry=entry) == SCALE
    assert _verify(lib, params(num_q_tokens=q1), ss=float("inf"), entry=entry) == SCALE
    assert _verify(lib, params(num_q_tokens=q1), ks=0.0, entry=entry) == SCALE
    assert _verify(lib, params(num_q_tokens=q1), ks=-1.0, entry=entry) == SCALE
    assert _verify(lib, params(num_q_tokens=q1), ks=float("nan"), entry=entry) == SCALE
    # workspace missing or too small when more than one split is used
    assert _verify(lib, params(num_q_tokens=q1, num_splits=4), entry=entry) == WS
    assert _verify(lib, params(num_q_tokens=q1, num_splits=4), ws=FAKE, wsb=100, entry=entry) == WS


def test_grid_size_limit(lib):
    # split launch: 256 splits x 65,535 sequences x 16 FP8 row blocks x 512
    # threads > 2^32 - 1 work-items; rejected before any pointer is touched
    big = params(batch=65535, num_q_tokens=8, num_heads=128, num_splits=256)
    assert _verify(lib, big) == UNSUPPORTED
    assert lib.mla_split(ctypes.byref(big), FAKE, FAKE, FAKE, FAKE, 0.07, 0.03, FAKE, FAKE,
                         None) == UNSUPPORTED
    # bf16, 48-row blocks of 256 threads: 22 blocks x 256 x 65,535 x 256 > 2^32 - 1
    assert _verify(lib, params(batch=65535, num_q_tokens=8, num_heads=128, num_splits=256,
                               kv_dtype=0)) == UNSUPPORTED
    # the split launch fits (33 x 65,535 x 2 row blocks x 512 = 2.2e9) but
    # the merge of 8.4 M rows at 1,024 threads per row (S > 32) does not
    fits_split = params(batch=65535, num_q_tokens=8, num_heads=16, num_splits=33)
    assert _verify(lib, fits_split) == UNSUPPORTED
    # a large call that fits both launches goes on to the workspace check
    assert _verify(lib, params(batch=65535, num_q_tokens=3, num_heads=12, num_splits=2)) == WS
    # mla_merge: 2^22 rows x 1,024 threads (S > 32) = 2^32 > 2^32 - 1
    assert lib.mla_merge(FAKE, FAKE, 64, 1 << 22, FAKE, FAKE, None) == UNSUPPORTED


def test_split_policy_validation(lib):
    """split_policy is MLA_SPLIT_PER_SEQUENCE (0) or MLA_SPLIT_BY_LENGTH (1);
    mla_split keeps its per-sequence partial layout and refuses the other."""
    assert _verify(lib, params(split_policy=2)) == SHAPE
    assert _verify(lib, params(split_policy=-1)) == SHAPE
    assert _verify(lib, params(split_policy=1, num_splits=4)) == WS     # valid: reaches the workspace check
    assert lib.mla_split(ctypes.byref(params(split_policy=1)), FAKE, FAKE, FAKE, FAKE, 0.07, 0.03,
                         FAKE, FAKE, None) == UNSUPPORTED
    # the split count and workspace do not depend on the policy
    for kw in (dict(), dict(batch=64, max_seq_len_hint=65536), dict(batch=32, kv_dtype=0)):
        a, b = params(**kw), params(split_policy=1, **kw)
        assert lib.mla_num_splits(ctypes.byref(a)) == lib.mla_num_splits(ctypes.byref(b))
        assert lib.mla_workspace_size(ctypes.byref(a)) == lib.mla_workspace_size(ctypes.byref(b))


def test_decode_rejects_multi_token(lib):
    assert _verify(lib, params(num_q_tokens=2), entry="mla_decode") == SHAPE


def test_bf16_ignores_kv_scale_but_checks_softmax_scale(lib):
    # bf16: kv_scale is not used, so 0 is accepted; the call then fails on the workspace check.
    assert _verify(lib, params(kv_dtype=0, num_splits=4), ks=0.0) == WS
    assert _verify(lib, params(kv_dtype=0, num_splits=4), ss=float("nan")) == SCALE


def test_split_and_merge_validation(lib):
    p = params()
    assert lib.mla_split(None, FAKE, FAKE, FAKE, FAKE, 0.07, 0.03, FAKE, FAKE, None) == NULL
    assert lib.mla_split(ctypes.byref(p), FAKE, FAKE, FAKE, FAKE, 0.07, 0.03, None, FAKE, None) == NULL
    assert lib.mla_split(ctypes.byref(params(num_heads=0)), FAKE, FAKE, FAKE, FAKE, 0.07, 0.03,
                         FAKE, FAKE, None) == SHAPE
    assert lib.mla_split(ctypes.byref(p), FAKE, FAKE, FAKE, FAKE, 0.07, -0.03, FAKE, FAKE, None) == SCALE
    assert lib.mla_merge(None, FAKE, 4, 10, FAKE, FAKE, None) == NULL
    assert lib.mla_merge(FAKE, FAKE, 0, 10, FAKE, FAKE, None) == SHAPE
    assert lib.mla_merge(FAKE, FAKE, 4097, 10, FAKE, FAKE, None) == SHAPE
    assert lib.mla_merge(FAKE, FAKE, 4, 0, FAKE, FAKE, None) == SHAPE
    assert lib.mla_merge(FAKE, FAKE, 4, (1 << 28) + 1, FAKE, FAKE, None) == SHAPE


def test_append_and_scale_validation(lib):
    p = params(num_heads=0, num_splits=-5)     # fields append ignores
    pb = ctypes.byref(p)
    A = lib.mla_kv_append
    assert A(None, FAKE, FAKE, FAKE, FAKE, 0.03, None) == NULL
    for i in range(4):
        args = [FAKE] * 4
        args[i] = None
        assert A(pb, *args, 0.03, None) == NULL, i
    for bad in (dict(batch=0), dict(num_q_tokens=0), dict(num_q_tokens=9), dict(num_blocks=0),
                dict(max_blocks_per_seq=0)):
        assert A(ctypes.byref(params(**bad)), FAKE, FAKE, FAKE, FAKE, 0.03, None) == SHAPE, bad
    assert A(ctypes.byref(params(kv_dtype=2)), FAKE, FAKE, FAKE, FAKE, 0.03, None) == DTYPE
    # 16-byte alignment of the new latents and of the cache
    assert A(pb, ctypes.c_void_p(0x1008), FAKE, FAKE, FAKE, 0.03, None) == SHAPE
    assert A(pb, FAKE, ctypes.c_void_p(0x1004), FAKE, FAKE, 0.03, None) == SHAPE
    for ks in (0.0, -1.0, float("nan"), float("inf")):
        assert A(pb, FAKE, FAKE, FAKE, FAKE, ks, None) == SCALE, ks
    D = lib.mla_kv_dynamic_scale
    assert D(None, 10, FAKE, None) == NULL
    assert D(FAKE, 10, None, None) == NULL
    assert D(FAKE, -1, FAKE, None) == SHAPE
    assert D(FAKE, (1 << 40) + 1, FAKE, None) == SHAPE
    assert D(FAKE, 10, ctypes.c_void_p(0x1002), None) == SHAPE


def test_binding_checks_caller_outputs():
    """The kernels write B*Q*H*512 bf16 and B*Q*H fp32 through raw pointers: a
    caller-supplied output of the wrong dtype, shape, layout or device is
    rejected before any call."""
    import torch
    dev = torch.device("cpu")
    good = torch.empty((2, 3, 12, 512), dtype=torch.bfloat16)
    _lib._check_out("out", good, torch.bfloat16, (2, 3, 12, 512), dev)
    bad = [
        torch.empty((2, 3, 12, 512), dtype=torch.float32),          # dtype
        torch.empty((2, 3, 12, 256), dtype=torch.bfloat16),         # too small
        torch.empty((2, 3, 512, 12), dtype=torch.bfloat16).transpose(2, 3),   # not contiguous
        torch.empty((1, 3, 12, 512), dtype=torch.bfloat16),         # batch
    ]
    for t in bad:
        with pytest.raises(mla.MLAError):
            _lib._check_out("out", t, torch.bfloat16, (2, 3, 12, 512), dev)
    with pytest.raises(mla.MLAError):
        _lib._check_out("out", good, torch.bfloat16, (2, 3, 12, 512), torch.device("meta"))


def test_merge_rejects_host_partials():
    import torch
    po = torch.zeros((2, 4, 512), dtype=torch.bfloat16)
    pl = torch.zeros((2, 4), dtype=torch.float32)
    with pytest.raises(mla.MLAError):
        mla.merge(po, pl)


def test_static_entry_rejects_partials_beyond_its_scratch(lib):
    """mla_verify_static refuses, before any HIP call, a request whose split
    partials exceed its static per-GPU array (MLA_STATIC_SCRATCH_BYTES)."""
    p = params(batch=65535, num_q_tokens=3, num_heads=12, max_seq_len_hint=65536,
               max_blocks_per_seq=4096, num_splits=8)
    assert lib.mla_workspace_size(ctypes.byref(p)) > mla.STATIC_SCRATCH_BYTES
    d = ctypes.c_void_p(16)
    st = lib.mla_verify_static(ctypes.byref(p), d, d, d, d, ctypes.c_float(0.07),
                               ctypes.c_float(1.0), d, d, None)
    assert st == 8, st
    assert b"static scratch" in lib.mla_status_string(8)
    # the long-context and B = 64 FP8 workloads fit
    for kw in (dict(), dict(batch=64, max_seq_len_hint=65536, max_blocks_per_seq=4096)):
        assert lib.mla_workspace_size(ctypes.byref(params(**kw))) <= mla.STATIC_SCRATCH_BYTES


def test_debug_library_exports_and_identifies_itself(lib):
    """The debug build (MLA_DEBUG=1) exports the same symbols; each library
    says which build it is, and the release build reports no flags without a
    HIP call."""
    dbg = _lib.load_debug()
    for n in _declared():
        assert hasattr(dbg, n), n
    assert dbg.mla_debug_build() == 1
    assert lib.mla_debug_build() == 0
    v = ctypes.c_uint32(123)
    assert lib.mla_debug_flags(ctypes.byref(v), 1) == OK and v.value == 0
    assert lib.mla_debug_flags(None, 0) == NULL
