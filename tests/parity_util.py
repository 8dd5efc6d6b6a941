"""Helpers shared by the GPU parity tests: run the HIP path, run the oracle on
the same bytes, compare at the stated tolerance.

Tolerance (BF16 / FP8 inputs, FP32 accumulation):
    max |out_gpu - out_ref| <= 1e-2 * max |out_ref|   (max over the compared tensor)
    max |lse_gpu - lse_ref| <= 1e-3                    (per element, natural log)
"""

import numpy as np
import torch

import oracle
from workloads import compact_for_oracle

OUT_REL_TOL = 1e-2
LSE_ABS_TOL = 1e-3


def split_page_ranges(seq_len, num_splits):
    """Position ranges of the splits, as include/mla.h defines them: sequence with
    P = ceil(L / 16) pages, split s covers pages [floor(sP/S), floor((s+1)P/S))."""
    P = -(-int(seq_len) // 16)
    out = []
    for s in range(num_splits):
        a = (s * P) // num_splits
        e = ((s + 1) * P) // num_splits
        out.append((min(16 * a, seq_len), min(16 * e, seq_len)))
    return out


def oracle_out(inp, batch_indices=None):
    d = compact_for_oracle(inp, batch_indices)
    out, lse = oracle.mla_reference(d["q_bits"], d["kv_raw"], d["page_table"], d["seq_lens"],
                                    d["softmax_scale"], d["kv_dtype"], d["kv_scale"])
    return out, lse, d


def oracle_partials(inp, num_splits, batch_indices=None):
    d = compact_for_oracle(inp, batch_indices)
    ranges = [split_page_ranges(L, num_splits) for L in d["seq_lens"]]
    return oracle.mla_partials(d["q_bits"], d["kv_raw"], d["page_table"], d["seq_lens"],
                               d["softmax_scale"], ranges, d["kv_dtype"], d["kv_scale"])


def compare(out_gpu, lse_gpu, out_ref, lse_ref, what="", lse_tol=LSE_ABS_TOL):
    """Assert the tolerance; returns (max|dout| / max|ref|, max|dlse|)."""
    og = out_gpu.detach().float().cpu().numpy().astype(np.float64)
    lg = lse_gpu.detach().float().cpu().numpy().astype(np.float64)
    assert og.shape == out_ref.shape, (og.shape, out_ref.shape)
    assert np.isfinite(og).all(), f"{what}: non-finite output"
    scale = np.abs(out_ref).max()
    dout = np.abs(og - out_ref).max() / scale
    fin = np.isfinite(lse_ref)
    assert np.array_equal(np.isfinite(lg), fin), f"{what}: lse finiteness differs"
    assert (lg[~fin] == lse_ref[~fin]).all()
    dlse = np.abs(lg[fin] - lse_ref[fin]).max() if fin.any() else 0.0
    assert dout <= OUT_REL_TOL, f"{what}: max|dout|/max|ref| = {dout:.3e}"
    assert dlse <= lse_tol, f"{what}: max|dlse| = {dlse:.3e}"
    return dout, dlse


def run_verify(mla, inp, **kw):
    fn = mla.decode if (inp.num_q == 1 and kw.pop("use_decode", False)) else mla.verify
    out, lse = fn(inp.q, inp.kv, inp.page_table, inp.seq_lens, inp.softmax_scale, inp.kv_scale,
                  **kw)
    torch.cuda.synchronize()
    return out, lse
