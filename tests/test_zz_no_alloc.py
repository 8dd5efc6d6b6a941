"""mla_verify_static (the entry point that allocates nothing: partials in a
static per-GPU array) against mla_verify on the same inputs, through the C
ABI: two calls in a row, the second with a smaller input, each bit for bit
equal to mla_verify and within the oracle tolerance.  Collected last so that
a failure here cannot hide the other GPU tests."""

import numpy as np
import pytest
import torch

from workloads import make_inputs
from parity_util import compare, oracle_out

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)


@pytest.mark.parametrize("dt", ["fp8", "bf16"])
def test_static_scratch_matches_verify(gpu_lib, dt):
    cases = [([35500, 35500, 35500, 35500], 3, 64),    # the long-context layer's shape
             ([300, 1000, 17], 3, 0)]                  # then a smaller one (fewer partials)
    for i, (lens, nq, S) in enumerate(cases):
        _say(f"static scratch {dt} call {i}: lens={lens} S={S}")
        inp = make_inputs(lens, nq, 12, dt, seed=900 + i, device="cuda", spare_blocks=1,
                          poison=True)
        hint = max(lens)
        ref_o, ref_l = gpu_lib.verify(inp.q, inp.kv, inp.page_table, inp.seq_lens,
                                      inp.softmax_scale, inp.kv_scale, num_splits=S,
                                      max_seq_len_hint=hint)
        out, lse = gpu_lib.verify_static(inp.q, inp.kv, inp.page_table, inp.seq_lens,
                                         inp.softmax_scale, inp.kv_scale, num_splits=S,
                                         max_seq_len_hint=hint)
        torch.cuda.synchronize()
        assert torch.equal(out, ref_o) and torch.equal(lse, ref_l), f"call {i}"
        ro, rl, _ = oracle_out(inp)
        compare(out, lse, ro, rl, f"static scratch {dt} call {i}")


def test_static_scratch_single_split_and_limit(gpu_lib):
    """One split (no partials: direct output) and a request beyond the array."""
    inp = make_inputs([200, 40], 1, 12, "bf16", seed=910, device="cuda")
    ref = gpu_lib.verify(inp.q, inp.kv, inp.page_table, inp.seq_lens, inp.softmax_scale,
                         inp.kv_scale, num_splits=1)
    got = gpu_lib.verify_static(inp.q, inp.kv, inp.page_table, inp.seq_lens, inp.softmax_scale,
                                inp.kv_scale, num_splits=1)
    torch.cuda.synchronize()
    assert torch.equal(got[0], ref[0]) and torch.equal(got[1], ref[1])
    big = make_inputs([64] * 4000, 3, 96, "fp8", seed=911, device="cuda")
    with pytest.raises(gpu_lib.MLAError) as e:
        gpu_lib.verify_static(big.q, big.kv, big.page_table, big.seq_lens, big.softmax_scale,
                              big.kv_scale, num_splits=16)
    assert e.value.status == 8
