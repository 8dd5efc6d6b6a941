"""Figures printed on the pages (tests/golden/page_figures.json) pin the byte
accounting, shapes and number formats used by the workloads and the oracle."""

import json
import os

import numpy as np
import torch

import oracle
import oracle.mla as om
import workloads
from workloads import mla_inputs as wi

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "page_figures.json")))


def test_kv_footprint_matches_page():
    g = GOLD["mla_kv_footprint"]
    total = g["layers"] * g["positions"] * g["fp8_bytes_per_position"]
    assert round(total / 1e9, 2) == g["total_gb_per_gpu_approx"]
    assert abs(total / 8 / 1e6 - g["dcp8_total_mb_approx"]) < 1.0
    # the long-context workload (24 layers x 4 x 35,500 positions) holds exactly that KV
    c = workloads.CONFIGS["c5"]
    per_layer_kv = c["batch"] * c["seq_lo"] * wi.LATENT_DIM * 1
    assert c["layers"] * per_layer_kv == total
    lens = [c["seq_lo"]] * c["batch"]
    kv_term = workloads.algorithmic_bytes(lens, 1, 0, "fp8") - int(np.sum(-(-np.array(lens) // 16))) * 4
    assert kv_term == per_layer_kv
    assert wi.LATENT_DIM == g["fp8_bytes_per_position"] == om.LATENT_DIM


def test_heads_per_rank_and_padding():
    g = GOLD["mla_heads"]
    assert g["total_mla_query_heads"] // g["tp"] == g["heads_per_gpu"]
    assert all(workloads.CONFIGS[k]["heads"] == g["heads_per_gpu"] for k in ("c1", "c2", "c3", "c4", "c5"))
    assert -(-g["heads_per_gpu"] // 16) * 16 == g["padded_heads"]


def test_fp8_halves_bytes_per_position():
    g = GOLD["fp8_vs_bf16_capacity"]
    ratio = g["fp8_tokens"] / g["bf16_tokens"]
    assert round(ratio, 2) == g["ratio_printed"]
    bf16_b = workloads.algorithmic_bytes([1000], 1, 0, "bf16")
    fp8_b = workloads.algorithmic_bytes([1000], 1, 0, "fp8")
    assert abs((bf16_b - 63 * 4) / (fp8_b - 63 * 4) - ratio) < 0.01


def test_bf16_rounding_example():
    g = GOLD["bf16_rounding_example"]
    x = torch.tensor([g["fp32_value"], 256.0], dtype=torch.float32)
    xb = x.to(torch.bfloat16)
    bits = xb.view(torch.int16).numpy().view(np.uint16)
    v = oracle.bf16_bits_to_f64(bits)
    assert v[0] == g["bf16_value"]
    assert float(x[0] - x[1]) == g["difference_fp32_inputs"]
    assert v[0] - v[1] == g["difference_bf16_inputs"]


def test_page_size():
    assert GOLD["page_size"]["block_size"] == wi.PAGE == om.PAGE
