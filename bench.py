"""Throughput of the MLA decode / verify hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config c5] [--num-splits S]

A step is one pass of the whole hot path over one batch of synthetic input
already resident in HBM: for the long-context workload (default, "c5"),
24 independent layer caches of 142,000 FP8 positions each (4 sequences x
35,500), 3 query tokens x 12 heads, each layer one mla_verify call
(split-KV kernel + log-sum-exp merge), back to back on one stream.  The
24 caches (1.96 GB) exceed the 256 MB Infinity Cache, so every layer reads
cold KV.

Printed: one JSON line with the metric (algorithmic KV-read GB/s, and us per
layer-step), a roofline object for the dominant kernel (the split kernel;
its average duration is measured with HIP events on the launch stream inside
a second timed region), and the float64 oracle timed on the host cores on a
bounded sample of the same workload.
"""

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MLA decode KV-read GB/s (% of 8 TB/s HBM) + µs per layer-step, 12 heads"
HBM_PEAK_GBS = 8000.0
PROFILES = os.path.join(ROOT, "profiles")
SPLIT_SRC = os.path.join(ROOT, "decode_attention_03_amd", "csrc", "mla_split.hip")


def _args():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", default="c5", choices=["c1", "c2", "c3", "c4", "c5", "c5b"])
    ap.add_argument("--num-splits", type=int, default=0, help="0 = library's choice")
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="CPU time budget of the oracle baseline sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain 1 GiB device copy (for HBM counter calibration)")
    return ap.parse_args()


def _layers(cfg, device):
    import torch
    import workloads
    from workloads import mla_inputs as wi
    c = workloads.CONFIGS[cfg]
    if "layers" in c:
        return [workloads.make_c5_layer(l, device=device, name=cfg) for l in range(c["layers"])], c
    base = workloads.make_config(cfg, device=device)
    # rotate copies of the pool so the timed footprint exceeds the 256 MB Infinity Cache
    per = base.kv.numel() * base.kv.element_size()
    copies = 1 if cfg == "c1" else max(1, -(-(1 << 30) // per))
    layers = [base]
    for i in range(1, copies):
        layers.append(wi.MLAInputs(q=base.q, kv=base.kv.clone(), page_table=base.page_table,
                                   seq_lens=base.seq_lens, kv_dtype=base.kv_dtype,
                                   kv_scale=base.kv_scale, softmax_scale=base.softmax_scale,
                                   meta=dict(base.meta, copy=i)))
    return layers, c


def _traffic(per_launch_alg_bytes):
    """HBM bytes per split-kernel launch from the committed counter summary, or
    None when the summary is missing or was taken on another kernel source."""
    path = os.path.join(PROFILES, "mla_split_c5_traffic.json")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path))
    src_hash = hashlib.sha256(open(SPLIT_SRC, "rb").read()).hexdigest()
    if rec.get("split_source_sha256") != src_hash:
        return None
    return float(rec["hbm_bytes_per_dispatch"])


def _cpu_baseline(layers, budget_s):
    """The float64 oracle on the host cores, on whole layers of the same workload
    until the time budget is spent; returns the rate in GB/s of algorithmic bytes."""
    import numpy as np
    import oracle
    import workloads
    from workloads import compact_for_oracle
    try:
        from threadpoolctl import threadpool_info
        blas_threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        blas_threads = None
    cores = len(os.sched_getaffinity(0))
    done_bytes, t_used, n_layers, n_seqs = 0, 0.0, 0, 0
    for inp in layers:
        for b in range(inp.batch):
            d = compact_for_oracle(inp, [b])
            t0 = time.perf_counter()
            oracle.mla_reference(d["q_bits"], d["kv_raw"], d["page_table"], d["seq_lens"],
                                 d["softmax_scale"], d["kv_dtype"], d["kv_scale"])
            t_used += time.perf_counter() - t0
            done_bytes += workloads.algorithmic_bytes(d["seq_lens"], inp.num_q, inp.heads,
                                                      inp.kv_dtype)
            n_seqs += 1
            if t_used >= budget_s:
                break
        n_layers += 1
        if t_used >= budget_s:
            break
    return {"value": round(done_bytes / t_used / 1e9, 4), "unit": "GB/s",
            "cores": int(blas_threads or cores), "kind": "oracle",
            "sample": f"{n_seqs} sequences over {n_layers} layer(s) of the same workload "
                      f"({done_bytes / 1e6:.1f} MB of algorithmic bytes, {t_used:.1f} s); "
                      f"float64 NumPy oracle, BLAS threads={blas_threads}, "
                      f"host cores visible={cores}"}


def main():
    args = _args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(--gpus must be 1).", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch
    import decode_attention_03_amd as mla
    import workloads

    assert torch.cuda.is_available(), "bench.py needs the GPU"
    mla.load()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    layers, cfg = _layers(args.config, dev)
    n_layers = len(layers)
    hint = cfg["seq_hi"]
    first = layers[0]
    S = mla.num_splits(first.q, first.kv, first.page_table, args.num_splits, hint)

    outs = [torch.empty((l.batch, l.num_q, l.heads, 512), dtype=torch.bfloat16, device=dev)
            for l in layers]
    lses = [torch.empty((l.batch, l.num_q, l.heads), dtype=torch.float32, device=dev)
            for l in layers]
    ws_bytes = max(mla.workspace_size(l.q, l.kv, l.page_table, args.num_splits, hint)
                   for l in layers)
    ws = torch.empty(max(ws_bytes, 256), dtype=torch.uint8, device=dev)

    def step():
        for i, l in enumerate(layers):
            mla.verify(l.q, l.kv, l.page_table, l.seq_lens, l.softmax_scale, l.kv_scale,
                       num_splits=args.num_splits, max_seq_len_hint=hint, out=outs[i],
                       lse=lses[i], workspace=ws)

    # Same kernels, same launch configuration as mla_verify (split kernel, then
    # merge when S > 1), issued as separate calls so each kernel can be timed.
    R = first.batch * first.num_q * first.heads
    po = torch.empty((S, R * 512), dtype=torch.float32, device=dev)
    pl = torch.empty((S, R), dtype=torch.float32, device=dev)

    def split_only():
        for l in layers:
            mla.split(l.q, l.kv, l.page_table, l.seq_lens, l.softmax_scale, l.kv_scale,
                      num_splits=S, max_seq_len_hint=hint, part_out=po, part_lse=pl)

    def merge_only():
        for i, l in enumerate(layers):
            mla.merge(po.view(S, l.batch, l.num_q, l.heads, 512),
                      pl.view(S, l.batch, l.num_q, l.heads), out=outs[i], lse=lses[i])

    # Eager issue (one Python call per layer) for reference.
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    eager_ms = (time.perf_counter() - t0) * 1e3 / args.steps

    # Timed region: the step captured once as a HIP graph (the library neither
    # allocates nor synchronises, so it is capturable) and replayed K times;
    # this removes host launch overhead, as decode serving does.
    stream = torch.cuda.Stream(device=dev)
    graphs = {}
    for name, fn in (("step", step), ("split", split_only), ("merge", merge_only)):
        stream.wait_stream(torch.cuda.current_stream(dev))
        with torch.cuda.stream(stream):
            fn()  # warm the capture stream
        torch.cuda.current_stream(dev).wait_stream(stream)
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=stream):
            fn()
        graphs[name] = g
    torch.cuda.synchronize()
    for _ in range(args.warmup):
        graphs["step"].replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        graphs["step"].replay()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    ms_per_step = elapsed * 1e3 / args.steps

    alg = [workloads.algorithmic_bytes(l.seq_lens.cpu().numpy(), l.num_q, l.heads, l.kv_dtype)
           for l in layers]
    flops = [workloads.algorithmic_flops(l.seq_lens.cpu().numpy(), l.num_q, l.heads)
             for l in layers]
    bytes_per_step = sum(alg)
    value = bytes_per_step / (ms_per_step * 1e-3) / 1e9
    us_per_layer = ms_per_step * 1e3 / n_layers

    # Per-kernel durations: HIP events on the launch stream around replays of
    # graphs holding only the split kernels, or only the merge kernels.
    cur = torch.cuda.current_stream(dev)

    def timed(g, reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        for _ in range(args.warmup):
            g.replay()
        e0.record(cur)
        for _ in range(reps):
            g.replay()
        e1.record(cur)
        e1.synchronize()
        return e0.elapsed_time(e1) / reps / n_layers * 1e3  # us per kernel launch

    split_us = timed(graphs["split"], args.steps)
    merge_us = timed(graphs["merge"], args.steps) if S > 1 else 0.0
    split_alg = float(np.mean(alg))     # one split launch processes one layer's batch
    achieved = split_alg / (split_us * 1e-6) / 1e9
    traffic = _traffic(split_alg)

    line = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "us_per_layer_step": round(us_per_layer, 3),
        "hbm_frac": round(value / HBM_PEAK_GBS, 4),
        "config": {
            "workload": cfg["desc"],
            "name": args.config,
            "layers_per_step": n_layers,
            "batch": first.batch,
            "num_q_tokens": first.num_q,
            "heads": first.heads,
            "kv_dtype": "fp8_e4m3fn" if first.kv_dtype == "fp8" else "bf16",
            "mfma_operands": "bf16, fp32 accumulate",
            "num_splits": S,
            "algorithmic_bytes_per_step": int(bytes_per_step),
            "algorithmic_flops_per_step": int(sum(flops)),
            "mfma_tflops_algorithmic": round(sum(flops) / (ms_per_step * 1e-3) / 1e12, 2),
            "split_kernel_us": round(split_us, 3),
            "merge_kernel_us": round(merge_us, 3),
            "timing": "HIP graph of the 24-layer step replayed K times; per-kernel times from "
                      "graphs of one kernel kind, HIP events on the launch stream",
            "eager_ms_per_step": round(eager_ms, 4),
        },
        "roofline": {
            "bound": "hbm",
            "kernel": "split_kernel",
            "achieved": round(achieved, 2),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": None if traffic is None else round(traffic),
        },
    }
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = _cpu_baseline(layers, args.cpu_seconds)
    if args.copy_calibration:
        n = 1 << 30
        a = torch.empty(n, dtype=torch.uint8, device=dev)
        b = torch.empty_like(a)
        for _ in range(3):
            b.copy_(a)
        torch.cuda.synchronize()
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
