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
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MLA decode KV-read GB/s (% of 8 TB/s HBM) + µs per layer-step, 12 heads"
HBM_PEAK_GBS = 8000.0
PROFILES = os.path.join(ROOT, "profiles")
DEVICE_CODE = os.path.join(ROOT, "decode_attention_03_amd", "_build", "device_code.json")


def _kernel_sha256(name):
    """sha256 of one split kernel's gfx950 assembly in the current build (by its
    demangled name, as the profiler reports it; written by the build next to
    the objects), or None if the build did not record it."""
    if not os.path.exists(DEVICE_CODE):
        return None
    return json.load(open(DEVICE_CODE)).get("kernels", {}).get("mla_split.hip", {}).get(name)


def _log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def _args():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", default="c5", choices=["c1", "c2", "c3", "c4", "c5", "c5b", "c6"])
    ap.add_argument("--num-splits", type=int, default=0, help="0 = library's choice")
    ap.add_argument("--split-policy", default="auto", choices=["auto", "per-sequence", "by-length"],
                    help="how the splits are spread over the sequences (auto: by length for "
                         "workloads of unequal lengths, else per sequence)")
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="CPU time budget of the oracle baseline sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-peaks", action="store_true",
                    help="skip the measured-peak microbenchmarks (HBM read, MFMA)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain 1 GiB elementwise copy (negation) for HBM counter "
                         "calibration")
    ap.add_argument("--summarize-profiles", nargs=4, metavar=("TRACE", "FETCH", "WRITE", "MFMA"),
                    help="no GPU: turn rocprofv3 output folders (kernel trace + stats, FETCH_SIZE, "
                         "WRITE_SIZE, MFMA counters) of a --copy-calibration run into the "
                         "summaries under profiles/")
    ap.add_argument("--profile-tag", default="long_ctx_fp8_4x35500_q3_h12",
                    help="workload tag in the summary file names")
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


def _profile_record(tag, num_splits, policy):
    """The committed counter summary of the split kernel for this workload, or
    None when it is missing or was taken on other device code of that kernel
    (its gfx950 assembly in the current build), another split count or
    another split policy."""
    path = os.path.join(PROFILES, f"split_traffic__{tag}.json")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path))
    dev = _kernel_sha256(rec.get("kernel"))
    if dev is None or rec.get("split_kernel_sha256") != dev or rec.get("num_splits") != num_splits:
        return None
    if rec.get("split_policy", "per-sequence") != policy:
        return None
    return rec


def _read_csvs(folder, suffix):
    import csv
    import glob
    rows = []
    for f in sorted(glob.glob(os.path.join(folder, "**", "*" + suffix), recursive=True)):
        rows.extend(csv.DictReader(open(f)))
    if not rows:
        raise SystemExit(f"no *{suffix} under {folder}")
    return rows


def _command_of(folder):
    p = os.path.join(folder, "command.txt")
    return open(p).read().strip() if os.path.exists(p) else "(command not recorded)"


def _per_kernel(rows, pick):
    """Mean counter values per dispatch of the kernels whose name satisfies pick."""
    import collections
    acc = collections.defaultdict(list)
    for r in rows:
        if pick(r["Kernel_Name"]):
            acc[r["Counter_Name"]].append(float(r["Counter_Value"]))
    return {k: (sum(v) / len(v), len(v)) for k, v in acc.items()}


def _is_split(name):
    return "split_kernel" in name


def _is_merge(name):
    return "merge_kernel" in name


def _is_calib(name):
    return "neg_kernel" in name


def summarize_profiles(trace_dir, fetch_dir, write_dir, mfma_dir, tag):
    """Writes profiles/kernel_stats__TAG.md, profiles/split_traffic__TAG.json/.md
    from rocprofv3 output of `bench.py --copy-calibration` runs (CPU only)."""
    import workloads
    if not os.path.exists(DEVICE_CODE):
        raise SystemExit("build the library first: the summary records the split kernel's "
                         "device-code hash of the current build")
    stats = _read_csvs(trace_dir, "kernel_stats.csv")
    trace = _read_csvs(trace_dir, "kernel_trace.csv")
    fetch = _read_csvs(fetch_dir, "counter_collection.csv")
    write = _read_csvs(write_dir, "counter_collection.csv")
    mfma = _read_csvs(mfma_dir, "counter_collection.csv")
    os.makedirs(PROFILES, exist_ok=True)

    # kernel time summary (rocprofv3 --stats), our kernels and the largest others
    stats.sort(key=lambda r: -float(r["TotalDurationNs"]))
    split_stat = [r for r in stats if _is_split(r["Name"])]
    merge_stat = [r for r in stats if _is_merge(r["Name"])]
    if not split_stat:
        raise SystemExit("no split kernel in the kernel stats")
    split_avg_us = float(split_stat[0]["AverageNs"]) / 1e3
    # grid of the split kernel from the trace (workgroups = grid / 256 threads)
    grids = sorted({int(r["Grid_Size_X"] if "Grid_Size_X" in r else r["Grid_Size"])
                    for r in trace if _is_split(r["Kernel_Name"])})
    lines = [f"# Kernel time: split + merge, workload {tag}", "",
             "Command (from the repository root on the GPU host):", "", "```",
             _command_of(trace_dir), "```", "",
             "| kernel | calls | average us | min us | max us | share of GPU time |",
             "|---|---|---|---|---|---|"]
    for r in stats[:8]:
        name = r["Name"]
        short = ("split: " if _is_split(name) else "merge: " if _is_merge(name) else "") + \
            (name if len(name) < 90 else name[:87] + "...")
        lines.append(f"| `{short}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | "
                     f"{float(r['MinNs']) / 1e3:.2f} | {float(r['MaxNs']) / 1e3:.2f} | "
                     f"{float(r['Percentage']):.1f}% |")
    lines += ["", f"Split kernel grid sizes (threads): {grids}"]
    open(os.path.join(PROFILES, f"kernel_stats__{tag}.md"), "w").write("\n".join(lines) + "\n")

    # HBM bytes, calibrated on the 1 GiB negation (reads 1 GiB, writes 1 GiB)
    cal_f = _per_kernel(fetch, _is_calib).get("FETCH_SIZE")
    cal_w = _per_kernel(write, _is_calib).get("WRITE_SIZE")
    spl_f = _per_kernel(fetch, _is_split)["FETCH_SIZE"]
    spl_w = _per_kernel(write, _is_split)["WRITE_SIZE"]
    mrg_f = _per_kernel(fetch, _is_merge).get("FETCH_SIZE", (0.0, 0))
    mrg_w = _per_kernel(write, _is_merge).get("WRITE_SIZE", (0.0, 0))
    if cal_f is None or cal_w is None:
        raise SystemExit("calibration kernel (neg_kernel) missing from the counter runs")
    gib = float(1 << 30)
    ff = gib / (cal_f[0] * 1024.0)
    fw = gib / (cal_w[0] * 1024.0)
    split_bytes = spl_f[0] * 1024.0 * ff + spl_w[0] * 1024.0 * fw
    merge_bytes = mrg_f[0] * 1024.0 * ff + mrg_w[0] * 1024.0 * fw

    # algorithmic bytes per split launch of this workload (one layer)
    cfg = tag_config(tag)
    c = workloads.CONFIGS[cfg]
    if "layers" in c:
        inp = workloads.make_c5_layer(0, device="cpu", name=cfg)
    else:
        inp = workloads.make_config(cfg, device="cpu")
    alg = workloads.algorithmic_bytes(inp.seq_lens.numpy(), inp.num_q, inp.heads, inp.kv_dtype)
    S = _recorded_splits(trace_dir)

    m = _per_kernel(mfma, _is_split)
    mops8 = m.get("SQ_INSTS_VALU_MFMA_MOPS_F8", (0.0, 0))[0]
    mops16 = m.get("SQ_INSTS_VALU_MFMA_MOPS_BF16", (0.0, 0))[0]
    busy = m.get("SQ_VALU_MFMA_BUSY_CYCLES", (0.0, 0))[0]
    gui = m.get("GRBM_GUI_ACTIVE", (0.0, 0))[0]
    lds_conf = m.get("SQ_LDS_BANK_CONFLICT", (0.0, 0))[0]
    lds_act = m.get("SQ_LDS_IDX_ACTIVE", (0.0, 0))[0]
    # MFMA busy: busy cycles per SIMD (the counter sums 1,024 SIMDs) over the
    # cycles the GPU was active per XCD (the counter sums 8 XCDs)
    mfma_busy_frac = (busy / 1024.0) / (gui / 8.0) if gui > 0 else None
    lds_conf_frac = lds_conf / lds_act if lds_act > 0 else None
    mfma_flops = (mops8 + mops16) * 512.0
    rec = {
        "kernel": split_stat[0]["Name"],
        "workload": tag,
        "config_key": cfg,
        "num_splits": S,
        "split_policy": _recorded_config(trace_dir).get("split_policy", "per-sequence"),
        "split_kernel_sha256": _kernel_sha256(split_stat[0]["Name"]),
        "split_avg_us": round(split_avg_us, 3),
        "merge_avg_us": round(float(merge_stat[0]["AverageNs"]) / 1e3, 3) if merge_stat else None,
        "fetch_kib_per_dispatch": round(spl_f[0], 1),
        "write_kib_per_dispatch": round(spl_w[0], 1),
        "dispatches_counted": spl_f[1],
        "calibration": {"kernel": "torch.neg on 2^28 float32 (1 GiB read, 1 GiB written)",
                        "fetch_kib": round(cal_f[0], 1), "write_kib": round(cal_w[0], 1),
                        "fetch_factor": round(ff, 4), "write_factor": round(fw, 4)},
        "hbm_bytes_per_dispatch": round(split_bytes),
        "algorithmic_bytes_per_dispatch": int(alg),
        "traffic_over_algorithmic": round(split_bytes / alg, 4),
        "achieved_gbs_from_profile": round(alg / (split_avg_us * 1e-6) / 1e9, 1),
        "merge_hbm_bytes_per_dispatch": round(merge_bytes),
        "mfma": {"executed_flops_per_dispatch": mfma_flops,
                 "executed_tflops": round(mfma_flops / (split_avg_us * 1e-6) / 1e12, 2),
                 "mfma_busy_cycles_per_dispatch": busy,
                 "grbm_gui_active_per_dispatch": gui,
                 "mfma_busy_fraction": None if mfma_busy_frac is None else round(mfma_busy_frac, 4),
                 "counters": "SQ_INSTS_VALU_MFMA_MOPS_F8/BF16 x 512 flops"},
        "lds": {"bank_conflict_cycles_per_dispatch": lds_conf,
                "lds_active_cycles_per_dispatch": lds_act,
                "bank_conflict_fraction": None if lds_conf_frac is None else round(lds_conf_frac, 4)},
        "commands": [_command_of(d) for d in (fetch_dir, write_dir, mfma_dir)],
    }
    json.dump(rec, open(os.path.join(PROFILES, f"split_traffic__{tag}.json"), "w"), indent=1)
    md = [f"# HBM traffic and MFMA work of the split kernel, workload {tag}", "",
          "Counter passes (each its own run, from the repository root on the GPU host):", ""]
    for cmd in rec["commands"]:
        md += ["```", cmd, "```"]
    md += ["", "Summarised with `python bench.py --summarize-profiles <trace> <fetch> <write> "
           f"<mfma> --profile-tag {tag}`.", "",
           "| quantity | value |", "|---|---|",
           f"| split kernel average duration (kernel trace) | {split_avg_us:.2f} us |",
           f"| split count | {S} ({rec['split_policy']} plan) |",
           f"| FETCH_SIZE per dispatch | {spl_f[0]:.0f} KiB |",
           f"| WRITE_SIZE per dispatch | {spl_w[0]:.0f} KiB |",
           f"| calibration: 1 GiB negation reads / writes | {cal_f[0]:.0f} / {cal_w[0]:.0f} KiB "
           f"(factors {ff:.3f} / {fw:.3f}) |",
           f"| HBM bytes per split dispatch (calibrated) | {split_bytes / 1e6:.2f} MB |",
           f"| algorithmic bytes per split dispatch | {alg / 1e6:.2f} MB |",
           f"| traffic / algorithmic | {split_bytes / alg:.3f} |",
           f"| achieved (algorithmic bytes / average duration) | "
           f"{alg / (split_avg_us * 1e-6) / 1e9:.0f} GB/s = "
           f"{alg / (split_avg_us * 1e-6) / 1e9 / HBM_PEAK_GBS * 100:.1f}% of 8 TB/s |",
           f"| HBM bytes per merge dispatch (calibrated) | {merge_bytes / 1e6:.2f} MB |",
           f"| executed MFMA flops per split dispatch | {mfma_flops / 1e9:.2f} GFLOP "
           f"({mfma_flops / (split_avg_us * 1e-6) / 1e12:.1f} TFLOP/s) |",
           f"| MFMA busy cycles per split dispatch (sum over SIMDs) | {busy:.3g} |",
           "| MFMA busy (SQ_VALU_MFMA_BUSY_CYCLES / 1024 SIMDs over GRBM_GUI_ACTIVE / 8 XCDs) | "
           + ("n/a" if mfma_busy_frac is None else f"{mfma_busy_frac * 100:.1f}%") + " |",
           "| LDS bank-conflict cycles / LDS active cycles (SQ_LDS_BANK_CONFLICT / SQ_LDS_IDX_ACTIVE) | "
           + ("n/a" if lds_conf_frac is None else f"{lds_conf:.3g} / {lds_act:.3g} = {lds_conf_frac * 100:.1f}%")
           + " |"]
    open(os.path.join(PROFILES, f"split_traffic__{tag}.md"), "w").write("\n".join(md) + "\n")
    print("\n".join(md))


TAGS = {"long_ctx_fp8_4x35500_q3_h12": "c5", "long_ctx_fp8_4x142000_q3_h12": "c5b",
        "fp8_verify_b64_q3_h12": "c4", "bf16_verify_b32_q3_h12": "c3",
        "bf16_decode_b32_q1_h12": "c2", "tiny_decode_b1_l256": "c1",
        "dcp8_fp8_verify_b64_q3_h96": "c6"}


def tag_config(tag):
    return TAGS[tag]


def config_tag(cfg):
    return {v: k for k, v in TAGS.items()}[cfg]


def _recorded_config(folder):
    """The config object of the bench JSON line saved beside the trace (bench.json)."""
    p = os.path.join(folder, "bench.json")
    if not os.path.exists(p):
        return {}
    for ln in open(p):
        if ln.startswith('{"metric"'):
            return json.loads(ln)["config"]
    return {}


def _recorded_splits(folder):
    """Split count from the bench JSON line saved beside the trace (bench.json)."""
    n = _recorded_config(folder).get("num_splits")
    return None if n is None else int(n)


def _cpu_model():
    """The host CPU's model name (from /proc/cpuinfo, as lscpu reports it)."""
    try:
        for ln in open("/proc/cpuinfo"):
            if ln.lower().startswith("model name"):
                return ln.split(":", 1)[1].strip()
    except OSError:  # pragma: no cover
        pass
    import platform
    return platform.processor() or "unknown"


def _oracle_rate(layers, budget_s):
    """The float64 oracle on whole sequences of the given layers until the time
    budget is spent: (GB/s of algorithmic bytes, sequences, layers, bytes, seconds)."""
    import oracle
    import workloads
    from workloads import compact_for_oracle
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
    return done_bytes / t_used / 1e9, n_seqs, n_layers, done_bytes, t_used


def _cpu_baseline(layers, budget_s):
    """The float64 oracle on the host cores, on whole layers of the same workload
    until the time budget is spent, then on one core (BLAS limited to one
    thread) for a quarter of the budget; rates in GB/s of algorithmic bytes."""
    try:
        from threadpoolctl import threadpool_info, threadpool_limits
        blas_threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threadpool_limits, blas_threads = None, None
    cores = len(os.sched_getaffinity(0))
    rate, n_seqs, n_layers, nbytes, t_used = _oracle_rate(layers, budget_s)
    out = {"value": round(rate, 4), "unit": "GB/s",
           "cores": int(blas_threads or cores), "kind": "oracle",
           "sample": f"{n_seqs} sequences over {n_layers} layer(s) of the same workload "
                     f"({nbytes / 1e6:.1f} MB of algorithmic bytes, {t_used:.1f} s); "
                     f"float64 NumPy oracle, BLAS threads={blas_threads}, "
                     f"host cores visible={cores}",
           "cpu_model": _cpu_model()}
    if threadpool_limits is not None:
        with threadpool_limits(limits=1):
            r1, s1, l1, b1, t1 = _oracle_rate(layers, max(1.0, budget_s / 4))
        out["single_core"] = {"value": round(r1, 4), "unit": "GB/s", "cores": 1,
                              "sample": f"{s1} sequence(s), {b1 / 1e6:.1f} MB, {t1:.1f} s, "
                                        "BLAS limited to one thread"}
    return out


def _measured_peaks(dev):
    """HBM read bandwidth and dense MFMA rate measured on this GPU with the
    library's microbenchmark kernels (include/mla_peaks.h), HIP events on the
    launch stream: a 2 GiB read (larger than the 256 MB last-level cache) with
    plain vector loads and with the split kernels' direct-to-LDS loads, and a
    stream of independent FP8 / bf16 MFMAs on every SIMD."""
    import torch
    from decode_attention_03_amd import _lib
    nbytes = 2 << 30
    buf = torch.ones(nbytes, dtype=torch.uint8, device=dev)
    wgs = 1024
    isink = torch.zeros(wgs, dtype=torch.int32, device=dev)
    fsink = torch.zeros(wgs, dtype=torch.float32, device=dev)
    cur = torch.cuda.current_stream(dev)

    def best_ms(fn, reps=5):
        fn()
        times = []
        for _ in range(reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(cur)
            fn()
            e1.record(cur)
            e1.synchronize()
            times.append(e0.elapsed_time(e1))
        return min(times)

    out = {}
    for name, mode in (("hbm_read_gbs", _lib.PEAK_READ_VGPR), ("hbm_read_lds_gbs", _lib.PEAK_READ_LDS)):
        ms = best_ms(lambda: _lib.peak_hbm_read(buf, mode, isink, wgs))
        out[name] = round(nbytes / (ms * 1e-3) / 1e9, 1)
    del buf
    iters = 4096
    for name, kind, flops in (("mfma_fp8_tflops", _lib.PEAK_MFMA_FP8, 131072),
                              ("mfma_bf16_tflops", _lib.PEAK_MFMA_BF16, 32768)):
        ms = best_ms(lambda: _lib.peak_mfma(kind, iters, fsink, wgs))
        total = wgs * 4 * iters * 4 * flops
        out[name] = round(total / (ms * 1e-3) / 1e12, 1)
    out["method"] = ("best of 5 launches, HIP events; read: 2 GiB once, 1024 workgroups of "
                     "256 threads, 16-byte loads; MFMA: 1024 workgroups x 4 waves x 4 independent "
                     "accumulators")
    return out


def _rank_merge(mla, first, dev, warmup, steps):
    """The merge a rank runs under context parallelism over ranks = heads / 12
    GPUs: after the exchange of partials it combines, for its own 12 heads,
    one partial per rank.  Timed on seeded partials of that shape."""
    import torch
    ranks = first.heads // 12
    rows = first.batch * first.num_q * 12
    g = torch.Generator(device="cpu").manual_seed(606)
    po = (torch.randn((ranks, rows * 512), generator=g) * 0.05).to(torch.bfloat16).to(dev)
    pl = (torch.randn((ranks, rows), generator=g) + 8.0).to(dev)
    out = torch.empty((first.batch, first.num_q, 12, 512), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((first.batch, first.num_q, 12), dtype=torch.float32, device=dev)

    def run():
        mla.merge(po.view(ranks, first.batch, first.num_q, 12, 512),
                  pl.view(ranks, first.batch, first.num_q, 12), out=out, lse=lse)

    per_graph = 20
    us = _graph_us(run, dev, warmup, steps, per_graph)
    nbytes = ranks * rows * (512 * 2 + 4) + rows * (512 * 2 + 4)
    return {"partials": ranks, "rows": rows, "us": round(us, 3),
            "gb_per_s": round(nbytes / (us * 1e-6) / 1e9, 1),
            "note": f"seeded partials; HIP graph of {per_graph} merges replayed, HIP events"}


def _graph_us(fn, dev, warmup, steps, per_graph=20):
    """Average duration of fn's kernels: a HIP graph of per_graph calls replayed,
    HIP events on the launch stream."""
    import torch
    stream = torch.cuda.Stream(device=dev)
    stream.wait_stream(torch.cuda.current_stream(dev))
    with torch.cuda.stream(stream):
        fn()
    torch.cuda.current_stream(dev).wait_stream(stream)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=stream):
        for _ in range(per_graph):
            fn()
    for _ in range(warmup):
        graph.replay()
    cur = torch.cuda.current_stream(dev)
    n = max(1, steps // per_graph)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(cur)
    for _ in range(n):
        graph.replay()
    e1.record(cur)
    e1.synchronize()
    return e0.elapsed_time(e1) / (n * per_graph) * 1e3


def _append_leg(mla, first, dev, warmup, steps):
    """The step before attention: the Q new latents of every sequence written
    into their cache slots (quantised for an FP8 cache), and the dynamic
    per-tensor scale of those latents.  Runs on a copy of the first cache."""
    import torch
    g = torch.Generator(device="cpu").manual_seed(707)
    new = (torch.randn((first.batch, first.num_q, 576), generator=g) * 0.5).to(torch.bfloat16).to(dev)
    kv = first.kv.clone()
    scale = torch.empty((1,), dtype=torch.float32, device=dev)
    ap_us = _graph_us(lambda: mla.kv_append(new, kv, first.page_table, first.seq_lens,
                                            kv_scale=first.kv_scale), dev, warmup, steps)
    sc_us = _graph_us(lambda: mla.kv_dynamic_scale(new, scale), dev, warmup, steps)
    elem = 1 if first.kv_dtype == "fp8" else 2
    nbytes = new.numel() * 2 + new.numel() * elem + first.batch * 4 * 2
    del kv
    return {"rows": first.batch * first.num_q, "append_us": round(ap_us, 3),
            "append_gb_per_s": round(nbytes / (ap_us * 1e-6) / 1e9, 2),
            "dynamic_scale_us": round(sc_us, 3),
            "note": "mla_kv_append of the step's new latents and mla_kv_dynamic_scale of them; "
                    "HIP graph of 20 calls replayed, HIP events"}


def main():
    args = _args()
    if args.summarize_profiles:
        summarize_profiles(*args.summarize_profiles, args.profile_tag)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
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
    _log(f"{n_layers} layer input(s) of {args.config} resident on {dev}")
    hint = cfg["seq_hi"]
    first = layers[0]
    S = mla.num_splits(first.q, first.kv, first.page_table, args.num_splits, hint)
    ragged = cfg["seq_lo"] != cfg["seq_hi"]
    policy_name = args.split_policy
    if policy_name == "auto":
        # by length for unequal lengths when the per-sequence plan runs at most
        # five rounds of workgroups (beyond that the rounds balance the work:
        # at eight rounds, B = 64 FP8 verify, both plans take the same time)
        rows = first.num_q * first.heads
        rblock = 64 if rows > 32 else (16 if rows <= 16 else 48)
        wgs = S * first.batch * -(-rows // rblock)
        policy_name = "by-length" if (ragged and wgs <= 5 * 256) else "per-sequence"
    policy = mla.SPLIT_BY_LENGTH if policy_name == "by-length" else mla.SPLIT_PER_SEQUENCE
    # the split and merge of the plan by length run only inside mla_verify:
    # the kernel legs below are timed together, as the layer-step
    joint = policy == mla.SPLIT_BY_LENGTH and S > 1

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
                       num_splits=args.num_splits, max_seq_len_hint=hint, split_policy=policy,
                       out=outs[i],
                       lse=lses[i], workspace=ws)

    # Same kernels, same launch configuration as mla_verify (split kernel, then
    # merge when S > 1), issued as separate calls so each kernel can be timed.
    R = first.batch * first.num_q * first.heads
    po = torch.empty((S, R * 512), dtype=torch.bfloat16, device=dev)
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
    _log(f"eager: {eager_ms:.3f} ms per step")

    # Timed region: the step captured as a HIP graph (the library neither
    # allocates nor synchronises, so it is capturable) and replayed; this
    # removes host launch overhead, as decode serving does.  A graph holds
    # `reps` consecutive steps (at least 24 layer calls) so that the graph
    # launch itself is amortised for small workloads; a timed step is still
    # one pass over the batch.
    reps = max(1, -(-24 // n_layers))

    def repeat(fn):
        def run():
            for _ in range(reps):
                fn()
        return run

    stream = torch.cuda.Stream(device=dev)
    graphs = {}
    kinds = [("step", repeat(step))]
    if not joint:
        kinds += [("split", repeat(split_only)), ("merge", repeat(merge_only))]
    for name, fn in kinds:
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
    n_replays = max(1, -(-args.steps // reps))
    t0 = time.perf_counter()
    for _ in range(n_replays):
        graphs["step"].replay()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    ms_per_step = elapsed * 1e3 / (n_replays * reps)
    _log(f"graph replay: {ms_per_step:.3f} ms per step")

    graph_ms = ms_per_step
    # Spread of the layer-step time: HIP events on the launch stream around
    # single replays of the step graph (at least 20), each replay's time per
    # layer-step; median and 10th / 90th percentiles.
    cur_stream = torch.cuda.current_stream(dev)
    spread = []
    for _ in range(max(20, n_replays)):
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(cur_stream)
        graphs["step"].replay()
        e1.record(cur_stream)
        e1.synchronize()
        spread.append(e0.elapsed_time(e1) * 1e3 / (reps * n_layers))
    spread.sort()

    def pct(q):
        return round(spread[min(len(spread) - 1, int(round(q * (len(spread) - 1))))], 3)

    # the headline is the faster of graph replay and eager issue
    timing_mode = "graph" if graph_ms <= eager_ms else "eager"
    ms_per_step = min(graph_ms, eager_ms)
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

    def timed(g, n):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        for _ in range(args.warmup):
            g.replay()
        e0.record(cur)
        for _ in range(n):
            g.replay()
        e1.record(cur)
        e1.synchronize()
        return e0.elapsed_time(e1) / (n * reps) / n_layers * 1e3  # us per kernel launch

    split_us = timed(graphs["step" if joint else "split"], n_replays)
    merge_us = timed(graphs["merge"], n_replays) if (S > 1 and not joint) else 0.0
    split_alg = float(np.mean(alg))     # one split launch processes one layer's batch
    achieved = split_alg / (split_us * 1e-6) / 1e9
    prof = _profile_record(config_tag(args.config), S, policy_name)
    traffic = None if prof is None else float(prof["hbm_bytes_per_dispatch"])
    # executed MFMA work of the split kernel (padded rows, two-term fp8 operands)
    fp8 = first.kv_dtype == "fp8"
    rows = first.num_q * first.heads
    # row blocks: 64 above 32 rows (the eight-wave kernels), else 16 or 48
    rblock = 64 if rows > 32 else 16 if rows <= 16 else 48
    exec_rows = rblock * -(-rows // rblock)
    terms = 2 if (fp8 and rows > 32) else 1
    # the FP8 kernel packs the second 32-row group of a 33..48-row block: both
    # terms share one 32-row operand, so that group executes one term's work
    packed = fp8 and 32 < rows <= 48
    row_terms = exec_rows * terms - (32 if packed else 0)
    positions = sum(int(l.seq_lens.sum().item()) for l in layers) / n_layers
    mfma_exec = positions * row_terms * 2 * (576 + 512)
    mfma_peak = 5000.0 if terms == 2 else 2500.0
    # The split kernel is bound by HBM below the MFMA ridge (peak flops / 8 TB/s)
    # and by the matrix cores above it (many heads, e.g. 96 heads at Q = 3).
    intensity = sum(flops) / bytes_per_step
    mfma_bound = intensity > mfma_peak * 1e12 / (HBM_PEAK_GBS * 1e9)
    split_flops = float(np.mean(flops))
    kname = ("split_kernel + merge_kernel (plan by length: timed together, as the layer-step)"
             if joint else "split_kernel")
    if mfma_bound:
        a_tf = split_flops / (split_us * 1e-6) / 1e12
        roofline = {"bound": "mfma", "kernel": kname, "achieved": round(a_tf, 2),
                    "peak": mfma_peak, "unit": "TFLOP/s", "frac": round(a_tf / mfma_peak, 4),
                    "traffic": None if traffic is None else round(traffic),
                    "intensity_flop_per_byte": round(intensity, 1)}
    else:
        roofline = {"bound": "hbm", "kernel": kname, "achieved": round(achieved, 2),
                    "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                    "traffic": None if traffic is None else round(traffic),
                    "intensity_flop_per_byte": round(intensity, 1)}
    # the same figure from the committed kernel trace of this build's split
    # kernel (rocprofv3 average duration), when there is one
    roofline["achieved_source"] = "HIP events on the launch stream around graph replays"
    if prof is not None:
        p_us = float(prof["split_avg_us"])
        if roofline["bound"] == "hbm":
            p_ach = split_alg / (p_us * 1e-6) / 1e9
        else:
            p_ach = split_flops / (p_us * 1e-6) / 1e12
        roofline["achieved_profile"] = round(p_ach, 2)
        roofline["frac_profile"] = round(p_ach / roofline["peak"], 4)
        roofline["profile_split_us"] = p_us

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
        "dtype": "fp8" if fp8 and terms == 2 else "bf16",
        "data": "synthetic",
        "us_per_layer_step": round(us_per_layer, 3),
        "us_per_layer_step_p10_p50_p90": [pct(0.1), pct(0.5), pct(0.9)],
        "hbm_frac": round(value / HBM_PEAK_GBS, 4),
        "config": {
            "workload": cfg["desc"],
            "name": args.config,
            "layers_per_step": n_layers,
            "batch": first.batch,
            "num_q_tokens": first.num_q,
            "heads": first.heads,
            "kv_dtype": "fp8_e4m3fn" if first.kv_dtype == "fp8" else "bf16",
            "mfma_operands": ("fp8 e4m3 (q and p each split into two fp8 terms), fp32 accumulate"
                              if terms == 2 else "bf16, fp32 accumulate"),
            "num_splits": S,
            "split_policy": policy_name,
            "algorithmic_bytes_per_step": int(bytes_per_step),
            "algorithmic_flops_per_step": int(sum(flops)),
            "mfma_tflops_algorithmic": round(sum(flops) / (ms_per_step * 1e-3) / 1e12, 2),
            "split_kernel_us": None if joint else round(split_us, 3),
            "merge_kernel_us": None if joint else round(merge_us, 3),
            "split_and_merge_us": round(split_us, 3) if joint else None,
            "timing": (f"{timing_mode} (faster of: HIP graph of {reps} step(s) "
                       f"({reps * n_layers} layer calls) replayed, {graph_ms:.4f} ms; eager "
                       f"issue of one call per layer, {eager_ms:.4f} ms); per-kernel times "
                       "from graphs of one kernel kind, HIP events on the launch stream"),
            "graph_ms_per_step": round(graph_ms, 4),
            "steps_timed": n_replays * reps,
            "eager_ms_per_step": round(eager_ms, 4),
        },
        "roofline": roofline,
        "mfma_roofline": {
            "kernel": kname,
            "executed_tflops": round(mfma_exec / (split_us * 1e-6) / 1e12, 2),
            "peak": mfma_peak,
            "unit": "TFLOP/s",
            "frac": round(mfma_exec / (split_us * 1e-6) / 1e12 / mfma_peak, 4),
            "note": f"executed = {exec_rows} padded rows x {terms} operand term(s)"
                    + (" (the second 32-row group packed: one term's work)" if packed else "")
                    + " x 2 x (576 + 512) flops per position",
        },
    }
    if joint:
        _log(f"split + merge (plan by length) {split_us:.2f} us per layer")
    else:
        _log(f"split {split_us:.2f} us, merge {merge_us:.2f} us per launch")
    line["config"]["kv_append"] = _append_leg(mla, first, dev, args.warmup, args.steps)
    if first.heads > 12 and first.heads % 12 == 0:
        line["config"]["rank_merge"] = _rank_merge(mla, first, dev, args.warmup, args.steps)
    if not args.no_peaks:
        peaks = _measured_peaks(dev)
        line["measured_peaks"] = peaks
        if roofline["bound"] == "hbm":
            best = max(peaks["hbm_read_gbs"], peaks["hbm_read_lds_gbs"])
            roofline["measured_peak"] = best
        else:
            best = peaks["mfma_fp8_tflops"] if fp8 else peaks["mfma_bf16_tflops"]
            roofline["measured_peak"] = best
        roofline["frac_of_measured"] = round(roofline["achieved"] / best, 4)
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = _cpu_baseline(layers, args.cpu_seconds)
    if args.copy_calibration:
        a = torch.ones(1 << 28, dtype=torch.float32, device=dev)   # 1 GiB
        b = torch.empty_like(a)
        for _ in range(3):
            torch.neg(a, out=b)
        torch.cuda.synchronize()
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
