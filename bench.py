"""Benchmark: paged decode KV-read throughput and chunked-prefill MFMA rate on
one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload 2]
                    [--splits S] [--no-cpu-baseline] [--no-prefill]
    python bench.py --copy-probe      (plain device copy of known size, for
                                       calibrating HBM byte counters)

A step is one pass of the hot path over one batch: pkv.attention on the
bf16 GQA packed-decode workload (64 sequences, lengths ~U[512, 8192],
Hq=32, Hkv=8, D=128, page size 16) with the split count pkv.tune_splits
measures fastest before timing starts: split-KV partials, then the
log-sum-exp merge.  Inputs are seeded
synthetic tensors resident in HBM before timing starts.  `value` is the
algorithmic K/V bytes of a step (every visible token row of every KV head
read once) divided by the wall time per step.

The JSON line also carries:
  roofline      the dominant kernel (the decode kernel) against the 8 TB/s
                HBM peak; its duration is measured live over the timed steps
                with HIP events that the kernel's own dispatch records on its
                stream (pkv_plan_timing_select; only that kernel is timed
                there).  `traffic` is the HBM bytes per launch from the
                committed rocprofv3 counter summary when it was taken on the
                current kernel source, else null.
  kernel_breakdown
                every kernel of a step (decode, merge), timed the same way
                over a few more steps after the timed region.
  prefill       the chunked-prefill tile kernel on the mixed prefill + decode
                workload (8 chunks x 512 queries + 120 decode rows): useful
                FLOPs of the chunk queries / tile-kernel time, against the
                dense bf16 MFMA peak.
With --workload 4 (that mixed workload as the step) the roofline is the tile
kernel's FLOP rate against the MFMA peak and `value` is useful TFLOP/s per
step; with --workload 5 (MLA) the roofline is HBM with the MFMA fraction
beside it.
  prefill_window
                the same tile kernel with every query limited to its last
                1024 keys (useful FLOPs inside the windows).
  prefill_fp8   the same tile kernel over E4M3 K/V caches of the same
                workload (codes widened to bf16 on the way into LDS).
  append, window, fp8
                the cache append, sliding-window decode and FP8-cache decode
                legs (per-kernel HIP-event durations).
  decode_step   one captured graph of append + attention on the packed
                decode workload: replay and eager times per step.
  f32_decode, long_decode, mla
                the f32 MHA decode (launch-bound), the long-context split
                decode (4 x 131072) and the MLA decode workloads, each with
                its tuned launch: dominant-kernel time (dispatch events),
                merge time, whole-step time, HBM fraction, and for MLA the
                MFMA fraction too.
  cpu_baseline  the float64 oracle timed on the host cores over a bounded
                sample of the same workload, in GB/s.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

import numpy as np

HBM_PEAK_GBS = 8000.0
MFMA_BF16_PEAK_TFS = 2500.0
HERE = os.path.dirname(os.path.abspath(__file__))
TRAFFIC_SUMMARY = os.path.join(HERE, "profiles", "decode_bf16_gqa_64seq_hbm_traffic.md")
# sources of the dominant (decode) kernel: the traffic figure is only used
# while these are unchanged
DECODE_SOURCES = ("decode_mfma.hip", "balanced.h", "device_common.h", "mfma_common.h", "kernels.h")


def _parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=50)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--workload", type=int, default=2, choices=[1, 2, 3, 4, 5])
    p.add_argument("--splits", default="tune",
                   help="tune: measured choice (pkv.tune_splits, balanced schedule included); "
                        "suggest: pkv.suggest_splits; balanced: balanced workspace; N: N parts")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-seconds", type=float, default=15.0)
    p.add_argument("--no-prefill", action="store_true")
    p.add_argument("--prefill-steps", type=int, default=20)
    p.add_argument("--copy-probe", action="store_true")
    p.add_argument("--legs", default="all",
                   help="comma-separated extra legs to run (" + ",".join(LEGS) + "), or all")
    args = p.parse_args()
    args.legs = set(LEGS) if args.legs == "all" else set(x for x in args.legs.split(",") if x)
    unknown = args.legs - set(LEGS)
    if unknown:
        raise SystemExit(f"unknown legs: {sorted(unknown)}")
    return args


LEGS = ("prefill", "prefill_window", "prefill_fp8", "append", "window", "fp8", "decode_step",
        "f32_decode", "long_decode", "mla")


def _fixed_splits(arg: str) -> int:
    """'balanced' -> 0 (balanced workspace), else a part count >= 1."""
    if arg == "balanced":
        return 0
    n = int(arg)
    if n < 1:
        raise SystemExit("--splits takes tune, suggest, balanced or a count >= 1")
    return n


def decode_source_hash() -> str:
    h = hashlib.sha256()
    for name in DECODE_SOURCES:
        with open(os.path.join(HERE, "paged_kv_cache_231_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def traffic_from_summary():
    """HBM bytes per decode launch from the committed counter summary, if it
    was taken on the current decode kernel source."""
    try:
        with open(TRAFFIC_SUMMARY) as f:
            text = f.read()
    except OSError:
        return None
    src = re.search(r"^source_hash:\s*(\w+)", text, re.M)
    val = re.search(r"^hbm_bytes_per_launch:\s*(\d+)", text, re.M)
    if not src or not val or src.group(1) != decode_source_hash():
        return None
    return int(val.group(1))


def copy_probe(torch):
    """Plain device-to-device copies of 1 GiB: the reference for scaling the
    FETCH_SIZE / WRITE_SIZE counters to bytes."""
    n = 1 << 30
    src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_probe_bytes_read": n, "copy_probe_bytes_written": n, "launches": 5}),
          flush=True)


def cpu_baseline(wl, budget_s: float):
    """Oracle throughput on a bounded sample: decode queries one at a time
    (cycling through the batch) until the time budget is spent."""
    import oracle
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:
        threads = 1
    affinity = len(os.sched_getaffinity(0))
    t = wl.tensors
    done_bytes, nq = 0, 0
    order = np.argsort(wl.qseq, kind="stable")
    if wl.kind == "attention":
        es = t["k"].element_size()
        row_bytes = wl.info["hkv"] * (wl.info["d"] + wl.info["dv"]) * es
    else:  # MLA: one latent row and one position row per token
        es = t["latent"].element_size()
        row_bytes = (wl.info["r"] + wl.info["p"]) * es
    args = (wl.lens, None, None, wl.table, wl.page_size, wl.scale, wl.causal)
    start = time.perf_counter()
    elapsed = 0.0
    while elapsed < budget_s:
        i = order[nq % len(order)]
        sl = np.array([i])
        a = (args[0], wl.qseq[sl], wl.qpos[sl]) + args[3:]
        if wl.kind == "attention":
            oracle.paged_attention(t["q"][sl], t["k"], t["v"], *a)
        else:
            oracle.paged_mla(t["q_abs"][sl], t["q_pos"][sl], t["latent"], t["k_pos"], *a)
        done_bytes += int(wl.visible()[i]) * row_bytes
        nq += 1
        elapsed = time.perf_counter() - start
    return {"value": round(done_bytes / elapsed / 1e9, 4), "unit": "GB/s",
            "cores": int(min(threads, affinity)), "affinity_cores": int(affinity),
            "blas_threads": int(threads), "kind": "oracle",
            "sample": f"{nq} single-query oracle calls cycling over the {wl.queries} queries "
                      f"(float64 numpy, {elapsed:.1f} s, {done_bytes / 1e9:.3f} GB of cache rows)"}


def tile_query_flops(plan, wl, window: int = 0) -> int:
    """Useful FLOPs of the queries the tile kernel owns: every query that is
    not a decode row of the plan (plan words: header, lens, qseq, qpos, rows);
    under a window each query counts only the keys inside it."""
    words = plan.words
    R = int(words[7])
    S, Q = int(words[3]), int(words[2])
    rows_off = 16 + S + 2 * Q
    in_rows = np.zeros(Q, dtype=bool)
    in_rows[np.asarray(words[rows_off:rows_off + R], dtype=np.int64)] = True
    vis = wl.visible().astype(np.int64)
    if window:
        vis = np.minimum(vis, window)
    hq, d, dv = wl.info["hq"], wl.info["d"], wl.info["dv"]
    return int(vis[~in_rows].sum()) * hq * 2 * (d + dv)


def prefill_measure(torch, pkv, workloads, steps: int, window: int = 0, fp8=None):
    """Tile-kernel TFLOP/s on the mixed chunked-prefill workload (with
    ``window``: every query limited to its last ``window`` keys; with
    ``fp8`` = (k_scale, v_scale): over E4M3 caches of the same K/V)."""
    wl = workloads.config(4)
    dev = {k: v.to("cuda") for k, v in wl.tensors.items()}
    if fp8:
        k8, v8 = workloads.fp8_caches(wl, *fp8)
        dev["k"], dev["v"] = k8.to("cuda"), v8.to("cuda")
    stream = torch.cuda.current_stream()
    plan = pkv.Plan(wl.lens, wl.qseq, wl.qpos, wl.table, wl.page_size, wl.pages, stream=stream)
    hq, hkv, d, dv = (wl.info[x] for x in ("hq", "hkv", "d", "dv"))
    out = torch.empty(wl.queries, hq, dv, dtype=wl.dtype, device="cuda")
    if window or fp8:
        splits = 0
    else:
        splits = pkv.tune_splits(plan, dev["q"], dev["k"], dev["v"], wl.scale, wl.causal, out=out)
    ws = pkv.Workspace.for_splits(wl.queries, hq, dv, splits)

    def step():
        if fp8:
            pkv.attention_fp8(plan, dev["q"], dev["k"], dev["v"], wl.scale, *fp8, wl.causal,
                              workspace=ws, out=out, window=window)
        else:
            pkv.attention(plan, dev["q"], dev["k"], dev["v"], wl.scale, wl.causal, workspace=ws,
                          out=out, window=window)

    for _ in range(3):
        step()
    torch.cuda.synchronize()
    plan.timing(True)
    for _ in range(steps):
        step()
    torch.cuda.synchronize()
    n_t, ms_t = plan.timing_read("tiles")
    n_r, ms_r = plan.timing_read("rows")
    plan.timing(False)
    T = int(plan.words[8])
    flops = tile_query_flops(plan, wl, window)
    avg_t = ms_t / max(1, n_t)
    tfs = flops / (avg_t * 1e-3) / 1e12
    return {"value": round(tfs, 1), "unit": "TFLOP/s", "peak": MFMA_BF16_PEAK_TFS,
            "frac": round(tfs / MFMA_BF16_PEAK_TFS, 4), "kernel": "chunked-prefill tiles",
            "avg_launch_us": round(avg_t * 1e3, 2), "launches": n_t, "flops_per_launch": flops,
            "tiles": T, "decode_rows_us": round(ms_r / max(1, n_r) * 1e3, 2),
            "workload": wl.name + (f", window {window}" if window else "")
            + (", E4M3 K/V cache" if fp8 else "")}


def append_measure(torch, pkv, workloads, steps: int):
    """Cache-append GB/s on the mixed workload's plan: every one of its 4216
    queries stores its new K/V rows (read once, written once)."""
    wl = workloads.config(4)
    dev = {k: v.to("cuda") for k, v in wl.tensors.items() if k in ("k", "v")}
    stream = torch.cuda.current_stream()
    plan = pkv.Plan(wl.lens, wl.qseq, wl.qpos, wl.table, wl.page_size, wl.pages, stream=stream)
    hkv, d, dv = (wl.info[x] for x in ("hkv", "d", "dv"))
    nk = torch.randn(wl.queries, hkv, d, device="cuda").to(wl.dtype)
    nv = torch.randn(wl.queries, hkv, dv, device="cuda").to(wl.dtype)
    for _ in range(3):
        pkv.append(plan, nk, nv, dev["k"], dev["v"])
    torch.cuda.synchronize()
    plan.timing(True)
    for _ in range(steps):
        pkv.append(plan, nk, nv, dev["k"], dev["v"])
    torch.cuda.synchronize()
    n, ms = plan.timing_read("append")
    plan.timing(False)
    nbytes = 2 * (nk.numel() + nv.numel()) * nk.element_size()
    avg_us = ms / max(1, n) * 1e3
    gbs = nbytes / (avg_us * 1e-6) / 1e9
    return {"value": round(gbs, 1), "unit": "GB/s", "peak": HBM_PEAK_GBS,
            "frac": round(gbs / HBM_PEAK_GBS, 4), "kernel": "cache append",
            "avg_launch_us": round(avg_us, 2), "launches": n, "bytes_per_launch": nbytes,
            "workload": f"append of the {wl.queries} queries of: {wl.name}"}


def window_measure(torch, pkv, workloads, steps: int, window: int = 1024):
    """Sliding-window decode GB/s: the packed-decode workload with each query
    limited to its last ``window`` keys, balanced schedule; bytes = the K/V
    rows inside the windows, each read once."""
    wl = workloads.config(2)
    dev = {k: v.to("cuda") for k, v in wl.tensors.items()}
    stream = torch.cuda.current_stream()
    plan = pkv.Plan(wl.lens, wl.qseq, wl.qpos, wl.table, wl.page_size, wl.pages, stream=stream)
    hq, hkv, d, dv = (wl.info[x] for x in ("hq", "hkv", "d", "dv"))
    out = torch.empty(wl.queries, hq, dv, dtype=wl.dtype, device="cuda")
    ws = pkv.Workspace(wl.queries, hq, dv, 0)

    def step():
        pkv.attention(plan, dev["q"], dev["k"], dev["v"], wl.scale, wl.causal, workspace=ws,
                      out=out, window=window)

    for _ in range(3):
        step()
    torch.cuda.synchronize()
    plan.timing(True)
    for _ in range(steps):
        step()
    torch.cuda.synchronize()
    n, ms = plan.timing_read("rows")
    plan.timing(False)
    es = torch.empty((), dtype=wl.dtype).element_size()
    nbytes = int(np.minimum(wl.visible(), window).sum()) * hkv * (d + dv) * es
    avg_us = ms / max(1, n) * 1e3
    gbs = nbytes / (avg_us * 1e-6) / 1e9
    return {"value": round(gbs, 1), "unit": "GB/s", "peak": HBM_PEAK_GBS,
            "frac": round(gbs / HBM_PEAK_GBS, 4), "kernel": "split-KV decode, window",
            "window": window, "avg_launch_us": round(avg_us, 2), "launches": n,
            "bytes_per_launch": nbytes, "workload": f"{wl.name}, window {window}, balanced"}


def fp8_measure(torch, pkv, workloads, steps: int, k_scale: float = 0.05, v_scale: float = 0.04):
    """Decode over an FP8 E4M3 cache: the packed-decode workload with its K/V
    quantised to one byte per element, balanced schedule; bytes = the visible
    cache bytes (1 per element), each read once."""
    wl = workloads.config(2)
    k8, v8 = workloads.fp8_caches(wl, k_scale, v_scale)
    k8, v8 = k8.to("cuda"), v8.to("cuda")
    q = wl.tensors["q"].to("cuda")
    stream = torch.cuda.current_stream()
    plan = pkv.Plan(wl.lens, wl.qseq, wl.qpos, wl.table, wl.page_size, wl.pages, stream=stream)
    hq, hkv, d, dv = (wl.info[x] for x in ("hq", "hkv", "d", "dv"))
    out = torch.empty(wl.queries, hq, dv, dtype=wl.dtype, device="cuda")
    ws = pkv.Workspace(wl.queries, hq, dv, 0)

    def step():
        pkv.attention_fp8(plan, q, k8, v8, wl.scale, k_scale, v_scale, wl.causal, workspace=ws,
                          out=out)

    for _ in range(3):
        step()
    torch.cuda.synchronize()
    plan.timing(True)
    for _ in range(steps):
        step()
    torch.cuda.synchronize()
    n, ms = plan.timing_read("rows")
    plan.timing(False)
    nbytes = int(wl.visible().sum()) * hkv * (d + dv)
    avg_us = ms / max(1, n) * 1e3
    gbs = nbytes / (avg_us * 1e-6) / 1e9
    return {"value": round(gbs, 1), "unit": "GB/s", "peak": HBM_PEAK_GBS,
            "frac": round(gbs / HBM_PEAK_GBS, 4), "kernel": "split-KV decode, FP8 E4M3 cache",
            "avg_launch_us": round(avg_us, 2), "launches": n, "bytes_per_launch": nbytes,
            "workload": f"{wl.name}, K/V as FP8 E4M3 bytes, balanced"}


def decode_step_measure(torch, pkv, workloads, steps: int):
    """A captured decode step on the packed-decode workload: one graph holds
    the append of every sequence's new K/V row at its own position and the
    attention over the grown caches (balanced schedule).  Reported: the
    replay time per step, the same calls launched eagerly, the per-step
    time of a graph holding two steps (what one launch costs shows as the
    difference), and the step's
    bytes (K/V rows read by the attention, plus the append's reads and
    writes) per replay time against the HBM peak."""
    wl = workloads.config(2)
    dev = {k: v.to("cuda") for k, v in wl.tensors.items()}
    hq, hkv, d, dv = (wl.info[x] for x in ("hq", "hkv", "d", "dv"))
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        plan = pkv.Plan(wl.lens, wl.qseq, wl.qpos, wl.table, wl.page_size, wl.pages, stream=s)
        ws = pkv.Workspace(wl.queries, hq, dv, 0, stream=s)
        nk = torch.randn(wl.queries, hkv, d, device="cuda").to(wl.dtype)
        nv = torch.randn(wl.queries, hkv, dv, device="cuda").to(wl.dtype)
        out = torch.empty(wl.queries, hq, dv, dtype=wl.dtype, device="cuda")

        def step():
            pkv.append(plan, nk, nv, dev["k"], dev["v"])
            pkv.attention(plan, dev["q"], dev["k"], dev["v"], wl.scale, wl.causal, workspace=ws,
                          out=out)

        def timed(run):
            for _ in range(3):
                run()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(s)
            for _ in range(steps):
                run()
            e1.record(s)
            s.synchronize()
            return e0.elapsed_time(e1) / steps * 1e3

        eager_us = timed(step)
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=s):
            step()
        graph_us = timed(g.replay)
        # the same step captured twice into one graph: per-step time when
        # one launch carries two steps
        g2 = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g2, stream=s):
            step()
            step()
        graph2_us = timed(g2.replay) / 2
    nbytes = workloads.attention_bytes(wl) + 2 * (nk.numel() + nv.numel()) * nk.element_size()
    gbs = nbytes / (graph_us * 1e-6) / 1e9
    return {"value": round(gbs, 1), "unit": "GB/s", "peak": HBM_PEAK_GBS,
            "frac": round(gbs / HBM_PEAK_GBS, 4),
            "kernel": "captured decode step: cache append + split-KV decode + merge",
            "graph_us": round(graph_us, 2), "eager_us": round(eager_us, 2),
            "graph_two_steps_per_launch_us": round(graph2_us, 2),
            "bytes_per_step": nbytes, "workload": f"{wl.name}, one new token per sequence"}


def workload_leg(torch, pkv, workloads, n: int, steps: int):
    """One more workload as its own leg: the tuned launch (split count or the
    balanced schedule), the whole step timed with stream events, the
    dominant kernel (decode rows, or MLA) with its own dispatch-recorded
    events inside those steps, and the merge timed the same way after
    them.  HBM fraction from the algorithmic bytes; MLA also reports its
    FLOP rate against the MFMA peak."""
    wl = workloads.config(n)
    dev = {k: v.to("cuda") for k, v in wl.tensors.items()}
    stream = torch.cuda.current_stream()
    plan = pkv.Plan(wl.lens, wl.qseq, wl.qpos, wl.table, wl.page_size, wl.pages, stream=stream)
    if wl.kind == "attention":
        hq, dv = wl.info["hq"], wl.info["dv"]
        out = torch.empty(wl.queries, hq, dv, dtype=wl.dtype, device="cuda")
        splits = pkv.tune_splits(plan, dev["q"], dev["k"], dev["v"], wl.scale, wl.causal, out=out)
        ws = pkv.Workspace.for_splits(wl.queries, hq, dv, splits)
        main = "rows"

        def step():
            pkv.attention(plan, dev["q"], dev["k"], dev["v"], wl.scale, wl.causal, workspace=ws,
                          out=out)
    else:
        h, r = wl.info["h"], wl.info["r"]
        out = torch.empty(wl.queries, h, r, dtype=wl.dtype, device="cuda")
        splits = pkv.tune_splits_mla(plan, dev["q_abs"], dev["q_pos"], dev["latent"], dev["k_pos"],
                                     wl.scale, wl.causal, out=out)
        ws = pkv.Workspace.for_splits(wl.queries, h, r, splits)
        main = "mla"

        def step():
            pkv.mla(plan, dev["q_abs"], dev["q_pos"], dev["latent"], dev["k_pos"], wl.scale,
                    wl.causal, workspace=ws, out=out)

    for _ in range(3):
        step()
    torch.cuda.synchronize()
    plan.timing(True, kernels=(main,))
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(steps):
        step()
    e1.record(stream)
    torch.cuda.synchronize()
    step_us = e0.elapsed_time(e1) / steps * 1e3
    n_m, ms_m = plan.timing_read(main)
    plan.timing(True, kernels=("merge",))
    for _ in range(steps):
        step()
    torch.cuda.synchronize()
    n_g, ms_g = plan.timing_read("merge")
    plan.timing(False)
    kern_us = ms_m / max(1, n_m) * 1e3
    nbytes = workloads.attention_bytes(wl)
    gbs = nbytes / (kern_us * 1e-6) / 1e9
    leg = {"value": round(gbs, 1), "unit": "GB/s", "peak": HBM_PEAK_GBS,
           "frac": round(gbs / HBM_PEAK_GBS, 4),
           "kernel": {"rows": "split-KV decode", "mla": "MLA decode"}[main],
           "splits": "balanced" if splits == 0 else splits,
           "avg_launch_us": round(kern_us, 2), "launches": n_m,
           "merge_us": round(ms_g / n_g * 1e3, 2) if n_g else None,
           "step_us": round(step_us, 2),
           "step_gbs": round(nbytes / (step_us * 1e-6) / 1e9, 1),
           "bytes_per_launch": nbytes, "workload": wl.name}
    if main == "mla":
        flops = workloads.attention_flops(wl)
        tfs = flops / (kern_us * 1e-6) / 1e12
        leg.update({"mfma_achieved_tflops": round(tfs, 1),
                    "mfma_frac": round(tfs / MFMA_BF16_PEAK_TFS, 4),
                    "flops_per_launch": flops})
    return leg


def main():
    args = _parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (got --gpus {args.gpus}): this build has no "
              "multi-GPU path; the design notes describe how it would shard.", file=sys.stderr)
        sys.exit(2)

    import torch
    import paged_kv_cache_231_amd as pkv
    import workloads

    torch.cuda.set_device(0)
    if args.copy_probe:
        copy_probe(torch)
        return

    wl = workloads.config(args.workload)
    dev = {k: v.to("cuda") for k, v in wl.tensors.items()}
    stream = torch.cuda.current_stream()
    plan = pkv.Plan(wl.lens, wl.qseq, wl.qpos, wl.table, wl.page_size, wl.pages, stream=stream)
    if wl.kind == "attention":
        hq, hkv, d, dv = (wl.info[x] for x in ("hq", "hkv", "d", "dv"))
        out = torch.empty(wl.queries, hq, dv, dtype=wl.dtype, device="cuda")
        if args.splits == "tune":
            splits = pkv.tune_splits(plan, dev["q"], dev["k"], dev["v"], wl.scale, wl.causal, out=out)
        elif args.splits == "suggest":
            splits = pkv.suggest_splits(plan, hq, hkv, dv)
        else:
            splits = _fixed_splits(args.splits)
        ws = pkv.Workspace.for_splits(wl.queries, hq, dv, splits)
        main_kernel = "tiles" if wl.info.get("prefill_queries") else "rows"

        def step():
            pkv.attention(plan, dev["q"], dev["k"], dev["v"], wl.scale, wl.causal,
                          workspace=ws, out=out)
    else:
        h, r = wl.info["h"], wl.info["r"]
        out = torch.empty(wl.queries, h, r, dtype=wl.dtype, device="cuda")
        if args.splits == "tune":
            splits = pkv.tune_splits_mla(plan, dev["q_abs"], dev["q_pos"], dev["latent"],
                                         dev["k_pos"], wl.scale, wl.causal, out=out)
        elif args.splits == "suggest":
            splits = pkv.suggest_splits(plan, h, 1, r)
        else:
            splits = _fixed_splits(args.splits)
        ws = pkv.Workspace.for_splits(wl.queries, h, r, splits)
        main_kernel = "mla"

        def step():
            pkv.mla(plan, dev["q_abs"], dev["q_pos"], dev["latent"], dev["k_pos"], wl.scale,
                    wl.causal, workspace=ws, out=out)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # Inside the timed steps only the dominant kernel records its events (a
    # timed launch costs a few microseconds of dispatch overhead).
    plan.timing(True, kernels=(main_kernel,))
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    n_main, ms_main = plan.timing_read(main_kernel)
    plan.timing(False)
    if n_main == 0:
        sys.exit(f"the {main_kernel} kernel did not run in the timed steps")
    ms_per_step = wall * 1e3 / args.steps
    avg_main_us = round(ms_main / n_main * 1e3, 2)

    # Per-kernel breakdown from a few more steps after the timed region, with
    # every kernel timed.
    plan.timing(True)
    for _ in range(min(args.steps, 10)):
        step()
    torch.cuda.synchronize()
    kernels = {}
    for name in ("rows", "tiles", "mla", "merge"):
        n, ms = plan.timing_read(name)
        if n:
            kernels[name] = {"launches": n, "avg_us": round(ms / n * 1e3, 2)}
    plan.timing(False)

    nbytes = workloads.attention_bytes(wl)
    if main_kernel == "tiles":
        # a step led by chunk queries, which re-read the same K/V rows: its
        # rate is useful FLOPs per second
        value, unit = workloads.attention_flops(wl) / (ms_per_step * 1e-3) / 1e12, "TFLOP/s"
    else:
        value, unit = nbytes / (ms_per_step * 1e-3) / 1e9, "GB/s"
    achieved = nbytes / (avg_main_us * 1e-6) / 1e9
    traffic = traffic_from_summary() if args.workload == 2 and main_kernel == "rows" else None
    kernel_name = {"rows": "split-KV decode", "tiles": "chunked-prefill tiles",
                   "mla": "MLA decode", "merge": "split merge"}[main_kernel]
    if main_kernel == "tiles":
        # the chunk queries' attention is a dense contraction: MFMA-bound
        flops = tile_query_flops(plan, wl)
        tfs = flops / (avg_main_us * 1e-6) / 1e12
        roofline = {"bound": "mfma", "achieved": round(tfs, 1), "peak": MFMA_BF16_PEAK_TFS,
                    "unit": "TFLOP/s", "frac": round(tfs / MFMA_BF16_PEAK_TFS, 4),
                    "traffic": None, "kernel": kernel_name,
                    "algorithmic_flops_per_launch": flops, "avg_launch_us": avg_main_us}
    else:
        roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                    "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic,
                    "kernel": kernel_name,
                    "algorithmic_bytes_per_launch": nbytes, "avg_launch_us": avg_main_us}
        if main_kernel == "mla":
            # near the ridge point: the matrix-core fraction beside the HBM one
            flops = workloads.attention_flops(wl)
            tfs = flops / (avg_main_us * 1e-6) / 1e12
            roofline.update({"mfma_achieved_tflops": round(tfs, 1),
                             "mfma_frac": round(tfs / MFMA_BF16_PEAK_TFS, 4),
                             "algorithmic_flops_per_launch": flops})
    line = {
        "metric": "paged decode KV-read GB/s (% of HBM peak); chunked-prefill TFLOP/s (% MFMA)",
        "value": round(value, 1),
        "unit": unit,
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": {torch.bfloat16: "bf16", torch.float16: "f16", torch.float32: "f32"}[wl.dtype],
        "data": "synthetic (seeded N(0,1) Q/K/V, shuffled pages)",
        "config": {"workload": wl.name, "queries": wl.queries,
                   "splits": "balanced" if splits == 0 else splits,
                   "kv_bytes_per_step": nbytes, "parallelism": "single GPU"},
        "roofline": roofline,
        "kernel_breakdown": kernels,
    }
    if not args.no_prefill and wl.kind == "attention":
        ps, legs = args.prefill_steps, args.legs
        runs = (("prefill", lambda: prefill_measure(torch, pkv, workloads, ps)),
                ("prefill_window", lambda: prefill_measure(torch, pkv, workloads, ps, window=1024)),
                ("prefill_fp8", lambda: prefill_measure(torch, pkv, workloads, ps, fp8=(0.05, 0.04))),
                ("append", lambda: append_measure(torch, pkv, workloads, ps)),
                ("window", lambda: window_measure(torch, pkv, workloads, ps)),
                ("fp8", lambda: fp8_measure(torch, pkv, workloads, ps)),
                ("decode_step", lambda: decode_step_measure(torch, pkv, workloads, ps)))
        for name, run in runs:
            if name in legs:
                line[name] = run()
        # the other workloads, each as a leg of its own (never the one timed above)
        for name, n in (("f32_decode", 1), ("long_decode", 3), ("mla", 5)):
            if n != args.workload and name in legs:
                line[name] = workload_leg(torch, pkv, workloads, n, ps)
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(wl, args.cpu_seconds)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
