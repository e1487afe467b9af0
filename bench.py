"""Benchmark: paged decode KV-read throughput on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload 2]
                    [--no-cpu-baseline] [--kernel-only]

A step is one pass of the hot path over one batch: pkv.attention on the
bf16 GQA packed-decode workload (64 sequences, lengths ~U[512, 8192],
Hq=32, Hkv=8, D=128, page size 16) with the split count pkv.suggest_splits
chooses (split-KV partials, then the log-sum-exp merge).  Inputs are seeded
synthetic tensors resident in HBM before timing starts.  `value` is the
algorithmic K/V bytes of a step (every visible token row of every KV head
read once) divided by the step time.

The JSON line also carries:
  roofline      the dominant kernel (split decode) against the 8 TB/s HBM
                peak, timed with HIP events on the plan's stream;
  cpu_baseline  the float64 oracle timed on the host cores over a bounded
                sample of the same workload (first sequences), in GB/s.
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

HBM_PEAK_GBS = 8000.0
MFMA_BF16_PEAK_TFS = 2500.0


def _parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=50)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--workload", type=int, default=2, choices=[1, 2, 3, 4, 5])
    p.add_argument("--splits", type=int, default=0, help="0: pkv.suggest_splits")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-seconds", type=float, default=15.0)
    return p.parse_args()


def _traffic_from_profile(kernel_prefix: str):
    """HBM bytes per launch from the committed counter summary, if current."""
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "profiles",
                        "decode_bf16_gqa_64seq_traffic.json")
    try:
        with open(path) as f:
            rec = json.load(f)
        if rec.get("kernel_prefix") == kernel_prefix and rec.get("source_hash") == _kernel_hash():
            return rec.get("bytes_per_launch")
    except Exception:
        pass
    return None


def _kernel_hash():
    import hashlib
    here = os.path.dirname(os.path.abspath(__file__))
    h = hashlib.sha256()
    for name in ("rows_fast.hip", "rows_generic.hip", "device_common.h"):
        with open(os.path.join(here, "paged_kv_cache_231_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def cpu_baseline(wl, budget_s: float):
    """Oracle throughput on the first sequences of the workload (bounded)."""
    import oracle
    from workloads import attention_bytes
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:
        threads = 1
    t = wl.tensors
    done_bytes, elapsed, nq = 0, 0.0, 0
    order = np.argsort(wl.qseq, kind="stable")
    # take queries one at a time (cycling) until the time budget is spent
    start = time.perf_counter()
    for j in range(10 ** 9):
        i = order[j % len(order)]
        sl = np.array([i])
        sub = dict(q=t["q"][sl], lens=wl.lens, qseq=wl.qseq[sl], qpos=wl.qpos[sl])
        oracle.paged_attention(sub["q"], t["k"], t["v"], sub["lens"], sub["qseq"], sub["qpos"],
                               wl.table, wl.page_size, wl.scale, wl.causal)
        n_vis = (wl.qpos[i] + 1) if wl.causal else wl.lens[wl.qseq[i]]
        es = t["k"].element_size()
        done_bytes += int(n_vis) * wl.info["hkv"] * (wl.info["d"] + wl.info["dv"]) * es
        nq += 1
        elapsed = time.perf_counter() - start
        if elapsed >= budget_s:
            break
    _ = attention_bytes
    return {"value": done_bytes / elapsed / 1e9, "unit": "GB/s", "cores": int(threads),
            "kind": "oracle",
            "sample": f"{nq} query evaluations over the {wl.queries} decode queries "
                      f"(float64 numpy oracle, "
                      f"{elapsed:.1f} s, {done_bytes / 1e9:.3f} GB of K/V)"}


def main():
    args = _parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (got --gpus {args.gpus}): this build has no "
              "multi-GPU path; see the design notes for how it would shard.", file=sys.stderr)
        sys.exit(2)

    import torch
    import paged_kv_cache_231_amd as pkv
    import workloads

    torch.cuda.set_device(0)
    wl = workloads.config(args.workload)
    dev = {k: v.to("cuda") for k, v in wl.tensors.items()}
    stream = torch.cuda.current_stream()
    plan = pkv.Plan(wl.lens, wl.qseq, wl.qpos, wl.table, wl.page_size, wl.pages, stream=stream)
    if wl.kind == "attention":
        hq, hkv, d, dv = (wl.info[x] for x in ("hq", "hkv", "d", "dv"))
        splits = args.splits or pkv.suggest_splits(plan, hq, hkv, dv)
        ws = pkv.Workspace(wl.queries, hq, dv, splits) if splits > 1 else None
        out = torch.empty(wl.queries, hq, dv, dtype=wl.dtype, device="cuda")

        def step():
            pkv.attention(plan, dev["q"], dev["k"], dev["v"], wl.scale, wl.causal,
                          workspace=ws, out=out)
    else:
        h, r = wl.info["h"], wl.info["r"]
        splits = args.splits or pkv.suggest_splits(plan, h, 1, r)
        ws = pkv.Workspace(wl.queries, h, r, splits) if splits > 1 else None
        out = torch.empty(wl.queries, h, r, dtype=wl.dtype, device="cuda")

        def step():
            pkv.mla(plan, dev["q_abs"], dev["q_pos"], dev["latent"], dev["k_pos"], wl.scale,
                    wl.causal, workspace=ws, out=out)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    starts = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for j in range(args.steps):
        starts[j].record(stream)
        step()
        ends[j].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    gpu_ms = [s.elapsed_time(e) for s, e in zip(starts, ends)]
    ms_per_step = wall * 1e3 / args.steps
    avg_kernel_ms = float(np.mean(gpu_ms))

    nbytes = workloads.attention_bytes(wl)
    value = nbytes / (ms_per_step * 1e-3) / 1e9
    achieved = nbytes / (avg_kernel_ms * 1e-3) / 1e9
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                "traffic": _traffic_from_profile("rows_fast_kernel"),
                "kernel": "split decode + merge (one attention call)",
                "avg_launch_us": round(avg_kernel_ms * 1e3, 2)}
    line = {
        "metric": "paged decode KV-read GB/s (% of HBM peak)",
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": {torch.bfloat16: "bf16", torch.float16: "f16", torch.float32: "f32"}[wl.dtype],
        "data": "synthetic (seeded N(0,1) Q/K/V, shuffled pages)",
        "config": {"workload": wl.name, "queries": wl.queries, "splits": splits,
                   "kv_bytes_per_step": nbytes, "parallelism": "single GPU"},
        "roofline": roofline,
    }
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(wl, args.cpu_seconds)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
