"""GPU parity of the benchmark workloads at full size, every output element
against the float64 oracle.

Workloads 2 (64 decode sequences of 512..8192 tokens), 3 (4 x 131072 tokens,
split-KV) and 4 (8 chunks of 512 queries behind priors of 0..4096 tokens
plus 120 decode rows) are compared in full: in the launch the benchmark
times (the split count pkv.tune_splits measures fastest), with the balanced
schedule and with the heuristic's split count.  The FP8-cache and
sliding-window legs of the benchmark (workload 2 with E4M3 caches; workload 2
with a 1024-key window) are compared in full with the balanced schedule and
with 8 parts.  Workload 5 (MLA, 128 sequences of 1024..32768 tokens, 128
heads) is compared on every query for 8 heads spread over both 64-head
groups of the kernel's blocks, tuned and balanced.

The oracle results are computed once per workload and shared by the tests
of this module (about 30 s of float64 work on the host in total).
Tolerance 1.5e-2 for bf16 outputs."""

import functools

import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_231_amd as pkv
from workloads import config, fp8_caches
from tests._gpu import assert_close, make_plan, run, to_dev

pytestmark = pytest.mark.gpu

KS, VS = 0.05, 0.04              # FP8 cache scales of the benchmark leg
WINDOW = 1024                    # window of the benchmark leg
MLA_HEADS = [0, 17, 34, 51, 64, 85, 102, 127]


@functools.lru_cache(maxsize=None)
def _workload(n):
    return config(n)


@functools.lru_cache(maxsize=None)
def _want(n, variant="plain"):
    wl = _workload(n)
    t = wl.tensors
    args = (wl.lens, wl.qseq, wl.qpos, wl.table, wl.page_size, wl.scale, wl.causal)
    if variant == "plain":
        return oracle.paged_attention(t["q"], t["k"], t["v"], *args)[0]
    if variant == "window":
        return oracle.paged_attention(t["q"], t["k"], t["v"], *args, window=WINDOW)[0]
    if variant == "fp8":
        k8, v8 = fp8_caches(wl, KS, VS)
        return oracle.paged_attention_fp8(t["q"], k8, v8, *args, KS, VS)[0]
    assert variant == "mla8"
    return oracle.paged_mla(t["q_abs"][:, MLA_HEADS], t["q_pos"][:, MLA_HEADS], t["latent"],
                            t["k_pos"], *args)[0]


@pytest.mark.parametrize("n", [2, 3, 4])
def test_attention_every_element(n):
    wl = _workload(n)
    print(f"full size: workload {n}", flush=True)
    dev = to_dev(wl)
    plan = make_plan(wl)
    hq, hkv, dv = wl.info["hq"], wl.info["hkv"], wl.info["dv"]
    tuned = pkv.tune_splits(plan, dev["q"], dev["k"], dev["v"], wl.scale, wl.causal, reps=2)
    suggested = pkv.suggest_splits(plan, hq, hkv, dv)
    want = _want(n)
    for splits in sorted({tuned, 0, suggested}):
        got = run(wl, splits=splits, plan=plan, dev=dev)
        assert_close(got, want, wl.dtype, f"workload {n} splits={splits}")


@pytest.mark.parametrize("splits", [0, 8])
def test_window_every_element(splits):
    wl = _workload(2)
    dev = to_dev(wl)
    plan = make_plan(wl)
    ws = pkv.Workspace.for_splits(wl.queries, wl.info["hq"], wl.info["dv"], splits)
    got = pkv.attention(plan, dev["q"], dev["k"], dev["v"], wl.scale, wl.causal, workspace=ws,
                        window=WINDOW)
    torch.cuda.synchronize()
    assert_close(got.double().cpu().numpy(), _want(2, "window"), wl.dtype, f"window splits={splits}")


@pytest.mark.parametrize("splits", [0, 8])
def test_fp8_every_element(splits):
    wl = _workload(2)
    k8, v8 = fp8_caches(wl, KS, VS)
    plan = make_plan(wl)
    ws = pkv.Workspace.for_splits(wl.queries, wl.info["hq"], wl.info["dv"], splits)
    got = pkv.attention_fp8(plan, wl.tensors["q"].cuda(), k8.cuda(), v8.cuda(), wl.scale, KS, VS,
                            wl.causal, workspace=ws)
    torch.cuda.synchronize()
    assert_close(got.double().cpu().numpy(), _want(2, "fp8"), wl.dtype, f"fp8 splits={splits}")


def test_mla_every_query_eight_heads():
    wl = _workload(5)
    dev = to_dev(wl)
    plan = make_plan(wl)
    tuned = pkv.tune_splits_mla(plan, dev["q_abs"], dev["q_pos"], dev["latent"], dev["k_pos"],
                                wl.scale, wl.causal, reps=2)
    want = _want(5, "mla8")
    for splits in sorted({tuned, 0}):
        got = run(wl, splits=splits, plan=plan, dev=dev)
        assert np.isfinite(got).all()
        assert_close(got[:, MLA_HEADS], want, wl.dtype, f"mla splits={splits}")
