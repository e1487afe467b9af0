"""Caches above 2^32 elements (the kernels address caches with 64-bit
offsets): every page the sequences use sits past element 2^32 of its cache
(bf16 K and V of 8.6 GB each, FP8 byte caches of 4.3 GB, an MLA latent of
8.6 GB), the rest of the pool is left unset but for page 0.  Decode rows
(unsplit, split, balanced), chunk queries on the tile kernel and MLA are
compared with the oracle run on a compact copy of the same pages."""

import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_231_amd as pkv
from workloads import build_attention, build_mla, decode_queries, fp8_caches
from tests._gpu import assert_close, expected

pytestmark = pytest.mark.gpu

U32 = 1 << 32


def _spread(cache, base, pool):
    """A device cache of `pool` pages holding the compact cache's page p at
    page base + p (page 0 zeroed, the others unset)."""
    big = torch.empty((pool,) + tuple(cache.shape[1:]), dtype=cache.dtype, device="cuda")
    big[0].zero_()
    big[base:base + cache.shape[0]] = cache.cuda()
    return big


def _plan(wl, base, pool):
    return pkv.Plan(wl.lens, wl.qseq, wl.qpos, wl.table + base, wl.page_size, pool)


def _mixed_queries(lens, chunk_seq, prior, c):
    q = [(s, n - 1) for s, n in enumerate(lens) if s != chunk_seq]
    return q + [(chunk_seq, prior + j) for j in range(c)]


@pytest.mark.parametrize("splits", [1, 3, 0])
def test_attention_pages_past_2_32_elements(splits):
    ps, hkv, d, g = 16, 8, 128, 4
    page_elems = ps * hkv * d
    lens = [700, 1500, 200 + 150, 33]
    queries = _mixed_queries(lens, 2, 200, 150)
    wl = build_attention("big", 9100, torch.bfloat16, lens, queries, hkv * g, hkv, d, d, ps,
                         poison=True)
    base = U32 // page_elems + 1  # first element of every used page is past 2^32
    pool = base + wl.pages
    assert base * page_elems >= U32
    k = _spread(wl.tensors["k"], base, pool)
    v = _spread(wl.tensors["v"], base, pool)
    plan = _plan(wl, base, pool)
    ws = pkv.Workspace.for_splits(wl.queries, hkv * g, d, splits)
    got = pkv.attention(plan, wl.tensors["q"].cuda(), k, v, wl.scale, wl.causal, workspace=ws)
    torch.cuda.synchronize()
    assert_close(got.double().cpu().numpy(), expected(wl), torch.bfloat16, f"big cache splits={splits}")
    del k, v
    torch.cuda.empty_cache()


def test_fp8_pages_past_2_32_bytes():
    ps, hkv, d, g = 16, 8, 128, 4
    ks, vs = 0.05, 0.04
    page_elems = ps * hkv * d
    lens = [900, 64, 100 + 130]
    queries = _mixed_queries(lens, 2, 100, 130)
    wl = build_attention("big8", 9200, torch.bfloat16, lens, queries, hkv * g, hkv, d, d, ps,
                         poison=True)
    k8, v8 = fp8_caches(wl, ks, vs)
    base = U32 // page_elems + 1
    pool = base + wl.pages
    bk, bv = _spread(k8, base, pool), _spread(v8, base, pool)
    plan = _plan(wl, base, pool)
    ws = pkv.Workspace.for_splits(wl.queries, hkv * g, d, 0)
    got = pkv.attention_fp8(plan, wl.tensors["q"].cuda(), bk, bv, wl.scale, ks, vs, wl.causal, workspace=ws)
    torch.cuda.synchronize()
    want = oracle.paged_attention_fp8(wl.tensors["q"], k8, v8, wl.lens, wl.qseq, wl.qpos, wl.table,
                                      wl.page_size, wl.scale, wl.causal, ks, vs)[0]
    assert_close(got.double().cpu().numpy(), want, torch.bfloat16, "big fp8 cache")
    del bk, bv
    torch.cuda.empty_cache()


@pytest.mark.parametrize("splits", [1, 0])
def test_mla_pages_past_2_32_elements(splits):
    ps, h, r, p = 64, 128, 512, 64
    lens = [3000, 40, 700]
    wl = build_mla("bigmla", 9300, torch.bfloat16, lens, decode_queries(lens), h, r, p, ps, poison=True)
    base = U32 // (ps * r) + 1
    pool = base + wl.pages
    lat = _spread(wl.tensors["latent"], base, pool)
    kp = _spread(wl.tensors["k_pos"], base, pool)
    plan = _plan(wl, base, pool)
    ws = pkv.Workspace.for_splits(wl.queries, h, r, splits)
    got = pkv.mla(plan, wl.tensors["q_abs"].cuda(), wl.tensors["q_pos"].cuda(), lat, kp, wl.scale,
                  wl.causal, workspace=ws)
    torch.cuda.synchronize()
    assert_close(got.double().cpu().numpy(), expected(wl), torch.bfloat16, f"big mla splits={splits}")
    del lat, kp
    torch.cuda.empty_cache()


def test_size_limits_launch_nothing():
    """Query and output tensors stay below 2^32 elements and a cache below
    2^63 bytes: both are refused with ERANGE before anything runs."""
    lib = pkv.lib()
    buf = torch.full((1 << 16,), 7.0, dtype=torch.bfloat16, device="cuda")
    ptr = buf.data_ptr()

    def call(plan, hq, hkv, d):
        return pkv.STATUS[lib.pkv_attention(plan.handle, 2, ptr, ptr, ptr, ptr, hq, hkv, d, d, 0.1, 1,
                                            None, None)]

    # 4097 queries x 1024 heads x 1024 dims: q and out above 2^32 elements
    n = 4097
    plan_q = pkv.Plan([n], [0] * n, list(range(n)), np.array([[0, 1]]), 4096, 2)
    assert call(plan_q, 1024, 1, 1024) == "ERANGE"
    # 2^32 - 1 pages of 4096 tokens x 1024 heads x 1024 dims: a cache of 2^66 bytes
    plan_k = pkv.Plan([1], [0], [0], np.array([[0]]), 4096, (1 << 32) - 1)
    assert call(plan_k, 1024, 1024, 1024) == "ERANGE"
    torch.cuda.synchronize()
    assert (buf == 7.0).all(), "a rejected call wrote memory"
