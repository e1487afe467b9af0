"""GPU parity of attention over an FP8 E4M3 cache (pkv_attention_fp8)
against the oracle's decoded-cache attention: every finite code through the
kernel's widening (bit for bit), head dims, GQA groups, page sizes,
unsplit / split / balanced, a window, chunk queries (run as rows) and the
argument errors (the decode workload at full size is checked in
test_gpu_full_size.py)."""

import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_231_amd as pkv
from workloads import build_attention, decode_queries, fp8_caches
from tests._gpu import assert_close, make_plan

pytestmark = pytest.mark.gpu

KS, VS = 0.05, 0.04


def _run(wl, k8, v8, splits=1, window=0, plan=None, ks=KS, vs=VS):
    plan = plan if plan is not None else make_plan(wl)
    q = wl.tensors["q"].cuda()
    ws = pkv.Workspace.for_splits(wl.queries, wl.info["hq"], wl.info["dv"], splits)
    o = pkv.attention_fp8(plan, q, k8.cuda(), v8.cuda(), wl.scale, ks, vs, wl.causal,
                          workspace=ws, window=window)
    torch.cuda.synchronize()
    return o.double().cpu().numpy()


def _want(wl, k8, v8, window=0, ks=KS, vs=VS):
    return oracle.paged_attention_fp8(wl.tensors["q"], k8, v8, wl.lens, wl.qseq, wl.qpos,
                                      wl.table, wl.page_size, wl.scale, wl.causal, ks, vs,
                                      window=window)[0]


def _wl(dtype, hq, hkv, d, ps, lens, seed, queries=None, causal=True):
    need = sum(-(-L // ps) for L in lens)
    wl = build_attention("f8", seed, dtype, lens, queries or decode_queries(lens), hq, hkv, d, d,
                         ps, pool=need + 3, causal=causal, poison=True)
    k8, v8 = fp8_caches(wl, KS, VS)
    return wl, k8, v8


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float16])
def test_every_code_widens_exactly(dtype):
    """Two sequences of one token each; the value rows hold all 254 finite
    codes; one visible key, so out = decode(v) * v_scale exactly."""
    d, ps = 128, 16
    wl = build_attention("f8", 5, dtype, [1, 1], [(0, 0), (1, 0)], 1, 1, d, d, ps, pool=2)
    codes = np.arange(256, dtype=np.uint8)
    codes[codes == 0x7F], codes[codes == 0xFF] = 0x7E, 0xFE
    k8 = torch.zeros(2, ps, 1, d, dtype=torch.uint8)
    v8 = torch.zeros(2, ps, 1, d, dtype=torch.uint8)
    for s in range(2):
        v8[int(wl.table[s, 0]), 0, 0] = torch.as_tensor(codes[128 * s:128 * (s + 1)])
        k8[int(wl.table[s, 0]), 0, 0] = torch.as_tensor(codes[128 * (1 - s):128 * (2 - s)])
    got = _run(wl, k8, v8, vs=1.0)
    want = oracle.e4m3_decode(codes).reshape(2, 1, d)
    np.testing.assert_array_equal(got, want)


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float16])
@pytest.mark.parametrize("d", [64, 128, 256])
@pytest.mark.parametrize("g", [1, 4, 32])
def test_fp8_decode_shapes(dtype, d, g):
    lens = [1, 15, 16, 17, 100, 257, 1000]
    wl, k8, v8 = _wl(dtype, 2 * g, 2, d, 16, lens, seed=4000 + d + g)
    assert_close(_run(wl, k8, v8), _want(wl, k8, v8), dtype, f"fp8 d={d} g={g}")


@pytest.mark.parametrize("ps", [12, 64])
@pytest.mark.parametrize("splits", [1, 3, 0])
def test_fp8_page_sizes_splits(ps, splits):
    lens = [7, 300, 64, 1001, 2000]
    wl, k8, v8 = _wl(torch.bfloat16, 32, 8, 128, ps, lens, seed=4100 + ps)
    assert_close(_run(wl, k8, v8, splits=splits), _want(wl, k8, v8), torch.bfloat16,
                 f"fp8 ps={ps} splits={splits}")
    assert_close(_run(wl, k8, v8, splits=splits, window=100), _want(wl, k8, v8, window=100),
                 torch.bfloat16, f"fp8 window ps={ps} splits={splits}")


def test_fp8_chunk_queries_run_as_rows():
    chunks = [(77, 150), (0, 20)]
    dec = [33, 300]
    lens = [p + c for p, c in chunks] + dec
    queries = []
    for s, (p, c) in enumerate(chunks):
        queries += [(s, p + j) for j in range(c)]
    queries += [(len(chunks) + j, L - 1) for j, L in enumerate(dec)]
    wl = build_attention("f8", 4200, torch.bfloat16, lens, queries, 16, 4, 128, 128, 16,
                         poison=True)
    k8, v8 = fp8_caches(wl, KS, VS)
    for splits in (1, 0):
        assert_close(_run(wl, k8, v8, splits=splits), _want(wl, k8, v8), torch.bfloat16, "chunks")


def test_fp8_argument_errors():
    lens = [40, 3]
    wl, k8, v8 = _wl(torch.bfloat16, 8, 2, 128, 16, lens, seed=4300)
    plan = make_plan(wl)
    q, k8d, v8d = wl.tensors["q"].cuda(), k8.cuda(), v8.cuda()
    with pytest.raises(pkv.PKVError) as e:
        pkv.attention_fp8(plan, q.float(), k8d, v8d, wl.scale, KS, VS)
    assert e.value.code == "EINVAL"
    with pytest.raises(pkv.PKVError) as e:
        pkv.attention_fp8(plan, q, k8d, v8d, wl.scale, 0.0, VS)
    assert e.value.code == "EINVAL"
    wl48 = build_attention("f8", 4301, torch.bfloat16, lens, decode_queries(lens), 4, 2, 48, 48, 16)
    k48, v48 = fp8_caches(wl48, KS, VS)
    with pytest.raises(pkv.PKVError) as e:
        pkv.attention_fp8(make_plan(wl48), wl48.tensors["q"].cuda(), k48.cuda(), v48.cuda(),
                          wl48.scale, KS, VS)
    assert e.value.code == "ESHAPE"
