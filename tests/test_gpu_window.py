"""GPU parity of the sliding window (pkv_attention_window) against the
oracle's windowed attention: windows shorter than a tile, on and off the
16-key grid, longer than the sequence; page sizes on and off the tile grid;
unsplit, split and balanced; chunk queries.  The benchmark workload at
full size is checked in test_gpu_full_size.py.  Tolerances as the other
parity tests; unused cache slots are NaN."""

import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_231_amd as pkv
from workloads import build_attention, decode_queries
from tests._gpu import assert_close, make_plan, to_dev

pytestmark = pytest.mark.gpu


def _run(wl, window, splits=1, plan=None, dev=None):
    dev = dev if dev is not None else to_dev(wl)
    plan = plan if plan is not None else make_plan(wl)
    ws = pkv.Workspace.for_splits(wl.queries, wl.info["hq"], wl.info["dv"], splits)
    o = pkv.attention(plan, dev["q"], dev["k"], dev["v"], wl.scale, wl.causal, workspace=ws,
                      window=window)
    torch.cuda.synchronize()
    return o.double().cpu().numpy()


def _want(wl, window):
    t = wl.tensors
    return oracle.paged_attention(t["q"], t["k"], t["v"], wl.lens, wl.qseq, wl.qpos, wl.table,
                                  wl.page_size, wl.scale, wl.causal, window=window)[0]


def _wl(dtype, hq, hkv, d, ps, lens, seed, queries=None, causal=True):
    need = sum(-(-L // ps) for L in lens)
    return build_attention("win", seed, dtype, lens, queries or decode_queries(lens), hq, hkv, d,
                           d, ps, pool=need + 3, causal=causal, poison=True)


WINDOWS = [1, 15, 16, 17, 100, 1 << 20]


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16, torch.float16])
@pytest.mark.parametrize("d", [64, 128, 256])
@pytest.mark.parametrize("g", [1, 4, 32])
def test_window_decode_shapes(dtype, d, g):
    lens = [1, 15, 16, 17, 40, 257, 1000]
    wl = _wl(dtype, 2 * g, 2, d, 16, lens, seed=3000 + d + g)
    for w in WINDOWS:
        assert_close(_run(wl, w), _want(wl, w), dtype, f"window {w} d={d} g={g}")


@pytest.mark.parametrize("ps", [12, 5, 64])
@pytest.mark.parametrize("causal", [True, False])
def test_window_page_sizes(ps, causal):
    lens = [7, 300, 64, 1001]
    wl = _wl(torch.bfloat16, 32, 8, 128, ps, lens, seed=3100 + ps, causal=causal)
    for w in (3, 33, 250):
        assert_close(_run(wl, w), _want(wl, w), torch.bfloat16, f"window {w} ps={ps}")


@pytest.mark.parametrize("splits", [3, 8, 0])
def test_window_split_and_balanced(splits):
    """Split parts wholly before the window are empty and skipped by the
    merge; the balanced schedule counts tiles from the window's first tile."""
    lens = [5, 700, 2000, 64, 1500]
    wl = _wl(torch.bfloat16, 32, 8, 128, 16, lens, seed=3200)
    for w in (1, 17, 300, 1024):
        assert_close(_run(wl, w, splits=splits), _want(wl, w), torch.bfloat16,
                     f"window {w} splits {splits}")


def _poison_outside_windows(wl, window):
    """NaN in every K/V cache slot that no query's window reaches (the pages
    in front of a sequence's earliest window start and the slots past its
    length; the workload already holds NaN in the latter)."""
    for s_ in range(wl.sequences):
        qs = np.flatnonzero(wl.qseq == s_)
        if qs.size == 0:
            continue
        starts = [oracle.window_start(oracle.visible_count(wl.lens, wl.qseq, wl.qpos, int(i), wl.causal),
                                      window) for i in qs]
        for t in range(min(starts)):
            page, slot = int(wl.table[s_, t // wl.page_size]), t % wl.page_size
            for name in ("k", "v"):
                wl.tensors[name][page, slot] = float("nan")
    return wl


@pytest.mark.parametrize("g,d,ps", [(4, 128, 16), (1, 128, 16), (8, 64, 16), (4, 128, 5)])
@pytest.mark.parametrize("causal", [True, False])
def test_window_chunk_queries_on_tiles(g, d, ps, causal):
    """Chunk queries under a window run on the tile kernel: windows inside
    one query block's span, a tile wide, across tiles and longer than the
    history, with the pages before every window poisoned with NaN (a block
    may not read them) and ragged tails; decode rows alongside."""
    chunks = [(77, 150), (0, 20), (1500, 200)]
    dec = [33, 300]
    lens = [p + c for p, c in chunks] + dec
    queries = []
    for s_, (p, c) in enumerate(chunks):
        queries += [(s_, p + j) for j in range(c)]
    queries += [(len(chunks) + j, L - 1) for j, L in enumerate(dec)]
    for w, splits in ((1, 1), (7, 0), (32, 1), (45, 3), (300, 0), (5000, 1)):
        wl = build_attention("win", 3300 + g + d + ps + w, torch.bfloat16, lens, queries, 2 * g, 2, d,
                             d, ps, causal=causal, poison=True)
        plan = make_plan(wl)
        assert plan.n_tiles > 0
        _poison_outside_windows(wl, w)
        assert_close(_run(wl, w, splits=splits, plan=plan), _want(wl, w), torch.bfloat16,
                     f"chunk window {w} g={g} d={d} ps={ps} causal={causal}")


def test_window_zero_is_attention():
    lens = [40, 300]
    wl = _wl(torch.bfloat16, 16, 4, 128, 16, lens, seed=3400)
    dev = to_dev(wl)
    plan = make_plan(wl)
    a = _run(wl, 0, plan=plan, dev=dev)
    b = pkv.attention(plan, dev["q"], dev["k"], dev["v"], wl.scale, wl.causal)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(a, b.double().cpu().numpy())
