"""GPU parity of the balanced decode schedule (pkv_workspace_create_balanced):
the row queries' 16-key tiles cut into equal ranges, one per resident wave,
with the pieces cut by range boundaries merged on the device.  Small inputs
give one tile per wave (every long segment is cut into many pieces); larger
ones give several tiles per wave.  Tolerance 1.5e-2 for f16/bf16; unused
cache slots are NaN."""

import numpy as np
import pytest
import torch

import paged_kv_cache_231_amd as pkv
from workloads import build_attention, build_mla, decode_queries
from tests._gpu import assert_close, expected, make_plan, run, to_dev

pytestmark = pytest.mark.gpu


def _wl(dtype, hq, hkv, d, ps, lens, seed, causal=True, queries=None):
    need = sum(-(-L // ps) for L in lens)
    q = queries if queries is not None else decode_queries(lens)
    return build_attention("bal", seed, dtype, lens, q, hq, hkv, d, d, ps, pool=need + 3,
                           causal=causal, poison=True)


@pytest.mark.parametrize("dtype", [torch.float16, torch.bfloat16])
@pytest.mark.parametrize("d", [64, 128, 256])
@pytest.mark.parametrize("g", [1, 3, 4, 32])
def test_balanced_decode_shapes(dtype, d, g):
    """Ragged lengths (inside a tile, on a tile edge, one token), GQA groups
    of 1..32 q heads (two 16-head groups at 32)."""
    hkv = 2
    lens = [1, 15, 16, 17, 100, 257, 33, 2000]
    wl = _wl(dtype, hkv * g, hkv, d, 16, lens, seed=1000 + d + g)
    assert_close(run(wl, splits=0), expected(wl), dtype, f"balanced d={d} g={g}")


@pytest.mark.parametrize("ps", [12, 64, 32])
@pytest.mark.parametrize("causal", [True, False])
def test_balanced_page_sizes(ps, causal):
    """Page sizes that are not a power of two (tiles straddle pages) and
    larger pages; causal and full visibility."""
    lens = [5, 700, 64, 1300, 31]
    wl = _wl(torch.bfloat16, 32, 8, 128, ps, lens, seed=1100 + ps, causal=causal)
    assert_close(run(wl, splits=0), expected(wl), torch.bfloat16, f"balanced ps={ps}")


def test_balanced_many_tiles_per_wave():
    """About 63k tiles, some 20 per wave: wave ranges that start and end
    inside segments and segments wholly inside one range."""
    rng = np.random.default_rng(5)
    lens = [int(x) for x in rng.integers(300, 6000, size=40)]
    wl = _wl(torch.bfloat16, 32, 8, 128, 16, lens, seed=1200)
    assert_close(run(wl, splits=0), expected(wl), torch.bfloat16, "balanced 25k tiles")


@pytest.mark.parametrize("n_rows", [300, 512, 513, 700])
@pytest.mark.parametrize("causal", [True, False])
def test_balanced_many_row_queries(n_rows, causal):
    """Hundreds of row queries: ranges that start in any of the first eight
    64-query chunks (kept in registers from the counting pass) and, past 512
    rows, in chunks found by the two-level search (512 and 513 are the two
    sides of that boundary); some queries see one token.  Causal and full
    visibility (the causal count reads no length)."""
    rng = np.random.default_rng(1250 + n_rows)
    lens = [int(x) for x in rng.integers(1, 400, size=n_rows)]
    wl = _wl(torch.bfloat16, 8, 2, 64, 16, lens, seed=1250 + n_rows, causal=causal)
    assert_close(run(wl, splits=0), expected(wl), torch.bfloat16, f"balanced {n_rows} rows")


def test_balanced_mixed_prefill_and_decode():
    """Chunk queries go to the tile kernel, decode rows to the balanced
    schedule over the plan's row list."""
    chunks = [(77, 150), (0, 20)]
    dec = [33, 300, 1500, 9]
    lens = [p + c for p, c in chunks] + dec
    queries = []
    for s, (p, c) in enumerate(chunks):
        queries += [(s, p + j) for j in range(c)]
    queries += [(len(chunks) + j, L - 1) for j, L in enumerate(dec)]
    wl = build_attention("bal", 1300, torch.bfloat16, lens, queries, 16, 4, 128, 128, 16,
                         poison=True)
    assert_close(run(wl, splits=0), expected(wl), torch.bfloat16, "balanced mixed")


def test_balanced_workspace_falls_back_to_unsplit():
    """Calls the balanced kernels do not take (f32, head dim 48, MLA of rank
    64) run unsplit with a balanced workspace and stay correct."""
    lens = [40, 300, 7]
    wl = _wl(torch.float32, 8, 2, 128, 16, lens, seed=1400)
    assert_close(run(wl, splits=0), expected(wl), torch.float32, "f32 balanced ws")
    wl = build_attention("bal", 1401, torch.bfloat16, lens, decode_queries(lens), 6, 3, 48, 48, 16,
                         poison=True)
    assert_close(run(wl, splits=0), expected(wl), torch.bfloat16, "d=48 balanced ws")
    mw = build_mla("bal", 1402, torch.bfloat16, lens, decode_queries(lens), 16, 64, 16, 16,
                   poison=True)
    assert_close(run(mw, splits=0), expected(mw), torch.bfloat16, "mla rank 64 balanced ws")


def test_balanced_launches_and_reuse():
    """The balanced path is the row kernel and one merge per call; repeated
    calls on one workspace stay correct."""
    wl = _wl(torch.bfloat16, 16, 2, 128, 16, [300, 77, 1000], seed=1500)
    dev = to_dev(wl)
    plan = make_plan(wl)
    ws = pkv.Workspace(wl.queries, 16, 128, 0)
    plan.timing(True)
    want = expected(wl)
    for _ in range(3):
        out = pkv.attention(plan, dev["q"], dev["k"], dev["v"], wl.scale, wl.causal, workspace=ws)
        torch.cuda.synchronize()
        assert_close(out.double().cpu().numpy(), want, torch.bfloat16, "balanced repeat")
    assert plan.timing_read("rows")[0] == 3
    assert plan.timing_read("merge")[0] == 3
    plan.timing(False)


def test_balanced_graph_capture_replays_with_new_lengths():
    """Captured once; lengths change through the plan words between replays,
    so the tile prefix, the wave ranges and the cut pieces all move; every
    replay equals an eager call bit for bit and the oracle within
    tolerance."""
    lens = [1700, 90, 300, 2500, 16]
    wl = _wl(torch.bfloat16, 32, 8, 128, 16, lens, seed=1600)
    dev = to_dev(wl)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        plan = make_plan(wl, stream=s)
        ws = pkv.Workspace(wl.queries, 32, 128, 0, stream=s)
        out = torch.empty(wl.queries, 32, 128, dtype=torch.bfloat16, device="cuda")
        eager = torch.empty_like(out)
        pkv.attention(plan, dev["q"], dev["k"], dev["v"], wl.scale, True, workspace=ws, out=out)
        s.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=s):
            pkv.attention(plan, dev["q"], dev["k"], dev["v"], wl.scale, True, workspace=ws,
                          out=out)
        rng = np.random.default_rng(9)
        for step in range(4):
            new_lens = np.array([int(rng.integers(1, L + 1)) for L in lens])
            plan.rebind(new_lens, wl.qseq, new_lens - 1, wl.table)
            g.replay()
            s.synchronize()
            got = out.double().cpu().numpy()
            pkv.attention(plan, dev["q"], dev["k"], dev["v"], wl.scale, True, workspace=ws,
                          out=eager)
            s.synchronize()
            _ = (dev["q"] * 2).sum().item()
            np.testing.assert_array_equal(got, eager.double().cpu().numpy())
            wl.lens, wl.qpos = new_lens, new_lens - 1
            assert_close(got, expected(wl), wl.dtype, f"balanced replay {step}")
