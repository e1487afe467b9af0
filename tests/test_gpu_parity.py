"""GPU parity: the HIP kernels through the C ABI against the float64 oracle.

Small cases compare every output element; every cache slot no query may see
is NaN (poisoned), so a kernel that reads one fails.  Tolerances: max abs
error 1e-5 for f32, 1.5e-2 for f16/bf16 (f32 accumulation).
"""

import numpy as np
import pytest
import torch

import paged_kv_cache_231_amd as pkv
from workloads import build_attention, build_mla, decode_queries, config
from tests._gpu import assert_close, expected, make_plan, run, to_dev

pytestmark = pytest.mark.gpu

DTYPES = [torch.float32, torch.float16, torch.bfloat16]


def _decode_wl(dtype, hq, hkv, d, dv, ps, lens, seed, causal=True, pool_extra=3):
    need = sum(-(-L // ps) for L in lens)
    return build_attention("t", seed, dtype, lens, decode_queries(lens), hq, hkv, d, dv, ps,
                           pool=need + pool_extra, causal=causal, poison=True)


def test_config1_full_parity():
    wl = config(1, poison=True)
    got = run(wl)
    assert_close(got, expected(wl), wl.dtype, "config 1")


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("d", [64, 128, 256])
@pytest.mark.parametrize("g", [1, 4, 8, 16])
def test_decode_fast_shapes(dtype, d, g):
    hkv = 2
    lens = [1, 15, 16, 17, 100, 257, 33]
    wl = _decode_wl(dtype, hkv * g, hkv, d, d, 16, lens, seed=100 + d + g)
    assert_close(run(wl), expected(wl), dtype, f"decode d={d} g={g}")


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("splits", [2, 3, 7, 64])
def test_decode_split_matches_oracle(dtype, splits):
    lens = [5, 64, 65, 300, 1000, 129]
    wl = _decode_wl(dtype, 8, 2, 128, 128, 16, lens, seed=7 + splits)
    want = expected(wl)
    assert_close(run(wl, splits=splits), want, dtype, f"split {splits}")


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("ps", [1, 5, 64])
def test_generic_shapes(dtype, ps):
    """Head dims with no specialised kernel (48 / 80) and odd page sizes."""
    lens = [1, 7, 40, 130]
    wl = _decode_wl(dtype, 6, 3, 48, 80, ps, lens, seed=300 + ps)
    assert_close(run(wl), expected(wl), dtype, "generic")
    assert_close(run(wl, splits=3), expected(wl), dtype, "generic split")


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("causal", [True, False])
def test_mixed_prefill_and_decode(dtype, causal):
    """Chunks at absolute positions after cached prefixes, plus decode rows."""
    priors = [0, 37, 100]
    chunk = [40, 9, 130]
    dec = [50, 16, 1]
    lens = [p + c for p, c in zip(priors, chunk)] + dec
    queries = []
    for s, (p, c) in enumerate(zip(priors, chunk)):
        queries += [(s, p + j) for j in range(c)]
    queries += [(3 + j, L - 1) for j, L in enumerate(dec)]
    wl = build_attention("t", 17, dtype, lens, queries, 8, 2, 128, 128, 16, causal=causal,
                         poison=True)
    assert_close(run(wl), expected(wl), dtype, "mixed")
    assert_close(run(wl, splits=4), expected(wl), dtype, "mixed split")


@pytest.mark.parametrize("dtype", DTYPES)
def test_mla_small(dtype):
    lens = [1, 64, 200, 77]
    wl = build_mla("t", 23, dtype, lens, decode_queries(lens), 16, 64, 16, 16, poison=True)
    assert_close(run(wl), expected(wl), dtype, "mla")
    assert_close(run(wl, splits=5), expected(wl), dtype, "mla split")


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float16])
@pytest.mark.parametrize("h,ps", [(128, 64), (16, 16), (40, 5), (256, 1)])
def test_mla_latent512(dtype, h, ps):
    """The MFMA MLA kernel's shape (rank 512, position dim 64): ragged head
    groups, page sizes 1/5/16/64, lengths that end inside a key tile, with
    and without splits."""
    lens = [1, 31, 32, 33, 300, 1000]
    queries = decode_queries(lens) + [(4, 17), (5, 500)]
    wl = build_mla("mla512", 29 + h + ps, dtype, lens, queries, h, 512, 64, ps, poison=True)
    want = expected(wl)
    assert_close(run(wl), want, dtype, "mla512")
    assert_close(run(wl, splits=3), want, dtype, "mla512 split 3")
    assert_close(run(wl, splits=16), want, dtype, "mla512 split 16")


def test_kernel_timing_records_each_launch():
    """pkv_plan_timing: one record per kernel launch, on the call's stream."""
    wl = _decode_wl(torch.bfloat16, 16, 2, 128, 128, 16, [300, 77, 1000], seed=43)
    dev = to_dev(wl)
    plan = make_plan(wl)
    plan.timing(True)
    for _ in range(4):
        run(wl, splits=3, plan=plan, dev=dev)
    torch.cuda.synchronize()
    n_rows, ms_rows = plan.timing_read("rows")
    n_merge, ms_merge = plan.timing_read("merge")
    assert n_rows == 4 and n_merge == 4
    assert ms_rows > 0 and ms_merge > 0
    assert plan.timing_read("tiles") == (0, 0.0)
    plan.timing(False)
    run(wl, plan=plan, dev=dev)
    assert plan.timing_read("rows") == (0, 0.0)
    # pkv_plan_timing_select: only the selected kernel records; the events
    # come from the kernel's own dispatch, so the time is positive
    plan.timing(True, kernels=("rows",))
    for _ in range(2):
        run(wl, splits=3, plan=plan, dev=dev)
    n_rows, ms_rows = plan.timing_read("rows")
    assert n_rows == 2 and ms_rows > 0
    assert plan.timing_read("merge") == (0, 0.0)
    plan.timing(False)
    with pytest.raises(pkv.PKVError):
        pkv.check(pkv.lib().pkv_plan_timing_select(plan.handle, 1 << 5))


def test_tune_splits_picks_a_candidate_and_leaves_the_result():
    """pkv_tune_splits / pkv_tune_splits_mla: the chosen count is one of the
    candidates, and `out` holds a correct result afterwards."""
    wl = _decode_wl(torch.bfloat16, 32, 8, 128, 128, 16, [3000, 77, 1000, 4096], seed=47)
    dev = to_dev(wl)
    plan = make_plan(wl)
    out = torch.empty(wl.queries, 32, 128, dtype=torch.bfloat16, device="cuda")
    s = pkv.tune_splits(plan, dev["q"], dev["k"], dev["v"], wl.scale, wl.causal, out=out, reps=2)
    assert s in (0, 1, 2, 3, 4, 6, 8, 12, 16, 24, 32, 48, 64) and s <= wl.table_width
    assert_close(out.double().cpu().numpy(), expected(wl), torch.bfloat16, "tuned attention")
    lens = [700, 64]
    mw = build_mla("tune", 31, torch.bfloat16, lens, decode_queries(lens), 128, 512, 64, 64)
    mdev = to_dev(mw)
    mplan = make_plan(mw)
    mout = torch.empty(2, 128, 512, dtype=torch.bfloat16, device="cuda")
    ms = pkv.tune_splits_mla(mplan, mdev["q_abs"], mdev["q_pos"], mdev["latent"], mdev["k_pos"],
                             mw.scale, mw.causal, out=mout, reps=2)
    assert ms == 0 or 1 <= ms <= mw.table_width
    assert_close(mout.double().cpu().numpy(), expected(mw), torch.bfloat16, "tuned mla")


def test_page_permutation_is_bitwise_invariant():
    """Moving pages in the pool (same logical content) gives identical bits."""
    wl = _decode_wl(torch.bfloat16, 16, 2, 128, 128, 16, [300, 77, 1000], seed=41, pool_extra=0)
    a = run(wl)
    rng = np.random.default_rng(1)
    perm = rng.permutation(wl.pages)  # new physical id of every page
    k2, v2 = torch.empty_like(wl.tensors["k"]), torch.empty_like(wl.tensors["v"])
    k2[torch.as_tensor(perm)] = wl.tensors["k"]
    v2[torch.as_tensor(perm)] = wl.tensors["v"]
    wl.tensors = dict(q=wl.tensors["q"], k=k2, v=v2)
    wl.table = perm[wl.table]
    b = run(wl)
    np.testing.assert_array_equal(a, b)
    c = run(wl, splits=3)
    assert_close(c, a, torch.bfloat16, "split vs unsplit")


def test_empty_plan_launches_nothing():
    plan = pkv.Plan([10], [], [], np.array([[0]]), 16, 1)
    q = torch.empty(0, 4, 64, device="cuda")
    k = torch.zeros(1, 16, 4, 64, device="cuda")
    out = pkv.attention(plan, q, k, k.clone(), 0.125)
    assert out.shape == (0, 4, 64)


def test_validation_errors_launch_nothing():
    wl = _decode_wl(torch.bfloat16, 8, 2, 128, 128, 16, [40, 3], seed=5)
    dev = to_dev(wl)
    plan = make_plan(wl)
    out = torch.full((wl.queries, 8, 128), 7.0, dtype=torch.bfloat16, device="cuda")
    lib = pkv.lib()
    base = dict(plan=plan.handle, dt=2, q=dev["q"].data_ptr(), k=dev["k"].data_ptr(),
                v=dev["v"].data_ptr(), out=out.data_ptr(), hq=8, hkv=2, d=128, dv=128,
                scale=0.1, causal=1, ws=None, stream=None)

    def call(**kw):
        a = dict(base, **kw)
        return pkv.STATUS[lib.pkv_attention(*a.values())]

    assert call() == "OK"
    torch.cuda.synchronize()
    out.fill_(7.0)
    assert call(hq=7) == "ESHAPE"  # 7 % 2 != 0
    assert call(d=0) == "ESHAPE" and call(dv=1025) == "ESHAPE"
    assert call(scale=0.0) == "EINVAL" and call(scale=float("nan")) == "EINVAL"
    assert call(dt=9) == "EINVAL"
    assert call(out=dev["q"].data_ptr()) == "EINVAL"  # output overlaps q
    ws_bad = pkv.Workspace(wl.queries, 4, 128, 2)
    assert call(ws=ws_bad.handle) == "EWORKSPACE"
    s2 = torch.cuda.Stream()
    assert call(stream=s2.cuda_stream) == "EDEVICE"
    torch.cuda.synchronize()
    assert (out == 7.0).all(), "a rejected call wrote the output"
    with pytest.raises(pkv.PKVError):
        pkv.Workspace(wl.queries, 0, 128, 0)  # balanced, zero heads
    with pytest.raises(pkv.PKVError):
        pkv.Workspace(wl.queries, 8, 128, 257)
    ws_bal = pkv.Workspace(wl.queries, 4, 128, 0)
    assert lib.pkv_workspace_splits(ws_bal.handle) == 0
    assert call(ws=ws_bal.handle) == "EWORKSPACE"  # built for 4 heads


def test_rebind_and_set_word():
    lens = [40, 100]
    wl = _decode_wl(torch.bfloat16, 8, 2, 128, 128, 16, lens, seed=61, pool_extra=4)
    dev = to_dev(wl)
    plan = make_plan(wl)
    assert_close(run(wl, plan=plan, dev=dev), expected(wl), wl.dtype, "before")
    # shorter lengths, same shape: rebind the whole word array
    wl.lens = np.array([33, 90])
    wl.qpos = wl.lens - 1
    plan.rebind(wl.lens, wl.qseq, wl.qpos, wl.table)
    assert_close(run(wl, plan=plan, dev=dev), expected(wl), wl.dtype, "rebind")
    # one more token in sequence 0 via two memsets (length, then position)
    w = plan.words
    plan.set_word(16 + 0, 34)
    plan.set_word(16 + 2 + 2 + 0, 33)
    wl.lens = np.array([34, 90])
    wl.qpos = wl.lens - 1
    got = run(wl, plan=plan, dev=dev)
    assert_close(got, expected(wl), wl.dtype, "set_word")
    with pytest.raises(pkv.PKVError):
        plan.set_word(16 + 2 + 2 + 0, 34)  # position == length: invalid
    assert w is plan.words


def test_graph_capture_replays_with_new_lengths():
    """Capture once; change lengths, positions and the block table through the
    plan words between replays; every replay matches the oracle."""
    lens = [700, 90, 300]
    wl = _decode_wl(torch.bfloat16, 16, 4, 128, 128, 16, lens, seed=71, pool_extra=10)
    dev = to_dev(wl)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        plan = make_plan(wl, stream=s)
        ws = pkv.Workspace(wl.queries, 16, 128, 4, stream=s)
        out = torch.empty(wl.queries, 16, 128, dtype=torch.bfloat16, device="cuda")
        pkv.attention(plan, dev["q"], dev["k"], dev["v"], wl.scale, True, workspace=ws, out=out)
        s.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=s):
            pkv.attention(plan, dev["q"], dev["k"], dev["v"], wl.scale, True, workspace=ws,
                          out=out)
        rng = np.random.default_rng(3)
        for step in range(4):
            new_lens = np.array([int(rng.integers(1, L + 1)) for L in lens])
            table = wl.table.copy()
            if step == 2:
                # move logical page 0 of sequence 1 to a free pool page (same
                # content): the graph reads the new table from the plan words
                spare, old = wl.pages - 1, int(wl.table[1, 0])
                for name in ("k", "v"):
                    wl.tensors[name][spare] = wl.tensors[name][old]
                    dev[name][spare] = dev[name][old]
                    wl.tensors[name][old] = float("nan")
                    dev[name][old] = float("nan")
                table[1, 0] = spare
            plan.rebind(new_lens, wl.qseq, new_lens - 1, table)
            g.replay()
            s.synchronize()
            wl.lens, wl.qpos, wl.table = new_lens, new_lens - 1, table
            got = out.double().cpu().numpy()
            assert_close(got, expected(wl), wl.dtype, f"replay {step}")


def _prefill_wl(dtype, hq, hkv, d, ps, chunks, dec_lens, seed, causal=True):
    """Chunks (prior, length) of consecutive queries plus decode rows."""
    lens = [p + c for p, c in chunks] + list(dec_lens)
    queries = []
    for s, (p, c) in enumerate(chunks):
        queries += [(s, p + j) for j in range(c)]
    queries += [(len(chunks) + j, L - 1) for j, L in enumerate(dec_lens)]
    return build_attention("t", seed, dtype, lens, queries, hq, hkv, d, d, ps, causal=causal,
                           poison=True)


@pytest.mark.parametrize("dtype", [torch.float16, torch.bfloat16])
@pytest.mark.parametrize("g", [1, 3, 4, 8, 16])
@pytest.mark.parametrize("d", [64, 128])
def test_prefill_tiles_gqa(dtype, g, d):
    """Tiles of the chunked-prefill kernel: a 150-query chunk (tiles of 128
    and 22 queries) after 77 cached tokens, a 20-query chunk from position 0,
    and two decode rows."""
    hkv = 2
    wl = _prefill_wl(dtype, hkv * g, hkv, d, 16, [(77, 150), (0, 20)], [33, 300], seed=900 + g + d)
    assert_close(run(wl), expected(wl), dtype, f"prefill g={g} d={d}")


@pytest.mark.parametrize("g", [32, 48, 128])
@pytest.mark.parametrize("d", [64, 128])
def test_prefill_tiles_wide_groups(g, d):
    """Groups of 32 to 128 q heads per KV head: a block's 128 q-rows are 4,
    2 (48 heads: 96 rows, the rest of the block idle) or 1 query, so a
    150-query tile spreads over up to 128 blocks."""
    wl = _prefill_wl(torch.bfloat16, g, 1, d, 16, [(77, 150), (0, 20)], [33, 300], seed=1900 + g + d)
    assert_close(run(wl), expected(wl), torch.bfloat16, f"prefill g={g} d={d}")


def test_prefill_groups_past_the_tile_limit_run_as_rows():
    """More than 128 q heads per KV head do not fit one block's q-rows: such
    chunk queries run on the per-query kernels, with the same results."""
    wl = _prefill_wl(torch.bfloat16, 192, 1, 64, 16, [(40, 24)], [9], seed=1990)
    dev = to_dev(wl)
    plan = make_plan(wl)
    assert plan.n_tiles > 0
    plan.timing(True)
    got = run(wl, plan=plan, dev=dev)
    assert plan.timing_read("tiles")[0] == 0 and plan.timing_read("rows")[0] == 1
    plan.timing(False)
    assert_close(got, expected(wl), torch.bfloat16, "prefill g=192 as rows")


@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("ps", [1, 5, 64])
def test_prefill_tiles_page_sizes(causal, ps):
    """Odd page sizes; with ps=1 the 1200-token prior needs more block-table
    entries than the kernel caches in LDS."""
    wl = _prefill_wl(torch.bfloat16, 8, 2, 128, ps, [(1200, 40), (3, 129)], [7], seed=950 + ps,
                     causal=causal)
    assert_close(run(wl), expected(wl), torch.bfloat16, f"prefill ps={ps}")
    assert_close(run(wl, splits=3), expected(wl), torch.bfloat16, f"prefill ps={ps} split")


def test_prefill_tiles_long_table():
    """A chunk behind a 16,600-token prior at page size 16: its block-table
    row (over 1,040 pages) is longer than the kernel's LDS copy, so whole
    tiles take their pages from the plan words directly and the last, partial
    tile reads entries past the copy one by one."""
    wl = _prefill_wl(torch.bfloat16, 8, 2, 128, 16, [(16600, 45)], [5], seed=977)
    assert_close(run(wl), expected(wl), torch.bfloat16, "prefill long table")


def test_graph_capture_mixed_prefill_and_decode():
    """A plan with prefill tiles, decode rows and a split merge, captured once
    into a graph and replayed after rebinding shorter priors and lengths
    (tile order and table lookups change), with eager work in between: every
    replay equals an eager call bit for bit and the oracle within
    tolerance."""
    chunks = [(200, 40), (90, 24)]
    dec_lens = [500, 77, 1200]
    wl = _prefill_wl(torch.bfloat16, 32, 8, 128, 16, chunks, dec_lens, seed=97)
    dev = to_dev(wl)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        plan = make_plan(wl, stream=s)
        assert plan.n_tiles > 0 and plan.n_rows > 0
        ws = pkv.Workspace(wl.queries, 32, 128, 3, stream=s)
        out = torch.empty(wl.queries, 32, 128, dtype=torch.bfloat16, device="cuda")
        eager = torch.empty_like(out)
        pkv.attention(plan, dev["q"], dev["k"], dev["v"], wl.scale, True, workspace=ws, out=out)
        s.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=s):
            pkv.attention(plan, dev["q"], dev["k"], dev["v"], wl.scale, True, workspace=ws,
                          out=out)
        n_chunk = sum(c for _, c in chunks)
        for step in range(3):
            shift = 30 * step
            new_chunks = [(p - shift, c) for p, c in chunks]
            new_dec = [L - 7 * step for L in dec_lens]
            lens = np.array([p + c for p, c in new_chunks] + new_dec)
            qpos = np.concatenate([np.arange(p, p + c) for p, c in new_chunks] +
                                  [np.array(new_dec) - 1])
            plan.rebind(lens, wl.qseq, qpos, wl.table)
            g.replay()
            s.synchronize()
            got = out.double().cpu().numpy()
            # eager call on the same plan, then some unrelated eager work
            pkv.attention(plan, dev["q"], dev["k"], dev["v"], wl.scale, True, workspace=ws,
                          out=eager)
            s.synchronize()
            _ = (dev["q"] * 2).sum().item()
            np.testing.assert_array_equal(got, eager.double().cpu().numpy())
            wl.lens, wl.qpos = lens, qpos
            assert_close(got, expected(wl), wl.dtype, f"mixed replay {step}")
            assert qpos.shape[0] == n_chunk + len(dec_lens)
