"""Pins of the oracle's sliding window (``window_start`` and the ``window``
argument of ``paged_attention`` / ``paged_attention_split`` /
``attention_one``), CPU only:

- a window at least as long as the visible range changes nothing (bitwise);
- a one-key window returns that key's value exactly;
- torch SDPA in float64 with an explicit band mask (keys p - W < t <= p);
- a page-aligned window equals plain attention on a sequence whose first
  pages were dropped from the block table (no mask involved at all);
- split + merge with a window equals the unsplit window;
- planted off-by-one and wrong-end windows each fail one of these.
"""

import numpy as np
import pytest
import torch

import oracle
from oracle import reference as ref
from workloads import build_attention, decode_queries


def test_window_start_values():
    assert oracle.window_start(10, 0) == 0
    assert oracle.window_start(10, 3) == 7
    assert oracle.window_start(10, 10) == 0
    assert oracle.window_start(10, 50) == 0
    assert oracle.window_start(1, 1) == 0


def test_long_window_changes_nothing():
    lens = [50, 9, 130]
    wl = build_attention("w", 31, torch.float64, lens, decode_queries(lens), 4, 2, 16, 8, 8)
    args = (wl.lens, wl.qseq, wl.qpos, wl.table, wl.page_size, wl.scale, True)
    a, la = oracle.paged_attention(wl.tensors["q"], wl.tensors["k"], wl.tensors["v"], *args)
    b, lb = oracle.paged_attention(wl.tensors["q"], wl.tensors["k"], wl.tensors["v"], *args,
                                   window=130)
    np.testing.assert_array_equal(a, b)
    np.testing.assert_array_equal(la, lb)


def test_one_key_window_returns_that_value():
    lens = [50, 9]
    wl = build_attention("w", 32, torch.float64, lens, decode_queries(lens), 4, 2, 16, 8, 8)
    q, k, v = (wl.tensors[x] for x in "qkv")
    out, lse = oracle.paged_attention(q, k, v, wl.lens, wl.qseq, wl.qpos, wl.table,
                                      wl.page_size, wl.scale, True, window=1)
    for i, L in enumerate(lens):
        p = L - 1
        page, slot = wl.table[i][p // 8], p % 8
        for h in range(4):
            np.testing.assert_array_equal(out[i, h], v[page, slot, h // 2].numpy())
            x = wl.scale * float(q[i, h] @ k[page, slot, h // 2])
            assert lse[i, h] == pytest.approx(x, abs=1e-14)


@pytest.mark.parametrize("window", [1, 5, 17, 40])
def test_matches_torch_sdpa_with_a_band_mask(window):
    """A chunk of 9 queries at positions 23..31 of one sequence: key t is
    visible to the query at p when p - window < t <= p."""
    L, ps, H, D = 32, 8, 3, 16
    wl = build_attention("w", 33, torch.float64, [L], [(0, 23 + j) for j in range(9)],
                         H, H, D, D, ps, pool=6)
    q, k, v = (wl.tensors[x] for x in "qkv")
    out, _ = oracle.paged_attention(q, k, v, wl.lens, wl.qseq, wl.qpos, wl.table, ps,
                                    wl.scale, True, window=window)
    pages = torch.as_tensor(wl.table[0, :L // ps])
    kc = k[pages].reshape(L, H, D).permute(1, 0, 2).contiguous()
    vc = v[pages].reshape(L, H, D).permute(1, 0, 2).contiguous()
    qc = q.permute(1, 0, 2).contiguous()
    t = torch.arange(L)[None, :]
    p = torch.as_tensor(wl.qpos)[:, None]
    mask = (t <= p) & (t > p - window)
    want = torch.nn.functional.scaled_dot_product_attention(qc, kc, vc, attn_mask=mask,
                                                            scale=wl.scale).permute(1, 0, 2)
    np.testing.assert_allclose(out, want.numpy(), rtol=0, atol=1e-12)


@pytest.mark.parametrize("causal", [True, False])
def test_page_aligned_window_equals_dropped_pages(causal):
    """A window that starts on a page boundary gives, bit for bit, the plain
    attention of a sequence whose block table starts at that page."""
    ps = 8
    lens = [64, 40]
    wl = build_attention("w", 34, torch.float64, lens, decode_queries(lens), 4, 2, 16, 8, ps)
    q, k, v = (wl.tensors[x] for x in "qkv")
    window = 24  # 3 pages: starts at 40 (page 5) and at 16 (page 2)
    out, lse = oracle.paged_attention(q, k, v, wl.lens, wl.qseq, wl.qpos, wl.table, ps,
                                      wl.scale, causal, window=window)
    for s, L in enumerate(lens):
        drop = (L - window) // ps
        table = wl.table[s:s + 1, drop:]
        o2, l2 = oracle.paged_attention(q[s:s + 1], k, v, [L - drop * ps], [0],
                                        [L - drop * ps - 1], table, ps, wl.scale, causal)
        np.testing.assert_array_equal(out[s], o2[0])
        np.testing.assert_array_equal(lse[s], l2[0])


@pytest.mark.parametrize("splits", [2, 3, 8])
def test_split_with_window_equals_unsplit(splits):
    lens = [64, 40, 5]
    wl = build_attention("w", 35, torch.float64, lens, decode_queries(lens), 4, 2, 16, 8, 8)
    args = (wl.tensors["q"], wl.tensors["k"], wl.tensors["v"], wl.lens, wl.qseq, wl.qpos,
            wl.table, wl.page_size, wl.scale, True)
    a, la = oracle.paged_attention(*args, window=21)
    b, lb = oracle.paged_attention_split(*args, splits, window=21)
    np.testing.assert_allclose(b, a, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(lb, la, rtol=1e-12, atol=1e-13)
    for i in range(len(lens)):
        for h in (0, 3):
            o1, l1 = oracle.attention_one(*args, i, h, window=21)
            np.testing.assert_allclose(o1, a[i, h], rtol=1e-12, atol=1e-13)


def _pins():
    """The window pins as callables, for the planted-mistake check."""
    return [test_one_key_window_returns_that_value,
            lambda: test_matches_torch_sdpa_with_a_band_mask(5),
            lambda: test_page_aligned_window_equals_dropped_pages(True)]


@pytest.mark.parametrize("planted", [
    lambda n, w: max(0, n - w - 1) if w > 0 else 0,   # one key too many
    lambda n, w: max(0, n - w + 1) if w > 0 else 0,   # one key too few
    lambda n, w: 0,                                   # the window ignored
])
def test_planted_window_mistakes_trip_a_pin(planted, monkeypatch):
    monkeypatch.setattr(ref, "window_start", planted)
    failed = 0
    for pin in _pins():
        try:
            pin()
        except AssertionError:
            failed += 1
    assert failed > 0
