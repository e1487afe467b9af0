"""Pins of the float64 oracle against facts fixed outside the oracle itself.

Each test states what it pins and why a plausible mistake would fail it:
closed forms (single visible key, equal scores, two keys, causal one-hot
means), a library routine (torch SDPA in float64 with an explicit mask),
invariances the pages fix (physical page permutation, GQA = MHA with repeated
K/V, split count, MLA = attention on [latent; k_pos]) and a few planted
mistakes that must trip at least one pin.
"""

import math

import numpy as np
import pytest
import torch

import oracle
from oracle import reference as ref
from workloads import build_attention, build_mla, decode_queries

RTOL = 1e-12


def _contiguous_layout(lens, ps):
    """Identity-like table: pages of sequence 0 first, in order."""
    need = [-(-L // ps) for L in lens]
    w = max(need)
    table = np.zeros((len(lens), w), dtype=np.int64)
    o = 0
    for s, n in enumerate(need):
        table[s, :n] = np.arange(o, o + n)
        o += n
    return table, o


def _place(cache_shape, lens, table, ps, token_values):
    """Cache with logical token t of sequence s at table[s][t//ps], slot t%ps."""
    cache = np.zeros(cache_shape)
    for s, L in enumerate(lens):
        for t in range(L):
            cache[table[s][t // ps], t % ps] = token_values(s, t)
    return cache


# ---------------------------------------------------------------- closed forms

def test_single_visible_key_returns_its_value():
    """Causal query at position 0 sees one key: out = v_0 exactly (exp(0)=1)."""
    wl = build_attention("t", 11, torch.float64, [37], [(0, 0)], 4, 2, 16, 24, 8)
    q, k, v = (wl.tensors[x] for x in "qkv")
    out, lse = oracle.paged_attention(q, k, v, wl.lens, wl.qseq, wl.qpos, wl.table,
                                      wl.page_size, wl.scale, True)
    page = wl.table[0, 0]
    for h in range(4):
        np.testing.assert_array_equal(out[0, h], v[page, 0, h // 2].numpy())
        x0 = wl.scale * float(q[0, h].double() @ k[page, 0, h // 2].double())
        assert lse[0, h] == pytest.approx(x0, abs=1e-14)


def test_equal_scores_give_mean_of_visible_values():
    """q = 0 makes every score equal: out = mean of the visible V rows.
    V at logical token t is (t+1) * ones, so the mean over n tokens is (n+1)/2.
    """
    lens, ps = [29, 7, 64], 8
    rng = np.random.default_rng(5)
    need = sum(-(-L // ps) for L in lens)
    perm = rng.permutation(need + 3)
    table = np.zeros((3, 8), dtype=np.int64)
    o = 0
    for s, L in enumerate(lens):
        n = -(-L // ps)
        table[s, :n] = perm[o:o + n]
        o += n
    pool = need + 3
    v = _place((pool, ps, 1, 5), lens, table, ps, lambda s, t: t + 1.0)
    k = rng.standard_normal((pool, ps, 1, 4))
    q = np.zeros((4, 3, 4))
    qseq = np.array([0, 1, 2, 2])
    qpos = np.array([28, 6, 0, 40])
    for causal in (False, True):
        out, lse = oracle.paged_attention(q, k, v, np.array(lens), qseq, qpos, table,
                                          ps, 0.3, causal)
        for i in range(4):
            n = qpos[i] + 1 if causal else lens[qseq[i]]
            np.testing.assert_allclose(out[i], np.full((3, 5), (n + 1) / 2), rtol=RTOL)
            np.testing.assert_allclose(lse[i], math.log(n), rtol=RTOL)


def test_two_keys_closed_form():
    """n = 2 by hand: scale 0.5, q = (1, 0), k0 = (2, 0), k1 = (0, 1):
    x0 = 1, x1 = 0; out = sigma(1) v0 + sigma(-1) v1, lse = log(e + 1)."""
    ps = 1
    table = np.array([[3, 1]])
    k = np.zeros((4, 1, 1, 2))
    v = np.zeros((4, 1, 1, 3))
    k[3, 0, 0] = [2.0, 0.0]
    k[1, 0, 0] = [0.0, 1.0]
    v[3, 0, 0] = [1.0, -2.0, 4.0]
    v[1, 0, 0] = [3.0, 5.0, -1.0]
    q = np.array([[[1.0, 0.0]]])
    out, lse = oracle.paged_attention(q, k, v, np.array([2]), np.array([0]), np.array([1]),
                                      table, ps, 0.5, True)
    s1 = 1.0 / (1.0 + math.exp(-1.0))
    expect = s1 * np.array([1.0, -2.0, 4.0]) + (1 - s1) * np.array([3.0, 5.0, -1.0])
    np.testing.assert_allclose(out[0, 0], expect, rtol=1e-15, atol=1e-15)
    assert lse[0, 0] == pytest.approx(math.log(math.e + 1.0), abs=1e-15)


def test_causal_uses_absolute_positions():
    """A causal chunk query at absolute position p sees exactly positions 0..p.
    With q = 0 and V at token t = one-hot(t), out[d] = 1/(p+1) for d <= p, else 0.
    """
    L, ps = 12, 4
    lens = [L]
    table = np.array([[2, 0, 1]])
    v = _place((3, ps, 1, L), lens, table, ps, lambda s, t: np.eye(L)[t])
    k = np.random.default_rng(1).standard_normal((3, ps, 1, 3))
    positions = [5, 6, 7, 8, 9]  # a prefill chunk after 5 cached tokens
    q = np.zeros((len(positions), 2, 3))
    out, _ = oracle.paged_attention(q, k, v, np.array(lens), np.zeros(5, dtype=int),
                                    np.array(positions), table, ps, 1.0, True)
    for i, p in enumerate(positions):
        expect = np.where(np.arange(L) <= p, 1.0 / (p + 1), 0.0)
        np.testing.assert_allclose(out[i, 0], expect, rtol=RTOL, atol=1e-15)
        np.testing.assert_allclose(out[i, 1], expect, rtol=RTOL, atol=1e-15)


# ------------------------------------------------------------ library routine

def _sdpa_reference(qc, kc, vc, qpos, causal, scale):
    """torch SDPA in float64 on contiguous [H, T, D] tensors, explicit mask."""
    n_keys = kc.shape[1]
    mask = torch.ones(qc.shape[1], n_keys, dtype=torch.bool)
    if causal:
        mask = torch.arange(n_keys)[None, :] <= torch.as_tensor(qpos)[:, None]
    return torch.nn.functional.scaled_dot_product_attention(
        qc, kc, vc, attn_mask=mask, scale=scale)


@pytest.mark.parametrize("causal", [True, False])
def test_matches_torch_sdpa_on_a_chunk(causal):
    """One sequence, a chunk of 9 queries after 23 cached tokens, MHA."""
    L, ps, H, D = 32, 8, 3, 16
    wl = build_attention("t", 21, torch.float64, [L], [(0, 23 + j) for j in range(9)],
                         H, H, D, D, ps, pool=7)
    q, k, v = (wl.tensors[x] for x in "qkv")
    out, _ = oracle.paged_attention(q, k, v, wl.lens, wl.qseq, wl.qpos, wl.table, ps,
                                    wl.scale, causal)
    # contiguous copies built with torch indexing (independent of the oracle)
    pages = torch.as_tensor(wl.table[0, :L // ps])
    kc = k[pages].reshape(L, H, D).permute(1, 0, 2).contiguous()
    vc = v[pages].reshape(L, H, D).permute(1, 0, 2).contiguous()
    qc = q.permute(1, 0, 2).contiguous()
    ref_out = _sdpa_reference(qc, kc, vc, wl.qpos, causal, wl.scale).permute(1, 0, 2)
    np.testing.assert_allclose(out, ref_out.numpy(), rtol=0, atol=1e-12)


# ------------------------------------------------------------- invariances

def test_paged_equals_contiguous_bitwise():
    """Physical page order does not change the result: the same logical K/V
    placed in an identity layout and in a shuffled pool give identical bits."""
    lens, ps, hq, hkv, d = [19, 40, 8], 8, 4, 2, 8
    rng = np.random.default_rng(3)
    kt = {(s, t): rng.standard_normal((hkv, d)) for s, L in enumerate(lens) for t in range(L)}
    vt = {(s, t): rng.standard_normal((hkv, d)) for s, L in enumerate(lens) for t in range(L)}
    q = rng.standard_normal((5, hq, d))
    qseq, qpos = np.array([0, 1, 1, 2, 1]), np.array([18, 3, 39, 7, 20])
    t_id, n_id = _contiguous_layout(lens, ps)
    perm = rng.permutation(n_id + 4)
    t_sh = np.where(t_id >= 0, perm[t_id], 0)
    outs = []
    for table, pool in ((t_id, n_id), (t_sh, n_id + 4)):
        k = _place((pool, ps, hkv, d), lens, table, ps, lambda s, t: kt[(s, t)])
        v = _place((pool, ps, hkv, d), lens, table, ps, lambda s, t: vt[(s, t)])
        outs.append(oracle.paged_attention(q, k, v, np.array(lens), qseq, qpos, table,
                                           ps, 0.25, True))
    np.testing.assert_array_equal(outs[0][0], outs[1][0])
    np.testing.assert_array_equal(outs[0][1], outs[1][1])


def test_gqa_equals_mha_with_repeated_kv():
    """GQA = MHA on K/V whose heads are repeated G times (oracle only)."""
    wl = build_attention("t", 31, torch.float64, [50, 17], [(0, 49), (1, 16), (0, 20)],
                         8, 2, 16, 12, 8)
    q, k, v = (wl.tensors[x] for x in "qkv")
    args = (wl.lens, wl.qseq, wl.qpos, wl.table, wl.page_size, wl.scale, True)
    gqa, _ = oracle.paged_attention(q, k, v, *args)
    mha, _ = oracle.paged_attention(q, k.repeat_interleave(4, dim=2),
                                    v.repeat_interleave(4, dim=2), *args)
    np.testing.assert_allclose(gqa, mha, rtol=RTOL, atol=1e-14)


def test_gqa_head_map_is_contiguous_groups():
    """KV head g serves q heads g*G .. g*G+G-1: with V of KV head g equal to
    g + 1 everywhere, out[:, h] = h // G + 1 (a map h % Hkv would fail)."""
    hq, hkv = 12, 3
    wl = build_attention("t", 41, torch.float64, [30], [(0, 29)], hq, hkv, 8, 4, 8)
    v = torch.zeros_like(wl.tensors["v"])
    for g in range(hkv):
        v[:, :, g, :] = g + 1.0
    out, _ = oracle.paged_attention(wl.tensors["q"], wl.tensors["k"], v, wl.lens, wl.qseq,
                                    wl.qpos, wl.table, wl.page_size, wl.scale, True)
    for h in range(hq):
        np.testing.assert_allclose(out[0, h], h // (hq // hkv) + 1.0, rtol=1e-14)


@pytest.mark.parametrize("splits", [1, 2, 3, 7, 64])
def test_split_merge_equals_unsplit(splits):
    """Split + log-sum-exp merge equals the unsplit result (empty parts too:
    with 64 parts over a 14-page table most parts are empty)."""
    lens = [100, 13, 60]
    wl = build_attention("t", 51, torch.float64, lens,
                         decode_queries(lens) + [(0, 40), (2, 3)], 6, 3, 16, 16, 8)
    q, k, v = (wl.tensors[x] for x in "qkv")
    args = (wl.lens, wl.qseq, wl.qpos, wl.table, wl.page_size, wl.scale, True)
    base, base_lse = oracle.paged_attention(q, k, v, *args)
    out, lse = ref.paged_attention_split(q, k, v, *args, splits=splits)
    np.testing.assert_allclose(out, base, rtol=RTOL, atol=1e-13)
    np.testing.assert_allclose(lse, base_lse, rtol=RTOL, atol=1e-13)


def test_merge_closed_form():
    """Two parts with sums of weights 1 and 3: out = (a + 3 b) / 4, lse = log 4;
    an empty part (lse = -inf) contributes nothing."""
    a, b = np.array([1.0, 2.0]), np.array([-3.0, 8.0])
    out, lse = oracle.merge_partials([a, b, np.zeros(2)], [0.0, math.log(3.0), -np.inf])
    np.testing.assert_allclose(out, (a + 3 * b) / 4, rtol=1e-15)
    assert lse == pytest.approx(math.log(4.0), abs=1e-15)


def test_split_ranges_cover_the_table():
    for w, s in [(7, 1), (7, 2), (7, 7), (7, 64), (2048, 128), (513, 16)]:
        rg = oracle.split_ranges(w, 16, s)
        assert len(rg) == s and rg[0][0] == 0
        assert all(rg[j][1] == rg[j + 1][0] for j in range(s - 1))
        assert rg[-1][1] >= w * 16


def test_mla_equals_attention_on_concatenated_keys():
    """MLA = attention with K = [latent; k_pos] (D = R + P), V = latent, Hkv = 1."""
    lens = [70, 33]
    wl = build_mla("t", 61, torch.float64, lens, decode_queries(lens) + [(0, 12)],
                   5, 24, 8, 16)
    t = wl.tensors
    args = (wl.lens, wl.qseq, wl.qpos, wl.table, wl.page_size, wl.scale, True)
    mla, mla_lse = oracle.paged_mla(t["q_abs"], t["q_pos"], t["latent"], t["k_pos"], *args)
    kcat = torch.cat([t["latent"], t["k_pos"]], dim=3)
    qcat = torch.cat([t["q_abs"], t["q_pos"]], dim=2)
    att, att_lse = oracle.paged_attention(qcat, kcat, t["latent"], *args)
    np.testing.assert_allclose(mla, att, rtol=RTOL, atol=1e-13)
    np.testing.assert_allclose(mla_lse, att_lse, rtol=RTOL, atol=1e-13)


def test_mla_split_equals_unsplit():
    lens = [200, 64]
    wl = build_mla("t", 62, torch.float64, lens, decode_queries(lens), 3, 16, 4, 16)
    t = wl.tensors
    args = (wl.lens, wl.qseq, wl.qpos, wl.table, wl.page_size, wl.scale, True)
    base, _ = oracle.paged_mla(t["q_abs"], t["q_pos"], t["latent"], t["k_pos"], *args)
    out, _ = ref.paged_mla_split(t["q_abs"], t["q_pos"], t["latent"], t["k_pos"], *args,
                                 splits=5)
    np.testing.assert_allclose(out, base, rtol=RTOL, atol=1e-13)


def test_single_row_helpers_match_full():
    lens = [90, 31]
    wl = build_attention("t", 71, torch.float64, lens, decode_queries(lens) + [(0, 5)],
                         4, 2, 8, 8, 16)
    q, k, v = (wl.tensors[x] for x in "qkv")
    args = (wl.lens, wl.qseq, wl.qpos, wl.table, wl.page_size, wl.scale, True)
    full, full_lse = oracle.paged_attention(q, k, v, *args)
    for i in range(3):
        for h in range(4):
            o, l = ref.attention_one(q, k, v, *args, i, h)
            np.testing.assert_allclose(o, full[i, h], rtol=RTOL)
            assert l == pytest.approx(full_lse[i, h], abs=1e-13)
    wm = build_mla("t", 72, torch.float64, lens, decode_queries(lens), 3, 16, 4, 16)
    t = wm.tensors
    margs = (wm.lens, wm.qseq, wm.qpos, wm.table, wm.page_size, wm.scale, True)
    mfull, _ = oracle.paged_mla(t["q_abs"], t["q_pos"], t["latent"], t["k_pos"], *margs)
    o, _ = ref.mla_one(t["q_abs"], t["q_pos"], t["latent"], t["k_pos"], *margs, 1, 2)
    np.testing.assert_allclose(o, mfull[1, 2], rtol=RTOL)


# ----------------------------------------------------- non-finite propagation

def test_invisible_nan_is_never_read_and_visible_nan_propagates():
    lens = [21, 9]
    base = build_attention("t", 81, torch.float64, lens, decode_queries(lens), 4, 2, 8, 8, 8,
                           pool=8)
    pois = build_attention("t", 81, torch.float64, lens, decode_queries(lens), 4, 2, 8, 8, 8,
                           pool=8, poison=True)
    assert torch.isnan(pois.tensors["k"]).any()
    args = (base.lens, base.qseq, base.qpos, base.table, 8, base.scale, True)
    a, _ = oracle.paged_attention(*(base.tensors[x] for x in "qkv"), *args)
    b, _ = oracle.paged_attention(*(pois.tensors[x] for x in "qkv"), *args)
    np.testing.assert_array_equal(a, b)
    v = base.tensors["v"].clone()
    v[int(base.table[1, 0]), 3, 1, 0] = float("nan")  # visible token 3 of seq 1, KV head 1
    c, _ = oracle.paged_attention(base.tensors["q"], base.tensors["k"], v, *args)
    # only element 0 of the value rows of KV head 1 is NaN: q heads 2, 3 of
    # query 1 get NaN there, everything else stays finite
    assert np.isnan(c[1, 2:4, 0]).all()
    assert np.isfinite(c[1, 2:4, 1:]).all() and np.isfinite(c[1, 0:2]).all()
    assert np.isfinite(c[0]).all()


# --------------------------------------------------------- planted mistakes

def test_planted_mistakes_trip_a_pin(monkeypatch):
    """A dropped '+1' in the causal count, swapped page/slot indices in the
    gather and an lse without its max term each make a pin above fail."""
    # 1. dropped +1: a causal query at position 0 would see nothing
    monkeypatch.setattr(ref, "visible_count",
                        lambda lens, qseq, qpos, i, causal: int(qpos[i]) if causal else int(lens[qseq[i]]))
    with pytest.raises(AssertionError):
        test_causal_uses_absolute_positions()
    monkeypatch.undo()

    # 2. swapped page/slot indices in the gather
    def bad_gather(cache, table_row, n, page_size):
        if n == 0:
            return np.zeros((0, cache.shape[2], cache.shape[3]))
        n_pages = -(-n // page_size)
        block = ref._f64(ref._take_pages(cache, np.asarray(table_row[:n_pages], dtype=np.int64)))
        return block.transpose(1, 0, 2, 3).reshape(n_pages * page_size, *block.shape[2:])[:n]
    monkeypatch.setattr(ref, "_gather_tokens", bad_gather)
    with pytest.raises(AssertionError):
        test_equal_scores_give_mean_of_visible_values()
    monkeypatch.undo()

    # 3. softmax without the max subtraction's matching lse term
    orig = ref._softmax_pv

    def bad_softmax(x, vals):
        o, l = orig(x, vals)
        return o, l - np.max(x, axis=-1) if x.shape[-1] else l
    monkeypatch.setattr(ref, "_softmax_pv", bad_softmax)
    with pytest.raises(AssertionError):
        test_two_keys_closed_form()
    monkeypatch.undo()


def _some_pin_fails(pins):
    for pin in pins:
        try:
            pin()
        except AssertionError:
            return True
    return False


def test_planted_operand_mistakes_trip_a_pin(monkeypatch):
    """A lost scale, a wrong q-head -> KV-head map (h % Hkv) and K/V used in
    each other's place each make at least one pin fail."""
    real = oracle.paged_attention
    pins = [test_single_visible_key_returns_its_value, test_two_keys_closed_form,
            test_gqa_head_map_is_contiguous_groups, lambda: test_matches_torch_sdpa_on_a_chunk(True)]

    # 1. scale dropped
    monkeypatch.setattr(oracle, "paged_attention",
                        lambda q, k, v, lens, qseq, qpos, table, ps, scale, causal, token_range=None:
                        real(q, k, v, lens, qseq, qpos, table, ps, 1.0, causal, token_range))
    assert _some_pin_fails(pins)
    monkeypatch.undo()

    # 2. q head h served by KV head h % Hkv (tiled instead of grouped heads)
    def tiled(q, k, v, lens, qseq, qpos, table, ps, scale, causal, token_range=None):
        g = q.shape[1] // k.shape[2]
        return real(q, k.repeat(1, 1, g, 1), v.repeat(1, 1, g, 1), lens, qseq, qpos, table, ps,
                    scale, causal, token_range)
    monkeypatch.setattr(oracle, "paged_attention", tiled)
    assert _some_pin_fails(pins)
    monkeypatch.undo()

    # 3. K and V exchanged where their shapes allow it
    def swapped(q, k, v, lens, qseq, qpos, table, ps, scale, causal, token_range=None):
        if k.shape == v.shape:
            k, v = v, k
        return real(q, k, v, lens, qseq, qpos, table, ps, scale, causal, token_range)
    monkeypatch.setattr(oracle, "paged_attention", swapped)
    assert _some_pin_fails(pins)
    monkeypatch.undo()
