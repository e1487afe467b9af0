"""Pins of the append oracle (oracle/append.py), CPU only.

- hand-derived write targets (tests/golden/append_targets.txt);
- the written rows read back through the attention oracle's own gather (an
  independent addressing path, itself pinned against SDPA and a contiguous
  cache), and every other slot bitwise unchanged, in f32 and bf16;
- the conflict rules of validate_writes (same slot twice, a slot of a page
  two sequences share, a position outside its sequence);
- the CacheAppendReport arithmetic;
- planted addressing mistakes, each caught by the golden targets.
"""

import numpy as np
import pytest
import torch

import oracle
from oracle import append as oa
from oracle import reference as ref
from tests._golden import read_append_fixture


def test_golden_write_targets():
    g = read_append_fixture("append_targets.txt")
    got = oracle.write_targets(g["lens"], g["qseq"], g["qpos"], g["table"], g["page_size"],
                               g["pages"])
    assert got == g["targets"]
    assert oracle.validate_writes(g["lens"], g["qseq"], g["qpos"], g["table"], g["page_size"],
                                  g["pages"]) == g["targets"]


def _schedule(rng, ps):
    """Sequences with distinct pages; queries: every sequence's last token
    plus a chunk of consecutive positions in some sequences."""
    lens = [int(x) for x in rng.integers(1, 60, size=5)]
    W = max(-(-L // ps) for L in lens) + 1
    n_pages = sum(-(-L // ps) for L in lens) + 3
    perm = rng.permutation(n_pages)
    table = np.full((len(lens), W), 0xFFFFFFFF, dtype=np.int64)
    k = 0
    for s, L in enumerate(lens):
        for j in range(-(-L // ps)):
            table[s, j] = perm[k]
            k += 1
    qseq, qpos = [], []
    for s, L in enumerate(lens):
        if s % 2 == 0 and L > 8:
            start = int(rng.integers(0, L - 8))
            qseq += [s] * 8
            qpos += list(range(start, start + 8))
        if s % 2 == 1 or L <= 8 or start + 8 < L:
            qseq.append(s)
            qpos.append(L - 1)
    return lens, qseq, qpos, table, n_pages


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("ps", [1, 4, 16])
def test_append_reads_back_through_the_attention_gather(dtype, ps):
    rng = np.random.default_rng(ps)
    lens, qseq, qpos, table, n_pages = _schedule(rng, ps)
    H, D, Dv = 3, 8, 5
    gen = torch.Generator().manual_seed(ps)
    k = torch.randn(n_pages, ps, H, D, generator=gen).to(dtype)
    v = torch.randn(n_pages, ps, H, Dv, generator=gen).to(dtype)
    new_k = torch.randn(len(qseq), H, D, generator=gen).to(dtype)
    new_v = torch.randn(len(qseq), H, Dv, generator=gen).to(dtype)
    k2, v2 = oracle.paged_append(new_k, new_v, k, v, lens, qseq, qpos, table, ps)
    written = {}
    for i, (s, p) in enumerate(zip(qseq, qpos)):
        written[(s, p)] = i
    for s, L in enumerate(lens):
        gk_old = ref._gather_tokens(k, table[s], L, ps)
        gk_new = ref._gather_tokens(k2, table[s], L, ps)
        gv_new = ref._gather_tokens(v2, table[s], L, ps)
        gv_old = ref._gather_tokens(v, table[s], L, ps)
        for p in range(L):
            if (s, p) in written:
                i = written[(s, p)]
                np.testing.assert_array_equal(gk_new[p], new_k[i].double().numpy())
                np.testing.assert_array_equal(gv_new[p], new_v[i].double().numpy())
            else:
                np.testing.assert_array_equal(gk_new[p], gk_old[p])
                np.testing.assert_array_equal(gv_new[p], gv_old[p])
    # slots of no sequence (unused tails, spare pages) are bitwise unchanged
    hit = np.zeros((n_pages, ps), dtype=bool)
    for page, slot in oracle.write_targets(lens, qseq, qpos, table, ps, n_pages):
        hit[page, slot] = True
    keep = torch.as_tensor(~hit)
    assert torch.equal(k2[keep], k[keep]) and torch.equal(v2[keep], v[keep])
    # the inputs are not modified
    assert not torch.equal(k2, k)


def test_conflicts():
    ps, pages = 4, 6
    table = np.array([[0, 1], [0, 2]])  # page 0 shared by both sequences
    lens = [8, 7]
    # distinct slots of the shared page: fine
    assert oracle.validate_writes(lens, [0, 1], [1, 2], table, ps, pages) == [(0, 1), (0, 2)]
    # the same slot of the shared page from two sequences
    with pytest.raises(oracle.WriteConflict):
        oracle.validate_writes(lens, [0, 1], [3, 3], table, ps, pages)
    # the same (sequence, position) twice
    with pytest.raises(oracle.WriteConflict):
        oracle.validate_writes(lens, [0, 0], [5, 5], table, ps, pages)
    # a position outside its sequence
    with pytest.raises(oracle.WriteConflict):
        oracle.write_targets(lens, [1], [7], table, ps, pages)
    # a page outside the pool
    with pytest.raises(oracle.WriteConflict):
        oracle.write_targets([4], [0], [0], np.array([[9]]), ps, pages)
    # no queries: nothing to check
    assert oracle.validate_writes(lens, [], [], table, ps, pages) == []


def test_report():
    assert oracle.append_report(False, False, 100, 60, 3) == \
        {"key_copied": False, "value_copied": False, "copied_bytes": 0}
    assert oracle.append_report(True, False, 100, 60, 3)["copied_bytes"] == 100
    assert oracle.append_report(True, True, 100, 60, 3) == \
        {"key_copied": True, "value_copied": True, "copied_bytes": 160}
    # an append with no queries copies nothing even when a copy is asked for
    assert oracle.append_report(True, True, 100, 60, 0)["copied_bytes"] == 0


def _swapped_page_slot(lens, qseq, qpos, table, ps, pages):
    return [(int(table[s][p % ps]), p // ps) for s, p in zip(qseq, qpos)]


def _table_by_query(lens, qseq, qpos, table, ps, pages):
    return [(int(table[i][p // ps]), p % ps) for i, p in enumerate(qpos) if i < len(table)] + \
        [(-1, -1)] * max(0, len(qpos) - len(table))


def _slot_off_by_one(lens, qseq, qpos, table, ps, pages):
    return [(int(table[s][p // ps]), (p + 1) % ps) for s, p in zip(qseq, qpos)]


@pytest.mark.parametrize("planted", [_swapped_page_slot, _table_by_query, _slot_off_by_one])
def test_planted_addressing_mistakes_fail_the_golden(planted, monkeypatch):
    g = read_append_fixture("append_targets.txt")
    monkeypatch.setattr(oa, "write_targets", planted)
    args = (g["lens"], g["qseq"], g["qpos"], g["table"], g["page_size"], g["pages"])
    try:
        got = oa.validate_writes(*args)
    except (oa.WriteConflict, IndexError):
        return
    assert got != g["targets"]
