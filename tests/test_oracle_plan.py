"""Pins of the oracle's independent plan encoder (spec v1).

The golden word lists in tests/golden/ are derived by hand from the spec, so
they pin the Python encoder against something other than itself; the C++
encoder is then checked bit-exactly against the Python one elsewhere.
"""

import numpy as np
import pytest

from oracle import plan as op
from tests._golden import FIXTURES, read_plan_fixture


@pytest.mark.parametrize("name", FIXTURES)
def test_golden_words(name):
    fx = read_plan_fixture(name)
    words = op.encode_plan(fx["lens"], fx["qseq"], fx["qpos"], fx["table"],
                           fx["page_size"], fx["pages"])
    assert words.dtype == np.uint32
    np.testing.assert_array_equal(words, fx["words"])


@pytest.mark.parametrize("name", FIXTURES)
def test_decode_roundtrip(name):
    fx = read_plan_fixture(name)
    d = op.decode_plan(fx["words"])
    assert d["lens"] == fx["lens"] and d["qseq"] == fx["qseq"] and d["qpos"] == fx["qpos"]
    assert d["page_size"] == fx["page_size"] and d["pages"] == fx["pages"]
    for s, L in enumerate(fx["lens"]):
        used = -(-L // fx["page_size"])
        np.testing.assert_array_equal(d["table"][s, :used], fx["table"][s, :used])
        assert (d["table"][s, used:] == 0xFFFFFFFF).all()
    covered = sorted(d["rows"] + [f + j for f, c in d["tiles"] for j in range(c)])
    assert covered == list(range(len(fx["qseq"])))


def test_tile_rule_boundaries():
    # a run of exactly TILE_MIN is a tile; one shorter is rows
    n = op.TILE_MIN
    rows, tiles = op.split_rows_tiles([0] * n, list(range(n)))
    assert rows == [] and tiles == [(0, n)]
    rows, tiles = op.split_rows_tiles([0] * (n - 1), list(range(n - 1)))
    assert rows == list(range(n - 1)) and tiles == []
    # a gap in positions or a change of sequence ends a run
    rows, tiles = op.split_rows_tiles([0] * 20 + [1] * 20, list(range(10)) + list(range(11, 21)) + list(range(20)))
    # listed heaviest first: works 20*0 + 210 = 210, 10*11 + 55 = 165, 55
    assert tiles == [(20, 20), (10, 10), (0, 10)] and rows == []
    # equal work: the earlier first query comes first
    rows, tiles = op.split_rows_tiles([0] * 10 + [1] * 10, list(range(10)) * 2)
    assert tiles == [(0, 10), (10, 10)] and rows == []
    # 2 * TILE_MAX + 1 consecutive queries -> 3 tiles
    m = 2 * op.TILE_MAX + 1
    rows, tiles = op.split_rows_tiles([0] * m, list(range(m)))
    # cut from the first query; the later full tile sees more keys, so it
    # is listed first
    assert tiles == [(op.TILE_MAX, op.TILE_MAX), (0, op.TILE_MAX), (2 * op.TILE_MAX, 1)]


def _ok_args():
    return dict(lens=[10, 3], qseq=[0, 1], qpos=[9, 2], table=np.array([[1, 0], [2, 3]]),
                page_size=8, pages=4)


@pytest.mark.parametrize("mutate,code", [
    (lambda a: a.update(page_size=0), "EINVAL"),
    (lambda a: a.update(lens=[17, 3]), "ESHAPE"),          # 17 > W * ps = 16
    (lambda a: a.update(qseq=[0, 2]), "EINVAL"),           # no sequence 2
    (lambda a: a.update(qpos=[10, 2]), "EINVAL"),          # position 10 not in a 10-token cache
    (lambda a: a.update(table=np.array([[1, 4], [2, 3]])), "EINVAL"),  # page 4 of 4
    (lambda a: a.update(qpos=[9]), "EINVAL"),              # qseq/qpos lengths differ
    (lambda a: a.update(lens=[10, 3], table=np.zeros((2, 0), dtype=np.int64)), "EINVAL"),
    (lambda a: a.update(pages=1 << 32), "ERANGE"),
])
def test_validation_errors(mutate, code):
    a = _ok_args()
    op.encode_plan(**a)
    mutate(a)
    with pytest.raises(op.PlanError) as e:
        op.encode_plan(**a)
    assert e.value.code == code


def test_unused_entries_are_not_validated():
    a = _ok_args()
    a["table"] = np.array([[1, 0], [2, 77]])  # seq 1 has 3 tokens: one page used
    words = op.encode_plan(**a)
    assert words[-1] == 0xFFFFFFFF


def test_empty_schedule():
    words = op.encode_plan([], [], [], np.zeros((0, 0), dtype=np.int64), 16, 0)
    assert list(words[:9]) == [op.MAGIC, 1, 0, 0, 0, 16, 0, 0, 0] and len(words) == 16
