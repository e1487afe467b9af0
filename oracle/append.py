"""Oracle of the paged cache append: test infrastructure, not product code.

Written from the ruDNN 0.1.7 ``paged_attention`` module page, the
``DevicePlan::append`` / ``append_with_report`` doc comments and the
``CacheAppendReport`` struct: every query of the plan stores its new key and
value rows (all KV heads) into the cache slot of its own absolute position,
found through the block table exactly as attention finds keys to read; the
write plan is validated first (``validate_writes``); a cache that is not
written in place is copied whole first, and the report states which caches
were copied and how many bytes.

The page shows ``validate_writes`` only by name.  Reading taken here: the
writes are valid when every query's position lies inside its sequence (the
plan already requires qpos < L) and no two queries target the same physical
(page, slot), whether through the same (sequence, position) or through a
page that two sequences share.  Two writes to one slot would leave the
result to the order the device happens to run them in.

Pins: ``tests/test_oracle_append.py`` (hand-derived golden targets, the
read-back through the attention oracle's own gather, untouched slots, the
conflict rules, the report arithmetic, planted mistakes).
"""

from __future__ import annotations

import numpy as np


class WriteConflict(ValueError):
    """The write plan of an append is not valid."""


def write_targets(lens, qseq, qpos, table, page_size: int, pages: int):
    """(page, slot) written by each query: slot qpos % page_size of page
    table[qseq][qpos // page_size].  Raises WriteConflict when a position is
    outside its sequence or its page outside the pool."""
    lens = np.asarray(lens, dtype=np.int64)
    qseq = np.asarray(qseq, dtype=np.int64)
    qpos = np.asarray(qpos, dtype=np.int64)
    table = np.asarray(table, dtype=np.int64)
    out = []
    for i in range(len(qseq)):
        s, p = int(qseq[i]), int(qpos[i])
        if not 0 <= s < len(lens) or not 0 <= p < int(lens[s]):
            raise WriteConflict(f"query {i}: position {p} outside its sequence")
        page = int(table[s, p // page_size])
        if not 0 <= page < pages:
            raise WriteConflict(f"query {i}: page {page} outside the pool")
        out.append((page, p % page_size))
    return out


def validate_writes(lens, qseq, qpos, table, page_size: int, pages: int):
    """The (page, slot) targets, after checking that no two queries share one."""
    targets = write_targets(lens, qseq, qpos, table, page_size, pages)
    seen = {}
    for i, t in enumerate(targets):
        if t in seen:
            raise WriteConflict(f"queries {seen[t]} and {i} write page {t[0]} slot {t[1]}")
        seen[t] = i
    return targets


def paged_append(new_k, new_v, k, v, lens, qseq, qpos, table, page_size: int):
    """New caches (copies of k and v, torch CPU tensors of any dtype) with
    new_k[i] / new_v[i] ([heads, D] / [heads, Dv]) stored at query i's slot.
    Pure copies: the result is exact in every dtype."""
    pages = int(k.shape[0])
    targets = validate_writes(lens, qseq, qpos, table, page_size, pages)
    k2, v2 = k.clone(), v.clone()
    for i, (page, slot) in enumerate(targets):
        k2[page, slot] = new_k[i]
        v2[page, slot] = new_v[i]
    return k2, v2


def append_report(copy_key: bool, copy_value: bool, key_bytes: int, value_bytes: int,
                  queries: int):
    """CacheAppendReport of an append: a cache not written in place is copied
    whole; an append with no queries copies nothing."""
    if queries == 0:
        return {"key_copied": False, "value_copied": False, "copied_bytes": 0}
    return {"key_copied": bool(copy_key), "value_copied": bool(copy_value),
            "copied_bytes": (key_bytes if copy_key else 0) + (value_bytes if copy_value else 0)}
