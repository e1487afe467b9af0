"""Independent encoder/decoder of the u32 plan words (test infrastructure).

The ruDNN 0.1.7 ``paged_attention`` page shows a ``HostPlan`` holding a
vector of u32 ``words`` plus ``queries``, ``sequences``, ``table_width``,
``page_size`` and ``pages``, uploaded once as U32 metadata
(``DevicePlan::upload``), but not the layout of the words.  The layout below
(spec v1) is this project's own; this module implements it in plain Python,
separately from the library's C++ encoder, and is the bit-exact reference
the C++ encoder is tested against.  It is itself pinned by hand-derived
golden word lists in ``tests/golden/``.

Spec v1 (little-endian u32 words):

    0       magic 0x564B5041
    1       version 1
    2..6    Q (queries), S (sequences), W (table width), ps (page size),
            N (pages in the pool)
    7       R, the number of row queries (attended one query at a time)
    8       T, the number of tiles (runs of consecutive queries)
    9..15   0
    16      lens[S]           tokens in the cache of each sequence
    +S      qseq[Q]           sequence of each query
    +Q      qpos[Q]           absolute position of each query
    +Q      rows[R]           indices of the row queries, ascending
    +R      tiles[T] x 2      {first query, query count}
    +2T     table[S*W]        row-major; entry j of sequence s is the
                              physical page of logical page j when
                              j < ceil(lens[s]/ps), else 0xFFFFFFFF

Tiles: scanning the queries in order, a run is a maximal range of queries of
one sequence whose positions increase by one from query to query.  A run of
at least TILE_MIN queries is cut, from its first query, into tiles of at
most TILE_MAX queries; the queries of shorter runs are rows.  Tiles are
listed heaviest first: by decreasing work, the sum over the tile's queries
of (position + 1), then by increasing first query (kernels take tiles in
list order, so long tiles start first).

Validation (each failure raises ``PlanError`` with the status name the C
ABI returns for it):
    ps == 0, or W == 0 while S > 0                         EINVAL
    any count or the word total above 2**32 - 1            ERANGE
    lens[s] > W * ps                                       ESHAPE
    qseq[i] >= S                                           EINVAL
    qpos[i] >= lens[qseq[i]]  (a query is in its cache)    EINVAL
    table[s][j] >= N for a used entry                      EINVAL
"""

from __future__ import annotations

import numpy as np

MAGIC = 0x564B5041
VERSION = 1
HEADER_WORDS = 16
UNUSED = 0xFFFFFFFF
TILE_MIN = 8
TILE_MAX = 128
U32_MAX = 0xFFFFFFFF


class PlanError(ValueError):
    """Invalid schedule; ``code`` is the C ABI status name (e.g. "EINVAL")."""

    def __init__(self, code: str, message: str):
        super().__init__(f"{code}: {message}")
        self.code = code
        self.message = message


def _runs(qseq, qpos):
    """Maximal runs [a, b) of queries of one sequence at consecutive positions."""
    q = len(qseq)
    a = 0
    while a < q:
        b = a + 1
        while b < q and qseq[b] == qseq[a] and qpos[b] == qpos[b - 1] + 1:
            b += 1
        yield a, b
        a = b


def split_rows_tiles(qseq, qpos):
    """(rows, tiles) per the tile rule of spec v1."""
    rows, tiles = [], []
    for a, b in _runs(qseq, qpos):
        if b - a >= TILE_MIN:
            for first in range(a, b, TILE_MAX):
                tiles.append((first, min(TILE_MAX, b - first)))
        else:
            rows.extend(range(a, b))

    def work(tile):  # sum of (position + 1) over the tile's queries
        first, count = tile
        return count * int(qpos[first]) + count * (count + 1) // 2

    tiles.sort(key=lambda t: (-work(t), t[0]))
    return rows, tiles


def encode_plan(lens, qseq, qpos, table, page_size: int, pages: int) -> np.ndarray:
    """Validate a schedule and return its spec-v1 words as a uint32 array.

    lens [S], qseq [Q], qpos [Q] integers; table [S, W] integers (entries
    past a sequence's last used page are ignored); ``page_size`` tokens per
    page; ``pages`` pages in the pool.
    """
    lens = [int(x) for x in np.asarray(lens).reshape(-1)]
    qseq = [int(x) for x in np.asarray(qseq).reshape(-1)]
    qpos = [int(x) for x in np.asarray(qpos).reshape(-1)]
    tab = np.asarray(table)
    s_n, q_n = len(lens), len(qseq)
    if len(qpos) != q_n:
        raise PlanError("EINVAL", "qseq and qpos differ in length")
    w = int(tab.shape[1]) if tab.ndim == 2 else 0
    if tab.ndim != 2 or tab.shape[0] != s_n:
        if not (s_n == 0 and tab.size == 0):
            raise PlanError("EINVAL", "block table must be [sequences, table_width]")
    page_size, pages = int(page_size), int(pages)
    if page_size <= 0:
        raise PlanError("EINVAL", "page size must be positive")
    if s_n > 0 and w == 0:
        raise PlanError("EINVAL", "table width must be positive")
    for x in (s_n, q_n, w, page_size, pages):
        if x > U32_MAX or x < 0:
            raise PlanError("ERANGE", "plan dimension exceeds u32")
    if s_n * w > U32_MAX:
        raise PlanError("ERANGE", "block table exceeds u32 indexing")
    for L in lens:
        if L < 0 or L > U32_MAX:
            raise PlanError("ERANGE", "sequence length exceeds u32")
        if L > w * page_size:
            raise PlanError("ESHAPE", "sequence longer than its block-table row")
    for s, p in zip(qseq, qpos):
        if s < 0 or s >= s_n:
            raise PlanError("EINVAL", "query sequence index out of range")
        if p < 0 or p >= lens[s]:
            raise PlanError("EINVAL", "query position outside its sequence")
    rows, tiles = split_rows_tiles(qseq, qpos)
    total = HEADER_WORDS + s_n + 2 * q_n + len(rows) + 2 * len(tiles) + s_n * w
    if total > U32_MAX:
        raise PlanError("ERANGE", "plan exceeds u32 word count")

    words = [MAGIC, VERSION, q_n, s_n, w, page_size, pages, len(rows), len(tiles)]
    words += [0] * (HEADER_WORDS - len(words))
    words += lens
    words += qseq
    words += qpos
    words += rows
    for first, count in tiles:
        words += [first, count]
    for s in range(s_n):
        used = -(-lens[s] // page_size)
        for j in range(w):
            if j < used:
                e = int(tab[s, j])
                if e < 0 or e >= pages:
                    raise PlanError("EINVAL", "block table entry outside the page pool")
                words.append(e)
            else:
                words.append(UNUSED)
    assert len(words) == total
    return np.array(words, dtype=np.uint32)


def decode_plan(words) -> dict:
    """Inverse of ``encode_plan`` (header checks only)."""
    wd = [int(x) for x in np.asarray(words, dtype=np.uint32).reshape(-1)]
    if len(wd) < HEADER_WORDS or wd[0] != MAGIC or wd[1] != VERSION:
        raise PlanError("EINVAL", "not a spec-v1 plan")
    q_n, s_n, w, ps, n, r_n, t_n = wd[2:9]
    o = HEADER_WORDS
    lens = wd[o:o + s_n]; o += s_n
    qseq = wd[o:o + q_n]; o += q_n
    qpos = wd[o:o + q_n]; o += q_n
    rows = wd[o:o + r_n]; o += r_n
    tiles = [(wd[o + 2 * j], wd[o + 2 * j + 1]) for j in range(t_n)]; o += 2 * t_n
    table = np.array(wd[o:o + s_n * w], dtype=np.uint32).reshape(s_n, w)
    o += s_n * w
    if o != len(wd):
        raise PlanError("EINVAL", "plan length does not match its header")
    return dict(queries=q_n, sequences=s_n, table_width=w, page_size=ps, pages=n,
                lens=lens, qseq=qseq, qpos=qpos, rows=rows, tiles=tiles, table=table)
