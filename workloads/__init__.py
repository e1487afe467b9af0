"""Seeded synthetic inputs for paged attention: schedules and tensors.

This module draws random numbers and lays out block tables; it holds none of
the attention arithmetic.  Both sides use it: the tests and the benchmark pass
the same tensors to the library and to the oracle.

Recipe (one ``numpy.random.default_rng(seed)`` per workload, fixed draw order):
  1. sequence lengths (and prior lengths of prefill chunks);
  2. one permutation of the page pool; the pages of sequence 0 take the first
     entries, then sequence 1, and so on (shuffled physical pages);
  3. tensors, each ~ N(0, 1) drawn in float32 then rounded to the workload's
     dtype (round-to-nearest-even, by torch).  A tensor is filled in fixed
     blocks of whole rows; block ``b`` of tensor ``j`` comes from
     ``default_rng([seed, j, b])``, so the values do not depend on how many
     threads fill it.
The MLA latent is RMS-normalised per token in float32 before rounding:
``x / sqrt(mean(x**2) + 1e-6)`` over the latent rank (no weight).
With ``poison=True`` every cache slot no query may see (pages outside every
sequence and slots at or past the length in a sequence's last page) is NaN,
so a kernel that reads them produces NaN.
"""

from __future__ import annotations

import math
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field

import numpy as np
import torch

_BLOCK_ELEMS = 1 << 22


@dataclass
class Workload:
    """A schedule plus its tensors (CPU torch tensors in ``dtype``)."""

    name: str
    kind: str                 # "attention" or "mla"
    dtype: torch.dtype
    lens: np.ndarray          # [S] int64
    qseq: np.ndarray          # [Q] int64
    qpos: np.ndarray          # [Q] int64
    table: np.ndarray         # [S, W] int64 (unused entries 0)
    page_size: int
    pages: int
    scale: float
    causal: bool
    tensors: dict = field(default_factory=dict)
    info: dict = field(default_factory=dict)

    @property
    def queries(self) -> int:
        return int(self.qseq.shape[0])

    @property
    def sequences(self) -> int:
        return int(self.lens.shape[0])

    @property
    def table_width(self) -> int:
        return int(self.table.shape[1])

    def visible(self) -> np.ndarray:
        """Visible keys per query (causal: position + 1; else the length)."""
        if self.causal:
            return self.qpos + 1
        return self.lens[self.qseq]


def _layout(rng, lens, page_size, pool):
    """Block table [S, W] from one permutation of a pool of ``pool`` pages."""
    need = [-(-int(L) // page_size) for L in lens]
    total = sum(need)
    assert pool >= total
    perm = rng.permutation(pool)
    w = max([1] + need)
    table = np.zeros((len(lens), w), dtype=np.int64)
    o = 0
    for s, n in enumerate(need):
        table[s, :n] = perm[o:o + n]
        o += n
    return table


def fill_normal(shape, dtype, seed, tensor_id, rms_norm=False, threads=8):
    """N(0,1) float32 draws rounded to ``dtype``; optional per-row RMS norm."""
    shape = tuple(int(x) for x in shape)
    numel = int(np.prod(shape)) if shape else 1
    last = shape[-1] if shape else 1
    rows_per_block = max(1, _BLOCK_ELEMS // max(last, 1))
    blk = rows_per_block * last
    out = torch.empty(numel, dtype=dtype)
    nblocks = -(-numel // blk) if numel else 0

    def one(b):
        a = b * blk
        e = min(numel, a + blk)
        rng = np.random.default_rng([seed, tensor_id, b])
        x = rng.standard_normal(e - a, dtype=np.float32)
        if rms_norm:
            x = x.reshape(-1, last)
            x = x / np.sqrt(np.mean(x * x, axis=1, keepdims=True) + np.float32(1e-6))
            x = x.reshape(-1)
        out[a:e] = torch.from_numpy(x).to(dtype)

    if nblocks:
        with ThreadPoolExecutor(max(1, threads)) as ex:
            list(ex.map(one, range(nblocks)))
    return out.reshape(shape)


def _poison(cache, lens, table, page_size):
    """NaN in every slot no query can see (unused pages, tails of last pages)."""
    used = np.zeros(cache.shape[0], dtype=bool)
    for s, L in enumerate(lens):
        n = -(-int(L) // page_size)
        used[table[s, :n]] = True
        if L % page_size and n:
            cache[int(table[s, n - 1]), int(L) % page_size:] = float("nan")
    cache[torch.from_numpy(~used)] = float("nan")


def build_attention(name, seed, dtype, lens, queries, hq, hkv, d, dv, page_size,
                    pool=None, scale=None, causal=True, poison=False, rng=None):
    """Workload for ``attention``.

    lens: lengths per sequence; queries: list of (sequence, position);
    pool: pages in the cache (default: exactly the pages needed).
    ``rng`` continues a generator that already drew the lengths.
    """
    rng = rng if rng is not None else np.random.default_rng(seed)
    lens = np.asarray(lens, dtype=np.int64)
    need = int(sum(-(-int(L) // page_size) for L in lens))
    pool = need if pool is None else int(pool)
    table = _layout(rng, lens, page_size, pool)
    qseq = np.array([s for s, _ in queries], dtype=np.int64)
    qpos = np.array([p for _, p in queries], dtype=np.int64)
    q = fill_normal((len(queries), hq, d), dtype, seed, 0)
    k = fill_normal((pool, page_size, hkv, d), dtype, seed, 1)
    v = fill_normal((pool, page_size, hkv, dv), dtype, seed, 2)
    if poison:
        _poison(k, lens, table, page_size)
        _poison(v, lens, table, page_size)
    return Workload(name=name, kind="attention", dtype=dtype, lens=lens, qseq=qseq,
                    qpos=qpos, table=table, page_size=page_size, pages=pool,
                    scale=float(scale if scale is not None else 1.0 / math.sqrt(d)),
                    causal=bool(causal), tensors=dict(q=q, k=k, v=v),
                    info=dict(hq=hq, hkv=hkv, d=d, dv=dv))


def build_mla(name, seed, dtype, lens, queries, h, r, p, page_size, pool=None,
              scale=None, causal=True, poison=False, rng=None):
    """Workload for ``mla`` (latent RMS-normalised per token)."""
    rng = rng if rng is not None else np.random.default_rng(seed)
    lens = np.asarray(lens, dtype=np.int64)
    need = int(sum(-(-int(L) // page_size) for L in lens))
    pool = need if pool is None else int(pool)
    table = _layout(rng, lens, page_size, pool)
    qseq = np.array([s for s, _ in queries], dtype=np.int64)
    qpos = np.array([pp for _, pp in queries], dtype=np.int64)
    q_abs = fill_normal((len(queries), h, r), dtype, seed, 0)
    q_pos = fill_normal((len(queries), h, p), dtype, seed, 1)
    latent = fill_normal((pool, page_size, 1, r), dtype, seed, 2, rms_norm=True)
    k_pos = fill_normal((pool, page_size, 1, p), dtype, seed, 3)
    if poison:
        _poison(latent, lens, table, page_size)
        _poison(k_pos, lens, table, page_size)
    return Workload(name=name, kind="mla", dtype=dtype, lens=lens, qseq=qseq,
                    qpos=qpos, table=table, page_size=page_size, pages=pool,
                    scale=float(scale if scale is not None else 1.0 / math.sqrt(r + p)),
                    causal=bool(causal),
                    tensors=dict(q_abs=q_abs, q_pos=q_pos, latent=latent, k_pos=k_pos),
                    info=dict(h=h, r=r, p=p))


def fp8_caches(wl: Workload, k_scale: float, v_scale: float):
    """The workload's K and V as FP8 E4M3 byte codes (uint8 tensors):
    round(k / k_scale), round(v / v_scale) to the nearest E4M3 value (torch's
    float8_e4m3fn cast; NaN poison stays NaN).  Holds no attention
    arithmetic: the caches are inputs."""
    k = (wl.tensors["k"].float() / k_scale).to(torch.float8_e4m3fn).view(torch.uint8)
    v = (wl.tensors["v"].float() / v_scale).to(torch.float8_e4m3fn).view(torch.uint8)
    return k.contiguous(), v.contiguous()


def decode_queries(lens):
    """One query per sequence at its last position (packed decode)."""
    return [(s, int(L) - 1) for s, L in enumerate(lens)]


# --- the five workloads of the benchmark description ----------------------

CONFIG_NAMES = {
    1: "f32 MHA decode L=100 Hq=Hkv=4 D=64 ps=16 (7 of 16 pages)",
    2: "bf16 GQA packed decode 64 seqs L~U[512,8192] Hq=32 Hkv=8 D=128 ps=16",
    3: "bf16 GQA split-KV decode 4 seqs x 131072 Hq=64 Hkv=8 D=128 ps=64",
    4: "bf16 causal chunked prefill 8x512 (prior~U[0,4096]) + 120 decode (L~U[256,4096]) Hq=32 Hkv=8 D=128 ps=16",
    5: "bf16 MLA decode 128 seqs L~U[1024,32768] H=128 R=512 P=64 ps=64",
}


def config(n: int, poison: bool = False, shuffle_queries: bool = False) -> Workload:
    """Workload ``n`` (1..5) drawn with seed ``1000 + n``."""
    seed = 1000 + n
    rng = np.random.default_rng(seed)
    bf16 = torch.bfloat16
    if n == 1:
        lens = [100]
        return build_attention(CONFIG_NAMES[1], seed, torch.float32, lens, [(0, 99)],
                               4, 4, 64, 64, 16, pool=16, scale=1 / 8.0,
                               causal=False, poison=poison, rng=rng)
    if n == 2:
        lens = rng.integers(512, 8192, size=64, endpoint=True)
        need = int(sum(-(-int(L) // 16) for L in lens))
        pool = int(math.ceil(1.1 * need))
        return build_attention(CONFIG_NAMES[2], seed, bf16, lens, decode_queries(lens),
                               32, 8, 128, 128, 16, pool=pool, causal=True,
                               poison=poison, rng=rng)
    if n == 3:
        lens = [131072] * 4
        return build_attention(CONFIG_NAMES[3], seed, bf16, lens, decode_queries(lens),
                               64, 8, 128, 128, 64, pool=8192, causal=True,
                               poison=poison, rng=rng)
    if n == 4:
        priors = rng.integers(0, 4096, size=8, endpoint=True)
        dec = rng.integers(256, 4096, size=120, endpoint=True)
        lens = [int(p) + 512 for p in priors] + [int(x) for x in dec]
        queries = []
        for s, p in enumerate(priors):
            queries += [(s, int(p) + j) for j in range(512)]
        queries += [(8 + j, int(x) - 1) for j, x in enumerate(dec)]
        if shuffle_queries:
            order = np.random.default_rng(seed + 100).permutation(len(queries))
            queries = [queries[i] for i in order]
        wl = build_attention(CONFIG_NAMES[4], seed, bf16, lens, queries, 32, 8, 128, 128,
                             16, causal=True, poison=poison, rng=rng)
        wl.info["prefill_queries"] = 8 * 512
        return wl
    if n == 5:
        lens = rng.integers(1024, 32768, size=128, endpoint=True)
        return build_mla(CONFIG_NAMES[5], seed, bf16, lens, decode_queries(lens),
                         128, 512, 64, 64, scale=1 / math.sqrt(192.0), causal=True,
                         poison=poison, rng=rng)
    raise ValueError(f"no workload {n}")


def attention_bytes(wl: Workload) -> int:
    """Algorithmic K/V bytes: every visible (query, KV head) token row read once."""
    es = torch.empty((), dtype=wl.dtype).element_size()
    n = int(wl.visible().sum())
    if wl.kind == "mla":
        r, p = wl.info["r"], wl.info["p"]
        return n * (r + p) * es
    hkv, d, dv = wl.info["hkv"], wl.info["d"], wl.info["dv"]
    return n * hkv * (d + dv) * es


def attention_flops(wl: Workload) -> int:
    """Useful FLOPs: 2 per multiply-add over visible (query, head, key) triples."""
    n = int(wl.visible().sum())
    if wl.kind == "mla":
        h, r, p = wl.info["h"], wl.info["r"], wl.info["p"]
        return n * h * 2 * ((r + p) + r)
    hq, d, dv = wl.info["hq"], wl.info["d"], wl.info["dv"]
    return n * hq * 2 * (d + dv)
