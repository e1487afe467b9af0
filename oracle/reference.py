"""Float64 oracle of paged attention (test infrastructure, not product code).

Written from the ruDNN 0.1.7 ``paged_attention`` module page:
  * module doc: a single module covers MHA, GQA and MLA, both packed decode
    and chunked prefill, with no padded KV gather and no per-head KV repeat;
    non-finite inputs propagate through ordinary arithmetic;
  * ``DevicePlan::attention`` doc: packed Q ``[queries,Hq,D]``, paged K
    ``[pages,page_size,Hkv,D]``, V ``[pages,page_size,Hkv,Dv]``, output
    ``[queries,Hq,Dv]``; ``causal`` masks by the absolute positions held in
    the plan, prefill chunks included;
  * ``execute_attention_into`` shape checks: ``Hq % Hkv == 0``;
  * ``DevicePlan::mla`` doc: MLA is attention with K = V = the shared latent
    head plus a position term, output is the compressed context ``[Q,H,R]``;
  * ``attention_into_split`` doc: the visible history is split into parts and
    the parts are merged through float32 statistics.

The definition computed, for query ``i`` and query head ``h``::

    s = qseq[i];  L = lens[s]
    n = qpos[i] + 1 if causal else L         # visible keys: positions 0..n-1
    g = h // (Hq // Hkv)                      # KV head shared by a q-head group
    for t in 0..n-1:  k_t = K[table[s][t // ps], t % ps, g, :]   (same for v_t)
    x_t = scale * <Q[i,h,:], k_t>
    out[i,h,:] = sum_t exp(x_t - m) v_t / sum_t exp(x_t - m),  m = max_t x_t
    lse[i,h]   = m + log(sum_t exp(x_t - m))

Readings of points the pages leave open (each also listed in the design
notes): the q-head -> KV-head map is contiguous groups ``g = h // G``; a
query's sequence is given explicitly per query; a causal query sees its own
position and every earlier one of its sequence; a split covers a contiguous,
page-aligned range of logical pages, ``ceil(W / splits)`` pages each, where W
is the table width.

Everything is computed in float64 with numpy; half-precision inputs are
widened exactly (bf16/f16 -> f64 is exact).  Queries of one sequence share
one gather of its pages; each query then uses the slice of visible
positions only (no masking by multiplication), with float64 products per
KV head.
"""

from __future__ import annotations

import numpy as np

try:  # torch is only used to widen CPU tensors (bf16 has no numpy dtype)
    import torch
except Exception:  # pragma: no cover - torch is always present in this image
    torch = None


def _f64(x) -> np.ndarray:
    """Widen a numpy array or a CPU torch tensor to a float64 numpy array."""
    if torch is not None and isinstance(x, torch.Tensor):
        return x.detach().to("cpu", torch.float64).numpy()
    return np.asarray(x, dtype=np.float64)


def _take_pages(cache, pages: np.ndarray):
    """cache[pages] for numpy or torch caches (pages: int64 array)."""
    if torch is not None and isinstance(cache, torch.Tensor):
        return cache[torch.as_tensor(pages, dtype=torch.long)]
    return cache[pages]


def visible_count(lens, qseq, qpos, i: int, causal: bool) -> int:
    """Number of keys query ``i`` attends to (positions ``0..n-1``).

    ``DevicePlan::attention`` doc: ``causal`` uses the absolute positions of
    the plan.  A causal query at absolute position ``p`` sees positions
    ``0..p``; a non-causal one sees its whole sequence of length ``L``.
    """
    s = int(qseq[i])
    return int(qpos[i]) + 1 if causal else int(lens[s])


def _gather_tokens(cache, table_row, n: int, page_size: int) -> np.ndarray:
    """Logical tokens ``0..n-1`` of one sequence as float64 ``[n, H, X]``.

    Token ``t`` lives at slot ``t % page_size`` of physical page
    ``table_row[t // page_size]`` (block-table addressing of the paged cache,
    ``DevicePlan::attention`` doc).  Only the first ``n`` slots are widened,
    so unused tail slots of the last page are never read into the result.
    """
    if n == 0:
        shape = tuple(cache.shape)
        return np.zeros((0, shape[2], shape[3]))
    n_pages = -(-n // page_size)
    pages = np.asarray(table_row[:n_pages], dtype=np.int64)
    block = _take_pages(cache, pages)  # [n_pages, ps, H, X]
    h, x = block.shape[2], block.shape[3]
    block = block.reshape(n_pages * page_size, h, x)[:n]
    return _f64(block)


def _softmax_pv(x: np.ndarray, vals: np.ndarray):
    """Softmax over the last axis of ``x`` and the weighted sum of ``vals``.

    x [..., T] scores of the visible keys only; vals [T, Dv] (or broadcastable
    batch ``[..., T, Dv]``).  Returns (out [..., Dv], lse [...]).  With T = 0
    (an empty part of a split) out = 0 and lse = -inf.  Only visible keys
    are passed in, so a NaN in a visible key or value propagates and nothing
    invisible is ever multiplied in.
    """
    if x.shape[-1] == 0:
        return np.zeros(x.shape[:-1] + (vals.shape[-1],)), np.full(x.shape[:-1], -np.inf)
    m = np.max(x, axis=-1, keepdims=True)
    w = np.exp(x - m)
    l = w.sum(axis=-1)
    out = (w @ vals) / l[..., None]
    lse = m[..., 0] + np.log(l)
    return out, lse


def _queries_by_sequence(qseq):
    groups: dict[int, list[int]] = {}
    for i, s in enumerate(np.asarray(qseq).tolist()):
        groups.setdefault(int(s), []).append(i)
    return groups


def window_start(n: int, window: int) -> int:
    """First visible position under a sliding window of ``window`` keys.

    Reading of the ``window`` field of the libmir-cuda 0.1.0 decode-attention
    geometry (its `Geometry` struct; the page shows the field, not its
    use): a query whose visible keys are positions ``[0, n)`` sees only the
    last ``window`` of them, ``[max(0, n - window), n)``; 0 means no window.
    """
    return max(0, n - window) if window > 0 else 0


def _visible_range(n: int, token_range, window: int = 0):
    """Logical positions ``[lo, hi)`` a query uses: ``[0, n)`` cut to the
    sliding window, then to the part."""
    w0 = window_start(n, window)
    if token_range is None:
        return w0, n
    lo, hi = token_range
    lo, hi = min(max(lo, w0), n), min(max(hi, 0), n)
    return lo, max(lo, hi)


def _is_torch(x) -> bool:
    return torch is not None and isinstance(x, torch.Tensor)


def _rows(x, idx):
    """x[idx] widened to float64 (idx: list of query indices)."""
    if _is_torch(x):
        return _f64(x[torch.as_tensor(idx, dtype=torch.long)])
    return _f64(np.asarray(x)[np.asarray(idx, dtype=np.int64)])


def paged_attention(q, k, v, lens, qseq, qpos, table, page_size: int,
                    scale: float, causal: bool, token_range=None, window: int = 0):
    """Paged MHA/GQA attention in float64.

    q [Q,Hq,D], k [N,ps,Hkv,D], v [N,ps,Hkv,Dv] (numpy or CPU torch);
    lens [S], qseq [Q], qpos [Q], table [S,W] integers.
    ``token_range = (lo, hi)`` restricts every query to the visible keys with
    logical position in ``[lo, hi)`` (one part of a split); parts with no
    visible key give out = 0 and lse = -inf.  ``window`` > 0 keeps only the
    last ``window`` visible keys (``window_start``).
    Returns (out [Q,Hq,Dv] float64, lse [Q,Hq] float64, natural log).
    """
    qn = int(q.shape[0])
    hq = int(q.shape[1])
    hkv, dv = int(k.shape[2]), int(v.shape[3])
    assert hq % hkv == 0, "Hq must be a multiple of Hkv"
    grp = hq // hkv
    out = np.zeros((qn, hq, dv))
    lse = np.full((qn, hq), -np.inf)
    table = np.asarray(table)
    for s, idx in _queries_by_sequence(qseq).items():
        n_max = max(visible_count(lens, qseq, qpos, i, causal) for i in idx)
        kk = _gather_tokens(k, table[s], n_max, page_size)  # [n, Hkv, D]
        vv = _gather_tokens(v, table[s], n_max, page_size)  # [n, Hkv, Dv]
        qq = _rows(q, idx)                                  # [nq, Hq, D]
        for j, i in enumerate(idx):
            lo, hi = _visible_range(visible_count(lens, qseq, qpos, i, causal), token_range, window)
            kg = kk[lo:hi].transpose(1, 2, 0)       # [Hkv, D, t]
            vg = vv[lo:hi].transpose(1, 0, 2)       # [Hkv, t, Dv]
            qg = qq[j].reshape(hkv, grp, -1)        # head h = g*G + r -> [g, r, :]
            x = scale * (qg @ kg)                   # [Hkv, G, t]
            o, l = _softmax_pv(x, vg)               # [Hkv, G, Dv], [Hkv, G]
            out[i] = o.reshape(hq, dv)
            lse[i] = l.reshape(hq)
    return out, lse


def paged_mla(q_abs, q_pos, latent, k_pos, lens, qseq, qpos, table,
              page_size: int, scale: float, causal: bool, token_range=None):
    """Absorbed MLA in float64 (``DevicePlan::mla`` doc).

    q_abs [Q,H,R], q_pos [Q,H,P], latent [N,ps,1,R], k_pos [N,ps,1,P].
    The single latent head is both key and value; the position part only
    adds to the score:
        x_t = scale * (<q_abs[i,h], latent_t> + <q_pos[i,h], k_pos_t>)
        out[i,h] = sum_t softmax(x)_t * latent_t        -> [Q,H,R]
    Returns (out, lse) as ``paged_attention`` does.
    """
    qn, hh, r = (int(x) for x in q_abs.shape)
    out = np.zeros((qn, hh, r))
    lse = np.full((qn, hh), -np.inf)
    table = np.asarray(table)
    for s, idx in _queries_by_sequence(qseq).items():
        n_max = max(visible_count(lens, qseq, qpos, i, causal) for i in idx)
        lat = _gather_tokens(latent, table[s], n_max, page_size)[:, 0, :]  # [n, R]
        kp = _gather_tokens(k_pos, table[s], n_max, page_size)[:, 0, :]    # [n, P]
        qa = _rows(q_abs, idx)
        qp = _rows(q_pos, idx)
        for j, i in enumerate(idx):
            lo, hi = _visible_range(visible_count(lens, qseq, qpos, i, causal), token_range)
            x = scale * (qa[j] @ lat[lo:hi].T + qp[j] @ kp[lo:hi].T)  # [H, t]
            o, l = _softmax_pv(x, lat[lo:hi])
            out[i] = o
            lse[i] = l
    return out, lse


def split_ranges(table_width: int, page_size: int, splits: int):
    """Logical token ranges of the parts of a split.

    Reading of the ``attention_into_split`` doc, which divides a query's
    visible keys among several parts: part ``j`` covers the contiguous, page-aligned
    pages ``[j*pp, (j+1)*pp)`` of the block-table row, ``pp = ceil(W/splits)``,
    i.e. tokens ``[j*pp*ps, (j+1)*pp*ps)``.  The partition depends only on
    the table width, so it is fixed for a plan's shape; parts past a query's
    visible range are empty.
    """
    assert splits >= 1 and table_width >= 1
    pp = -(-table_width // splits)
    return [(j * pp * page_size, (j + 1) * pp * page_size) for j in range(splits)]


def merge_partials(o_parts, lse_parts):
    """Merge normalised partial outputs through their log-sum-exp statistics.

    o_parts [S, ..., Dv], lse_parts [S, ...] (natural log, -inf = empty part):
        M = max_s lse_s,  w_s = exp(lse_s - M)
        out = sum_s w_s o_s / sum_s w_s,   lse = M + log(sum_s w_s)
    This is the float32-statistics merge of the ``attention_into_split``
    doc, here in float64.
    """
    o_parts = np.asarray(o_parts, dtype=np.float64)
    lse_parts = np.asarray(lse_parts, dtype=np.float64)
    m = np.max(lse_parts, axis=0)
    safe_m = np.where(np.isfinite(m), m, 0.0)
    w = np.where(np.isfinite(lse_parts), np.exp(lse_parts - safe_m[None]), 0.0)
    wsum = w.sum(axis=0)
    empty = wsum == 0  # every part empty: no visible key at all
    denom = np.where(empty, 1.0, wsum)
    out = np.where(empty[..., None], 0.0, (w[..., None] * o_parts).sum(axis=0) / denom[..., None])
    lse = np.where(empty, -np.inf, safe_m + np.log(denom))
    return out, lse


def paged_attention_split(q, k, v, lens, qseq, qpos, table, page_size: int,
                          scale: float, causal: bool, splits: int, window: int = 0):
    """Split-KV attention: per-part attention, then ``merge_partials``."""
    w = int(np.asarray(table).shape[1])
    parts = [paged_attention(q, k, v, lens, qseq, qpos, table, page_size, scale,
                             causal, token_range=rg, window=window)
             for rg in split_ranges(w, page_size, splits)]
    return merge_partials([p[0] for p in parts], [p[1] for p in parts])


def paged_mla_split(q_abs, q_pos, latent, k_pos, lens, qseq, qpos, table,
                    page_size: int, scale: float, causal: bool, splits: int):
    """Split-KV MLA: per-part MLA, then ``merge_partials``."""
    w = int(np.asarray(table).shape[1])
    parts = [paged_mla(q_abs, q_pos, latent, k_pos, lens, qseq, qpos, table,
                       page_size, scale, causal, token_range=rg)
             for rg in split_ranges(w, page_size, splits)]
    return merge_partials([p[0] for p in parts], [p[1] for p in parts])


def attention_one(q, k, v, lens, qseq, qpos, table, page_size, scale, causal, i, h,
                  window: int = 0):
    """One output row ``out[i, h, :]`` computed on its own (for sampling big
    workloads): the same definition as ``paged_attention``, one query, one head.
    """
    hq, hkv = int(q.shape[1]), int(k.shape[2])
    g = h // (hq // hkv)
    s = int(qseq[i])
    n = visible_count(lens, qseq, qpos, i, causal)
    lo = window_start(n, window)
    kk = _gather_tokens(k, np.asarray(table)[s], n, page_size)[lo:, g, :]
    vv = _gather_tokens(v, np.asarray(table)[s], n, page_size)[lo:, g, :]
    qv = _f64(q[i, h])
    x = scale * (kk @ qv)
    o, l = _softmax_pv(x[None, :], vv)
    return o[0], float(l[0])


def mla_one(q_abs, q_pos, latent, k_pos, lens, qseq, qpos, table, page_size,
            scale, causal, i, h):
    """One MLA output row ``out[i, h, :]`` (same definition as ``paged_mla``)."""
    s = int(qseq[i])
    n = visible_count(lens, qseq, qpos, i, causal)
    row = np.asarray(table)[s]
    lat = _gather_tokens(latent, row, n, page_size)[:, 0, :]
    kp = _gather_tokens(k_pos, row, n, page_size)[:, 0, :]
    x = scale * (lat @ _f64(q_abs[i, h]) + kp @ _f64(q_pos[i, h]))
    o, l = _softmax_pv(x[None, :], lat)
    return o[0], float(l[0])


__all__ = [
    "visible_count", "window_start", "paged_attention", "paged_mla", "split_ranges",
    "merge_partials", "paged_attention_split", "paged_mla_split",
    "attention_one", "mla_one",
]

