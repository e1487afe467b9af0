"""Oracle of attention over an 8-bit (FP8 E4M3) KV cache: test
infrastructure, not product code.

The libmir-cuda 0.1.0 attention ``graph`` page keeps its K and V caches as
byte buffers (``DeviceBuffer<u8>``) next to bf16 queries and outputs, and
shows no encoding.  Reading taken here: one byte per element in the OCP FP8
E4M3 format (1 sign bit, 4 exponent bits with bias 7, 3 mantissa bits;
exponent 0 is subnormal; S.1111.111 is NaN; there is no infinity), and one
f32 scale per cache: key = decode(byte) * k_scale, value = decode(byte) *
v_scale.  Attention is then exactly ``paged_attention`` on the decoded
caches.

Pins: ``tests/test_oracle_fp8.py`` (all 256 codes against torch's
float8_e4m3fn conversion, hand values, attention = attention on the decoded
caches, scale folding).
"""

from __future__ import annotations

import numpy as np

try:
    import torch
except ImportError:  # numpy caches only
    torch = None

from .reference import paged_attention, attention_one


def e4m3_decode(codes) -> np.ndarray:
    """float64 values of E4M3 byte codes (any integer array)."""
    c = np.asarray(codes, dtype=np.int64) & 0xFF
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = c & 0x7
    normal = sign * np.ldexp(1.0 + m / 8.0, (e - 7).astype(np.int64))
    sub = sign * np.ldexp(m / 8.0, -6)
    out = np.where(e == 0, sub, normal)
    return np.where((c & 0x7F) == 0x7F, np.nan, out)


def _decoded(cache_codes, scale: float):
    x = cache_codes.numpy() if hasattr(cache_codes, "numpy") else np.asarray(cache_codes)
    return e4m3_decode(x) * float(scale)


def paged_attention_fp8(q, k8, v8, lens, qseq, qpos, table, page_size: int, scale: float,
                        causal: bool, k_scale: float, v_scale: float, window: int = 0):
    """Attention over E4M3 caches: ``paged_attention`` on the decoded,
    scaled caches (float64).  k8 [N,ps,Hkv,D], v8 [N,ps,Hkv,Dv] byte codes."""
    return paged_attention(q, _decoded(k8, k_scale), _decoded(v8, v_scale), lens, qseq, qpos,
                           table, page_size, scale, causal, window=window)


def attention_one_fp8(q, k8, v8, lens, qseq, qpos, table, page_size, scale, causal, i, h,
                      k_scale, v_scale, window: int = 0):
    """One output row of ``paged_attention_fp8``: only the pages of query i's
    sequence are decoded (the same definition, on a one-sequence cache)."""
    s = int(qseq[i])
    n_pages = -(-int(lens[s]) // page_size)
    pages = np.asarray(table)[s, :n_pages].astype(np.int64)
    idx = torch.as_tensor(pages) if torch is not None and isinstance(k8, torch.Tensor) else pages
    k_c, v_c = _decoded(k8[idx], k_scale), _decoded(v8[idx], v_scale)
    return attention_one(q[i:i + 1], k_c, v_c, [int(lens[s])], [0], [int(qpos[i])],
                         np.arange(n_pages)[None, :], page_size, scale, causal, 0, h,
                         window=window)
