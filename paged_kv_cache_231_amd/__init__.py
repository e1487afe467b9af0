"""Attention over a paged (block-table) KV cache on MI355X — Python binding.

A thin layer over the C ABI of libpkv.so (include/pkv.h): it turns torch
tensors into device pointers, sizes and the current HIP stream, and status
codes into ``PKVError``.  Every step of the computation runs in the
library's HIP kernels; there is no Python or CPU fallback.

    plan = Plan(lens, qseq, qpos, table, page_size, pages)   # one upload
    out = attention(plan, q, k, v, scale, causal=True)        # unsplit
    ws = Workspace(plan.queries, q_heads, value_dim, splits)
    out = attention(plan, q, k, v, scale, workspace=ws)       # split-KV
    out = mla(plan, q_abs, q_pos, latent, k_pos, scale)
    k, v, report = append(plan, new_k, new_v, k, v)          # cache append

Shapes (ruDNN 0.1.7 ``paged_attention`` page, ``DevicePlan::attention`` and
``DevicePlan::mla`` docs): q [Q,Hq,D], k [N,ps,Hkv,D], v [N,ps,Hkv,Dv],
out [Q,Hq,Dv]; MLA q_abs [Q,H,R], q_pos [Q,H,P], latent [N,ps,1,R],
k_pos [N,ps,1,P], out [Q,H,R].
"""

from __future__ import annotations

import ctypes

import numpy as np
import torch

from ._lib import LIB_PATH, AppendReport, PKVError, STATUS, check, lib  # noqa: F401

__all__ = ["Plan", "Workspace", "attention", "attention_noalloc", "attention_fp8", "mla", "append", "encode_plan", "validate_plan",
           "validate_writes", "suggest_splits", "PKVError", "LIB_PATH", "lib", "HEADER_WORDS",
           "MAX_SPLITS"]

HEADER_WORDS = 16
MAX_SPLITS = 256
_DTYPES = {torch.float32: 0, torch.float16: 1, torch.bfloat16: 2}


def _u32_array(x) -> np.ndarray:
    a = np.ascontiguousarray(np.asarray(x).reshape(-1))
    if a.size and (a.min() < 0 or a.max() > 0xFFFFFFFF):
        raise PKVError("ERANGE", "value outside u32")
    return np.ascontiguousarray(a.astype(np.uint32))


def _ptr32(a: np.ndarray):
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_uint32))


def encode_plan(lens, qseq, qpos, table, page_size: int, pages: int) -> np.ndarray:
    """Spec-v1 plan words of a schedule (host only, C++ encoder)."""
    lens_a, qs, qp = _u32_array(lens), _u32_array(qseq), _u32_array(qpos)
    tab = np.asarray(table)
    if tab.ndim != 2 or tab.shape[0] != lens_a.size:
        raise PKVError("EINVAL", "block table must be [sequences, table_width]")
    if qs.size != qp.size:
        raise PKVError("EINVAL", "qseq and qpos differ in length")
    width = int(tab.shape[1])
    for x in (width, int(page_size), int(pages)):
        if x < 0 or x > 0xFFFFFFFF:
            raise PKVError("ERANGE", "plan dimension exceeds u32")
    tab_a = _u32_array(np.where(tab < 0, 0, tab)) if tab.size else np.zeros(0, np.uint32)
    n = ctypes.c_size_t(0)
    args = (lens_a.size, _ptr32(lens_a), qs.size, _ptr32(qs), _ptr32(qp), width, _ptr32(tab_a),
            int(page_size), int(pages))
    check(lib().pkv_plan_encode(*args, None, ctypes.byref(n)))
    words = np.zeros(n.value, dtype=np.uint32)
    check(lib().pkv_plan_encode(*args, _ptr32(words), ctypes.byref(n)))
    return words


def validate_plan(words) -> None:
    w = _u32_array(words)
    check(lib().pkv_plan_validate(_ptr32(w), w.size))


def _stream_handle(stream, device=None) -> int:
    if stream is None:
        stream = torch.cuda.current_stream(device)
    if isinstance(stream, torch.cuda.Stream):
        return int(stream.cuda_stream)
    return int(stream)


class Plan:
    """Immutable uploaded schedule (block table, lengths, positions).

    Bound to the device and stream current at creation; use it on that
    stream.  ``rebind`` / ``set_word`` change the device words in place,
    stream-ordered, keeping the grid-defining header (graph replays stay
    valid).
    """

    def __init__(self, lens, qseq, qpos, table, page_size: int, pages: int, stream=None,
                 words=None):
        self.words = encode_plan(lens, qseq, qpos, table, page_size, pages) if words is None \
            else _u32_array(words)
        self.device = torch.cuda.current_device()
        self.stream = _stream_handle(stream)
        h = ctypes.c_void_p()
        check(lib().pkv_plan_create(_ptr32(self.words), self.words.size,
                                    ctypes.c_void_p(self.stream), ctypes.byref(h)))
        self._h = h
        self._pinned = None
        self._event = None

    @classmethod
    def from_words(cls, words, stream=None) -> "Plan":
        return cls(None, None, None, None, 0, 0, stream=stream, words=words)

    # header fields
    @property
    def queries(self) -> int: return int(self.words[2])
    @property
    def sequences(self) -> int: return int(self.words[3])
    @property
    def table_width(self) -> int: return int(self.words[4])
    @property
    def page_size(self) -> int: return int(self.words[5])
    @property
    def pages(self) -> int: return int(self.words[6])
    @property
    def n_rows(self) -> int: return int(self.words[7])
    @property
    def n_tiles(self) -> int: return int(self.words[8])

    @property
    def handle(self) -> ctypes.c_void_p:
        if self._h is None:
            raise PKVError("EINVAL", "plan is closed")
        return self._h

    def rebind(self, lens, qseq, qpos, table) -> None:
        """New schedule of the same shape, copied stream-ordered from pinned memory."""
        self.rebind_words(encode_plan(lens, qseq, qpos, table, self.page_size, self.pages))

    def rebind_words(self, words) -> None:
        w = _u32_array(words)
        if self._pinned is None or self._pinned.numel() != w.size:
            self._pinned = torch.empty(w.size, dtype=torch.int32, pin_memory=True)
            self._event = torch.cuda.Event()
        else:
            self._event.synchronize()  # the previous copy has read the buffer
        self._pinned.numpy().view(np.uint32)[:] = w
        check(lib().pkv_plan_rebind_async(self.handle, ctypes.c_void_p(self._pinned.data_ptr()),
                                          w.size, ctypes.c_void_p(self.stream)))
        self._event.record(torch.cuda.ExternalStream(self.stream) if self.stream else
                           torch.cuda.default_stream())
        self.words = w.copy()

    def set_word(self, index: int, value: int) -> None:
        """One word, set with hipMemsetD32Async (value passed by copy)."""
        check(lib().pkv_plan_set_word_async(self.handle, int(index), int(value),
                                            ctypes.c_void_p(self.stream)))
        self.words[int(index)] = int(value)

    KERNELS = {"rows": 0, "tiles": 1, "mla": 2, "merge": 3, "append": 4}

    def timing(self, enable: bool = True, kernels=None) -> None:
        """Record HIP events at the start and end of every kernel launched
        with this plan (pkv_plan_timing), or only of the named ``kernels``
        (pkv_plan_timing_select); enabling clears earlier records."""
        if kernels is None:
            check(lib().pkv_plan_timing(self.handle, 1 if enable else 0))
        else:
            mask = sum(1 << self.KERNELS[k] for k in set(kernels)) if enable else 0
            check(lib().pkv_plan_timing_select(self.handle, mask))

    def timing_read(self, kernel: str):
        """(launches, summed milliseconds) of one kernel since timing was enabled."""
        n = ctypes.c_uint32(0)
        ms = ctypes.c_double(0.0)
        check(lib().pkv_plan_timing_read(self.handle, self.KERNELS[kernel], ctypes.byref(n), ctypes.byref(ms)))
        return int(n.value), float(ms.value)

    def close(self) -> None:
        if getattr(self, "_h", None) is not None:
            lib().pkv_plan_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


class Workspace:
    """f32 split partials for ``splits`` parts; reusable across plans with the
    same queries, heads and value dim on the same stream.  ``splits=0`` makes
    a balanced workspace (pkv_workspace_create_balanced): the row queries'
    tiles are cut into equal ranges, one per resident decode wave (attention)
    or per group of 64-head-group blocks, one block per CU (MLA)."""

    def __init__(self, queries: int, heads: int, dv: int, splits: int, stream=None):
        self.stream = _stream_handle(stream)
        self.queries, self.heads, self.dv, self.splits = int(queries), int(heads), int(dv), int(splits)
        h = ctypes.c_void_p()
        if self.splits == 0:
            check(lib().pkv_workspace_create_balanced(self.queries, self.heads, self.dv,
                                                      ctypes.c_void_p(self.stream), ctypes.byref(h)))
        else:
            check(lib().pkv_workspace_create(self.queries, self.heads, self.dv, self.splits,
                                             ctypes.c_void_p(self.stream), ctypes.byref(h)))
        self._h = h

    @classmethod
    def for_splits(cls, queries: int, heads: int, dv: int, splits: int, stream=None):
        """Workspace for a split choice as pkv_tune_splits reports it: None for
        1 (unsplit), balanced for 0, else ``splits`` parts."""
        if splits == 1:
            return None
        return cls(queries, heads, dv, splits, stream=stream)

    @property
    def handle(self):
        if self._h is None:
            raise PKVError("EINVAL", "workspace is closed")
        return self._h

    def close(self) -> None:
        if getattr(self, "_h", None) is not None:
            lib().pkv_workspace_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def suggest_splits(plan: Plan, q_heads: int, kv_heads: int, value_dim: int) -> int:
    """Split count that fills the GPU for this plan (heuristic, capped by the
    workspace limit)."""
    return int(lib().pkv_suggest_splits(plan.handle, int(q_heads), int(kv_heads), int(value_dim)))


def tune_splits(plan: Plan, q, k, v, scale: float, causal: bool = True, out=None,
                reps: int = 5) -> int:
    """Fastest split count for this call, measured on these tensors
    (pkv_tune_splits): 0 means the balanced schedule (``Workspace.for_splits``
    turns the answer into a workspace); synchronises the plan's stream."""
    qn, hq, d = q.shape
    hkv, dv = k.shape[2], v.shape[3]
    if out is None:
        out = torch.empty((qn, hq, dv), dtype=q.dtype, device=q.device)
    code = _dtype_code(q, k, v, out)
    s = ctypes.c_uint32(1)
    check(lib().pkv_tune_splits(plan.handle, code, q.data_ptr(), k.data_ptr(), v.data_ptr(),
                                out.data_ptr(), hq, hkv, d, dv, float(scale), int(bool(causal)),
                                int(reps), ctypes.c_void_p(plan.stream), ctypes.byref(s)))
    return int(s.value)


def tune_splits_mla(plan: Plan, q_abs, q_pos, latent, k_pos, scale: float, causal: bool = True,
                    out=None, reps: int = 5) -> int:
    """Fastest split count for this MLA call (pkv_tune_splits_mla); 0 means
    the balanced schedule."""
    qn, h, r = q_abs.shape
    p = q_pos.shape[2]
    if out is None:
        out = torch.empty((qn, h, r), dtype=q_abs.dtype, device=q_abs.device)
    code = _dtype_code(q_abs, q_pos, latent, k_pos, out)
    s = ctypes.c_uint32(1)
    check(lib().pkv_tune_splits_mla(plan.handle, code, q_abs.data_ptr(), q_pos.data_ptr(),
                                    latent.data_ptr(), k_pos.data_ptr(), out.data_ptr(), h, r, p,
                                    float(scale), int(bool(causal)), int(reps),
                                    ctypes.c_void_p(plan.stream), ctypes.byref(s)))
    return int(s.value)


def _dtype_code(*ts) -> int:
    dt = ts[0].dtype
    for t in ts:
        if t.dtype != dt or not t.is_cuda or not t.is_contiguous():
            raise PKVError("EINVAL", "operands must be contiguous device tensors of one float dtype on one device")
        if t.device != ts[0].device:
            raise PKVError("EINVAL", "operands must be contiguous device tensors of one float dtype on one device")
    if dt not in _DTYPES:
        raise PKVError("EINVAL", "paged operands must be F32, F16 or BF16")
    return _DTYPES[dt]


def attention(plan: Plan, q, k, v, scale: float, causal: bool = True, workspace=None, out=None,
              window: int = 0):
    """Paged MHA/GQA attention; returns ``out`` [Q, Hq, Dv].  ``window`` > 0:
    each query sees only the last ``window`` of its visible keys
    (pkv_attention_window)."""
    if q.dim() != 3 or k.dim() != 4 or v.dim() != 4:
        raise PKVError("EINVAL", "q must be 3-D and the caches 4-D")
    qn, hq, d = q.shape
    n, ps, hkv, dk = k.shape
    dv = v.shape[3]
    if qn != plan.queries or n != plan.pages or ps != plan.page_size or dk != d \
            or tuple(v.shape[:3]) != (n, ps, hkv):
        raise PKVError("ESHAPE", "head counts, head dims or tensor shapes do not fit together")
    if out is None:
        out = torch.empty((qn, hq, dv), dtype=q.dtype, device=q.device)
    elif tuple(out.shape) != (qn, hq, dv):
        raise PKVError("ESHAPE", "head counts, head dims or tensor shapes do not fit together")
    code = _dtype_code(q, k, v, out)
    ws = workspace.handle if workspace is not None else None
    if window:
        if not 0 < int(window) <= 0xFFFFFFFF:
            raise PKVError("ERANGE", "window outside u32")
        check(lib().pkv_attention_window(plan.handle, code, q.data_ptr(), k.data_ptr(),
                                         v.data_ptr(), out.data_ptr(), hq, hkv, d, dv,
                                         float(scale), int(bool(causal)), int(window), ws,
                                         ctypes.c_void_p(plan.stream)))
    else:
        check(lib().pkv_attention(plan.handle, code, q.data_ptr(), k.data_ptr(), v.data_ptr(),
                                  out.data_ptr(), hq, hkv, d, dv, float(scale),
                                  int(bool(causal)), ws, ctypes.c_void_p(plan.stream)))
    return out


def attention_noalloc(plan: Plan, q, k, v, scale: float, causal: bool = True, out=None):
    """pkv_attention_noalloc: the balanced schedule with the library's static
    per-GPU scratch array as its workspace (no device allocation in the
    call; ``out`` must be given for that).  Calls that overlap on one GPU
    race on the array."""
    if q.dim() != 3 or k.dim() != 4 or v.dim() != 4:
        raise PKVError("EINVAL", "q must be 3-D and the caches 4-D")
    qn, hq, d = q.shape
    n, ps, hkv, dk = k.shape
    dv = v.shape[3]
    if qn != plan.queries or n != plan.pages or ps != plan.page_size or dk != d \
            or tuple(v.shape[:3]) != (n, ps, hkv):
        raise PKVError("ESHAPE", "head counts, head dims or tensor shapes do not fit together")
    if out is None:
        out = torch.empty((qn, hq, dv), dtype=q.dtype, device=q.device)
    elif tuple(out.shape) != (qn, hq, dv):
        raise PKVError("ESHAPE", "head counts, head dims or tensor shapes do not fit together")
    code = _dtype_code(q, k, v, out)
    check(lib().pkv_attention_noalloc(plan.handle, code, q.data_ptr(), k.data_ptr(), v.data_ptr(),
                                      out.data_ptr(), hq, hkv, d, dv, float(scale),
                                      int(bool(causal)), ctypes.c_void_p(plan.stream)))
    return out


def attention_fp8(plan: Plan, q, k8, v8, scale: float, k_scale: float, v_scale: float,
                  causal: bool = True, workspace=None, out=None, window: int = 0):
    """Attention over an FP8 E4M3 cache (pkv_attention_fp8): k8 / v8 are
    uint8 tensors [N, ps, Hkv, D] of E4M3 codes, keys = decode * k_scale,
    values = decode * v_scale; q and out F16 or BF16.  Returns ``out``."""
    if q.dim() != 3 or k8.dim() != 4 or v8.dim() != 4:
        raise PKVError("EINVAL", "q must be 3-D and the caches 4-D")
    if k8.dtype != torch.uint8 or v8.dtype != torch.uint8:
        raise PKVError("EINVAL", "FP8 caches are uint8 tensors of E4M3 codes")
    qn, hq, d = q.shape
    n, ps, hkv, dk = k8.shape
    dv = v8.shape[3]
    if qn != plan.queries or n != plan.pages or ps != plan.page_size or dk != d \
            or tuple(v8.shape[:3]) != (n, ps, hkv):
        raise PKVError("ESHAPE", "head counts, head dims or tensor shapes do not fit together")
    if out is None:
        out = torch.empty((qn, hq, dv), dtype=q.dtype, device=q.device)
    elif tuple(out.shape) != (qn, hq, dv):
        raise PKVError("ESHAPE", "head counts, head dims or tensor shapes do not fit together")
    code = _dtype_code(q, out)
    for t in (k8, v8):
        if not t.is_cuda or not t.is_contiguous() or t.device != q.device:
            raise PKVError("EINVAL", "operands must be contiguous device tensors of one float dtype on one device")
    check(lib().pkv_attention_fp8(plan.handle, code, q.data_ptr(), k8.data_ptr(), v8.data_ptr(),
                                  out.data_ptr(), hq, hkv, d, dv, float(scale), float(k_scale),
                                  float(v_scale), int(bool(causal)), int(window),
                                  workspace.handle if workspace is not None else None,
                                  ctypes.c_void_p(plan.stream)))
    return out


def mla(plan: Plan, q_abs, q_pos, latent, k_pos, scale: float, causal: bool = True,
        workspace=None, out=None):
    """Absorbed MLA over one shared latent head; returns ``out`` [Q, H, R]."""
    if latent.dim() != 4 or latent.shape[2] != 1:
        raise PKVError("EINVAL", "the latent cache is [pages, page_size, 1, rank]: one head")
    if q_abs.dim() != 3 or q_pos.dim() != 3 or k_pos.dim() != 4:
        raise PKVError("EINVAL", "q must be 3-D and the caches 4-D")
    qn, h, r = q_abs.shape
    p = q_pos.shape[2]
    n, ps = latent.shape[0], latent.shape[1]
    if qn != plan.queries or n != plan.pages or ps != plan.page_size or latent.shape[3] != r \
            or tuple(q_pos.shape[:2]) != (qn, h) or tuple(k_pos.shape[:3]) != (n, ps, 1) \
            or k_pos.shape[3] != p:
        raise PKVError("ESHAPE", "position dim must be 1..256 and match between q_pos and k_pos")
    if out is None:
        out = torch.empty((qn, h, r), dtype=q_abs.dtype, device=q_abs.device)
    elif tuple(out.shape) != (qn, h, r):
        raise PKVError("ESHAPE", "head counts, head dims or tensor shapes do not fit together")
    code = _dtype_code(q_abs, q_pos, latent, k_pos, out)
    check(lib().pkv_mla(plan.handle, code, q_abs.data_ptr(), q_pos.data_ptr(), latent.data_ptr(),
                        k_pos.data_ptr(), out.data_ptr(), h, r, p, float(scale),
                        int(bool(causal)), workspace.handle if workspace is not None else None,
                        ctypes.c_void_p(plan.stream)))
    return out


def append(plan: Plan, new_k, new_v, k, v, copy=False):
    """Cache append (pkv_append): query i's new_k[i] / new_v[i] ([Hkv, D] /
    [Hkv, Dv]) go to the cache slot of its own position.  ``copy`` (a bool,
    or a (key, value) pair of bools): copy that cache first and append into
    the copy (copy-on-write for a cache that is not uniquely owned), leaving
    the original unchanged.  Returns (k, v, report) with the caches written
    and the report as a dict."""
    if new_k.dim() != 3 or new_v.dim() != 3 or k.dim() != 4 or v.dim() != 4:
        raise PKVError("EINVAL", "append takes 3-D new rows and 4-D caches")
    copy_k, copy_v = (copy, copy) if isinstance(copy, bool) else (bool(copy[0]), bool(copy[1]))
    n, ps, hkv, d = k.shape
    dv = v.shape[3]
    if (n, ps) != (plan.pages, plan.page_size) or tuple(v.shape[:3]) != (n, ps, hkv) \
            or tuple(new_k.shape) != (plan.queries, hkv, d) \
            or tuple(new_v.shape) != (plan.queries, hkv, dv):
        raise PKVError("ESHAPE", "new rows and caches do not match the plan or each other")
    code = _dtype_code(new_k, new_v, k, v)
    kc = torch.empty_like(k) if copy_k and plan.queries else None
    vc = torch.empty_like(v) if copy_v and plan.queries else None
    rep = AppendReport()
    check(lib().pkv_append(plan.handle, code, new_k.data_ptr(), new_v.data_ptr(), k.data_ptr(),
                           v.data_ptr(), kc.data_ptr() if kc is not None else None,
                           vc.data_ptr() if vc is not None else None, hkv, d, dv,
                           ctypes.byref(rep), ctypes.c_void_p(plan.stream)))
    report = {"key_copied": bool(rep.key_copied), "value_copied": bool(rep.value_copied),
              "copied_bytes": int(rep.copied_bytes)}
    return (kc if kc is not None else k), (vc if vc is not None else v), report


def validate_writes(words) -> None:
    """pkv_plan_validate_writes on plan words (host only): raises PKVError
    when two queries would write one cache slot."""
    w = _u32_array(words)
    check(lib().pkv_plan_validate_writes(_ptr32(w), w.size))
