"""Paged Multi-head Latent Attention for AMD MI355X (gfx950).

A thin Python binding over the C ABI of ``libmla.so`` (include/mla.h).  It
only marshals arguments: every step of the attention runs in the library's
HIP kernels; PyTorch supplies device memory and streams.  The functions keep
the C names (``mla_plan_create``, ``mla_plan``, ``mla_run``,
``mla_merge_state``, ``mla_plan_destroy``); :class:`MLAPlan` bundles them.

Interface after the m-star page "mstar.engine.resources.attn.flashinfer_mla"
(FlashInferMLAWrapper: constructor, plan, run).
"""

from __future__ import annotations

import ctypes
from ctypes import c_int32, c_int64, c_void_p
from typing import Optional

import numpy as np

from . import _native

KV_LORA_RANK = 512
QK_ROPE_HEAD_DIM = 64

__all__ = [
    "MLAPlan", "mla_plan_create", "mla_plan", "mla_run", "mla_append_kv", "mla_merge_state",
    "mla_absorb_query", "mla_up_project", "absorb_query", "up_project",
    "mla_plan_destroy", "mla_plan_stats", "merge_state", "schedule", "append_rows", "library",
    "mla_run_noalloc", "run_noalloc", "mla_run_fp8", "mla_append_kv_fp8",
]


def library():
    """The loaded product library (raises if it is not built)."""
    return _native.load(_native.LIB_PATH)


def _host_i32(x) -> np.ndarray:
    """Index arrays are read on the host.  A GPU tensor costs a device sync."""
    try:
        import torch
        if isinstance(x, torch.Tensor):
            x = x.detach().to("cpu").numpy()
    except ImportError:  # pragma: no cover
        pass
    return np.ascontiguousarray(np.asarray(x), dtype=np.int32)


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.POINTER(c_int32))


def _stream_handle(stream) -> Optional[int]:
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _dev_ptr(t, name, dtype, shape):
    import torch
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be on the GPU")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t.data_ptr()


# ----------------------------------------------------------------------------
# C-named functions
# ----------------------------------------------------------------------------

def mla_plan_create(device: int, num_heads: int, kv_lora_rank: int = KV_LORA_RANK,
                    qk_rope_head_dim: int = QK_ROPE_HEAD_DIM, page_size: int = 64) -> int:
    lib = library()
    h = c_void_p()
    _native.check(lib, lib.mla_plan_create(ctypes.byref(h), device, num_heads, kv_lora_rank,
                                           qk_rope_head_dim, page_size))
    return h.value


def mla_plan(handle: int, qo_indptr, kv_indptr, kv_indices, kv_last_page_len, causal: bool,
             sm_scale: float, num_cache_pages: int, stream: int) -> None:
    lib = library()
    qo, kv = _host_i32(qo_indptr), _host_i32(kv_indptr)
    idx, last = _host_i32(kv_indices), _host_i32(kv_last_page_len)
    batch = qo.shape[0] - 1
    if kv.shape[0] != batch + 1 or last.shape[0] != batch:
        raise ValueError("qo_indptr, kv_indptr and kv_last_page_len disagree on the batch size")
    if idx.size == 0:
        idx = np.zeros(1, np.int32)
    _native.check(lib, lib.mla_plan(handle, _ptr(qo), _ptr(kv), _ptr(idx), _ptr(last), batch,
                                    1 if causal else 0, float(sm_scale), int(num_cache_pages),
                                    stream))


def mla_run(handle: int, q_nope_ptr: int, q_pe_ptr: int, kv_cache_ptr: int, out_ptr: int,
            lse_ptr: Optional[int], stream: int) -> None:
    lib = library()
    _native.check(lib, lib.mla_run(handle, q_nope_ptr, q_pe_ptr, kv_cache_ptr, out_ptr,
                                   lse_ptr, stream))


def mla_run_fp8(handle: int, q_nope_ptr: int, q_pe_ptr: int, kv_cache_ptr: int, kv_scale: float,
                out_ptr: int, lse_ptr: Optional[int], stream: int) -> None:
    lib = library()
    _native.check(lib, lib.mla_run_fp8(handle, q_nope_ptr, q_pe_ptr, kv_cache_ptr,
                                       float(kv_scale), out_ptr, lse_ptr, stream))


def mla_append_kv(handle: int, ckv_ptr: int, kpe_ptr: int, kv_cache_ptr: int,
                  stream: int) -> None:
    lib = library()
    _native.check(lib, lib.mla_append_kv(handle, ckv_ptr, kpe_ptr, kv_cache_ptr, stream))


def mla_append_kv_fp8(handle: int, ckv_ptr: int, kpe_ptr: int, kv_cache_ptr: int,
                      kv_scale: float, stream: int) -> None:
    lib = library()
    _native.check(lib, lib.mla_append_kv_fp8(handle, ckv_ptr, kpe_ptr, kv_cache_ptr,
                                             float(kv_scale), stream))


def _kv_dtype(kv_dtype):
    """The cache dtype a plan is made for: None / bfloat16 (the default) or
    an fp8 E4M3 cache ("fp8_e4m3" or torch.float8_e4m3fn)."""
    if kv_dtype is None:
        return "bf16"
    name = str(kv_dtype).replace("torch.", "")
    if name in ("bf16", "bfloat16"):
        return "bf16"
    if name in ("fp8_e4m3", "float8_e4m3fn", "e4m3"):
        return "fp8_e4m3"
    raise ValueError(f"unsupported kv_dtype {kv_dtype!r} (bf16 or fp8_e4m3)")


def mla_merge_state(v_a: int, s_a: int, v_b: int, s_b: int, v_out: int, s_out: int,
                    num_tokens: int, num_heads: int, stream: int) -> None:
    lib = library()
    _native.check(lib, lib.mla_merge_state(v_a, s_a, v_b, s_b, v_out, s_out, num_tokens,
                                           num_heads, stream))


def mla_plan_destroy(handle: int) -> None:
    if handle:
        library().mla_plan_destroy(handle)


def mla_plan_stats(handle: int) -> dict:
    lib = library()
    w, n, s, p = c_int32(), c_int64(), c_int64(), c_int64()
    _native.check(lib, lib.mla_plan_stats(handle, ctypes.byref(w), ctypes.byref(n),
                                          ctypes.byref(s), ctypes.byref(p)))
    return {"num_workers": w.value, "num_items": n.value, "num_split_tokens": s.value,
            "num_partials": p.value}


# ----------------------------------------------------------------------------
# Torch-facing wrapper
# ----------------------------------------------------------------------------

class MLAPlan:
    """One plan handle: ``plan(...)`` on host index arrays, then ``run(...)``.

    Mirrors FlashInferMLAWrapper(num_qo_heads, kv_lora_rank, qk_rope_head_dim,
    page_size) with ``plan(qo_indptr, paged_kv_indptr, paged_kv_indices,
    paged_kv_last_page_len, causal=True)`` and ``run(q_nope, q_pe,
    kv_cache_layer, return_lse=False)``.
    """

    def __init__(self, num_heads: int, page_size: int, kv_lora_rank: int = KV_LORA_RANK,
                 qk_rope_head_dim: int = QK_ROPE_HEAD_DIM, device: Optional[int] = None):
        import torch
        if device is None:
            device = torch.cuda.current_device()
        self.device = int(device)
        self.num_heads = int(num_heads)
        self.page_size = int(page_size)
        self._h = mla_plan_create(self.device, self.num_heads, kv_lora_rank, qk_rope_head_dim,
                                  self.page_size)
        self._planned = None
        self.kv_dtype = "bf16"

    def reserve(self, max_batch: int, max_tokens: int, max_kv_indices: int) -> None:
        """Fix the plan's capacity so that a captured ``run`` stays valid while
        later ``plan`` calls change the batch (see mla_plan_reserve)."""
        lib = library()
        _native.check(lib, lib.mla_plan_reserve(self._h, int(max_batch), int(max_tokens),
                                                int(max_kv_indices)))
        self._planned = None
        self._reserved_tokens = int(max_tokens)

    def plan(self, qo_indptr, kv_indptr, kv_indices, kv_last_page_len, causal: bool = True,
             sm_scale: float = 192.0 ** -0.5, num_cache_pages: Optional[int] = None,
             stream=None, kv_dtype=None) -> None:
        """``kv_dtype`` None (bf16 cache) or "fp8_e4m3" (E4M3 codes with one
        fp32 scale, given to ``run`` / ``append_kv`` as ``kv_scale``)."""
        qo = _host_i32(qo_indptr)
        if num_cache_pages is None:
            raise ValueError("num_cache_pages is required (page ids are validated against it)")
        dt = _kv_dtype(kv_dtype)
        mla_plan(self._h, qo, kv_indptr, kv_indices, kv_last_page_len, causal, sm_scale,
                 num_cache_pages, _stream_handle(stream))
        self._planned = (int(qo[-1]), int(num_cache_pages))
        self.kv_dtype = dt

    def _cache_ptr(self, kv_cache, pages, kv_scale):
        import torch
        if kv_cache.dim() != 3 or kv_cache.shape[0] < pages:
            raise ValueError(f"kv_cache must be [>= {pages}, page_size, 576]")
        shape = (kv_cache.shape[0], self.page_size, KV_LORA_RANK + QK_ROPE_HEAD_DIM)
        if self.kv_dtype == "bf16":
            if kv_scale is not None:
                raise ValueError("kv_scale is for an fp8 cache (plan with kv_dtype='fp8_e4m3')")
            return _dev_ptr(kv_cache, "kv_cache", torch.bfloat16, shape)
        if kv_scale is None:
            raise ValueError("an fp8 cache needs kv_scale")
        if kv_cache.dtype not in (torch.uint8, torch.float8_e4m3fn):
            raise ValueError(f"an fp8 cache is uint8 or float8_e4m3fn, got {kv_cache.dtype}")
        return _dev_ptr(kv_cache, "kv_cache", kv_cache.dtype, shape)

    def run(self, q_nope, q_pe, kv_cache, return_lse: bool = False, out=None, lse=None,
            stream=None, kv_scale: Optional[float] = None):
        import torch
        if self._planned is None:
            raise RuntimeError("run() before plan()")
        T, pages = self._planned
        H = self.num_heads
        if getattr(self, "_reserved_tokens", None):
            T = self._reserved_tokens  # tensors sized for the reserved capacity
        kv = self._cache_ptr(kv_cache, pages, kv_scale)
        qn = _dev_ptr(q_nope, "q_nope", torch.bfloat16, (T, H, KV_LORA_RANK))
        qp = _dev_ptr(q_pe, "q_pe", torch.bfloat16, (T, H, QK_ROPE_HEAD_DIM))
        if out is None:
            out = torch.empty((T, H, KV_LORA_RANK), dtype=torch.bfloat16, device=q_nope.device)
        op = _dev_ptr(out, "out", torch.bfloat16, (T, H, KV_LORA_RANK))
        lp = None
        if return_lse or lse is not None:
            if lse is None:
                lse = torch.empty((T, H), dtype=torch.float32, device=q_nope.device)
            lp = _dev_ptr(lse, "lse", torch.float32, (T, H))
        if self.kv_dtype == "bf16":
            mla_run(self._h, qn, qp, kv, op, lp, _stream_handle(stream))
        else:
            mla_run_fp8(self._h, qn, qp, kv, kv_scale, op, lp, _stream_handle(stream))
        return (out, lse) if (return_lse or lp is not None) else out

    def append_kv(self, ckv, kpe, kv_cache, stream=None, kv_scale: Optional[float] = None) -> None:
        """Write this step's latent rows (``ckv [T, 512]``, ``kpe [T, 64]``
        bf16) into ``kv_cache`` in place: token i of a row with Q tokens and
        L keys becomes the row's key L - Q + i (mirrors the KV write a layer
        makes before ``run``).  An fp8 cache stores the E4M3 codes of
        ``x / kv_scale``."""
        import torch
        if self._planned is None:
            raise RuntimeError("append_kv() before plan()")
        T, pages = self._planned
        kv = self._cache_ptr(kv_cache, pages, kv_scale)
        cp = _dev_ptr(ckv, "ckv", torch.bfloat16, (T, KV_LORA_RANK))
        pp = _dev_ptr(kpe, "kpe", torch.bfloat16, (T, QK_ROPE_HEAD_DIM))
        if self.kv_dtype == "bf16":
            mla_append_kv(self._h, cp, pp, kv, _stream_handle(stream))
        else:
            mla_append_kv_fp8(self._h, cp, pp, kv, kv_scale, _stream_handle(stream))

    def stats(self) -> dict:
        return mla_plan_stats(self._h)

    def close(self) -> None:
        if getattr(self, "_h", None):
            mla_plan_destroy(self._h)
            self._h = None

    def __del__(self):  # pragma: no cover
        try:
            self.close()
        except Exception:
            pass


def mla_absorb_query(q_nope: int, w_uk: int, q_abs: int, num_tokens: int, num_heads: int,
                     stream: int) -> None:
    lib = library()
    _native.check(lib, lib.mla_absorb_query(q_nope, w_uk, q_abs, num_tokens, num_heads, stream))


def mla_up_project(o: int, w_uv: int, v: int, num_tokens: int, num_heads: int,
                   stream: int) -> None:
    lib = library()
    _native.check(lib, lib.mla_up_project(o, w_uv, v, num_tokens, num_heads, stream))


NOPE_HEAD_DIM = 128
V_HEAD_DIM = 128


def absorb_query(q_nope, w_uk, out=None, stream=None):
    """``q_nope [T, H, 128] @ w_uk [H, 128, 512]`` per head -> ``[T, H, 512]``
    (bf16 tensors on the GPU)."""
    import torch
    T, H = int(q_nope.shape[0]), int(q_nope.shape[1])
    if out is None:
        out = torch.empty((T, H, KV_LORA_RANK), dtype=torch.bfloat16, device=q_nope.device)
    mla_absorb_query(_dev_ptr(q_nope, "q_nope", torch.bfloat16, (T, H, NOPE_HEAD_DIM)),
                     _dev_ptr(w_uk, "w_uk", torch.bfloat16, (H, NOPE_HEAD_DIM, KV_LORA_RANK)),
                     _dev_ptr(out, "out", torch.bfloat16, (T, H, KV_LORA_RANK)), T, H,
                     _stream_handle(stream))
    return out


def up_project(o, w_uv, out=None, stream=None):
    """``o [T, H, 512] @ w_uv [H, 512, 128]`` per head -> ``[T, H, 128]``
    (bf16 tensors on the GPU)."""
    import torch
    T, H = int(o.shape[0]), int(o.shape[1])
    if out is None:
        out = torch.empty((T, H, V_HEAD_DIM), dtype=torch.bfloat16, device=o.device)
    mla_up_project(_dev_ptr(o, "o", torch.bfloat16, (T, H, KV_LORA_RANK)),
                   _dev_ptr(w_uv, "w_uv", torch.bfloat16, (H, KV_LORA_RANK, V_HEAD_DIM)),
                   _dev_ptr(out, "out", torch.bfloat16, (T, H, V_HEAD_DIM)), T, H,
                   _stream_handle(stream))
    return out


def merge_state(v_a, s_a, v_b, s_b, v_out=None, s_out=None, stream=None):
    """LSE merge of two results over disjoint key segments (bf16 v, fp32 s)."""
    import torch
    if v_a.dim() != 3 or v_a.shape[-1] != KV_LORA_RANK:
        raise ValueError("v_a must be [T, H, 512]")
    T, H = int(v_a.shape[0]), int(v_a.shape[1])
    if v_out is None:
        v_out = torch.empty_like(v_a)
    if s_out is None:
        s_out = torch.empty_like(s_a)
    ptrs = [
        _dev_ptr(v_a, "v_a", torch.bfloat16, (T, H, KV_LORA_RANK)),
        _dev_ptr(s_a, "s_a", torch.float32, (T, H)),
        _dev_ptr(v_b, "v_b", torch.bfloat16, (T, H, KV_LORA_RANK)),
        _dev_ptr(s_b, "s_b", torch.float32, (T, H)),
        _dev_ptr(v_out, "v_out", torch.bfloat16, (T, H, KV_LORA_RANK)),
        _dev_ptr(s_out, "s_out", torch.float32, (T, H)),
    ]
    mla_merge_state(*ptrs, T, H, _stream_handle(stream))
    return v_out, s_out


def mla_run_noalloc(qo_indptr: int, kv_indptr: int, kv_indices: int, kv_last_page_len: int,
                    batch: int, num_tokens: int, num_kv_indices: int, causal: bool,
                    sm_scale: float, num_cache_pages: int, max_kv_len: int, num_heads: int,
                    page_size: int, q_nope: int, q_pe: int, kv_cache: int, out: int, lse: int,
                    stream: Optional[int]) -> None:
    lib = library()
    _native.check(lib, lib.mla_run_noalloc(qo_indptr, kv_indptr, kv_indices, kv_last_page_len,
                                           batch, num_tokens, num_kv_indices, 1 if causal else 0,
                                           sm_scale, num_cache_pages, max_kv_len, num_heads,
                                           page_size, q_nope, q_pe, kv_cache, out, lse, stream))


def run_noalloc(qo_indptr, kv_indptr, kv_indices, kv_last_page_len, q_nope, q_pe, kv_cache,
                page_size: int, max_kv_len: int, causal: bool = True, sm_scale: float = None,
                out=None, lse=None, return_lse: bool = False, stream=None):
    """mla_run_noalloc with torch tensors: the page table as int32 GPU
    tensors, everything else as for MLAPlan.run.  Allocates only what the
    caller did not pass (out, lse); the library allocates nothing."""
    import torch
    if sm_scale is None:
        raise ValueError("sm_scale is required")
    if q_nope.dim() != 3 or q_nope.shape[-1] != KV_LORA_RANK:
        raise ValueError("q_nope must be [T, H, 512]")
    T, H = int(q_nope.shape[0]), int(q_nope.shape[1])
    B = int(qo_indptr.shape[0]) - 1
    nnz = int(kv_indices.shape[0])
    if kv_cache.dim() != 3 or kv_cache.shape[1:] != (page_size, KV_LORA_RANK + QK_ROPE_HEAD_DIM):
        raise ValueError("kv_cache must be [pages, page_size, 576]")
    pages = int(kv_cache.shape[0])
    if out is None:
        out = torch.empty((T, H, KV_LORA_RANK), dtype=torch.bfloat16, device=q_nope.device)
    if lse is None and return_lse:
        lse = torch.empty((T, H), dtype=torch.float32, device=q_nope.device)
    mla_run_noalloc(
        _dev_ptr(qo_indptr, "qo_indptr", torch.int32, (B + 1,)),
        _dev_ptr(kv_indptr, "kv_indptr", torch.int32, (B + 1,)),
        _dev_ptr(kv_indices, "kv_indices", torch.int32, (nnz,)) if nnz else None,
        _dev_ptr(kv_last_page_len, "kv_last_page_len", torch.int32, (B,)),
        B, T, nnz, causal, float(sm_scale), pages, int(max_kv_len), H, page_size,
        _dev_ptr(q_nope, "q_nope", torch.bfloat16, (T, H, KV_LORA_RANK)),
        _dev_ptr(q_pe, "q_pe", torch.bfloat16, (T, H, QK_ROPE_HEAD_DIM)),
        _dev_ptr(kv_cache, "kv_cache", torch.bfloat16, tuple(kv_cache.shape)),
        _dev_ptr(out, "out", torch.bfloat16, (T, H, KV_LORA_RANK)),
        _dev_ptr(lse, "lse", torch.float32, (T, H)) if lse is not None else None,
        _stream_handle(stream))
    return (out, lse) if return_lse else out


# ----------------------------------------------------------------------------
# Host-only planner output (no GPU needed)
# ----------------------------------------------------------------------------

def schedule(qo_indptr, kv_indptr, kv_indices, kv_last_page_len, page_size: int,
             num_cache_pages: int, num_heads: int, num_workers: int, causal: bool = True,
             lib_path: Optional[str] = None) -> dict:
    """Run the host planner and return its schedule as numpy arrays:
    worker_indptr [num_workers + 2] (the last two entries bound the shared
    pool), items [num_items, 8], merges [num_merges, 4]."""
    lib = _native.load(lib_path or _native.LIB_PATH, host_only=True)
    qo, kv = _host_i32(qo_indptr), _host_i32(kv_indptr)
    idx, last = _host_i32(kv_indices), _host_i32(kv_last_page_len)
    if idx.size == 0:
        idx = np.zeros(1, np.int32)
    h = c_void_p()
    _native.check(lib, lib.mla_schedule_build(ctypes.byref(h), _ptr(qo), _ptr(kv), _ptr(idx),
                                              _ptr(last), qo.shape[0] - 1, 1 if causal else 0,
                                              page_size, num_cache_pages, num_heads, num_workers))
    try:
        w, n, m, s = c_int32(), c_int64(), c_int64(), c_int64()
        lib.mla_schedule_sizes(h, ctypes.byref(w), ctypes.byref(n), ctypes.byref(m),
                               ctypes.byref(s))
        wi = np.zeros(w.value + 2, np.int32)
        items = np.zeros((n.value, 8), np.int32)
        merges = np.zeros((m.value, 4), np.int32)
        lib.mla_schedule_copy(h, _ptr(wi), _ptr(items), _ptr(merges))
    finally:
        lib.mla_schedule_destroy(h)
    return {"worker_indptr": wi, "items": items, "merges": merges, "num_slots": s.value}


def append_rows(qo_indptr, kv_indptr, kv_indices, kv_last_page_len, page_size: int,
                num_cache_pages: int, lib_path: Optional[str] = None) -> np.ndarray:
    """The cache row (page * page_size + slot) the KV append writes for each
    query token, from the host planner; raises MLAError if the page table
    cannot take an append."""
    lib = _native.load(lib_path or _native.LIB_PATH, host_only=True)
    qo, kv = _host_i32(qo_indptr), _host_i32(kv_indptr)
    idx, last = _host_i32(kv_indices), _host_i32(kv_last_page_len)
    if idx.size == 0:
        idx = np.zeros(1, np.int32)
    h = c_void_p()
    _native.check(lib, lib.mla_schedule_build(ctypes.byref(h), _ptr(qo), _ptr(kv), _ptr(idx),
                                              _ptr(last), qo.shape[0] - 1, 1, page_size,
                                              num_cache_pages, 1, 1))
    try:
        rows = np.zeros(max(1, int(qo[-1])), np.int32)
        _native.check(lib, lib.mla_schedule_append_rows(h, _ptr(rows)))
    finally:
        lib.mla_schedule_destroy(h)
    return rows[:int(qo[-1])]
