"""Chunked-prefill + decode paged attention for AMD MI355X (gfx950).

A thin binding over the C ABI of ``libcb.so`` (declared in include/cb.h):
every step of the attention path runs in the library's HIP kernels, and the
FIFO batch builder runs in its C++ host code.  This module only checks and
marshals arguments.  ``torch`` is used for device memory and streams.

    kv_append(...)              -> cb_kv_append
    attention_workspace_bytes() -> cb_attention_workspace_bytes
    attention_step(...)         -> cb_attention_step
    Builder                     -> cb_builder_* (FIFO batch builder)
"""
from __future__ import annotations

import ctypes as C
from dataclasses import dataclass

import numpy as np

from ._lib import (BuilderConfig, BuilderStats, CbError, StepDesc, check, load,
                   CB_F32, CB_BF16, CB_POLICY_FIFO, CB_POLICY_PREFILL_FIRST, PAGE_SIZE, LIB_PATH)

__all__ = ["kv_append", "attention_step", "attention_step_noalloc", "attention_workspace_bytes", "Builder", "Step", "builder_config",
           "CbError", "CB_F32", "CB_BF16", "PAGE_SIZE", "LIB_PATH", "load"]


def _torch():
    import torch
    return torch


def _dtype_code(t) -> int:
    torch = _torch()
    if t.dtype == torch.float32:
        return CB_F32
    if t.dtype == torch.bfloat16:
        return CB_BF16
    raise TypeError(f"unsupported dtype {t.dtype}; use float32 or bfloat16")


def _dev(t, name, dtype=None):
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    return C.c_void_p(t.data_ptr())


def _stream(stream):
    torch = _torch()
    s = stream if stream is not None else torch.cuda.current_stream()
    return C.c_void_p(s.cuda_stream)


def kv_append(k_new, v_new, k_cache, v_cache, slot_mapping, stream=None) -> None:
    """Write rows ``k_new/v_new[T, Hkv, D]`` into ``k_cache[P, Hkv, 16, D]`` and
    ``v_cache[P, Hkv, D, 16]`` at ``slot_mapping[T]`` (int32; < 0 skips)."""
    torch = _torch()
    T, hkv, d = k_new.shape
    dt = _dtype_code(k_new)
    for t, n in ((v_new, "v_new"), (k_cache, "k_cache"), (v_cache, "v_cache")):
        if t.dtype != k_new.dtype:
            raise TypeError(f"{n} dtype differs from k_new")
    if tuple(v_new.shape) != (T, hkv, d) or k_cache.shape[1:] != (hkv, PAGE_SIZE, d) \
            or tuple(v_cache.shape) != (k_cache.shape[0], hkv, d, PAGE_SIZE):
        raise ValueError("shape mismatch between new rows and caches")
    if slot_mapping.numel() != T:
        raise ValueError("slot_mapping must have one entry per token")
    check(load().cb_kv_append(_dev(k_new, "k_new"), _dev(v_new, "v_new"), _dev(k_cache, "k_cache"),
                              _dev(v_cache, "v_cache"), _dev(slot_mapping, "slot_mapping", torch.int32),
                              T, hkv, d, k_cache.shape[0], PAGE_SIZE, dt, _stream(stream)))


def attention_workspace_bytes(num_seqs, num_decodes, num_tokens, num_q_heads, num_kv_heads, head_dim,
                              max_context_len, dtype_code) -> int:
    n = load().cb_attention_workspace_bytes(num_seqs, num_decodes, num_tokens, num_q_heads, num_kv_heads,
                                            head_dim, max_context_len, dtype_code)
    if n == C.c_size_t(-1).value:
        raise CbError(-1, "invalid arguments to cb_attention_workspace_bytes")
    return n


def attention_step(q, k_cache, v_cache, block_tables, query_start_loc, context_lens, q_offsets,
                   num_decodes: int, max_context_len: int, scale: float, out=None, workspace=None,
                   stream=None, sliding_window: int = 0):
    """Causal attention of every query row ``q[T, Hq, D]`` over its sequence's pages.

    ``block_tables[B, stride]``, ``query_start_loc[B+1]``, ``context_lens[B]``,
    ``q_offsets[B]`` are int32 device tensors.  Returns ``out[T, Hq, D]``.
    ``workspace`` (uint8 device tensor) is allocated here when not given.
    ``sliding_window`` > 0 limits row ``p`` to keys ``p - W < j <= p``.
    """
    torch = _torch()
    T, hq, d = q.shape
    P, hkv = k_cache.shape[0], k_cache.shape[1]
    B = context_lens.numel()
    dt = _dtype_code(q)
    if k_cache.dtype != q.dtype or v_cache.dtype != q.dtype:
        raise TypeError("q, k_cache and v_cache must share a dtype")
    if block_tables.dim() != 2 or block_tables.shape[0] != B:
        raise ValueError("block_tables must be [num_seqs, stride]")
    if query_start_loc.numel() != B + 1 or q_offsets.numel() != B:
        raise ValueError("query_start_loc must be [B+1] and q_offsets [B]")
    if out is None:
        out = torch.empty_like(q)
    elif out.shape != q.shape or out.dtype != q.dtype:
        raise ValueError("out must match q")
    need = attention_workspace_bytes(B, num_decodes, T, hq, hkv, d, max_context_len, dt)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    ws_ptr = _dev(workspace, "workspace") if workspace is not None else C.c_void_p(0)
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    check(load().cb_attention_step(
        _dev(q, "q"), _dev(k_cache, "k_cache"), _dev(v_cache, "v_cache"),
        _dev(block_tables, "block_tables", torch.int32), block_tables.shape[1],
        _dev(query_start_loc, "query_start_loc", torch.int32), _dev(context_lens, "context_lens", torch.int32),
        _dev(q_offsets, "q_offsets", torch.int32), B, num_decodes, T, max_context_len, hq, hkv, d,
        PAGE_SIZE, P, float(scale), int(sliding_window), dt, _dev(out, "out"), ws_ptr, ws_bytes,
        _stream(stream)))
    return out


def attention_step_noalloc(q, k_cache, v_cache, block_tables, query_start_loc, context_lens, q_offsets,
                           num_decodes: int, max_context_len: int, scale: float, out=None, stream=None,
                           sliding_window: int = 0):
    """``attention_step`` through cb_attention_step_noalloc: no workspace; the
    library's fixed per-device scratch array is used instead (``out`` is still
    allocated here when not given)."""
    torch = _torch()
    T, hq, d = q.shape
    P, hkv = k_cache.shape[0], k_cache.shape[1]
    B = context_lens.numel()
    dt = _dtype_code(q)
    if k_cache.dtype != q.dtype or v_cache.dtype != q.dtype:
        raise TypeError("q, k_cache and v_cache must share a dtype")
    if block_tables.dim() != 2 or block_tables.shape[0] != B:
        raise ValueError("block_tables must be [num_seqs, stride]")
    if query_start_loc.numel() != B + 1 or q_offsets.numel() != B:
        raise ValueError("query_start_loc must be [B+1] and q_offsets [B]")
    if out is None:
        out = torch.empty_like(q)
    elif out.shape != q.shape or out.dtype != q.dtype:
        raise ValueError("out must match q")
    check(load().cb_attention_step_noalloc(
        _dev(q, "q"), _dev(k_cache, "k_cache"), _dev(v_cache, "v_cache"),
        _dev(block_tables, "block_tables", torch.int32), block_tables.shape[1],
        _dev(query_start_loc, "query_start_loc", torch.int32), _dev(context_lens, "context_lens", torch.int32),
        _dev(q_offsets, "q_offsets", torch.int32), B, num_decodes, T, max_context_len, hq, hkv, d,
        PAGE_SIZE, P, float(scale), int(sliding_window), dt, _dev(out, "out"), _stream(stream)))
    return out


@dataclass
class Step:
    """Host copy of one step descriptor emitted by the builder."""
    num_seqs: int
    num_decodes: int
    num_tokens: int
    max_query_len: int
    max_context_len: int
    block_table_stride: int
    new_pages: int
    req_ids: np.ndarray
    query_start_loc: np.ndarray
    context_lens: np.ndarray
    q_offsets: np.ndarray
    block_tables: np.ndarray     # [num_seqs, stride]
    slot_mapping: np.ndarray
    finished_ids: np.ndarray
    stalled_ids: np.ndarray
    prefix_hit_tokens: int = 0

    @property
    def q_lens(self) -> np.ndarray:
        return np.diff(self.query_start_loc)


def _arr(ptr, n, dtype):
    if n == 0:
        return np.zeros(0, dtype)
    return np.ctypeslib.as_array(ptr, shape=(n,)).copy().astype(dtype, copy=False)


POLICIES = {"fifo": CB_POLICY_FIFO, "prefill_first": CB_POLICY_PREFILL_FIRST}


def builder_config(max_batch_tokens, max_requests_per_batch, num_pages, max_prefill_chunk=0,
                   safety_margin=0.0, page_shuffle_seed=0, policy="fifo", max_partial_prefills=0,
                   max_long_partial_prefills=0, long_prefill_threshold=0,
                   allow_block_sharing=False, sliding_window=0) -> BuilderConfig:
    """The builder's C configuration; argument meanings as in include/cb.h."""
    if policy not in POLICIES:
        raise ValueError(f"policy must be one of {sorted(POLICIES)}")
    return BuilderConfig(max_batch_tokens, max_requests_per_batch, num_pages, PAGE_SIZE,
                         max_prefill_chunk, safety_margin, page_shuffle_seed, POLICIES[policy],
                         max_partial_prefills, max_long_partial_prefills, long_prefill_threshold,
                         1 if allow_block_sharing else 0, sliding_window)


class Builder:
    """Batch builder (C++): token budget, request cap, page budget, safety margin,
    FIFO or PrefillFirst policy, partial-prefill caps, prefix block sharing."""

    def __init__(self, max_batch_tokens, max_requests_per_batch, num_pages, max_prefill_chunk=0,
                 safety_margin=0.0, page_shuffle_seed=0, _handle=None, _owned=True, **policy_kw):
        self._lib = load()
        self._owned = _owned
        if _handle is not None:
            self._h = C.c_void_p(_handle) if isinstance(_handle, int) else _handle
            return
        cfg = builder_config(max_batch_tokens, max_requests_per_batch, num_pages, max_prefill_chunk,
                             safety_margin, page_shuffle_seed, **policy_kw)
        h = C.c_void_p()
        check(self._lib.cb_builder_create(C.byref(cfg), C.byref(h)))
        self._h = h

    def clone(self) -> "Builder":
        h = C.c_void_p()
        check(self._lib.cb_builder_clone(self._h, C.byref(h)))
        return Builder(0, 0, 0, _handle=h)

    def close(self):
        if getattr(self, "_h", None):
            if self._owned:
                self._lib.cb_builder_destroy(self._h)
            self._h = None

    __del__ = close

    def submit(self, req_id: int, prompt_len: int, output_len: int, tokens_cached: int = 0,
               tokens=None) -> None:
        """Queue a request; with ``tokens`` (the whole prompt) it may share prefix blocks."""
        if tokens is None:
            check(self._lib.cb_builder_submit(self._h, req_id, prompt_len, output_len, tokens_cached))
            return
        if tokens_cached:
            raise ValueError("tokens are given for new requests only")
        t = np.ascontiguousarray(tokens, dtype=np.int32)
        if t.shape != (prompt_len,):
            raise ValueError("tokens must hold prompt_len ids")
        check(self._lib.cb_builder_submit_tokens(self._h, req_id, t.ctypes.data_as(C.POINTER(C.c_int32)),
                                                 prompt_len, output_len))

    def step(self) -> Step:
        d = StepDesc()
        check(self._lib.cb_builder_step(self._h, C.byref(d)))
        n, T, st = d.num_seqs, d.num_tokens, d.block_table_stride
        return Step(n, d.num_decodes, T, d.max_query_len, d.max_context_len, st, d.new_pages,
                    _arr(d.req_ids, n, np.int64), _arr(d.query_start_loc, n + 1, np.int32),
                    _arr(d.context_lens, n, np.int32), _arr(d.q_offsets, n, np.int32),
                    _arr(d.block_tables, n * st, np.int32).reshape(n, st),
                    _arr(d.slot_mapping, T, np.int32), _arr(d.finished_ids, d.num_finished, np.int64),
                    _arr(d.stalled_ids, d.num_stalled, np.int64), d.prefix_hit_tokens)

    def block_table(self, req_id: int) -> np.ndarray:
        n = C.c_int32()
        check(self._lib.cb_builder_block_table(self._h, req_id, None, 0, C.byref(n)))
        buf = np.zeros(max(n.value, 1), np.int32)
        check(self._lib.cb_builder_block_table(self._h, req_id, buf.ctypes.data_as(C.POINTER(C.c_int32)),
                                               n.value, C.byref(n)))
        return buf[:n.value]

    def slots(self, req_id: int, start: int, end: int) -> np.ndarray:
        """Cache slots of logical positions ``start .. end-1`` of a request (int32)."""
        out = np.zeros(max(end - start, 1), np.int32)
        check(self._lib.cb_builder_slots(self._h, req_id, start, end, out.ctypes.data_as(C.POINTER(C.c_int32))))
        return out[:max(end - start, 0)]

    def stats(self) -> dict:
        s = BuilderStats()
        check(self._lib.cb_builder_stats_get(self._h, C.byref(s)))
        return {f: getattr(s, f) for f, _ in BuilderStats._fields_}
