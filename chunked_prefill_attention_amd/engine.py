"""One attention layer's engine step, driven by the native ``cb_engine``.

Hugging Face transformers, "Continuous batching architecture" ("Request
lifecycle", "Scheduler"): every generation step the scheduler picks the
requests and tokens of the next forward pass; AI Engineering from Scratch,
"vLLM serving internals" ("What the scheduler looks like"): the chosen
decode tokens and prefill chunks then run as one fused GPU call.

``PagedAttentionLayer`` owns (as torch tensors) the paged K/V caches of one
layer, two pinned-host and two device metadata slots and the workspace; the
C++ engine owns the FIFO builder.  A step is two library calls:

    desc = layer.schedule()                   # builder + packed async upload
    out  = layer.attend(q, k_new, v_new)      # cb_kv_append + cb_attention_step

All compute runs in the HIP library; this module only hands over buffers.
"""
from __future__ import annotations

import ctypes as C

import numpy as np

from . import Builder, Step, builder_config, kv_append, CB_BF16, CB_F32, PAGE_SIZE
from ._lib import EngineConfig, EngineStats, StepDesc, CbError, check, load, CB_ERR_CAPACITY, CB_ERR_WORKSPACE


def _arr(ptr, n, dtype):
    if n == 0:
        return np.zeros(0, dtype)
    return np.ctypeslib.as_array(ptr, shape=(n,)).copy().astype(dtype, copy=False)


class StepView:
    """The scheduled step: scalars at once, host arrays copied on first use.

    The arrays live in the engine's builder until the next ``schedule``; a
    view read after that raises instead of returning the next step's data.
    ``copy()`` returns a view that stays valid.
    """

    def __init__(self, d: StepDesc, layer=None):
        self._d = d
        self._layer = layer
        self._gen = layer._gen if layer is not None else None
        self.num_seqs, self.num_decodes, self.num_tokens = d.num_seqs, d.num_decodes, d.num_tokens
        self.max_query_len, self.max_context_len = d.max_query_len, d.max_context_len
        self.block_table_stride, self.new_pages = d.block_table_stride, d.new_pages
        self.prefix_hit_tokens = d.prefix_hit_tokens
        self._cache = {}

    def _get(self, name, n, dtype):
        if name not in self._cache:
            if self._layer is not None and self._layer._gen != self._gen:
                raise RuntimeError("step descriptor read after the next schedule()")
            self._cache[name] = _arr(getattr(self._d, name), n, dtype)
        return self._cache[name]

    def copy(self) -> "StepView":
        for name, n, dt in (("req_ids", self.num_seqs, np.int64), ("query_start_loc", self.num_seqs + 1, np.int32),
                            ("context_lens", self.num_seqs, np.int32), ("q_offsets", self.num_seqs, np.int32),
                            ("slot_mapping", self.num_tokens, np.int32),
                            ("block_tables", self.num_seqs * self.block_table_stride, np.int32),
                            ("finished_ids", self._d.num_finished, np.int64),
                            ("stalled_ids", self._d.num_stalled, np.int64)):
            self._get(name, n, dt)
        v = StepView.__new__(StepView)
        v.__dict__.update(self.__dict__)
        v._cache = dict(self._cache)
        v._layer = None
        return v

    req_ids = property(lambda self: self._get("req_ids", self.num_seqs, np.int64))
    query_start_loc = property(lambda self: self._get("query_start_loc", self.num_seqs + 1, np.int32))
    context_lens = property(lambda self: self._get("context_lens", self.num_seqs, np.int32))
    q_offsets = property(lambda self: self._get("q_offsets", self.num_seqs, np.int32))
    slot_mapping = property(lambda self: self._get("slot_mapping", self.num_tokens, np.int32))
    finished_ids = property(lambda self: self._get("finished_ids", self._d.num_finished, np.int64))
    stalled_ids = property(lambda self: self._get("stalled_ids", self._d.num_stalled, np.int64))

    @property
    def block_tables(self):
        return self._get("block_tables", self.num_seqs * self.block_table_stride,
                         np.int32).reshape(self.num_seqs, self.block_table_stride)

    @property
    def q_lens(self):
        return np.diff(self.query_start_loc)


class PagedAttentionLayer:
    def __init__(self, num_q_heads: int, num_kv_heads: int, head_dim: int, num_pages: int,
                 max_batch_tokens: int, max_requests_per_batch: int, dtype: str = "bf16",
                 max_prefill_chunk: int = 0, safety_margin: float = 0.0, page_shuffle_seed: int = 0,
                 device=None, cache_fill: float = 0.0, meta_pages_per_request: int = 2048,
                 graph_q_interval: int = 0, graph_kv_interval: int = 0, graph_capture: bool = True,
                 **policy_kw):
        import torch
        self.torch = torch
        self._lib = load()
        self.hq, self.hkv, self.d = num_q_heads, num_kv_heads, head_dim
        self.num_pages = num_pages
        self.tdtype = {"bf16": torch.bfloat16, "f32": torch.float32}[dtype]
        self.code = CB_BF16 if dtype == "bf16" else CB_F32
        self.device = device if device is not None else torch.device("cuda", torch.cuda.current_device())
        self.k_cache = torch.full((num_pages, num_kv_heads, PAGE_SIZE, head_dim), cache_fill,
                                  dtype=self.tdtype, device=self.device)
        self.v_cache = torch.full((num_pages, num_kv_heads, head_dim, PAGE_SIZE), cache_fill,
                                  dtype=self.tdtype, device=self.device)
        self.scale = float(np.float32(1.0 / np.sqrt(head_dim)))
        B, T = max_requests_per_batch, max_batch_tokens
        slot_ints = 3 * B + 1 + T + B * min(num_pages, meta_pages_per_request) + 64
        self._alloc_meta(2 * slot_ints)
        self._ws = None
        cfg = EngineConfig(builder_config(max_batch_tokens, max_requests_per_batch, num_pages,
                                          max_prefill_chunk, safety_margin, page_shuffle_seed,
                                          **policy_kw),
                           num_q_heads, num_kv_heads, head_dim, self.code, self.scale,
                           self.k_cache.data_ptr(), self.v_cache.data_ptr(), self._meta_dev.data_ptr(),
                           self._meta_host.data_ptr(), self._meta_dev.numel() * 4, None, 0)
        h = C.c_void_p()
        check(self._lib.cb_engine_create(C.byref(cfg), C.byref(h)))
        self._h = h
        self.builder = Builder(0, 0, 0, _handle=self._lib.cb_engine_builder(h), _owned=False)
        self._desc = StepDesc()
        self._gen = 0
        # graph replay: padded step shapes, static buffers, a capturable stream
        self.graphs = graph_q_interval > 0 or graph_kv_interval > 0
        if self.graphs:
            check(self._lib.cb_engine_set_graphs(h, graph_q_interval, graph_kv_interval, int(graph_capture)))
            rows = max_batch_tokens + max(graph_q_interval, 16)   # >= any padded token count
            self.static_q = torch.zeros((rows, num_q_heads, head_dim), dtype=self.tdtype, device=self.device)
            self.static_k = torch.zeros((rows, num_kv_heads, head_dim), dtype=self.tdtype, device=self.device)
            self.static_v = torch.zeros_like(self.static_k)
            self.static_out = torch.zeros_like(self.static_q)
            self.graph_stream = torch.cuda.Stream(self.device)     # default priority

    def _alloc_meta(self, ints):
        torch = self.torch
        self._meta_host = torch.empty(ints, dtype=torch.int32, pin_memory=True)
        self._meta_dev = torch.empty(ints, dtype=torch.int32, device=self.device)

    def close(self):
        if getattr(self, "_h", None):
            self._lib.cb_engine_destroy(self._h)
            self._h = None

    __del__ = close

    def _stream(self, stream):
        if stream is None:
            stream = self.graph_stream if self.graphs else self.torch.cuda.current_stream(self.device)
        return C.c_void_p(stream.cuda_stream)

    def graph_stats(self) -> dict:
        c, r, n = C.c_int64(), C.c_int64(), C.c_int64()
        check(self._lib.cb_engine_graph_stats(self._h, C.byref(c), C.byref(r), C.byref(n)))
        return {"captures": c.value, "replays": r.value, "cached": n.value}

    def reserve_workspace(self, nbytes: int) -> None:
        """Hold at least ``nbytes`` of attention workspace now, so that no later
        step has to grow it (growing synchronises the device)."""
        if self._ws is not None and self._ws.numel() >= nbytes:
            return
        self.torch.cuda.synchronize(self.device)
        self._ws = self.torch.empty(int(nbytes), dtype=self.torch.uint8, device=self.device)
        check(self._lib.cb_engine_set_workspace(self._h, self._ws.data_ptr(), self._ws.numel()))

    def stats(self) -> dict:
        """Engine counters (cb_engine_stats_get): steps scheduled and attended,
        waits for a staging slot, graph captures and replays."""
        s = EngineStats()
        check(self._lib.cb_engine_stats_get(self._h, C.byref(s)))
        return {f: getattr(s, f) for f, _ in EngineStats._fields_}

    # -- a1 + a2: builder step and metadata upload -----------------------------------------
    def schedule(self, stream=None) -> StepView:
        self._gen += 1
        self._desc = StepDesc()
        st = self._lib.cb_engine_schedule(self._h, self._stream(stream), C.byref(self._desc))
        for _ in range(32):
            if st != CB_ERR_CAPACITY:
                break
            # grow the metadata slots (the builder state is unchanged), schedule again
            self.torch.cuda.synchronize(self.device)
            self._alloc_meta(2 * self._meta_dev.numel())
            check(self._lib.cb_engine_set_metadata(self._h, self._meta_dev.data_ptr(),
                                                   self._meta_host.data_ptr(), self._meta_dev.numel() * 4))
            st = self._lib.cb_engine_schedule(self._h, self._stream(stream), C.byref(self._desc))
        check(st)
        return StepView(self._desc, self)

    # -- a3 .. a7: append + attention --------------------------------------------------------
    def attend(self, q, k_new, v_new, out=None, stream=None):
        if self.graphs:
            return self._attend_padded(q, k_new, v_new, out, stream)
        if out is None:
            out = self.torch.empty_like(q)
        return self._attend(q, k_new, v_new, out, stream)

    def _attend_padded(self, q, k_new, v_new, out, stream):
        """Padded (graph) mode: the step runs on the static buffers, on the
        layer's stream (or ``stream``), ordered after the caller's current stream."""
        torch = self.torch
        T = self._desc.num_tokens
        cur = torch.cuda.current_stream(self.device)
        for src, dst in ((q, self.static_q), (k_new, self.static_k), (v_new, self.static_v)):
            if src.data_ptr() != dst.data_ptr():
                dst[:T].copy_(src[:T])
        gs = stream if stream is not None else self.graph_stream
        gs.wait_stream(cur)
        self._attend(self.static_q, self.static_k, self.static_v, self.static_out, gs)
        cur.wait_stream(gs)
        if out is None:
            return self.static_out[:T]
        out[:T].copy_(self.static_out[:T])
        return out

    def _attend(self, q, k_new, v_new, out, stream):
        args = (q.data_ptr(), k_new.data_ptr(), v_new.data_ptr(), out.data_ptr(), self._stream(stream))
        st = self._lib.cb_engine_attend(self._h, *args)
        if st == CB_ERR_WORKSPACE:
            need = self._lib.cb_engine_workspace_bytes(self._h)
            # earlier steps (possibly on another stream) may still use the old one
            self.torch.cuda.synchronize(self.device)
            self._ws = self.torch.empty(int(need * 1.25) + 256, dtype=self.torch.uint8, device=self.device)
            check(self._lib.cb_engine_set_workspace(self._h, self._ws.data_ptr(), self._ws.numel()))
            st = self._lib.cb_engine_attend(self._h, *args)
        check(st)
        return out

    def load_builder(self, snapshot: Builder) -> None:
        """Restore the scheduler state from a builder snapshot (``Builder.clone()``)."""
        check(self._lib.cb_engine_load_builder(self._h, snapshot._h))

    def write_positions(self, req_id: int, start: int, end: int, k_rows, v_rows, stream=None):
        """Write K/V rows of logical positions start..end-1 of request ``req_id``
        into its pages (used to import in-flight requests); the slots come from
        the builder (cb_builder_slots)."""
        slots = self.builder.slots(req_id, start, end)
        sm = self.torch.from_numpy(slots).to(self.device)
        kv_append(k_rows, v_rows, self.k_cache, self.v_cache, sm, stream=stream)
