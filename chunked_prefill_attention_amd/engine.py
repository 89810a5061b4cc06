"""One attention layer's engine step: builder -> metadata upload -> append -> attention.

Hugging Face transformers, "Continuous batching architecture" ("Request
lifecycle", "Scheduler"): every generation step the scheduler picks the
requests and tokens of the next forward pass; AI Engineering from Scratch,
"vLLM serving internals" ("What the scheduler looks like"): the chosen
decode tokens and prefill chunks then run as one fused GPU call.

``PagedAttentionLayer`` owns the paged K/V caches of one layer, the C++ FIFO
builder, a pinned host staging buffer and the device workspace.  A step is

    desc = layer.schedule()                 # host: C++ builder
    meta = layer.upload(desc)               # one async H2D copy of all int32 metadata
    out  = layer.forward(meta, q, k_new, v_new)   # cb_kv_append + cb_attention_step

All compute runs in the HIP library; this module only moves buffers.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

from . import Builder, Step, attention_step, attention_workspace_bytes, kv_append, CB_BF16, CB_F32, PAGE_SIZE


@dataclass
class DeviceStep:
    """Device views of one step descriptor (int32), plus host scalars."""
    desc: Step
    query_start_loc: "object"
    context_lens: "object"
    q_offsets: "object"
    block_tables: "object"
    slot_mapping: "object"


class PagedAttentionLayer:
    def __init__(self, num_q_heads: int, num_kv_heads: int, head_dim: int, num_pages: int,
                 max_batch_tokens: int, max_requests_per_batch: int, dtype: str = "bf16",
                 max_prefill_chunk: int = 0, safety_margin: float = 0.0, page_shuffle_seed: int = 0,
                 device=None, cache_fill: float = 0.0, staging_slots: int = 2):
        import torch
        self.torch = torch
        self.hq, self.hkv, self.d = num_q_heads, num_kv_heads, head_dim
        self.num_pages = num_pages
        self.tdtype = {"bf16": torch.bfloat16, "f32": torch.float32}[dtype]
        self.code = CB_BF16 if dtype == "bf16" else CB_F32
        self.device = device if device is not None else torch.device("cuda", torch.cuda.current_device())
        self.builder = Builder(max_batch_tokens, max_requests_per_batch, num_pages, max_prefill_chunk,
                               safety_margin, page_shuffle_seed)
        self.k_cache = torch.full((num_pages, num_kv_heads, PAGE_SIZE, head_dim), cache_fill,
                                  dtype=self.tdtype, device=self.device)
        self.v_cache = torch.full((num_pages, num_kv_heads, head_dim, PAGE_SIZE), cache_fill,
                                  dtype=self.tdtype, device=self.device)
        self.scale = float(np.float32(1.0 / np.sqrt(head_dim)))
        self._ws = None
        self._staging = [None] * staging_slots   # (pinned host buffer, device buffer) pairs
        self._slot = 0

    # -- a1: batch build on the host --------------------------------------------------
    def schedule(self) -> Step:
        return self.builder.step()

    # -- a2: metadata upload -------------------------------------------------------------
    def upload(self, desc: Step, stream=None) -> DeviceStep:
        """Pack every int32 array of the descriptor and copy it in one transfer.

        Staging buffers rotate so the host can pack step N+1 while step N's
        copy is still in flight on ``stream``.
        """
        torch = self.torch
        parts = [desc.query_start_loc, desc.context_lens, desc.q_offsets,
                 desc.block_tables.reshape(-1), desc.slot_mapping]
        sizes = [p.size for p in parts]
        total = int(sum(sizes))
        slot = self._slot
        self._slot = (slot + 1) % len(self._staging)
        buf = self._staging[slot]
        if buf is not None:
            buf[2].synchronize()      # the copy that last read this host buffer has finished
        if buf is None or buf[0].numel() < total:
            n = max(total, 1 << 16)
            host = torch.empty(n, dtype=torch.int32, pin_memory=True)
            devb = torch.empty(n, dtype=torch.int32, device=self.device)
            buf = self._staging[slot] = (host, devb, torch.cuda.Event())
        host, devb, done = buf
        hv = host.numpy()
        off = 0
        for p, n in zip(parts, sizes):
            hv[off:off + n] = p
            off += n
        s = stream if stream is not None else torch.cuda.current_stream(self.device)
        with torch.cuda.stream(s):
            devb[:total].copy_(host[:total], non_blocking=True)
            done.record(s)
        views, off = [], 0
        for n in sizes:
            views.append(devb[off:off + n])
            off += n
        qsl, ctx, qo, bt, sm = views
        return DeviceStep(desc, qsl, ctx, qo, bt.view(desc.num_seqs, desc.block_table_stride), sm)

    def workspace(self, desc: Step):
        need = attention_workspace_bytes(desc.num_seqs, desc.num_decodes, desc.num_tokens, self.hq,
                                         self.hkv, self.d, max(desc.max_context_len, 1), self.code)
        if need and (self._ws is None or self._ws.numel() < need):
            self._ws = self.torch.empty(int(need * 1.25), dtype=self.torch.uint8, device=self.device)
        return self._ws if need else None

    # -- a3..a7: append + attention -------------------------------------------------------
    def forward(self, meta: DeviceStep, q, k_new, v_new, out=None, stream=None):
        d = meta.desc
        if d.num_tokens == 0:
            return q
        kv_append(k_new, v_new, self.k_cache, self.v_cache, meta.slot_mapping, stream=stream)
        return attention_step(q, self.k_cache, self.v_cache, meta.block_tables, meta.query_start_loc,
                              meta.context_lens, meta.q_offsets, d.num_decodes, d.max_context_len,
                              self.scale, out=out, workspace=self.workspace(d), stream=stream)

    def write_positions(self, req_pages: np.ndarray, start: int, end: int, k_rows, v_rows, stream=None):
        """Write K/V rows of logical positions start..end-1 of a request whose
        block table is ``req_pages`` (used to import in-flight requests)."""
        torch = self.torch
        pos = np.arange(start, end)
        slots = (req_pages[pos // PAGE_SIZE].astype(np.int64) * PAGE_SIZE + pos % PAGE_SIZE).astype(np.int32)
        sm = torch.from_numpy(slots).to(self.device, non_blocking=False)
        kv_append(k_rows, v_rows, self.k_cache, self.v_cache, sm, stream=stream)
