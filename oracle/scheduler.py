"""Plain-Python FIFO batch builder (test infrastructure only).

Follows these passages of the pages:

* Hugging Face transformers, "Continuous batching architecture":
  - "Request lifecycle": a request goes PENDING -> PREFILLING -> DECODING ->
    FINISHED; it leaves the queue when the scheduler has enough token budget
    and cache room; a prompt too long for one step is split over several
    forward passes.
  - "Chunked prefill": a prompt longer than the remaining token budget takes
    every token that still fits; the rest resumes in the next step from
    where it stopped.
  - "Scheduler": three limits per forward pass -- the token budget
    (``max_batch_tokens``), the cache budget (KV pages), and the request
    cap (``max_requests_per_batch``).
  - "FIFO": active decodes first, then active prefills, then waiting
    requests in arrival order.
  - "Admission": a request that any allocator cannot hold is rejected and
    nothing is allocated; below ``safety_margin`` of free capacity new
    prefills are deferred and only active work continues.
* Ultralytics glossary, "Chunked Prefill", "How chunked prefill works": one
  token per running decode first, then the remaining budget is filled with
  chunks of waiting prompts.
* AI Engineering from Scratch, "vLLM serving internals", section "What the
  scheduler looks like": finished sequences release their blocks at the top
  of the loop; waiting sequences are admitted from the head of the queue
  while blocks are free (strict head of line).

Readings where the pages are silent or ambiguous (also listed in the design doc):

* chunk = min(remaining prompt, remaining token budget, ``max_prefill_chunk``
  when it is > 0); an active prefill is further cut to the tokens its held
  pages plus the free pages can hold, and is "stalled" if that is zero;
* a decode needs one new page when its cached length is a multiple of the
  page size; with no free page it is stalled (skipped, counted), not
  offloaded;
* admission of a waiting request needs its first chunk's pages to be free and
  ``free - needed >= safety_margin * num_pages``; the margin does not gate
  active decodes or active prefills;
* a request that finishes in a step keeps its pages until the start of the
  next step, where it is reported as finished and its pages are freed;
* the prefill step that completes the prompt yields the first output token;
  each decode step yields one more, so a request takes ``output_len - 1``
  decode steps and its KV never exceeds ``prompt_len + output_len - 1``;
* ``submit`` with ``tokens_cached > 0`` imports an in-flight request whose
  pages are allocated at once: an active prefill if ``tokens_cached <
  prompt_len``, else a decode that has produced ``tokens_cached - prompt_len
  + 1`` tokens; imports and submissions share one arrival order.

Physical page ids are not unique (any free page is correct), so this model
tracks page *counts* only.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

WAITING, PREFILLING, DECODING, FINISHED = "waiting", "prefilling", "decoding", "finished"


class SchedulerError(ValueError):
    def __init__(self, kind: str, msg: str):
        super().__init__(msg)
        self.kind = kind          # "invalid" or "capacity"


@dataclass
class Request:
    req_id: int
    prompt_len: int
    output_len: int
    arrival: int
    cached: int = 0
    generated: int = 0
    pages: int = 0
    state: str = WAITING


@dataclass
class ScheduledSeq:
    req_id: int
    q_len: int
    q_offset: int          # KV length before this step's tokens
    context_len: int       # KV length after this step's tokens
    is_decode: bool
    pages: int             # pages the request holds after this step's allocation


@dataclass
class Step:
    seqs: list = field(default_factory=list)
    finished: list = field(default_factory=list)   # released at the start of this step
    stalled: list = field(default_factory=list)
    new_pages: int = 0

    @property
    def num_decodes(self) -> int:
        return sum(1 for s in self.seqs if s.is_decode)

    @property
    def num_tokens(self) -> int:
        return sum(s.q_len for s in self.seqs)


def _ceil_div(a: int, b: int) -> int:
    return -(-a // b)


class FifoScheduler:
    def __init__(self, max_batch_tokens: int, max_requests_per_batch: int, num_pages: int,
                 page_size: int = 16, max_prefill_chunk: int = 0, safety_margin: float = 0.0):
        if max_batch_tokens < 1 or max_requests_per_batch < 1 or num_pages < 1 or page_size < 1:
            raise SchedulerError("invalid", "budgets and pool size must be positive")
        if max_prefill_chunk < 0 or not (0.0 <= safety_margin < 1.0):
            raise SchedulerError("invalid", "bad chunk cap or safety margin")
        self.max_batch_tokens = max_batch_tokens
        self.max_requests = max_requests_per_batch
        self.num_pages = num_pages
        self.page = page_size
        self.chunk_cap = max_prefill_chunk
        # the margin is a float32 configuration value; compare in float64
        self.margin = float(np.float32(safety_margin))
        self.free = num_pages
        self.requests: dict[int, Request] = {}
        self._arrivals = 0
        self.total_stalls = 0

    # -- submission ---------------------------------------------------------------
    def submit(self, req_id: int, prompt_len: int, output_len: int, tokens_cached: int = 0):
        if req_id in self.requests:
            raise SchedulerError("invalid", f"duplicate request id {req_id}")
        if prompt_len < 1 or output_len < 1 or tokens_cached < 0:
            raise SchedulerError("invalid", "lengths must be positive")
        final_kv = prompt_len + output_len - 1
        if tokens_cached >= final_kv and tokens_cached > 0:
            raise SchedulerError("invalid", "request has nothing left to do")
        if _ceil_div(final_kv, self.page) > self.num_pages:
            raise SchedulerError("capacity", "request can never fit the page pool")
        r = Request(req_id, prompt_len, output_len, self._arrivals)
        if tokens_cached > 0:
            need = _ceil_div(tokens_cached, self.page)
            if need > self.free:
                raise SchedulerError("capacity", "not enough free pages to import")
            self.free -= need
            r.pages = need
            r.cached = tokens_cached
            if tokens_cached < prompt_len:
                r.state = PREFILLING
            else:
                r.state = DECODING
                r.generated = tokens_cached - prompt_len + 1
        self._arrivals += 1
        self.requests[req_id] = r

    # -- one engine step ----------------------------------------------------------
    def _ordered(self, state):
        return sorted((r for r in self.requests.values() if r.state == state),
                      key=lambda r: r.arrival)

    def step(self) -> Step:
        st = Step()
        # release what finished last step
        for r in self._ordered(FINISHED):
            self.free += r.pages
            st.finished.append(r.req_id)
            del self.requests[r.req_id]

        tokens_left = self.max_batch_tokens
        slots_left = self.max_requests
        scheduled = []        # (request, q_len, is_decode)

        # 1. active decodes, one token each
        for r in self._ordered(DECODING):
            if tokens_left < 1 or slots_left < 1:
                break
            need = 1 if r.cached % self.page == 0 else 0
            if need > self.free:
                st.stalled.append(r.req_id)
                continue
            self.free -= need
            r.pages += need
            st.new_pages += need
            scheduled.append((r, 1, True))
            tokens_left -= 1
            slots_left -= 1

        # 2. active prefills, each taking every token that still fits
        for r in self._ordered(PREFILLING):
            if tokens_left < 1 or slots_left < 1:
                break
            chunk = min(r.prompt_len - r.cached, tokens_left)
            if self.chunk_cap > 0:
                chunk = min(chunk, self.chunk_cap)
            chunk = min(chunk, (r.pages + self.free) * self.page - r.cached)
            if chunk <= 0:
                st.stalled.append(r.req_id)
                continue
            need = _ceil_div(r.cached + chunk, self.page) - r.pages
            self.free -= need
            r.pages += need
            st.new_pages += need
            scheduled.append((r, chunk, False))
            tokens_left -= chunk
            slots_left -= 1

        # 3. waiting requests in arrival order, strict head of line
        for r in self._ordered(WAITING):
            if tokens_left < 1 or slots_left < 1:
                break
            chunk = min(r.prompt_len, tokens_left)
            if self.chunk_cap > 0:
                chunk = min(chunk, self.chunk_cap)
            need = _ceil_div(chunk, self.page)
            if need > self.free:
                break
            if self.margin > 0.0 and (self.free - need) < self.margin * self.num_pages:
                break
            self.free -= need
            r.pages = need
            r.state = PREFILLING
            st.new_pages += need
            scheduled.append((r, chunk, False))
            tokens_left -= chunk
            slots_left -= 1

        # emit in scheduling order and advance each request
        for r, n, is_decode in scheduled:
            st.seqs.append(ScheduledSeq(r.req_id, n, r.cached, r.cached + n, is_decode, r.pages))
            r.cached += n
            if is_decode:
                r.generated += 1
            elif r.cached == r.prompt_len:
                r.generated = 1
            if r.generated >= 1:
                r.state = FINISHED if r.generated >= r.output_len else DECODING
        self.total_stalls += len(st.stalled)
        return st

    # -- accounting ---------------------------------------------------------------
    def pages_in_use(self) -> int:
        return self.num_pages - self.free

    def used_slots(self) -> int:
        return sum(r.cached for r in self.requests.values())

    def idle(self) -> bool:
        return not self.requests
