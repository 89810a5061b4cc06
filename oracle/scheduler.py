"""Plain-Python batch builder (test infrastructure only).

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
  - "PrefillFirst": split prefills are carried to completion before decoding
    resumes.
  - "Admission": a request that any allocator cannot hold is rejected and
    nothing is allocated; below ``safety_margin`` of free capacity new
    prefills are deferred and only active work continues.
  - "Prefix caching": every full block gets a hash of its content; a later
    request with the same prompt prefix reuses those blocks and skips their
    prefill; shared blocks are reference counted and go back to the free pool
    only when no request uses them any more.
  - "Eviction" (of cached blocks): released blocks keep their content and
    hash so that a later prefix can still match them; when uninitialised
    blocks run out, the newest initialised ones lose their hash and are
    handed out again.
* Ultralytics glossary, "Chunked Prefill", "How chunked prefill works": one
  token per running decode first, then the remaining budget is filled with
  chunks of waiting prompts.
* AI Engineering from Scratch, "vLLM serving internals", section "What the
  scheduler looks like": finished sequences release their blocks at the top
  of the loop; waiting sequences are admitted from the head of the queue
  while blocks are free (strict head of line).
* TNG blog on LLM serving performance, "Request-parallel prefill": prefills
  of several requests may share a step, with a cap on how many of them have
  a long prompt (the example: four prefills, at most one above 10,000
  tokens), so that short prompts need not wait behind a long one.

Readings where the pages are silent or ambiguous:

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
  + 1`` tokens; imports and submissions share one arrival order;
* PrefillFirst picks active prefills, then active decodes, then waiting
  requests; under every policy the step lists its decodes first;
* the partial-prefill caps count the prefill chunks of one step (active and
  newly admitted); a prefill over a cap is skipped (not stalled) and the
  requests behind it are still considered; "long" means a prompt longer
  than ``long_prefill_threshold`` tokens;
* prefix sharing applies to requests submitted with their prompt tokens; a
  block's identity is its tokens together with the identity of the block
  before it, and only blocks wholly inside the prompt are hashed; a match
  stops short of the last prompt token, which is always computed, so no
  step writes into a shared page; blocks are registered when the step that
  fills them is built, in order, and a request stops registering at its
  first block whose identity is already registered; a reused block that no
  request held counts against the free pages at admission; an allocation
  takes a page that holds no registered block when there is one, else the
  most recently released registered block, whose registration ends;
* sliding window (transformers, "Memory management": sliding layers keep a
  fixed window of recent tokens by recycling a small set of pages, and do not
  share blocks): at the start of a step, after finished requests are
  released, every live request releases the pages that lie wholly below
  ``cached - W + 1``, the lowest key any of its later rows can see; released
  pages leave holes in its block table (the kernel never reads them); an
  import allocates only the pages still inside its window; a request is
  rejected as never fitting only if even its largest simultaneous need (its
  window plus one chunk) exceeds the pool; a window together with block
  sharing is invalid.

Physical page ids are not unique (any free page is correct), so this model
tracks page *counts* and block identities, not page ids.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Optional

import numpy as np

WAITING, PREFILLING, DECODING, FINISHED = "waiting", "prefilling", "decoding", "finished"
FIFO, PREFILL_FIRST = "fifo", "prefill_first"
RELEASED = "released"        # a block-table entry whose page went back to the pool


class SchedulerError(ValueError):
    def __init__(self, kind: str, msg: str):
        super().__init__(msg)
        self.kind = kind          # "invalid" or "capacity"


@dataclass(eq=False)
class Block:
    """A registered full prompt block: the page that holds it is shared."""
    serial: int                   # identity; never reused
    key: tuple                    # (parent block's serial or -1, its tokens)
    ref: int = 1                  # requests holding it


@dataclass
class Request:
    req_id: int
    prompt_len: int
    output_len: int
    arrival: int
    cached: int = 0
    generated: int = 0
    state: str = WAITING
    tokens: Optional[tuple] = None
    # one entry per logical page: a Block when the page holds a registered
    # block, None for a page private to this request, RELEASED for a page
    # below the sliding window that went back to the pool
    blocks: list = field(default_factory=list)
    registered: int = 0           # leading blocks that are registered or matched
    stop_registering: bool = False
    released: int = 0             # leading entries that are RELEASED

    @property
    def pages(self) -> int:
        """Length of the block table (logical pages)."""
        return len(self.blocks)

    @property
    def held(self) -> int:
        return len(self.blocks) - self.released


@dataclass
class ScheduledSeq:
    req_id: int
    q_len: int
    q_offset: int          # KV length before this step's tokens
    context_len: int       # KV length after this step's tokens
    is_decode: bool
    pages: int             # block-table length after this step's allocation
    blocks: tuple = ()     # per logical page: block serial, -1 if private, -2 if released
    prefix_hit: int = 0    # tokens reused from shared blocks at admission
    held: int = 0          # pages actually held (pages minus released ones)


@dataclass
class Step:
    seqs: list = field(default_factory=list)
    finished: list = field(default_factory=list)   # released at the start of this step
    stalled: list = field(default_factory=list)
    new_pages: int = 0     # pages taken from the free pool (fresh or reused blocks)

    @property
    def num_decodes(self) -> int:
        return sum(1 for s in self.seqs if s.is_decode)

    @property
    def num_tokens(self) -> int:
        return sum(s.q_len for s in self.seqs)


def _ceil_div(a: int, b: int) -> int:
    return -(-a // b)


class Scheduler:
    def __init__(self, max_batch_tokens: int, max_requests_per_batch: int, num_pages: int,
                 page_size: int = 16, max_prefill_chunk: int = 0, safety_margin: float = 0.0,
                 policy: str = FIFO, max_partial_prefills: int = 0,
                 max_long_partial_prefills: int = 0, long_prefill_threshold: int = 0,
                 allow_block_sharing: bool = False, sliding_window: int = 0):
        if max_batch_tokens < 1 or max_requests_per_batch < 1 or num_pages < 1 or page_size < 1:
            raise SchedulerError("invalid", "budgets and pool size must be positive")
        if max_prefill_chunk < 0 or not (0.0 <= safety_margin < 1.0):
            raise SchedulerError("invalid", "bad chunk cap or safety margin")
        if policy not in (FIFO, PREFILL_FIRST):
            raise SchedulerError("invalid", f"unknown policy {policy!r}")
        if min(max_partial_prefills, max_long_partial_prefills, long_prefill_threshold) < 0:
            raise SchedulerError("invalid", "prefill caps must be >= 0")
        if sliding_window < 0 or (sliding_window > 0 and allow_block_sharing):
            raise SchedulerError("invalid", "window must be >= 0 and excludes block sharing")
        self.max_batch_tokens = max_batch_tokens
        self.max_requests = max_requests_per_batch
        self.num_pages = num_pages
        self.page = page_size
        self.chunk_cap = max_prefill_chunk
        # the margin is a float32 configuration value; compare in float64
        self.margin = float(np.float32(safety_margin))
        self.policy = policy
        self.max_partial = max_partial_prefills
        self.max_long = max_long_partial_prefills
        self.long_threshold = long_prefill_threshold
        self.sharing = bool(allow_block_sharing)
        self.window = sliding_window
        self.clean = num_pages            # free pages holding no registered block
        self.cached: list[Block] = []     # released registered blocks, newest last
        self.index: dict[tuple, Block] = {}
        self._serials = 0
        self.requests: dict[int, Request] = {}
        self._arrivals = 0
        self.total_stalls = 0
        self.prefix_hit_tokens = 0

    # -- the page pool ------------------------------------------------------------
    @property
    def free(self) -> int:
        return self.clean + len(self.cached)

    def _take(self):
        """One page for private use: a clean page if any, else the newest cached block."""
        assert self.free > 0
        if self.clean > 0:
            self.clean -= 1
        else:
            blk = self.cached.pop()
            if self.index.get(blk.key) is blk:
                del self.index[blk.key]
        return None

    def _release(self, entry):
        if entry is None:
            self.clean += 1
            return
        entry.ref -= 1
        if entry.ref == 0:
            self.cached.append(entry)

    def _key(self, parent, tokens, i):
        return (parent.serial if parent is not None else -1,
                tuple(tokens[i * self.page:(i + 1) * self.page]))

    def _match(self, r):
        """Registered blocks matching r's prompt, leaving its last token to compute."""
        found, parent = [], None
        for i in range((r.prompt_len - 1) // self.page):
            blk = self.index.get(self._key(parent, r.tokens, i))
            if blk is None:
                break
            found.append(blk)
            parent = blk
        return found

    def _register(self, r):
        full = min(r.cached, r.prompt_len) // self.page
        while r.registered < full and not r.stop_registering:
            i = r.registered
            parent = r.blocks[i - 1] if i > 0 else None
            key = self._key(parent, r.tokens, i)
            if key in self.index:
                r.stop_registering = True
                break
            blk = Block(self._serials, key)
            self._serials += 1
            self.index[key] = blk
            r.blocks[i] = blk
            r.registered += 1

    # -- submission ---------------------------------------------------------------
    def submit(self, req_id: int, prompt_len: int, output_len: int, tokens_cached: int = 0,
               tokens=None):
        if req_id in self.requests:
            raise SchedulerError("invalid", f"duplicate request id {req_id}")
        if prompt_len < 1 or output_len < 1 or tokens_cached < 0:
            raise SchedulerError("invalid", "lengths must be positive")
        if tokens is not None and (len(tokens) != prompt_len or tokens_cached > 0):
            raise SchedulerError("invalid", "tokens must hold the whole prompt of a new request")
        final_kv = prompt_len + output_len - 1
        if tokens_cached >= final_kv and tokens_cached > 0:
            raise SchedulerError("invalid", "request has nothing left to do")
        peak = _ceil_div(final_kv, self.page)
        if self.window > 0:    # the window plus one chunk (+1 page for misalignment)
            chunk = min(prompt_len, self.max_batch_tokens)
            if self.chunk_cap > 0:
                chunk = min(chunk, self.chunk_cap)
            peak = min(peak, _ceil_div(self.window - 1 + chunk, self.page) + 1)
        if peak > self.num_pages:
            raise SchedulerError("capacity", "request can never fit the page pool")
        r = Request(req_id, prompt_len, output_len, self._arrivals,
                    tokens=tuple(int(t) for t in tokens) if tokens is not None else None)
        if tokens_cached > 0:
            first = self._window_floor(tokens_cached)
            need = _ceil_div(tokens_cached, self.page) - first
            if need > self.free:
                raise SchedulerError("capacity", "not enough free pages to import")
            r.blocks = [RELEASED] * first + [self._take() for _ in range(need)]
            r.released = first
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

    def _window_floor(self, cached: int) -> int:
        """Logical pages wholly below every later row's window."""
        if self.window <= 0:
            return 0
        return max(0, cached - self.window + 1) // self.page

    def _is_long(self, r) -> bool:
        return r.prompt_len > self.long_threshold

    def step(self) -> Step:
        st = Step()
        # release what finished last step
        for r in self._ordered(FINISHED):
            for entry in r.blocks:
                if entry is not RELEASED:
                    self._release(entry)
            st.finished.append(r.req_id)
            del self.requests[r.req_id]
        # pages that fell out of every live request's window
        for r in sorted(self.requests.values(), key=lambda r: r.arrival):
            lim = min(self._window_floor(r.cached), len(r.blocks))
            while r.released < lim:
                self._release(r.blocks[r.released])
                r.blocks[r.released] = RELEASED
                r.released += 1

        budget = {"tokens": self.max_batch_tokens, "slots": self.max_requests,
                  "prefills": 0, "long": 0}
        scheduled = []        # (request, q_len, is_decode, prefix_hit)

        def room() -> bool:
            return budget["tokens"] >= 1 and budget["slots"] >= 1

        def prefill_capped(r) -> bool:
            if self.max_partial > 0 and budget["prefills"] >= self.max_partial:
                return True
            return self.max_long > 0 and self._is_long(r) and budget["long"] >= self.max_long

        def take_prefill(r, n):
            budget["tokens"] -= n
            budget["slots"] -= 1
            budget["prefills"] += 1
            budget["long"] += 1 if self._is_long(r) else 0

        # active decodes, one token each
        def decodes():
            for r in self._ordered(DECODING):
                if not room():
                    break
                need = 1 if r.cached % self.page == 0 else 0
                if need > self.free:
                    st.stalled.append(r.req_id)
                    continue
                for _ in range(need):
                    r.blocks.append(self._take())
                st.new_pages += need
                scheduled.append((r, 1, True, 0))
                budget["tokens"] -= 1
                budget["slots"] -= 1

        # active prefills, each taking every token that still fits
        def active_prefills():
            for r in self._ordered(PREFILLING):
                if not room():
                    break
                if prefill_capped(r):
                    continue
                chunk = min(r.prompt_len - r.cached, budget["tokens"])
                if self.chunk_cap > 0:
                    chunk = min(chunk, self.chunk_cap)
                chunk = min(chunk, (len(r.blocks) + self.free) * self.page - r.cached)
                if chunk <= 0:
                    st.stalled.append(r.req_id)
                    continue
                need = _ceil_div(r.cached + chunk, self.page) - len(r.blocks)
                for _ in range(need):
                    r.blocks.append(self._take())
                st.new_pages += need
                scheduled.append((r, chunk, False, 0))
                take_prefill(r, chunk)

        # waiting requests in arrival order, strict head of line on pages
        def waiting():
            for r in self._ordered(WAITING):
                if not room():
                    break
                if prefill_capped(r):
                    continue
                matched = self._match(r) if (self.sharing and r.tokens is not None) else []
                start = len(matched) * self.page
                chunk = min(r.prompt_len - start, budget["tokens"])
                if self.chunk_cap > 0:
                    chunk = min(chunk, self.chunk_cap)
                fresh = _ceil_div(chunk, self.page)
                reused = sum(1 for b in matched if b.ref == 0)
                need = fresh + reused
                if need > self.free:
                    break
                if self.margin > 0.0 and (self.free - need) < self.margin * self.num_pages:
                    break
                for b in matched:
                    if b.ref == 0:
                        self.cached.remove(b)
                    b.ref += 1
                r.blocks = list(matched) + [self._take() for _ in range(fresh)]
                r.cached = start
                r.registered = len(matched)
                r.state = PREFILLING
                st.new_pages += need
                self.prefix_hit_tokens += start
                scheduled.append((r, chunk, False, start))
                take_prefill(r, chunk)

        if self.policy == FIFO:
            decodes()
            active_prefills()
        else:
            active_prefills()
            decodes()
        waiting()

        # emit decodes first, each class in scheduling order, and advance
        ordered = [x for x in scheduled if x[2]] + [x for x in scheduled if not x[2]]
        for r, n, is_decode, hit in ordered:
            r.cached += n
            if is_decode:
                r.generated += 1
            elif r.cached == r.prompt_len:
                r.generated = 1
            if r.generated >= 1:
                r.state = FINISHED if r.generated >= r.output_len else DECODING
            if self.sharing and r.tokens is not None:
                self._register(r)
            st.seqs.append(ScheduledSeq(
                r.req_id, n, r.cached - n, r.cached, is_decode, r.pages,
                tuple(-2 if b is RELEASED else (b.serial if b is not None else -1) for b in r.blocks),
                hit, r.held))
        self.total_stalls += len(st.stalled)
        return st

    # -- accounting ---------------------------------------------------------------
    def pages_in_use(self) -> int:
        return self.num_pages - self.free

    def used_slots(self) -> int:
        """Cached tokens held in pages; a shared block counts once."""
        total, shared = 0, {}
        for r in self.requests.values():
            for i, e in enumerate(r.blocks):
                fill = max(0, min(self.page, r.cached - i * self.page))
                if e is RELEASED:
                    continue
                if e is None:
                    total += fill
                else:
                    shared[id(e)] = max(shared.get(id(e), 0), fill)
        return total + sum(shared.values())

    def idle(self) -> bool:
        return not self.requests


# the pages' default scheduler
FifoScheduler = Scheduler
