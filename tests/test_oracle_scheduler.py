"""Pins of the plain-Python FIFO batch builder to the pages' rules and examples."""
import numpy as np
import pytest

from oracle.scheduler import FifoScheduler, SchedulerError
import workloads as wl


def _drive(s, max_steps=10000):
    steps = []
    for _ in range(max_steps):
        st = s.step()
        if not st.seqs and s.idle():
            break
        steps.append(st)
    return steps


def test_page_example_chunks_256_256_256_232():
    """A lone 1000-token prompt under a 256-token budget (the pages' example)."""
    s = FifoScheduler(256, 128, 63)
    s.submit(0, 1000, 1)
    steps = _drive(s)
    assert [st.num_tokens for st in steps] == [256, 256, 256, 232]
    assert [st.seqs[0].q_offset for st in steps] == [0, 256, 512, 768]
    assert [st.seqs[0].context_len for st in steps] == [256, 512, 768, 1000]
    assert s.free == 63 and s.idle()


def test_mixed_step_composition():
    """64 decodes, then the active 1500-token prefill at 1024, then 700 and 6000."""
    w = wl.mixed()
    s = FifoScheduler(w.max_batch_tokens, w.max_requests, w.pool_pages)
    for i, (p, o, c) in enumerate(w.requests):
        s.submit(i, p, o, c)
    st = s.step()
    assert st.num_decodes == 64 and st.num_tokens == 2048
    pf = st.seqs[64:]
    assert [(x.q_offset, x.q_len) for x in pf] == [(1024, 476), (0, 700), (0, 808)]
    assert all(x.q_len == 1 for x in st.seqs[:64])


def test_long_prompt_forty_chunks_of_512():
    w = wl.long_prompt()
    s = FifoScheduler(w.max_batch_tokens, w.max_requests, w.pool_pages,
                      max_prefill_chunk=w.max_prefill_chunk)
    for i, (p, o, c) in enumerate(w.requests):
        s.submit(i, p, o, c)
    chunks = []
    for _ in range(40):
        st = s.step()
        assert st.num_decodes == 127
        pf = [x for x in st.seqs if not x.is_decode]
        chunks.append((pf[0].q_offset, pf[0].q_len))
    assert chunks == [(512 * k, 512) for k in range(39)] + [(19968, 32)]


def test_decodes_first_then_active_prefills_then_waiting_fifo():
    s = FifoScheduler(10, 128, 1000)
    s.submit(1, 5, 3)          # waiting
    s.submit(2, 30, 2)         # waiting, long
    st = s.step()              # 1 admitted (5), 2 admitted with 5 tokens
    assert [(x.req_id, x.q_len) for x in st.seqs] == [(1, 5), (2, 5)]
    s.submit(3, 4, 2)
    st = s.step()              # decode of 1 first, then 2's next chunk, 3 waits for budget
    assert [(x.req_id, x.q_len, x.is_decode) for x in st.seqs] == [(1, 1, True), (2, 9, False)]
    st = s.step()
    assert [(x.req_id, x.q_len) for x in st.seqs] == [(1, 1), (2, 9), ]
    st = s.step()              # 1 finished (3 outputs -> 2 decodes) and released now
    assert st.finished == [1]
    assert [(x.req_id, x.q_len, x.q_offset) for x in st.seqs] == [(2, 7, 23), (3, 3, 0)]


def test_strict_head_of_line_and_request_cap():
    s = FifoScheduler(100, 2, 10)
    s.submit(1, 16 * 9, 1)     # needs 9 pages for its first chunk (100 tokens -> 7 pages)
    s.submit(2, 10, 1)
    s.submit(3, 10, 1)
    st = s.step()
    assert [x.req_id for x in st.seqs] == [1]      # 1 takes 100 tokens; budget gone
    s2 = FifoScheduler(1000, 2, 100)
    for i in range(4):
        s2.submit(i, 10, 1)
    assert [x.req_id for x in s2.step().seqs] == [0, 1]   # request cap
    s3 = FifoScheduler(1000, 8, 4)
    s3.submit(0, 64, 1)        # 4 pages: fits exactly
    s3.submit(1, 1, 1)         # no page left -> head of line blocks
    assert [x.req_id for x in s3.step().seqs] == [0]


def test_safety_margin_defers_new_prefills_but_not_decodes():
    s = FifoScheduler(1000, 8, 100, safety_margin=0.15)
    s.submit(0, 16 * 80, 5, 16 * 80)     # imported decode holding 80 pages
    s.submit(1, 16 * 10, 1)              # would leave 10 pages free (< 15) -> deferred
    st = s.step()
    assert [x.req_id for x in st.seqs] == [0] and st.new_pages == 1
    s0 = FifoScheduler(1000, 8, 100, safety_margin=0.0)
    s0.submit(0, 16 * 80, 5, 16 * 80)
    s0.submit(1, 16 * 10, 1)
    assert [x.req_id for x in s0.step().seqs] == [0, 1]


def test_decode_stalls_without_a_free_page():
    s = FifoScheduler(100, 8, 2)
    s.submit(0, 16, 4, 16)     # holds 1 page, next token needs a new page
    s.submit(1, 16, 4, 16)     # holds the other page
    st = s.step()
    assert st.seqs == [] and st.stalled == [0, 1]


def test_lifecycle_counts_and_page_conservation():
    rng = np.random.default_rng(0)
    s = FifoScheduler(64, 6, 60, max_prefill_chunk=24, safety_margin=0.1)
    outs = {}
    for i in range(30):
        p, o = int(rng.integers(1, 120)), int(rng.integers(1, 20))
        s.submit(i, p, o)
        outs[i] = (p, o)
    decode_steps = {i: 0 for i in outs}
    prefill_tokens = {i: 0 for i in outs}
    for st in _drive(s):
        assert st.num_tokens <= 64 and len(st.seqs) <= 6
        assert all(x.is_decode for x in st.seqs[:st.num_decodes])
        for x in st.seqs:
            assert x.pages == -(-x.context_len // 16)
            if x.is_decode:
                decode_steps[x.req_id] += 1
            else:
                prefill_tokens[x.req_id] += x.q_len
                assert x.q_len <= 24
        assert s.pages_in_use() == sum(r.pages for r in s.requests.values())
    assert s.free == 60
    for i, (p, o) in outs.items():
        assert prefill_tokens[i] == p and decode_steps[i] == o - 1


def test_submit_errors():
    s = FifoScheduler(10, 2, 4)
    s.submit(1, 5, 1)
    with pytest.raises(SchedulerError) as e:
        s.submit(1, 5, 1)
    assert e.value.kind == "invalid"
    with pytest.raises(SchedulerError) as e:
        s.submit(2, 64, 2)             # 65 KV tokens > 4 pages
    assert e.value.kind == "capacity"
    with pytest.raises(SchedulerError):
        s.submit(3, 0, 1)


# --- scheduler variants ------------------------------------------------------
def test_prefill_first_serves_active_prefills_before_decodes():
    """PrefillFirst: the split prefill takes the budget first; decodes get the rest."""
    def build(policy, budget):
        s = FifoScheduler(budget, 128, 100, policy=policy)
        s.submit(0, 20, 5, tokens_cached=4)          # active prefill, 16 tokens left
        for i in (1, 2, 3):
            s.submit(i, 8, 5, tokens_cached=10)      # decodes
        return s.step()
    fifo = build("fifo", 10)
    assert [(x.req_id, x.q_len) for x in fifo.seqs] == [(1, 1), (2, 1), (3, 1), (0, 7)]
    pf = build("prefill_first", 10)
    assert [(x.req_id, x.q_len) for x in pf.seqs] == [(0, 10)]
    pf = build("prefill_first", 18)                  # 16 for the prefill, 2 decodes
    assert [(x.req_id, x.q_len) for x in pf.seqs] == [(1, 1), (2, 1), (0, 16)]
    assert pf.num_decodes == 2                       # decodes are listed first


def test_partial_prefill_caps_four_prefills_one_long():
    """The page's example: up to four prefills per step, at most one over 10,000 tokens."""
    s = FifoScheduler(2048, 128, 10000, max_prefill_chunk=512, max_partial_prefills=4,
                      max_long_partial_prefills=1, long_prefill_threshold=10000)
    s.submit(0, 20000, 2)     # long
    s.submit(1, 15000, 2)     # long: must wait for 0's prefill
    s.submit(2, 500, 2)       # short: fast lane past request 1
    s.submit(3, 300, 2)
    s.submit(4, 200, 2)
    s.submit(5, 100, 2)       # fifth prefill: over the cap of four
    st = s.step()
    assert [(x.req_id, x.q_offset, x.q_len) for x in st.seqs] == [
        (0, 0, 512), (2, 0, 500), (3, 0, 300), (4, 0, 200)]
    st = s.step()
    # 2, 3, 4 decode; 0 continues; 1 stays behind the long cap; 5 fits now
    assert [(x.req_id, x.q_len) for x in st.seqs] == [(2, 1), (3, 1), (4, 1), (0, 512), (5, 100)]
    # with one prefill per step, prefills run one request at a time
    s = FifoScheduler(2048, 128, 10000, max_prefill_chunk=512, max_partial_prefills=1)
    s.submit(0, 700, 2)
    s.submit(1, 10, 2)
    assert [(x.req_id, x.q_len) for x in s.step().seqs] == [(0, 512)]
    assert [(x.req_id, x.q_len) for x in s.step().seqs] == [(0, 188)]
    assert [(x.req_id, x.q_len) for x in s.step().seqs] == [(0, 1), (1, 10)]


# --- prefix sharing -------------------------------------------------------------
def _prompt(n, seed=0, vocab=1000):
    return [int(t) for t in np.random.default_rng(seed).integers(0, vocab, n)]


def _sharing(pages=100, budget=256, **kw):
    return FifoScheduler(budget, 128, pages, allow_block_sharing=True, **kw)


def test_shared_prefix_skips_matched_blocks():
    s = _sharing()
    p = _prompt(40)
    s.submit(0, 40, 4, tokens=p)
    a = s.step().seqs[0]
    assert (a.q_offset, a.q_len, a.prefix_hit) == (0, 40, 0)
    assert a.blocks[2] == -1 and a.blocks[0] >= 0 and a.blocks[1] >= 0   # 2 full blocks registered
    s.submit(1, 40, 4, tokens=p)
    st = s.step()
    b = [x for x in st.seqs if x.req_id == 1][0]
    # blocks 0 and 1 (32 tokens) are reused; the last 8 prompt tokens are computed
    assert (b.q_offset, b.q_len, b.context_len, b.prefix_hit) == (32, 8, 40, 32)
    assert b.blocks[:2] == a.blocks[:2] and b.blocks[2] == -1
    # 3 pages for request 0, 1 more for its decode at 40 -> no; 40 % 16 != 0, so 3,
    # plus 1 private page for request 1
    assert s.pages_in_use() == 4 and s.prefix_hit_tokens == 32


def test_last_prompt_token_is_always_computed():
    s = _sharing()
    p = _prompt(32, seed=1)
    s.submit(0, 32, 3, tokens=p)
    s.step()
    s.submit(1, 32, 3, tokens=p)
    b = [x for x in s.step().seqs if x.req_id == 1][0]
    # two full blocks are registered, but only one can be reused: the second
    # holds the last prompt token, which must be computed
    assert (b.q_offset, b.q_len, b.prefix_hit) == (16, 16, 16)
    assert b.blocks[1] == -1


def test_partial_match_and_no_match():
    s = _sharing()
    p = _prompt(64, seed=2)
    s.submit(0, 64, 2, tokens=p)
    s.step()
    q = list(p)
    q[20] += 1                              # differs inside block 1
    s.submit(1, 64, 2, tokens=q)
    r = list(p)
    r[0] += 1                               # differs in block 0
    s.submit(2, 64, 2, tokens=r)
    st = s.step()
    hits = {x.req_id: (x.q_offset, x.prefix_hit) for x in st.seqs if not x.is_decode}
    assert hits == {1: (16, 16), 2: (0, 0)}


def test_shared_blocks_are_reference_counted_and_reusable_after_release():
    s = _sharing(pages=20)
    p = _prompt(48, seed=3)
    s.submit(0, 48, 2, tokens=p)            # prefill step, then one decode step
    s.step()
    s.submit(1, 48, 2, tokens=p)
    s.step()                                # 0 decodes (finishes); 1 reuses 2 blocks
    held = s.pages_in_use()
    st = s.step()                           # 0 released; its shared blocks stay held by 1
    assert st.finished == [0]
    # 0's block 2 (registered, now unheld) and its decode page are free; 1's
    # decode at 48 takes a fresh page
    assert s.pages_in_use() == held - 2 + 1
    s.step()                                # 1 (finished last step) released
    assert s.pages_in_use() == 0 and s.free == 20
    assert len(s.cached) == 3               # blocks 0, 1, 2 keep their registration
    s.submit(2, 48, 2, tokens=p)
    b = s.step().seqs[0]
    assert (b.q_offset, b.prefix_hit) == (32, 32)   # released blocks still match
    assert s.pages_in_use() == 3


def test_newest_cached_block_is_demoted_first():
    s = _sharing(pages=6, budget=128)
    p, q = _prompt(33, seed=4), _prompt(33, seed=5)
    s.submit(0, 33, 1, tokens=p)            # output 1: finishes with its prefill
    s.submit(1, 33, 1, tokens=q)
    s.step()
    s.step()                                # both released: 0's then 1's pages
    assert s.free == 6 and s.clean == 2 and len(s.cached) == 4
    s.submit(2, 40, 1, tokens=_prompt(40, seed=6))   # 3 pages: 2 clean + 1 demoted
    s.step()
    # the newest cached block (1's block 1) lost its registration
    s.step()
    s.submit(3, 33, 1, tokens=q)
    s.submit(4, 33, 1, tokens=p)
    st = s.step()
    hits = {x.req_id: x.prefix_hit for x in st.seqs}
    assert hits == {3: 16, 4: 32}


def test_identical_prompts_admitted_together_do_not_share():
    s = _sharing()
    p = _prompt(40, seed=7)
    s.submit(0, 40, 3, tokens=p)
    s.submit(1, 40, 3, tokens=p)
    st = s.step()
    a, b = st.seqs
    assert a.prefix_hit == b.prefix_hit == 0
    assert a.blocks[:2] != b.blocks[:2] and b.blocks == (-1, -1, -1)   # 1 stops registering
    s.submit(2, 40, 3, tokens=p)
    c = [x for x in s.step().seqs if x.req_id == 2][0]
    assert c.blocks[:2] == a.blocks[:2] and c.prefix_hit == 32


def test_sharing_off_or_without_tokens_changes_nothing():
    p = _prompt(40, seed=8)
    for kw in ({"allow_block_sharing": False}, {"allow_block_sharing": True}):
        s = FifoScheduler(256, 128, 100, **kw)
        s.submit(0, 40, 3, tokens=p)
        s.step()
        s.submit(1, 40, 3, tokens=p if not kw["allow_block_sharing"] else None)
        b = [x for x in s.step().seqs if x.req_id == 1][0]
        assert (b.q_offset, b.prefix_hit) == (0, 0)


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_sharing_pool_invariants_on_random_traces(seed):
    """Pages are conserved and every block's count equals the requests holding it."""
    rng = np.random.default_rng(100 + seed)
    base = [_prompt(int(rng.integers(16, 120)), seed=1000 * seed + k, vocab=50) for k in range(4)]
    s = FifoScheduler(96, 16, 60, max_prefill_chunk=int(rng.integers(0, 3)) * 24,
                      allow_block_sharing=True)
    rid = 0
    for _ in range(300):
        if rng.random() < 0.5:
            b = base[int(rng.integers(0, 4))]
            n = int(rng.integers(1, len(b) + 1))
            toks = list(b[:n]) + _prompt(int(rng.integers(0, 20)), seed=rid, vocab=50)
            try:
                s.submit(rid, len(toks), int(rng.integers(1, 12)), tokens=toks)
            except Exception:
                pass
            rid += 1
        s.step()
        held = {}
        private = 0
        for r in s.requests.values():
            for e in r.blocks:
                if e is None:
                    private += 1
                else:
                    held[id(e)] = held.get(id(e), 0) + 1
                    assert e.ref >= 1
        objs = {id(e): e for r in s.requests.values() for e in r.blocks if e is not None}
        assert all(objs[k].ref == v for k, v in held.items())
        assert all(c.ref == 0 and id(c) not in held for c in s.cached)
        assert s.pages_in_use() == private + len(held)
        assert 0 <= s.clean and s.free <= s.num_pages
    assert s.prefix_hit_tokens > 0


# --- sliding window: pages recycled below the window ----------------------------
def test_window_releases_pages_below_every_later_row():
    s = FifoScheduler(256, 8, 100, sliding_window=32)
    s.submit(0, 100, 40)
    st = s.step()                          # prefill 0..99: pages 0..6
    assert (st.seqs[0].pages, st.seqs[0].held) == (7, 7)
    st = s.step()                          # later rows see keys >= 100 - 31 = 69: pages 0..3 go
    assert st.seqs[0].blocks[:4] == (-2, -2, -2, -2)
    assert (st.seqs[0].pages, st.seqs[0].held, s.pages_in_use()) == (7, 3, 3)
    # decodes at 100..111 stay in page 6; the decode at 112 adds page 7 and, its
    # keys starting at 81, releases page 4 (64..79)
    for _ in range(11):
        s.step()
    st = s.step()
    assert (st.seqs[0].q_offset, st.seqs[0].pages, st.seqs[0].held, s.pages_in_use()) == (112, 8, 3, 3)
    for _ in range(14):                    # decodes at 113..126
        st = s.step()
    assert st.seqs[0].q_offset == 126 and st.seqs[0].held == 3
    st = s.step()                          # at 127 keys start at 96: page 5 (80..95) goes
    assert (st.seqs[0].held, s.pages_in_use()) == (2, 2)
    st = s.step()                          # at 128 a new page
    assert (st.seqs[0].pages, st.seqs[0].held) == (9, 3)


def test_window_lets_a_long_request_run_in_a_small_pool():
    # 200 + 20 - 1 tokens need 14 pages; the pool has 8
    with pytest.raises(SchedulerError) as e:
        FifoScheduler(64, 8, 8).submit(0, 200, 20)
    assert e.value.kind == "capacity"
    s = FifoScheduler(64, 8, 8, max_prefill_chunk=64, sliding_window=32)
    s.submit(0, 200, 20)                  # peak: ceil((31 + 64) / 16) + 1 = 7 pages
    steps = _drive(s)
    assert [x.seqs[0].q_len for x in steps[:4]] == [64, 64, 64, 8]
    assert len(steps) == 4 + 19 and s.free == 8
    assert max(x.seqs[0].held for x in steps) <= 7


def test_window_import_allocates_only_the_window():
    s = FifoScheduler(256, 8, 20, sliding_window=32)
    s.submit(0, 100, 5, tokens_cached=100)   # keys from 69 on: pages 4, 5, 6
    assert s.pages_in_use() == 3
    st = s.step()
    assert st.seqs[0].blocks[:4] == (-2, -2, -2, -2) and st.seqs[0].held == 3


def test_window_excludes_block_sharing():
    with pytest.raises(SchedulerError):
        FifoScheduler(64, 8, 8, sliding_window=16, allow_block_sharing=True)


@pytest.mark.parametrize("seed", [0, 1])
def test_window_pool_invariants_on_random_traces(seed):
    rng = np.random.default_rng(300 + seed)
    W = int(rng.choice([1, 16, 17, 40]))
    s = FifoScheduler(80, 8, 40, max_prefill_chunk=int(rng.choice([0, 24])), sliding_window=W)
    rid = 0
    for _ in range(400):
        if rng.random() < 0.4:
            p = int(rng.integers(1, 300))
            c = int(rng.integers(0, p + 20)) if rng.random() < 0.2 else 0
            try:
                s.submit(rid, p, int(rng.integers(1, 30)), tokens_cached=c)
            except SchedulerError:
                pass
            rid += 1
        st = s.step()
        assert s.pages_in_use() == sum(r.held for r in s.requests.values())
        for x in st.seqs:   # every page a row of this step can see is held
            first_key = max(0, x.q_offset - W + 1)
            assert all(b != -2 for b in x.blocks[first_key // 16:])
    assert s.idle() or rid > 0


# -- cached-token accounting (the fragmentation figure) --------------------------------
#
# AI Engineering from Scratch, "vLLM serving internals", "PagedAttention as
# virtual memory": with 16-token pages the only waste is the unused tail of
# each sequence's last page (under 4% in practice).  Fragmentation here is
# (pages in use * 16 - cached tokens held) / (pages in use * 16), with a
# shared page counted once and a page released below a sliding window not
# counted at all.  The expected numbers below are worked out by hand.

def _acct(s):
    alloc = s.pages_in_use() * s.page
    return s.used_slots(), alloc


def test_used_slots_counts_a_shared_block_once_and_a_partial_page_by_its_fill():
    toks_a = list(range(100, 140))                       # 40 prompt tokens
    toks_b = list(range(100, 132)) + [7, 8, 9, 10]       # same first 32, own 4
    s = FifoScheduler(64, 8, 20, allow_block_sharing=True)
    s.submit(0, 40, 3, tokens=toks_a)
    s.step()
    # A holds tokens 0..39 in 3 pages (16 + 16 + 8); blocks 0 and 1 are registered
    assert _acct(s) == (40, 48)
    s.submit(1, 36, 2, tokens=toks_b)
    st = s.step()
    assert [(x.req_id, x.q_offset, x.q_len) for x in st.seqs] == [(0, 40, 1), (1, 32, 4)]
    # pages: the two shared prompt blocks, A's third page (41 - 32 = 9 tokens)
    # and B's third page (36 - 32 = 4 tokens).  Shared blocks count once.
    used, alloc = _acct(s)
    assert alloc == 4 * 16
    assert used == 16 + 16 + 9 + 4                     # not 16*4 + 9 + 4 = 77
    assert s.pages_in_use() == 4


def test_used_slots_skips_pages_released_below_the_window():
    s = FifoScheduler(64, 8, 20, sliding_window=20)
    s.submit(0, 40, 10)
    s.step()
    assert _acct(s) == (40, 48)                          # 16 + 16 + 8 in 3 pages
    s.step()
    # at the step's start the lowest key any later row sees is 40 - 20 + 1 = 21,
    # so page 0 (keys 0..15) is released; the decode then caches token 40:
    # page 1 holds 16 tokens, page 2 holds 41 - 32 = 9
    used, alloc = _acct(s)
    assert (used, alloc) == (16 + 9, 2 * 16)            # not 41 over 48

