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
