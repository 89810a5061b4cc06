"""The five workloads at full size, through the whole step (C++ builder ->
metadata upload -> cb_kv_append -> cb_attention_step), against the oracle.

Decode rows are checked for every sequence; prefill chunks are checked on
sampled query rows (first, last and seeded random rows), which the oracle
computes one by one.  The long prompt is checked on all 40 steps and the FIFO
trace on every one of its steps, its appends bit for bit.
"""
import math

import numpy as np
import pytest
import torch

from gpu_util import compare, dev, say
from oracle import attention as ora
from oracle import paging
from chunked_prefill_attention_amd.engine import PagedAttentionLayer
import workloads as wl

pytestmark = pytest.mark.gpu


class Run:
    """A workload whose K/V values are fixed per (request, position)."""

    def __init__(self, w: wl.Workload):
        self.w = w
        self.layer = PagedAttentionLayer(w.n_q_heads, w.n_kv_heads, w.head_dim, w.pool_pages,
                                         w.max_batch_tokens, w.max_requests, w.dtype, w.max_prefill_chunk,
                                         w.safety_margin, page_shuffle_seed=w.seed, cache_fill=float("nan"))
        self.hist = {}
        for i, (p, o, c) in enumerate(w.requests):
            self.layer.builder.submit(i, p, o, c)
            k, v = wl.seq_kv(w.seed, i, 0, p + o - 1, w.n_kv_heads, w.head_dim, w.dtype)
            self.hist[i] = (k, v)
            if c > 0:
                self.layer.write_positions(i, 0, c, self._dev(k[:c]),
                                           self._dev(v[:c]))
        self.steps = 0

    def _dev(self, x):
        return torch.from_numpy(np.ascontiguousarray(x)).to(dev()).to(self.layer.tdtype)

    def step(self):
        L, w = self.layer, self.w
        desc = L.schedule()
        ks, vs = [], []
        for s in range(desc.num_seqs):
            i = int(desc.req_ids[s])
            a, e = int(desc.q_offsets[s]), int(desc.context_lens[s])
            ks.append(self.hist[i][0][a:e])
            vs.append(self.hist[i][1][a:e])
        q = wl.step_q(w.seed, self.steps, desc.num_tokens, w.n_q_heads, w.head_dim, w.dtype)
        out = L.attend(self._dev(q), self._dev(np.concatenate(ks)), self._dev(np.concatenate(vs)))
        torch.cuda.synchronize()
        self.steps += 1
        return desc, q, out.float().cpu().numpy()

    def check(self, desc, q, out, n_rows=24, rng_seed=0):
        w = self.w
        scale = wl.softmax_scale(w.head_dim)
        rng = np.random.default_rng(rng_seed)
        worst = 0.0
        for s in range(desc.num_seqs):
            i = int(desc.req_ids[s])
            a, e = int(desc.query_start_loc[s]), int(desc.query_start_loc[s + 1])
            ctx = int(desc.context_lens[s])
            k, v = self.hist[i][0][:ctx], self.hist[i][1][:ctx]
            if e - a == 1:
                ref = ora.attend(q[a:e], k, v, scale)
                am = ora.attend(q[a:e], k, np.abs(v), scale)
                worst = max(worst, compare(out[a:e], ref, w.dtype, f"decode seq {s}", am))
            else:
                L = e - a
                pick = sorted(set([0, L - 1] + rng.integers(0, L, size=n_rows).tolist()))
                rows = [(ii, h) for ii in pick for h in range(w.n_q_heads)]
                ref = ora.attend_rows(q[a:e], k, v, scale, rows=rows)
                am = ora.attend_rows(q[a:e], k, np.abs(v), scale, rows=rows)
                worst = max(worst, compare(out[a:e][pick], ref[pick], w.dtype, f"prefill seq {s} rows {pick[:4]}..",
                                           am[pick]))
        return worst

    def check_groups(self, desc, q, out, n_rows=4, rng_seed=0):
        """Every decode row and ``n_rows`` + 2 rows of each prefill chunk (its
        first, last and seeded others), each on one seeded KV head and the
        query heads that read it."""
        w = self.w
        G = w.n_q_heads // w.n_kv_heads
        scale = wl.softmax_scale(w.head_dim)
        rng = np.random.default_rng(rng_seed)
        worst = 0.0
        for s in range(desc.num_seqs):
            i = int(desc.req_ids[s])
            a, e = int(desc.query_start_loc[s]), int(desc.query_start_loc[s + 1])
            ctx, L = int(desc.context_lens[s]), e - a
            pick = [0] if L == 1 else sorted(set([0, L - 1] + rng.integers(0, L, size=n_rows).tolist()))
            for ii in pick:
                g = int(rng.integers(0, w.n_kv_heads))
                heads = slice(g * G, (g + 1) * G)
                pos = ctx - L + ii
                k = self.hist[i][0][:pos + 1, g:g + 1]
                v = self.hist[i][1][:pos + 1, g:g + 1]
                qr = q[a + ii:a + ii + 1, heads]
                ref = ora.attend(qr, k, v, scale)
                am = ora.attend(qr, k, np.abs(v), scale)
                worst = max(worst, compare(out[a + ii:a + ii + 1, heads], ref, w.dtype,
                                           f"seq {s} row {ii} kv head {g}", am))
        return worst


def test_decode_only_128_sequences():
    say("decode-only: 128 seqs, ctx U[512,4096], 32q/8kv, D128, bf16")
    r = Run(wl.decode_only())
    desc, q, out = r.step()
    assert desc.num_decodes == 128 and desc.num_tokens == 128
    say(f"  max abs err {r.check(desc, q, out):.2e}")


def test_mixed_step():
    say("mixed: 64 decodes + 476@1024 + 700 + 808, 32q/8kv, D128, bf16")
    r = Run(wl.mixed())
    desc, q, out = r.step()
    assert desc.num_tokens == 2048 and desc.num_decodes == 64
    assert desc.q_lens[64:].tolist() == [476, 700, 808]
    say(f"  max abs err {r.check(desc, q, out, n_rows=48):.2e}")


@pytest.mark.timeout(900)
def test_long_prompt_forty_steps():
    """Every one of the 40 steps is checked: all 127 decode rows and six rows
    of the chunk, each on a seeded KV head's group of 8 query heads; steps 0,
    1, 19, 38 and 39 also on every head of every decode row and of 26 chunk
    rows."""
    say("long prompt: 127 decodes + 20000-token prompt in 512-token chunks, 64q/8kv, D128, bf16")
    r = Run(wl.long_prompt())
    for k in range(40):
        desc, q, out = r.step()
        pf = desc.q_lens[desc.num_decodes:]
        assert desc.num_decodes == 127 and pf.tolist() == ([512] if k < 39 else [32])
        err = r.check_groups(desc, q, out, rng_seed=100 + k)
        if k in (0, 1, 19, 38, 39):
            err = max(err, r.check(desc, q, out, rng_seed=k))
        say(f"  step {k}: chunk at {desc.q_offsets[-1]}, max abs err {err:.2e}")
    # the later chunks are a large share of their steps: those run with the
    # prefill and decode workgroups split by CU (and were checked above)
    n = r.layer.stats()["cu_split_steps"]
    say(f"  {n} of 40 steps split by CU")
    assert 0 < n < 40


def _bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    return (bits.astype(np.uint32) << 16).view(np.float32)


def _pages_of(cache: torch.Tensor, pages: np.ndarray) -> np.ndarray:
    """Host copy (bf16 bits) of the given physical pages of a device cache."""
    idx = torch.from_numpy(pages.astype(np.int64)).to(cache.device)
    return cache[idx].view(torch.int16).cpu().numpy().view(np.uint16)


@pytest.mark.timeout(900)
def test_fifo_trace_every_step():
    """256 requests, Poisson arrivals, lognormal prompts, geometric outputs, pool 200k pages.

    K, V and Q of each step are drawn on the device; the host keeps a copy of
    every request's K/V history for the oracle.  Every step is checked:
    * append: the pages the step wrote are read back and every slot of its
      slot mapping must hold the token's K and V bits (oracle/paging.append
      onto the read-back pages changes nothing);
    * attention, on every query head: one seeded decode row, and the first,
      last and three seeded interior rows of one prefill chunk;
    * paging: the sampled sequences' whole histories, gathered through their
      block tables (oracle/paging.gather), equal the host copies bit for bit.
    """
    hq, hkv, d, dtype = 64, 8, 128, "bf16"
    reqs = wl.fifo_trace()
    L = PagedAttentionLayer(hq, hkv, d, 200_000, 2048, 128, dtype, 0, 0.15, page_shuffle_seed=5,
                            cache_fill=float("nan"))
    scale = wl.softmax_scale(d)
    pending = list(reqs)
    hist = {}
    step = 0
    rng = np.random.default_rng(55)
    worst = 0.0
    checked_rows = appended = 0
    frag = []

    def busy():
        st = L.builder.stats()
        return st["num_waiting"] + st["num_prefilling"] + st["num_decoding"] + st["num_finished_pending"] > 0

    while pending or busy():
        while pending and pending[0].arrival_step <= step:
            r = pending.pop(0)
            L.builder.submit(r.req_id, r.prompt_len, r.output_len)
            hist[r.req_id] = np.zeros((2, r.prompt_len + r.output_len - 1, hkv, d), np.uint16)
        desc = L.schedule()
        for f in desc.finished_ids.tolist():
            del hist[f]
        if desc.num_tokens == 0:
            step += 1
            continue
        T = desc.num_tokens
        kn = wl.device_normal((T, hkv, d), dtype, dev(), 5, step, 1)
        vn = wl.device_normal((T, hkv, d), dtype, dev(), 5, step, 2)
        qd = wl.device_normal((T, hq, d), dtype, dev(), 5, step, 3)
        out = L.attend(qd, kn, vn)
        torch.cuda.synchronize()
        kh = kn.view(torch.int16).cpu().numpy().view(np.uint16)
        vh = vn.view(torch.int16).cpu().numpy().view(np.uint16)
        for s in range(desc.num_seqs):
            i = int(desc.req_ids[s])
            a, e = desc.query_start_loc[s], desc.query_start_loc[s + 1]
            hist[i][0, desc.q_offsets[s]:desc.context_lens[s]] = kh[a:e]
            hist[i][1, desc.q_offsets[s]:desc.context_lens[s]] = vh[a:e]

        # the append: every slot written holds its token's bits
        slots = desc.slot_mapping.astype(np.int64)
        pages = np.unique(slots // 16)
        kp, vp = _pages_of(L.k_cache, pages), _pages_of(L.v_cache, pages)
        local = np.searchsorted(pages, slots // 16) * 16 + slots % 16
        ke, ve = kp.copy(), vp.copy()
        paging.append(ke, ve, kh, vh, local)
        assert np.array_equal(ke, kp) and np.array_equal(ve, vp), f"trace step {step}: appended slots differ"
        appended += T

        # sampled rows, every query head
        picks = []
        if desc.num_decodes:
            picks.append((int(rng.integers(0, desc.num_decodes)), [0]))
        if desc.num_seqs > desc.num_decodes:
            s = int(rng.integers(desc.num_decodes, desc.num_seqs))
            n = int(desc.q_lens[s])
            picks.append((s, sorted({0, n - 1} | set(rng.integers(0, n, size=3).tolist()))))
        if picks:
            qh = qd.float().cpu().numpy()
            out_h = out.float().cpu().numpy()
        for s, rows in picks:
            i = int(desc.req_ids[s])
            a, ctx = int(desc.query_start_loc[s]), int(desc.context_lens[s])
            n = int(desc.q_lens[s])
            # the sequence's history through its block table == the host copy
            row = desc.block_tables[s][: -(-ctx // 16)].astype(np.int64)
            kq, vq = _pages_of(L.k_cache, row), _pages_of(L.v_cache, row)
            kg, vg = paging.gather(kq, vq, np.arange(len(row)), ctx)
            assert np.array_equal(kg, hist[i][0, :ctx]) and np.array_equal(vg, hist[i][1, :ctx]), \
                f"trace step {step} seq {s}: paged history differs"
            k, v = _bf16_bits_to_f32(hist[i][0, :ctx]), _bf16_bits_to_f32(hist[i][1, :ctx])
            for ii in rows:
                pos = ctx - n + ii
                qr = qh[a + ii:a + ii + 1]
                ref = ora.attend(qr, k[:pos + 1], v[:pos + 1], scale)
                am = ora.attend(qr, k[:pos + 1], np.abs(v[:pos + 1]), scale)
                worst = max(worst, compare(out_h[a + ii:a + ii + 1], ref, dtype,
                                           f"trace step {step} seq {s} row {ii}", am))
            checked_rows += len(rows)
        st = L.builder.stats()
        if st["allocated_slots"]:
            frag.append(st["fragmentation"])
        if step % 200 == 0:
            say(f"  trace step {step}: T={T} decodes={desc.num_decodes} seqs={desc.num_seqs} worst={worst:.2e}")
        step += 1
        assert step < 5000
    say(f"  trace done: {step} steps, {appended} appended tokens read back, {checked_rows} rows x {hq} heads "
        f"checked, mean fragmentation {np.mean(frag):.4f}")
    assert L.builder.stats()["total_finished"] == len(reqs)
    n = L.stats()["cu_split_steps"]
    say(f"  {n} of {step} steps split by CU")
    assert 0 < n < step
