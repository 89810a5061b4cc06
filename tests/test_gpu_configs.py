"""The five workloads at full size, through the whole step (C++ builder ->
metadata upload -> cb_kv_append -> cb_attention_step), against the oracle.

Decode rows are checked for every sequence; prefill chunks are checked on
sampled query rows (first, last and seeded random rows, every head), which
the oracle computes one by one.  The FIFO trace checks sampled rows of every
one of its steps.
"""
import math

import numpy as np
import pytest
import torch

from gpu_util import compare, dev, say
from oracle import attention as ora
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
                self.layer.write_positions(self.layer.builder.block_table(i), 0, c, self._dev(k[:c]),
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


def test_long_prompt_forty_steps():
    say("long prompt: 127 decodes + 20000-token prompt in 512-token chunks, 64q/8kv, D128, bf16")
    r = Run(wl.long_prompt())
    for k in range(40):
        desc, q, out = r.step()
        pf = desc.q_lens[desc.num_decodes:]
        assert desc.num_decodes == 127 and pf.tolist() == ([512] if k < 39 else [32])
        if k in (0, 1, 19, 38, 39):
            say(f"  step {k}: chunk at {desc.q_offsets[-1]}, max abs err {r.check(desc, q, out, rng_seed=k):.2e}")
        else:
            assert np.isfinite(out).all()


@pytest.mark.timeout(900)
def test_fifo_trace_every_step():
    """256 requests, Poisson arrivals, lognormal prompts, geometric outputs, pool 200k pages.

    K, V and Q of each step are drawn on the device; the host keeps a copy of
    every request's K/V history for the oracle.  Every step is checked on
    sampled rows: one decode sequence and, when present, the first and last
    rows of one prefill chunk, each on the query heads of one seeded KV head.
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
    checked_rows = 0
    frag = []
    while pending or L.builder.stats()["num_waiting"] + L.builder.stats()["num_prefilling"] \
            + L.builder.stats()["num_decoding"] + L.builder.stats()["num_finished_pending"] > 0:
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
        kh = kn.view(torch.int16).cpu().numpy().view(np.uint16)
        vh = vn.view(torch.int16).cpu().numpy().view(np.uint16)
        for s in range(desc.num_seqs):
            i = int(desc.req_ids[s])
            a, e = desc.query_start_loc[s], desc.query_start_loc[s + 1]
            hist[i][0, desc.q_offsets[s]:desc.context_lens[s]] = kh[a:e]
            hist[i][1, desc.q_offsets[s]:desc.context_lens[s]] = vh[a:e]
        # sampled rows: one decode sequence, one prefill chunk (first and last rows)
        picks = []
        if desc.num_decodes:
            picks.append((int(rng.integers(0, desc.num_decodes)), [0]))
        if desc.num_seqs > desc.num_decodes:
            s = int(rng.integers(desc.num_decodes, desc.num_seqs))
            n = int(desc.q_lens[s])
            picks.append((s, sorted({0, n - 1})))
        qh = out_h = None
        for s, rows in picks:
            if qh is None:
                torch.cuda.synchronize()
                qh = qd.float().cpu().numpy()
                out_h = out.float().cpu().numpy()
            i = int(desc.req_ids[s])
            a, e, ctx = int(desc.query_start_loc[s]), int(desc.query_start_loc[s + 1]), int(desc.context_lens[s])
            # one KV head and its query-head group (a seeded choice per check)
            g = int(rng.integers(0, hkv))
            G = hq // hkv
            heads = slice(g * G, (g + 1) * G)
            k = torch.from_numpy(hist[i][0, :ctx, g:g + 1].view(np.int16)).view(torch.bfloat16).float().numpy()
            v = torch.from_numpy(hist[i][1, :ctx, g:g + 1].view(np.int16)).view(torch.bfloat16).float().numpy()
            pairs = [(ii, h) for ii in rows for h in range(G)]
            qg = qh[a:e][:, heads]
            ref = ora.attend_rows(qg, k, v, scale, rows=pairs)
            am = ora.attend_rows(qg, k, np.abs(v), scale, rows=pairs)
            worst = max(worst, compare(out_h[a:e][rows][:, heads], ref[rows], dtype,
                                       f"trace step {step} seq {s} kv head {g}", am[rows]))
            checked_rows += len(rows)
        st = L.builder.stats()
        if st["allocated_slots"]:
            frag.append(st["fragmentation"])
        if step % 200 == 0:
            say(f"  trace step {step}: T={T} decodes={desc.num_decodes} seqs={desc.num_seqs} worst={worst:.2e}")
        step += 1
        assert step < 5000
    say(f"  trace done: {step} steps, {checked_rows} rows checked, mean fragmentation {np.mean(frag):.4f}")
    assert L.builder.stats()["total_finished"] == len(reqs)
