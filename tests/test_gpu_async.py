"""Async stepping through the native engine, checked against the oracle.

Hugging Face transformers, "Continuous batching architecture", "Async
batching": the host prepares step N+1 while the device computes step N.  The
engine keeps two pinned staging slots; scheduling step N+2 reuses step N's
slot and waits (on the host) only if step N's upload -- done by its append
kernel -- has not run yet.  Here ten distinct steps are enqueued back to back
behind a device backlog (after one warm-up step), with no host synchronisation
between them, each into
its own output buffer; the engine must report that a schedule waited for a
slot, and every step's output is then compared with the oracle.  The same
runs with graph replay ([CBA] "CUDA graphs"): padded step shapes recorded
and replayed on the layer's stream while earlier steps are still pending.
"""
import time

import numpy as np
import pytest
import torch

import chunked_prefill_attention_amd as cb
from gpu_util import compare, dev, say
from oracle import attention as ora
from chunked_prefill_attention_amd.engine import PagedAttentionLayer
import workloads as wl

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("graphs", [(0, 0), (64, 1024)], ids=["direct", "graphs"])
def test_overlapped_engine_steps_match_the_oracle(graphs):
    hq, hkv, d, seed = 32, 8, 128, 41
    budget, max_req = 640, 64
    # 24 decodes (contexts 1,500 .. 4,000) and two prompts of 1,500 and 2,600
    # tokens chunked under the budget: every step differs (chunks advance,
    # decode contexts grow by one)
    ctx = wl.uniform_ints(seed, 24, 1500, 4000)
    reqs = [(int(c) - 1, 40, int(c) - 1) for c in ctx] + [(1500, 4, 0), (2600, 4, 0)]
    pool = sum(-(-(p + o) // 16) for p, o, _ in reqs) + 64
    L = PagedAttentionLayer(hq, hkv, d, pool, budget, max_req, "bf16", page_shuffle_seed=seed,
                            cache_fill=float("nan"), graph_q_interval=graphs[0], graph_kv_interval=graphs[1])
    hist = {}
    for i, (p, o, c) in enumerate(reqs):
        L.builder.submit(i, p, o, c)
        n = p + o - 1
        hist[i] = (wl.device_normal((n, hkv, d), "bf16", dev(), seed, i, 1),
                   wl.device_normal((n, hkv, d), "bf16", dev(), seed, i, 2))
        if c > 0:
            L.write_positions(i, 0, c, hist[i][0][:c], hist[i][1][:c])
    max_ctx = max(p + o for p, o, _ in reqs)
    L.reserve_workspace(max(cb.attention_workspace_bytes(max_req, nd, budget, hq, hkv, d, max_ctx, cb.CB_BF16)
                            for nd in range(max_req + 1)))
    torch.cuda.synchronize()

    def enqueue(s):
        desc = L.schedule().copy()
        rows = list(zip(desc.req_ids.tolist(), desc.q_offsets.tolist(), desc.context_lens.tolist()))
        kn = torch.cat([hist[r][0][a:e] for r, a, e in rows])
        vn = torch.cat([hist[r][1][a:e] for r, a, e in rows])
        q = wl.device_normal((desc.num_tokens, hq, d), "bf16", dev(), seed, 1000 + s, 3)
        out = torch.empty_like(q)
        L.attend(q, kn, vn, out=out)
        return desc, q, out

    # one step first, synchronised: every kernel and library routine the loop
    # uses has been loaded and run once before the overlapped steps
    runs = [enqueue(0)]
    torch.cuda.synchronize()
    # a backlog on the stream (about 20 ms of writes): the host enqueues the
    # next steps long before the device reaches them
    scratch = torch.empty(1 << 30, dtype=torch.uint8, device=dev())
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    ev[0].record()
    for r in range(100):
        scratch.fill_(r)
    ev[1].record()
    n_steps = 10
    trail = []
    t0 = time.perf_counter()
    for s in range(1, n_steps + 1):
        runs.append(enqueue(s))
        trail.append((round((time.perf_counter() - t0) * 1e3, 2), L.stats()["slot_waits"]))
    stats = L.stats()               # read before any synchronisation
    torch.cuda.synchronize()
    say(f"  host ms and slot waits after each overlapped step: {trail}")
    say(f"  engine stats: {stats}; backlog {ev[0].elapsed_time(ev[1]):.1f} ms on the device; "
        f"all drained {1e3 * (time.perf_counter() - t0):.1f} ms after the first enqueue")
    assert stats["steps_attended"] == n_steps + 1
    assert stats["slot_waits"] >= 1, "no schedule had to wait: the steps did not overlap"
    if graphs[0]:
        assert stats["graph_replays"] == n_steps + 1 and stats["graph_captures"] >= 1

    scale = wl.softmax_scale(d)
    host = {i: (k.float().cpu().numpy(), v.float().cpu().numpy()) for i, (k, v) in hist.items()}
    shapes = set()
    for s, (desc, q, out) in enumerate(runs):
        qh, oh = q.float().cpu().numpy(), out.float().cpu().numpy()
        shapes.add((tuple(desc.q_lens.tolist()), tuple(desc.context_lens.tolist())))
        worst = 0.0
        for j in range(desc.num_seqs):
            i = int(desc.req_ids[j])
            a, e, c = int(desc.query_start_loc[j]), int(desc.query_start_loc[j + 1]), int(desc.context_lens[j])
            k, v = host[i][0][:c], host[i][1][:c]
            ref = ora.attend(qh[a:e], k, v, scale)
            am = ora.attend(qh[a:e], k, np.abs(v), scale)
            worst = max(worst, compare(oh[a:e], ref, "bf16", f"step {s} seq {j}", am))
        say(f"  step {s}: {desc.num_decodes} decodes + chunks {desc.q_lens[desc.num_decodes:].tolist()}, "
            f"max abs err {worst:.2e}")
    assert len(shapes) == n_steps + 1        # eleven distinct steps (chunks and contexts)
