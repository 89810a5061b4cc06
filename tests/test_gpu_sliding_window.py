"""Sliding window through the whole engine step (builder -> upload -> append
-> attention) against the oracle.

The pool is small, so pages that fall below a request's window are released
and handed to other requests, which overwrite them.  Every row of every step
must still equal the windowed oracle on the request's own full history.
"""
import numpy as np
import pytest
import torch

from gpu_util import compare, dev, say
from oracle import attention as ora
from chunked_prefill_attention_amd.engine import PagedAttentionLayer
import workloads as wl

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("window,dtype,seed", [(64, "bf16", 21), (17, "bf16", 22), (200, "f32", 23)])
def test_sliding_window_engine_matches_oracle(window, dtype, seed):
    HQ, HKV, D = 8, 2, 128 if dtype == "bf16" else 64
    rng = np.random.default_rng(seed)
    layer = PagedAttentionLayer(HQ, HKV, D, 60, 128, 3, dtype, 64, 0.0, page_shuffle_seed=seed,
                                cache_fill=float("nan"), sliding_window=window)
    scale = wl.softmax_scale(D)
    tdt = layer.tdtype
    hist, nid, worst, reused = {}, 0, 0.0, 0
    seen_pages = {}

    def tdev(x):
        return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(dev()).to(tdt)

    for step in range(600):
        if nid < 10 and step % 3 == 0:
            p, o = int(rng.integers(100, 700)), int(rng.integers(5, 60))
            layer.builder.submit(nid, p, o)
            hist[nid] = wl.seq_kv(seed, nid, 0, p + o - 1, HKV, D, dtype)
            nid += 1
        desc = layer.schedule()
        if desc.num_seqs == 0:
            st = layer.builder.stats()
            if nid >= 10 and st["num_waiting"] + st["num_prefilling"] + st["num_decoding"] == 0:
                break
            continue
        ks, vs = [], []
        for s in range(desc.num_seqs):
            i, a, e = int(desc.req_ids[s]), int(desc.q_offsets[s]), int(desc.context_lens[s])
            ks.append(hist[i][0][a:e])
            vs.append(hist[i][1][a:e])
            for pg in desc.block_tables[s].tolist():       # pages seen under another request
                if pg >= 0:
                    if seen_pages.setdefault(pg, i) != i:
                        reused += 1
                        seen_pages[pg] = i
        q = wl.step_q(seed, step, desc.num_tokens, HQ, D, dtype)
        out = layer.attend(tdev(q), tdev(np.concatenate(ks)), tdev(np.concatenate(vs)))
        torch.cuda.synchronize()
        out = out.float().cpu().numpy()
        for s in range(desc.num_seqs):
            i = int(desc.req_ids[s])
            a, e = int(desc.query_start_loc[s]), int(desc.query_start_loc[s + 1])
            ctx = int(desc.context_lens[s])
            k, v = hist[i][0][:ctx], hist[i][1][:ctx]
            ref = ora.attend(q[a:e], k, v, scale, window=window)
            am = ora.attend(q[a:e], k, np.abs(v), scale, window=window) if dtype == "bf16" else None
            worst = max(worst, compare(out[a:e], ref, dtype, f"step {step} req {i}", am))
    st = layer.builder.stats()
    say(f"[window {window} {dtype}] steps {step} pages reused across requests {reused} worst {worst:.3g}")
    assert st["total_finished"] == 10 and reused > 0
    layer.close()
