"""Prefix block sharing through the whole engine step (builder -> upload ->
append -> attention) against the oracle.

Requests take prefixes of a few base prompts.  A request that reuses shared
blocks never writes their K/V; its rows must still equal the oracle computed
on its own full history, which the generator makes identical to what the
first owner wrote (K/V rows are keyed by the whole prompt prefix).  The cache
starts as NaN, so a block table pointing at a page nobody wrote shows up.
"""
import numpy as np
import pytest
import torch

from gpu_util import compare, dev, say
from oracle import attention as ora
from chunked_prefill_attention_amd.engine import PagedAttentionLayer
import workloads as wl

pytestmark = pytest.mark.gpu

HQ, HKV, D, DT = 8, 2, 128, "bf16"


def _run(policy, max_partial, seed):
    rng = np.random.default_rng(seed)
    layer = PagedAttentionLayer(HQ, HKV, D, 48, 96, 8, DT, 0, 0.0, page_shuffle_seed=seed,
                                cache_fill=float("nan"), policy=policy, max_partial_prefills=max_partial,
                                allow_block_sharing=True)
    base = [rng.integers(0, 30, n).tolist() for n in (70, 45, 100)]
    scale = wl.softmax_scale(D)
    hist, nid, hits, started_late, worst = {}, 0, 0, 0, 0.0

    def tdev(x):
        return torch.from_numpy(np.ascontiguousarray(x)).to(dev()).to(torch.bfloat16)

    for step in range(400):
        if nid < 14 and (step % 2 == 0):
            fam = base[int(rng.integers(0, 3))]
            n = int(rng.integers(17, len(fam) + 1))
            toks = fam[:n] + rng.integers(0, 30, int(rng.integers(0, 6))).tolist()
            out_len = int(rng.integers(2, 9))
            layer.builder.submit(nid, len(toks), out_len, tokens=toks)
            hist[nid] = wl.prompt_kv(seed, nid, toks, len(toks) + out_len - 1, HKV, D, DT)
            nid += 1
        desc = layer.schedule()
        if desc.num_seqs == 0:
            st = layer.builder.stats()
            if nid >= 14 and st["num_waiting"] + st["num_prefilling"] + st["num_decoding"] == 0:
                break
            continue
        ks, vs = [], []
        for s in range(desc.num_seqs):
            i, a, e = int(desc.req_ids[s]), int(desc.q_offsets[s]), int(desc.context_lens[s])
            ks.append(hist[i][0][a:e])
            vs.append(hist[i][1][a:e])
            if s >= desc.num_decodes and a > 0 and a % 16 == 0:
                started_late += 1
        q = wl.step_q(seed, step, desc.num_tokens, HQ, D, DT)
        out = layer.attend(tdev(q), tdev(np.concatenate(ks)), tdev(np.concatenate(vs)))
        torch.cuda.synchronize()
        out = out.float().cpu().numpy()
        hits += desc.prefix_hit_tokens
        for s in range(desc.num_seqs):
            i = int(desc.req_ids[s])
            a, e = int(desc.query_start_loc[s]), int(desc.query_start_loc[s + 1])
            ctx = int(desc.context_lens[s])
            k, v = hist[i][0][:ctx], hist[i][1][:ctx]
            ref = ora.attend(q[a:e], k, v, scale)
            am = ora.attend(q[a:e], k, np.abs(v), scale)
            worst = max(worst, compare(out[a:e], ref, DT, f"step {step} req {i}", am))
    st = layer.builder.stats()
    say(f"[sharing {policy}/{max_partial}] steps {step} hits {hits} late starts {started_late} "
        f"worst {worst:.3g} cached pages {st['cached_pages']}")
    assert hits > 0 and hits == st["prefix_hit_tokens"]
    assert started_late > 0
    assert st["num_prefilling"] == st["num_decoding"] == st["num_waiting"] == 0
    layer.close()


@pytest.mark.parametrize("policy,max_partial,seed", [("fifo", 0, 11), ("prefill_first", 2, 12)])
def test_prefix_sharing_engine_matches_oracle(policy, max_partial, seed):
    _run(policy, max_partial, seed)
