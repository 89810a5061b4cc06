"""Graph replay: padded step shapes recorded once into HIP graphs and replayed.

Two engines with the same configuration run the same trace in lockstep: one
launches each padded step directly, the other records a graph per padded
shape and replays it.  Every step must agree bit for bit (same kernels, same
arguments), and with the oracle within the stated tolerance.  Eager work runs
on the graph stream between steps, and one step is replayed several times
from the same starting state.
"""
import numpy as np
import pytest
import torch

from gpu_util import compare, dev, say
from oracle import attention as ora
from chunked_prefill_attention_amd.engine import PagedAttentionLayer
import workloads as wl

pytestmark = pytest.mark.gpu


def _layer(hq, hkv, d, dtype, seed, capture):
    return PagedAttentionLayer(hq, hkv, d, 400, 256, 16, dtype, 0, 0.0, page_shuffle_seed=seed,
                               cache_fill=float("nan"), graph_q_interval=64, graph_kv_interval=256,
                               graph_capture=capture)


def _inputs(layer, desc, hist, seed, step, hq, d, dtype):
    ks = np.concatenate([hist[int(r)][0][a:e] for r, a, e in zip(desc.req_ids, desc.q_offsets, desc.context_lens)])
    vs = np.concatenate([hist[int(r)][1][a:e] for r, a, e in zip(desc.req_ids, desc.q_offsets, desc.context_lens)])
    q = wl.step_q(seed, step, desc.num_tokens, hq, d, dtype)

    def t(x):
        return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(dev()).to(layer.tdtype)
    return q, t(q), t(ks), t(vs)


@pytest.mark.parametrize("dtype,d", [("bf16", 128), ("f32", 64)])
def test_graph_replay_matches_direct_padded_steps_bitwise(dtype, d):
    hq, hkv, seed = 8, 2, 31
    rng = np.random.default_rng(seed)
    direct, graph = _layer(hq, hkv, d, dtype, seed, False), _layer(hq, hkv, d, dtype, seed, True)
    scale = wl.softmax_scale(d)
    hist, nid, worst = {}, 0, 0.0
    noise = torch.randn((512, 512), device=dev())
    for step in range(200):
        if nid < 24 and step % 2 == 0:
            p, o = int(rng.integers(30, 400)), int(rng.integers(5, 40))
            for L in (direct, graph):
                L.builder.submit(nid, p, o)
            hist[nid] = wl.seq_kv(seed, nid, 0, p + o - 1, hkv, d, dtype)
            nid += 1
        da, db = direct.schedule(), graph.schedule()
        assert np.array_equal(da.req_ids, db.req_ids) and np.array_equal(da.query_start_loc, db.query_start_loc)
        if da.num_tokens == 0:
            if nid >= 24 and graph.builder.stats()["num_decoding"] + graph.builder.stats()["num_prefilling"] \
                    + graph.builder.stats()["num_waiting"] == 0:
                break
            continue
        q, qt, kt, vt = _inputs(graph, db, hist, seed, step, hq, d, dtype)
        oa = direct.attend(qt, kt, vt).float().cpu().numpy()
        with torch.cuda.stream(graph.graph_stream):      # eager work between replays
            noise = torch.tanh(noise @ noise.T * 1e-3)
        ob = graph.attend(qt, kt, vt).float().cpu().numpy()
        torch.cuda.synchronize()
        assert np.array_equal(oa, ob), f"step {step}: replay differs from the direct launch"
        for s in range(db.num_seqs):
            i = int(db.req_ids[s])
            a, e, ctx = int(db.query_start_loc[s]), int(db.query_start_loc[s + 1]), int(db.context_lens[s])
            ref = ora.attend(q[a:e], hist[i][0][:ctx], hist[i][1][:ctx], scale)
            am = ora.attend(q[a:e], hist[i][0][:ctx], np.abs(hist[i][1][:ctx]), scale) if dtype == "bf16" else None
            worst = max(worst, compare(ob[a:e], ref, dtype, f"step {step} req {i}", am))
    gs = graph.graph_stats()
    say(f"[graphs {dtype}] steps {step}: {gs}; worst {worst:.3g}")
    assert gs["replays"] > gs["captures"] > 0
    assert direct.graph_stats()["captures"] == 0


def test_same_step_replayed_repeatedly_is_identical():
    hq, hkv, d, dtype, seed = 8, 2, 128, "bf16", 32
    layer = _layer(hq, hkv, d, dtype, seed, True)
    hist = {}
    for i, (p, o) in enumerate([(300, 20), (90, 20), (1000, 20), (17, 20)]):
        layer.builder.submit(i, p, o)
        hist[i] = wl.seq_kv(seed, i, 0, p + o - 1, hkv, d, dtype)
    for step in range(5):                      # prefills done, decodes running
        desc = layer.schedule()
        _, qt, kt, vt = _inputs(layer, desc, hist, seed, step, hq, d, dtype)
        layer.attend(qt, kt, vt)
    snap = layer.builder.clone()
    outs = []
    for rep in range(4):
        layer.load_builder(snap)
        desc = layer.schedule()
        _, qt, kt, vt = _inputs(layer, desc, hist, seed, 99, hq, d, dtype)
        outs.append(layer.attend(qt, kt, vt).float().cpu().numpy())
        torch.cuda.synchronize()
        x = torch.randn(1 << 20, device=dev()).sum().item()    # eager work and a sync between
        assert np.isfinite(x)
    assert all(np.array_equal(outs[0], o) for o in outs[1:])
    gs = layer.graph_stats()
    assert gs["replays"] >= 4
