"""cb_attention_step on the GPU against the fp64 oracle, element by element.

Small and medium steps that span several tiles and ragged tails, every edge
case of the method (one-token contexts, page-aligned and unaligned ends,
single-query prefill rows, decodes with many splits, empty sequences,
grouped-query sizes 1..16), bit-exact indexing probes, and invariances
(physical page permutation, determinism, NaN in unused slots).
"""
import zlib

import numpy as np
import pytest
import torch

from gpu_util import Step, compare, i32, new_cache, say, to_dev, write_history
from oracle import attention as ora
import chunked_prefill_attention_amd as cb
import workloads as wl

pytestmark = pytest.mark.gpu


def _check_all(st: Step, out, what, window=0):
    worst = 0.0
    for s, (c, n) in enumerate(st.seqs):
        if n == 0:
            continue
        ref = ora.attend(st.q[s], st.k_hist[s], st.v_hist[s], st.scale, window=window)
        am = ora.attend(st.q[s], st.k_hist[s], np.abs(st.v_hist[s]), st.scale,
                        window=window) if st.dtype == "bf16" else None
        worst = max(worst, compare(st.out_rows(out, s), ref, st.dtype, f"{what} seq {s} (ctx {c}, q {n})", am))
    return worst


CASES = {
    # name: (seqs [(ctx, q_len)], Hq, Hkv, D)
    "decode_gqa4": ([(1, 1), (15, 1), (16, 1), (17, 1), (255, 1), (256, 1), (257, 1), (1000, 1), (3000, 1)], 32, 8, 128),
    "decode_long_splits": ([(9000, 1), (4097, 1), (130, 1)] + [(2000 + 37 * i, 1) for i in range(40)], 16, 2, 128),
    "prefill_only_gqa4": ([(476 + 1024, 476), (700, 700), (808, 808)], 32, 8, 128),
    "mixed_small": ([(33, 1), (600, 1), (129, 1), (1500, 476), (70, 70), (1, 1), (300, 17)], 32, 8, 128),
    "mixed_d64_g1": ([(40, 1), (513, 1), (260, 130), (64, 64), (1000, 5)], 4, 4, 64),
    "mixed_g2": ([(100, 1), (2100, 1), (777, 250), (31, 31)], 8, 4, 128),
    "mixed_g8": ([(1100, 1), (5000, 1), (20000 - 19968 + 19968, 32), (1536, 512)], 64, 8, 128),
    "mixed_g16": ([(800, 1), (77, 1), (300, 45)], 16, 1, 128),
    "g3_odd": ([(90, 1), (500, 200)], 6, 2, 64),
    "qlen1_in_prefill_set": ([(500, 1), (20, 1), (1, 1)], 8, 2, 128),
    "empty_seq_in_prefill_set": ([(300, 1), (50, 0), (200, 60), (10, 0)], 8, 2, 128),
}


@pytest.mark.parametrize("name", sorted(CASES))
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_step_matches_oracle(name, dtype):
    seqs, hq, hkv, d = CASES[name]
    say(f"step {name} {dtype}")
    st = Step(seqs, hq, hkv, d, dtype, seed=zlib.crc32(name.encode()) % 1000)
    if name == "qlen1_in_prefill_set":
        st.num_decodes = 1            # later q_len == 1 rows go down the prefill path
    kc, vc = st.upload()
    out = st.run(kc, vc)
    worst = _check_all(st, out, name)
    say(f"  max abs err {worst:.2e}")


WINDOW_CASES = [("decode_gqa4", 1), ("decode_gqa4", 100), ("decode_long_splits", 1000),
                ("decode_long_splits", 16), ("prefill_only_gqa4", 100), ("prefill_only_gqa4", 1),
                ("mixed_small", 17), ("mixed_small", 300), ("mixed_d64_g1", 64), ("mixed_g8", 1000),
                ("mixed_g8", 130), ("g3_odd", 5), ("mixed_g16", 50), ("mixed_g2", 100000)]


@pytest.mark.parametrize("name,window", WINDOW_CASES)
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("holes", [False, True])
def test_sliding_window_matches_oracle(name, window, dtype, holes):
    """Row p sees keys p-W < j <= p.  Pages wholly below a sequence's first
    row's window are NaN-filled (and, with ``holes``, their block-table
    entries become -1, as the builder leaves them): they must not matter."""
    seqs, hq, hkv, d = CASES[name]
    say(f"window {name} W={window} {dtype} holes={holes}")
    st = Step(seqs, hq, hkv, d, dtype, seed=zlib.crc32(name.encode()) % 1000 + window)
    kc, vc = st.upload()
    bt = st.bt.copy()
    dropped = 0
    for s, (c, n) in enumerate(st.seqs):
        first_key = max(0, c - n - window + 1)
        for pg in range(first_key // 16):
            kc[int(st.bt[s, pg])] = float("nan")
            vc[int(st.bt[s, pg])] = float("nan")
            if holes:
                bt[s, pg] = -1
            dropped += 1
    q = to_dev(np.concatenate(st.q), dtype)
    out = cb.attention_step(q, kc, vc, i32(bt), i32(st.qsl), i32(st.ctx), i32(st.off), st.num_decodes,
                            st.max_ctx, st.scale, sliding_window=window)
    torch.cuda.synchronize()
    worst = _check_all(st, out, f"window {window}", window=window)
    say(f"  {dropped} pages below the windows; max abs err {worst:.2e}")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_peaky_scores(dtype):
    """Large-magnitude queries concentrate the softmax; outputs are O(1)."""
    st = Step([(700, 1), (2500, 1), (900, 300)], 32, 8, 128, dtype, seed=11, q_std=4.0)
    kc, vc = st.upload()
    _check_all(st, st.run(kc, vc), "peaky")


def test_page_example_through_builder_f32():
    """The pages' worked example as four engine steps (fp32, 8 heads x 64, budget 256).

    Each step: builder -> kv_append of the chunk -> attention over the pages.
    The concatenated outputs must equal one-shot causal attention (the oracle).
    """
    w = wl.page_example()
    q, k, v = wl.page_example_tensors()
    b = cb.Builder(w.max_batch_tokens, w.max_requests, w.pool_pages + 7, page_shuffle_seed=12345)
    b.submit(0, 1000, 1)
    kc, vc = new_cache(w.pool_pages + 7, 8, 64, "f32")   # 7 spare pages stay NaN
    outs, sizes = [], []
    while True:
        s = b.step()
        if s.num_seqs == 0:
            break
        a, e = int(s.q_offsets[0]), int(s.context_lens[0])
        sizes.append(e - a)
        cb.kv_append(to_dev(k[a:e], "f32"), to_dev(v[a:e], "f32"), kc, vc, i32(s.slot_mapping))
        o = cb.attention_step(to_dev(q[a:e], "f32"), kc, vc, i32(s.block_tables), i32(s.query_start_loc),
                              i32(s.context_lens), i32(s.q_offsets), s.num_decodes, s.max_context_len,
                              wl.softmax_scale(64))
        outs.append(o.cpu().numpy())
    assert sizes == [256, 256, 256, 232]
    got = np.concatenate(outs)
    ref = ora.attend(q, k, v, wl.softmax_scale(64))
    compare(got, ref, "f32", "page example")


def test_one_hot_probe_is_bit_exact():
    """A dominant key at position j makes every row that sees it return V[j] exactly."""
    d, hkv, hq = 128, 2, 8
    ctx_list = [1, 16, 17, 100, 255, 4100]
    for j_frac in (0.0, 0.37, 0.999):
        seqs = [(c, 1) for c in ctx_list] + [(700, 300)]
        st = Step(seqs, hq, hkv, d, "bf16", seed=3)
        for s, (c, n) in enumerate(st.seqs):
            j = min(int(j_frac * c), c - n)      # visible to every query of the sequence
            st.k_hist[s][:] = 0.0
            st.k_hist[s][j, :, 0] = 16.0
            st.q[s][:] = 0.0
            st.q[s][:, :, 0] = 128.0              # score gap 2048*scale ~ 181 (log2 units ~ 261)
        kc, vc = st.upload()
        out = st.run(kc, vc)
        for s, (c, n) in enumerate(st.seqs):
            j = min(int(j_frac * c), c - n)
            got = st.out_rows(out, s)
            for h in range(hq):
                want = np.broadcast_to(st.v_hist[s][j, h // (hq // hkv)], got[:, h].shape)
                assert np.array_equal(got[:, h], want), (s, c, j, h)


def test_physical_permutation_and_determinism_bitwise():
    st = Step([(3000, 1), (517, 1), (64, 1), (1500, 476), (700, 700)], 32, 8, 128, "bf16", seed=5)
    kc, vc = st.upload()
    o1 = st.run(kc, vc).clone()
    o2 = st.run(kc, vc).clone()
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))
    alt = st.permuted_table(99)
    kc2, vc2 = st.upload(table=alt)
    o3 = st.run(kc2, vc2, table=alt)
    assert torch.equal(o1.view(torch.int16), o3.view(torch.int16))


def test_chunk_size_invariance_bf16():
    """One prompt prefilled in different chunkings matches the oracle each time."""
    hq, hkv, d, n = 32, 8, 128, 1100
    k, v = wl.seq_kv(21, 0, 0, n, hkv, d, "bf16")
    q = wl.seq_q(21, 0, 0, n, hq, d, "bf16")
    ref = ora.attend(q, k, v, wl.softmax_scale(d))
    am = ora.attend(q, k, np.abs(v), wl.softmax_scale(d))
    for chunk in (1100, 512, 256, 100, 17):
        pages = -(-n // 16) + 5
        row = wl.permutation(chunk, pages)[: -(-n // 16)].astype(np.int32)
        kc, vc = new_cache(pages, hkv, d, "bf16")
        outs = []
        for a in range(0, n, chunk):
            e = min(a + chunk, n)
            write_history(kc, vc, k, v, row, a, e, "bf16")
            o = cb.attention_step(to_dev(q[a:e], "bf16"), kc, vc, i32(row[None]), i32([0, e - a]), i32([e]),
                                  i32([a]), 0, e, wl.softmax_scale(d))
            outs.append(o.float().cpu().numpy())
        compare(np.concatenate(outs), ref, "bf16", f"chunk {chunk}", am)


@pytest.mark.parametrize("d", [64, 128])
def test_nan_in_unused_slots_does_not_leak(d):
    """Garbage (NaN) in partial-page tails and in unreferenced pages is masked
    (prefill: the V tokens of the tile that holds the context end are zeroed
    as they are read from LDS)."""
    st = Step([(17, 1), (33, 1), (4097, 1), (45, 13), (129, 129), (300, 77)], 16, 4, d, "bf16", seed=8,
              fill=float("nan"))
    kc, vc = st.upload()
    out = st.run(kc, vc)
    assert torch.isfinite(out.float()).all()
    _check_all(st, out, "nan tails")


@pytest.mark.parametrize("d", [64, 128])
def test_nan_tails_decode_only(d):
    """A decode-only step (the decode-only launch, its splits and the
    combine): NaN in partial-page tails and in unreferenced pages stays
    masked, also for sequences of one to three pages."""
    st = Step([(17, 1), (33, 1), (4097, 1), (1, 1), (48, 1), (49, 1), (2000, 1)], 16, 4, d, "bf16", seed=9,
              fill=float("nan"))
    kc, vc = st.upload()
    out = st.run(kc, vc)
    assert torch.isfinite(out.float()).all()
    _check_all(st, out, "nan tails decode-only")


@pytest.mark.parametrize("with_prefill", [False, True])
def test_long_decode_splits_match_oracle(with_prefill):
    """256 decode sequences, two of them long (1,025 and 1,000 pages): with
    2,048 (sequence, KV head) lanes the planner picks 128-page decode splits
    in the decode-only launch (full splits plus a short last one of 1 and 104
    pages) and 64-page splits beside a prefill chunk (last ones of 1 and 40
    pages), listed by the device plan kernel of a direct call."""
    seqs = [(16400, 1), (16000, 1)] + [(17 + 13 * i, 1) for i in range(254)]
    if with_prefill:
        seqs.append((300, 77))
    st = Step(seqs, 32, 8, 128, "bf16", seed=21)
    kc, vc = st.upload()
    out = st.run(kc, vc)
    _check_all(st, out, "long decode splits")


@pytest.mark.parametrize("d,window", [(64, 0), (128, 9000), (64, 2500)])
def test_long_decode_splits_d64_and_window(d, window):
    """128-page decode splits at D 64 and under a sliding window (a split's
    pages then start at the window's first page, and the second page-id
    register holds pages 64..127 of the split)."""
    seqs = [(16400, 1), (16000, 1)] + [(17 + 13 * i, 1) for i in range(254)]
    st = Step(seqs, 16, 8, d, "bf16", seed=22 + d + window)
    kc, vc = st.upload()
    q = to_dev(np.concatenate(st.q), "bf16")
    out = cb.attention_step(q, kc, vc, i32(st.bt), i32(st.qsl), i32(st.ctx), i32(st.off), st.num_decodes,
                            st.max_ctx, st.scale, sliding_window=window)
    torch.cuda.synchronize()
    _check_all(st, out, f"long splits d{d} w{window}", window=window)



@pytest.mark.parametrize("dtype,d,hq,hkv,window", [("bf16", 128, 16, 2, 0), ("f32", 128, 16, 2, 0),
                                                   ("bf16", 64, 4, 4, 0), ("bf16", 128, 16, 2, 5000)])
def test_very_long_contexts_match_oracle(dtype, d, hq, hkv, window):
    """Contexts far past the other cases: decodes over 200,000 and 150,001
    keys (12,500 and 9,376 pages, cut into 196 and 147 splits for the
    combine to merge) and a 64-token chunk at offset 131,072 (its GQA-packed
    rows in row tiles each cut into ~100 key ranges); at D 128 with eight
    query heads per KV head, at D 64 with one, and under a 5,000-token
    sliding window (the splits then cover only the window's pages).  Every
    head of every decode row and of the chunk's first, second, middle and
    last rows against the row-by-row oracle.  Queries are drawn with std 4,
    so that a few keys anywhere in the context carry most of a row's weight
    (the heaviest 1,024-key stretch of a decode row holds ~0.3 of it): a
    dropped, repeated or misplaced split moves the output well past the
    tolerance."""
    seqs = [(200_000, 1), (150_001, 1), (131_072 + 64, 64)]
    say(f"very long contexts {dtype} d{d} {hq}/{hkv} window {window}")
    st = Step(seqs, hq, hkv, d, dtype, seed=31 + d + window, q_std=4.0)
    kc, vc = st.upload()
    q = to_dev(np.concatenate(st.q), dtype)
    out = cb.attention_step(q, kc, vc, i32(st.bt), i32(st.qsl), i32(st.ctx), i32(st.off), st.num_decodes,
                            st.max_ctx, st.scale, sliding_window=window)
    torch.cuda.synchronize()
    for s, (c, n) in enumerate(seqs):
        rows = [(i, h) for i in sorted({0, min(1, n - 1), n // 2, n - 1}) for h in range(hq)]
        ii = [i for i, _ in rows]
        hh = [h for _, h in rows]
        ref = ora.attend_rows(st.q[s], st.k_hist[s], st.v_hist[s], st.scale, rows=rows, window=window)[ii, hh]
        am = ora.attend_rows(st.q[s], st.k_hist[s], np.abs(st.v_hist[s]), st.scale, rows=rows,
                             window=window)[ii, hh] if dtype == "bf16" else None
        err = compare(st.out_rows(out, s)[ii, hh], ref, dtype, f"seq {s} (ctx {c}, q {n})", am)
        say(f"  seq {s}: ctx {c}, {len(rows)} rows, max abs err {err:.2e}")

def test_bad_page_ids_do_not_fault():
    """Out-of-range block-table entries (a broken precondition) must not fault:
    they read page 0, so with finite cache contents the output stays finite."""
    st = Step([(40, 1), (60, 20)], 8, 2, 128, "bf16", seed=9, fill=0.0)
    kc, vc = st.upload()
    bad = st.bt.copy()
    bad[:, 1] = st.num_pages + 1000
    out = st.run(kc, vc, table=bad)
    assert torch.isfinite(out.float()).all()


def test_engine_page_example_with_buffer_growth():
    """The pages' example through the native engine (schedule + attend), with
    metadata slots sized to force one CB_ERR_CAPACITY regrowth and a workspace
    grown on first use."""
    from chunked_prefill_attention_amd.engine import PagedAttentionLayer
    q, k, v = wl.page_example_tensors()
    layer = PagedAttentionLayer(8, 8, 64, 70, 256, 128, "f32", page_shuffle_seed=3, cache_fill=float("nan"),
                                meta_pages_per_request=0)
    layer.builder.submit(0, 1000, 1)
    outs = []
    while True:
        d = layer.schedule()
        if d.num_tokens == 0:
            break
        a, e = int(d.q_offsets[0]), int(d.context_lens[0])
        outs.append(layer.attend(to_dev(q[a:e], "f32"), to_dev(k[a:e], "f32"), to_dev(v[a:e], "f32")).cpu().numpy())
    compare(np.concatenate(outs), ora.attend(q, k, v, wl.softmax_scale(64)), "f32", "engine page example")


def test_engine_mixed_bf16_matches_direct_calls_bitwise():
    """Engine step == builder + cb_kv_append + cb_attention_step called directly."""
    from chunked_prefill_attention_amd.engine import PagedAttentionLayer
    hq, hkv, d = 32, 8, 128
    reqs = [(900, 5, 899), (300, 5, 299), (1500, 5, 1024), (700, 5, 0)]
    layer = PagedAttentionLayer(hq, hkv, d, 400, 600, 16, "bf16", page_shuffle_seed=9)
    ref_b = cb.Builder(600, 16, 400, page_shuffle_seed=9)
    kc2, vc2 = new_cache(400, hkv, d, "bf16", 0.0)
    hist = {}
    for i, (p, o, c) in enumerate(reqs):
        layer.builder.submit(i, p, o, c)
        ref_b.submit(i, p, o, c)
        k, v = wl.seq_kv(31, i, 0, p + o, hkv, d, "bf16")
        hist[i] = (k, v)
        if c:
            layer.write_positions(i, 0, c, to_dev(k[:c], "bf16"), to_dev(v[:c], "bf16"))
            write_history(kc2, vc2, k, v, ref_b.block_table(i), 0, c, "bf16")
    for step in range(3):
        dsc = layer.schedule().copy()
        rs = ref_b.step()
        assert rs.req_ids.tolist() == dsc.req_ids.tolist() and np.array_equal(rs.block_tables, dsc.block_tables)
        kn = np.concatenate([hist[int(r)][0][a:e] for r, a, e in zip(dsc.req_ids, dsc.q_offsets, dsc.context_lens)])
        vn = np.concatenate([hist[int(r)][1][a:e] for r, a, e in zip(dsc.req_ids, dsc.q_offsets, dsc.context_lens)])
        qq = wl.step_q(31, step, dsc.num_tokens, hq, d, "bf16")
        o1 = layer.attend(to_dev(qq, "bf16"), to_dev(kn, "bf16"), to_dev(vn, "bf16"))
        cb.kv_append(to_dev(kn, "bf16"), to_dev(vn, "bf16"), kc2, vc2, i32(rs.slot_mapping))
        o2 = cb.attention_step(to_dev(qq, "bf16"), kc2, vc2, i32(rs.block_tables), i32(rs.query_start_loc),
                               i32(rs.context_lens), i32(rs.q_offsets), rs.num_decodes, rs.max_context_len,
                               wl.softmax_scale(d))
        torch.cuda.synchronize()
        assert torch.equal(o1.view(torch.int16), o2.view(torch.int16)), step
    # the chunks dominate these steps: the engine ran them split by CU, the
    # direct calls in block order, with the same bits
    assert layer.stats()["cu_split_steps"] > 0


def test_interleaved_block_order_matches_oracle():
    """More live prefill workgroups than the device holds at once, beside
    decodes: the mixed launch alternates prefill and decode blocks.  The work
    lists' header (at the front of the workspace) records the order used."""
    seqs = [(300 + 97 * i, 1) for i in range(8)] + [(8048, 2048)]
    hq, hkv, d = 32, 8, 128
    say("interleaved block order: 8 decodes + 2048 tokens at offset 6000")
    st = Step(seqs, hq, hkv, d, "bf16", seed=11)
    kc, vc = st.upload()
    ws = torch.empty(cb.attention_workspace_bytes(len(seqs), st.num_decodes, st.T, hq, hkv, d, st.max_ctx, 1),
                     dtype=torch.uint8, device=kc.device)
    q = to_dev(np.concatenate(st.q), "bf16")
    out = cb.attention_step(q, kc, vc, i32(st.bt), i32(st.qsl), i32(st.ctx), i32(st.off), st.num_decodes,
                            st.max_ctx, st.scale, workspace=ws)
    torch.cuda.synchronize()
    live_pf, live_dec, order = (int(x) for x in ws[:16].view(torch.int32).cpu()[:3])
    assert live_dec > 0 and live_pf * hkv > 512 and order == 1, (live_pf, live_dec, order)
    worst = 0.0
    for s in range(st.num_decodes):
        ref = ora.attend(st.q[s], st.k_hist[s], st.v_hist[s], st.scale)
        worst = max(worst, compare(st.out_rows(out, s), ref, "bf16", f"decode {s}"))
    s = len(seqs) - 1
    pick = sorted(set([0, 1, 1023, 2046, 2047] + wl.uniform_ints(5, 8, 0, 2047).tolist()))
    rows = [(i, h) for i in pick for h in range(hq)]
    ref = ora.attend_rows(st.q[s], st.k_hist[s], st.v_hist[s], st.scale, rows=rows)
    am = ora.attend_rows(st.q[s], st.k_hist[s], np.abs(st.v_hist[s]), st.scale, rows=rows)
    worst = max(worst, compare(st.out_rows(out, s)[pick], ref[pick], "bf16", "prefill rows", am[pick]))
    say(f"  live prefill items {live_pf}, decode items {live_dec}; max abs err {worst:.2e}")
