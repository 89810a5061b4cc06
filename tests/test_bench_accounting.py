"""bench.py's algorithmic work per step (the numerator of every roofline
fraction) against brute-force counts and the workloads' stated figures.

A step's flops are 4·D·Hq per visible (query row, key) pair (QKᵀ and P·V,
2·D each); its bytes are the KV history read once per sequence and KV head,
q read, out written, and the step's tables.
"""
import types

import numpy as np
import pytest

import bench


def _desc(seqs):
    """A step descriptor with (context_len, q_len) per sequence."""
    ctx = np.array([c for c, _ in seqs], dtype=np.int32)
    ql = np.array([n for _, n in seqs], dtype=np.int32)
    return types.SimpleNamespace(context_lens=ctx, q_lens=ql, num_tokens=int(ql.sum()), num_seqs=len(seqs))


def _brute_pairs(seqs, window=0):
    n = 0
    for c, q in seqs:
        off = c - q
        for i in range(q):
            p = off + i
            n += sum(1 for j in range(c) if j <= p and (window <= 0 or j > p - window))
    return n


@pytest.mark.parametrize("window", [0, 1, 5, 40])
def test_pairs_and_flops_match_brute_force(window):
    seqs = [(1, 1), (17, 1), (90, 33), (64, 64), (130, 7), (5, 0)]
    hq, hkv, d = 8, 2, 64
    nbytes, flops, pairs = bench.algorithmic(_desc(seqs), hq, hkv, d, 2, window)[:3]
    assert pairs == _brute_pairs(seqs, window)
    assert flops == 4 * d * hq * pairs


@pytest.mark.parametrize("window", [0, 3, 50])
def test_bytes_match_their_definition(window):
    seqs = [(1, 1), (17, 1), (90, 33), (64, 64), (130, 7)]
    hq, hkv, d, e = 8, 2, 64, 2
    nbytes, _, _ = bench.algorithmic(_desc(seqs), hq, hkv, d, e, window)[:3]
    kv = meta = 0
    for c, q in seqs:
        off = c - q
        # the first key any row of the sequence sees (the first row's window start)
        first = min(max(0, off + i - window + 1) if window > 0 else 0 for i in range(q))
        kv += (c - first) * 2 * hkv * d * e
        meta += (-(-c // 16) - first // 16) * 4        # the block-table entries read
    meta += (3 * len(seqs) + 1) * 4                     # query_start_loc, context_lens, q_offsets
    qo = 2 * sum(q for _, q in seqs) * hq * d * e
    assert nbytes == kv + qo + meta


def test_mixed_step_prefill_figures():
    """The mixed step's three prefill chunks: 476 tokens at offset 1024, 700
    and 808 at offset 0 (32 q heads, D 128): 1,173,136 visible pairs, 19.2 GFLOP."""
    _, flops, pairs = bench.algorithmic(_desc([(1500, 476), (700, 700), (808, 808)]), 32, 8, 128, 2)[:3]
    assert pairs == 1_173_136
    assert round(flops / 1e9, 1) == 19.2


def test_long_prompt_chunk_figures():
    """Chunk k of the 20,000-token prompt in 512-token chunks has 512·512k +
    131,328 visible pairs; k = 38 (offset 19,456, 64 q heads, D 128) is 330.7 GFLOP."""
    for k in (0, 1, 19, 38):
        _, _, pairs = bench.algorithmic(_desc([(512 * k + 512, 512)]), 64, 8, 128, 2)[:3]
        assert pairs == 512 * 512 * k + 131_328
    _, flops, _ = bench.algorithmic(_desc([(19456 + 512, 512)]), 64, 8, 128, 2)[:3]
    assert round(flops / 1e9, 1) == 330.7


def test_decode_kv_bytes_are_four_kib_per_token():
    """A decode token with 8 KV heads of 128 dims in bf16 reads 4 KiB of KV per context token."""
    nbytes, _, _ = bench.algorithmic(_desc([(1000, 1)]), 32, 8, 128, 2)[:3]
    kv = nbytes - 2 * 32 * 128 * 2 - (63 + 4) * 4
    assert kv == 1000 * 4096
    assert bench.algorithmic(_desc([(1000, 1)]), 32, 8, 128, 2)[3] == 1000 * 4096   # the KV part on its own
