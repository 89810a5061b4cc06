"""Pins of the host paged-KV model: permuted pools reproduce the contiguous history."""
import numpy as np

from oracle import paging


def _history(ctx, Hkv, D, seed):
    r = np.random.default_rng(seed)
    return (r.standard_normal((ctx, Hkv, D)).astype(np.float32),
            r.standard_normal((ctx, Hkv, D)).astype(np.float32))


def test_append_then_gather_is_identity_bitwise_for_two_permutations():
    ctx, Hkv, D = 203, 3, 8
    k, v = _history(ctx, Hkv, D, 0)
    n_pages = -(-ctx // 16)
    outs = []
    for seed in (1, 2):
        pool = 2 * n_pages
        kc = np.full((pool, Hkv, 16, D), np.nan, np.float32)
        vc = np.full((pool, Hkv, D, 16), np.nan, np.float32)
        bt = np.random.default_rng(seed).permutation(pool)[:n_pages]
        # append in three uneven chunks through the slot mapping
        for a, b in ((0, 50), (50, 51), (51, ctx)):
            paging.append(kc, vc, k[a:b], v[a:b], paging.slots_for(bt, a, b))
        gk, gv = paging.gather(kc, vc, bt, ctx)
        assert np.array_equal(gk, k) and np.array_equal(gv, v)
        outs.append((gk, gv))
    assert np.array_equal(outs[0][0], outs[1][0])


def test_negative_slot_writes_nothing_and_layout_is_documented():
    kc = np.zeros((2, 1, 16, 4), np.float32)
    vc = np.zeros((2, 1, 4, 16), np.float32)
    kn = np.arange(8, dtype=np.float32).reshape(2, 1, 4) + 1
    paging.append(kc, vc, kn, -kn, np.array([17, -1]))
    assert np.array_equal(kc[1, 0, 1], kn[0, 0])          # page 1, offset 1, token-major K
    assert np.array_equal(vc[1, 0, :, 1], -kn[0, 0])      # token-minor V
    assert np.count_nonzero(kc) == 4 and np.count_nonzero(vc) == 4


def test_slot_of_matches_page_arithmetic():
    bt = np.array([5, 2, 9])
    assert [paging.slot_of(bt, p) for p in (0, 15, 16, 33, 47)] == [80, 95, 32, 145, 159]
