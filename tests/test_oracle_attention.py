"""Pins of the fp64 attention oracle to facts that do not come from it.

* the facts the pages state about their worked example (tests/golden/page_example.txt);
* a library routine (torch scaled_dot_product_attention in float64 on CPU);
* closed forms (one key, zero query -> prefix mean, constant V, a dominant key);
* brute force with pure-Python arithmetic on tiny inputs;
* invariants (chunking, grouped-query == repeated-KV multi-head).
"""
import math
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as F

from oracle import attention as ora
import workloads as wl

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "page_example.txt")


def _golden():
    out = {}
    for line in open(GOLDEN):
        if line.startswith("#") or ":" not in line:
            continue
        k, v = line.split(":", 1)
        out[k.strip()] = v.strip()
    return out


def _rand(shape, seed, scale=1.0):
    return np.random.default_rng(seed).standard_normal(shape) * scale


def _sdpa64(q, k, v, scale):
    """torch SDPA in float64 (the library routine) with an explicit causal mask
    over absolute positions."""
    L, Hq, D = q.shape
    ctx, Hkv, _ = k.shape
    G = Hq // Hkv
    qt = torch.from_numpy(np.ascontiguousarray(q.transpose(1, 0, 2))).double()[None]
    kt = torch.from_numpy(np.ascontiguousarray(k.transpose(1, 0, 2))).double()
    vt = torch.from_numpy(np.ascontiguousarray(v.transpose(1, 0, 2))).double()
    kt = kt.repeat_interleave(G, dim=0)[None]
    vt = vt.repeat_interleave(G, dim=0)[None]
    start = ctx - L
    # query row i sits at position start + i and sees keys 0 .. start + i
    mask = torch.arange(ctx)[None, :] <= (start + torch.arange(L))[:, None]
    o = F.scaled_dot_product_attention(qt, kt, vt, attn_mask=mask, scale=scale)
    return o[0].permute(1, 0, 2).numpy()


# -- the pages' worked example ---------------------------------------------------

def test_page_example_facts():
    """The section's stated facts, checked on the oracle: a 1000-token prompt
    of 8 heads x 64 dims, prefilled in chunks 256/256/256/232, equals one-pass
    prefill within the stated tolerance."""
    g = _golden()
    n, heads, dim = int(g["prompt_len"]), int(g["heads"]), int(g["head_dim"])
    sizes = [int(x) for x in g["chunks"].split()]
    assert sum(sizes) == n
    q, k, v = wl.page_example_tensors()
    assert q.shape == k.shape == v.shape == (n, heads, dim)
    scale = wl.softmax_scale(dim)
    whole = ora.attend(q, k, v, scale)
    parts, end = [], 0
    for size in sizes:                      # each chunk sees the cache up to its own end
        start, end = end, end + size
        parts.append(ora.attend(q[start:end], k[:end], v[:end], scale))
    chunked = np.concatenate(parts)
    agree = bool(np.max(np.abs(chunked - whole)) <= float(g["atol"]))
    assert agree == (g["chunked_equals_one_shot"] == "true")


def test_oracle_matches_page_example_library_result():
    """The oracle on the page's tensors agrees with the page's one-shot SDPA call."""
    q, k, v = wl.page_example_tensors()
    scale = wl.softmax_scale(64)
    assert scale == 0.125
    ref = ora.attend(q, k, v, scale)
    tq, tk, tv = (torch.from_numpy(x).permute(1, 0, 2)[None] for x in (q, k, v))
    full = F.scaled_dot_product_attention(tq, tk, tv, is_causal=True)[0].permute(1, 0, 2).numpy()
    assert np.max(np.abs(ref - full)) < 2e-6        # fp32 library vs fp64 oracle


def test_oracle_chunked_equals_one_shot_bitwise():
    """Chunks 256/256/256/232 of the page's prompt reproduce one-shot exactly."""
    q, k, v = wl.page_example_tensors()
    scale = wl.softmax_scale(64)
    rows = [(i, h) for i in range(0, 1000, 7) for h in range(8)]
    one = ora.attend_rows(q, k, v, scale, rows=rows)
    for chunk in (256, 1000, 512, 128, 100, 17, 1):
        got = np.full_like(one, np.nan)
        for start in range(0, 1000, chunk):
            end = min(start + chunk, 1000)
            sub = [(i - start, h) for (i, h) in rows if start <= i < end]
            if not sub:
                continue
            part = ora.attend_rows(q[start:end], k[:end], v[:end], scale, rows=sub)
            got[start:end] = np.where(np.isnan(part), got[start:end], part)
        sel = tuple(np.array(rows).T)
        assert np.array_equal(got[sel], one[sel]), chunk


def test_matrix_form_equals_row_form():
    q, k, v = wl.page_example_tensors()
    scale = wl.softmax_scale(64)
    a = ora.attend(q[768:], k, v, scale)
    b = ora.attend_rows(q[768:], k, v, scale)
    assert np.max(np.abs(a - b)) < 1e-13


# -- library routine --------------------------------------------------------------

@pytest.mark.parametrize("L,ctx,Hq,Hkv,D", [
    (1, 1, 1, 1, 8), (1, 37, 4, 1, 16), (5, 5, 2, 2, 8), (7, 40, 8, 2, 32),
    (33, 70, 32, 8, 64), (16, 16, 4, 4, 128), (3, 100, 6, 3, 16),
])
def test_oracle_matches_sdpa_fp64(L, ctx, Hq, Hkv, D):
    q = _rand((L, Hq, D), 1 + L)
    k = _rand((ctx, Hkv, D), 2 + ctx)
    v = _rand((ctx, Hkv, D), 3 + ctx)
    scale = wl.softmax_scale(D)
    ref = _sdpa64(q, k, v, scale)
    assert np.max(np.abs(ora.attend(q, k, v, scale) - ref)) < 1e-12
    assert np.max(np.abs(ora.attend_rows(q, k, v, scale) - ref)) < 1e-12


# -- closed forms -----------------------------------------------------------------

def test_single_key_returns_its_value():
    q = _rand((1, 4, 16), 5)
    k = _rand((1, 2, 16), 6)
    v = _rand((1, 2, 16), 7)
    out = ora.attend(q, k, v, 0.25)
    for h in range(4):
        assert np.array_equal(out[0, h], v[0, h // 2])


def test_zero_query_gives_prefix_mean():
    ctx, L, Hkv, G, D = 50, 20, 2, 3, 8
    q = np.zeros((L, Hkv * G, D))
    k = _rand((ctx, Hkv, D), 8)
    v = _rand((ctx, Hkv, D), 9)
    out = ora.attend(q, k, v, 0.3)
    off = ctx - L
    csum = np.cumsum(v, axis=0)
    for i in range(L):
        n = off + i + 1
        for h in range(Hkv * G):
            np.testing.assert_allclose(out[i, h], csum[n - 1, h // G] / n, rtol=0, atol=1e-14)


def test_constant_values_give_the_constant():
    c = _rand((2, 16), 10)
    k = _rand((30, 2, 16), 11)
    v = np.broadcast_to(c, (30, 2, 16)).copy()
    out = ora.attend(_rand((30, 4, 16), 12), k, v, 0.25)
    for h in range(4):
        np.testing.assert_allclose(out[:, h], np.broadcast_to(c[h // 2], (30, 16)), atol=1e-14)


def test_dominant_key_selects_its_value_exactly():
    ctx, D = 40, 16
    k = np.zeros((ctx, 1, D))
    v = _rand((ctx, 1, D), 13)
    j = 23
    k[j, 0, 0] = 32.0
    q = np.zeros((ctx - j, 1, D))
    q[:, 0, 0] = 32.0                     # score gap 32*32*scale = 256 * 4 -> weights exactly 0
    out = ora.attend(q, k, v, 1.0)
    for i in range(ctx - j):
        assert np.array_equal(out[i, 0], v[j, 0])


# -- brute force --------------------------------------------------------------------

def _brute(q, k, v, scale):
    L, Hq, D = q.shape
    ctx, Hkv, _ = k.shape
    G = Hq // Hkv
    out = np.zeros((L, Hq, D))
    for i in range(L):
        p = ctx - L + i
        for h in range(Hq):
            g = h // G
            xs = [scale * math.fsum(q[i, h, d] * k[j, g, d] for d in range(D)) for j in range(p + 1)]
            m = max(xs)
            ws = [math.exp(x - m) for x in xs]
            z = math.fsum(ws)
            for d in range(D):
                out[i, h, d] = math.fsum(w * v[j, g, d] for j, w in enumerate(ws)) / z
    return out


@pytest.mark.parametrize("L,ctx,Hq,Hkv,D", [(1, 1, 1, 1, 1), (3, 7, 2, 1, 3), (4, 12, 4, 2, 4), (12, 12, 2, 2, 2)])
def test_oracle_matches_brute_force(L, ctx, Hq, Hkv, D):
    q = _rand((L, Hq, D), 20 + L)
    k = _rand((ctx, Hkv, D), 21 + ctx)
    v = _rand((ctx, Hkv, D), 22 + D)
    b = _brute(q, k, v, 0.7)
    assert np.max(np.abs(ora.attend(q, k, v, 0.7) - b)) < 1e-13
    assert np.max(np.abs(ora.attend_rows(q, k, v, 0.7) - b)) < 1e-13


# -- invariants --------------------------------------------------------------------

def test_gqa_equals_mha_with_repeated_kv_bitwise():
    q = _rand((9, 8, 16), 30)
    k = _rand((25, 2, 16), 31)
    v = _rand((25, 2, 16), 32)
    g = ora.attend_rows(q, k, v, 0.25)
    m = ora.attend_rows(q, np.repeat(k, 4, axis=1), np.repeat(v, 4, axis=1), 0.25)
    assert np.array_equal(g, m)


def test_rejects_bad_shapes():
    with pytest.raises(ValueError):
        ora.attend(np.zeros((3, 3, 4)), np.zeros((5, 2, 4)), np.zeros((5, 2, 4)), 1.0)
    with pytest.raises(ValueError):
        ora.attend(np.zeros((6, 2, 4)), np.zeros((5, 2, 4)), np.zeros((5, 2, 4)), 1.0)


# -- sliding window ---------------------------------------------------------------

def _sdpa64_window(q, k, v, scale, window):
    """torch SDPA in float64 with the band mask p - W < j <= p."""
    L, Hq, D = q.shape
    ctx, Hkv, _ = k.shape
    G = Hq // Hkv
    qt = torch.from_numpy(np.ascontiguousarray(q.transpose(1, 0, 2))).double()[None]
    kt = torch.from_numpy(np.ascontiguousarray(k.transpose(1, 0, 2))).double().repeat_interleave(G, 0)[None]
    vt = torch.from_numpy(np.ascontiguousarray(v.transpose(1, 0, 2))).double().repeat_interleave(G, 0)[None]
    start = ctx - L
    pos = (start + torch.arange(L))[:, None]
    j = torch.arange(ctx)[None, :]
    band = (j <= pos) & (j > pos - window)
    o = F.scaled_dot_product_attention(qt, kt, vt, attn_mask=band, scale=scale)
    return o[0].permute(1, 0, 2).numpy()


def _brute_window(q, k, v, scale, window):
    L, Hq, D = q.shape
    ctx, Hkv, _ = k.shape
    G = Hq // Hkv
    out = np.zeros((L, Hq, D))
    for i in range(L):
        p = ctx - L + i
        for h in range(Hq):
            g = h // G
            keys = [j for j in range(ctx) if p - window < j <= p]
            x = [scale * math.fsum(float(q[i, h, d]) * float(k[j, g, d]) for d in range(D)) for j in keys]
            m = max(x)
            w = [math.exp(t - m) for t in x]
            sw = math.fsum(w)
            for d in range(D):
                out[i, h, d] = math.fsum(wj * float(v[j, g, d]) for wj, j in zip(w, keys)) / sw
    return out


@pytest.mark.parametrize("L,ctx,W", [(1, 9, 3), (5, 12, 4), (7, 7, 2), (6, 11, 16), (3, 10, 1)])
def test_window_matches_brute_force_and_sdpa(L, ctx, W):
    q, k, v = _rand((L, 4, 3), 1), _rand((ctx, 2, 3), 2), _rand((ctx, 2, 3), 3)
    for f in (ora.attend, ora.attend_rows):
        got = f(q, k, v, 0.6, window=W)
        assert np.abs(got - _brute_window(q, k, v, 0.6, W)).max() <= 1e-13
        assert np.abs(got - _sdpa64_window(q, k, v, 0.6, W)).max() <= 1e-12


def test_window_at_least_context_is_full_attention_bitwise():
    q, k, v = _rand((20, 4, 8), 4), _rand((50, 2, 8), 5), _rand((50, 2, 8), 6)
    for W in (50, 51, 1000):
        assert np.array_equal(ora.attend_rows(q, k, v, 0.3, window=W), ora.attend_rows(q, k, v, 0.3))
        assert np.array_equal(ora.attend(q, k, v, 0.3, window=W), ora.attend(q, k, v, 0.3))


def test_window_one_returns_own_value_exactly():
    q, k, v = _rand((9, 4, 8), 7), _rand((30, 2, 8), 8), _rand((30, 2, 8), 9)
    for f in (ora.attend, ora.attend_rows):
        out = f(q, k, v, 0.5, window=1)
        for i in range(9):
            for h in range(4):
                assert np.array_equal(out[i, h], v[21 + i, h // 2])


def test_window_zero_query_gives_windowed_mean():
    k, v = _rand((40, 1, 5), 10), _rand((40, 1, 5), 11)
    q = np.zeros((10, 2, 5))
    out = ora.attend(q, k, v, 0.7, window=6)
    for i in range(10):
        p = 30 + i
        assert np.abs(out[i, 0] - v[p - 5:p + 1, 0].mean(axis=0)).max() <= 1e-14


def test_window_row_equals_full_attention_on_its_window():
    """A windowed row is the unwindowed definition on keys p-W+1..p, bit for bit."""
    q, k, v = _rand((12, 4, 8), 12), _rand((64, 2, 8), 13), _rand((64, 2, 8), 14)
    W = 9
    out = ora.attend_rows(q, k, v, 0.4, window=W)
    for i in (0, 5, 11):
        p = 52 + i
        for h in range(4):
            ref = ora.attend_row(q[i, h], k[p - W + 1:], v[p - W + 1:], W - 1, h // 2, 0.4)
            assert np.array_equal(out[i, h], ref)


def test_window_chunked_equals_one_shot_bitwise():
    q, k, v = _rand((60, 4, 8), 15), _rand((60, 2, 8), 16), _rand((60, 2, 8), 17)
    full = ora.attend_rows(q, k, v, 0.25, window=13)
    for size in (7, 16, 25):
        parts = [ora.attend_rows(q[a:a + size], k[:a + size][:min(60, a + size)],
                                 v[:min(60, a + size)], 0.25, window=13)
                 for a in range(0, 60, size)]
        assert np.array_equal(np.concatenate(parts), full)


def test_window_ignores_values_below_every_row():
    """Keys no row can see may hold anything, NaN included."""
    q, k, v = _rand((4, 2, 8), 18), _rand((40, 1, 8), 19), _rand((40, 1, 8), 20)
    W = 5
    k2, v2 = k.copy(), v.copy()
    k2[:32] = np.nan          # rows sit at 36..39, so keys below 32 are never visible
    v2[:32] = np.nan
    assert np.array_equal(ora.attend(q, k2, v2, 0.3, window=W), ora.attend(q, k, v, 0.3, window=W))
    assert np.array_equal(ora.attend_rows(q, k2, v2, 0.3, window=W), ora.attend_rows(q, k, v, 0.3, window=W))
