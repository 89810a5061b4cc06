"""fp64 reference attention for one engine step (test infrastructure only).

What is computed
----------------
Ultralytics glossary, "Chunked Prefill", section "How chunked prefill works":
splitting a prompt changes only *when* its tokens are processed.  Each chunk
attends, under a causal mask over absolute positions, to the cached keys and
values of every earlier chunk plus its own, so the output equals one-shot
causal prefill.  A decode request is the special case of a one-token chunk
whose offset is its cached length.

For one sequence with query rows ``q[L, Hq, D]`` and the full KV history
``k, v[ctx, Hkv, D]`` (this step's tokens included), the offset of the chunk
is ``off = ctx - L`` and query row ``i`` sits at absolute position
``p = off + i``.  For every query head ``h``:

    g      = h // (Hq // Hkv)                   (grouped-query head mapping)
    x_j    = scale * sum_d q[i, h, d] * k[j, g, d]      for j = 0 .. p
    m      = max_j x_j
    w_j    = exp(x_j - m)
    out    = sum_j w_j * v[j, g, :] / sum_j w_j

Readings of points the pages leave open:
* the causal boundary is inclusive (the page's example masks only keys at
  later absolute positions, so a query keeps its own key), so every query
  sees at least itself and no row is empty;
* ``scale`` is passed in; the pages' code uses the library default
  ``1/sqrt(D)``, and callers pass that value rounded to fp32, the same value
  the GPU receives;
* grouped-query attention (absent from the pages) uses contiguous groups:
  query head ``h`` reads KV head ``h // (Hq // Hkv)``.

Sliding window (Hugging Face transformers, "Continuous batching
architecture", section "Memory management": sliding-attention layers keep only
a fixed window of the most recent tokens).  With a window of ``W`` tokens the
row at position ``p`` sees keys ``j`` with ``p - W < j <= p`` (the ``W`` most
recent positions, itself included); ``W = 0`` means no window.  Reading: the
window counts the query's own position, so ``W = 1`` sees only itself.

Two forms are given.  ``attend_rows`` is the definition taken row by row: a
row's arithmetic depends only on that row's query and on keys ``0..p``, so
chunked and one-shot prefill agree bit for bit.  ``attend`` is the same
definition in matrix form (masked score matrix, row softmax, weighted sum of
values), used where many rows are needed.  Both run in float64 on inputs that
are exactly the values the GPU holds (bf16 and fp32 widen exactly).
"""
from __future__ import annotations

import numpy as np


def _as64(a) -> np.ndarray:
    return np.asarray(a, dtype=np.float64)


def _check(q, k, v):
    if q.ndim != 3 or k.ndim != 3 or v.ndim != 3:
        raise ValueError("q must be [L, Hq, D] and k, v [ctx, Hkv, D]")
    L, Hq, D = q.shape
    ctx, Hkv, Dk = k.shape
    if v.shape != k.shape or Dk != D:
        raise ValueError("k and v must both be [ctx, Hkv, D] with q's D")
    if Hkv == 0 or Hq % Hkv != 0:
        raise ValueError("Hq must be a multiple of Hkv")
    if L > ctx:
        raise ValueError("the history must include this step's query tokens")
    return L, Hq, D, ctx, Hkv


def _first_key(pos: int, window: int) -> int:
    return max(0, pos - window + 1) if window > 0 else 0


def attend_row(q_row, k, v, pos: int, kv_head: int, scale: float, window: int = 0) -> np.ndarray:
    """One query row at absolute position ``pos`` against keys ``0..pos``
    (``pos-window+1 .. pos`` with a sliding window).

    ``q_row`` is ``[D]``; ``k, v`` are ``[ctx, Hkv, D]``.  Returns ``[D]``.
    This is the five-line definition in the module docstring, nothing else.
    """
    lo = _first_key(pos, window)
    qr = _as64(q_row)
    kk = _as64(k[lo: pos + 1, kv_head, :])    # keys lo..pos (inclusive)
    vv = _as64(v[lo: pos + 1, kv_head, :])
    x = scale * (kk @ qr)                      # x_j, j = 0..pos
    m = x.max()
    w = np.exp(x - m)
    return (w @ vv) / w.sum()


def attend_rows(q, k, v, scale: float, rows=None, window: int = 0) -> np.ndarray:
    """Row-by-row form.  ``q[L, Hq, D]``, ``k, v[ctx, Hkv, D]`` -> ``[L, Hq, D]``.

    ``rows`` optionally restricts the work to a list of ``(i, h)`` pairs;
    other entries of the result are NaN.
    """
    L, Hq, D, ctx, Hkv = _check(q, k, v)
    G = Hq // Hkv
    off = ctx - L
    out = np.full((L, Hq, D), np.nan)
    todo = rows if rows is not None else [(i, h) for i in range(L) for h in range(Hq)]
    for i, h in todo:
        out[i, h] = attend_row(q[i, h], k, v, off + i, h // G, scale, window)
    return out


def attend(q, k, v, scale: float, window: int = 0) -> np.ndarray:
    """Matrix form of the same definition.  Shapes as ``attend_rows``.

    For each query head: scores ``S = scale * Q K^T`` over the whole history,
    entries with key position > query position (or, with a window, at or
    below query position - window) set to -inf, a softmax along each row,
    then ``P V``.  Masked entries are replaced, never multiplied, so values
    outside a row's keys cannot reach it.
    """
    L, Hq, D, ctx, Hkv = _check(q, k, v)
    G = Hq // Hkv
    off = ctx - L
    q64, k64, v64 = _as64(q), _as64(k), _as64(v)
    pos = off + np.arange(L)
    j = np.arange(ctx)[None, :]
    visible = j <= pos[:, None]                                # [L, ctx]
    if window > 0:
        visible &= j > pos[:, None] - window
    out = np.empty((L, Hq, D))
    for h in range(Hq):
        g = h // G
        s = scale * (q64[:, h, :] @ k64[:, g, :].T)            # [L, ctx]
        s = np.where(visible, s, -np.inf)
        m = s.max(axis=1, keepdims=True)
        w = np.exp(s - m)                                      # masked -> 0
        vg = v64[:, g, :]
        if window > 0:   # keys below every row's window may hold anything
            vg = np.where(visible.any(axis=0)[:, None], vg, 0.0)
        out[:, h, :] = (w @ vg) / w.sum(axis=1, keepdims=True)
    return out

