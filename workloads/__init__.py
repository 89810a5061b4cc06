"""Seeded synthetic inputs shared by the tests, the smoke check and the bench.

This module draws random numbers and lengths and fixes the shapes of the
workloads; it holds none of the attention arithmetic, no page mapping and no
scheduling logic.  Both the HIP path and the oracle take their inputs from
here (and from nothing else that the other side computes).

Values: Q, K and V are standard normal.  For bf16 workloads they are drawn
in float32 and rounded to bfloat16 by round-to-nearest-even (through
``torch``'s dtype conversion), and returned as float32 arrays holding exactly
the bf16 values, so the oracle widens exactly what the GPU holds.

K/V of a sequence are generated per 256-token block from a seed made of
``(seed, stream, seq, block)``: any token range of any sequence can be
regenerated independently, and re-chunking a prompt never changes its
values.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

BLOCK = 256   # tokens per independently seeded block of K/V or Q values
_K, _V, _Q = 1, 2, 3


def _rng(*key: int) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence([int(x) for x in key]))


def round_bf16(x: np.ndarray) -> np.ndarray:
    """float32 array -> float32 array of the nearest bfloat16 values (RNE)."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.bfloat16).to(torch.float32).numpy()


def _finish(x: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "bf16":
        return round_bf16(x)
    if dtype == "f32":
        return x.astype(np.float32, copy=False)
    raise ValueError(dtype)


def normal(shape, dtype: str, *key: int, std: float = 1.0) -> np.ndarray:
    x = _rng(*key).standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        x *= np.float32(std)
    return _finish(x, dtype)


def seq_kv(seed: int, seq: int, start: int, end: int, n_kv_heads: int, head_dim: int,
           dtype: str, std: float = 1.0):
    """K, V ``[end-start, Hkv, D]`` of tokens ``start..end-1`` of sequence ``seq``."""
    if end <= start:
        z = np.zeros((0, n_kv_heads, head_dim), np.float32)
        return z, z.copy()
    b0, b1 = start // BLOCK, (end - 1) // BLOCK + 1
    ks, vs = [], []
    for b in range(b0, b1):
        ks.append(_rng(seed, _K, seq, b).standard_normal((BLOCK, n_kv_heads, head_dim), np.float32))
        vs.append(_rng(seed, _V, seq, b).standard_normal((BLOCK, n_kv_heads, head_dim), np.float32))
    lo = start - b0 * BLOCK
    k = np.concatenate(ks)[lo:lo + end - start]
    v = np.concatenate(vs)[lo:lo + end - start]
    if std != 1.0:
        k = k * np.float32(std)
    return _finish(np.ascontiguousarray(k), dtype), _finish(np.ascontiguousarray(v), dtype)


def prompt_kv(seed: int, req_id: int, tokens, end: int, n_kv_heads: int, head_dim: int, dtype: str):
    """K, V ``[end, Hkv, D]`` of a request whose prompt is ``tokens``.

    Row ``p < len(tokens)`` is drawn from a seed made of the whole prompt prefix
    ``tokens[:p+1]`` (a 64-bit FNV-1a chain), so requests that share a prefix
    hold identical rows there and different prefixes give different rows; rows
    past the prompt depend on the request.
    """
    k = np.empty((end, n_kv_heads, head_dim), np.float32)
    v = np.empty_like(k)
    h = 0xCBF29CE484222325
    for p in range(end):
        if p < len(tokens):
            h = ((h ^ (int(tokens[p]) & 0xFFFFFFFF)) * 0x100000001B3) & 0xFFFFFFFFFFFFFFFF
            key = (seed, 7, h & 0xFFFFFFFF, h >> 32, p)
        else:
            key = (seed, 8, req_id, p)
        g = _rng(*key)
        k[p] = g.standard_normal(size=(n_kv_heads, head_dim), dtype=np.float32)
        v[p] = g.standard_normal(size=(n_kv_heads, head_dim), dtype=np.float32)
    return _finish(k, dtype), _finish(v, dtype)


def seq_q(seed: int, seq: int, start: int, end: int, n_q_heads: int, head_dim: int,
          dtype: str, std: float = 1.0):
    """Q ``[end-start, Hq, D]`` of tokens ``start..end-1`` of sequence ``seq``."""
    if end <= start:
        return np.zeros((0, n_q_heads, head_dim), np.float32)
    b0, b1 = start // BLOCK, (end - 1) // BLOCK + 1
    qs = [_rng(seed, _Q, seq, b).standard_normal((BLOCK, n_q_heads, head_dim), np.float32)
          for b in range(b0, b1)]
    lo = start - b0 * BLOCK
    q = np.concatenate(qs)[lo:lo + end - start]
    if std != 1.0:
        q = q * np.float32(std)
    return _finish(np.ascontiguousarray(q), dtype)


def uniform_ints(seed: int, n: int, lo: int, hi: int, stream: int = 0) -> np.ndarray:
    """``n`` integers uniform on ``lo..hi`` inclusive."""
    return _rng(seed, 7, stream).integers(lo, hi + 1, size=n).astype(np.int64)


def permutation(seed: int, n: int, stream: int = 0) -> np.ndarray:
    return _rng(seed, 11, stream).permutation(n).astype(np.int64)


def softmax_scale(head_dim: int) -> float:
    """The library-default softmax scale 1/sqrt(D), rounded to float32."""
    return float(np.float32(1.0 / math.sqrt(head_dim)))


def page_example_tensors():
    """Inputs of the pages' worked example: one layer of 8 heads x 64 dims
    and a 1000-token prompt (Ultralytics glossary, "Chunked Prefill", "How
    chunked prefill works"), drawn N(0, 1) in float32 from this module's own
    seeded generator (seed 0).  Returns ``q, k, v[1000, 8, 64]``, token-major.
    """
    k, v = seq_kv(0, 0, 0, 1000, 8, 64, "f32")
    q = seq_q(0, 0, 0, 1000, 8, 64, "f32")
    return q, k, v


# -- workload descriptors ------------------------------------------------------------

@dataclass
class Workload:
    """Shapes and scheduling knobs of one synthetic engine step (or trace)."""
    name: str
    seed: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    dtype: str
    max_batch_tokens: int
    max_requests: int = 128
    max_prefill_chunk: int = 0
    safety_margin: float = 0.0
    # requests in arrival order: (prompt_len, output_len, tokens_cached)
    requests: list = field(default_factory=list)
    pool_pages: int = 0
    description: str = ""


def _pages(n: int) -> int:
    return -(-n // 16)


def decode_only(seed: int = 2, n: int = 128, lo: int = 512, hi: int = 4096) -> Workload:
    """128 decodes, context uniform on [512, 4096], 32 q / 8 kv heads, D 128, bf16.

    Each request is imported with ``ctx - 1`` tokens cached, so the step
    appends one token per sequence and its context length is ``ctx``.
    """
    ctx = uniform_ints(seed, n, lo, hi)
    reqs = [(int(c) - 1, 64, int(c) - 1) for c in ctx]
    need = sum(_pages(int(c)) for c in ctx)
    return Workload("decode_128x[512,4096]_gqa32/8_d128_bf16", seed, 32, 8, 128, "bf16",
                    max_batch_tokens=2048, max_requests=128, requests=reqs,
                    pool_pages=int(math.ceil(1.1 * need)),
                    description="decode-only step: 128 sequences, one query token each")


def mixed(seed: int = 3) -> Workload:
    """64 decodes (context uniform [256, 8192]) + prompts 1500 (1024 cached), 700, 6000."""
    ctx = uniform_ints(seed, 64, 256, 8192)
    reqs = [(int(c) - 1, 64, int(c) - 1) for c in ctx]
    reqs += [(1500, 256, 1024), (700, 256, 0), (6000, 256, 0)]
    need = sum(_pages(int(c)) for c in ctx) + _pages(1500) + _pages(700) + _pages(6000)
    return Workload("mixed_64dec+476/700/808_gqa32/8_d128_bf16", seed, 32, 8, 128, "bf16",
                    max_batch_tokens=2048, max_requests=128, requests=reqs,
                    pool_pages=int(math.ceil(1.1 * need)),
                    description="mixed step: 64 decodes + three prefill chunks, T = 2048")


def long_prompt(seed: int = 4) -> Workload:
    """127 decodes (context uniform [1024, 8192]) + one 20,000-token prompt, 512-token chunks."""
    ctx = uniform_ints(seed, 127, 1024, 8192)
    reqs = [(int(c) - 1, 64, int(c) - 1) for c in ctx]
    reqs += [(20000, 16, 0)]
    need = sum(_pages(int(c) + 40) for c in ctx) + _pages(20000 + 16)
    return Workload("longprompt_127dec+20000@512_gqa64/8_d128_bf16", seed, 64, 8, 128, "bf16",
                    max_batch_tokens=2048, max_requests=128, max_prefill_chunk=512,
                    requests=reqs, pool_pages=int(math.ceil(1.1 * need)),
                    description="127 decodes + one 20k prompt in 512-token chunks, 40 steps")


def page_example() -> Workload:
    """The pages' worked example as an engine run: one 1000-token prompt, budget 256."""
    return Workload("page_example_1000@256_mha8_d64_f32", 0, 8, 8, 64, "f32",
                    max_batch_tokens=256, max_requests=128, requests=[(1000, 1, 0)],
                    pool_pages=63, description="1000-token prompt in chunks 256/256/256/232")


@dataclass
class TraceRequest:
    req_id: int
    arrival_step: int
    prompt_len: int
    output_len: int


def fifo_trace(seed: int = 5, n: int = 256, rate: float = 0.5, median_prompt: int = 1500,
               sigma: float = 1.0, max_prompt: int = 32768, mean_output: int = 256):
    """256 requests: Poisson arrivals (per step), lognormal prompts, geometric outputs."""
    rng = _rng(seed, 13)
    gaps = rng.exponential(1.0 / rate, size=n)
    arrive = np.floor(np.cumsum(gaps)).astype(np.int64)
    prompts = np.clip(np.round(rng.lognormal(math.log(median_prompt), sigma, size=n)),
                      1, max_prompt).astype(np.int64)
    outputs = rng.geometric(1.0 / mean_output, size=n).astype(np.int64)
    return [TraceRequest(i, int(a), int(p), int(o)) for i, (a, p, o)
            in enumerate(zip(arrive, prompts, outputs))]


def step_q(seed: int, step: int, n_tokens: int, n_q_heads: int, head_dim: int, dtype: str) -> np.ndarray:
    """Query rows of one engine step ``[T, Hq, D]`` (queries are not cached)."""
    return normal((n_tokens, n_q_heads, head_dim), dtype, seed, 17, step)


def device_normal(shape, dtype: str, device, *key: int):
    """Standard normal values drawn directly in device memory by torch's
    counter-based generator, seeded from ``key``; bf16 by RNE conversion.

    Used where host generation would dominate a long trace: the oracle side
    receives a host copy of exactly these values.
    """
    import torch
    seed = int(np.random.SeedSequence([int(k) for k in key]).generate_state(1, dtype=np.uint64)[0]) & ((1 << 63) - 1)
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    x = torch.randn(tuple(shape), generator=g, device=device, dtype=torch.float32)
    return x.to(torch.bfloat16) if dtype == "bf16" else x
