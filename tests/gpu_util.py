"""Helpers for the GPU tests: device copies of seeded inputs and paged steps.

Inputs come from ``workloads`` (seeded generators); expected values come from
``oracle``.  Nothing here computes attention.
"""
from __future__ import annotations

import sys

import numpy as np
import torch

import chunked_prefill_attention_amd as cb
import workloads as wl

TORCH_DT = {"bf16": torch.bfloat16, "f32": torch.float32}
BF16_ATOL, BF16_RTOL = 2e-2, 1e-2      # the stated bf16 tolerance (allclose form)
F32_ATOL = 1e-4


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def dev():
    return torch.device("cuda", 0)


def to_dev(x: np.ndarray, dtype: str) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(dev()).to(TORCH_DT[dtype])


def i32(x) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.int32)).to(dev())


def new_cache(num_pages: int, hkv: int, d: int, dtype: str, fill=float("nan")):
    k = torch.full((num_pages, hkv, 16, d), fill, dtype=TORCH_DT[dtype], device=dev())
    v = torch.full((num_pages, hkv, d, 16), fill, dtype=TORCH_DT[dtype], device=dev())
    return k, v


def slots_from_table(row, start, end):
    pos = np.arange(start, end)
    return (np.asarray(row)[pos // 16] * 16 + pos % 16).astype(np.int32)


def write_history(kc, vc, k_hist, v_hist, row, start, end, dtype):
    """Write tokens start..end-1 of a sequence through the append kernel."""
    if end <= start:
        return
    cb.kv_append(to_dev(k_hist[start:end], dtype), to_dev(v_hist[start:end], dtype), kc, vc,
                 i32(slots_from_table(row, start, end)))


class Step:
    """A synthetic engine step: per-sequence histories, queries and page tables."""

    def __init__(self, seqs, hq, hkv, d, dtype, seed=0, pool_extra=1.25, table_seed=1,
                 kv_std=1.0, q_std=1.0, fill=float("nan"), history_via="append"):
        # seqs: list of (ctx, q_len); decodes (q_len == 1 first) are the leading entries
        self.seqs = list(seqs)
        self.hq, self.hkv, self.d, self.dtype = hq, hkv, d, dtype
        # the leading q_len == 1 sequences take the decode path
        nd = 0
        for c, n in self.seqs:
            if n != 1:
                break
            nd += 1
        self.num_decodes = nd
        need = sum(-(-c // 16) for c, _ in self.seqs)
        self.num_pages = max(1, int(need * pool_extra) + 1)
        perm = wl.permutation(table_seed, self.num_pages)
        self.rows, cur = [], 0
        for c, _ in self.seqs:
            n = -(-c // 16)
            self.rows.append(perm[cur:cur + n].astype(np.int32))
            cur += n
        self.stride = max([len(r) for r in self.rows] + [1])
        self.bt = np.zeros((len(self.seqs), self.stride), np.int32)
        for s, r in enumerate(self.rows):
            self.bt[s, :len(r)] = r
        self.k_hist, self.v_hist, self.q = [], [], []
        for s, (c, n) in enumerate(self.seqs):
            k, v = wl.seq_kv(seed, s, 0, c, hkv, d, dtype, std=kv_std)
            self.k_hist.append(k)
            self.v_hist.append(v)
            self.q.append(wl.seq_q(seed, s, c - n, c, hq, d, dtype, std=q_std))
        self.qsl = np.concatenate([[0], np.cumsum([n for _, n in self.seqs])]).astype(np.int32)
        self.ctx = np.array([c for c, _ in self.seqs], np.int32)
        self.off = np.array([c - n for c, n in self.seqs], np.int32)
        self.T = int(self.qsl[-1])
        self.max_ctx = int(self.ctx.max()) if len(self.seqs) else 0
        self.fill = fill
        self.scale = wl.softmax_scale(d)

    def upload(self, table=None):
        """Allocate the caches, write every history, return them."""
        kc, vc = new_cache(self.num_pages, self.hkv, self.d, self.dtype, self.fill)
        bt = self.bt if table is None else table
        for s, (c, n) in enumerate(self.seqs):
            row = bt[s]
            write_history(kc, vc, self.k_hist[s], self.v_hist[s], row, 0, c - n, self.dtype)
            write_history(kc, vc, self.k_hist[s], self.v_hist[s], row, c - n, c, self.dtype)
        return kc, vc

    def run(self, kc, vc, table=None, out=None):
        q = to_dev(np.concatenate(self.q) if self.T else np.zeros((0, self.hq, self.d)), self.dtype)
        bt = self.bt if table is None else table
        o = cb.attention_step(q, kc, vc, i32(bt), i32(self.qsl), i32(self.ctx), i32(self.off),
                              self.num_decodes, self.max_ctx, self.scale, out=out)
        torch.cuda.synchronize()
        return o

    def permuted_table(self, seed):
        """The same logical pages on a different physical permutation."""
        perm = wl.permutation(seed, self.num_pages)
        bt = np.zeros_like(self.bt)
        cur = 0
        for s, r in enumerate(self.rows):
            bt[s, :len(r)] = perm[cur:cur + len(r)]
            cur += len(r)
        return bt

    def out_rows(self, out: torch.Tensor, s: int) -> np.ndarray:
        a, b = self.qsl[s], self.qsl[s + 1]
        return out[a:b].float().cpu().numpy()


def compare(got: np.ndarray, ref: np.ndarray, dtype: str, what: str = "", absmean=None):
    """Assert the stated tolerance; for bf16 also the bound derived from the
    kernel's arithmetic when ``absmean`` (attention over |V|) is given.

    Derived bound: the probabilities enter the P V product rounded to bf16
    (relative error <= 2^-9 each); the normaliser sums them in fp32 (decode)
    or sums the same rounded values (prefill).  Either way the pre-rounding
    output error is at most 2 * 2^-9 * sum_j w_j |v_j| / sum_j w_j; the final
    rounding to bf16 adds 2^-9 |out|.  The check allows twice that.
    """
    assert got.shape == ref.shape, (got.shape, ref.shape)
    assert np.isfinite(got).all(), f"{what}: non-finite output"
    err = np.abs(got.astype(np.float64) - ref)
    if dtype == "f32":
        assert err.max() <= F32_ATOL, f"{what}: max abs err {err.max():.3e}"
        return err.max()
    bad = err > BF16_ATOL + BF16_RTOL * np.abs(ref)
    assert not bad.any(), f"{what}: {bad.sum()} elements outside the stated bf16 tolerance, max {err.max():.3e}"
    if absmean is not None:
        bound = 2.0 ** -7 * absmean + 2.0 ** -8 * np.abs(ref) + 1e-6
        tight = err > bound
        assert not tight.any(), (f"{what}: {tight.sum()} elements outside the derived bound; "
                                 f"worst err/bound {(err / bound).max():.2f}")
    return err.max()
