"""Host model of the paged KV cache (test infrastructure only).

Pages (Hugging Face transformers, "Continuous batching architecture",
section "Memory management"): the KV cache is cut into pages of
``page_size`` tokens of one layer so requests of different lengths share one
fixed pool.  AI Engineering from Scratch, "vLLM serving internals", section
"PagedAttention as virtual memory": each sequence has a block table mapping
its logical token positions to physical blocks of 16 tokens; a sequence that
grows past its last block gets one more block.

The physical layout inside a page is not on the pages; the library fixes it
and this model follows the library's documented layout:

    k_cache[num_pages, Hkv, 16, D]   token-major: one (page, head) slab is
                                     16 rows of D values
    v_cache[num_pages, Hkv, D, 16]   token-minor: one (page, head) slab is
                                     D rows of 16 token values

A slot is ``page * 16 + offset``.  Appending token ``t`` writes its K and V
rows to slot ``slot_mapping[t]``; a negative slot writes nothing.  All copies
here are exact (the arrays keep the caller's dtype; no arithmetic is done on
values), which is what the append kernel must reproduce bit for bit.
"""
from __future__ import annotations

import numpy as np

PAGE = 16


def slot_of(block_table_row, pos: int, page_size: int = PAGE) -> int:
    """Physical slot of logical position ``pos`` through a block table row."""
    return int(block_table_row[pos // page_size]) * page_size + pos % page_size


def append(k_cache, v_cache, k_new, v_new, slot_mapping, page_size: int = PAGE):
    """Copy each new token's K/V rows into its slot, in place.

    ``k_new, v_new[T, Hkv, D]``; ``slot_mapping[T]`` (int).  Later tokens win
    if two tokens name one slot (the library forbids duplicates; the model
    needs no rule for them).
    """
    for t, slot in enumerate(np.asarray(slot_mapping).tolist()):
        if slot < 0:
            continue
        page, off = divmod(int(slot), page_size)
        k_cache[page, :, off, :] = k_new[t]
        v_cache[page, :, :, off] = v_new[t]


def gather(k_cache, v_cache, block_table_row, ctx: int, page_size: int = PAGE):
    """Contiguous ``K, V[ctx, Hkv, D]`` of one sequence, read through its table."""
    num_pages, Hkv, _, D = k_cache.shape
    k = np.empty((ctx, Hkv, D), dtype=k_cache.dtype)
    v = np.empty((ctx, Hkv, D), dtype=v_cache.dtype)
    for pos in range(ctx):
        page, off = divmod(slot_of(block_table_row, pos, page_size), page_size)
        k[pos] = k_cache[page, :, off, :]
        v[pos] = v_cache[page, :, :, off]
    return k, v


def slots_for(block_table_row, start: int, end: int, page_size: int = PAGE):
    """Slot mapping of logical positions ``start .. end-1`` of one sequence."""
    return np.array([slot_of(block_table_row, p, page_size) for p in range(start, end)],
                    dtype=np.int32)
