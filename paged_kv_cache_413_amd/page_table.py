"""Host-side page-table maintenance for limited attention windows.

Under a window of W tokens a query at position p attends to keys p - W + 1 .. p only,
so the blocks wholly before every window of a sequence can be released and reused
("NVIDIA TensorRT-LLM详解：架构、KV Cache、调度与部署实践", §11, limited attention window).
The attention kernels never read the table entries of pages that end at or before
32 * floor(lo / 32), lo = the first key the call's earliest query of the sequence sees
(they fetch keys in 32-token blocks); those pages are what release_out_of_window frees.
"""
from __future__ import annotations

import numpy as np


def window_lo(pos: int, window: int) -> int:
    """First key a query at position pos attends to under `window` (0 = no window)."""
    return max(0, pos - window + 1) if window > 0 else 0


def releasable_pages(context_len: int, num_queries: int, window: int, page_size: int) -> int:
    """Number of leading logical pages of a sequence whose K/V no query of this or any
    later step reads: the call's earliest query sits at context_len - num_queries, and
    later steps' windows start later still."""
    if window <= 0:
        return 0
    lo = window_lo(context_len - num_queries, window)
    return ((lo // 32) * 32) // page_size


def release_out_of_window(block_tables: np.ndarray, context_lens: np.ndarray, new_lens: np.ndarray,
                          window: int, page_size: int):
    """Return (tables, freed): a copy of the int32 block tables with the releasable
    leading entries of every sequence set to -1, and the physical pages that no entry
    references any more (a page shared by several sequences, such as a common prefix,
    is freed only once every sequence has dropped it)."""
    tables = np.array(block_tables, dtype=np.int32, copy=True)
    dropped = []
    for s in range(tables.shape[0]):
        n = releasable_pages(int(context_lens[s]), int(new_lens[s]), window, page_size)
        row = tables[s, :n]
        dropped.extend(int(p) for p in row[row >= 0])
        tables[s, :n] = -1
    still = np.unique(tables[tables >= 0])
    freed = np.setdiff1d(np.unique(np.array(dropped, dtype=np.int64)), still)
    return tables, freed


def shared_pages(block_tables: np.ndarray, context_lens: np.ndarray, page_size: int) -> np.ndarray:
    """Physical pages that the used part of two or more sequences' tables name: the blocks
    of a common prefix several requests reuse ("NVIDIA TensorRT-LLM详解：架构、KV Cache、
    调度与部署实践", §10, cross-request KV reuse)."""
    used = []
    for s in range(block_tables.shape[0]):
        n = -(-int(context_lens[s]) // page_size)
        used.append(np.unique(block_tables[s, :n]))
    pages, counts = np.unique(np.concatenate(used) if used else np.zeros(0, np.int32), return_counts=True)
    return pages[counts > 1]


def check_append_targets(block_tables: np.ndarray, context_lens: np.ndarray, new_lens: np.ndarray,
                         page_size: int, shared=None):
    """Host-side check before kv_append: no appended row may land in a page other
    sequences share (a shared prefix page is read by all of them; a request writes only
    pages of its own, copying a partly matched page first, §11 of the same page), and no two appended rows may
    name the same (page, slot).  `shared` defaults to shared_pages(...).  Raises
    ValueError naming the first offending sequence."""
    if shared is None:
        shared = shared_pages(block_tables, context_lens, page_size)
    shared = set(int(p) for p in np.asarray(shared).reshape(-1))
    seen = {}
    for s in range(block_tables.shape[0]):
        L, n = int(context_lens[s]), int(new_lens[s])
        for t in range(L - n, L):
            page, slot = int(block_tables[s, t // page_size]), t % page_size
            if page in shared:
                raise ValueError(f"sequence {s} appends position {t} into page {page}, which other sequences share")
            if (page, slot) in seen:
                raise ValueError(f"sequences {seen[(page, slot)]} and {s} both append into page {page}, slot {slot}")
            seen[(page, slot)] = s
