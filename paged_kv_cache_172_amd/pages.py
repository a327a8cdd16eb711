"""Host side of the page pool: a free list and the lazy page step.

Physical pages are handed out only when a sequence's next token opens a new
page, and an exhausted pool is refused with a clear error instead of
preempting anything ("Hours of YouTube and 85 handtyped pages of notes on LLM
Inference - Start here", section "現在のスコープ": admission credits are kept
apart from physical pages, which are allocated lazily; a request that does
not fit is rejected with a clear error; --stats reports pool size, peak
allocated pages and final free pages).
"""
from __future__ import annotations

import collections

import numpy as np

PAGE_TOKENS = 16


class PoolExhausted(RuntimeError):
    pass


class FreeList:
    """FIFO free list of physical page ids with allocation statistics."""

    def __init__(self, pages, pool_size: int):
        self._free = collections.deque(int(p) for p in pages)
        self.pool_size = int(pool_size)
        self.allocated = self.pool_size - len(self._free)
        self.peak_allocated = self.allocated

    def __len__(self) -> int:
        return len(self._free)

    def pop(self) -> int:
        if not self._free:
            raise PoolExhausted(
                f"KV page pool exhausted: all {self.pool_size} pages are allocated")
        self.allocated += 1
        self.peak_allocated = max(self.peak_allocated, self.allocated)
        return self._free.popleft()

    def push(self, page: int) -> None:
        self._free.append(int(page))
        self.allocated -= 1

    def stats(self) -> dict:
        return {"pool_pages": self.pool_size, "peak_allocated_pages": self.peak_allocated,
                "free_pages": len(self._free)}


def lazy_page_step(block_tables: np.ndarray, context_lens: np.ndarray, free: FreeList):
    """Give every sequence whose new token (position ctx-1) opens a logical
    page it does not hold yet one physical page per layer.

    block_tables: int32 [L][B][bt_stride], -1 = not held; edited in place.
    context_lens: int32 [B], lengths after this step's append.
    Returns the sorted list of sequence ids whose rows changed."""
    L, B, W = block_tables.shape
    changed = set()
    for s in range(B):
        n = int(context_lens[s])
        if n < 1:
            continue
        j = (n - 1) // PAGE_TOKENS
        if j >= W:
            raise ValueError(f"sequence {s}: context {n} exceeds the table width {W * PAGE_TOKENS}")
        for layer in range(L):
            if block_tables[layer, s, j] < 0:
                block_tables[layer, s, j] = free.pop()
                changed.add(s)
    return sorted(changed)
