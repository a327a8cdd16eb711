"""Host side of the page pool: thin bindings of the native page management in
libpagedkv.so (include/paged_kv_pager.h).

- ``FreeList``: the FIFO free list of physical pages.
- ``lazy_page_step``: the lazy page step of a decode batch.
- ``Pager``: admission credits, lazy physical pages, FIFO waiting, early
  release and prefix sharing with copy-on-write, plus the statistics the
  pages list ("Hours of YouTube and 85 handtyped pages of notes on LLM
  Inference - Start here", section "現在のスコープ").

Argument marshalling only; every decision is made in the C++ code.
"""
from __future__ import annotations

import ctypes

import numpy as np

from . import _lib

PAGE_TOKENS = 16


class PoolExhausted(_lib.PagedKVError):
    pass


class RequestRejected(_lib.PagedKVError):
    pass


def _raise(status: int, where: str):
    if status == _lib.PKV_OK:
        return
    if status == _lib.PKV_ERR_EXHAUSTED:
        raise PoolExhausted(status, where)
    if status == _lib.PKV_ERR_REJECTED:
        raise RequestRejected(status, where)
    raise _lib.PagedKVError(status, where)


def _i32(a) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=np.int32)


class FreeList:
    """FIFO free list of physical page ids with allocation statistics."""

    def __init__(self, pages, pool_size: int):
        lib = _lib.load()
        ids = _i32(pages)
        h = ctypes.c_void_p()
        _raise(lib.paged_kv_free_list_create(ids.ctypes.data_as(ctypes.c_void_p), ids.size,
                                             int(pool_size), ctypes.byref(h)),
               "paged_kv_free_list_create")
        self._h = h
        self._lib = lib
        self.pool_size = int(pool_size)

    def __del__(self):
        h = getattr(self, "_h", None)
        if h is not None and h.value:
            self._lib.paged_kv_free_list_destroy(h)
            self._h = None

    def _stats(self):
        pool, peak, free = ctypes.c_int64(), ctypes.c_int64(), ctypes.c_int64()
        _raise(self._lib.paged_kv_free_list_stats(self._h, ctypes.byref(pool), ctypes.byref(peak),
                                                  ctypes.byref(free)), "paged_kv_free_list_stats")
        return pool.value, peak.value, free.value

    def __len__(self) -> int:
        return self._stats()[2]

    def pop(self) -> int:
        page = ctypes.c_int32()
        _raise(self._lib.paged_kv_free_list_pop(self._h, ctypes.byref(page)),
               "paged_kv_free_list_pop")
        return page.value

    def push(self, page: int) -> None:
        _raise(self._lib.paged_kv_free_list_push(self._h, int(page)), "paged_kv_free_list_push")

    def stats(self) -> dict:
        pool, peak, free = self._stats()
        return {"pool_pages": pool, "peak_allocated_pages": peak, "free_pages": free}


def lazy_page_step(block_tables: np.ndarray, context_lens: np.ndarray, free: FreeList):
    """Give every sequence whose new token (position ctx-1) opens a logical
    page it does not hold yet one physical page per layer (all or nothing).

    block_tables: int32 [L][B][bt_stride], -1 = not held; edited in place.
    context_lens: int32 [B], lengths after this step's append.
    Returns the sorted list of sequence ids whose rows changed."""
    if block_tables.dtype != np.int32 or not block_tables.flags.c_contiguous:
        raise TypeError("block_tables must be a C-contiguous int32 array")
    L, B, W = block_tables.shape
    ctx = _i32(context_lens)
    changed = np.empty(max(B, 1), np.int32)
    n = ctypes.c_int32()
    _raise(free._lib.paged_kv_lazy_page_step(
        free._h, block_tables.ctypes.data_as(ctypes.c_void_p), L, B, W,
        ctx.ctypes.data_as(ctypes.c_void_p), changed.ctypes.data_as(ctypes.c_void_p),
        ctypes.byref(n)), "paged_kv_lazy_page_step")
    return changed[:n.value].tolist()


class Pager:
    """Request pager: admission credits, lazy pages, FIFO waiting, early
    release, prefix sharing with copy-on-write.  Table rows are host int32
    arrays [num_layers][row_width] the pager writes into."""

    def __init__(self, num_pages: int, num_layers: int, max_context: int = 2048):
        lib = _lib.load()
        h = ctypes.c_void_p()
        _raise(lib.paged_kv_pager_create(int(num_pages), int(num_layers), int(max_context),
                                         ctypes.byref(h)), "paged_kv_pager_create")
        self._h = h
        self._lib = lib
        self.num_layers = int(num_layers)

    def __del__(self):
        h = getattr(self, "_h", None)
        if h is not None and h.value:
            self._lib.paged_kv_pager_destroy(h)
            self._h = None

    def submit(self, prompt_tokens: int, max_new_tokens: int):
        """Queue a request; returns (request id, allowed new tokens)."""
        rid, allowed = ctypes.c_int64(), ctypes.c_int32()
        _raise(self._lib.paged_kv_pager_submit(self._h, int(prompt_tokens), int(max_new_tokens),
                                               ctypes.byref(rid), ctypes.byref(allowed)),
               "paged_kv_pager_submit")
        return rid.value, allowed.value

    def admit(self, capacity: int = 1 << 20):
        """Admit waiting requests in FIFO order; returns their ids."""
        ids = np.empty(max(int(capacity), 1), np.int64)
        n = ctypes.c_int32()
        _raise(self._lib.paged_kv_pager_admit(self._h, ids.ctypes.data_as(ctypes.c_void_p),
                                              int(capacity), ctypes.byref(n)),
               "paged_kv_pager_admit")
        return ids[:n.value].tolist()

    def _copy_bufs(self, n):
        return np.empty(max(n, 1), np.int32), np.empty(max(n, 1), np.int32)

    def reserve(self, rid: int, length: int, table: np.ndarray):
        """Hold the pages of tokens [0, length); writes the table row
        ([num_layers][width] int32, in place).  Returns the copy-on-write
        page pairs [(src, dst), ...] to copy on the device first."""
        self._check_table(table)
        src, dst = self._copy_bufs(self.num_layers)
        n = ctypes.c_int32()
        _raise(self._lib.paged_kv_pager_reserve(
            self._h, int(rid), int(length), table.ctypes.data_as(ctypes.c_void_p),
            table.shape[-1], src.ctypes.data_as(ctypes.c_void_p),
            dst.ctypes.data_as(ctypes.c_void_p), ctypes.byref(n)), "paged_kv_pager_reserve")
        return list(zip(src[:n.value].tolist(), dst[:n.value].tolist()))

    def decode_step(self, rids, lengths, tables: np.ndarray):
        """reserve() for one decode batch; tables [n][num_layers][width]."""
        ids = np.ascontiguousarray(rids, np.int64)
        lens = _i32(lengths)
        n = ids.size
        if tables.dtype != np.int32 or not tables.flags.c_contiguous or tables.shape[0] < n:
            raise TypeError("tables must be a C-contiguous int32 array [n][layers][width]")
        src, dst = self._copy_bufs(n * self.num_layers)
        nc = ctypes.c_int32()
        _raise(self._lib.paged_kv_pager_decode_step(
            self._h, ids.ctypes.data_as(ctypes.c_void_p), lens.ctypes.data_as(ctypes.c_void_p),
            n, tables.ctypes.data_as(ctypes.c_void_p), tables.shape[1] * tables.shape[2],
            tables.shape[2], src.ctypes.data_as(ctypes.c_void_p),
            dst.ctypes.data_as(ctypes.c_void_p), ctypes.byref(nc)), "paged_kv_pager_decode_step")
        return list(zip(src[:nc.value].tolist(), dst[:nc.value].tolist()))

    def share_prefix(self, src_rid: int, dst_rid: int, tokens: int, table: np.ndarray) -> None:
        self._check_table(table)
        _raise(self._lib.paged_kv_pager_share_prefix(
            self._h, int(src_rid), int(dst_rid), int(tokens),
            table.ctypes.data_as(ctypes.c_void_p), table.shape[-1]), "paged_kv_pager_share_prefix")

    def finish(self, rid: int) -> None:
        _raise(self._lib.paged_kv_pager_finish(self._h, int(rid)), "paged_kv_pager_finish")

    def stats(self) -> dict:
        st = _lib.PagerStats()
        _raise(self._lib.paged_kv_pager_get_stats(self._h, ctypes.byref(st)),
               "paged_kv_pager_get_stats")
        return {name: getattr(st, name) for name, _ in _lib.PagerStats._fields_}

    def _check_table(self, table):
        if (table.dtype != np.int32 or not table.flags.c_contiguous or table.ndim != 2
                or table.shape[0] != self.num_layers):
            raise TypeError("table must be a C-contiguous int32 array [num_layers][width]")
