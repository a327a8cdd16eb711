"""ctypes binding of libpagedkv.so (include/paged_kv.h).

Argument marshalling only: each function takes device pointers (ints) or
objects with ``data_ptr()`` (torch tensors), converts them and calls the C
entry point of the same name.  A non-zero status raises ``PagedKVError``.
There is no fallback: if the library is not built, loading raises.
"""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libpagedkv.so")

PKV_OK = 0
PKV_ERR_INVALID_ARG = -1
PKV_ERR_ALIGNMENT = -2
PKV_ERR_WORKSPACE = -3
PKV_ERR_UNSUPPORTED = -4
PKV_ERR_HIP = -5
PKV_ERR_EXHAUSTED = -6
PKV_ERR_REJECTED = -7
PKV_ERR_BUDGET = -8
PKV_ERR_STATE = -9

EXPORTED = (
    "paged_kv_rope_table",
    "paged_kv_append",
    "paged_decode_attn_num_splits",
    "paged_decode_attn_workspace_size",
    "paged_decode_attn_workspace_init",
    "paged_decode_attn_order",
    "paged_decode_attn_order_round",
    "paged_decode_attn_order_host",
    "paged_decode_attn",
    "paged_decode_attn_split",
    "paged_decode_attn_combine",
    "paged_kv_append_decode_attn",
    "paged_kv_append_decode_attn_noalloc",
    "paged_kv_prefill",
    "paged_kv_copy_pages",
    "paged_kv_status_string",
    # host page management (include/paged_kv_pager.h)
    "paged_kv_free_list_create",
    "paged_kv_free_list_destroy",
    "paged_kv_free_list_pop",
    "paged_kv_free_list_push",
    "paged_kv_free_list_stats",
    "paged_kv_lazy_page_step",
    "paged_kv_pager_create",
    "paged_kv_pager_destroy",
    "paged_kv_pager_submit",
    "paged_kv_pager_admit",
    "paged_kv_pager_reserve",
    "paged_kv_pager_decode_step",
    "paged_kv_pager_share_prefix",
    "paged_kv_pager_finish",
    "paged_kv_pager_get_stats",
)


class PagerStats(ctypes.Structure):
    """paged_kv_pager_stats."""
    _fields_ = [
        ("pool_pages", ctypes.c_int64),
        ("free_pages", ctypes.c_int64),
        ("live_pages", ctypes.c_int64),
        ("peak_live_pages", ctypes.c_int64),
        ("credit_pages", ctypes.c_int64),
        ("shared_refs", ctypes.c_int64),
        ("copies", ctypes.c_int64),
        ("active_requests", ctypes.c_int32),
        ("peak_active_requests", ctypes.c_int32),
        ("waiting_requests", ctypes.c_int32),
        ("largest_decode_batch", ctypes.c_int32),
        ("submitted", ctypes.c_int64),
        ("admitted", ctypes.c_int64),
        ("rejected", ctypes.c_int64),
        ("finished", ctypes.c_int64),
        ("wait_max_us", ctypes.c_double),
        ("wait_total_us", ctypes.c_double),
    ]


class PagedKVError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {status_string(status)} (status {status})")


class Pool(ctypes.Structure):
    """paged_kv_pool: pointers are device addresses, strides in elements."""
    _fields_ = [
        ("k_pool", ctypes.c_void_p),
        ("v_pool", ctypes.c_void_p),
        ("num_pages", ctypes.c_int64),
        ("page_stride", ctypes.c_int64),
        ("head_stride", ctypes.c_int64),
        ("slot_stride", ctypes.c_int64),
    ]


_lib = None


def load(path: str = LIB_PATH):
    """Load libpagedkv.so (built by ``python -m paged_kv_cache_172_amd.build``)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with "
                           "`python -m paged_kv_cache_172_amd.build` (needs hipcc)")
    # torch ships its own HIP runtime under the same soname as the system's
    # (libamdhip64.so.7).  Whichever is loaded first serves the whole process,
    # and torch's bundled HSA runtime works only with its own, so torch (the
    # caller's device memory and streams) is loaded before this library.
    try:
        import torch  # noqa: F401
    except ImportError:
        pass
    lib = ctypes.CDLL(path)
    P, i32, i64, f32, f64 = (ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float,
                             ctypes.c_double)
    PP = ctypes.POINTER(Pool)
    sig = {
        "paged_kv_rope_table": ([f64, i32, P, P], ctypes.c_int),
        "paged_kv_append": ([PP, P, i64, P, i32, P, i64, P, i64, P, i64, P, P, i32, P],
                            ctypes.c_int),
        "paged_decode_attn_num_splits": ([i32, i32], i32),
        "paged_decode_attn_workspace_size": ([i32, i32], ctypes.c_size_t),
        "paged_decode_attn_workspace_init": ([P, ctypes.c_size_t, P], ctypes.c_int),
        "paged_decode_attn_order": ([P, i32, i32, P, P], ctypes.c_int),
        "paged_decode_attn_order_round": ([], i32),
        "paged_decode_attn_order_host": ([P, i32, i32, i32, P], ctypes.c_int),
        "paged_decode_attn": ([PP, P, i64, P, P, i32, i32, P, i64, f32, P, i64, P,
                               ctypes.c_size_t, P], ctypes.c_int),
        "paged_decode_attn_split": ([PP, P, i64, P, P, i32, i32, P, i64, f32, P, i64, P,
                                     ctypes.c_size_t, P], ctypes.c_int),
        "paged_decode_attn_combine": ([P, i32, i32, P, i64, P, ctypes.c_size_t, P], ctypes.c_int),
        "paged_kv_append_decode_attn": ([PP, P, i64, P, P, i32, i32, P, i64, P, i64, P, i64, P,
                                         P, i32, f32, P, i64, P, ctypes.c_size_t, P],
                                        ctypes.c_int),
        "paged_kv_append_decode_attn_noalloc": ([PP, P, i64, P, P, i32, i32, P, i64, P, i64, P,
                                                 i64, P, P, i32, f32, P, i64, P], ctypes.c_int),
        "paged_kv_prefill": ([PP, P, i64, P, P, i32, i32, P, i64, P, i64, P, i64, P, P, i32, P],
                             ctypes.c_int),
        "paged_kv_copy_pages": ([PP, P, P, i32, P], ctypes.c_int),
        "paged_kv_status_string": ([ctypes.c_int], ctypes.c_char_p),
        "paged_kv_free_list_create": ([P, i64, i64, ctypes.POINTER(P)], ctypes.c_int),
        "paged_kv_free_list_destroy": ([P], None),
        "paged_kv_free_list_pop": ([P, ctypes.POINTER(i32)], ctypes.c_int),
        "paged_kv_free_list_push": ([P, i32], ctypes.c_int),
        "paged_kv_free_list_stats": ([P, ctypes.POINTER(i64), ctypes.POINTER(i64),
                                      ctypes.POINTER(i64)], ctypes.c_int),
        "paged_kv_lazy_page_step": ([P, P, i32, i32, i64, P, P, ctypes.POINTER(i32)],
                                    ctypes.c_int),
        "paged_kv_pager_create": ([i32, i32, i32, ctypes.POINTER(P)], ctypes.c_int),
        "paged_kv_pager_destroy": ([P], None),
        "paged_kv_pager_submit": ([P, i32, i32, ctypes.POINTER(i64), ctypes.POINTER(i32)],
                                  ctypes.c_int),
        "paged_kv_pager_admit": ([P, P, i32, ctypes.POINTER(i32)], ctypes.c_int),
        "paged_kv_pager_reserve": ([P, i64, i32, P, i64, P, P, ctypes.POINTER(i32)],
                                   ctypes.c_int),
        "paged_kv_pager_decode_step": ([P, P, P, i32, P, i64, i64, P, P, ctypes.POINTER(i32)],
                                       ctypes.c_int),
        "paged_kv_pager_share_prefix": ([P, i64, i64, i32, P, i64], ctypes.c_int),
        "paged_kv_pager_finish": ([P, i64], ctypes.c_int),
        "paged_kv_pager_get_stats": ([P, ctypes.POINTER(PagerStats)], ctypes.c_int),
    }
    for name, (args, res) in sig.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = res
    _lib = lib
    return lib


def _p(x):
    """Device pointer of a tensor-like (data_ptr()) or a plain int, as an int
    (the declared c_void_p arguments take ints); None -> NULL."""
    if x is None or type(x) is int:
        return x
    dp = getattr(x, "data_ptr", None)
    return dp() if dp is not None else int(x)


def _stream(stream):
    """A stream object (cuda_stream), a raw handle (int) or None (NULL)."""
    if stream is None or type(stream) is int:
        return stream
    cs = getattr(stream, "cuda_stream", None)
    return cs if cs is not None else int(stream)


def _check(status: int, where: str) -> int:
    if status != PKV_OK:
        raise PagedKVError(status, where)
    return status


def status_string(status: int) -> str:
    return load().paged_kv_status_string(int(status)).decode()


def make_pool(k_pool, v_pool, num_pages, page_stride, head_stride, slot_stride) -> Pool:
    return Pool(_p(k_pool), _p(v_pool),
                int(num_pages), int(page_stride), int(head_stride), int(slot_stride))


def paged_kv_rope_table(theta: float, max_pos: int, cos_out, sin_out) -> None:
    """cos_out/sin_out: host buffers (numpy float32 [max_pos][32] or addresses)."""
    def hp(a):
        if a is None:
            return None
        if hasattr(a, "ctypes"):
            return a.ctypes.data_as(ctypes.c_void_p)
        return ctypes.c_void_p(int(a))
    _check(load().paged_kv_rope_table(float(theta), int(max_pos), hp(cos_out), hp(sin_out)),
           "paged_kv_rope_table")


def paged_kv_append(pool: Pool, block_table, bt_stride, context_lens, num_seqs, q, q_stride,
                    k_new, k_stride, v_new, v_stride, rope_cos, rope_sin, max_pos,
                    stream=None) -> None:
    _check(load().paged_kv_append(
        ctypes.byref(pool), _p(block_table), int(bt_stride), _p(context_lens), int(num_seqs),
        _p(q), int(q_stride), _p(k_new), int(k_stride), _p(v_new), int(v_stride),
        _p(rope_cos), _p(rope_sin), int(max_pos), _stream(stream)), "paged_kv_append")


def paged_decode_attn_num_splits(num_seqs: int, max_context_len: int) -> int:
    return int(load().paged_decode_attn_num_splits(int(num_seqs), int(max_context_len)))


def paged_decode_attn_workspace_size(num_seqs: int, max_context_len: int) -> int:
    return int(load().paged_decode_attn_workspace_size(int(num_seqs), int(max_context_len)))


def paged_decode_attn_workspace_init(workspace, workspace_bytes, stream=None) -> None:
    _check(load().paged_decode_attn_workspace_init(_p(workspace), int(workspace_bytes),
                                                   _stream(stream)),
           "paged_decode_attn_workspace_init")


def paged_decode_attn_order(context_lens, num_seqs, max_context_len, seq_order,
                            stream=None) -> None:
    _check(load().paged_decode_attn_order(_p(context_lens), int(num_seqs), int(max_context_len),
                                          _p(seq_order), _stream(stream)),
           "paged_decode_attn_order")


def paged_decode_attn_order_round() -> int:
    return int(load().paged_decode_attn_order_round())


def paged_decode_attn_order_host(context_lens, max_context_len, round_len):
    """The start order on the host: context_lens is a host int32 array;
    returns the int32 order array."""
    import numpy as np
    ctx = np.ascontiguousarray(context_lens, np.int32)
    out = np.empty(ctx.size, np.int32)
    _check(load().paged_decode_attn_order_host(ctx.ctypes.data, int(ctx.size), int(max_context_len),
                                                int(round_len), out.ctypes.data),
           "paged_decode_attn_order_host")
    return out


def _attn_args(pool, block_table, bt_stride, context_lens, seq_order, num_seqs, max_context_len,
               q, q_stride, scale, out, out_stride, workspace, workspace_bytes, stream):
    return (ctypes.byref(pool), _p(block_table), int(bt_stride), _p(context_lens), _p(seq_order),
            int(num_seqs), int(max_context_len), _p(q), int(q_stride), float(scale), _p(out),
            int(out_stride), _p(workspace), int(workspace_bytes), _stream(stream))


def paged_decode_attn(pool: Pool, block_table, bt_stride, context_lens, num_seqs,
                      max_context_len, q, q_stride, scale, out, out_stride, workspace=None,
                      workspace_bytes=0, stream=None, seq_order=None) -> None:
    """seq_order (the C argument after context_lens) is a keyword here."""
    _check(load().paged_decode_attn(*_attn_args(
        pool, block_table, bt_stride, context_lens, seq_order, num_seqs, max_context_len, q,
        q_stride, scale, out, out_stride, workspace, workspace_bytes, stream)),
        "paged_decode_attn")


def paged_decode_attn_split(pool: Pool, block_table, bt_stride, context_lens, num_seqs,
                            max_context_len, q, q_stride, scale, out, out_stride, workspace=None,
                            workspace_bytes=0, stream=None, seq_order=None) -> None:
    _check(load().paged_decode_attn_split(*_attn_args(
        pool, block_table, bt_stride, context_lens, seq_order, num_seqs, max_context_len, q,
        q_stride, scale, out, out_stride, workspace, workspace_bytes, stream)),
        "paged_decode_attn_split")


def paged_decode_attn_combine(context_lens, num_seqs, max_context_len, out, out_stride,
                              workspace=None, workspace_bytes=0, stream=None) -> None:
    _check(load().paged_decode_attn_combine(
        _p(context_lens), int(num_seqs), int(max_context_len), _p(out), int(out_stride),
        _p(workspace), int(workspace_bytes), _stream(stream)), "paged_decode_attn_combine")


def paged_kv_append_decode_attn(pool: Pool, block_table, bt_stride, context_lens, num_seqs,
                                max_context_len, q, q_stride, k_new, k_stride, v_new, v_stride,
                                rope_cos, rope_sin, max_pos, scale, out, out_stride,
                                workspace=None, workspace_bytes=0, stream=None,
                                seq_order=None) -> None:
    _check(load().paged_kv_append_decode_attn(
        ctypes.byref(pool), _p(block_table), int(bt_stride), _p(context_lens), _p(seq_order),
        int(num_seqs),
        int(max_context_len), _p(q), int(q_stride), _p(k_new), int(k_stride), _p(v_new),
        int(v_stride), _p(rope_cos), _p(rope_sin), int(max_pos), float(scale), _p(out),
        int(out_stride), _p(workspace), int(workspace_bytes), _stream(stream)),
        "paged_kv_append_decode_attn")


def paged_kv_append_decode_attn_noalloc(pool: Pool, block_table, bt_stride, context_lens,
                                        num_seqs, max_context_len, q, q_stride, k_new, k_stride,
                                        v_new, v_stride, rope_cos, rope_sin, max_pos, scale, out,
                                        out_stride, stream=None, seq_order=None) -> None:
    _check(load().paged_kv_append_decode_attn_noalloc(
        ctypes.byref(pool), _p(block_table), int(bt_stride), _p(context_lens), _p(seq_order),
        int(num_seqs),
        int(max_context_len), _p(q), int(q_stride), _p(k_new), int(k_stride), _p(v_new),
        int(v_stride), _p(rope_cos), _p(rope_sin), int(max_pos), float(scale), _p(out),
        int(out_stride), _stream(stream)), "paged_kv_append_decode_attn_noalloc")


def paged_kv_prefill(pool: Pool, block_table, bt_stride, start_pos, cu_tokens, num_seqs,
                     total_tokens, q, q_stride, k_new, k_stride, v_new, v_stride, rope_cos,
                     rope_sin, max_pos, stream=None) -> None:
    """q may be None (K/V only)."""
    _check(load().paged_kv_prefill(
        ctypes.byref(pool), _p(block_table), int(bt_stride), _p(start_pos), _p(cu_tokens),
        int(num_seqs), int(total_tokens), _p(q), int(q_stride), _p(k_new), int(k_stride),
        _p(v_new), int(v_stride), _p(rope_cos), _p(rope_sin), int(max_pos), _stream(stream)),
        "paged_kv_prefill")


def paged_kv_copy_pages(pool: Pool, src, dst, num_pairs, stream=None) -> None:
    _check(load().paged_kv_copy_pages(ctypes.byref(pool), _p(src), _p(dst), int(num_pairs),
                                      _stream(stream)), "paged_kv_copy_pages")
