"""MI355X-native decode step over a paged BF16 KV cache.

The product is ``libpagedkv.so`` (HIP kernels for gfx950 behind the C ABI in
``include/paged_kv.h``).  This package holds its sources (``csrc/``), the
build step (``build.py``), the thin ctypes binding (``_lib.py``, re-exported
here), the bindings of the native host page management (``pages.py``), and the
seeded synthetic workload generator (``workload.py``).
"""
from ._lib import (  # noqa: F401
    EXPORTED,
    LIB_PATH,
    PKV_ERR_ALIGNMENT,
    PKV_ERR_BUDGET,
    PKV_ERR_EXHAUSTED,
    PKV_ERR_HIP,
    PKV_ERR_INVALID_ARG,
    PKV_ERR_REJECTED,
    PKV_ERR_STATE,
    PKV_ERR_UNSUPPORTED,
    PKV_ERR_WORKSPACE,
    PKV_OK,
    PagedKVError,
    Pool,
    load,
    make_pool,
    paged_decode_attn,
    paged_decode_attn_combine,
    paged_decode_attn_num_splits,
    paged_decode_attn_order,
    paged_decode_attn_order_round,
    paged_decode_attn_order_host,
    paged_decode_attn_split,
    paged_decode_attn_workspace_init,
    paged_decode_attn_workspace_size,
    paged_kv_append,
    paged_kv_append_decode_attn,
    paged_kv_append_decode_attn_noalloc,
    paged_kv_prefill,
    paged_kv_copy_pages,
    paged_kv_rope_table,
    status_string,
)

NUM_Q_HEADS = 32
NUM_KV_HEADS = 8
HEAD_DIM = 64
PAGE_TOKENS = 16
MAX_CONTEXT = 2048
