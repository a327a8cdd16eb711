"""Device buffers of one decode batch and the calls of one decode step.

``DecodeBatch`` owns, in device memory, the page pool, the per-layer block
tables, the context lengths, the new-token q/k/v rows of every layer, the RoPE
table, one FP32 output row set per layer and the split workspace -- all
allocated once up front and reused ("Tiny-vLLMでゼロから構築する高性能LLM推論
エンジン", section "GPUメモリ管理").  ``step()`` runs, layer by layer, the
append then the attention on one stream.  torch is used for device memory
and streams only; every computation runs in libpagedkv.so.
"""
from __future__ import annotations

import numpy as np

from . import _lib

Q_ROW = 32 * 64
KV_ROW = 8 * 64
PAGE_ELEMS = 2 * 8 * 16 * 64
HALF_PAGE = 8 * 16 * 64


def rope_table_host(theta: float = 500000.0, max_pos: int = 2048):
    cos = np.empty((max_pos, 32), np.float32)
    sin = np.empty((max_pos, 32), np.float32)
    _lib.paged_kv_rope_table(theta, max_pos, cos, sin)
    return cos, sin


def _to_dev_i16(a, device):
    import torch
    if isinstance(a, torch.Tensor):
        return a.to(device=device, dtype=torch.int16).contiguous()
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(device)


class DecodeBatch:
    def __init__(self, pool_pages, block_tables, context_lens, q, k, v, *, rope=None,
                 scale: float = 0.125, max_context_len: int | None = None, device="cuda"):
        """pool_pages: int16/uint16 [P][2][8][16][64] (tensor on device or numpy);
        block_tables: int32 [L][B][W]; context_lens: int32 [B];
        q/k/v: uint16 [L][B][2048 | 512 | 512]; rope: optional (cos, sin) FP32
        [max_pos][32] host tables (default: paged_kv_rope_table(500000, 2048))."""
        import torch
        self.device = torch.device(device)
        self.pool_pages = _to_dev_i16(pool_pages, self.device)
        P = self.pool_pages.shape[0]
        self.num_pages = P
        bt = np.ascontiguousarray(block_tables, np.int32)
        self.num_layers, self.num_seqs, self.bt_stride = bt.shape
        self.block_tables = torch.from_numpy(bt).to(self.device)
        self.context_lens_host = np.ascontiguousarray(context_lens, np.int32).copy()
        self.context_lens = torch.from_numpy(self.context_lens_host).to(self.device)
        self.q = _to_dev_i16(q, self.device)
        self.k = _to_dev_i16(k, self.device)
        self.v = _to_dev_i16(v, self.device)
        cos, sin = rope if rope is not None else rope_table_host()
        self.max_pos = cos.shape[0]
        self.rope_cos = torch.from_numpy(np.ascontiguousarray(cos, np.float32)).to(self.device)
        self.rope_sin = torch.from_numpy(np.ascontiguousarray(sin, np.float32)).to(self.device)
        self.scale = float(scale)
        mcl = int(self.context_lens_host.max()) if max_context_len is None else int(max_context_len)
        self.max_context_len = max(1, mcl)
        self.out = torch.zeros((self.num_layers, self.num_seqs, Q_ROW), dtype=torch.float32,
                               device=self.device)
        self.ws_bytes = _lib.paged_decode_attn_workspace_size(self.num_seqs, self.max_context_len)
        self.workspace = torch.empty(max(self.ws_bytes, 16), dtype=torch.uint8, device=self.device)
        _lib.paged_decode_attn_workspace_init(self.workspace, self.ws_bytes,
                                              torch.cuda.current_stream(self.device))
        base = self.pool_pages.data_ptr()
        self.pool = _lib.make_pool(base, base + HALF_PAGE * 2, P, PAGE_ELEMS, 16 * 64, 64)
        # start order of the sequences (paged_decode_attn_order), used by the
        # attention calls once order() has run
        self.seq_order = torch.empty(self.num_seqs, dtype=torch.int32, device=self.device)
        self.ordered = False
        # Every device address a call passes, as a plain int, per layer where
        # it depends on the layer: the buffers above never move, and a call
        # then costs the host no tensor indexing.
        def rows(t):
            step = t.stride(0) * t.element_size()
            return [t.data_ptr() + layer * step for layer in range(t.shape[0])]
        self._bt = rows(self.block_tables)
        self._q, self._k, self._v, self._out = rows(self.q), rows(self.k), rows(self.v), rows(self.out)
        self._ctx = self.context_lens.data_ptr()
        self._ws = self.workspace.data_ptr()
        self._order_ptr = self.seq_order.data_ptr()
        self._cos, self._sin = self.rope_cos.data_ptr(), self.rope_sin.data_ptr()

    @property
    def splits(self) -> int:
        return _lib.paged_decode_attn_num_splits(self.num_seqs, self.max_context_len)

    def upload_tables(self, block_tables: np.ndarray, rows=None) -> None:
        """Copy changed table rows (all when rows is None) and the lengths."""
        import torch
        bt = np.ascontiguousarray(block_tables, np.int32)
        if rows is None:
            self.block_tables.copy_(torch.from_numpy(bt))
        else:
            for s in rows:
                self.block_tables[:, s].copy_(torch.from_numpy(np.ascontiguousarray(bt[:, s])))
        self.context_lens.copy_(torch.from_numpy(self.context_lens_host))

    def _stream(self, stream):
        if stream is not None:
            return stream
        import torch
        return torch.cuda.current_stream(self.device)

    def order(self, stream=None) -> None:
        """Rank the sequences once for this step's attention calls (longest
        first); every later attention call of this batch starts them in that
        order."""
        _lib.paged_decode_attn_order(self._ctx, self.num_seqs, self.max_context_len,
                                     self._order_ptr, self._stream(stream))
        self.ordered = True

    def _order(self):
        return self._order_ptr if self.ordered else None

    def append(self, layer: int, stream=None) -> None:
        _lib.paged_kv_append(
            self.pool, self._bt[layer], self.bt_stride, self._ctx, self.num_seqs,
            self._q[layer], Q_ROW, self._k[layer], KV_ROW, self._v[layer], KV_ROW,
            self._cos, self._sin, self.max_pos, self._stream(stream))

    def attn(self, layer: int, stream=None) -> None:
        _lib.paged_decode_attn(
            self.pool, self._bt[layer], self.bt_stride, self._ctx, self.num_seqs,
            self.max_context_len, self._q[layer], Q_ROW, self.scale, self._out[layer], Q_ROW,
            self._ws, self.ws_bytes, self._stream(stream), seq_order=self._order())

    def attn_split(self, layer: int, stream=None) -> None:
        _lib.paged_decode_attn_split(
            self.pool, self._bt[layer], self.bt_stride, self._ctx, self.num_seqs,
            self.max_context_len, self._q[layer], Q_ROW, self.scale, self._out[layer], Q_ROW,
            self._ws, self.ws_bytes, self._stream(stream), seq_order=self._order())

    def attn_combine(self, layer: int, stream=None) -> None:
        _lib.paged_decode_attn_combine(
            self._ctx, self.num_seqs, self.max_context_len, self._out[layer], Q_ROW,
            self._ws, self.ws_bytes, self._stream(stream))

    def append_attn(self, layer: int, stream=None) -> None:
        """The fused append + attention of one layer (q is left unrotated)."""
        _lib.paged_kv_append_decode_attn(
            self.pool, self._bt[layer], self.bt_stride, self._ctx, self.num_seqs,
            self.max_context_len, self._q[layer], Q_ROW, self._k[layer], KV_ROW,
            self._v[layer], KV_ROW, self._cos, self._sin, self.max_pos, self.scale,
            self._out[layer], Q_ROW, self._ws, self.ws_bytes, self._stream(stream),
            seq_order=self._order())

    def step(self, stream=None) -> None:
        """One decode step: for every layer, append then attention."""
        for layer in range(self.num_layers):
            self.append(layer, stream)
            self.attn(layer, stream)

    def step_fused(self, stream=None, order: bool = False) -> None:
        """One decode step with the fused call per layer; with order, the
        sequences are ranked once first (paged_decode_attn_order)."""
        if order:
            self.order(stream)
        for layer in range(self.num_layers):
            self.append_attn(layer, stream)
