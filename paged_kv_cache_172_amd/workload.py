"""Seeded synthetic workloads for the paged BF16 KV-cache decode step.

This module draws random numbers and lays them out in the page pool; it holds
none of the method's arithmetic (no RoPE, no dot products, no softmax).  It is
the one module that both the oracle-side tests and the GPU side use for inputs.

Shapes follow the pages: the Llama-3.2-1B attention geometry (32 query heads,
8 KV heads, head_dim 64), a fixed 2,048-token context, 16 layers, and a pool
of 16-token physical pages shared by every sequence and layer with one block
table per (sequence, layer) ("Hours of YouTube and 85 handtyped pages of notes
on LLM Inference - Start here", sections "これまでの進捗" and "現在のスコープ").
No public benchmark or dataset is involved.

Layout convention of the pool built here (the format both sides read):
  page p holds [K | V][kv head 8][slot 16][dim 64] BF16 bits (32 KiB);
  logical token t of (sequence s, layer l) sits in page block_table[l][s][t div 16],
  slot t mod 16.  Unused slots, free pages and table tails are poisoned
  (BF16 quiet NaN 0x7FC0, table entry -1).

Draw order from numpy PCG64(seed): lengths -> placement -> new-token q, k, v
rows (layer-major, then sequence) -> outlier mask of the new k -> cached K
(layer-major, sequence, token) -> cached V -> outlier masks of cached K.
Large pools (configs 3-5) draw the cached K/V on the GPU from a torch
generator seeded with the same seed instead; their new-token rows still come
from the numpy stream above.
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np

NUM_Q_HEADS = 32
NUM_KV_HEADS = 8
HEAD_DIM = 64
PAGE_TOKENS = 16
MAX_CONTEXT = 2048
NUM_LAYERS = 16
ROPE_THETA = 500000.0
SCALE = 0.125                      # 1/sqrt(64)
BF16_NAN = 0x7FC0
PAGE_ELEMS = 2 * NUM_KV_HEADS * PAGE_TOKENS * HEAD_DIM   # 16384 BF16 = 32 KiB
BT_STRIDE = MAX_CONTEXT // PAGE_TOKENS                    # 128 table entries
Q_ROW = NUM_Q_HEADS * HEAD_DIM                            # 2048
KV_ROW = NUM_KV_HEADS * HEAD_DIM                          # 512
SEED_BASE = 172000

CONFIG_NAMES = {
    1: "tiny: 1 seq x 1 layer, ctx 37, 64-page pool",
    2: "batch 8 x 1 layer, ctx in [1,2048] with 1/16/17",
    3: "batch 64 x 16 layers, ctx 2048 (4 GiB KV)",
    4: "continuous batching: 256 seqs x 16 layers, log-uniform ctx, 16 page crossers",
    5: "stress: 1024 seqs x ctx 2048 x 1 layer, K outliers x30, q x4, 25% free pages",
}


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round FP32 draws to BF16 bit patterns with torch's conversion
    (round to nearest even), returned as uint16."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16).copy()


def _pages_for(n_tokens: int) -> int:
    return -(-int(n_tokens) // PAGE_TOKENS) if n_tokens > 0 else 0


@dataclasses.dataclass
class Spec:
    """What a workload is made of, before any value is drawn."""
    index: int                       # config number, 0 for ad-hoc workloads
    seed: int
    ctx: np.ndarray                  # int32 [B], context length AFTER the append
    num_layers: int
    num_pages: int
    block_tables: np.ndarray         # int32 [L][B][BT_STRIDE]
    free_pages: np.ndarray           # int32, pop order (front first)
    crossers: np.ndarray             # int32 sequence ids whose new token needs a new page
    q_mult: float = 1.0
    k_outlier_p: float = 0.0
    k_outlier_mult: float = 30.0
    rng_state: dict | None = None    # numpy bit-generator state after lengths+placement

    @property
    def num_seqs(self) -> int:
        return int(self.ctx.shape[0])

    @property
    def name(self) -> str:
        return CONFIG_NAMES.get(self.index, "ad-hoc")

    def kv_bytes_per_step(self) -> int:
        """Algorithmic KV bytes read by attention: K and V of valid tokens."""
        return int(self.ctx.astype(np.int64).sum()) * self.num_layers * 2 * KV_ROW * 2


# ----------------------------------------------------------------- specs --

def _finish_placement(rng, ctx, num_layers, held_counts, num_pages, interleave_free=True):
    """Assign distinct physical pages to every held (layer, seq, logical page)
    from one seeded permutation of the pool; the rest is the free list."""
    B = ctx.shape[0]
    perm = rng.permutation(num_pages).astype(np.int32)
    bt = np.full((num_layers, B, BT_STRIDE), -1, np.int32)
    cursor = 0
    for l in range(num_layers):
        for s in range(B):
            c = int(held_counts[l, s])
            bt[l, s, :c] = perm[cursor:cursor + c]
            cursor += c
    return bt, perm[cursor:].copy()


def make_spec(lengths, num_layers: int = 1, seed: int = SEED_BASE, extra_free: int = 0,
              crossers_lazy: bool = False, q_mult: float = 1.0, k_outlier_p: float = 0.0,
              index: int = 0, rng=None) -> Spec:
    """Ad-hoc workload: every (layer, seq) holds pages for its ctx tokens.

    crossers_lazy: sequences whose new token opens a new page (ctx-1 divisible
    by 16) do not hold that page yet; it comes from the free list later."""
    rng = np.random.Generator(np.random.PCG64(seed)) if rng is None else rng
    ctx = np.asarray(lengths, np.int32).copy()
    B = ctx.shape[0]
    held = np.zeros((num_layers, B), np.int64)
    crossers = []
    for s in range(B):
        n = int(ctx[s])
        need = _pages_for(n)
        if crossers_lazy and n >= 1 and (n - 1) % PAGE_TOKENS == 0:
            need -= 1
            crossers.append(s)
        held[:, s] = need
    n_cross_pages = len(crossers) * num_layers
    num_pages = int(held.sum()) + n_cross_pages + int(extra_free)
    bt, free = _finish_placement(rng, ctx, num_layers, held, max(num_pages, 1))
    return Spec(index=index, seed=seed, ctx=ctx, num_layers=num_layers,
                num_pages=max(num_pages, 1), block_tables=bt, free_pages=free,
                crossers=np.asarray(crossers, np.int32), q_mult=q_mult,
                k_outlier_p=k_outlier_p, rng_state=rng.bit_generator.state)


def config_spec(k: int) -> Spec:
    """The five workload configurations."""
    seed = SEED_BASE + k
    rng = np.random.Generator(np.random.PCG64(seed))
    if k == 1:
        ctx = np.array([37], np.int32)
        num_pages = 64
        perm = rng.permutation(num_pages).astype(np.int32)
        bt = np.full((1, 1, BT_STRIDE), -1, np.int32)
        bt[0, 0, :3] = perm[:3]
        return Spec(1, seed, ctx, 1, num_pages, bt, perm[3:].copy(),
                    np.zeros(0, np.int32), rng_state=rng.bit_generator.state)
    if k == 2:
        ctx = np.empty(8, np.int32)
        ctx[:3] = [1, 16, 17]
        ctx[3:] = rng.integers(1, MAX_CONTEXT + 1, size=5)
        return make_spec(ctx, 1, seed, index=2, rng=rng)
    if k == 3:
        ctx = np.full(64, MAX_CONTEXT, np.int32)
        return make_spec(ctx, NUM_LAYERS, seed, index=3, rng=rng)
    if k == 4:
        B = 256
        u = rng.uniform(math.log(16), math.log(MAX_CONTEXT), size=B)
        ctx = np.clip(np.rint(np.exp(u)), 16, MAX_CONTEXT).astype(np.int32)
        cross = rng.choice(B, size=16, replace=False)
        is_cross = np.zeros(B, bool)
        is_cross[cross] = True
        for s in range(B):
            if is_cross[s]:
                kk = max((int(ctx[s]) - 1) // PAGE_TOKENS, 1)
                ctx[s] = kk * PAGE_TOKENS + 1
            elif (int(ctx[s]) - 1) % PAGE_TOKENS == 0:
                ctx[s] += 1
        held = int(sum(_pages_for(int(n) - 1) for n in ctx)) * NUM_LAYERS
        slack = (held + 16 * NUM_LAYERS) // 10
        return make_spec(ctx, NUM_LAYERS, seed, extra_free=slack, crossers_lazy=True,
                         index=4, rng=rng)
    if k == 5:
        ctx = np.full(1024, MAX_CONTEXT, np.int32)
        used = 1024 * BT_STRIDE
        free = 174763 - used
        return make_spec(ctx, 1, seed, extra_free=free, q_mult=4.0, k_outlier_p=1e-3,
                         index=5, rng=rng)
    raise ValueError(f"unknown config {k}")


# ------------------------------------------------------------ host values --

@dataclasses.dataclass
class HostWorkload:
    spec: Spec
    pages: np.ndarray        # uint16 [num_pages][2][8][16][64]
    q: np.ndarray            # uint16 [L][B][2048]   new token's q (before RoPE)
    k: np.ndarray            # uint16 [L][B][512]    new token's k (before RoPE)
    v: np.ndarray            # uint16 [L][B][512]
    k_cached: list           # [L][B] uint16 [ctx-1][8][64], logical order
    v_cached: list


def draw_bf16(rng, shape, mult: float = 1.0) -> np.ndarray:
    x = rng.standard_normal(shape, dtype=np.float32)
    if mult != 1.0:
        x = x * np.float32(mult)
    return f32_to_bf16_bits(x)


def make_host_workload(spec: Spec) -> HostWorkload:
    """Draw every value on the host (small and medium workloads)."""
    rng = np.random.Generator(np.random.PCG64(spec.seed))
    if spec.rng_state is not None:
        rng.bit_generator.state = spec.rng_state
    L, B = spec.num_layers, spec.num_seqs
    q, k, v = _draw_new_rows(rng, spec)
    k_cached_f, v_cached = [], []
    for l in range(L):
        k_cached_f.append([rng.standard_normal((max(int(n) - 1, 0), NUM_KV_HEADS, HEAD_DIM),
                                               dtype=np.float32) for n in spec.ctx])
    for l in range(L):
        v_cached.append([draw_bf16(rng, (max(int(n) - 1, 0), NUM_KV_HEADS, HEAD_DIM))
                         for n in spec.ctx])
    if spec.k_outlier_p > 0.0:
        m = np.float32(spec.k_outlier_mult)
        for l in range(L):
            for s in range(B):
                a = k_cached_f[l][s]
                k_cached_f[l][s] = np.where(rng.random(a.shape) < spec.k_outlier_p, a * m, a)
    k_cached = [[f32_to_bf16_bits(a) for a in row] for row in k_cached_f]

    pages = np.full((spec.num_pages, 2, NUM_KV_HEADS, PAGE_TOKENS, HEAD_DIM), BF16_NAN,
                    np.uint16)
    for l in range(L):
        for s in range(B):
            scatter_tokens(pages, spec.block_tables[l, s], k_cached[l][s], v_cached[l][s])
    return HostWorkload(spec, pages, q, k, v, k_cached, v_cached)


def scatter_tokens(pages, bt_row, k_tok, v_tok) -> None:
    """Write tokens 0..T-1 (arrays [T][8][64]) into their pages: token t goes
    to page bt_row[t div 16], slot t mod 16 (pages are [2][8][16][64])."""
    T = k_tok.shape[0]
    full = T // PAGE_TOKENS
    if full:
        idx = bt_row[:full]
        kk = k_tok[:full * PAGE_TOKENS].reshape(full, PAGE_TOKENS, NUM_KV_HEADS, HEAD_DIM)
        vv = v_tok[:full * PAGE_TOKENS].reshape(full, PAGE_TOKENS, NUM_KV_HEADS, HEAD_DIM)
        pages[idx, 0] = kk.transpose(0, 2, 1, 3)
        pages[idx, 1] = vv.transpose(0, 2, 1, 3)
    rem = T - full * PAGE_TOKENS
    if rem:
        p = bt_row[full]
        pages[p, 0, :, :rem] = k_tok[full * PAGE_TOKENS:].transpose(1, 0, 2)
        pages[p, 1, :, :rem] = v_tok[full * PAGE_TOKENS:].transpose(1, 0, 2)


# ---------------------------------------------------------- device values --

def make_device_pool(spec: Spec, device="cuda", chunk_pages: int = 8192):
    """Draw the cached K/V of a large workload directly in device memory.

    Every held page is filled with N(0,1) BF16 (K with the spec's outlier
    rule), then the slots that hold no cached token yet (the new token's slot
    and anything after it), every free page and every page no table uses are
    set to BF16 NaN.  Returns an int16 tensor [num_pages][2][8][16][64]."""
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(spec.seed)
    P = spec.num_pages
    pool = torch.empty((P, 2, NUM_KV_HEADS, PAGE_TOKENS, HEAD_DIM), dtype=torch.int16,
                       device=device)
    for a in range(0, P, chunk_pages):
        b = min(P, a + chunk_pages)
        x = torch.randn((b - a, 2, NUM_KV_HEADS, PAGE_TOKENS, HEAD_DIM), generator=g,
                        device=device, dtype=torch.float32)
        if spec.k_outlier_p > 0.0:
            u = torch.rand(x[:, 0].shape, generator=g, device=device)
            x[:, 0] = torch.where(u < spec.k_outlier_p, x[:, 0] * spec.k_outlier_mult, x[:, 0])
        pool[a:b] = x.to(torch.bfloat16).view(torch.int16)
        del x
    poison_device_pool(pool, spec)
    return pool


def poison_device_pool(pool, spec: Spec) -> None:
    import torch
    nan = BF16_NAN                   # 0x7FC0 fits a positive int16
    used = np.zeros(spec.num_pages, bool)
    tail_pages, tail_from = [], []
    for l in range(spec.num_layers):
        for s in range(spec.num_seqs):
            n_cached = max(int(spec.ctx[s]) - 1, 0)
            row = spec.block_tables[l, s]
            held = row[row >= 0]
            used[held] = True
            full = n_cached // PAGE_TOKENS
            if full < held.shape[0]:
                tail_pages.append(int(row[full]))
                tail_from.append(n_cached - full * PAGE_TOKENS)
    unused = np.nonzero(~used)[0]
    if unused.size:
        idx = torch.from_numpy(unused.astype(np.int64)).to(pool.device)
        pool.index_fill_(0, idx, nan)
    if tail_pages:
        tp = np.asarray(tail_pages, np.int64)
        tf = np.asarray(tail_from, np.int64)
        for start in np.unique(tf):
            sel = torch.from_numpy(tp[tf == start]).to(pool.device)
            view = pool.index_select(0, sel)
            view[:, :, :, int(start):] = nan
            pool.index_copy_(0, sel, view)


def _draw_new_rows(rng, spec: Spec):
    L, B = spec.num_layers, spec.num_seqs
    q = draw_bf16(rng, (L, B, Q_ROW), spec.q_mult)
    k_new = rng.standard_normal((L, B, KV_ROW), dtype=np.float32)
    v = draw_bf16(rng, (L, B, KV_ROW))
    if spec.k_outlier_p > 0.0:
        k_new = np.where(rng.random(k_new.shape) < spec.k_outlier_p,
                         k_new * np.float32(spec.k_outlier_mult), k_new)
    return q, f32_to_bf16_bits(k_new), v


def draw_new_tokens(spec: Spec):
    """New-token q/k/v rows [L][B][...] as uint16 BF16 bits, drawn on the host
    from the spec's generator state (cheap even for the large configs).  They
    equal the rows make_host_workload draws for the same spec."""
    rng = np.random.Generator(np.random.PCG64(spec.seed))
    if spec.rng_state is not None:
        rng.bit_generator.state = spec.rng_state
    return _draw_new_rows(rng, spec)
