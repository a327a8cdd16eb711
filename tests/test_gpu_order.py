"""GPU: the start order of a mixed-length batch (paged_decode_attn_order) and
the attention calls that follow it.

The ranking is index work, so the bar is bit-exact: seq_order must equal the
stable descending sort of the page counts ceil(min(ctx, max_context_len)/16)
(numpy's stable argsort on the host, ties in batch order), placed by the
documented start positions when the batch holds a whole first round of R
sequences (R from paged_decode_attn_order_round).  The order only
decides which workgroups start first, so every attention call (plain, split,
fused, allocation-free) must give the same output and pool bits with and
without it, on batches whose grid exceeds what the GPU holds at once (so the
order is actually followed); and an order whose entries are all out of range
(each rank then serves itself) must too.
"""
import numpy as np
import pytest

import paged_kv_cache_172_amd as pkv
from paged_kv_cache_172_amd import workload as wl

from tests.gpu_util import host_batch, say
from tests.order_ref import host_rank

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def torch_gpu():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU (run with -m 'not gpu' on CPU)"
    pkv.load()
    return torch


@pytest.fixture(scope="module")
def rope():
    from paged_kv_cache_172_amd.runner import rope_table_host
    return rope_table_host()


ORDER_CASES = {
    "one": ([37], 2048),
    "config4": (None, 2048),
    "two_rounds_1025": ("rand1025", 2048),
    "many_5000": ("rand5000", 2048),
    "all_equal_300": ([2048] * 300, 2048),
    "one_round_128": ("rand128", 2048),
    "one_short_of_a_round_127": ("rand127", 2048),
    "round_and_a_quarter_160": ("rand160", 2048),
    "clamped_and_empty": ([0, -3, 5000, 2048, 17, 16, 1, 0, 3000, 33] * 7, 700),
}


@pytest.mark.parametrize("name", list(ORDER_CASES))
def test_order_is_the_stable_descending_sort(torch_gpu, name):
    torch = torch_gpu
    lens, mcl = ORDER_CASES[name]
    rng = np.random.default_rng(880)
    if lens is None:
        lens = wl.config_spec(4).ctx
    elif isinstance(lens, str):
        lens = rng.integers(-5, 2200, int(lens[4:]))
    ctx = np.asarray(lens, np.int32)
    dev_ctx = torch.from_numpy(ctx).cuda()
    out = torch.full((ctx.size,), -7, dtype=torch.int32, device="cuda")
    pkv.paged_decode_attn_order(dev_ctx, ctx.size, mcl, out)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    R = pkv.paged_decode_attn_order_round()
    assert R >= 2 and R % 2 == 0, R
    want = host_rank(ctx, mcl, R)
    say(f"[order] {name}: B={ctx.size}, round {R}")
    assert np.array_equal(got, want), (name, got[:16], want[:16])
    # the library's host order is the same, entry for entry
    assert np.array_equal(pkv.paged_decode_attn_order_host(ctx, mcl, R), got), name


def _outputs(torch, b, how, seq_order):
    """Run one layer of batch b with the given call and order; return
    (out, pool) copies.  The plain and split calls get the append first
    (the new token's slot holds NaN until it is written)."""
    if how in ("attn", "split"):
        b.append(0)
    if how == "attn":
        pkv.paged_decode_attn(b.pool, b.block_tables[0], b.bt_stride, b.context_lens, b.num_seqs,
                              b.max_context_len, b.q[0], 2048, b.scale, b.out[0], 2048, b.workspace,
                              b.ws_bytes, seq_order=seq_order)
    elif how == "split":
        pkv.paged_decode_attn_split(b.pool, b.block_tables[0], b.bt_stride, b.context_lens,
                                    b.num_seqs, b.max_context_len, b.q[0], 2048, b.scale, b.out[0],
                                    2048, b.workspace, b.ws_bytes, seq_order=seq_order)
        pkv.paged_decode_attn_combine(b.context_lens, b.num_seqs, b.max_context_len, b.out[0], 2048,
                                      b.workspace, b.ws_bytes)
    else:
        fn = pkv.paged_kv_append_decode_attn if how == "fused" else \
            pkv.paged_kv_append_decode_attn_noalloc
        args = (b.pool, b.block_tables[0], b.bt_stride, b.context_lens, b.num_seqs,
                b.max_context_len, b.q[0], 2048, b.k[0], 512, b.v[0], 512, b.rope_cos, b.rope_sin,
                b.max_pos, b.scale, b.out[0], 2048)
        if how == "fused":
            fn(*args, b.workspace, b.ws_bytes, seq_order=seq_order)
        else:
            fn(*args, seq_order=seq_order)
    torch.cuda.synchronize()
    return b.out[0].clone(), b.pool_pages.clone()


@pytest.mark.parametrize("how", ["attn", "split", "fused", "noalloc"])
def test_order_changes_no_bit(torch_gpu, rope, how):
    """1,500 sequences of log-uniform lengths (12,000 workgroups: more than
    the GPU holds at once), one layer: the same bits in batch order, in the
    library's order, in a random order, and with every entry out of range."""
    torch = torch_gpu
    rng = np.random.default_rng(881)
    lengths = np.clip(np.rint(np.exp(rng.uniform(np.log(16), np.log(2048), 1500))), 16,
                      2048).astype(int)
    spec = wl.make_spec(lengths, 1, seed=881)
    hw = wl.make_host_workload(spec)
    B = spec.num_seqs
    ranked = torch.empty(B, dtype=torch.int32, device="cuda")
    results = {}
    for name in ("none", "library", "random", "out_of_range"):
        b = host_batch(hw, rope)
        if name == "library":
            pkv.paged_decode_attn_order(b.context_lens, B, b.max_context_len, ranked)
            order = ranked
        elif name == "random":
            order = torch.from_numpy(rng.permutation(B).astype(np.int32)).cuda()
        elif name == "out_of_range":
            order = torch.full((B,), B + 5, dtype=torch.int32, device="cuda")
        else:
            order = None
        results[name] = _outputs(torch, b, how, order)
        del b
    say(f"[order] {how}: B={B} grid={B * 8} workgroups")
    out0, pool0 = results["none"]
    assert torch.isfinite(out0).all()
    for name, (out, pool) in results.items():
        assert torch.equal(out.view(torch.int32), out0.view(torch.int32)), (how, name)
        assert torch.equal(pool, pool0), (how, name)
    assert np.array_equal(ranked.cpu().numpy(),
                          host_rank(spec.ctx, spec.ctx.max(), pkv.paged_decode_attn_order_round()))


def test_issue_priority_changes_no_bit(torch_gpu, rope):
    """Waves take their issue priority from their pages left only in launches
    of at most two rounds of resident workgroups.  The same 64 sequences, alone
    (512 workgroups: priority on) and as the first rows of a 1,024-sequence
    batch (8,192 workgroups: priority off), must give the same output bits,
    for the plain and the fused call."""
    torch = torch_gpu
    from paged_kv_cache_172_amd.runner import DecodeBatch
    rng = np.random.default_rng(990)
    lens = rng.integers(1, 300, 1024)
    lens[::97] = 2048
    spec = wl.make_spec(lens, 1, seed=990)
    pool = wl.make_device_pool(spec)
    q0, k0, v0 = wl.draw_new_tokens(spec)
    big = DecodeBatch(pool, spec.block_tables, spec.ctx, q0, k0, v0, rope=rope, max_context_len=2048)
    small = DecodeBatch(big.pool_pages, spec.block_tables[:, :64], spec.ctx[:64], q0[:, :64],
                        k0[:, :64], v0[:, :64], rope=rope, max_context_len=2048)
    assert big.pool_pages.data_ptr() == small.pool_pages.data_ptr()
    assert big.splits == small.splits == 1
    # the fused call first: it writes each new token's K/V row, which the
    # device pool leaves NaN until then
    for how in ("fused", "attn"):
        say(f"[priority] {how}: B=1024 against its first 64 sequences")
        for b in (big, small):
            b.out.fill_(float("nan"))
            if how == "attn":
                b.attn(0)
            else:
                b.append_attn(0)
        torch.cuda.synchronize()
        got_big = big.out[0, :64].view(torch.int32)
        got_small = small.out[0].view(torch.int32)
        assert torch.equal(got_big, got_small), how
        assert torch.isfinite(small.out[0]).all(), how
