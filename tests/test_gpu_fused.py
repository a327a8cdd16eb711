"""GPU parity of the fused call paged_kv_append_decode_attn.

It must give, bit for bit, the output and the pool of paged_kv_append
followed by paged_decode_attn on the same inputs (both checked against the
FP64 oracle elsewhere), leave q unrotated, and meet the oracle's attention
tolerance on its own.  Edge cases: new tokens past max_context_len, positions
outside the RoPE table, a bad page id for the new token, empty rows, and the
split + combine plan.
"""
import numpy as np
import pytest

import oracle
from oracle import PoolView
import paged_kv_cache_172_amd as pkv
from paged_kv_cache_172_amd import workload as wl
from paged_kv_cache_172_amd.runner import DecodeBatch

from tests.gpu_util import assert_attn_close, host_batch, say, to_u16
from tests.test_gpu_parity import SMALL

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def torch_gpu():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU (run with -m 'not gpu' on CPU)"
    pkv.load()
    return torch


@pytest.fixture(scope="module")
def orc():
    return oracle.default()


@pytest.fixture(scope="module")
def rope(orc):
    return orc.rope_table(500000.0, 2048)


def same_bits(torch, a, b) -> bool:
    """Bitwise equality of two tensors; for FP32, NaN must sit in the same
    places in both (its payload may differ: a row that reads a bad page id
    is NaN whichever way the NaN arose)."""
    if a.dtype != torch.float32:
        return bool(torch.equal(a, b))
    na, nb = torch.isnan(a), torch.isnan(b)
    if not torch.equal(na, nb):
        return False
    keep = ~na
    return bool(torch.equal(a[keep].view(torch.int32), b[keep].view(torch.int32)))


def run_both(torch, make_batch, num_layers):
    """Two batches built from the same inputs: append + attention on one,
    the fused call on the other."""
    sep, fus = make_batch(), make_batch()
    q_before = fus.q.clone()
    for layer in range(num_layers):
        sep.append(layer)
        sep.attn(layer)
        fus.append_attn(layer)
    torch.cuda.synchronize()
    assert same_bits(torch, fus.q, q_before), "the fused call must leave q as given"
    return sep, fus


@pytest.mark.parametrize("name", list(SMALL))
def test_fused_equals_append_then_attn(torch_gpu, rope, name):
    torch = torch_gpu
    spec = SMALL[name]()
    hw = wl.make_host_workload(spec)
    sep, fus = run_both(torch, lambda: host_batch(hw, rope), spec.num_layers)
    say(f"[fused] {name}: B={spec.num_seqs} L={spec.num_layers} splits={fus.splits}")
    assert same_bits(torch, fus.out, sep.out), "output differs from append + attention"
    assert same_bits(torch, fus.pool_pages, sep.pool_pages), "pool differs from append"


@pytest.mark.parametrize("name", ["cfg1", "cfg2", "edges"])
def test_fused_matches_oracle(torch_gpu, orc, rope, name):
    spec = SMALL[name]()
    hw = wl.make_host_workload(spec)
    batch = host_batch(hw, rope)
    for layer in range(spec.num_layers):
        batch.append_attn(layer)
    out = batch.out.cpu().numpy()
    pages = hw.pages.copy()
    q = hw.q.copy()
    for layer in range(spec.num_layers):
        bt = np.ascontiguousarray(spec.block_tables[layer])
        orc.append(PoolView.from_pages(pages), bt, spec.ctx, q[layer],
                   np.ascontiguousarray(hw.k[layer]), np.ascontiguousarray(hw.v[layer]),
                   rope[0], rope[1])
        ref = orc.attn(PoolView.from_pages(pages), bt, spec.ctx, np.ascontiguousarray(q[layer]),
                       0.125)
        assert_attn_close(out[layer], ref, f"fused {name} layer {layer}")
    assert np.array_equal(to_u16(batch.pool_pages).reshape(pages.shape), pages)


def test_fused_edge_cases(torch_gpu, rope):
    """Lengths past max_context_len (written, not attended), positions past
    the RoPE table (not rotated, not written), a bad page id for one new
    token (NaN row, nothing written) and an empty row."""
    torch = torch_gpu
    lengths = [40, 70, 100, 33, 1, 64]
    spec = wl.make_spec(lengths, 1, seed=520)
    hw = wl.make_host_workload(spec)
    ctx = spec.ctx.copy()
    ctx[4] = 0                                   # empty row
    bt = spec.block_tables.copy()
    bt[0, 3, (33 - 1) // 16] = spec.num_pages + 3   # new token's page id out of range
    short_rope = (rope[0][:90].copy(), rope[1][:90].copy())   # positions >= 90 not in the table

    def make():
        return DecodeBatch(hw.pages, bt, ctx, hw.q, hw.k, hw.v, rope=short_rope,
                           max_context_len=64)
    sep, fus = run_both(torch, make, 1)
    assert same_bits(torch, fus.out, sep.out)
    assert same_bits(torch, fus.pool_pages, sep.pool_pages)
    out = fus.out[0].cpu().numpy()
    assert np.isnan(out[3]).all() and not out[4].any()
    assert np.isfinite(out[[0, 1, 2, 5]]).all()


def test_fused_strided_layouts(torch_gpu, rope):
    """Packed QKV rows ([B][3072]), padded output rows and a [slot][head][dim]
    page layout: the fused call gives the bits of append + attention on the
    default layout, writes the K/V rows through the strides, and leaves the
    packed q, k and v as given."""
    torch = torch_gpu
    spec = wl.make_spec([5, 16, 17, 300, 2048, 64], 1, seed=511)
    hw = wl.make_host_workload(spec)
    base = host_batch(hw, rope)
    base.step()
    torch.cuda.synchronize()
    ref_out = base.out[0].clone()
    ref_pool = base.pool_pages.clone()
    B = spec.num_seqs
    dev = base.device
    # pool with [K|V][slot 16][head 8][dim 64] pages
    inter = torch.from_numpy(np.ascontiguousarray(hw.pages.transpose(0, 1, 3, 2, 4)).view(np.int16)).to(dev)
    half = 16 * 8 * 64
    pool = pkv.make_pool(inter.data_ptr(), inter.data_ptr() + 2 * half, spec.num_pages,
                         2 * half, 64, 512)
    qkv = torch.zeros((B, 3072), dtype=torch.int16, device=dev)
    qkv[:, :2048] = torch.from_numpy(hw.q[0].view(np.int16)).to(dev)
    qkv[:, 2048:2560] = torch.from_numpy(hw.k[0].view(np.int16)).to(dev)
    qkv[:, 2560:] = torch.from_numpy(hw.v[0].view(np.int16)).to(dev)
    qkv_before = qkv.clone()
    bt = torch.from_numpy(np.ascontiguousarray(spec.block_tables[0])).to(dev)
    ctx = torch.from_numpy(spec.ctx).to(dev)
    out = torch.zeros((B, 2056), dtype=torch.float32, device=dev)   # padded rows
    ws_bytes = pkv.paged_decode_attn_workspace_size(B, base.max_context_len)
    ws = torch.zeros(max(ws_bytes, 16), dtype=torch.uint8, device=dev)
    say(f"fused strided layouts: B={B} ctx={spec.ctx.tolist()}")
    pkv.paged_kv_append_decode_attn(pool, bt, 128, ctx, B, base.max_context_len, qkv, 3072,
                                    qkv[:, 2048:], 3072, qkv[:, 2560:], 3072, base.rope_cos,
                                    base.rope_sin, 2048, base.scale, out, 2056, ws, ws_bytes)
    torch.cuda.synchronize()
    assert same_bits(torch, out[:, :2048].contiguous(), ref_out), "output differs from append + attention"
    assert torch.equal(out[:, 2048:], torch.zeros_like(out[:, 2048:])), "padding written"
    back = inter.view(spec.num_pages, 2, 16, 8, 64).permute(0, 1, 3, 2, 4).contiguous()
    assert torch.equal(back, ref_pool.view(back.shape)), "pool differs from append"
    assert torch.equal(qkv, qkv_before), "the fused call must leave q, k and v as given"


def test_fused_rotation_rounding_edges(torch_gpu):
    """The fused kernel's rotation on the rounding edges (exact BF16 ties,
    values beside a half-way point by less than an FP32 ulp, overflow,
    subnormals, zeros, infinities, NaN; RoPE table rows built for them):
    pool bits and output equal append + attention (NaN where NaN)."""
    from tests.test_gpu_prefill import _edge_bf16, _edge_table
    torch = torch_gpu
    rng = np.random.Generator(np.random.PCG64(721))
    lengths = list(range(1, 33))                 # new tokens at positions 0..31
    spec = wl.make_spec(lengths, 1, seed=721)
    hw = wl.make_host_workload(spec)
    B = spec.num_seqs
    hw.q[0] = _edge_bf16(rng, (B, 2048))
    hw.k[0] = _edge_bf16(rng, (B, 512))
    hw.v[0] = _edge_bf16(rng, (B, 512))
    table = _edge_table(rng, 32)

    def make():
        return DecodeBatch(hw.pages, spec.block_tables, spec.ctx, hw.q, hw.k, hw.v, rope=table,
                           max_context_len=32)
    sep, fus = run_both(torch, make, 1)
    assert same_bits(torch, fus.pool_pages, sep.pool_pages), "pool differs from append"
    assert same_bits(torch, fus.out, sep.out), "output differs from append + attention"
