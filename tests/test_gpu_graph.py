"""GPU: the decode step captured in a HIP graph and replayed.

The library's calls enqueue plain kernel launches on the caller's stream
(no memory operations, no allocation), so a step can be captured once and
replayed.  Each replay must equal the eagerly run step bit for bit, with the
program's own eager work and synchronizations between replays: a batch with
S > 1 (the in-launch merge and its counters, reset by every merging
workgroup), the start order of a mixed-length batch (its ranking launch
inside the graph), and the allocation-free call (its fixed scratch array).
Bar: bit-exact.
"""
import numpy as np
import pytest

import paged_kv_cache_172_amd as pkv
from paged_kv_cache_172_amd import workload as wl

from tests.gpu_util import host_batch, say

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


def _noalloc_step(b, stream):
    for layer in range(b.num_layers):
        pkv.paged_kv_append_decode_attn_noalloc(
            b.pool, b.block_tables[layer], b.bt_stride, b.context_lens, b.num_seqs,
            b.max_context_len, b.q[layer], 2048, b.k[layer], 512, b.v[layer], 512, b.rope_cos,
            b.rope_sin, b.max_pos, b.scale, b.out[layer], 2048, stream)


CASES = {
    "split_merge_cfg2": (lambda: wl.config_spec(2), "fused"),
    "ordered_mix_1200": (lambda: wl.make_spec(
        np.clip(np.rint(np.exp(np.random.default_rng(960).uniform(np.log(16), np.log(2048), 1200))),
                16, 2048).astype(int), 1, seed=960), "ordered"),
    "noalloc_two_layers": (lambda: wl.make_spec([2048, 5, 700, 33, 1400, 17, 9, 1990], 2, seed=961),
                           "noalloc"),
}


@pytest.mark.parametrize("name", list(CASES))
def test_graph_replays_equal_the_eager_step(torch_gpu, rope, name):
    torch = torch_gpu
    make, how = CASES[name]
    spec = make()
    hw = wl.make_host_workload(spec)
    eager = host_batch(hw, rope)
    graphed = host_batch(hw, rope)
    stream = torch.cuda.Stream()

    def step(b):
        if how == "noalloc":
            _noalloc_step(b, torch.cuda.current_stream())
        else:
            b.step_fused(order=(how == "ordered"))

    with torch.cuda.stream(stream):
        step(eager)
    torch.cuda.synchronize()
    ref_out = eager.out.clone()
    ref_pool = eager.pool_pages.clone()
    say(f"[graph] {name}: B={spec.num_seqs} L={spec.num_layers} splits={eager.splits}")
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        step(graphed)
    torch.cuda.synchronize()
    for r in range(4):
        graphed.out.fill_(float("nan"))            # eager work between replays
        junk = torch.randn(1 << 20, device="cuda").sum()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.isfinite(junk)
        assert torch.equal(graphed.out.view(torch.int32), ref_out.view(torch.int32)), (name, r)
        assert torch.equal(graphed.pool_pages, ref_pool), (name, r)
    if graphed.ws_bytes:
        assert not graphed.workspace[:2048].view(torch.int32).any(), "merge counters left nonzero"
    del g
