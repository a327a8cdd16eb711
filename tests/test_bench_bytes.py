"""bench.py's algorithmic byte counts (the roofline's numerator) on the CPU,
derived here from the model geometry: 32 query heads and 8 KV heads of 64
dims, BF16 K/V/q, FP32 output, 16-token pages, int32 table entries, and an
FP32 partial of 64 accumulators plus (max, sum) per (sequence, query head,
split)."""
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import bench  # noqa: E402
from paged_kv_cache_172_amd import workload as wl  # noqa: E402

HQ, HKV, D, BF16, F32, PAGE = 32, 8, 64, 2, 4, 16


def expected_attention_bytes(ctx, splits):
    kv_per_token = HKV * D * 2 * BF16               # K and V of one token, all KV heads
    per_seq = []
    for n in np.asarray(ctx, np.int64):
        pages = -(-int(n) // PAGE)
        out = HQ * D * F32 if splits == 1 else splits * HQ * (D + 2) * F32
        per_seq.append(int(n) * kv_per_token + HQ * D * BF16 + pages * 4 + out)
    return sum(per_seq)


def test_config3_attention_and_fused_bytes():
    ctx = wl.config_spec(3).ctx
    assert ctx.size == 64 and (ctx == 2048).all()
    got = bench.split_bytes_per_launch(ctx, 1)
    assert got == expected_attention_bytes(ctx, 1) == 269_254_656
    # the fused kernel also reads the new k and v rows and the two RoPE rows
    # (32 FP32 each) and writes the K and V rows into the pages
    extra = 64 * (2 * HKV * D * BF16 + 2 * HKV * D * BF16 + 2 * 32 * F32)
    assert bench.append_bytes_per_launch(64) == extra
    assert got + extra == 269_533_184
    # the headline's KV bytes: K and V of every valid token of every layer
    assert wl.config_spec(3).kv_bytes_per_step() == 64 * 2048 * 16 * HKV * D * 2 * BF16 == 4 * 2 ** 30


def test_mixed_and_split_bytes():
    spec = wl.config_spec(4)
    assert bench.split_bytes_per_launch(spec.ctx, 1) == expected_attention_bytes(spec.ctx, 1)
    assert spec.kv_bytes_per_step() // spec.num_layers == int(spec.ctx.astype(np.int64).sum()) * 2048
    ctx = np.array([1, 16, 17, 37, 2048, 0], np.int32)
    for s in (1, 2, 5, 8):
        assert bench.split_bytes_per_launch(ctx, s) == expected_attention_bytes(ctx, s)


def test_prefill_bytes():
    per_token = bench.prefill_bytes_per_token(True)
    # k and v rows read and written (1 KiB each way each), q read and written back (4 KiB each way)
    assert per_token == 2 * 2 * HKV * D * BF16 + 2 * HQ * D * BF16
    assert bench.prefill_bytes_per_token(False) == 2 * 2 * HKV * D * BF16
    assert bench.ROPE_TABLE_BYTES == 2 * 2048 * 32 * F32
    assert 64 * 2048 * per_token + bench.ROPE_TABLE_BYTES == 1_610_612_736 + 524_288
