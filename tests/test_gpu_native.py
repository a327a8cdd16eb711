"""GPU: the C ABI called from native code (tests/native/abi_caller.cpp), with
no Python in the call path.

The caller checks a mixed batch of 8 sequences (1 to 2,048 tokens) against
the FP64 oracle library: the fused call's pool bytes bit-exact, its output
within 2e-3 absolute / 1e-2 relative (to max(|oracle|, 1e-3)), the two-call
path equal to the fused call bit for bit and paged_kv_append's rotated q
bit-exact; and the library's RoPE table equal to the oracle's.  It then times
back-to-back calls of one 37-token sequence from C.  The binary is built by
``__graft_entry__.build()`` (tests/native/build_native.py).
"""
import json
import os
import subprocess

import pytest

from tests.gpu_util import say

pytestmark = pytest.mark.gpu

BINARY = os.path.join(os.path.dirname(os.path.abspath(__file__)), "native", "abi_caller")


def test_native_caller_parity_and_latency():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU (run with -m 'not gpu' on CPU)"
    assert os.path.exists(BINARY), f"{BINARY} is missing: run __graft_entry__.build()"
    say("[native] running tests/native/abi_caller")
    r = subprocess.run([BINARY], capture_output=True, text=True, timeout=120)
    say(r.stderr[-2000:])
    assert r.returncode == 0, f"native caller failed ({r.returncode}): {r.stderr[-2000:]}"
    res = json.loads(r.stdout.strip().splitlines()[-1])
    say(f"[native] {json.dumps(res)}")
    assert res["failures"] == 0
    assert res["parity"]["pool_bit_exact"] and res["parity"]["two_calls_bit_exact"]
    assert res["parity"]["max_abs"] <= 2e-3 and res["parity"]["max_rel"] <= 1e-2
    for leg in res["latency_us_per_call"].values():
        assert leg["device"] > 0.0
