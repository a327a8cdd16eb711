"""The native page management under AddressSanitizer and UBSan: its C++
source and a randomised stress driver built with g++ (host code only) and
run for 20,000 steps."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.skipif(shutil.which("g++") is None, reason="needs g++")
def test_pager_under_sanitizers(tmp_path):
    exe = tmp_path / "pager_stress"
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fsanitize=address,undefined",
           "-fno-sanitize-recover=all", "-I", os.path.join(ROOT, "include"),
           os.path.join(ROOT, "paged_kv_cache_172_amd", "csrc", "pager.cpp"),
           os.path.join(ROOT, "tests", "pager_stress.cpp"), "-o", str(exe)]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    r = subprocess.run([str(exe), "20000"], capture_output=True, text=True, timeout=300,
                       env=dict(os.environ, ASAN_OPTIONS="detect_leaks=1"))
    assert r.returncode == 0, r.stderr[-3000:]
    assert r.stdout.startswith("ok:")
