"""The FP64 oracle against its pins, and the pins against planted mistakes.

Every pin compares the oracle with something fixed independently of it
(hand-derived golden values, closed forms, invariants, library routines,
brute force on contiguous arrays).  The mutation test plants plausible
mistakes in copies of the oracle's C source, on the CPU, and requires that
each one breaks at least one pin.
"""
import concurrent.futures
import os
import subprocess
import sys
import tempfile

import pytest

import oracle
from tests import oracle_pins

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def orc():
    return oracle.default()


@pytest.mark.parametrize("pin", oracle_pins.ALL_PINS, ids=lambda p: p.__name__)
def test_pin(orc, pin):
    pin(orc)


# (what the correct source says, a plausible mistake)
MUTATIONS = {
    "rope_sign": ("y[i] = x1 * c - x2 * s;", "y[i] = x1 * c + x2 * s;"),
    "rope_sign_second": ("y[i + HALF] = x2 * c + x1 * s;", "y[i + HALF] = x2 * c - x1 * s;"),
    "rope_pairing": ("double x2 = x[i + HALF];", "double x2 = x[(i + 1) % HD];"),
    "rope_frequency": ("-(2.0 * (double)i) / (double)HD", "-((double)i) / (double)HD"),
    "rope_cos_sin_swap": ("cos_out[(int64_t)pos * HALF + i] = (float)cos(angle);",
                          "cos_out[(int64_t)pos * HALF + i] = (float)sin(angle);"),
    "position_off_by_one": ("int32_t pos = ctx - 1;\n    *page_index", "int32_t pos = ctx;\n    *page_index"),
    "slot_formula": ("*slot = pos % PTOK;", "*slot = pos / PTOK % PTOK;"),
    "append_pos_table_row": ("const float* crow = rope_cos + (int64_t)pos * HALF;",
                             "const float* crow = rope_cos + (int64_t)n * HALF;"),
    "v_copy_from_k": ("memcpy(v_pool + off, vg, HD * sizeof(uint16_t));",
                      "memcpy(v_pool + off, kg, HD * sizeof(uint16_t));"),
    "head_offset": ("return page * page_stride + (int64_t)g * head_stride",
                    "return page * page_stride + (int64_t)g * slot_stride"),
    "gqa_mapping": ("int g = h / (HQ / HKV);", "int g = h % HKV;"),
    "scale_dropped": ("z[tau] = scale * dot;", "z[tau] = dot;"),
    "no_max_subtraction": ("w[tau] = exp(z[tau] - m);", "w[tau] = exp(z[tau]);"),
    "exp2_for_exp": ("w[tau] = exp(z[tau] - m);", "w[tau] = exp2(z[tau] - m);"),
    "no_normalisation": ("for (int d = 0; d < HD; ++d) o[d] /= total;", ""),
    "page_lookup_mod": ("block_table[(int64_t)s * bt_stride + tau / PTOK];\n                    if",
                        "block_table[(int64_t)s * bt_stride + tau % PTOK];\n                    if"),
    "slot_lookup_div": ("k_pool + elem_offset(page, g, tau % PTOK,", "k_pool + elem_offset(page, g, tau / PTOK,"),
    "causal_range": ("for (int32_t tau = 0; tau < n; ++tau) {\n                    w[tau]",
                     "for (int32_t tau = 0; tau < n - 1; ++tau) {\n                    w[tau]"),
    "bf16_truncate": ("double r = nearbyint(units) * spacing;", "double r = floor(units) * spacing;"),
    "bf16_ties_away": ("double r = nearbyint(units) * spacing;", "double r = round(units) * spacing;"),
    "bf16_precision": ("double spacing = ldexp(1.0, binade - 7);", "double spacing = ldexp(1.0, binade - 8);"),
    "bf16_subnormal_clamp": ("if (binade < -126) binade = -126;", ""),
    "q_not_rotated": ("memcpy(qh, rotated, sizeof rotated);", ""),
    "prefill_position_off_by_one": ("const int32_t n = start_pos[s] + (row - cu_tokens[s]) + 1;",
                                    "const int32_t n = start_pos[s] + (row - cu_tokens[s]);"),
    "prefill_row_of_first_sequence": ("k + (int64_t)row * k_stride, k_stride,",
                                      "k + (int64_t)(row - cu_tokens[s]) * k_stride, k_stride,"),
    "k_from_q_row": ("const uint16_t* kg = k + (int64_t)s * k_stride + (int64_t)g * HD;",
                     "const uint16_t* kg = k + (int64_t)s * k_stride + (int64_t)(g / 2) * HD;"),
}


def _run_mutant(name, find, repl, tmp):
    src = open(oracle.SOURCE).read()
    assert src.count(find) == 1, f"mutation {name}: anchor must occur exactly once"
    path = os.path.join(tmp, f"{name}.c")
    with open(path, "w") as f:
        f.write(src.replace(find, repl))
    lib = oracle.compile_source(path, os.path.join(tmp, f"lib{name}.so"))
    r = subprocess.run([sys.executable, "-m", "tests.oracle_pins", "--lib", lib], cwd=ROOT,
                       capture_output=True, text=True, timeout=600)
    return name, r.returncode, r.stdout[-2000:]


def test_planted_mistakes_are_caught():
    with tempfile.TemporaryDirectory() as tmp:
        with concurrent.futures.ThreadPoolExecutor(max_workers=4) as ex:
            futs = [ex.submit(_run_mutant, n, f, r, tmp) for n, (f, r) in MUTATIONS.items()]
            results = [fu.result() for fu in futs]
    survivors = [(n, out) for n, rc, out in results if rc == 0]
    assert not survivors, "mutants no pin caught: " + ", ".join(n for n, _ in survivors)
