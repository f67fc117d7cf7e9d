"""Planted mistakes in copies of the oracle source must each fail some pin.

Every mutant below is a plausible slip in the oracle (wrong head grouping, a
dropped scale, an off-by-one slot, K read for V, no max shift, a missing
normalisation, a reversed operand, a wrong stride, a dropped token, a wrong
log base, a squared weight).  Each is compiled on the CPU and the whole pin
suite runs against it in a child process, so a mutant that reads out of bounds
fails by crashing rather than taking the test run down.
"""
import os
import subprocess
import sys

import pytest

from oracle import build as obuild

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

MUTANTS = {
    "interleaved_heads": [("const int32_t kv = h / group;", "const int32_t kv = h % s->num_kv_heads;")],
    "no_scale": [("z[t] = scale * dot;", "z[t] = dot;")],
    "slot_off_by_one": [("const int32_t slot = t % s->page_size;",
                         "const int32_t slot = (t + 1) % s->page_size;")],
    "k_for_v": [("vrow[t] = v_pool + row;", "vrow[t] = k_pool + row;")],
    "no_max_shift": [("z[t] = exp(z[t] - m);", "z[t] = exp(z[t]);")],
    "no_normalise": [("out_row[d] /= l;", "out_row[d] /= 1.0;")],
    "reversed_key": [("dot += bf16_value(qh[d]) * bf16_value(k[d]);",
                      "dot += bf16_value(qh[d]) * bf16_value(k[dim - 1 - d]);")],
    "query_of_kv_head": [("const uint16_t *qh = q + ((size_t)b * s->num_q_heads + h) * dim;",
                          "const uint16_t *qh = q + ((size_t)b * s->num_q_heads + kv) * dim;")],
    "drops_last_token": [("const int32_t n = context_lens[b];\n    const size_t slot_stride",
                          "const int32_t n = context_lens[b] - (context_lens[b] > 1);\n"
                          "    const size_t slot_stride")],
    "lse_without_max": [("*lse = m + log(l);", "*lse = log(l);")],
    "lse_log2": [("*lse = m + log(l);", "*lse = m + log2(l);")],
    "squared_weight": [("l += z[t];", "l += z[t] * z[t];")],
    "table_row_stride": [("block_table[(size_t)b * s->max_blocks + t / s->page_size]",
                          "block_table[(size_t)b * (s->max_blocks - 1) + t / s->page_size]")],
}


def test_unmutated_copy_passes(tmp_path):
    lib = obuild.build_variant([], out_dir=str(tmp_path))
    r = subprocess.run([sys.executable, "-m", "tests.oracle_pins", "--lib", lib],
                       cwd=ROOT, capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stdout + r.stderr


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, tmp_path):
    lib = obuild.build_variant(MUTANTS[name], out_dir=str(tmp_path))
    r = subprocess.run([sys.executable, "-m", "tests.oracle_pins", "--lib", lib],
                       cwd=ROOT, capture_output=True, text=True, timeout=600)
    assert r.returncode != 0, f"mutant {name} passed every pin:\n{r.stdout}"
