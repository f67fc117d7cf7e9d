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


# Slips in the append oracle: the RoPE pairing, sign, frequency, base or
# position; the rounding's precision, direction or subnormal range; a slot off
# by one; V rotated; q left unrotated; stale rows.
APPEND_MUTANTS = {
    "rope_sign": [("x[i + half] = second * c + first * s;", "x[i + half] = second * c - first * s;")],
    "rope_adjacent_pairs": [("const double first = x[i];\n        const double second = x[i + half];",
                             "const double first = x[i];\n        const double second = x[i ^ 1];")],
    "rope_frequency_exponent": [("pow(theta, -2.0 * (double)i / (double)head_dim)",
                                 "pow(theta, -(double)i / (double)head_dim)")],
    "rope_default_base": [("pow(theta, -2.0", "pow(10000.0, -2.0")],
    "rope_angle_sign": [("const double angle = pos * freq;", "const double angle = -pos * freq;")],
    "rope_at_context_length": [("dim, rope, (double)pos, theta, scratch);\n                memcpy",
                                "dim, rope, (double)c, theta, scratch);\n                memcpy")],
    "round_truncates": [("r = ldexp(nearbyint(ldexp(x, -step)), step);", "r = ldexp(trunc(ldexp(x, -step)), step);")],
    "round_nine_bits": [("int step = e - 8;", "int step = e - 9;")],
    "round_no_subnormals": [("if (step < -133)\n            step = -133;", "if (step < -126)\n            step = -126;")],
    "slot_off_by_one": [("const size_t slot = (size_t)page * s->page_size + pos % s->page_size;",
                         "const size_t slot = (size_t)page * s->page_size + (pos + 1) % s->page_size;")],
    "position_off_by_one": [("const int32_t pos = c - n + j;", "const int32_t pos = c - n + j - 1 + (c - n + j == 0);")],
    "v_rotated": [("memcpy(v_pool + slot * kv_row + (size_t)g * dim, v_new + row * kv_row + (size_t)g * dim,\n"
                   "                       (size_t)dim * sizeof *v_pool);",
                   "rotate_head(v_new + row * kv_row + (size_t)g * dim, v_pool + slot * kv_row + (size_t)g * dim,\n"
                   "                            dim, rope, (double)pos, theta, scratch);")],
    "q_not_rotated": [("if (q && rope)", "if (q && !rope)")],
    "row_ignores_start": [("const size_t row = (size_t)start + j;", "const size_t row = (size_t)b + j;")],
}


# Slips in the prefill oracle: the causal cut off by one, positions counted
# from the chunk start, the query of the request instead of the row, the
# first request's table row for everyone, and (in the listed-pairs entry
# point) a pair's neighbouring query head.
PREFILL_MUTANTS = {
    "cut_excludes_own_token": [("const int32_t visible = pos + 1;", "const int32_t visible = pos;")],
    "positions_from_chunk_start": [("*pos_out = context_lens[b] - n + (r - start);", "*pos_out = r - start;")],
    "query_of_request": [("q + (size_t)r * s->num_q_heads * s->head_dim", "q + (size_t)b * s->num_q_heads * s->head_dim")],
    "first_table_row": [("block_table + (size_t)b * s->max_blocks, &visible", "block_table, &visible")],
    "pairs_neighbouring_head": [("pairs[2 * i + 1], scale,", "pairs[2 * i + 1] ^ 1, scale,")],
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


def test_unmutated_append_copy_passes(tmp_path):
    lib = obuild.build_variant([], out_dir=str(tmp_path), source=obuild.APPEND_SRC)
    r = subprocess.run([sys.executable, "-m", "tests.oracle_append_pins", "--lib", lib],
                       cwd=ROOT, capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stdout + r.stderr


@pytest.mark.parametrize("name", sorted(APPEND_MUTANTS))
def test_append_mutant_is_caught(name, tmp_path):
    lib = obuild.build_variant(APPEND_MUTANTS[name], out_dir=str(tmp_path), source=obuild.APPEND_SRC)
    r = subprocess.run([sys.executable, "-m", "tests.oracle_append_pins", "--lib", lib],
                       cwd=ROOT, capture_output=True, text=True, timeout=600)
    assert r.returncode != 0, f"mutant {name} passed every pin:\n{r.stdout}"


def test_unmutated_prefill_copy_passes(tmp_path):
    lib = obuild.build_variant([], out_dir=str(tmp_path), source=obuild.PREFILL_SRC)
    r = subprocess.run([sys.executable, "-m", "tests.oracle_prefill_pins", "--lib", lib],
                       cwd=ROOT, capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stdout + r.stderr


@pytest.mark.parametrize("name", sorted(PREFILL_MUTANTS))
def test_prefill_mutant_is_caught(name, tmp_path):
    lib = obuild.build_variant(PREFILL_MUTANTS[name], out_dir=str(tmp_path), source=obuild.PREFILL_SRC)
    r = subprocess.run([sys.executable, "-m", "tests.oracle_prefill_pins", "--lib", lib],
                       cwd=ROOT, capture_output=True, text=True, timeout=600)
    assert r.returncode != 0, f"mutant {name} passed every pin:\n{r.stdout}"
