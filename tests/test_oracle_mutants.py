"""Planted mistakes: each mutant is a copy of the oracle source with one
plausible bug (a dropped term, a wrong sign, index or alignment, a transposed
operand), built on the CPU into a temporary directory. The pin suite must
reject every one of them."""
import os
import subprocess

import pytest

import oracle
from oracle import build as obuild
from tests import test_oracle as pins

MUTANTS = {
    "block_offset_off_by_one": ("int64_t off = t % bs;", "int64_t off = (t + 1) % bs;"),
    "block_and_head_swapped": ("return ((blk * H + h) * bs + off) * d;", "return ((h * H + blk) * bs + off) * d;"),
    "scale_dropped": ("x[t] = scale * dot;", "x[t] = dot;"),
    "normalisation_dropped": ("out[e] = acc / sum;", "out[e] = acc;"),
    "max_subtracted_with_wrong_sign": ("x[t] = exp(x[t] - m);", "x[t] = exp(m - x[t]);"),
    "causal_off_by_one": ("int visible = ctx[s] - L + j + 1;", "int visible = ctx[s] - L + j;"),
    "causal_top_left_aligned": ("int visible = ctx[s] - L + j + 1;", "int visible = j + 1;"),
    "query_head_transposed": ("qd[e] = elem(q, dtype, ((int64_t)s * H + h) * d + e);",
                              "qd[e] = elem(q, dtype, ((int64_t)h * S + s) * d + e);"),
    "values_read_from_key_cache": ("V[(int64_t)t * d + e] = elem(v_cache, dtype, base + e);",
                                   "V[(int64_t)t * d + e] = elem(k_cache, dtype, base + e);"),
    "last_token_dropped": ("attend(out + (int64_t)i * d, qd, K, V, ctx[s], d, scale, x);",
                           "attend(out + (int64_t)i * d, qd, K, V, ctx[s] - 1, d, scale, x);"),
    "half_exponent_bias": ("mag = ldexp((double)(fr | 0x400), ex - 25);", "mag = ldexp((double)(fr | 0x400), ex - 24);"),
    "half_subnormal_scale": ("mag = ldexp((double)fr, -24);", "mag = ldexp((double)fr, -25);"),
    "bf16_shift": ("uint32_t u = (uint32_t)b << 16;", "uint32_t u = (uint32_t)b << 15;"),
    "slot_block_offset_swapped": ("int64_t blk = s / bs, off = s % bs;", "int64_t blk = s % bs, off = s / bs;"),
    "duplicate_slots_accepted": ("if (seen[s]) { free(seen); return O_DUP_SLOT; }", ""),
    "copy_source_and_destination_swapped": (
        "size_t src = (size_t)pairs[2 * i] * block_bytes, dst = (size_t)pairs[2 * i + 1] * block_bytes;",
        "size_t dst = (size_t)pairs[2 * i] * block_bytes, src = (size_t)pairs[2 * i + 1] * block_bytes;"),
    "copy_of_values_skipped": ("memcpy((char*)v_cache + dst, (const char*)v_cache + src, block_bytes);", ""),
    "softmax_sum_skips_first_token": ("    sum += x[t];", "    if (t) sum += x[t];"),
    "scale_applied_twice": ("x[t] = scale * dot;", "x[t] = scale * scale * dot;"),
    "new_values_written_from_keys": ("memcpy((char*)v_cache + dst, (const char*)v + src, row);",
                                     "memcpy((char*)v_cache + dst, (const char*)k + src, row);"),
}

PINS = [
    (pins.test_widen_f16_every_bit_pattern_matches_numpy, ()),
    (pins.test_widen_bf16_every_bit_pattern_matches_torch, ()),
    (pins.test_decode_matches_dense_brute_force, ("f16", 16)),
    (pins.test_decode_matches_dense_brute_force, ("bf16", 32)),
    (pins.test_prefill_matches_dense_brute_force_with_explicit_mask, ("f16",)),
    (pins.test_prefill_with_prior_equals_torch_sdpa_bottom_right_mask, ()),
    (pins.test_golden_closed_form_example, ()),
    (pins.test_single_token_returns_its_value_row_exactly, ()),
    (pins.test_affine_map_of_values_passes_through, ()),
    (pins.test_reshape_and_cache_round_trip_and_untouched_slots, ()),
    (pins.test_reshape_and_cache_skips_negative_and_rejects_bad_slots, ()),
    (pins.test_gather_matches_independent_index_arithmetic, ()),
    (pins.test_copy_blocks_matches_numpy_block_assignment_and_rejects_ambiguous_maps, ()),
]


def _build_mutant(tmp_path, name, old, new):
    src = open(obuild.SRC).read()
    assert src.count(old) >= 1, f"mutation site for {name} not found"
    path = tmp_path / f"{name}.c"
    path.write_text(src.replace(old, new))
    lib = tmp_path / f"lib{name}.so"
    subprocess.run(["gcc", "-std=c11", "-O2", "-fopenmp", "-fPIC", "-shared", "-o", str(lib), str(path), "-lm"],
                   check=True)
    return str(lib)


def _caught():
    for fn, args in PINS:
        try:
            fn(*args)
        except (AssertionError, oracle.OracleError, pytest.fail.Exception):
            return fn.__name__
    return None


def test_unmutated_source_passes_the_pins(tmp_path):
    lib = _build_mutant(tmp_path, "identity", "#include <math.h>", "#include <math.h>")
    oracle.use_library(lib)
    try:
        assert _caught() is None
    finally:
        oracle.use_library(None)


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_reject_planted_mistake(tmp_path, name):
    old, new = MUTANTS[name]
    lib = _build_mutant(tmp_path, name, old, new)
    oracle.use_library(lib)
    try:
        assert _caught() is not None, f"mutant {name} passed every pin"
    finally:
        oracle.use_library(None)
