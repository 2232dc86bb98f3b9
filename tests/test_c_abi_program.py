"""The library driven from C++ through include/pagedattn.h alone (no Python
binding, no torch): tests/c_abi/decode_from_c.cpp writes new tokens with
pa_reshape_and_cache, runs a split-K pa_paged_attention_decode and a causal
pa_paged_attention_prefill and compares their fp32 outputs with the fp64
oracle, then runs the same work as one pa_attention_step (in order and with
a side stream) and checks it equals the separate calls bit for bit and
matches the oracle on both outputs."""
import os
import subprocess

import pytest

from tests.c_abi import build as c_abi_build


def test_c_program_compiles_against_the_header():
    exe = c_abi_build.build()
    assert os.path.exists(exe)


@pytest.mark.gpu
def test_c_program_matches_the_oracle_and_the_step_call():
    if not os.path.exists(c_abi_build.EXE):
        c_abi_build.build()
    r = subprocess.run([c_abi_build.EXE], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    vals = dict(line.split() for line in r.stdout.split("\n") if line.strip())
    assert float(vals["max_abs_err"]) <= 2e-3
    assert float(vals["prefill_max_abs_err"]) <= 2e-3
    assert vals["step_bit_identical"] == "1"
    assert float(vals["step_max_abs_err"]) <= 2e-3
    assert float(vals["step_prefill_max_abs_err"]) <= 2e-3


def test_kernel_index_arithmetic_stays_in_bounds():
    """Lengths, block ids and query ranges far outside the preconditions
    (negative, past max_context_len, past the pool, INT_MIN/INT_MAX) are
    clamped by the functions every kernel and launch plan uses, so no table
    entry, workspace slot, query row or block outside the validated sizes is
    touched. Host code only (tests/c_abi/bounds_check.cpp)."""
    exe = c_abi_build.build_bounds()
    r = subprocess.run([exe], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    assert r.stdout.startswith("bounds ok")
