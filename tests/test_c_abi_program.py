"""The library driven from C++ through include/pagedattn.h alone (no Python
binding, no torch): tests/c_abi/decode_from_c.cpp writes new tokens with
pa_reshape_and_cache, runs a split-K pa_paged_attention_decode and compares
the fp32 output with the fp64 oracle."""
import os
import subprocess

import pytest

from tests.c_abi import build as c_abi_build


def test_c_program_compiles_against_the_header():
    exe = c_abi_build.build()
    assert os.path.exists(exe)


@pytest.mark.gpu
def test_c_program_decode_matches_the_oracle():
    if not os.path.exists(c_abi_build.EXE):
        c_abi_build.build()
    r = subprocess.run([c_abi_build.EXE], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    err = float(r.stdout.split("max_abs_err")[1].split()[0])
    assert err <= 2e-3
