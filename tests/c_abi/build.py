"""Compile decode_from_c.cpp (host code; links the library, the HIP runtime
and the oracle) into tests/c_abi/decode_from_c, and bounds_check.cpp (host
code over the kernels' index arithmetic, no GPU) into
tests/c_abi/bounds_check. Test infrastructure."""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
SRC = os.path.join(HERE, "decode_from_c.cpp")
EXE = os.path.join(HERE, "decode_from_c")
BOUNDS_SRC = os.path.join(HERE, "bounds_check.cpp")
BOUNDS_EXE = os.path.join(HERE, "bounds_check")


def build(verbose: bool = False) -> str:
    tmp = EXE + ".tmp%d" % os.getpid()
    cmd = ["g++", "-std=c++17", "-O2", "-Wall", "-D__HIP_PLATFORM_AMD__",
           "-I", os.path.join(ROOT, "include"), "-I", "/opt/rocm/include", SRC, "-o", tmp,
           "-L", os.path.join(ROOT, "paged_kv_cache_391_amd"), "-lpagedattn",
           "-L", os.path.join(ROOT, "oracle"), "-loracle",
           "-L", "/opt/rocm/lib", "-lamdhip64",
           "-Wl,-rpath,$ORIGIN/../../paged_kv_cache_391_amd:$ORIGIN/../../oracle:/opt/rocm/lib"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, EXE)
    return EXE


def build_bounds(verbose: bool = False) -> str:
    """The index-arithmetic check: pa_bounds.h is host-and-device code, so
    it is compiled by hipcc (its device pass holds no kernel)."""
    tmp = BOUNDS_EXE + ".tmp%d" % os.getpid()
    cmd = ["/opt/rocm/bin/hipcc", "-std=c++17", "-O1", "-x", "hip", "--offload-arch=gfx950", BOUNDS_SRC, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, BOUNDS_EXE)
    return BOUNDS_EXE


if __name__ == "__main__":
    build(verbose=True)
    build_bounds(verbose=True)
    sys.exit(0)
