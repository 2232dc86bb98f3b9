"""Build libpagedattn.so (HIP, gfx950) in-tree with hipcc."""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libpagedattn.so")
SOURCES = ["pa_api.hip", "pa_cache.hip", "pa_decode.hip", "pa_prefill.hip", "pa_shared.hip", "pa_alloc.cpp"]
ARCH = "gfx950"


def hipcc_flags(extra=()):
    return [
        "--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC", "-shared",
        # no packed-fp32 VALU ops: keep every fp32 op scalar per lane
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        # matrix-core accumulators in ordinary VGPRs: the online softmax
        # rescales them every tile, which would otherwise copy them out of
        # and back into the accumulation registers
        "-mllvm", "-amdgpu-mfma-vgpr-form=1",
        "-Wall", "-Wno-unused-function",
        *extra,
    ]


def build(out: str = LIB, defines=(), verbose: bool = False) -> str:
    srcs = [os.path.join(CSRC, s) for s in SOURCES]
    tmp = out + ".tmp%d" % os.getpid()
    cmd = ["hipcc", *hipcc_flags(["-D" + d for d in defines]), "-o", tmp, *srcs]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True, stderr=None if verbose else subprocess.PIPE)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
