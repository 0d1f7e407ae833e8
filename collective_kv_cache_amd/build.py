"""Build the tdx HIP library (libtdx.so) in-tree for gfx950 with hipcc.

Usage: python -m collective_kv_cache_amd.build  (or call build()).
Every call recompiles; the library lands next to this file.
"""

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
SOURCES = ["api.hip", "rerotate.hip", "select.hip", "encode.hip", "attn.hip", "attn_f32.hip", "transfer.hip",
           "round.cpp"]
LIB = os.path.join(HERE, "libtdx.so")

FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    "-Wall",
    "-Wno-unused-function",
    # keep hipcc from forming packed fp32 arithmetic (v_pk_*_f32)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # MFMA accumulators in ordinary VGPRs: the online-softmax rescale then
    # multiplies them in place instead of copying them out of and back into AGPRs
    "-mllvm", "-amdgpu-mfma-vgpr-form",
    # keep a single-lane atomic a single-lane atomic: the optimizer's rewrite
    # uses the returned value at once, which waits for every load in flight
    "-mllvm", "-amdgpu-atomic-optimizer-strategy=None",
    "-I" + os.path.join(ROOT, "include"),
]


def hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    return os.path.join(rocm, "bin", "hipcc")


def build(verbose: bool = False) -> str:
    srcs = [os.path.join(CSRC, s) for s in SOURCES]
    tmp = LIB + ".tmp"
    cmd = [hipcc(), *FLAGS, *srcs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError("hipcc failed building libtdx.so")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
