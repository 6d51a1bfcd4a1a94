"""Build libnvfp4.so (the C ABI + HIP kernels) for gfx950 with hipcc, in-tree.

Each source is compiled to an object in its own process (in parallel), then the
objects are linked into the shared library.  Every call rebuilds everything.

    python nvfp4_w4a4_quantized_amd/build.py

It imports nothing from the package, whose import needs the built library.
"""

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libnvfp4.so")
OBJDIR = os.path.join(ROOT, "_build")

SOURCES = ["abi.cpp", "quant.hip", "gemm.hip", "gemv.hip", "skinny.hip", "requant.hip", "mx.hip", "noalloc.hip", "gdn.hip", "probe.hip", "soloq.hip"]

COMPILE_FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++20",
    "-fPIC",
    "-fvisibility=hidden",
    # the quantizer relies on exactly rounded float64/fp32 operations: no contraction
    "-ffp-contract=off",
    # keep the compiler from forming packed-fp32 (v_pk_*_f32) instructions
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
]
LINK_FLAGS = ["--offload-arch=gfx950", "-shared", "-fPIC"]


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + " ".join(cmd) + "\n" + res.stdout + res.stderr)


def build(verbose: bool = False) -> str:
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    os.makedirs(OBJDIR, exist_ok=True)
    objs = [os.path.join(OBJDIR, os.path.splitext(s)[0] + ".o") for s in SOURCES]
    cmds = [[hipcc] + COMPILE_FLAGS + ["-c", "-o", o, os.path.join(CSRC, s)] for s, o in zip(SOURCES, objs)]
    with ThreadPoolExecutor(max_workers=len(cmds)) as ex:
        for f in [ex.submit(_run, c, verbose) for c in cmds]:
            f.result()
    tmp = LIB + ".tmp"
    _run([hipcc] + LINK_FLAGS + ["-o", tmp] + objs, verbose)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
