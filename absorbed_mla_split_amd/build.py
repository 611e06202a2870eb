"""Build the HIP library ``libamla.so`` (gfx950) in-tree.

Three translation units, compiled separately and linked into one shared library:
  csrc/amla.hip       the plan, the reducers, the steps next to the decode and the C ABI of
                      include/amla.h; MFMA results in VGPRs;
  csrc/decode_stream.hip  the 32- and 64-row decodes; MFMA results in VGPRs (their output
                      tiles and scores live there);
  csrc/decode128.hip  the 128-row decode; MFMA results in AGPRs (its 256 output
                      accumulators per lane live there, its score tiles in VGPRs).
Packed-FP32 instructions are disabled for all device code.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libamla.so")
ARCH = "gfx950"

COMMON = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-result", "-Wno-unknown-warning-option",
    f"-I{os.path.join(ROOT, 'include')}",
]
UNITS = [
    ("amla.hip", ["-mllvm", "-amdgpu-mfma-vgpr-form=1"]),
    ("decode_stream.hip", ["-mllvm", "-amdgpu-mfma-vgpr-form=1"]),
    ("decode128.hip", ["-mllvm", "-amdgpu-mfma-vgpr-form=0"]),
]
NOISE = "packed-fp32-ops"


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    msgs = [l for l in (res.stdout + res.stderr).splitlines() if NOISE not in l]
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + "\n".join(msgs))
    if verbose and msgs:
        print("\n".join(msgs))


def build(verbose: bool = False, extra=()) -> str:
    objs = []
    for src, flags in UNITS:
        obj = os.path.join(CSRC, os.path.splitext(src)[0] + ".o")
        _run(["hipcc", *COMMON, *flags, *extra, "-c", os.path.join(CSRC, src), "-o", obj], verbose)
        objs.append(obj)
    _run(["hipcc", "-shared", f"--offload-arch={ARCH}", *objs, "-o", LIB + ".tmp"], verbose)
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True, extra=sys.argv[1:])
