"""Build the HIP library ``libamla.so`` (gfx950) in-tree.

One translation unit (csrc/amla.hip) holds the plan, decode and combine kernels and the
C ABI of include/amla.h.  Packed-FP32 instructions are disabled for the device code.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SRC = os.path.join(HERE, "csrc", "amla.hip")
LIB = os.path.join(HERE, "libamla.so")
ARCH = "gfx950"

FLAGS = [
    "-O3", "-std=c++17", "-fPIC", "-shared", f"--offload-arch={ARCH}",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # MFMA results in the VGPR form: lets the 128-row decode keep its 256 output
    # accumulators and the score tiles without spilling (Q fragments go to AGPRs).
    "-mllvm", "-amdgpu-mfma-vgpr-form=1",
    "-Wall", "-Wno-unused-result", "-Wno-unknown-warning-option",
    f"-I{os.path.join(ROOT, 'include')}",
]


def build(verbose: bool = False, extra=()) -> str:
    cmd = ["hipcc", *FLAGS, *extra, SRC, "-o", LIB + ".tmp"]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    noise = "packed-fp32-ops"
    msgs = [l for l in (res.stdout + res.stderr).splitlines() if noise not in l]
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + "\n".join(msgs))
    if verbose and msgs:
        print("\n".join(msgs))
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True, extra=sys.argv[1:])
