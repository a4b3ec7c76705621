"""Build libzpq.so (HIP, gfx950) in-tree, next to this file.

  python -m block_quantized_communication_amd.build [-v] [--save-temps]

Flags: -O3 for gfx950 only; packed-FP32 instructions disabled; no fast-math
(IEEE division, denormals kept); -fPIC shared library with a C ABI.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SRC = os.path.join(HERE, "csrc", "zpq.hip")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "libzpq.so")
ARCH = "gfx950"

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-fno-gpu-flush-denormals-to-zero", "-ffp-contract=off",
    "-fconstexpr-steps=100000000", "-Wall", "-Wno-unused-function",
]


def build(verbose: bool = False, save_temps: bool = False) -> str:
    tmp = LIB + ".tmp"
    cmd = ["hipcc", *HIPCC_FLAGS, f"-I{INCLUDE}", SRC, "-o", tmp]
    if save_temps:
        cmd.insert(1, "--save-temps")
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True,
                         cwd=os.path.join(HERE, "csrc") if save_temps else None)
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in res.stderr.splitlines() if noise not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{err}")
    if err.strip() and verbose:
        print(err, file=sys.stderr)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    build(verbose="-v" in sys.argv, save_temps="--save-temps" in sys.argv)
