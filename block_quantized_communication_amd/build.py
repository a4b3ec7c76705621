"""Build libzpq.so (HIP, gfx950) in-tree, next to this file.

  python -m block_quantized_communication_amd.build [-v] [--save-temps]
  python -m block_quantized_communication_amd.build --variants

--variants builds, into variants/, the receive-kernel launch-shape variants
that bench.py --study receive-shapes compares (RECEIVE_VARIANTS), the
qgZ-quantizer code-store cache policies that bench.py --study store-policy
compares (QGZ_STORE_VARIANTS) and the wave-timeline recording builds of
bench.py --study timeline (TIMELINE_VARIANTS), one build-time override each, with the
compiler's register, LDS and occupancy report for the kernels concerned in
variants/resources.json.

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


# Launch-shape variants of the receive kernels (k_dequant_reduce): name ->
# build-time overrides of the defaults in csrc/zpq.hip.
RECEIVE_VARIANTS = {
    "default": [],
    "i4_pf1": ["-DZPQ_REDUCE_PF_I4=1"],
    "i4_pf3": ["-DZPQ_REDUCE_PF_I4=3"],
    "i4_pf4": ["-DZPQ_REDUCE_PF_I4=4"],
    "i4_epl16": ["-DZPQ_REDUCE_EPL_I4=16"],
    "i4_epl16_pf4": ["-DZPQ_REDUCE_EPL_I4=16", "-DZPQ_REDUCE_PF_I4=4"],
    "fl_narrow_pf2": ["-DZPQ_REDUCE_PF_FL_NARROW=2"],
    "fl_narrow_pf8": ["-DZPQ_REDUCE_PF_FL_NARROW=8"],
    "fl_wide_pf3": ["-DZPQ_REDUCE_PF_FL=3"],
    "fl_wide_pf4": ["-DZPQ_REDUCE_PF_FL=4"],
    "fl_wide_epl32": ["-DZPQ_REDUCE_EPL_FL=32"],
    "fl_wide_xcd": ["-DZPQ_XCD_REDUCE=1"],
    "fl_never_narrow": ["-DZPQ_REDUCE_NARROW_WAVES=0"],
    "fl_always_narrow": ["-DZPQ_REDUCE_NARROW_WAVES=1048576"],
    "wg3": ["-DZPQ_REDUCE_WG3=1"],
}
# Wave-timeline recording builds of the receive kernel (bench.py --study
# timeline): timeline_w7 holds the occupancy target at 7 waves per SIMD, where
# the recording code would otherwise change the INT4 kernel's registers (the
# shipped INT4 kernel's 92 scalar registers also give it 7 waves per SIMD).
TIMELINE_VARIANTS = {
    "timeline": ["-DZPQ_TIMELINE=1"],
    "timeline_w7": ["-DZPQ_TIMELINE=1", "-DZPQ_TIMELINE_WAVES=7"],
}
# The qgZ quantizer's code stores (default: buffer stores with sc0 sc1 nt).
QGZ_STORE_VARIANTS = {
    "qgz_global_nt": ["-DZPQ_CPOL_QGZ=-1"],      # non-temporal global stores
    "qgz_nt": ["-DZPQ_CPOL_QGZ=2"],
    "qgz_sc1": ["-DZPQ_CPOL_QGZ=16"],
    "qgz_sc0_sc1": ["-DZPQ_CPOL_QGZ=17"],
}
VARIANTS_DIR = os.path.join(HERE, "variants")


def _resources(stderr, only="k_dequant_reduce"):
    """Per-kernel register, LDS and occupancy report from the compiler's
    kernel-resource-usage remarks: {mangled name: {field: int}}, for the
    kernels whose name contains `only` (all of them for "")."""
    import re
    out, cur = {}, None
    fields = {"TotalSGPRs": "sgprs", "VGPRs": "vgprs", "AGPRs": "agprs",
              "ScratchSize [bytes/lane]": "scratch_bytes_per_lane",
              "Occupancy [waves/SIMD]": "waves_per_simd", "LDS Size [bytes/block]": "lds_bytes"}
    for line in stderr.splitlines():
        m = re.search(r"remark: Function Name: (\S+)", line)
        if m:
            cur = m.group(1) if only in m.group(1) else None
            if cur:
                out[cur] = {}
            continue
        if cur:
            m = re.search(r"remark:\s+([^:]+(?:\[[^]]*\])?): (\d+)", line)
            if m and m.group(1).strip() in fields:
                out[cur][fields[m.group(1).strip()]] = int(m.group(2))
    return out


def build_variants(names=None, jobs=8, verbose=False):
    """Build the RECEIVE_VARIANTS and QGZ_STORE_VARIANTS libraries (all, or
    `names`) into variants/libzpq_<name>.so, `jobs` compilers at a time; write
    the compiler's resource report of each variant's receive kernels (or qgZ
    quantizer kernels) to variants/resources.json, with the variant's group
    ("receive" or "qgz_store").  Returns the paths."""
    import concurrent.futures
    import json
    os.makedirs(VARIANTS_DIR, exist_ok=True)
    table = {**RECEIVE_VARIANTS, **QGZ_STORE_VARIANTS, **TIMELINE_VARIANTS}
    names = list(table) if names is None else list(names)

    def one(name):
        out = os.path.join(VARIANTS_DIR, f"libzpq_{name}.so")
        cmd = ["hipcc", *HIPCC_FLAGS, *table[name], "-Rpass-analysis=kernel-resource-usage",
               f"-I{INCLUDE}", SRC, "-o", out + ".tmp"]
        if verbose:
            print(" ".join(cmd), flush=True)
        res = subprocess.run(cmd, capture_output=True, text=True)
        if res.returncode != 0:
            raise RuntimeError(f"hipcc failed for variant {name} ({res.returncode}):\n{res.stderr[-4000:]}")
        os.replace(out + ".tmp", out)
        only = "k_reorder_quant_i4" if name in QGZ_STORE_VARIANTS else "k_dequant_reduce"
        return name, out, _resources(res.stderr, only)

    report, paths = {}, []
    with concurrent.futures.ThreadPoolExecutor(max_workers=max(1, jobs)) as ex:
        for name, out, res in ex.map(one, names):
            report[name] = {"defines": table[name], "kernels": res,
                            "group": ("receive" if name in RECEIVE_VARIANTS else
                                      "qgz_store" if name in QGZ_STORE_VARIANTS else "timeline")}
            paths.append(out)
    rpath = os.path.join(VARIANTS_DIR, "resources.json")
    old = {}
    if os.path.exists(rpath):
        with open(rpath) as f:
            old = json.load(f)
    old.update(report)
    with open(rpath, "w") as f:
        json.dump(old, f, indent=1)
    return paths


if __name__ == "__main__":
    if "--variants" in sys.argv:
        for p in build_variants(verbose="-v" in sys.argv):
            print(p)
    else:
        build(verbose="-v" in sys.argv, save_temps="--save-temps" in sys.argv)
