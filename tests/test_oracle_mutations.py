"""The oracle's pins catch plausible mistakes.  Each case plants one mistake
in a copy of oracle/zpq_ref.c (rounding mode, reciprocal instead of
division, a dropped clamp, nibble order or sign, the slice permutation, the
summation order, a scale index, the absmax range, qmax, the accumulator
start, the bf16 rounding), rebuilds that copy and runs the
oracle's pin tests against it: every mutant must fail at least one pin by an
assertion (not by a build or import error), and the unmutated copy must pass.
Runs on the CPU only, in temporary directories.  (Adding in double and
rounding to fp32 is not a mistake to plant: for two fp32 operands it returns
the fp32 sum exactly, since double has more than 2*24 + 2 significand bits.)"""
import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
PIN_TESTS = ["tests/test_oracle_quant.py", "tests/test_oracle_qgz.py",
             "tests/test_oracle_convert.py"]

# name -> (text in oracle/zpq_ref.c, replacement)
MUTANTS = {
    "round_half_away": ("float r = rintf(t);", "float r = roundf(t);"),
    "truncate": ("float r = rintf(t);", "float r = truncf(t);"),
    "scale_by_reciprocal": ("float s = a / fq;", "float s = a * (1.0f / fq);"),
    "code_by_reciprocal": ("float t = xb[i] / s;", "float t = xb[i] * (1.0f / s);"),
    "no_clamp": ("if (r > fq) r = fq;", ";"),
    "nibbles_swapped": ("packed[k] = (uint8_t)(lo | (hi << 4));",
                        "packed[k] = (uint8_t)(hi | (lo << 4));"),
    "nibble_unsigned": ("return (int8_t)(v >= 8 ? (int)v - 16 : (int)v);", "return (int8_t)v;"),
    "reorder_source_formula": ("int64_t s = (int64_t)m * L + j;", "int64_t s = (int64_t)j * N + m;"),
    "reorder_position_formula": ("int64_t p = (int64_t)j * N + m;",
                                 "int64_t p = (int64_t)m * L + j;"),
    "sources_reversed": ("for (int32_t i = 0; i < K && rc == REF_OK; ++i) {",
                         "for (int32_t i = K - 1; i >= 0 && rc == REF_OK; --i) {"),
    "average_by_reciprocal": ("out[i] = acc[i] / divisor;",
                              "out[i] = acc[i] * (1.0f / divisor);"),
    "wrong_scale_index": ("float s = scales[i / block];",
                          "float s = scales[(i + 1) / block < n / block ? (i + 1) / block : "
                          "i / block];"),
    "absmax_skips_last": ("for (int32_t i = 0; i < block; ++i) {\n            float v = fabsf(xb[i]);",
                          "for (int32_t i = 0; i < block - 1; ++i) {\n            float v = "
                          "fabsf(xb[i]);"),
    "f16_round_half_away": ("float r = rintf(m);", "float r = roundf(m);"),
    "int4_qmax_8": ("rc = zpq_ref_block_quant(xf, n, block, 7, q, scales);",
                    "rc = zpq_ref_block_quant(xf, n, block, 8, q, scales);"),
    "requant_qmax_6": ("rc = zpq_ref_block_quant(acc, chunk, block, 7, q, out_scales);",
                       "rc = zpq_ref_block_quant(acc, chunk, block, 6, q, out_scales);"),
    "accumulator_not_zero": ("for (int64_t e = 0; e < chunk; ++e) acc[e] = 0.0f;",
                             "for (int64_t e = 0; e < chunk; ++e) acc[e] = 1e-30f;"),
    "bf16_truncates": ("float r = round_to_quantum(a, quantum);   /* overflows",
                       "float r = truncf(a / quantum) * quantum;   /* overflows"),
}


def run_pins(workdir, name, source):
    """Copy the oracle and its pin tests to workdir/name with `source` as the
    oracle's C file; run the pins; return (returncode, summary line, output)."""
    d = os.path.join(workdir, name)
    shutil.copytree(os.path.join(ROOT, "oracle"), os.path.join(d, "oracle"),
                    ignore=shutil.ignore_patterns("*.so", "__pycache__"))
    shutil.copytree(HERE, os.path.join(d, "tests"),
                    ignore=shutil.ignore_patterns("__pycache__", "*.so"))
    shutil.copy(os.path.join(ROOT, "pytest.ini"), d)
    with open(os.path.join(d, "oracle", "zpq_ref.c"), "w") as f:
        f.write(source)
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-m", "not slow", *PIN_TESTS],
                       cwd=d, capture_output=True, text=True, timeout=600)
    lines = [l for l in r.stdout.splitlines() if l.strip()]
    return r.returncode, (lines[-1] if lines else ""), r.stdout + r.stderr


@pytest.mark.slow
def test_pins_catch_every_planted_mistake(tmp_path):
    src = open(os.path.join(ROOT, "oracle", "zpq_ref.c")).read()
    jobs = {"unmutated": src}
    for name, (a, b) in MUTANTS.items():
        assert src.count(a) == 1, f"{name}: the text to mutate is not in the oracle exactly once"
        jobs[name] = src.replace(a, b, 1)
    workers = max(1, min(6, (os.cpu_count() or 2) - 1))
    with ThreadPoolExecutor(workers) as ex:
        futs = {name: ex.submit(run_pins, str(tmp_path), name, s) for name, s in jobs.items()}
        res = {name: f.result() for name, f in futs.items()}
    rc, summary, out = res.pop("unmutated")
    assert rc == 0, f"the unmutated copy fails its pins: {summary}\n{out[-2000:]}"
    missed = [n for n, (rc, _, _) in res.items() if rc == 0]
    assert not missed, f"mutants not caught by any pin: {missed}"
    # caught by a failing assertion, not by a broken build or collection
    broken = [n for n, (rc, s, _) in res.items() if rc != 1 or "failed" not in s or "error" in s]
    assert not broken, {n: res[n][1] for n in broken}
