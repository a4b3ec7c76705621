"""The CPU oracle and the input generator under AddressSanitizer and
UndefinedBehaviorSanitizer: both C libraries are rebuilt with
-fsanitize=address,undefined (gcc, host code only) in a temporary copy of the
tree, and the oracle's pin tests, the generator's tests and the range-split
oracle runs execute there with the sanitizer runtime preloaded.  Any invalid
memory access or undefined behaviour aborts the run."""
import os
import shutil
import subprocess
import sys

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
TESTS = ["tests/test_oracle_quant.py", "tests/test_oracle_qgz.py", "tests/test_oracle_convert.py",
         "tests/test_synth.py", "tests/test_oracle_ranges.py", "tests/test_hop_count.py"]
SAN = ["-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
       "-fno-sanitize-recover=all"]


def runtime(name):
    path = subprocess.run(["gcc", f"-print-file-name={name}"], capture_output=True,
                          text=True).stdout.strip()
    return path if os.path.isabs(path) and os.path.exists(path) else None


@pytest.mark.slow
def test_oracle_and_generator_under_sanitizers(tmp_path):
    asan = runtime("libasan.so")
    if asan is None:
        pytest.skip("gcc has no AddressSanitizer runtime here")
    d = str(tmp_path)
    for sub in ("oracle", "synth"):
        shutil.copytree(os.path.join(ROOT, sub), os.path.join(d, sub),
                        ignore=shutil.ignore_patterns("*.so", "__pycache__"))
    shutil.copytree(HERE, os.path.join(d, "tests"),
                    ignore=shutil.ignore_patterns("__pycache__", "*.so", "native"))
    shutil.copy(os.path.join(ROOT, "pytest.ini"), d)
    # the same build scripts, with the optimisation flag swapped for the sanitizers
    for script in ("oracle/build.py", "synth/build.py"):
        p = os.path.join(d, script)
        src = open(p).read()
        assert src.count('"-O2"') == 1, script
        open(p, "w").write(src.replace('"-O2"', ", ".join(f'"{f}"' for f in SAN)))
    env = dict(os.environ)
    env.update(LD_PRELOAD=asan, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1", ZPQ_SYNTH_THREADS="4",
               ZPQ_TEST_THREADS="4")
    build = subprocess.run([sys.executable, "-c",
                            "from oracle import build as o; from synth import build as s; "
                            "o.build(); s.build()"], cwd=d, env=env, capture_output=True,
                           text=True, timeout=600)
    assert build.returncode == 0, build.stdout + build.stderr
    for lib in ("oracle/libzpq_ref.so", "synth/libzpq_synth.so"):      # really instrumented
        syms = subprocess.run(["nm", "-D", os.path.join(d, lib)], capture_output=True,
                              text=True).stdout
        assert "__asan_report" in syms and "__ubsan_handle" in syms, lib
    # the runtime catches a planted out-of-bounds read in this environment
    bad = os.path.join(d, "oob.c")
    open(bad, "w").write("#include <stdlib.h>\nint main(int c, char** v) {\n"
                         "  int* a = malloc(4 * sizeof(int));\n  return a[c + 3];\n}\n")
    subprocess.run(["gcc", *SAN, bad, "-o", bad[:-2]], check=True)
    probe = subprocess.run([bad[:-2]], capture_output=True, text=True, env=env)
    assert probe.returncode != 0 and ("heap-buffer-overflow" in probe.stderr or
                                      "runtime error" in probe.stderr), probe.stderr[-2000:]
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-m", "not slow and not gpu",
                        *TESTS], cwd=d, env=env, capture_output=True, text=True, timeout=1800)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    assert "AddressSanitizer" not in out and "runtime error" not in out, out[-4000:]
