"""The GPU quantizer's arithmetic shortcuts for 16-bit inputs, checked by
exhaustion on the CPU (tests/div_check.c): for every positive finite fp16 or
bf16 absmax a, the scale fl32(a/qmax) from a product and one residual
correction (a >= 2^-90) equals the IEEE quotient; and for every a with
s = fl32(a/qmax) >= 2^-100, every value 0 <= x <= a of the same type and
either float next to the exact 1/s, one residual correction of x * r rounds
to the same integer as the IEEE quotient fl32(x/s).  (fp32 values take a
binary64 route instead, checked by tests/test_div_f64.py.)"""
import os
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))


@pytest.fixture(scope="module")
def checker(tmp_path_factory):
    exe = str(tmp_path_factory.mktemp("div") / "div_check")
    subprocess.run(["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-pthread",
                    os.path.join(HERE, "div_check.c"), "-o", exe, "-lm"], check=True)
    return exe


@pytest.mark.slow
@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("qmax", [127, 7])
def test_one_correction_is_exact_for_16bit_inputs(checker, dtype, qmax):
    threads = str(max(1, min(8, os.cpu_count() or 1)))
    out = subprocess.run([checker, dtype, str(qmax), threads], check=True, capture_output=True,
                         text=True).stdout.split()
    assert out[0] == "mismatches" and int(out[1]) == 0, out
    assert int(out[3]) > 10 ** 9              # about half of all (a, x) pairs, x >= 0, two r each
    assert out[4] == "scale_mismatches" and int(out[5]) == 0, out
    assert int(out[7]) > 27000                 # every absmax >= 2^-90
