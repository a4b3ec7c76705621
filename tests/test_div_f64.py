"""The binary64 route the GPU kernels take for divisions with binary32
operands -- the scale of fp32 blocks and of the hop-1 requantization of fp32
sums, their codes, and the hop-2 average -- checked on the CPU against IEEE
binary32 division (tests/div_f64_check.c): the scale for every positive
finite fp32 absmax (qmax 7 and 127), codes for every value within 16 ulp of
every rounding boundary of quantizer-produced scales in every binade, and
the average for sums next to rounding boundaries of the quotient across
65 536 integer, 81 power-of-two and 200 000 random divisors.  Also the
hop-1 requantization's faster code route (one binary32 product, the
binary64 route only for values within 2^-19 of a half-integer quotient) on
the same near-boundary values.  A planted binary32 product and a planted
too-narrow margin must be caught."""
import os
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
THREADS = str(max(1, min(8, os.cpu_count() or 1)))


def build(tmp_path_factory, name, defines=()):
    exe = str(tmp_path_factory.mktemp("divf64") / name)
    subprocess.run(["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-pthread", *defines,
                    os.path.join(HERE, "div_f64_check.c"), "-o", exe, "-lm"], check=True)
    return exe


@pytest.fixture(scope="module")
def checker(tmp_path_factory):
    return build(tmp_path_factory, "div_f64_check")


@pytest.fixture(scope="module")
def planted(tmp_path_factory):
    return build(tmp_path_factory, "div_f64_planted", ["-DPLANT_FP32_PRODUCT"])


@pytest.fixture(scope="module")
def planted_margin(tmp_path_factory):
    return build(tmp_path_factory, "div_f64_planted_margin", ["-DPLANT_NARROW_MARGIN"])


def run(exe, *args):
    out = subprocess.run([exe, *args], check=True, capture_output=True, text=True).stdout.split()
    assert out[0] == "mismatches" and out[2] == "cases", out
    return int(out[1]), int(out[3])


@pytest.mark.slow
@pytest.mark.parametrize("qmax", [7, 127])
def test_scale_every_fp32_absmax(checker, qmax):
    bad, cases = run(checker, "scale", str(qmax), THREADS)
    assert cases == 0x7F7FFFFF and bad == 0, (bad, cases)


@pytest.mark.slow
@pytest.mark.parametrize("qmax", [7, 127])
def test_codes_next_to_rounding_boundaries(checker, qmax):
    bad, cases = run(checker, "codes", str(qmax), THREADS)
    assert bad == 0 and cases > (2 * 10 ** 8 if qmax == 7 else 4 * 10 ** 9), (bad, cases)


def test_fast_requant_codes_next_to_rounding_boundaries(checker):
    """qmax 7 (the hop-1 requantization): every value takes the route the
    kernel gives it, and each code equals the definition's."""
    bad, cases = run(checker, "fastcodes", "7", THREADS)
    assert bad == 0 and cases > 2 * 10 ** 8, (bad, cases)


@pytest.mark.slow
def test_average_next_to_rounding_boundaries(checker):
    bad, cases = run(checker, "mean", THREADS)
    assert bad == 0 and cases > 4 * 10 ** 8, (bad, cases)


def test_planted_binary32_product_is_caught(planted):
    for args in (("codes", "7", THREADS), ("mean", THREADS)):
        bad, cases = run(planted, *args)
        assert bad > 0, (args, cases)


def test_planted_narrow_margin_is_caught(planted_margin):
    bad, cases = run(planted_margin, "fastcodes", "7", THREADS)
    assert bad > 0, cases
