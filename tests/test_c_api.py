"""libzpq used from plain C (tests/native/c_api_check.c): the five entry
points through include/zpq.h and the HIP C API, no Python on the path,
compared byte for byte with the oracle's C functions."""
import os
import subprocess

import pytest

EXE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "native", "c_api_check")


def test_c_program_links_against_the_header():
    """Built by __graft_entry__.build(); links libzpq, the oracle and the HIP runtime."""
    assert os.path.exists(EXE), "run __graft_entry__.build() (builds tests/native/c_api_check)"
    out = subprocess.run(["ldd", EXE], capture_output=True, text=True).stdout
    assert "libzpq.so" in out and "libzpq_ref.so" in out and "not found" not in out, out


@pytest.mark.gpu
def test_c_program_matches_oracle():
    print("c_api_check", flush=True)
    r = subprocess.run([EXE], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0 and "c_api_check: ok" in r.stdout, r.stdout + r.stderr
