"""Build tests/native/c_api_check (test infrastructure): a plain C program
using libzpq through include/zpq.h and the HIP runtime's C API, linked with
the CPU oracle for the expected bytes.  Host code only (gcc); needs
libzpq.so and the oracle's library built first."""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
EXE = os.path.join(HERE, "c_api_check")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


def build(verbose: bool = False) -> str:
    pkg = os.path.join(ROOT, "block_quantized_communication_amd")
    orc = os.path.join(ROOT, "oracle")
    cmd = ["gcc", "-O2", "-std=c11", "-Wall", "-D__HIP_PLATFORM_AMD__",
           f"-I{ROCM}/include", f"-I{os.path.join(ROOT, 'include')}",
           os.path.join(HERE, "c_api_check.c"), "-o", EXE + ".tmp",
           f"-L{pkg}", "-lzpq", f"-L{orc}", "-lzpq_ref", f"-L{ROCM}/lib", "-lamdhip64", "-lm",
           "-Wl,-rpath,$ORIGIN/../../block_quantized_communication_amd",
           "-Wl,-rpath,$ORIGIN/../../oracle", f"-Wl,-rpath,{ROCM}/lib"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(EXE + ".tmp", EXE)
    return EXE


if __name__ == "__main__":
    build(verbose="-v" in sys.argv)
