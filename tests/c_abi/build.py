"""Builds tests/c_abi/dit_c_check, a host program that drives libdit.so through
its C ABI and compares with the CPU oracle (test infrastructure).  Needs
libdit.so and oracle/liboracle.so built first."""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
PKG = os.path.join(ROOT, "modulation_bf16_row_amd")
ORACLE = os.path.join(ROOT, "oracle")
OUT = os.path.join(HERE, "dit_c_check")


def build(verbose=False, out=OUT):
    # Host code only: the program includes the C headers and links the
    # libraries, so the plain host compiler builds it.
    cmd = ["g++", "-std=c++17", "-O2", "-Wall", "-Wextra", "-D__HIP_PLATFORM_AMD__",
           "-I", "/opt/rocm/include", "-I", os.path.join(ROOT, "include"), "-I", ORACLE,
           os.path.join(HERE, "dit_c_check.cpp"), "-o", out + ".tmp",
           "-L", PKG, "-ldit", "-L", ORACLE, "-loracle", "-L", "/opt/rocm/lib", "-lamdhip64",
           "-Wl,-rpath,/opt/rocm/lib",
           "-Wl,-rpath,$ORIGIN/../../modulation_bf16_row_amd", "-Wl,-rpath,$ORIGIN/../../oracle",
           "-Wl,-rpath," + PKG, "-Wl,-rpath," + ORACLE]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("building the C-ABI check failed:\n" + res.stderr[-3000:])
    os.replace(out + ".tmp", out)
    return out


if __name__ == "__main__":
    build(verbose="-v" in sys.argv)
