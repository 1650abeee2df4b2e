"""CPU check of the exact multiply-high division the flat kernels use to split a
lane's group index (csrc/dit_divide.hpp): for 1 <= d < 2^32, floor(n M / 2^64)
with M = reciprocal(d) equals floor(n / d) for every n < 2^32.  The library's
own reciprocal() is compiled for the host (tests/divide_check.cpp) with a host
stand-in for the 64-bit multiply-high; all 2^32 numerators for the divisors of
the Wan 720p table (1280 groups per row, 75600 tokens), edge, exact-multiple
and pseudo-random numerators for others (1, powers of two, odd primes, the
Qwen-Image shapes, values near 2^31 and 2^32)."""
import os
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "modulation_bf16_row_amd", "csrc")


@pytest.fixture(scope="module")
def checker(tmp_path_factory):
    exe = str(tmp_path_factory.mktemp("div") / "divide_check")
    cmd = ["/opt/rocm/bin/hipcc", "-std=c++17", "-O2", "-D__HIP_PLATFORM_AMD__", "-I", CSRC,
           os.path.join(ROOT, "tests", "divide_check.cpp"), "-o", exe]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr
    return exe


def _run(exe, args):
    res = subprocess.run([exe] + [str(a) for a in args], capture_output=True, text=True,
                         timeout=600)
    assert res.returncode == 0, res.stdout + res.stderr


def test_edge_and_random_numerators(checker):
    divisors = [1, 2, 3, 4, 5, 7, 8, 640, 768, 1024, 1280, 3, 4608, 9216, 75600, 453600, 65535,
                65536, 1000003, (1 << 31) - 1, 1 << 31, (1 << 31) + 1, (1 << 32) - 1,
                3000000019]
    _run(checker, divisors)


def test_all_numerators_for_the_wan_divisors(checker):
    _run(checker, ["--all", 1280, 75600])
