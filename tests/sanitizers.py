"""Sanitized CPU builds of the host guards and the oracle (test helpers).

The C-ABI guard layer (csrc/dit_abi.cpp and csrc/dit_probe_abi.cpp, linked
with the stand-in launchers of tests/host_stub.cpp) and the oracle
(oracle/dit_oracle.c) are compiled for the host only with AddressSanitizer
and UndefinedBehaviorSanitizer, every finding fatal.  No GPU code is built
here.  The libraries depend on the compiler's shared ASan runtime, which a
Python process must preload (``runtime()``).
"""
import glob
import os
import subprocess

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
INCLUDE = os.path.join(ROOT, "include")
CSRC = os.path.join(ROOT, "modulation_bf16_row_amd", "csrc")
LLVM = "/opt/rocm/llvm/bin"

# Environment variable naming a folder that holds sanitized builds; the test
# fixtures load them from there instead of the ordinary builds.
ENV_DIR = "DIT_SANITIZED_LIBS"

SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-shared-libasan",
       "-fno-omit-frame-pointer", "-g", "-O1", "-fPIC", "-shared"]


def runtime():
    """Path of the shared ASan runtime that matches the compiler."""
    hits = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    if not hits:
        raise FileNotFoundError("clang's shared ASan runtime is not installed")
    return hits[-1]


def build_stub(out):
    cmd = [os.path.join(LLVM, "clang++"), "-x", "c++", "-std=c++17", *SAN, "-w",
           "-D__HIP_PLATFORM_AMD__", "-I", "/opt/rocm/include", "-I", INCLUDE, "-I", CSRC,
           os.path.join(CSRC, "dit_abi.cpp"), os.path.join(CSRC, "dit_probe_abi.cpp"),
           os.path.join(ROOT, "tests", "host_stub.cpp"), "-L", "/opt/rocm/lib", "-lamdhip64",
           "-Wl,-rpath,/opt/rocm/lib", "-o", out]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    return out


def build_oracle(out):
    here = os.path.join(ROOT, "oracle")
    cmd = [os.path.join(LLVM, "clang"), "-std=c11", *SAN, "-ffp-contract=off", "-fno-fast-math",
           "-mfpmath=sse", "-msse2", "-Wall", "-I", here, os.path.join(here, "dit_oracle.c"),
           "-o", out, "-lm"]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    return out


def sanitized_dir():
    """The folder of sanitized builds this process should use, or None."""
    return os.environ.get(ENV_DIR) or None
