"""Builds the HIP epilogue library, modulation_bf16_row_amd/libdit.so, for gfx950.

Every source is compiled with hipcc for gfx950 only, in parallel, into
_build/, then linked into one shared library with a plain C ABI.

Floating-point flags: no contraction into fused multiply-add
(-ffp-contract=off; FAST-mode code writes fmaf explicitly), no fast-math,
correctly rounded fp32 division and square root, fp32 denormals kept, and
no packed-fp32 instructions (-packed-fp32-ops; the host pass prints a
harmless warning that it does not know this feature).
"""
import concurrent.futures
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libdit.so")

SOURCES = ["dit_ln.hip", "dit_gate_ln.hip", "dit_rms.hip", "dit_gate.hip", "dit_mod.hip",
           "dit_qkv.hip", "dit_modtab.hip", "dit_probe.hip", "dit_abi.cpp"]

ARCH = "gfx950"
COMMON = [
    "-std=c++17", "-O3", "-fPIC", "-Wall",
    "-ffp-contract=off", "-fno-fast-math",
    "-fhip-fp32-correctly-rounded-divide-sqrt", "-fno-gpu-flush-denormals-to-zero",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", INCLUDE, "-I", CSRC,
]


def _hipcc():
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", "hipcc"):
        if cand and (os.path.sep not in cand or os.path.exists(cand)):
            return cand
    raise RuntimeError("hipcc not found")


def _compile(src, verbose, build_dir, extra):
    obj = os.path.join(build_dir, os.path.splitext(src)[0] + ".o")
    cmd = [_hipcc(), f"--offload-arch={ARCH}", *COMMON, *extra, "-c", os.path.join(CSRC, src),
           "-o", obj]
    if src.endswith(".cpp"):
        cmd = [_hipcc(), *COMMON, *extra, "-D__HIP_PLATFORM_AMD__", "-c",
               os.path.join(CSRC, src), "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in res.stderr.splitlines() if noise not in l)
    if res.returncode != 0:
        raise RuntimeError(f"compile failed: {src}\n{err}")
    if verbose and err.strip():
        print(err, flush=True)
    return obj


def build(verbose: bool = False, jobs: int = 7, lib: str = LIB, extra_flags=()) -> str:
    """Compiles and links the library; `lib` and `extra_flags` allow side
    builds (e.g. with -D macros) without touching the default one."""
    build_dir = BUILD if lib == LIB else os.path.join(BUILD, os.path.basename(lib) + ".d")
    os.makedirs(build_dir, exist_ok=True)
    extra = list(extra_flags)
    with concurrent.futures.ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose, build_dir, extra), SOURCES))
    tmp = lib + ".tmp"
    cmd = [_hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, lib)
    return lib


if __name__ == "__main__":
    build(verbose="-v" in sys.argv)
