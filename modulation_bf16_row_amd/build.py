"""Builds the HIP epilogue library for gfx950.

Every source is compiled with hipcc for gfx950 only, in parallel, into
_build/, then linked twice from the same objects:

  libdit.so        the product: the entry points of include/dit.h and
                   include/dit_producers.h, nothing else exported;
  libdit_probe.so  the same kernel and guard objects plus the probes of the
                   device primitives (include/dit_probe.h) and the
                   dispatch-timing hook (include/dit_timing.h), for the tests
                   and the benchmark's per-kernel timing.

A linker version script limits each library's dynamic symbols to the
declared entry points (and the compiler's per-translation-unit
__hip_cuid_* markers).

Floating-point flags: no contraction into fused multiply-add
(-ffp-contract=off; FAST-mode code writes fmaf explicitly), no fast-math,
correctly rounded fp32 division and square root, fp32 denormals kept, and
no packed-fp32 instructions (-packed-fp32-ops; the host pass prints a
harmless warning that it does not know this feature).
"""
import concurrent.futures
import os
import re
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libdit.so")
PROBE_LIB = os.path.join(PKG, "libdit_probe.so")

# Kernels and the C-ABI guards, shared by both libraries.
KERNELS = ["dit_ln.hip", "dit_gate_ln.hip", "dit_rms.hip", "dit_gate.hip", "dit_mod.hip",
           "dit_qkv.hip", "dit_modtab.hip", "dit_abi.cpp"]
PRODUCT_ONLY = ["dit_timing_off.cpp"]
PROBE_ONLY = ["dit_probe.hip", "dit_probe_abi.cpp"]
SOURCES = KERNELS + PRODUCT_ONLY + PROBE_ONLY

PRODUCT_HEADERS = ["dit.h", "dit_producers.h"]
PROBE_HEADERS = PRODUCT_HEADERS + ["dit_probe.h", "dit_timing.h"]

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


def declared_entry_points(headers):
    """Names of the functions the given include/ headers declare."""
    names = set()
    for h in headers:
        text = re.sub(r"/\*.*?\*/", "", open(os.path.join(INCLUDE, h)).read(), flags=re.S)
        names |= set(re.findall(r"\b(dit_\w+)\s*\(", text))
    return sorted(names)


def _link(objs, headers, out, build_dir, verbose):
    script = os.path.join(build_dir, os.path.basename(out) + ".map")
    with open(script, "w") as f:
        f.write("{\n  global:\n")
        for n in declared_entry_points(headers):
            f.write(f"    {n};\n")
        f.write("    __hip_cuid_*;\n")          # the compiler's per-TU ids stay as they were
        f.write("  local:\n    *;\n};\n")
    tmp = out + ".tmp"
    cmd = [_hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs,
           f"-Wl,--version-script={script}", "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)


def build(verbose: bool = False, jobs: int = 7) -> str:
    """Compiles every source and links libdit.so and libdit_probe.so."""
    os.makedirs(BUILD, exist_ok=True)
    with concurrent.futures.ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = dict(zip(SOURCES, ex.map(lambda s: _compile(s, verbose, BUILD, []), SOURCES)))
    _link([objs[s] for s in KERNELS + PRODUCT_ONLY], PRODUCT_HEADERS, LIB, BUILD, verbose)
    _link([objs[s] for s in KERNELS + PROBE_ONLY], PROBE_HEADERS, PROBE_LIB, BUILD, verbose)
    return LIB


if __name__ == "__main__":
    build(verbose="-v" in sys.argv)
