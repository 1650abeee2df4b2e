"""Every kernel the library builds runs without private memory: each csrc/*.hip
is compiled for gfx950 with the library's own flags to device assembly, and
the code-object metadata of every kernel must show no VGPR or SGPR spills and
no private segment (scratch).  Scratch is the failure mode to guard against:
a per-lane table or an unrolled fix-up loop lowered to private memory adds
HBM traffic to a bandwidth-bound kernel (it once cost the tanh epilogue
6.3 MB of writes per launch)."""
import os
import re
import subprocess
from concurrent.futures import ThreadPoolExecutor

import pytest

from modulation_bf16_row_amd import build

SOURCES = [s for s in build.SOURCES if s.endswith(".hip")]


def _kernels(asm):
    meta = asm[asm.find("amdhsa.kernels"):]
    out = {}
    for blk in re.split(r"\n\s+- \.", meta):
        name = re.search(r"\.name:\s+(\S+)", blk)
        if not name:
            continue
        field = lambda k: int((re.search(r"\." + k + r":\s+(\d+)", blk) or [None, "-1"])[1])
        out[name.group(1)] = dict(vgpr_spill=field("vgpr_spill_count"),
                                  sgpr_spill=field("sgpr_spill_count"),
                                  scratch=field("private_segment_fixed_size"))
    return out


@pytest.fixture(scope="module")
def kernels(tmp_path_factory):
    d = tmp_path_factory.mktemp("asm")

    def compile_one(src):
        out = str(d / (src + ".s"))
        cmd = [build._hipcc(), f"--offload-arch={build.ARCH}", *build.COMMON,
               "--cuda-device-only", "-S", os.path.join(build.CSRC, src), "-o", out]
        res = subprocess.run(cmd, capture_output=True, text=True)
        assert res.returncode == 0, res.stderr[-2000:]
        with open(out) as f:
            return _kernels(f.read())

    with ThreadPoolExecutor(min(8, len(SOURCES))) as ex:
        found = {}
        for ks in ex.map(compile_one, SOURCES):
            found.update(ks)
    return found


def test_every_source_has_kernels(kernels):
    assert len(kernels) > 100           # the row kernels alone instantiate NC = 1..16


def test_no_kernel_spills_or_uses_scratch(kernels):
    bad = {k: v for k, v in kernels.items()
           if v["vgpr_spill"] != 0 or v["sgpr_spill"] != 0 or v["scratch"] != 0}
    assert not bad, sorted(bad.items())[:8]
