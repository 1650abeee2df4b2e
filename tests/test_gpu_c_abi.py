"""The library driven from C: tests/c_abi/dit_c_check (built by
__graft_entry__.build()) calls the C entry points with hipMalloc'd buffers on
a HIP stream, with no Python or torch in the process, and compares every
output bit for bit with the CPU oracle.  Every entry point of dit.h and
dit_producers.h: LN + AdaLN modulate, RMSNorm-scale, RMSNorm-tanh-residual,
residual gate-add, standalone modulate, the gated residual + LN producer
and both E4M3 producers (codes byte for byte) on [37 x 1032] (strided and
per-token), [9 x 8192] and [64 x 3072]; Q/K RMSNorm + RoPE on two streams
of a [2, 3+5, 3, 128] joint buffer and its destination-major form (three
destinations); the Wan modulation table on [6, 1, 37, 1040]; and the
statuses of bad calls as a C caller sees them."""
import os
import re
import subprocess
import sys

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
BIN = os.path.join(HERE, "c_abi", "dit_c_check")


@pytest.mark.gpu
def test_c_program_matches_the_oracle():
    assert os.path.exists(BIN), "tests/c_abi/dit_c_check is not built (run __graft_entry__.build())"
    print("running", BIN, flush=True)
    res = subprocess.run([BIN], capture_output=True, text=True, timeout=120)
    sys.stdout.write(res.stdout[-4000:])
    assert res.returncode == 0, res.stdout[-3000:] + res.stderr[-2000:]
    assert re.search(r"^c-abi check: [1-9]\d* cases, 0 failed$", res.stdout, re.M), res.stdout[-2000:]
