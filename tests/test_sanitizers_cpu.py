"""The host guard tests and the oracle pins, run again against builds made
with AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

A signed overflow, an out-of-bounds access or any other finding in the guard
arithmetic (dit_abi.cpp, dit_probe_abi.cpp) or in the oracle aborts the inner
pytest run, so this test fails.  The sweep over all 2^32 binary32 inputs is
left out (it adds minutes and no new code path).
"""
import os
import subprocess
import sys

import pytest

import sanitizers

HERE = os.path.dirname(os.path.abspath(__file__))


def test_guards_and_oracle_are_clean_under_asan_and_ubsan(tmp_path):
    try:
        rt = sanitizers.runtime()
    except FileNotFoundError as e:
        pytest.skip(str(e))
    sanitizers.build_stub(str(tmp_path / "libstub.so"))
    sanitizers.build_oracle(str(tmp_path / "liboracle.so"))
    env = dict(os.environ)
    env.update({
        "LD_PRELOAD": rt,
        "ASAN_OPTIONS": "detect_leaks=0:abort_on_error=1",
        "UBSAN_OPTIONS": "print_stacktrace=1:halt_on_error=1",
        sanitizers.ENV_DIR: str(tmp_path),
    })
    cmd = [sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider", "-m", "not gpu",
           os.path.join(HERE, "test_abi_cpu.py"), os.path.join(HERE, "test_oracle_pins.py"),
           "-k", "not all_binary32 and not library_exports and not check_program"]
    res = subprocess.run(cmd, env=env, capture_output=True, text=True, timeout=900)
    out = res.stdout + res.stderr
    assert res.returncode == 0, out[-6000:]
    assert "runtime error" not in out and "AddressSanitizer" not in out, out[-6000:]
    assert " passed" in out
