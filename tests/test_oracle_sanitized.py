"""The oracle's pins run again against a copy of the C oracle built with
AddressSanitizer and UndefinedBehaviorSanitizer, every report fatal: an
out-of-bounds access, a use after free, a signed overflow or an invalid shift
in the oracle fails this test."""
import os
import subprocess
import sys

import pytest

from conftest import ROOT


def test_oracle_pins_under_asan_and_ubsan(tmp_path):
    import oracle
    lib = oracle.build(out=str(tmp_path / "_liborc_san.so"), sanitize=True)
    env = dict(os.environ)
    env["WQ_ORACLE_LIB"] = lib
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=1"
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1"
    if env.get("LD_PRELOAD"):
        # the ASan runtime must be loaded first; a preload set by the
        # environment is left as it is, and this run is skipped
        pytest.skip("LD_PRELOAD is already set by the environment")
    libasan = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True, text=True,
                             check=True).stdout.strip()
    env["LD_PRELOAD"] = libasan
    res = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                          os.path.join(ROOT, "tests", "test_oracle_pins.py")],
                         cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    out = res.stdout + res.stderr
    assert "AddressSanitizer" not in out and "runtime error" not in out, out[-4000:]
    assert res.returncode == 0, out[-4000:]
    assert " passed" in out
