"""The checked build of the host logic, run on the CPU.

``build_hostcheck.py`` compiles ``sq_host.cpp`` with its bounds asserts
(SQ_HOSTCHECK) and AddressSanitizer + UndefinedBehaviorSanitizer on the host
code, with stub launchers that check every launch's arguments and start no
kernel.  A child process with the ASan runtime preloaded then runs the host
ABI tests and ``test_entry_points.py`` against that library; any sanitizer
report, failed assert or test failure fails this test."""
import os
import subprocess
import sys

import pytest

from conftest import ROOT

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, HERE)
import build_hostcheck as B  # noqa: E402


def test_host_logic_under_sanitizers_and_bounds_asserts():
    rt = B.asan_runtime()
    if rt is None or not os.path.exists(B.HIPCC):
        pytest.skip("no hipcc or clang ASan runtime in this image")
    lib = B.build(os.path.join(ROOT, "_build", "hostcheck"))
    env = dict(os.environ)
    env.update({
        "SQ_LIBRARY": lib,
        "SQ_HOSTCHECK_CHILD": "1",
        "LD_PRELOAD": rt,
        "ASAN_OPTIONS": "detect_leaks=0:abort_on_error=1",
        "UBSAN_OPTIONS": "print_stacktrace=1:halt_on_error=1",
    })
    env.pop("SQ_VALIDATE", None)  # slot validation copies from the device
    cmd = [sys.executable, "-m", "pytest", "-q", "-s", "-p", "no:cacheprovider",
           os.path.join(ROOT, "tests", "test_abi_host.py"),
           os.path.join(ROOT, "tests", "test_calib_stats_pins.py"),
           os.path.join(HERE, "test_entry_points.py")]
    r = subprocess.run(cmd, cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-6000:]
    assert "SQ_CHECK failed" not in out and "runtime error" not in out, out[-6000:]
    assert "ERROR: AddressSanitizer" not in out, out[-6000:]
