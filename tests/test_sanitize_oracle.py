"""The oracle built with gcc's address and undefined-behaviour sanitizers
(host code only) and driven over edge inputs by tests/sanitize/oracle_driver.c:
memory errors, leaks and undefined behaviour in the test oracle abort the
driver."""
import os
import shutil
import subprocess

import pytest

from tests.conftest import ROOT

FLAGS = ["-std=c11", "-O1", "-g", "-ffp-contract=off", "-fno-fast-math",
         "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer"]


def test_oracle_under_sanitizers(tmp_path):
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("gcc is not available")
    exe = str(tmp_path / "oracle_driver")
    build = subprocess.run(
        [gcc, *FLAGS, "-I", os.path.join(ROOT, "oracle"), "-o", exe,
         os.path.join(ROOT, "oracle", "oracle.c"),
         os.path.join(ROOT, "tests", "sanitize", "oracle_driver.c"), "-lm"],
        capture_output=True, text=True)
    if build.returncode != 0 and ("asan" in build.stderr or "ubsan" in build.stderr):
        pytest.skip("sanitizer runtimes are not installed: " + build.stderr[-300:])
    assert build.returncode == 0, build.stderr
    # another preloaded library may come first; the driver itself links the runtime
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:verify_asan_link_order=0",
               UBSAN_OPTIONS="print_stacktrace=1")
    run = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=600)
    assert run.returncode == 0 and run.stdout.strip() == "ok", (
        run.returncode, run.stdout[-500:], run.stderr[-3000:])
