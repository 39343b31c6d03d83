"""The CPU oracle's C code (oracle/gdr_oracle.c) built with gcc's
AddressSanitizer and UndefinedBehaviorSanitizer and driven through every
gate and decay mode, head and column selections, one and several threads,
and its argument checks (tests/c_oracle/sanitize_driver.c). A memory error,
a leak or undefined behaviour makes the run fail."""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)


def test_oracle_under_address_and_undefined_behaviour_sanitizers(tmp_path):
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("gcc not found")
    exe = str(tmp_path / "oracle_sanitize")
    cmd = [gcc, "-std=c11", "-O1", "-g", "-fno-omit-frame-pointer", "-ffp-contract=off",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-pthread",
           os.path.join(HERE, "c_oracle", "sanitize_driver.c"), os.path.join(ROOT, "oracle", "gdr_oracle.c"),
           "-o", exe, "-lm"]
    build = subprocess.run(cmd, capture_output=True, text=True)
    if build.returncode != 0 and "asan" in (build.stderr or "").lower() and "cannot find" in build.stderr:
        pytest.skip("the sanitizer runtimes are not installed")
    assert build.returncode == 0, build.stderr
    # verify_asan_link_order=0: the run does not require the sanitizer
    # runtime to be the first library the process loads.
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=1:verify_asan_link_order=0",
               UBSAN_OPTIONS="print_stacktrace=1")
    run = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    assert run.returncode == 0, run.stdout + run.stderr
    assert "all checks passed" in run.stdout
