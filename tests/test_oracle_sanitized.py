"""The CPU oracle built with AddressSanitizer and UndefinedBehaviorSanitizer (gcc), driven
through every entry point on small ragged inputs by tests/sanitize/oracle_driver.c: no
out-of-bounds access, use after free, leak, signed overflow or other undefined behaviour."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
def test_oracle_under_asan_and_ubsan(tmp_path):
    exe = tmp_path / "oracle_driver"
    cmd = ["gcc", "-std=c11", "-O1", "-g", "-fno-omit-frame-pointer", "-ffp-contract=off",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           os.path.join(ROOT, "oracle", "cfz_oracle.c"),
           os.path.join(ROOT, "tests", "sanitize", "oracle_driver.c"), "-lm", "-o", str(exe)]
    build = subprocess.run(cmd, capture_output=True, text=True)
    if build.returncode != 0 and "sanitize" in build.stderr:
        pytest.skip("this gcc cannot build sanitizer binaries: " + build.stderr[-300:])
    assert build.returncode == 0, build.stderr
    # a library preloaded by the environment may come before the ASan runtime; ASan's own
    # option accepts that order
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:verify_asan_link_order=0",
               UBSAN_OPTIONS="print_stacktrace=1")
    run = subprocess.run([str(exe)], capture_output=True, text=True, env=env, timeout=300)
    assert run.returncode == 0 and run.stdout.strip() == "OK", run.stdout + run.stderr
