"""The C ABI from C: include/cfz.h compiles on its own as C11 and as C++17 with warnings
as errors, and a plain C client (tests/abi_c/abi_check.c) links against libcfz.so and
exercises the host-side entry points (sizes, status strings, validation) without a GPU."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
INC = os.path.join(ROOT, "include")
LIBDIR = os.path.join(ROOT, "diffusion_activation_residual_amd")


@pytest.mark.skipif(shutil.which("gcc") is None or shutil.which("g++") is None,
                    reason="gcc/g++ not available")
def test_header_is_self_contained_c_and_cxx(tmp_path):
    for comp, std, ext in (("gcc", "-std=c11", "c"), ("g++", "-std=c++17", "cpp")):
        src = tmp_path / f"inc.{ext}"
        src.write_text('#include "cfz.h"\nint main(void) { return cfz_abi_version() < 0; }\n')
        r = subprocess.run([comp, std, "-Wall", "-Wextra", "-Werror", "-pedantic", "-I", INC,
                            "-c", str(src), "-o", str(tmp_path / f"inc_{ext}.o")],
                           capture_output=True, text=True)
        assert r.returncode == 0, r.stderr


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
def test_c_client_links_and_validates(tmp_path):
    if not os.path.exists(os.path.join(LIBDIR, "libcfz.so")):
        pytest.skip("libcfz.so is not built")
    exe = tmp_path / "abi_check"
    r = subprocess.run(["gcc", "-std=c11", "-Wall", "-Wextra", "-Werror", "-I", INC,
                        os.path.join(ROOT, "tests", "abi_c", "abi_check.c"), "-L", LIBDIR,
                        "-lcfz", "-Wl,-rpath," + LIBDIR, "-o", str(exe)],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    run = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120)
    assert run.returncode == 0 and run.stdout.strip() == "OK", run.stdout + run.stderr
