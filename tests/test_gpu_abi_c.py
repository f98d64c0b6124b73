"""The codec from a plain C program on the GPU: tests/abi_c/gpu_client.c allocates
device memory with the HIP runtime API, calls libcfz only through include/cfz.h
(no Python, no torch) and compares every step's codes, scales, states and bf16
output byte for byte with the C oracle, over int4/int2, group sizes 32-128, the
three error-feedback modes and fp32/bf16 state; then cfz_lowrank from C, its
reconstruction within 1e-3 of the oracle's; then the low-rank error-feedback loop
with the plain and the deferred sender, bit-identical step by step."""
import os
import shutil
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
INC = os.path.join(ROOT, "include")
LIBDIR = os.path.join(ROOT, "diffusion_activation_residual_amd")
ORACLE_DIR = os.path.join(ROOT, "oracle")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


def test_c_client_runs_the_codec_bit_exact(tmp_path):
    import torch
    if torch.cuda.device_count() == 0:  # counting devices does not initialise the GPU here
        pytest.skip("no GPU")
    if shutil.which("gcc") is None:
        pytest.skip("gcc not available")
    for lib in (os.path.join(LIBDIR, "libcfz.so"), os.path.join(ORACLE_DIR, "libcfz_oracle.so")):
        assert os.path.exists(lib), f"{lib} is not built"
    exe = tmp_path / "gpu_client"
    rpath = ":".join((LIBDIR, ORACLE_DIR, os.path.join(ROCM, "lib")))
    r = subprocess.run(["gcc", "-std=c11", "-Wall", "-Wextra", "-Werror", "-D__HIP_PLATFORM_AMD__",
                        "-I", os.path.join(ROCM, "include"), "-I", INC,
                        os.path.join(ROOT, "tests", "abi_c", "gpu_client.c"),
                        "-L", LIBDIR, "-lcfz", "-L", ORACLE_DIR, "-l:libcfz_oracle.so",
                        "-L", os.path.join(ROCM, "lib"), "-lamdhip64", "-lm", "-Wl,-rpath," + rpath,
                        "-o", str(exe)], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    print("[gpu] C client", file=sys.stderr, flush=True)
    run = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120)
    print(run.stdout, file=sys.stderr, flush=True)
    assert run.returncode == 0 and run.stdout.strip().endswith("OK"), run.stdout + run.stderr
