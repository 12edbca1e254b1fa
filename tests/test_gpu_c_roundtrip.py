"""The C ABI from a plain C program on the GPU (no Python, no torch in it).

gcc builds tests/c_abi/gpu_roundtrip.c against include/qknorm_rope.h, HIP's C
runtime API, the built libqknorm_rope.so and the CPU oracle; the program
uploads a fused QKV buffer, calls qknorm_rope_fused, and checks Q and K
against the oracle (bf16 bar, max_abs <= 1.6e-2) and V bit for bit; then the
AdaLN step and group norm + SiLU in its two-pass and lagged schedules, each
against the oracle.
"""
import os
import shutil
import subprocess

import pytest

import diffusion_transformer_qk_amd as qkr

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_c_program_runs_the_pass_on_the_gpu(tmp_path, oracle_lib):
    lib_dir = os.path.dirname(qkr.LIB_PATH)
    oracle_dir = os.path.dirname(oracle_lib.LIB)
    exe = os.path.join(tmp_path, "gpu_roundtrip")
    subprocess.run(["gcc", "-std=c99", "-O1", "-Wall", "-Werror", "-D__HIP_PLATFORM_AMD__",
                    "-I", os.path.join(ROOT, "include"), "-I", os.path.join(ROCM, "include"),
                    os.path.join(ROOT, "tests", "c_abi", "gpu_roundtrip.c"),
                    "-L", lib_dir, "-lqknorm_rope", "-L", oracle_dir, "-lqkr_oracle",
                    "-L", os.path.join(ROCM, "lib"), "-lamdhip64", "-lm",
                    "-Wl,-rpath," + lib_dir, "-Wl,-rpath," + oracle_dir,
                    "-Wl,-rpath," + os.path.join(ROCM, "lib"), "-o", exe], check=True)
    out = subprocess.run([exe], capture_output=True, text=True, timeout=120)
    assert out.returncode == 0 and out.stdout.strip().endswith("ok"), out.stdout + out.stderr
    print(out.stdout.strip())
