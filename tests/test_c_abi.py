"""The public headers compile as C and the library links from a C program.

gcc builds tests/c_abi/abi_check.c against include/*.h and the built
libqknorm_rope.so; the program exercises the argument checks (no GPU call).
"""
import os
import shutil
import subprocess

import pytest

import diffusion_transformer_qk_amd as qkr

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_c_program_builds_and_gets_the_documented_codes(tmp_path):
    lib_dir = os.path.dirname(qkr.LIB_PATH)
    exe = os.path.join(tmp_path, "abi_check")
    subprocess.run(["gcc", "-std=c99", "-Wall", "-Werror", "-pedantic",
                    "-I", os.path.join(ROOT, "include"),
                    os.path.join(ROOT, "tests", "c_abi", "abi_check.c"),
                    "-L", lib_dir, "-lqknorm_rope", "-Wl,-rpath," + lib_dir, "-o", exe],
                   check=True)
    out = subprocess.run([exe], capture_output=True, text=True, timeout=60)
    assert out.returncode == 0 and out.stdout.strip() == "ok", out.stdout + out.stderr
