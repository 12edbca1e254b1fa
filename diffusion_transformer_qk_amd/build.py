"""Compile the HIP library ``libqknorm_rope.so`` for gfx950 with hipcc (and,
beside it, bench.py's data-movement probe ``bench_floor.so``).

Usage:  python -m diffusion_transformer_qk_amd.build [--save-temps DIR]
"""
from __future__ import annotations

import argparse
import os
import shutil
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
SRCS = [os.path.join(PKG, "csrc", "qknorm_rope.hip"),
        os.path.join(PKG, "csrc", "fuse_scale_shift.hip"),
        os.path.join(PKG, "csrc", "group_norm_silu.hip")]
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libqknorm_rope.so")
# bench.py's data-movement probe: its own library, outside libqknorm_rope.so
FLOOR_SRC = os.path.join(ROOT, "bench_floor.hip")
FLOOR_LIB = os.path.join(ROOT, "bench_floor.so")
ARCH = "gfx950"

HIPCC_FLAGS = [
    "--offload-arch=" + ARCH,
    "-O3", "-std=c++17", "-fPIC", "-shared",
    # exact fp32 operation order: no implicit fma contraction, so both cos/sin
    # layouts execute identical arithmetic
    "-ffp-contract=off",
    # no packed fp32 instructions on this target
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall",
]


def hipcc() -> str:
    path = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(path):
        raise RuntimeError("hipcc not found")
    return path


OBJ_DIR = os.path.join(PKG, "_build")


def build(save_temps: str | None = None) -> str:
    """Build the library in-tree and return its path.

    Each source compiles to its own object in parallel (they share no device
    code), then one link makes the shared library.  With ``save_temps`` the
    whole build runs as one hipcc call that keeps its ISA/IR there.
    """
    tmp = LIB + ".tmp%d" % os.getpid()
    if save_temps:
        os.makedirs(save_temps, exist_ok=True)
        cmd = [hipcc(), "--save-temps", *HIPCC_FLAGS, "-I", INCLUDE, *SRCS, "-o", tmp]
        subprocess.run(cmd, check=True, cwd=save_temps)
        os.replace(tmp, LIB)
        return LIB
    os.makedirs(OBJ_DIR, exist_ok=True)
    compile_flags = [f for f in HIPCC_FLAGS if f != "-shared"]
    objs, procs = [], []
    for src in SRCS:
        obj = os.path.join(OBJ_DIR, os.path.basename(src) + ".o")
        objs.append(obj)
        procs.append((src, subprocess.Popen([hipcc(), *compile_flags, "-I", INCLUDE, "-c", src,
                                             "-o", obj])))
    floor_tmp = FLOOR_LIB + ".tmp%d" % os.getpid()
    procs.append((FLOOR_SRC, subprocess.Popen([hipcc(), *HIPCC_FLAGS, "-I", INCLUDE, "-I",
                                               os.path.join(PKG, "csrc"), FLOOR_SRC, "-o",
                                               floor_tmp])))
    failed = [src for src, proc in procs if proc.wait() != 0]
    if failed:
        raise RuntimeError("hipcc failed on " + ", ".join(failed))
    subprocess.run([hipcc(), "--offload-arch=" + ARCH, "-shared", "-fPIC", *objs, "-o", tmp],
                   check=True)
    os.replace(tmp, LIB)
    os.replace(floor_tmp, FLOOR_LIB)
    return LIB


if __name__ == "__main__":
    ap = argparse.ArgumentParser()
    ap.add_argument("--save-temps", default=None, help="keep ISA/IR in this directory")
    print(build(ap.parse_args().save_temps))
