"""Kernel resources read from the built library's own gfx950 code objects (CPU).

The library embeds one offload bundle per HIP source file in its
``.hip_fatbin`` section.  Each gfx950 code object's AMDGPU metadata note lists
every kernel with its register, LDS and scratch use.  A kernel that spills
(registers to scratch) loses much of its bandwidth, and spills have crept in
unnoticed from small source changes, so every kernel is held to zero scratch
here, without a GPU.
"""
import os
import re
import shutil
import subprocess

import pytest
import yaml

from diffusion_transformer_qk_amd import binding

LLVM = "/opt/rocm/llvm/bin"
TOOLS = ("llvm-objcopy", "clang-offload-bundler", "llvm-readelf")
MAGIC = b"__CLANG_OFFLOAD_BUNDLE__"
TARGET = "hipv4-amdgcn-amd-amdhsa--gfx950"

pytestmark = pytest.mark.skipif(
    not all(os.path.exists(os.path.join(LLVM, t)) for t in TOOLS)
    or not os.path.exists(binding.LIB_PATH),
    reason="ROCm LLVM tools or the built library not available")


def _code_objects(tmp_path):
    """Paths of the library's gfx950 code objects, one per HIP source file."""
    fat = os.path.join(tmp_path, "fat.bin")
    subprocess.run([os.path.join(LLVM, "llvm-objcopy"), "--dump-section",
                    ".hip_fatbin=" + fat, binding.LIB_PATH], check=True)
    data = open(fat, "rb").read()
    starts = [m.start() for m in re.finditer(re.escape(MAGIC), data)] + [len(data)]
    paths = []
    for n, (a, b) in enumerate(zip(starts, starts[1:])):
        part = os.path.join(tmp_path, "bundle%d" % n)
        with open(part, "wb") as f:
            f.write(data[a:b])
        co = os.path.join(tmp_path, "co%d.o" % n)
        subprocess.run([os.path.join(LLVM, "clang-offload-bundler"), "--unbundle", "--type=o",
                        "--targets=" + TARGET, "--input=" + part, "--output=" + co], check=True)
        paths.append(co)
    return paths


def _kernels(tmp_path):
    kernels = []
    for co in _code_objects(tmp_path):
        notes = subprocess.run([os.path.join(LLVM, "llvm-readelf"), "--notes", co], check=True,
                               capture_output=True, text=True).stdout
        doc = notes[notes.index("---"):]
        if "\n..." in doc:
            doc = doc[:doc.index("\n...")]
        kernels += yaml.safe_load(doc)["amdhsa.kernels"]
    return kernels


def _family(name):
    for fam in ("qknorm_rope_kernel", "fuse_scale_shift_kernel", "gn_single_kernel",
                "gn_stats_kernel", "gn_apply_kernel", "gn_lagged_kernel", "gn_clear_kernel"):
        if fam in name:
            return fam
    return name


@pytest.fixture(scope="module")
def kernels(tmp_path_factory):
    return _kernels(str(tmp_path_factory.mktemp("code_object")))


def test_every_source_file_contributes_its_kernels(kernels):
    fams = {}
    for k in kernels:
        fams[_family(k[".name"])] = fams.get(_family(k[".name"]), 0) + 1
    # 3 head dims x 2 styles x 2 table dtypes x 2 data dtypes x 2 block orders x
    # (4 unroll depths, shared layout + 3, per-head layout)
    assert fams.get("qknorm_rope_kernel") == 336, fams
    # 8 row lengths x 2 data dtypes x 3 modulation dtypes x {1, 4} rows per
    # workgroup x {rows of exactly 512 * vectors per lane, other rows}
    assert fams.get("fuse_scale_shift_kernel") == 192, fams
    assert fams.get("gn_single_kernel") == 6, fams   # 2 data dtypes x 3 affine dtypes
    assert fams.get("gn_apply_kernel") == 18, fams   # ... x 3 chunk sizes
    assert fams.get("gn_stats_kernel") == 6, fams    # 2 data dtypes x 3 chunk sizes
    assert fams.get("gn_lagged_kernel") == 6, fams   # 2 data dtypes x 3 affine dtypes
    assert fams.get("gn_clear_kernel") == 1, fams


def test_no_kernel_uses_scratch_or_spills(kernels):
    bad = [(k[".name"], k[".private_segment_fixed_size"], k[".vgpr_spill_count"],
            k[".sgpr_spill_count"]) for k in kernels
           if k[".private_segment_fixed_size"] or k[".vgpr_spill_count"] or k[".sgpr_spill_count"]
           or k[".uses_dynamic_stack"]]
    assert not bad, bad


def test_wave64_and_block_sizes(kernels):
    for k in kernels:
        assert k[".wavefront_size"] == 64, k[".name"]
        # one-row AdaLN workgroups are a single wave; every other kernel runs 4 waves
        one_wave = "fuse_scale_shift_kernel" in k[".name"] and "Li1ELb" in k[".name"][-30:]
        assert k[".max_flat_workgroup_size"] == (64 if one_wave else 256), k[".name"]
        assert k[".agpr_count"] == 0, k[".name"]
        # LDS: the largest is the staged cos/sin rows of 2 tokens at head_dim 256
        assert k[".group_segment_fixed_size"] <= 8192, k[".name"]


def waves_per_simd(vgprs: int) -> int:
    """Waves a SIMD holds by VGPRs: 512 per lane, allocated in blocks of 8."""
    return min(8, 512 // (-(-vgprs // 8) * 8))


def test_headline_kernel_occupancy(kernels):
    """The fused-QKV interleaved bf16 kernel with 10 heads in flight and die
    runs leaves room for at least 5 waves per SIMD by its registers.  Its
    long launches hold 2 workgroups per CU through an LDS reservation; the
    register headroom keeps that a choice of the launch, not of the
    allocation."""
    match = [k for k in kernels if "qknorm_rope_kernel" in k[".name"]
             and "ILi128ELi0ELb0ELb0ELb0ELi10ELi4ELi3ELin1E" in k[".name"]]
    assert len(match) == 1
    assert waves_per_simd(match[0][".vgpr_count"]) >= 5, match[0][".vgpr_count"]
