"""Instruction checks on the built library's own gfx950 code (CPU, no GPU).

Disassembles every kernel of the library (the code objects extracted as in
test_code_object.py) and checks properties the design depends on:
  * no kernel writes through the scalar data cache (no scalar stores,
    scalar atomics, or scalar-cache write-back/discard): all writes are
    vector stores;
  * no packed fp32 arithmetic (v_pk_add_f32 / v_pk_mul_f32 / v_pk_fma_f32):
    the build disables it;
  * no matrix-core instructions: every step is memory-bound elementwise or
    reduction work;
  * the bf16 outputs use the hardware round-to-nearest-even packed convert.
This file names those instructions, so it stays off the GPU runs.
"""
import os
import re
import subprocess

import pytest

from tests.test_code_object import LLVM, TOOLS, _code_objects

OBJDUMP = os.path.join(LLVM, "llvm-objdump")

pytestmark = pytest.mark.skipif(
    not all(os.path.exists(os.path.join(LLVM, t)) for t in TOOLS) or not os.path.exists(OBJDUMP),
    reason="ROCm LLVM tools not available")

SCALAR_WRITES = re.compile(r"^\s*(s_store_|s_buffer_store|s_atomic|s_buffer_atomic|s_dcache_wb|"
                           r"s_dcache_discard|s_scratch_store)")
PACKED_FP32 = re.compile(r"^\s*v_pk_(add|mul|fma)_f32")
MATRIX = re.compile(r"^\s*v_(mfma|smfmac)")


@pytest.fixture(scope="module")
def disassembly(tmp_path_factory):
    """{kernel symbol: [instruction lines]} over every code object."""
    out = {}
    for co in _code_objects(str(tmp_path_factory.mktemp("isa"))):
        text = subprocess.run([OBJDUMP, "-d", "--mcpu=gfx950", co], check=True,
                              capture_output=True, text=True).stdout
        current = None
        for line in text.splitlines():
            m = re.match(r"^[0-9a-f]+ <(\w+)>:", line)
            if m:
                current = m.group(1)
                out[current] = []
            elif current and line.startswith("\t"):
                out[current].append(line.strip())
    return out


def test_every_kernel_disassembled(disassembly):
    names = list(disassembly)
    assert sum("qknorm_rope_kernel" in n for n in names) == 336
    assert sum("fuse_scale_shift_kernel" in n for n in names) == 192
    assert sum("gn_" in n for n in names) == 37


def test_no_scalar_cache_writes(disassembly):
    bad = {k: [i for i in v if SCALAR_WRITES.match(i)] for k, v in disassembly.items()}
    assert not any(bad.values()), {k: v[:3] for k, v in bad.items() if v}


def test_no_packed_fp32_or_matrix_instructions(disassembly):
    for k, v in disassembly.items():
        assert not any(PACKED_FP32.match(i) for i in v), k
        assert not any(MATRIX.match(i) for i in v), k


def test_bf16_outputs_use_the_packed_rne_convert(disassembly):
    # template argument lists mark the data dtype: qknorm_rope_kernel<..., X_FP16, ...>
    # is the 5th argument; bf16 kernels must convert with v_cvt_pk_bf16_f32
    bf16 = [k for k in disassembly
            if re.search(r"qknorm_rope_kernelILi\d+ELi\dELb[01]ELb[01]ELb0E", k)]
    assert len(bf16) == 168
    for k in bf16:
        assert any(i.startswith("v_cvt_pk_bf16_f32") for i in disassembly[k]), k
