"""The floor probes' library (bench_floor.so, measurement only) rejects bad
arguments before any HIP call, so these checks need no GPU.  Pointers are fake
integers that are never dereferenced."""
import ctypes
import os

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
FLOOR_LIB = os.path.join(ROOT, "bench_floor.so")

A = 0x10000          # a 16-byte aligned fake device address
B = 0x20000          # another one
MIS = 0x10008        # 8-byte aligned only


@pytest.fixture(scope="module")
def floor():
    if not os.path.exists(FLOOR_LIB):
        pytest.skip("bench_floor.so is not built")
    lib = ctypes.CDLL(FLOOR_LIB)
    vp, i64, i32, u32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_uint32
    lib.qkr_floor.argtypes = [vp, vp, i64, i32, i64, vp, vp, vp, u32, i32, i32, vp, vp]
    lib.qkr_floor.restype = ctypes.c_int

    def call(x0=A, x1=None, tokens=100, heads=40, row_stride=40 * 128, cos=A, sin=A, sink=A,
             mode=0, cap=1, y=None):
        return lib.qkr_floor(x0, x1, tokens, heads, row_stride, cos, sin, sink, 0, mode, cap, y,
                             None)
    return call


def test_null_pointers(floor):
    assert floor(x0=None) == -1
    assert floor(mode=1, cos=None) == -1
    assert floor(mode=3, sink=None) == -1
    assert floor(mode=6, y=None) == -1


def test_sizes_modes_and_cap(floor):
    assert floor(tokens=0) == -2
    assert floor(tokens=1 << 24) == -2
    assert floor(heads=0) == -2
    assert floor(heads=49) == -2
    assert floor(row_stride=40 * 128 - 8) == -2
    # a fused buffer (x1 = x0 + heads * 128 elements) needs room for Q and K
    assert floor(x1=A + 40 * 128 * 2, row_stride=40 * 128) == -2
    assert floor(mode=-1) == -2 and floor(mode=7) == -2
    assert floor(cap=2) == -2 and floor(cap=-1) == -2
    # out of place takes a single tensor
    assert floor(mode=6, x1=B, y=B + 0x100000) == -2


def test_alignment(floor):
    assert floor(x0=MIS) == -3
    assert floor(x1=MIS, row_stride=40 * 128) == -3
    assert floor(mode=1, cos=MIS) == -3
    assert floor(mode=6, y=MIS) == -3
    assert floor(row_stride=40 * 128 + 4) == -3
