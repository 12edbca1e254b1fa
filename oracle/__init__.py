"""CPU oracle for the fused QK-norm + RoPE pass, the adaptive layer norm with
scale/shift and the group norm followed by SiLU: TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The product path (the HIP library and
its binding) never touches it, and the two share no code.

The arithmetic lives in ``qkr_oracle.c`` (plain C, fp64, OpenMP over rows);
this module compiles it with gcc and marshals numpy arrays.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "qkr_oracle.c")
LIB = os.path.join(HERE, "libqkr_oracle.so")

BF16, FP16, FP32 = 0, 1, 2
SHARED, PER_HEAD = 0, 1
INTERLEAVED, ROTATE_HALF = 0, 1

DTYPE_CODE = {"bf16": BF16, "fp16": FP16, "fp32": FP32}
LAYOUT_CODE = {"shared": SHARED, "per_head": PER_HEAD}
STYLE_CODE = {"interleaved": INTERLEAVED, "rotate_half": ROTATE_HALF}


def compile_source(src: str, out: str) -> str:
    """gcc the oracle source ``src`` into the shared library ``out``."""
    tmp = out + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp",
           "-ffp-contract=off", "-fno-fast-math", src, "-o", tmp, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


def build(force: bool = True) -> str:
    """Compile the oracle into ``libqkr_oracle.so`` next to its source."""
    if not force and os.path.exists(LIB) and os.path.getmtime(LIB) >= os.path.getmtime(SRC):
        return LIB
    return compile_source(SRC, LIB)


def _ptr(a: np.ndarray):
    return ctypes.c_void_p(a.ctypes.data)


def _table_array(t, cos_dtype: str) -> np.ndarray:
    """fp32 tables as float32; bf16 tables as their uint16 bit patterns."""
    a = np.ascontiguousarray(t)
    if cos_dtype == "fp32":
        assert a.dtype == np.float32, a.dtype
    else:
        assert a.dtype == np.uint16, a.dtype
    return a


class Oracle:
    """ctypes front end of one compiled oracle library."""

    def __init__(self, lib_path: str):
        lib = ctypes.CDLL(lib_path)
        p = ctypes.c_void_p
        i64, i32, c_int = ctypes.c_int64, ctypes.c_int32, ctypes.c_int
        lib.qkr_oracle_qknorm_rope.argtypes = [p, c_int, i64, i64, i64, i64, i32, i32, p,
                                               ctypes.c_float, p, p, c_int, c_int, c_int, p]
        lib.qkr_oracle_qknorm_rope.restype = c_int
        lib.qkr_oracle_decode.argtypes = [p, i64, c_int, p]
        lib.qkr_oracle_decode.restype = None
        lib.qkr_oracle_round.argtypes = [p, i64, c_int]
        lib.qkr_oracle_round.restype = None
        lib.qkr_oracle_adaln.argtypes = [p, c_int, i64, i64, i64, i64, p, p, c_int,
                                         ctypes.c_float, p]
        lib.qkr_oracle_adaln.restype = c_int
        lib.qkr_oracle_group_norm_silu.argtypes = [p, c_int, i64, i64, i64, i64, i64, p, p,
                                                   c_int, ctypes.c_float, p]
        lib.qkr_oracle_group_norm_silu.restype = c_int
        lib.qkr_oracle_max_threads.argtypes = []
        lib.qkr_oracle_max_threads.restype = c_int
        lib.qkr_oracle_set_threads.argtypes = [c_int]
        lib.qkr_oracle_set_threads.restype = None
        self.lib = lib
        self.path = lib_path

    def max_threads(self) -> int:
        return int(self.lib.qkr_oracle_max_threads())

    def set_threads(self, n: int) -> None:
        """Threads for the following calls (for single-core timing)."""
        self.lib.qkr_oracle_set_threads(int(n))

    def decode(self, bits: np.ndarray, dtype: str) -> np.ndarray:
        """Exact fp64 values of bf16/fp16 bit patterns (uint16 array)."""
        bits = np.ascontiguousarray(bits, dtype=np.uint16)
        out = np.empty(bits.shape, dtype=np.float64)
        self.lib.qkr_oracle_decode(_ptr(bits), bits.size, DTYPE_CODE[dtype], _ptr(out))
        return out

    def round_to(self, values: np.ndarray, dtype: str) -> np.ndarray:
        """Nearest bf16/fp16 value (ties to even) of each fp64 value, as fp64."""
        out = np.array(values, dtype=np.float64, copy=True, order="C")
        self.lib.qkr_oracle_round(_ptr(out), out.size, DTYPE_CODE[dtype])
        return out

    def qknorm_rope(self, x_bits: np.ndarray, x_dtype: str, *, row_stride: int, col0: int,
                    heads: int, head_dim: int, gamma: np.ndarray, eps: float,
                    cos, sin, cos_dtype: str = "fp32", cos_layout: str = "shared",
                    style: str = "interleaved", t_begin: int = 0, t_end: int | None = None,
                    out: np.ndarray | None = None) -> np.ndarray:
        """fp64 output [t_end - t_begin, heads, head_dim] of the pass on one tensor.

        ``x_bits`` is the whole tensor's uint16 storage (any shape, C-contiguous);
        head h of token t starts at element ``t*row_stride + col0 + h*head_dim``.
        """
        x = np.ascontiguousarray(x_bits, dtype=np.uint16).reshape(-1)
        span = heads * head_dim
        n_tokens = (x.size - col0 - span) // row_stride + 1 if x.size >= col0 + span else 0
        if t_end is None:
            t_end = n_tokens
        assert 0 <= t_begin <= t_end
        if t_end > t_begin:
            last = (t_end - 1) * row_stride + col0 + heads * head_dim
            assert last <= x.size, "tensor too small for the requested tokens"
        g = np.ascontiguousarray(gamma, dtype=np.float32)
        assert g.size == head_dim
        c = _table_array(cos, cos_dtype)
        s = _table_array(sin, cos_dtype)
        rows = c.size // head_dim
        need = t_end * (heads if cos_layout == "per_head" else 1)
        assert c.size == s.size and rows >= need, "cos/sin table too small"
        shape = (t_end - t_begin, heads, head_dim)
        if out is None:
            out = np.empty(shape, dtype=np.float64)
        assert out.shape == shape and out.dtype == np.float64 and out.flags.c_contiguous
        rc = self.lib.qkr_oracle_qknorm_rope(
            _ptr(x), DTYPE_CODE[x_dtype], row_stride, col0, t_begin, t_end, heads, head_dim,
            _ptr(g), ctypes.c_float(eps), _ptr(c), _ptr(s), DTYPE_CODE[cos_dtype],
            LAYOUT_CODE[cos_layout], STYLE_CODE[style], _ptr(out))
        if rc != 0:
            raise ValueError("oracle rejected its arguments")
        return out

    def adaln(self, x_bits: np.ndarray, x_dtype: str, *, hidden: int, rows_per_batch: int,
              scale, shift, mod_dtype: str, eps: float, row_begin: int = 0,
              row_end: int | None = None, out: np.ndarray | None = None) -> np.ndarray:
        """fp64 [row_end - row_begin, hidden] adaptive layer norm with scale/shift.

        ``scale``/``shift``: [batches, hidden] as float32 (mod_dtype "fp32") or
        their 16-bit patterns (uint16, "bf16"/"fp16"); row r uses batch
        r // rows_per_batch.
        """
        x = np.ascontiguousarray(x_bits, dtype=np.uint16).reshape(-1)
        rows = x.size // hidden
        if row_end is None:
            row_end = rows
        assert 0 <= row_begin <= row_end <= rows and x.size == rows * hidden
        want = np.float32 if mod_dtype == "fp32" else np.uint16
        sc = np.ascontiguousarray(scale)
        sh = np.ascontiguousarray(shift)
        assert sc.dtype == want and sh.dtype == want and sc.size == sh.size
        batches_needed = (row_end - 1) // rows_per_batch + 1 if row_end > row_begin else 0
        assert sc.size >= batches_needed * hidden, "scale/shift too small"
        shape = (row_end - row_begin, hidden)
        if out is None:
            out = np.empty(shape, dtype=np.float64)
        assert out.shape == shape and out.dtype == np.float64 and out.flags.c_contiguous
        rc = self.lib.qkr_oracle_adaln(_ptr(x), DTYPE_CODE[x_dtype], row_begin, row_end, hidden,
                                       rows_per_batch, _ptr(sc), _ptr(sh), DTYPE_CODE[mod_dtype],
                                       ctypes.c_float(eps), _ptr(out))
        if rc != 0:
            raise ValueError("oracle rejected its arguments")
        return out

    def group_norm_silu(self, x_bits: np.ndarray, x_dtype: str, *, channels: int, spatial: int,
                        groups: int, gamma, beta, param_dtype: str, eps: float,
                        group_begin: int = 0, group_end: int | None = None,
                        out: np.ndarray | None = None) -> np.ndarray:
        """fp64 [(group_end - group_begin) * (channels // groups) * spatial] output.

        ``x_bits``: the whole [n, channels, spatial] tensor's uint16 storage;
        groups are the n*groups (sample, group) pairs in memory order.
        ``gamma``/``beta``: [channels] float32 ("fp32") or uint16 patterns.
        """
        x = np.ascontiguousarray(x_bits, dtype=np.uint16).reshape(-1)
        gsize = channels // groups * spatial
        total = x.size // gsize
        assert x.size == total * gsize and channels % groups == 0
        if group_end is None:
            group_end = total
        assert 0 <= group_begin <= group_end <= total
        want = np.float32 if param_dtype == "fp32" else np.uint16
        g = np.ascontiguousarray(gamma)
        b = np.ascontiguousarray(beta)
        assert g.dtype == want and b.dtype == want and g.size == channels == b.size
        n = (group_end - group_begin) * gsize
        if out is None:
            out = np.empty(n, dtype=np.float64)
        assert out.size == n and out.dtype == np.float64 and out.flags.c_contiguous
        rc = self.lib.qkr_oracle_group_norm_silu(
            _ptr(x), DTYPE_CODE[x_dtype], channels, spatial, groups, group_begin, group_end,
            _ptr(g), _ptr(b), DTYPE_CODE[param_dtype], ctypes.c_float(eps), _ptr(out))
        if rc != 0:
            raise ValueError("oracle rejected its arguments")
        return out

    def fused_qk(self, qkv_bits: np.ndarray, x_dtype: str, *, heads: int, head_dim: int,
                 q_gamma, k_gamma, eps: float, cos, sin, cos_dtype="fp32",
                 cos_layout="shared", style="interleaved", t_begin=0, t_end=None):
        """(q_out, k_out) fp64 for a fused [T, 3*heads*head_dim] QKV buffer."""
        hd = heads * head_dim
        kw = dict(row_stride=3 * hd, heads=heads, head_dim=head_dim, eps=eps, cos=cos,
                  sin=sin, cos_dtype=cos_dtype, cos_layout=cos_layout, style=style,
                  t_begin=t_begin, t_end=t_end)
        q = self.qknorm_rope(qkv_bits, x_dtype, col0=0, gamma=q_gamma, **kw)
        k = self.qknorm_rope(qkv_bits, x_dtype, col0=hd, gamma=k_gamma, **kw)
        return q, k


_default: Oracle | None = None


def default() -> Oracle:
    """The oracle built from ``qkr_oracle.c`` (compiled on first use if missing)."""
    global _default
    if _default is None:
        build(force=False)
        _default = Oracle(LIB)
    return _default


def max_threads() -> int:
    return default().max_threads()


def set_threads(n: int) -> None:
    default().set_threads(n)


def decode(bits, dtype):
    return default().decode(bits, dtype)


def round_to(values, dtype):
    return default().round_to(values, dtype)


def qknorm_rope(x_bits, x_dtype, **kw):
    return default().qknorm_rope(x_bits, x_dtype, **kw)


def fused_qk(qkv_bits, x_dtype, **kw):
    return default().fused_qk(qkv_bits, x_dtype, **kw)


def adaln(x_bits, x_dtype, **kw):
    return default().adaln(x_bits, x_dtype, **kw)


def group_norm_silu(x_bits, x_dtype, **kw):
    return default().group_norm_silu(x_bits, x_dtype, **kw)
