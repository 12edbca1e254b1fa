"""Pins for the oracle of the group norm followed by SiLU.

Independent of the oracle: torch's fp64 group_norm and silu (library
routines, including the instance-norm and layer-norm special cases), exact
closed forms (gamma = 0 gives silu(beta); a constant group gives silu(beta)),
the SiLU odd-part identity silu(y) - silu(-y) = y, and brute force in exact
arithmetic (Fractions, 60-digit Decimal sqrt and exp).
"""
import struct
import zlib
from decimal import Decimal, getcontext
from fractions import Fraction

import numpy as np
import pytest
import torch

import workloads as wl


def _bits(a, dtype):
    return wl.u16(torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(wl.DTYPES[dtype]))


def _np_decode(bits, dtype):
    bits = np.asarray(bits, dtype=np.uint16)
    if dtype == "fp16":
        return bits.view(np.float16).astype(np.float64)
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def _params(rng, channels, param_dtype):
    g = (1 + 0.3 * rng.standard_normal(channels)).astype(np.float32)
    b = (0.5 * rng.standard_normal(channels)).astype(np.float32)
    if param_dtype == "fp32":
        return g, b, g.astype(np.float64), b.astype(np.float64)
    gb, bb = _bits(g, param_dtype), _bits(b, param_dtype)
    return gb, bb, _np_decode(gb, param_dtype), _np_decode(bb, param_dtype)


def _torch_ref(xv, channels, spatial, groups, gv, bv, eps):
    n = xv.size // (channels * spatial)
    t = torch.from_numpy(xv.reshape(n, channels, spatial))
    y = torch.nn.functional.group_norm(t, groups, weight=torch.from_numpy(gv),
                                       bias=torch.from_numpy(bv), eps=eps)
    return torch.nn.functional.silu(y).numpy().reshape(-1)


@pytest.mark.parametrize("groups", [1, 4, 16])
@pytest.mark.parametrize("x_dtype,param_dtype", [("bf16", "fp32"), ("fp16", "bf16"),
                                                 ("bf16", "fp16")])
def test_matches_torch_group_norm_silu(oracle_lib, groups, x_dtype, param_dtype):
    """groups = 1 is a layer norm over (C, S); groups = C (16) an instance norm."""
    rng = np.random.default_rng(zlib.crc32(repr((groups, x_dtype, param_dtype)).encode()))
    n, channels, spatial = 3, 16, 40
    x = _bits(rng.standard_normal((n, channels, spatial)) * 2 + 0.5, x_dtype)
    gb, bb, gv, bv = _params(rng, channels, param_dtype)
    eps = 1e-3
    out = oracle_lib.group_norm_silu(x, x_dtype, channels=channels, spatial=spatial,
                                     groups=groups, gamma=gb, beta=bb, param_dtype=param_dtype,
                                     eps=eps)
    ref = _torch_ref(_np_decode(x, x_dtype), channels, spatial, groups, gv, bv,
                     float(np.float32(eps)))
    assert np.max(np.abs(out - ref)) <= 1e-13


def test_instance_norm_special_case(oracle_lib):
    rng = np.random.default_rng(2)
    n, channels, spatial = 2, 6, 64
    x = _bits(rng.standard_normal((n, channels, spatial)), "bf16")
    ones, zeros = np.ones(channels, np.float32), np.zeros(channels, np.float32)
    out = oracle_lib.group_norm_silu(x, "bf16", channels=channels, spatial=spatial,
                                     groups=channels, gamma=ones, beta=zeros, param_dtype="fp32",
                                     eps=1e-5)
    t = torch.from_numpy(_np_decode(x, "bf16").reshape(n, channels, spatial))
    ref = torch.nn.functional.silu(torch.nn.functional.instance_norm(
        t, eps=float(np.float32(1e-5)))).numpy().reshape(-1)
    assert np.max(np.abs(out - ref)) <= 1e-13


def test_zero_gamma_and_constant_groups_give_silu_of_beta(oracle_lib):
    rng = np.random.default_rng(3)
    n, channels, spatial, groups = 2, 8, 16, 2
    x = _bits(rng.standard_normal((n, channels, spatial)) * 3, "fp16")
    beta = rng.standard_normal(channels).astype(np.float32)
    out = oracle_lib.group_norm_silu(x, "fp16", channels=channels, spatial=spatial, groups=groups,
                                     gamma=np.zeros(channels, np.float32), beta=beta,
                                     param_dtype="fp32", eps=1e-6).reshape(n, channels, spatial)
    b = beta.astype(np.float64)
    want = b / (1 + np.exp(-b))
    assert np.array_equal(out, np.broadcast_to(want[None, :, None], out.shape))
    const = _bits(np.full((n, channels, spatial), -1.75, np.float32), "bf16")
    out2 = oracle_lib.group_norm_silu(const, "bf16", channels=channels, spatial=spatial,
                                      groups=groups, gamma=np.ones(channels, np.float32),
                                      beta=beta, param_dtype="fp32",
                                      eps=1e-6).reshape(n, channels, spatial)
    assert np.array_equal(out2, np.broadcast_to(want[None, :, None], out2.shape))


def test_silu_odd_part_identity(oracle_lib):
    """Negating beta and gamma negates y; silu(y) - silu(-y) = y recovers it."""
    rng = np.random.default_rng(4)
    n, channels, spatial, groups = 1, 12, 50, 3
    x = _bits(rng.standard_normal((n, channels, spatial)), "bf16")
    g = rng.standard_normal(channels).astype(np.float32)
    b = rng.standard_normal(channels).astype(np.float32)
    kw = dict(channels=channels, spatial=spatial, groups=groups, param_dtype="fp32", eps=1e-6)
    pos = oracle_lib.group_norm_silu(x, "bf16", gamma=g, beta=b, **kw)
    neg = oracle_lib.group_norm_silu(x, "bf16", gamma=-g, beta=-b, **kw)
    v = _np_decode(x, "bf16").reshape(n, groups, -1)
    mean = v.mean(axis=2, keepdims=True)
    var = v.var(axis=2, keepdims=True)
    y = ((v - mean) / np.sqrt(var + float(np.float32(1e-6)))).reshape(n, channels, spatial)
    y = y * g.astype(np.float64)[None, :, None] + b.astype(np.float64)[None, :, None]
    assert np.max(np.abs((pos - neg) - y.reshape(-1))) <= 1e-12


def _dec(bits, dtype):
    b = int(bits)
    if dtype == "fp16":
        return Fraction(struct.unpack("<e", struct.pack("<H", b))[0])
    return Fraction(struct.unpack("<f", struct.pack("<I", b << 16))[0])


@pytest.mark.parametrize("x_dtype,param_dtype", [("bf16", "fp32"), ("fp16", "fp16")])
def test_brute_force(oracle_lib, x_dtype, param_dtype):
    getcontext().prec = 60
    rng = np.random.default_rng(zlib.crc32(repr((x_dtype, param_dtype)).encode()))
    n, channels, spatial, groups = 2, 6, 5, 3
    x = _bits(rng.standard_normal((n, channels, spatial)) * 1.5 + 0.3, x_dtype)
    gb, bb, gv, bv = _params(rng, channels, param_dtype)
    eps = np.float32(1e-2)
    out = oracle_lib.group_norm_silu(x, x_dtype, channels=channels, spatial=spatial,
                                     groups=groups, gamma=gb, beta=bb, param_dtype=param_dtype,
                                     eps=float(eps)).reshape(n, channels, spatial)
    cg = channels // groups
    for i in range(n):
        for g in range(groups):
            vals = [_dec(x[i, c, s], x_dtype) for c in range(g * cg, (g + 1) * cg)
                    for s in range(spatial)]
            mean = sum(vals) / len(vals)
            var = sum((v - mean) ** 2 for v in vals) / len(vals) + Fraction(float(eps))
            root = (Decimal(var.numerator) / Decimal(var.denominator)).sqrt()
            for k, v in enumerate(vals):
                c = g * cg + k // spatial
                d = v - mean
                y = (Decimal(d.numerator) / Decimal(d.denominator) / root * Decimal(float(gv[c]))
                     + Decimal(float(bv[c])))
                want = float(y / (1 + (-y).exp()))
                assert abs(out[i, c, k % spatial] - want) <= 1e-12


def test_group_range_is_a_slice(oracle_lib):
    rng = np.random.default_rng(6)
    n, channels, spatial, groups = 3, 8, 24, 4
    x = _bits(rng.standard_normal((n, channels, spatial)), "bf16")
    gb, bb, _, _ = _params(rng, channels, "fp32")
    kw = dict(channels=channels, spatial=spatial, groups=groups, gamma=gb, beta=bb,
              param_dtype="fp32", eps=1e-6)
    full = oracle_lib.group_norm_silu(x, "bf16", **kw)
    gs = channels // groups * spatial
    part = oracle_lib.group_norm_silu(x, "bf16", group_begin=5, group_end=10, **kw)
    assert np.array_equal(full[5 * gs:10 * gs], part)


def test_rejects_bad_arguments(oracle_lib):
    """The C code refuses groups that do not divide the channels."""
    import ctypes
    x = np.zeros(2 * 6 * 8, np.uint16)
    p = np.ones(6, np.float32)
    out = np.zeros(x.size, np.float64)
    ptr = lambda a: ctypes.c_void_p(a.ctypes.data)  # noqa: E731
    rc = oracle_lib.default().lib.qkr_oracle_group_norm_silu(
        ptr(x), 0, 6, 8, 4, 0, 2, ptr(p), ptr(p), 2, ctypes.c_float(1e-6), ptr(out))
    assert rc == -1
