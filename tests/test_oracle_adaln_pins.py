"""Pins for the oracle of the adaptive layer norm with scale and shift (AdaLN).

Independent of the oracle: torch's fp64 layer_norm (library routine), exact
closed forms (scale = -1 gives the shift; a constant row gives the shift),
the output's mean/variance identity, the affine-invariance identity, and
brute force in exact arithmetic with several batches and every modulation
dtype.
"""
import struct
import zlib
from decimal import Decimal, getcontext
from fractions import Fraction

import numpy as np
import pytest
import torch

import workloads as wl


def _bits(a: np.ndarray, dtype: str) -> np.ndarray:
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(wl.DTYPES[dtype])
    return wl.u16(t)


def _np_decode(bits, dtype):
    bits = np.asarray(bits, dtype=np.uint16)
    if dtype == "fp16":
        return bits.view(np.float16).astype(np.float64)
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def _mods(rng, batches, hidden, mod_dtype, scale_sd=0.5):
    sc = (scale_sd * rng.standard_normal((batches, hidden))).astype(np.float32)
    sh = (0.5 * rng.standard_normal((batches, hidden))).astype(np.float32)
    if mod_dtype == "fp32":
        return sc, sh, sc.astype(np.float64), sh.astype(np.float64)
    scb, shb = _bits(sc, mod_dtype), _bits(sh, mod_dtype)
    return scb, shb, _np_decode(scb, mod_dtype), _np_decode(shb, mod_dtype)


@pytest.mark.parametrize("x_dtype", ["bf16", "fp16"])
@pytest.mark.parametrize("hidden", [64, 5120])
def test_zero_modulation_is_torch_layer_norm(oracle_lib, x_dtype, hidden):
    rng = np.random.default_rng(hidden)
    rows = 33
    x = _bits((rng.standard_normal((rows, hidden)) * 2 + 0.7), x_dtype)
    zero = np.zeros((1, hidden), np.float32)
    eps = 1e-3
    y = oracle_lib.adaln(x, x_dtype, hidden=hidden, rows_per_batch=rows, scale=zero, shift=zero,
                         mod_dtype="fp32", eps=eps)
    v = torch.from_numpy(_np_decode(x, x_dtype))
    ref = torch.nn.functional.layer_norm(v, (hidden,), eps=float(np.float32(eps))).numpy()
    assert np.max(np.abs(y - ref)) <= 1e-12


def test_scale_minus_one_gives_shift_exactly(oracle_lib):
    rng = np.random.default_rng(1)
    rows, hidden = 10, 128
    x = _bits(rng.standard_normal((rows, hidden)) * 3, "bf16")
    sc = -np.ones((2, hidden), np.float32)
    sh = rng.standard_normal((2, hidden)).astype(np.float32)
    y = oracle_lib.adaln(x, "bf16", hidden=hidden, rows_per_batch=5, scale=sc, shift=sh,
                         mod_dtype="fp32", eps=1e-6)
    assert np.array_equal(y[:5], np.broadcast_to(sh[0].astype(np.float64), (5, hidden)))
    assert np.array_equal(y[5:], np.broadcast_to(sh[1].astype(np.float64), (5, hidden)))


def test_constant_row_gives_shift_exactly(oracle_lib):
    rows, hidden = 4, 96
    x = _bits(np.full((rows, hidden), 2.5, np.float32), "fp16")
    rng = np.random.default_rng(2)
    scb, shb, _, shv = _mods(rng, 1, hidden, "bf16")
    y = oracle_lib.adaln(x, "fp16", hidden=hidden, rows_per_batch=rows, scale=scb, shift=shb,
                         mod_dtype="bf16", eps=1e-6)
    assert np.array_equal(y, np.broadcast_to(shv[0], (rows, hidden)))


def test_output_moments(oracle_lib):
    """scale = shift = 0: each row has mean 0 and variance var / (var + eps)."""
    rng = np.random.default_rng(3)
    rows, hidden = 20, 1000
    x = _bits(rng.standard_normal((rows, hidden)) * 0.05 + 0.3, "bf16")
    zero = np.zeros((1, hidden), np.float32)
    eps = 1e-3
    y = oracle_lib.adaln(x, "bf16", hidden=hidden, rows_per_batch=rows, scale=zero, shift=zero,
                         mod_dtype="fp32", eps=eps)
    v = _np_decode(x, "bf16")
    var = v.var(axis=1)
    assert np.max(np.abs(y.mean(axis=1))) <= 1e-13
    want = var / (var + float(np.float32(eps)))
    assert np.max(np.abs(y.var(axis=1) / want - 1)) <= 1e-12


def test_affine_invariance(oracle_lib):
    """y(a x + b; eps a^2) = y(x; eps): the mean is removed and the scale divided out."""
    rng = np.random.default_rng(4)
    rows, hidden = 12, 256
    k = rng.integers(-32, 33, (rows, hidden)).astype(np.float32)
    x = k / 8                       # exact in bf16 and fp16
    a, b = 2.0, 2.0                 # a x + b = k/4 + 2: still exact
    sc = rng.standard_normal((1, hidden)).astype(np.float32)
    sh = rng.standard_normal((1, hidden)).astype(np.float32)
    for dt in ("bf16", "fp16"):
        y1 = oracle_lib.adaln(_bits(x, dt), dt, hidden=hidden, rows_per_batch=rows, scale=sc,
                              shift=sh, mod_dtype="fp32", eps=1.0 / 64)
        y2 = oracle_lib.adaln(_bits(a * x + b, dt), dt, hidden=hidden, rows_per_batch=rows,
                              scale=sc, shift=sh, mod_dtype="fp32", eps=a * a / 64)
        assert np.max(np.abs(y1 - y2)) <= 1e-13


def _dec(bits, dtype):
    b = int(bits)
    if dtype == "fp16":
        return Fraction(struct.unpack("<e", struct.pack("<H", b))[0])
    return Fraction(struct.unpack("<f", struct.pack("<I", b << 16))[0])


def _brute_row(xs, sc, sh, eps):
    """Exact mean and variance (Fractions), root in 60-digit Decimal."""
    getcontext().prec = 60
    C = len(xs)
    mean = sum(xs) / C
    var = sum((x - mean) ** 2 for x in xs) / C
    q = var + eps
    root = (Decimal(q.numerator) / Decimal(q.denominator)).sqrt()
    out = []
    for x, s, h in zip(xs, sc, sh):
        d = x - mean
        n = Decimal(d.numerator) / Decimal(d.denominator) / root
        out.append(float(n * (1 + Decimal(s)) + Decimal(h)))
    return out


@pytest.mark.parametrize("x_dtype,mod_dtype", [("bf16", "fp32"), ("fp16", "bf16"),
                                               ("bf16", "fp16"), ("fp16", "fp32")])
@pytest.mark.parametrize("hidden", [8, 24])
def test_brute_force(oracle_lib, x_dtype, mod_dtype, hidden):
    rng = np.random.default_rng(zlib.crc32(repr((x_dtype, mod_dtype, hidden)).encode()))
    rows, rpb = 7, 3                 # batches 0, 0, 0, 1, 1, 1, 2
    x = _bits(rng.standard_normal((rows, hidden)) * 1.5 + 0.4, x_dtype)
    scb, shb, scv, shv = _mods(rng, 3, hidden, mod_dtype)
    eps = np.float32(1e-2)
    y = oracle_lib.adaln(x, x_dtype, hidden=hidden, rows_per_batch=rpb, scale=scb, shift=shb,
                         mod_dtype=mod_dtype, eps=float(eps))
    for r in range(rows):
        b = r // rpb
        xs = [_dec(v, x_dtype) for v in x[r]]
        want = _brute_row(xs, [float(v) for v in scv[b]], [float(v) for v in shv[b]],
                          Fraction(float(eps)))
        assert np.max(np.abs(y[r] - np.array(want))) <= 1e-12, r


def test_row_range_is_a_slice(oracle_lib):
    rng = np.random.default_rng(6)
    rows, hidden = 19, 40
    x = _bits(rng.standard_normal((rows, hidden)), "bf16")
    scb, shb, _, _ = _mods(rng, 4, hidden, "fp32")
    kw = dict(hidden=hidden, rows_per_batch=5, scale=scb, shift=shb, mod_dtype="fp32", eps=1e-6)
    full = oracle_lib.adaln(x, "bf16", **kw)
    part = oracle_lib.adaln(x, "bf16", row_begin=6, row_end=17, **kw)
    assert np.array_equal(full[6:17], part)


def test_rejects_bad_arguments(oracle_lib):
    x = np.zeros((2, 16), np.uint16)
    z = np.zeros((1, 16), np.float32)
    with pytest.raises(ValueError):
        oracle_lib.adaln(x, "bf16", hidden=16, rows_per_batch=0, scale=z, shift=z,
                         mod_dtype="fp32", eps=1e-6, row_end=0)
