"""Pins for the CPU oracle: checks against things other than the oracle itself.

Each test fixes the oracle to something independent of it: exhaustive decode
against numpy / IEEE bit layouts, brute force in exact arithmetic with a dense
rotation matrix, a library RMSNorm, the complex-multiply and rotate-half
textbook forms of RoPE, closed forms and invariants.  The pages print no
worked numeric example, so none can be used.
"""
import struct
import zlib
from decimal import Decimal, getcontext
from fractions import Fraction

import numpy as np
import pytest
import torch

import workloads as wl

# ----------------------------------------------------------------------------- helpers


def _bf16_bits(a: np.ndarray) -> np.ndarray:
    return wl.u16(torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(torch.bfloat16))


def _fp16_bits(a: np.ndarray) -> np.ndarray:
    return wl.u16(torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(torch.float16))


def _bits(a, dtype):
    return _bf16_bits(a) if dtype == "bf16" else _fp16_bits(a)


def _np_decode(bits: np.ndarray, dtype: str) -> np.ndarray:
    """Decode through numpy's own float views (independent of the oracle)."""
    bits = np.asarray(bits, dtype=np.uint16)
    with np.errstate(invalid="ignore"):     # NaN patterns widen to NaN, as intended
        if dtype == "fp16":
            return bits.view(np.float16).astype(np.float64)
        return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def _random_tensor(rng, shape, dtype, scale=1.0):
    x = (rng.standard_normal(shape) * scale).astype(np.float32)
    return _bits(x, dtype)


def _identity_tables(rows, d):
    return np.ones((rows, d), np.float32), np.zeros((rows, d), np.float32)


# ----------------------------------------------------------------------------- decode


def test_decode_bf16_exhaustive(oracle_lib):
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    got = oracle_lib.decode(bits, "bf16")
    want = _np_decode(bits, "bf16")
    nan = np.isnan(want)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], want[~nan])


def test_decode_fp16_exhaustive(oracle_lib):
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    got = oracle_lib.decode(bits, "fp16")
    want = _np_decode(bits, "fp16")
    nan = np.isnan(want)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], want[~nan])
    # spot values from the binary16 layout itself
    assert got[0x0001] == 2.0 ** -24 and got[0x03FF] == 1023 * 2.0 ** -24
    assert got[0x3C00] == 1.0 and got[0x7BFF] == 65504.0 and got[0xC000] == -2.0


# ----------------------------------------------------------------------------- rounding


def test_round_fp16_matches_numpy(oracle_lib):
    rng = np.random.default_rng(7)
    mags = 10.0 ** rng.uniform(-9, 4.9, 200000)
    v = mags * rng.choice([-1.0, 1.0], mags.size)
    # exact ties between neighbouring fp16 values, normal and subnormal
    grid = np.arange(-4096, 4096, dtype=np.float64)
    ties = np.concatenate([(grid + 0.5) * 2.0 ** -24, 1.0 + (grid[grid > 0] + 0.5) * 2.0 ** -10])
    v = np.concatenate([v, ties, [1 + 2.0 ** -11, 1 + 3 * 2.0 ** -11, 65519.99, 65520.0]])
    got = oracle_lib.round_to(v, "fp16")
    with np.errstate(over="ignore"):        # 65520 rounds to inf, as the oracle does
        want = v.astype(np.float16).astype(np.float64)
    assert np.array_equal(got, want)
    assert oracle_lib.round_to(np.array([1 + 2.0 ** -11]), "fp16")[0] == 1.0
    assert oracle_lib.round_to(np.array([1 + 3 * 2.0 ** -11]), "fp16")[0] == 1 + 2.0 ** -9


def test_round_bf16_properties(oracle_lib):
    rng = np.random.default_rng(8)
    v = 10.0 ** rng.uniform(-30, 30, 100000) * rng.choice([-1.0, 1.0], 100000)
    r = oracle_lib.round_to(v, "bf16")
    # representable: exactly a float32 whose low 16 bits are zero
    r32 = r.astype(np.float32)
    assert np.array_equal(r32.astype(np.float64), r)
    assert not np.any(r32.view(np.uint32) & 0xFFFF)
    # nearest: within half a quantum of the binade (8 significant bits)
    e = np.floor(np.log2(np.abs(v)))
    half_q = 2.0 ** (e - 8)
    assert np.all(np.abs(v - r) <= half_q * (1 + 1e-12))
    # ties go to the even significand
    assert oracle_lib.round_to(np.array([1 + 2.0 ** -8]), "bf16")[0] == 1.0
    assert oracle_lib.round_to(np.array([1 + 3 * 2.0 ** -8]), "bf16")[0] == 1 + 2.0 ** -6
    assert oracle_lib.round_to(np.array([-(1 + 2.0 ** -8)]), "bf16")[0] == -1.0
    # smallest subnormal quantum 2^-133; half of it ties to zero
    sub = oracle_lib.round_to(np.array([2.0 ** -133, 1.5 * 2.0 ** -133, 2.0 ** -134]), "bf16")
    assert list(sub) == [2.0 ** -133, 2.0 ** -132, 0.0]


# ----------------------------------------------------------------------------- brute force


def _dec(bits, dtype):
    """Exact decode through Python's struct module (IEEE layouts)."""
    b = int(bits)
    if dtype == "fp16":
        return Fraction(struct.unpack("<e", struct.pack("<H", b))[0])
    return Fraction(struct.unpack("<f", struct.pack("<I", b << 16))[0])


def _pairs(style, d):
    if style == "interleaved":
        return [(2 * i, 2 * i + 1) for i in range(d // 2)]
    return [(i, i + d // 2) for i in range(d // 2)]


def _brute_head(v, gamma, eps, c, s, style):
    """Exact-arithmetic reference for one head via a dense rotation matrix.

    RMSNorm as x / sqrt(mean(x^2) + eps) * gamma (Decimal, 60 digits), then
    the block-diagonal rotation R built from the pairs, applied as R @ n.
    """
    getcontext().prec = 60
    d = len(v)
    mean_sq = sum(x * x for x in v) / d                       # exact Fraction
    denom = (Decimal(mean_sq.numerator) / Decimal(mean_sq.denominator)
             + Decimal(eps.numerator) / Decimal(eps.denominator)).sqrt()
    n = [Decimal(x.numerator) / Decimal(x.denominator) / denom
         * (Decimal(g.numerator) / Decimal(g.denominator)) for x, g in zip(v, gamma)]
    R = [[Decimal(0)] * d for _ in range(d)]
    for a, b in _pairs(style, d):
        R[a][a] = Decimal(float(c[a]))
        R[a][b] = -Decimal(float(s[a]))
        R[b][b] = Decimal(float(c[b]))
        R[b][a] = Decimal(float(s[b]))
    return [float(sum(R[i][j] * n[j] for j in range(d) if R[i][j] != 0)) for i in range(d)]


def _bf16_table_bits(a):
    return _bf16_bits(a)


@pytest.mark.parametrize("style", ["interleaved", "rotate_half"])
@pytest.mark.parametrize("cos_layout", ["shared", "per_head"])
@pytest.mark.parametrize("x_dtype,cos_dtype,head_dim", [
    ("bf16", "fp32", 64), ("fp16", "fp32", 64), ("bf16", "bf16", 64), ("fp16", "fp32", 128)])
def test_brute_force_fused_qkv(oracle_lib, style, cos_layout, x_dtype, cos_dtype, head_dim):
    """P-a: whole oracle vs exact arithmetic on a tiny fused QKV buffer.

    General tables (no pair duplication, distinct per-head rows, tokens != heads)
    so a wrong table index, a swapped q/k gamma or a wrong partner shows up.
    """
    rng = np.random.default_rng(zlib.crc32(repr((style, cos_layout, x_dtype, cos_dtype, head_dim)).encode()))
    T, H, D = 3, 2, head_dim
    x = _random_tensor(rng, (T, 3 * H * D), x_dtype, 2.0)
    qg = (1 + 0.3 * rng.standard_normal(D)).astype(np.float32)
    kg = (1 + 0.3 * rng.standard_normal(D)).astype(np.float32)
    rows = T * (H if cos_layout == "per_head" else 1)
    c = rng.uniform(-1, 1, (rows, D)).astype(np.float32)
    s = rng.uniform(-1, 1, (rows, D)).astype(np.float32)
    if cos_dtype == "bf16":
        c_in, s_in = _bf16_table_bits(c), _bf16_table_bits(s)
        c_val, s_val = _np_decode(c_in, "bf16"), _np_decode(s_in, "bf16")
    else:
        c_in, s_in, c_val, s_val = c, s, c.astype(np.float64), s.astype(np.float64)
    eps = np.float32(1e-3)
    q_out, k_out = oracle_lib.fused_qk(x, x_dtype, heads=H, head_dim=D, q_gamma=qg,
                                       k_gamma=kg, eps=float(eps), cos=c_in, sin=s_in,
                                       cos_dtype=cos_dtype, cos_layout=cos_layout, style=style)
    eps_f = Fraction(float(eps))
    for t in range(T):
        for si, (out, gam) in enumerate([(q_out, qg), (k_out, kg)]):
            for h in range(H):
                col = si * H * D + h * D
                v = [_dec(b, x_dtype) for b in x[t, col:col + D]]
                row = t if cos_layout == "shared" else t * H + h
                want = _brute_head(v, [Fraction(float(g)) for g in gam], eps_f,
                                   c_val[row], s_val[row], style)
                assert np.max(np.abs(out[t, h] - np.array(want))) <= 1e-12


# ----------------------------------------------------------------------------- library / textbook forms


@pytest.mark.parametrize("x_dtype", ["bf16", "fp16"])
@pytest.mark.parametrize("head_dim", [64, 128])
def test_norm_matches_torch_rms_norm(oracle_lib, x_dtype, head_dim):
    """P-i: with cos = 1, sin = 0 the output is torch's fp64 RMSNorm."""
    rng = np.random.default_rng(11 + head_dim)
    T, H, D = 37, 5, head_dim
    x = _random_tensor(rng, (T, H, D), x_dtype, 3.0)
    g = (1 + 0.1 * rng.standard_normal(D)).astype(np.float32)
    c, s = _identity_tables(T, D)
    eps = 1e-2   # large enough that its placement matters
    out = oracle_lib.qknorm_rope(x, x_dtype, row_stride=H * D, col0=0, heads=H, head_dim=D,
                                 gamma=g, eps=eps, cos=c, sin=s)
    v = torch.from_numpy(_np_decode(x, x_dtype))
    ref = torch.nn.functional.rms_norm(v, (D,), weight=torch.from_numpy(g.astype(np.float64)),
                                       eps=float(np.float32(eps)))
    assert np.max(np.abs(out - ref.numpy())) <= 1e-13


def _norm_only(oracle_lib, x, x_dtype, H, D, g, eps, style="interleaved"):
    T = x.shape[0]
    c, s = _identity_tables(T, D)
    return oracle_lib.qknorm_rope(x, x_dtype, row_stride=H * D, col0=0, heads=H, head_dim=D,
                                  gamma=g, eps=eps, cos=c, sin=s, style=style)


def test_interleaved_is_complex_multiply(oracle_lib):
    """P-h: interleaved RoPE is (n_2i + i n_2i+1) * (cos + i sin) per pair."""
    rng = np.random.default_rng(12)
    T, H, D = 64, 3, 128
    x = _random_tensor(rng, (T, H, D), "bf16", 1.5)
    g = (1 + 0.1 * rng.standard_normal(D)).astype(np.float32)
    pos = rng.integers(0, 5000, T)
    c, s = (t.numpy() for t in wl.rope_tables(pos, (D // 2,), D, "interleaved"))
    out = oracle_lib.qknorm_rope(x, "bf16", row_stride=H * D, col0=0, heads=H, head_dim=D,
                                 gamma=g, eps=1e-6, cos=c, sin=s, style="interleaved")
    v = torch.from_numpy(_np_decode(x, "bf16"))
    n = torch.nn.functional.rms_norm(v, (D,), weight=torch.from_numpy(g.astype(np.float64)),
                                     eps=float(np.float32(1e-6))).numpy()
    z = n[..., 0::2] + 1j * n[..., 1::2]
    w = c[:, None, 0::2].astype(np.float64) + 1j * s[:, None, 0::2].astype(np.float64)
    zr = z * w
    want = np.empty_like(n)
    want[..., 0::2], want[..., 1::2] = zr.real, zr.imag
    assert np.max(np.abs(out - want)) <= 1e-13


def test_rotate_half_textbook_form(oracle_lib):
    """Rotate-half RoPE is n * cos + cat(-n2, n1) * sin (the split-halves form)."""
    rng = np.random.default_rng(13)
    T, H, D = 50, 4, 64
    x = _random_tensor(rng, (T, H, D), "fp16", 0.7)
    g = (1 + 0.1 * rng.standard_normal(D)).astype(np.float32)
    pos = rng.integers(0, 3000, T)
    c, s = (t.numpy() for t in wl.rope_tables(pos, (D // 2,), D, "rotate_half"))
    out = oracle_lib.qknorm_rope(x, "fp16", row_stride=H * D, col0=0, heads=H, head_dim=D,
                                 gamma=g, eps=1e-6, cos=c, sin=s, style="rotate_half")
    v = torch.from_numpy(_np_decode(x, "fp16"))
    n = torch.nn.functional.rms_norm(v, (D,), weight=torch.from_numpy(g.astype(np.float64)),
                                     eps=float(np.float32(1e-6))).numpy()
    rot = np.concatenate([-n[..., D // 2:], n[..., :D // 2]], axis=-1)
    want = n * c[:, None, :].astype(np.float64) + rot * s[:, None, :].astype(np.float64)
    assert np.max(np.abs(out - want)) <= 1e-13


# ----------------------------------------------------------------------------- closed forms and invariants


def test_rms_closed_form(oracle_lib):
    """P-b: gamma = 1, cos = 1, sin = 0 -> RMS of each head is sqrt(ms / (ms + eps))."""
    rng = np.random.default_rng(14)
    T, H, D = 40, 6, 128
    x = _random_tensor(rng, (T, H, D), "bf16", 0.01)
    g = np.ones(D, np.float32)
    eps = 1e-4
    out = _norm_only(oracle_lib, x, "bf16", H, D, g, eps)
    v = _np_decode(x, "bf16")
    ms = np.mean(v * v, axis=-1)
    rms = np.sqrt(np.mean(out * out, axis=-1))
    want = np.sqrt(ms / (ms + float(np.float32(eps))))
    assert np.max(np.abs(rms - want)) <= 1e-12


def test_zero_head_is_zero(oracle_lib):
    """P-c: an all-zero head stays exactly zero, whatever the tables and gamma."""
    rng = np.random.default_rng(15)
    T, H, D = 5, 3, 64
    x = _random_tensor(rng, (T, H, D), "fp16")
    x[2, 1, :] = 0
    x[4, 0, :] = 0x8000   # negative zeros
    g = (1 + 0.1 * rng.standard_normal(D)).astype(np.float32)
    c = rng.uniform(-1, 1, (T, D)).astype(np.float32)
    s = rng.uniform(-1, 1, (T, D)).astype(np.float32)
    for style in ("interleaved", "rotate_half"):
        out = oracle_lib.qknorm_rope(x, "fp16", row_stride=H * D, col0=0, heads=H, head_dim=D,
                                     gamma=g, eps=1e-6, cos=c, sin=s, style=style)
        assert np.all(out[2, 1] == 0) and np.all(out[4, 0] == 0)
        assert np.count_nonzero(out[0]) > 0.9 * out[0].size


def test_scale_relation(oracle_lib):
    """P-d: o(a x) = a sqrt(ms + eps) / sqrt(a^2 ms + eps) * o(x) for a power of two a."""
    rng = np.random.default_rng(16)
    T, H, D = 20, 4, 128
    xv = (rng.standard_normal((T, H, D))).astype(np.float32)
    x = _bf16_bits(xv)
    a = 8.0
    xa = _bf16_bits(_np_decode(x, "bf16").astype(np.float32) * np.float32(a))
    g = (1 + 0.1 * rng.standard_normal(D)).astype(np.float32)
    pos = rng.integers(0, 100, T)
    c, s = (t.numpy() for t in wl.rope_tables(pos, (D // 2,), D, "interleaved"))
    eps = 0.05
    kw = dict(row_stride=H * D, col0=0, heads=H, head_dim=D, gamma=g, eps=eps, cos=c, sin=s)
    o1 = oracle_lib.qknorm_rope(x, "bf16", **kw)
    o2 = oracle_lib.qknorm_rope(xa, "bf16", **kw)
    v = _np_decode(x, "bf16")
    ms = np.mean(v * v, axis=-1, keepdims=True)
    e = float(np.float32(eps))
    ratio = a * np.sqrt(ms + e) / np.sqrt(a * a * ms + e)
    assert np.max(np.abs(o2 - ratio * o1)) <= 1e-12


@pytest.mark.parametrize("style", ["interleaved", "rotate_half"])
def test_pair_norm_identity(oracle_lib, style):
    """P-e: |(o_a, o_b)|^2 = |(n_a, n_b)|^2 (c^2 + s^2) for pair-duplicated tables."""
    rng = np.random.default_rng(17)
    T, H, D = 30, 4, 128
    x = _random_tensor(rng, (T, H, D), "bf16", 2.0)
    g = (1 + 0.1 * rng.standard_normal(D)).astype(np.float32)
    pos = rng.integers(0, 10000, T)
    c, s = (t.numpy() for t in wl.rope_tables(pos, (D // 2,), D, style))
    kw = dict(row_stride=H * D, col0=0, heads=H, head_dim=D, gamma=g, eps=1e-6, style=style)
    o = oracle_lib.qknorm_rope(x, "bf16", cos=c, sin=s, **kw)
    ones, zeros = _identity_tables(T, D)
    n = oracle_lib.qknorm_rope(x, "bf16", cos=ones, sin=zeros, **kw)
    a, b = zip(*_pairs(style, D))
    a, b = list(a), list(b)
    lhs = o[..., a] ** 2 + o[..., b] ** 2
    cs = (c[:, a].astype(np.float64) ** 2 + s[:, a].astype(np.float64) ** 2)[:, None, :]
    rhs = (n[..., a] ** 2 + n[..., b] ** 2) * cs
    assert np.max(np.abs(lhs - rhs) / np.maximum(rhs, 1e-300)) <= 1e-13
    assert np.max(np.abs(cs - 1)) <= 2.4e-7


def test_position_zero_is_norm_only(oracle_lib):
    """P-f: the text tokens (all axes at position 0) get cos = 1, sin = 0 exactly."""
    w = wl.WORKLOADS["flux"]
    c, s = (t.numpy() for t in wl.workload_tables(w, "interleaved"))
    assert np.all(c[:w.text_tokens] == 1) and np.all(s[:w.text_tokens] == 0)
    rng = np.random.default_rng(18)
    T, H, D = 8, 3, 128
    x = _random_tensor(rng, (T, H, D), "fp16")
    g = (1 + 0.1 * rng.standard_normal(D)).astype(np.float32)
    kw = dict(row_stride=H * D, col0=0, heads=H, head_dim=D, gamma=g, eps=1e-6)
    o = oracle_lib.qknorm_rope(x, "fp16", cos=c[:T], sin=s[:T], **kw)
    n = _norm_only(oracle_lib, x, "fp16", H, D, g, 1e-6)
    assert np.array_equal(o, n)


def test_styles_agree_under_permutation(oracle_lib):
    """P-g: rotate_half(P x; P gamma, P c, P s) = P interleaved(x; gamma, c, s),
    with P sending dim 2i -> i and 2i+1 -> i + D/2."""
    rng = np.random.default_rng(19)
    T, H, D = 24, 5, 128
    x = _random_tensor(rng, (T, H, D), "bf16", 1.0)
    g = (1 + 0.1 * rng.standard_normal(D)).astype(np.float32)
    c = rng.uniform(-1, 1, (T, D)).astype(np.float32)
    s = rng.uniform(-1, 1, (T, D)).astype(np.float32)
    perm = np.empty(D, np.int64)              # perm[k] = rotate-half slot of interleaved dim k
    perm[0::2] = np.arange(D // 2)
    perm[1::2] = np.arange(D // 2) + D // 2
    inv = np.argsort(perm)                    # rotate-half slot j holds interleaved dim inv[j]
    kw = dict(row_stride=H * D, col0=0, heads=H, head_dim=D, eps=1e-6)
    o_int = oracle_lib.qknorm_rope(x, "bf16", gamma=g, cos=c, sin=s, style="interleaved", **kw)
    o_rh = oracle_lib.qknorm_rope(np.ascontiguousarray(x[..., inv]), "bf16", gamma=g[inv],
                                  cos=np.ascontiguousarray(c[:, inv]),
                                  sin=np.ascontiguousarray(s[:, inv]), style="rotate_half", **kw)
    assert np.max(np.abs(o_rh - o_int[..., inv])) <= 1e-12


def test_relative_position_invariance(oracle_lib):
    """<o_q(m), o_k(n)> depends only on m - n (1-D RoPE is a rotation group)."""
    rng = np.random.default_rng(20)
    D, H = 128, 1
    q = _random_tensor(rng, (1, H, D), "bf16")
    k = _random_tensor(rng, (1, H, D), "bf16")
    g = np.ones(D, np.float32)
    dots = {}
    for m, n in [(0, 3), (10, 13), (500, 503), (7, 0), (1007, 1000)]:
        cq, sq = (t.numpy() for t in wl.rope_tables(np.array([m]), (D // 2,), D, "interleaved"))
        ck, sk = (t.numpy() for t in wl.rope_tables(np.array([n]), (D // 2,), D, "interleaved"))
        kw = dict(row_stride=D, col0=0, heads=H, head_dim=D, gamma=g, eps=1e-6)
        oq = oracle_lib.qknorm_rope(q, "bf16", cos=cq, sin=sq, **kw)
        ok = oracle_lib.qknorm_rope(k, "bf16", cos=ck, sin=sk, **kw)
        dots[(m, n)] = float(np.sum(oq * ok))
    assert abs(dots[(0, 3)] - dots[(10, 13)]) < 1e-4
    assert abs(dots[(0, 3)] - dots[(500, 503)]) < 1e-4
    assert abs(dots[(7, 0)] - dots[(1007, 1000)]) < 1e-4
    assert abs(dots[(0, 3)] - dots[(7, 0)]) > 1e-3   # the offset itself does matter


# ----------------------------------------------------------------------------- addressing


def test_fused_k_slice_equals_separate_tensor(oracle_lib):
    rng = np.random.default_rng(21)
    T, H, D = 9, 3, 64
    qkv = _random_tensor(rng, (T, 3 * H * D), "bf16")
    g = (1 + 0.1 * rng.standard_normal(D)).astype(np.float32)
    c = rng.uniform(-1, 1, (T, D)).astype(np.float32)
    s = rng.uniform(-1, 1, (T, D)).astype(np.float32)
    _, k_fused = oracle_lib.fused_qk(qkv, "bf16", heads=H, head_dim=D, q_gamma=g, k_gamma=g,
                                     eps=1e-6, cos=c, sin=s)
    k_sep = np.ascontiguousarray(qkv[:, H * D:2 * H * D])
    k_alone = oracle_lib.qknorm_rope(k_sep, "bf16", row_stride=H * D, col0=0, heads=H,
                                     head_dim=D, gamma=g, eps=1e-6, cos=c, sin=s)
    assert np.array_equal(k_fused, k_alone)


def test_token_range_is_a_slice(oracle_lib):
    rng = np.random.default_rng(22)
    T, H, D = 17, 2, 128
    x = _random_tensor(rng, (T, H, D), "fp16")
    g = np.ones(D, np.float32)
    c = rng.uniform(-1, 1, (T * H, D)).astype(np.float32)
    s = rng.uniform(-1, 1, (T * H, D)).astype(np.float32)
    kw = dict(row_stride=H * D, col0=0, heads=H, head_dim=D, gamma=g, eps=1e-6, cos=c, sin=s,
              cos_layout="per_head", style="rotate_half")
    full = oracle_lib.qknorm_rope(x, "fp16", **kw)
    part = oracle_lib.qknorm_rope(x, "fp16", t_begin=5, t_end=11, **kw)
    assert np.array_equal(full[5:11], part)


def test_expanded_table_equals_shared(oracle_lib):
    rng = np.random.default_rng(23)
    T, H, D = 6, 4, 64
    x = _random_tensor(rng, (T, H, D), "bf16")
    g = (1 + 0.1 * rng.standard_normal(D)).astype(np.float32)
    c, s = wl.rope_tables(np.arange(T), (D // 2,), D, "interleaved")
    kw = dict(row_stride=H * D, col0=0, heads=H, head_dim=D, gamma=g, eps=1e-6)
    a = oracle_lib.qknorm_rope(x, "bf16", cos=c.numpy(), sin=s.numpy(), **kw)
    b = oracle_lib.qknorm_rope(x, "bf16", cos=wl.expand_per_head(c, H).numpy(),
                               sin=wl.expand_per_head(s, H).numpy(), cos_layout="per_head", **kw)
    assert np.array_equal(a, b)


def test_rejects_bad_arguments(oracle_lib):
    """Odd head_dim or zero heads are refused by the C code, not computed."""
    g = np.ones(63, np.float32)
    c, s = _identity_tables(2, 63)
    with pytest.raises(ValueError):
        oracle_lib.qknorm_rope(np.zeros((2, 63), np.uint16), "bf16", row_stride=63, col0=0,
                               heads=1, head_dim=63, gamma=g, eps=1e-6, cos=c, sin=s)
    c, s = _identity_tables(2, 64)
    with pytest.raises(ValueError):
        oracle_lib.qknorm_rope(np.zeros((2, 64), np.uint16), "bf16", row_stride=64, col0=0,
                               heads=0, head_dim=64, gamma=np.ones(64, np.float32), eps=1e-6,
                               cos=c, sin=s, t_begin=0, t_end=2)


def test_thread_count_does_not_change_results(oracle_lib):
    """Every output element is computed by one thread from its own row, so the
    oracle's bits do not depend on how many threads run (the bench times it
    on one core and on all)."""
    T, H, D = 37, 3, 64
    qkv = wl.fused_qkv(71, T, H, D, "bf16")
    qg, kg = wl.norm_weights(71, D)
    cos, sin = wl.rope_tables(np.arange(T), (D // 2,), D, "interleaved")
    args = dict(heads=H, head_dim=D, q_gamma=qg.numpy(), k_gamma=kg.numpy(), eps=wl.EPS,
                cos=cos.numpy(), sin=sin.numpy(), style="interleaved")
    many = oracle_lib.fused_qk(wl.u16(qkv), "bf16", **args)
    threads = oracle_lib.max_threads()
    oracle_lib.set_threads(1)
    try:
        one = oracle_lib.fused_qk(wl.u16(qkv), "bf16", **args)
    finally:
        oracle_lib.set_threads(threads)
    assert all(np.array_equal(a, b) for a, b in zip(many, one))
