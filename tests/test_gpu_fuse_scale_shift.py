"""GPU parity of the AdaLN modulation (dit_fuse_scale_shift) against the fp64 oracle.

Calls of 8192 rows or more run workgroups of 4 rows that stage the
modulation in LDS; smaller calls run one-row workgroups that read it from L2.
Both schedules are covered, including rows whose batch differs from the one
their workgroup staged.

Bar (no fixed tolerance is given for this step, so it follows from the
arithmetic): every output within half an ulp of the exact value plus fp32
noise, the noise bounded by 8e-6 times the largest term |n (1 + scale)| +
|shift| of its row; and the output equal to the oracle's round-to-nearest-even
image on all but <= 1e-3 of the elements.  In place and out of place must agree
bit for bit; x (out of place), scale and shift stay unchanged; nothing outside
y is written.
"""
import numpy as np
import pytest
import torch

import diffusion_transformer_qk_amd as qkr
import oracle
import workloads as wl
from tests.gpu_common import decode as _decode, same_bits, ulp as _ulp

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")
PAD = 4096
CANARY = 0x6A1B
FP32_NOISE = 8e-6


def _mod_np(t):
    return t.numpy() if t.dtype == torch.float32 else wl.u16(t)


def _mod_name(t):
    return {torch.float32: "fp32", torch.bfloat16: "bf16", torch.float16: "fp16"}[t.dtype]


def _mod_values(t):
    return t.float().numpy().astype(np.float64)


def oracle_rows(x, dtype, sc, sh, rows_per_batch, eps, r0=0, r1=None):
    hidden = x.shape[-1]
    kw = dict(hidden=hidden, rows_per_batch=rows_per_batch, mod_dtype=_mod_name(sc), eps=eps,
              row_begin=r0, row_end=r1)
    y = oracle.adaln(wl.u16(x), dtype, scale=_mod_np(sc), shift=_mod_np(sh), **kw)
    z = np.zeros_like(_mod_np(sc))
    n = oracle.adaln(wl.u16(x), dtype, scale=z, shift=z, **kw)
    return y, n


def check_rows(got, y, n, sc, sh, rows_per_batch, r0, dtype, what):
    rows = y.shape[0]
    b = (np.arange(r0, r0 + rows) // rows_per_batch)
    scv, shv = _mod_values(sc)[b], _mod_values(sh)[b]
    terms = np.abs(n) * np.abs(1 + scv) + np.abs(shv)
    bound = 0.5 * _ulp(y, dtype) + FP32_NOISE * terms.max(axis=1, keepdims=True)
    got = got.reshape(y.shape)
    err = np.abs(got - y)
    over = err > bound
    assert not over.any(), "%s: %d outside the rounding model, worst excess %.3g" % (
        what, int(over.sum()), float((err - bound).max()))
    rne = oracle.round_to(y, dtype)
    n_diff = int(np.count_nonzero(got != rne))
    assert n_diff <= max(2, 1e-3 * got.size), "%s: %d of %d differ from RNE" % (what, n_diff, got.size)
    return float(err.max())


def guarded_empty(shape, dtype):
    n = int(np.prod(shape))
    buf = torch.full((n + 2 * PAD,), CANARY, dtype=torch.int16, device=DEV)
    return buf[PAD:PAD + n].view(dtype).view(shape), buf


def canaries_intact(buf):
    return bool((buf[:PAD] == CANARY).all()) and bool((buf[-PAD:] == CANARY).all())


def run(x, sc, sh, rows_per_batch=None, eps=wl.EPS, inplace=False):
    xd, scd, shd = x.to(DEV), sc.to(DEV), sh.to(DEV)
    keep = [t.clone() for t in (xd, scd, shd)]
    if inplace:
        out = qkr.fuse_scale_shift(xd, scd, shd, out=xd, eps=eps, rows_per_batch=rows_per_batch)
        torch.cuda.synchronize()
        assert same_bits(scd, keep[1]) and same_bits(shd, keep[2])
        return out.cpu()
    y, buf = guarded_empty(x.shape, x.dtype)
    qkr.fuse_scale_shift(xd, scd, shd, out=y, eps=eps, rows_per_batch=rows_per_batch)
    torch.cuda.synchronize()
    assert canaries_intact(buf), "write outside y"
    for a, b in zip(keep, (xd, scd, shd)):
        assert same_bits(a, b), "input changed"
    return y.cpu()


@pytest.mark.parametrize("dtype,mod", [("bf16", "fp32"), ("bf16", "bf16"), ("fp16", "fp32"),
                                       ("fp16", "fp16"), ("bf16", "fp16")])
def test_flux_shape_full(dtype, mod):
    w = wl.ADALN_WORKLOADS["adaln_flux"]
    x, sc, sh = wl.adaln_inputs(w.seed, w.rows, w.hidden, w.batches, dtype, mod)
    out = run(x, sc, sh)
    y, n = oracle_rows(x, dtype, sc, sh, w.rows_per_batch, wl.EPS)
    m = check_rows(_decode(out, dtype), y, n, sc, sh, w.rows_per_batch, 0, dtype, "flux")
    print("flux", dtype, mod, "max_abs", m, "max|y|", np.abs(y).max())


def _windows(rows, rng, n=10, width=40, extra=()):
    starts = sorted(set(rng.integers(0, rows - width, n).tolist()) | set(extra))
    return [(0, width)] + [(s, s + width) for s in starts] + [(rows - width, rows)]


@pytest.mark.parametrize("key", ["adaln_wan", "adaln_wan_cfg2"])
def test_wan_shapes_sampled(key):
    w = wl.ADALN_WORKLOADS[key]
    x, sc, sh = wl.adaln_inputs(w.seed, w.rows, w.hidden, w.batches, "bf16", "fp32")
    out = run(x, sc, sh)
    rng = np.random.default_rng(w.seed)
    boundary = [w.rows_per_batch - 20] if w.batches > 1 else []
    worst = 0.0
    for a, b in _windows(w.rows, rng, extra=boundary):
        y, n = oracle_rows(x, "bf16", sc, sh, w.rows_per_batch, wl.EPS, a, b)
        worst = max(worst, check_rows(_decode(out[a:b], "bf16"), y, n, sc, sh, w.rows_per_batch,
                                      a, "bf16", "%s rows %d:%d" % (key, a, b)))
    print(key, "sampled max_abs", worst)


@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
def test_in_place_equals_out_of_place(dtype):
    x, sc, sh = wl.adaln_inputs(77, 300, 5120, 3, dtype, "bf16")
    a = run(x, sc, sh)
    b = run(x, sc, sh, inplace=True)
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))


@pytest.mark.parametrize("rows,hidden,rpb,batches", [
    (1, 8, 1, 1), (3, 64, 1, 3), (257, 1000, 100, 3), (65, 2048, 13, 5), (17, 6152, 4, 5),
    (9, 8192, 9, 1), (40, 24, 7, 6), (128, 3072, 64, 2), (5, 2056, 2, 3)])
@pytest.mark.parametrize("dtype,mod", [("bf16", "fp32"), ("fp16", "bf16")])
def test_ragged_widths_and_batches(rows, hidden, rpb, batches, dtype, mod):
    x, sc, sh = wl.adaln_inputs(rows * 7 + hidden, rows, hidden, batches, dtype, mod)
    out = run(x, sc, sh, rows_per_batch=rpb)
    y, n = oracle_rows(x, dtype, sc, sh, rpb, wl.EPS)
    check_rows(_decode(out, dtype), y, n, sc, sh, rpb, 0, dtype, "ragged")


def test_constant_rows_and_large_eps():
    rows, hidden = 6, 512
    x = torch.full((rows, hidden), 3.25, dtype=torch.bfloat16)
    x[3] = torch.linspace(-4, 4, hidden).to(torch.bfloat16)
    sc = torch.randn(1, hidden, generator=torch.Generator().manual_seed(3)) * 0.5
    sh = torch.randn(1, hidden, generator=torch.Generator().manual_seed(4)) * 0.5
    for eps in (1e-6, 0.5):
        out = run(x, sc, sh, eps=eps)
        y, n = oracle_rows(x, "bf16", sc, sh, rows, eps)
        check_rows(_decode(out, "bf16"), y, n, sc, sh, rows, 0, "bf16", "constant eps=%g" % eps)
        # a constant row normalises to zero: its output is the shift, rounded once
        assert np.array_equal(_decode(out[0], "bf16"), oracle.round_to(_mod_values(sh)[0], "bf16"))


def test_zero_rows_is_a_no_op():
    x = torch.zeros(0, 64, dtype=torch.bfloat16, device=DEV)
    s = torch.zeros(1, 64, device=DEV)
    out = qkr.fuse_scale_shift(x, s, s, rows_per_batch=1)
    torch.cuda.synchronize()
    assert out.shape == (0, 64)


def test_partial_overlap_and_misalignment_are_rejected():
    rows, hidden = 8, 64
    buf = torch.zeros(2 * rows * hidden + 8, dtype=torch.bfloat16, device=DEV)
    x = buf[:rows * hidden].view(rows, hidden)
    y = buf[hidden:hidden + rows * hidden].view(rows, hidden)        # overlaps x by 7 rows
    s = torch.zeros(1, hidden, device=DEV)
    with pytest.raises(qkr.QkrError) as e:
        qkr.fuse_scale_shift(x, s, s, out=y)
    assert e.value.status == qkr.binding.QKR_ERR_ARG
    xm = buf[1:1 + rows * hidden].view(rows, hidden)                 # 2-byte offset
    with pytest.raises(qkr.QkrError) as e:
        qkr.fuse_scale_shift(xm, s, s)
    assert e.value.status == qkr.binding.QKR_ERR_ALIGN


def test_byte_offsets_beyond_4gib_in_place():
    """[420000, 5120] bf16 = 4.3 GB in place: rows on both sides of the 2^32-byte
    offset (row 419430 straddles it) against the oracle.  The rows repeat a
    1024-row block; one modulation row."""
    rows, hidden, B = 420000, 5120, 1024
    block, sc, sh = wl.adaln_inputs(4343, B, hidden, 1, "bf16", "fp32")
    blk = block.to(DEV)
    x = torch.empty((rows, hidden), dtype=torch.bfloat16, device=DEV)
    for i in range(0, rows, B):
        x[i:i + B].copy_(blk[:min(B, rows - i)])
    qkr.fuse_scale_shift(x, sc.to(DEV), sh.to(DEV), out=x, rows_per_batch=rows)
    torch.cuda.synchronize()
    samples = [0, 1, 1023, 1024, 209715, 419429, 419430, 419431, rows - 1]
    assert max(samples) < rows
    idx = torch.tensor(samples)
    xs = block[idx % B]
    y, n = oracle_rows(xs, "bf16", sc, sh, len(samples), wl.EPS)
    m = check_rows(_decode(x[idx.to(DEV)], "bf16"), y, n, sc, sh, len(samples), 0, "bf16",
                   ">4GiB rows")
    print("beyond 4 GiB max_abs", m)


@pytest.mark.parametrize("rows,hidden,rpb,mod", [
    (16390, 512, 4097, "fp32"),      # staged; workgroups straddle every batch boundary
    (8195, 64, 5, "bf16"),           # staged; most rows outside the staged batch
    (8192, 8192, 8192, "fp32"),      # staged 64 KB of modulation, widest rows
    (8200, 5128, 4100, "fp16"),      # staged, a row tail (641 vectors)
    (8191, 5128, 4095, "fp32"),      # one below the staging threshold, same tail
    (300, 8, 7, "fp32"),             # one vector per row
])
def test_staging_schedules_and_tails(rows, hidden, rpb, mod):
    batches = -(-rows // rpb)
    x, sc, sh = wl.adaln_inputs(rows + hidden, rows, hidden, batches, "bf16", mod)
    out = run(x, sc, sh, rows_per_batch=rpb)
    rng = np.random.default_rng(rows)
    edges = sorted({b * rpb + d for b in range(1, batches) for d in (-3, -1, 0, 2)} |
                   set(rng.integers(0, rows, 6).tolist()) | {0, rows - 1})
    worst = 0.0
    for a in edges:
        a = max(0, min(a, rows - 4))
        y, n = oracle_rows(x, "bf16", sc, sh, rpb, wl.EPS, a, a + 4)
        worst = max(worst, check_rows(_decode(out[a:a + 4], "bf16"), y, n, sc, sh, rpb, a, "bf16",
                                      "rows %d:%d" % (a, a + 4)))
    print("staging", rows, hidden, rpb, mod, "max_abs", worst)


@pytest.mark.parametrize("rows", [300, 9000])      # one-row and staging schedules
def test_graph_capture_replays_match_eager(rows):
    """The call holds no allocation, copy or synchronisation: captured into a
    graph, every replay (with eager work and synchronisation between them)
    equals the eager result bit for bit."""
    hidden = 1024
    x, sc, sh = wl.adaln_inputs(rows, rows, hidden, 3, "bf16", "fp32")
    xd, scd, shd = x.to(DEV), sc.to(DEV), sh.to(DEV)
    rpb = -(-rows // 3)
    eager = qkr.fuse_scale_shift(xd, scd, shd, rows_per_batch=rpb)
    out = torch.empty_like(xd)
    st = torch.cuda.Stream()
    graph = torch.cuda.CUDAGraph()
    torch.cuda.synchronize()
    with torch.cuda.graph(graph, stream=st):
        qkr.fuse_scale_shift(xd, scd, shd, out=out, rows_per_batch=rpb)
    torch.cuda.synchronize()
    for replay in range(3):
        out.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), eager.view(torch.int16)), replay


def test_concurrent_streams_are_independent():
    """Calls on four streams over different buffers, both schedules, at once."""
    cases = []
    for i in range(4):
        rows = (300, 9000)[i % 2]
        x, sc, sh = wl.adaln_inputs(500 + i, rows, 2048, 1, "fp16", "bf16")
        cases.append((x, sc, sh, x.to(DEV), sc.to(DEV), sh.to(DEV), torch.cuda.Stream()))
    torch.cuda.synchronize()
    outs = []
    for x, sc, sh, xd, scd, shd, st in cases:
        with torch.cuda.stream(st):
            outs.append(qkr.fuse_scale_shift(xd, scd, shd, stream=st))
    torch.cuda.synchronize()
    for (x, sc, sh, *_), out in zip(cases, outs):
        rows = x.shape[0]
        y, n = oracle_rows(x, "fp16", sc, sh, rows, wl.EPS, 0, 64)
        check_rows(_decode(out[:64], "fp16"), y, n, sc, sh, rows, 0, "fp16", "stream")
        y, n = oracle_rows(x, "fp16", sc, sh, rows, wl.EPS, rows - 64, rows)
        check_rows(_decode(out[rows - 64:], "fp16"), y, n, sc, sh, rows, rows - 64, "fp16",
                   "stream tail")


def test_maximum_rows():
    """The largest row count the library takes: rows = 2^24 - 1 of hidden 8
    (268 MB), three batches of 5,592,405 rows, 2^22 staging workgroups.
    Sampled rows at both ends, the middle and every batch boundary against the
    oracle.  Rows repeat a 4096-row block (the step is per row)."""
    rows, hidden, B, batches = (1 << 24) - 1, 8, 4096, 3
    rpb = rows // batches
    block, sc, sh = wl.adaln_inputs(4747, B, hidden, batches, "bf16", "fp32")
    blk = block.to(DEV)
    n = rows // B
    x = torch.empty((rows, hidden), dtype=torch.bfloat16, device=DEV)
    x[:n * B].view(n, B, hidden).copy_(blk.unsqueeze(0).expand(n, -1, -1))
    x[n * B:].copy_(blk[:rows - n * B])
    y = qkr.fuse_scale_shift(x, sc.to(DEV), sh.to(DEV), rows_per_batch=rpb)
    torch.cuda.synchronize()
    rng = np.random.default_rng(4748)
    samples = sorted({0, 1, B, rpb - 1, rpb, 2 * rpb - 1, 2 * rpb, rows // 2, rows - 2,
                      rows - 1, *rng.integers(0, rows, 20).tolist()})
    assert max(samples) < rows
    got_all = _decode(y[torch.tensor(samples, device=DEV)], "bf16")
    m = 0.0
    for i, r in enumerate(samples):
        b = r // rpb
        yr, nr = oracle_rows(block[r % B:r % B + 1], "bf16", sc[b:b + 1], sh[b:b + 1], 1, wl.EPS)
        m = max(m, check_rows(got_all[i:i + 1], yr, nr, sc[b:b + 1], sh[b:b + 1], 1, 0, "bf16",
                              "row %d" % r))
    print("maximum rows max_abs", m)


@pytest.mark.parametrize("dtype,mod", [("bf16", "fp32"), ("bf16", "bf16"), ("bf16", "fp16"),
                                       ("fp16", "fp32"), ("fp16", "bf16"), ("fp16", "fp16")])
def test_every_kernel_instantiation(dtype, mod):
    """Every compiled kernel of one (data, modulation) dtype pair: 2..16 row
    vectors per lane, rows of exactly that many vectors and rows 8 elements
    short (tail masks), one-row workgroups (203 rows) and workgroups of 4
    staging the modulation (8200 rows), each over batches that split inside a
    workgroup.  Sampled rows against the oracle.  Rows repeat a 256-row block
    (the step is per row)."""
    B = 256
    rng = np.random.default_rng(6000)
    hit = set()
    for vpl in range(2, 17, 2):
        for hidden in (vpl * 512, vpl * 512 - 8):
            block, sc3, sh3 = wl.adaln_inputs(6000 + hidden, B, hidden, 3, dtype, mod)
            blk = block.to(DEV)
            for rows, rpb in ((203, 101), (8200, 4099)):
                batches = -(-rows // rpb)
                sc, sh = sc3[:batches], sh3[:batches]
                n = rows // B
                x = torch.empty((rows, hidden), dtype=blk.dtype, device=DEV)
                if n:
                    x[:n * B].view(n, B, hidden).copy_(blk.unsqueeze(0).expand(n, -1, -1))
                x[n * B:].copy_(blk[:rows - n * B])
                y = qkr.fuse_scale_shift(x, sc.to(DEV), sh.to(DEV), rows_per_batch=rpb)
                torch.cuda.synchronize()
                # the dispatch rule: vectors per lane, whole rows of them, staged schedule
                hit.add((vpl, hidden == vpl * 512, rows >= 8192))
                samples = sorted(r for r in {0, 1, 2, 3, rpb - 1, rpb, rows // 2, rows - 2,
                                             rows - 1, *rng.integers(0, rows, 6).tolist()}
                                 if r < rows)
                assert samples[-1] < rows          # checked before indexing on the GPU
                got_all = _decode(y[torch.tensor(samples, device=DEV)], dtype)
                refs = [oracle_rows(block[r % B:r % B + 1], dtype, sc[r // rpb:r // rpb + 1],
                                    sh[r // rpb:r // rpb + 1], 1, wl.EPS) for r in samples]
                bsel = torch.tensor([r // rpb for r in samples])
                # one row of modulation per sampled row; the RNE-agreement
                # fraction is taken over all of the case's sampled rows
                check_rows(got_all, np.concatenate([a for a, _ in refs]),
                           np.concatenate([b for _, b in refs]), sc[bsel], sh[bsel], 1, 0, dtype,
                           "hidden %d rows %d" % (hidden, rows))
    assert hit == {(v, f, s) for v in range(2, 17, 2) for f in (True, False)
                   for s in (True, False)}


# ----------------------------------------------------------------------------- large and tiny finite values


def _rows_with_peaks(rng, rows, hidden, peaks):
    """fp64 [rows, hidden]: N(0.5, 1) rows rescaled so that each row's largest
    |x| is one of `peaks`, cycling over the rows."""
    raw = rng.standard_normal((rows, hidden)) + 0.5
    raw /= np.abs(raw).max(axis=1, keepdims=True)
    return raw * np.asarray(peaks, dtype=np.float64)[np.arange(rows) % len(peaks)][:, None]


def _special_rows(raw, rng):
    """A constant row at 3e38 (zero variance), an O(1) row with one element
    at 3.3e38, and a row alternating +-3.3e38."""
    hidden = raw.shape[1]
    raw[1] = 3e38
    raw[2] = rng.standard_normal(hidden)
    raw[2, 5] = 3.3e38
    raw[3] = 3.3e38 * np.where(np.arange(hidden) % 2 == 0, 1.0, -1.0)
    return raw


@pytest.mark.parametrize("rows,hidden", [(64, 5120), (70, 1000), (8200, 1024)])
def test_large_finite_bf16_rows(rows, hidden):
    """bf16 rows whose fp32 sums or squared deviations overflow (largest |x|
    1e18, 1e30, 3e38) between O(1) rows, in the one-row schedule (with a full
    and a ragged row width) and in the 4-row staging schedule; plus a constant
    row of 3e38, a spike and an alternating +-3.3e38 row.  Every element
    against the oracle."""
    rng = np.random.default_rng(800 + rows)
    raw = _special_rows(_rows_with_peaks(rng, rows, hidden, [1.0, 1e18, 1e30, 3e38, 7.0]), rng)
    x = torch.from_numpy(raw.astype(np.float32)).to(torch.bfloat16)
    assert torch.isfinite(x.float()).all()
    sc = torch.from_numpy((0.5 * rng.standard_normal((1, hidden))).astype(np.float32))
    sh = torch.from_numpy((0.5 * rng.standard_normal((1, hidden))).astype(np.float32))
    out = run(x, sc, sh)
    y, n = oracle_rows(x, "bf16", sc, sh, rows, wl.EPS)
    got = _decode(out, "bf16")
    m = check_rows(got, y, n, sc, sh, rows, 0, "bf16", "large rows %dx%d" % (rows, hidden))
    # the constant row is the shift alone (up to its rounding)
    assert np.all(got.reshape(rows, hidden)[1] == oracle.round_to(_mod_values(sh)[0], "bf16"))
    inplace = run(x, sc, sh, inplace=True)
    assert torch.equal(inplace.view(torch.int16), out.view(torch.int16))
    print("large finite bf16 rows", rows, hidden, "max_abs", m)


@pytest.mark.parametrize("eps", [1e-6, 1e-38, 1.4e-45])
@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
def test_tiny_rows_and_tiny_eps(eps, dtype):
    """Rows of tiny values (down to bf16 subnormals near 1e-40, fp16
    subnormals near 1e-7) with eps down to the smallest fp32 subnormal; an
    all-zero row.  Every element against the oracle."""
    rows, hidden = 48, 2048
    rng = np.random.default_rng(810)
    peaks = ([1.0, 1e-12, 1e-20, 1e-30, 1e-38, 1e-40] if dtype == "bf16"
             else [1.0, 1e-3, 1e-5, 3e-7, 5.0])
    raw = _rows_with_peaks(rng, rows, hidden, peaks)
    raw[0] = 0.0
    x = torch.from_numpy(raw.astype(np.float32)).to(wl.DTYPES[dtype])
    sc = torch.from_numpy((0.5 * rng.standard_normal((1, hidden))).astype(np.float32))
    sh = torch.from_numpy((0.5 * rng.standard_normal((1, hidden))).astype(np.float32))
    out = run(x, sc, sh, eps=eps)
    y, n = oracle_rows(x, dtype, sc, sh, rows, eps)
    m = check_rows(_decode(out, dtype), y, n, sc, sh, rows, 0, dtype, "tiny rows eps %g" % eps)
    print("tiny rows", dtype, "eps", eps, "max_abs", m)
