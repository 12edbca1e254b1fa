"""GPU parity of the group norm + SiLU step (dit_group_norm_silu) against the fp64 oracle.

Bar (no fixed tolerance is given for this step, so it follows from the
arithmetic): every output within half an ulp of the exact value plus fp32
noise, bounded by 8e-6 times (1 + the largest |output| of its group) -- the
normalised value t carries a relative fp32 error of a few ulp and SiLU's slope
is at most 1.1 -- and the output equal to the oracle's round-to-nearest-even
image on all but <= 1e-3 of the elements.  In place and out of place agree bit
for bit; x (out of place), gamma and beta stay unchanged; nothing outside y is
written.
"""
import numpy as np
import pytest
import torch

import diffusion_transformer_qk_amd as qkr
import oracle
import workloads as wl
from tests import gn_hooks
from tests.gpu_common import decode as _decode, same_bits, ulp as _ulp

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")
PAD = 4096
CANARY = 0x5C3D
FP32_NOISE = 8e-6


def _pnp(t):
    return t.numpy() if t.dtype == torch.float32 else wl.u16(t)


def _pname(t):
    return {torch.float32: "fp32", torch.bfloat16: "bf16", torch.float16: "fp16"}[t.dtype]


def check_groups(got, ref, gsize, dtype, what, rne_check=True):
    """got, ref: flat arrays covering whole groups of gsize elements."""
    ref_g = ref.reshape(-1, gsize)
    got_g = got.reshape(ref_g.shape)
    scale = 1.0 + np.abs(ref_g).max(axis=1, keepdims=True)
    bound = 0.5 * _ulp(ref_g, dtype) + FP32_NOISE * scale
    err = np.abs(got_g - ref_g)
    over = err > bound
    assert not over.any(), "%s: %d outside the rounding model, worst excess %.3g" % (
        what, int(over.sum()), float((err - bound).max()))
    if rne_check:
        rne = oracle.round_to(ref_g, dtype)
        n_diff = int(np.count_nonzero(got_g != rne))
        assert n_diff <= max(2, 1e-3 * got_g.size), "%s: %d of %d differ from RNE" % (
            what, n_diff, got_g.size)
    return float(err.max())


def run(x, gamma, beta, groups, eps=wl.EPS, inplace=False):
    xd, gd, bd = x.to(DEV), gamma.to(DEV), beta.to(DEV)
    keep = [t.clone() for t in (xd, gd, bd)]
    if inplace:
        out = qkr.group_norm_silu(xd, gd, bd, groups, out=xd, eps=eps)
        torch.cuda.synchronize()
        assert same_bits(gd, keep[1]) and same_bits(bd, keep[2])
        return out.cpu()
    n = x.numel()
    buf = torch.full((n + 2 * PAD,), CANARY, dtype=torch.int16, device=DEV)
    y = buf[PAD:PAD + n].view(x.dtype).view(x.shape)
    qkr.group_norm_silu(xd, gd, bd, groups, out=y, eps=eps)
    torch.cuda.synchronize()
    assert bool((buf[:PAD] == CANARY).all()) and bool((buf[-PAD:] == CANARY).all()), "write outside y"
    for a, b in zip(keep, (xd, gd, bd)):
        assert same_bits(a, b), "input changed"
    return y.cpu()


def oracle_groups(x, dtype, channels, spatial, groups, gamma, beta, eps, g0=0, g1=None):
    return oracle.group_norm_silu(wl.u16(x), dtype, channels=channels, spatial=spatial,
                                  groups=groups, gamma=_pnp(gamma), beta=_pnp(beta),
                                  param_dtype=_pname(gamma), eps=eps, group_begin=g0,
                                  group_end=g1)


@pytest.mark.parametrize("dtype,param_dtype", [("bf16", "fp32"), ("fp16", "bf16")])
def test_vae_mid_full(dtype, param_dtype):
    w = wl.GN_WORKLOADS["gn_vae_mid"]
    x, g, b = wl.gn_inputs(w.seed, w.n, w.channels, w.spatial, dtype, param_dtype)
    out = run(x, g, b, w.groups)
    ref = oracle_groups(x, dtype, w.channels, w.spatial, w.groups, g, b, wl.EPS)
    gsize = w.channels // w.groups * w.spatial
    m = check_groups(_decode(out, dtype), ref, gsize, dtype, "vae mid")
    print("vae mid", dtype, param_dtype, "max_abs", m)


@pytest.mark.parametrize("key,dtype", [("gn_vae_up", "bf16"), ("gn_vae_up", "fp16"),
                                       ("gn_vae_out", "bf16")])
def test_vae_large_sampled_groups(key, dtype):
    """Many chunks per group; the oracle checks first, last and a few inner groups."""
    w = wl.GN_WORKLOADS[key]
    x, g, b = wl.gn_inputs(w.seed, w.n, w.channels, w.spatial, dtype, "fp32")
    out = run(x, g, b, w.groups)
    gsize = w.channels // w.groups * w.spatial
    pairs = w.n * w.groups
    flat = out.reshape(-1)
    worst = 0.0
    for q in sorted({0, 1, 11, 12, pairs // 2, pairs - 1}):
        ref = oracle_groups(x, dtype, w.channels, w.spatial, w.groups, g, b, wl.EPS, q, q + 1)
        got = _decode(flat[q * gsize:(q + 1) * gsize], dtype)
        worst = max(worst, check_groups(got, ref, gsize, dtype, "%s group %d" % (key, q)))
    print(key, dtype, "sampled max_abs", worst)


@pytest.mark.parametrize("n,channels,h,w,groups", [
    (2, 64, 8, 8, 8),          # one chunk per group (single-kernel path)
    (3, 32, 16, 16, 32),       # instance norm
    (2, 16, 8, 16, 1),         # layer norm over (C, S)
    (1, 4, 64, 64, 1),         # group of exactly one chunk (16384)
    (1, 8, 16392, 1, 4),       # 2 x 16392 = 32784 elements: last chunk of 16
    (2, 6, 40, 200, 3),        # 16000: one chunk, ragged thread tail
    (1, 12, 96, 96, 2),        # 55296: 4 chunks, last partial
    (1, 256, 8, 8, 1),         # 16384 in one group
])
@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
def test_chunk_boundaries(n, channels, h, w, groups, dtype):
    spatial = h * w
    x, g, b = wl.gn_inputs(n * 1000 + channels + spatial, n, channels, spatial, dtype, "fp32")
    x = x.view(n, channels, h, w)
    out = run(x, g, b, groups)
    ref = oracle_groups(x, dtype, channels, spatial, groups, g, b, wl.EPS)
    check_groups(_decode(out, dtype), ref, channels // groups * spatial, dtype, "boundary")


@pytest.mark.parametrize("shape,groups", [((1, 64, 128, 128), 32), ((2, 32, 24, 24), 8)])
def test_in_place_equals_out_of_place(shape, groups):
    n, c = shape[0], shape[1]
    x, g, b = wl.gn_inputs(55, n, c, shape[2] * shape[3], "bf16", "bf16")
    x = x.view(shape)
    a = run(x, g, b, groups)
    b2 = run(x, g, b, groups, inplace=True)
    assert torch.equal(a.view(torch.int16), b2.view(torch.int16))


def test_constant_groups_and_zero_gamma():
    """A constant group, or gamma = 0, leaves t = beta exactly: y = silu(beta) per channel."""
    n, channels, spatial, groups = 1, 16, 2048, 4
    b = torch.linspace(-3, 3, channels)
    bd = b.double().numpy()
    want = np.broadcast_to((bd / (1 + np.exp(-bd)))[None, :, None], (n, channels, spatial))
    gsize = channels // groups * spatial
    x = torch.full((n, channels, spatial), -0.625, dtype=torch.bfloat16)
    out = run(x, torch.ones(channels), b, groups)
    # every element of a channel is the same value, so one rounding tie would move
    # 2048 elements at once: only the per-element rounding model applies here
    check_groups(_decode(out, "bf16"), want.reshape(-1), gsize, "bf16", "constant group",
                 rne_check=False)
    x2, _, _ = wl.gn_inputs(9, n, channels, spatial, "bf16", "fp32")
    out2 = run(x2, torch.zeros(channels), b, groups)
    check_groups(_decode(out2, "bf16"), want.reshape(-1), gsize, "bf16", "zero gamma",
                 rne_check=False)


def test_workspace_errors_and_explicit_workspace():
    n, channels, spatial, groups = 1, 64, 64 * 64, 32     # 8192-element groups: no workspace
    assert qkr.group_norm_silu_workspace_size(n, channels, spatial, groups) == 0
    n, channels, spatial, groups = 1, 32, 128 * 128, 8    # 65536-element groups: 16 chunks
    need = qkr.group_norm_silu_workspace_size(n, channels, spatial, groups)
    assert need == 8 * 16 * 8
    x, g, b = wl.gn_inputs(10, n, channels, spatial, "bf16", "fp32")
    xd, gd, bd = x.to(DEV), g.to(DEV), b.to(DEV)
    short = torch.empty(need - 8, dtype=torch.uint8, device=DEV)
    with pytest.raises(qkr.QkrError) as e:
        qkr.group_norm_silu(xd, gd, bd, groups, workspace=short)
    assert e.value.status == qkr.binding.QKR_ERR_WORKSPACE
    ws = torch.full((need,), 0x7F, dtype=torch.uint8, device=DEV)     # garbage contents
    out = qkr.group_norm_silu(xd, gd, bd, groups, workspace=ws)
    torch.cuda.synchronize()
    ref = oracle_groups(x, "bf16", channels, spatial, groups, g, b, wl.EPS)
    check_groups(_decode(out, "bf16"), ref, channels // groups * spatial, "bf16", "workspace")


def test_zero_samples_is_a_no_op():
    x = torch.zeros(0, 8, 8, 8, dtype=torch.bfloat16, device=DEV)
    p = torch.ones(8, device=DEV)
    out = qkr.group_norm_silu(x, p, p, 4)
    torch.cuda.synchronize()
    assert out.shape == x.shape


def test_repeated_calls_reuse_one_workspace():
    """Back-to-back calls on one workspace, then in place: identical bits."""
    n, channels, spatial, groups = 2, 64, 64 * 64, 8            # 8 groups of 2 chunks
    x, g, b = wl.gn_inputs(31, n, channels, spatial, "bf16", "fp32")
    xd, gd, bd = x.to(DEV), g.to(DEV), b.to(DEV)
    ws = torch.empty(qkr.group_norm_silu_workspace_size(n, channels, spatial, groups),
                     dtype=torch.uint8, device=DEV)
    outs = [qkr.group_norm_silu(xd, gd, bd, groups, workspace=ws) for _ in range(4)]
    qkr.group_norm_silu(xd, gd, bd, groups, out=xd, workspace=ws)
    torch.cuda.synchronize()
    for o in outs[1:] + [xd]:
        assert torch.equal(o.view(torch.int16), outs[0].view(torch.int16))
    ref = oracle_groups(x, "bf16", channels, spatial, groups, g, b, wl.EPS)
    check_groups(_decode(outs[0], "bf16"), ref, channels // groups * spatial, "bf16", "repeat")


def test_graph_capture_replays_match_eager():
    """The two-pass kernels recorded into a graph: every replay, with eager
    work and synchronisation between replays, equals the eager result."""
    n, channels, spatial, groups = 1, 64, 128 * 128, 8             # 8 chunks per group
    x, g, b = wl.gn_inputs(77, n, channels, spatial, "bf16", "fp32")
    xd, gd, bd = x.to(DEV), g.to(DEV), b.to(DEV)
    eager = qkr.group_norm_silu(xd, gd, bd, groups)
    ws = torch.empty(qkr.group_norm_silu_workspace_size(n, channels, spatial, groups),
                     dtype=torch.uint8, device=DEV)
    out = torch.empty_like(xd)
    stream = torch.cuda.Stream()
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(stream):
        with torch.cuda.graph(graph, stream=stream):
            qkr.group_norm_silu(xd, gd, bd, groups, out=out, workspace=ws)
    torch.cuda.synchronize()
    for _ in range(3):
        out.zero_()
        ws.fill_(0x7F)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), eager.view(torch.int16))


def test_byte_offsets_beyond_4gib_in_place():
    """[260, 128, 256, 256] bf16 = 4.4 GB in place, 32 groups of 16 chunks:
    8320 groups, 133,120 chunks (the lagged schedule: 133,120 + 768
    workgroups); groups on both sides of the 2^32-byte offset
    (group 8192 starts there) against the oracle.  The samples repeat a
    4-sample block."""
    n, channels, spatial, groups, B = 260, 128, 256 * 256, 32, 4
    assert qkr.group_norm_silu_schedule(n, channels, spatial, groups)[0] == "lagged"
    block, g, b = wl.gn_inputs(4444, B, channels, spatial, "bf16", "fp32")
    blk = block.to(DEV)
    x = torch.empty((n, channels, spatial), dtype=torch.bfloat16, device=DEV)
    for i in range(0, n, B):
        x[i:i + B].copy_(blk[:min(B, n - i)])
    qkr.group_norm_silu(x, g.to(DEV), b.to(DEV), groups, out=x)
    torch.cuda.synchronize()
    gsize = channels // groups * spatial
    flat = x.view(-1)
    for q in (0, 8191, 8192, 8193, n * groups - 1):
        ref = oracle_groups(block, "bf16", channels, spatial, groups, g, b, wl.EPS,
                            q % (B * groups), q % (B * groups) + 1)
        got = _decode(flat[q * gsize:(q + 1) * gsize], "bf16")
        check_groups(got, ref, gsize, "bf16", ">4GiB group %d" % q)


def test_concurrent_streams_are_independent():
    """Group-norm calls on four streams (own workspaces) at once."""
    cases = []
    for i in range(4):
        n, channels, spatial, groups = 1, 32, (64 * 64, 256 * 256)[i % 2], 4
        x, g, b = wl.gn_inputs(600 + i, n, channels, spatial, "bf16", "fp32")
        cases.append((x, g, b, spatial, x.to(DEV), g.to(DEV), b.to(DEV), torch.cuda.Stream()))
    torch.cuda.synchronize()
    outs = []
    for x, g, b, spatial, xd, gd, bd, st in cases:
        with torch.cuda.stream(st):
            outs.append(qkr.group_norm_silu(xd, gd, bd, 4, stream=st))
    torch.cuda.synchronize()
    for (x, g, b, spatial, *_), out in zip(cases, outs):
        ref = oracle_groups(x, "bf16", 32, spatial, 4, g, b, wl.EPS)
        check_groups(_decode(out, "bf16"), ref, 32 // 4 * spatial, "bf16", "stream")


@pytest.mark.parametrize("n,channels,spatial,chunk", [
    (4, 512, 16392, 16384),     # 2176 workgroups at 16384: a 128-element last chunk
    (4, 256, 30000, 8192),      # 1920 at 16384, so 8192: a 2432-element last chunk
    (1, 512, 128 * 128, 4096),  # the VAE mid stage: 4096-element chunks
])
def test_chunk_size_follows_call_size(n, channels, spatial, chunk):
    groups = 32
    gsize = channels // groups * spatial
    chunks = -(-gsize // chunk)
    assert qkr.group_norm_silu_workspace_size(n, channels, spatial, groups) == n * groups * chunks * 8
    x, g, b = wl.gn_inputs(n * 31 + spatial, n, channels, spatial, "bf16", "fp32")
    out = run(x, g, b, groups)
    flat = out.reshape(-1)
    for q in sorted({0, 1, n * groups // 2, n * groups - 1}):
        ref = oracle_groups(x, "bf16", channels, spatial, groups, g, b, wl.EPS, q, q + 1)
        check_groups(_decode(flat[q * gsize:(q + 1) * gsize], "bf16"), ref, gsize, "bf16",
                     "chunk %d group %d" % (chunk, q))


def test_maximum_workgroups():
    """The largest grid the library launches: n = 2^24 - 1 samples of one
    8-element group ([16777215, 1, 8] bf16, 268 MB), one single-read workgroup
    each, 2^24 - 1 workgroups of 256 threads (the most a launch grid holds).
    Sampled groups at both ends and the middle against the oracle.  Samples
    repeat a 4096-sample block (the step is per group)."""
    n, channels, spatial, groups, B = (1 << 24) - 1, 1, 8, 1, 4096
    assert qkr.group_norm_silu_workspace_size(n, channels, spatial, groups) == 0
    block, g, b = wl.gn_inputs(4949, B, channels, spatial, "bf16", "fp32")
    blk = block.to(DEV).view(B, -1)
    k = n // B
    x = torch.empty((n, channels, spatial), dtype=torch.bfloat16, device=DEV)
    flat = x.view(n, -1)
    flat[:k * B].view(k, B, -1).copy_(blk.unsqueeze(0).expand(k, -1, -1))
    flat[k * B:].copy_(blk[:n - k * B])
    y = qkr.group_norm_silu(x, g.to(DEV), b.to(DEV), groups)
    torch.cuda.synchronize()
    rng = np.random.default_rng(4950)
    samples = sorted({0, 1, B - 1, B, n // 2, n - 2, n - 1, *rng.integers(0, n, 20).tolist()})
    assert max(samples) < n
    got_all = _decode(y.view(n, -1)[torch.tensor(samples, device=DEV)], "bf16")
    m = 0.0
    for i, q in enumerate(samples):
        ref = oracle_groups(block, "bf16", channels, spatial, groups, g, b, wl.EPS,
                            q % B, q % B + 1)
        m = max(m, check_groups(got_all[i], ref, spatial, "bf16", "group %d" % q))
    print("maximum workgroups max_abs", m)


# (n, channels, spatial, groups, vectors per thread or 0 for one chunk per group, schedule)
GN_SWEEP = [
    (2, 64, 512, 32, 0, "one_read"),        # 1,024-element groups
    (4, 512, 16384, 32, 8, "two_pass"),     # channels of exactly one 16,384-element chunk
    (4, 512, 16392, 32, 8, "two_pass"),     # channel boundaries inside chunks (two-channel select)
    (64, 512, 1000, 8, 8, "two_pass"),      # channels shorter than a chunk (per-vector division)
    (2, 512, 16384, 32, 4, "two_pass"),     # 2,048 workgroups only with 8,192-element chunks
    (1, 512, 16384, 32, 2, "two_pass"),     # ... only with 4,096-element chunks
    (8, 512, 16384, 32, 8, "lagged"),       # 4,096 chunks: the lagged single read
    (8, 512, 16392, 32, 8, "lagged"),       # ... channel boundaries inside chunks
    (128, 512, 1000, 8, 8, "lagged"),       # ... channels shorter than a chunk
]


@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
@pytest.mark.parametrize("param", ["fp32", "bf16", "fp16"])
def test_every_kernel_instantiation(dtype, param):
    """Every compiled kernel of one (data, affine) dtype pair: the one-read
    kernel, the stats + apply pair at each chunk size and the lagged kernel,
    with channels longer and shorter than a chunk.  The chunk size is confirmed through the
    workspace size it implies; sampled groups against the oracle.  Samples
    repeat a block of at most 2 (the step is per group)."""
    for n, channels, spatial, groups, vpt, sched in GN_SWEEP:
        gsize = channels // groups * spatial
        chunk = 2048 * vpt
        want_ws = 0 if vpt == 0 else n * groups * -(-gsize // chunk) * 8
        assert qkr.group_norm_silu_workspace_size(n, channels, spatial, groups) == want_ws
        assert qkr.group_norm_silu_schedule(n, channels, spatial, groups) == (sched,
                                                                             chunk or 16384)
        nb = min(n, 2)
        block, g, b = wl.gn_inputs(7000 + spatial + n, nb, channels, spatial, dtype, param)
        blk = block.to(DEV)
        x = blk.repeat(n // nb, 1, 1)
        y = qkr.group_norm_silu(x, g.to(DEV), b.to(DEV), groups)
        torch.cuda.synchronize()
        flat = y.reshape(-1)
        got, ref = [], []
        for q in sorted({0, 1, n * groups // 2 + 1, n * groups - 1}):
            qb = q % (nb * groups)
            ref.append(oracle_groups(block, dtype, channels, spatial, groups, g, b, wl.EPS, qb,
                                     qb + 1))
            got.append(_decode(flat[q * gsize:(q + 1) * gsize], dtype))
        # per-group bounds; the RNE-agreement fraction over all sampled groups
        check_groups(np.concatenate(got), np.concatenate(ref), gsize, dtype,
                     "%s vpt %d" % ((n, channels, spatial, groups), vpt))


# ---------------------------------------------------------------- lagged schedule

LAGGED = (8, 512, 16384, 32)            # 256 groups of 16 chunks: 4,096 chunks


def _lagged_inputs(seed, dtype="bf16", param="fp32", shape=LAGGED):
    n, channels, spatial, groups = shape
    assert qkr.group_norm_silu_schedule(n, channels, spatial, groups)[0] == "lagged"
    x, g, b = wl.gn_inputs(seed, n, channels, spatial, dtype, param)
    return x, g, b


@pytest.mark.parametrize("spatial", [16384, 16392])
def test_lagged_and_two_pass_give_identical_bits(spatial):
    """The first 4 samples of an 8-sample call (lagged) equal a 4-sample call
    of the same samples (two passes) bit for bit: both combine the same chunk
    partials in the same order."""
    n, channels, groups = 8, 512, 32
    assert qkr.group_norm_silu_schedule(n, channels, spatial, groups)[0] == "lagged"
    assert qkr.group_norm_silu_schedule(4, channels, spatial, groups) == ("two_pass", 16384)
    x, g, b = wl.gn_inputs(8100 + spatial, n, channels, spatial, "bf16", "fp32")
    xd, gd, bd = x.to(DEV), g.to(DEV), b.to(DEV)
    lagged = qkr.group_norm_silu(xd, gd, bd, groups)
    two = qkr.group_norm_silu(xd[:4].contiguous(), gd, bd, groups)
    torch.cuda.synchronize()
    assert torch.equal(lagged[:4].view(torch.int16), two.view(torch.int16))


def test_lagged_in_place_and_any_workspace_contents():
    """In place equals out of place bit for bit, whatever the workspace held
    before the call (all ones is the unpublished mark itself, zeros would
    read as published statistics); sampled groups against the oracle."""
    n, channels, spatial, groups = LAGGED
    x, g, b = _lagged_inputs(8200)
    xd, gd, bd = x.to(DEV), g.to(DEV), b.to(DEV)
    need = qkr.group_norm_silu_workspace_size(n, channels, spatial, groups)
    ws = torch.empty(need, dtype=torch.uint8, device=DEV)
    outs = []
    for fill in (0x00, 0x7F, 0xFF):
        ws.fill_(fill)
        outs.append(qkr.group_norm_silu(xd, gd, bd, groups, workspace=ws))
    xi = xd.clone()
    ws.fill_(0x00)
    qkr.group_norm_silu(xi, gd, bd, groups, out=xi, workspace=ws)
    torch.cuda.synchronize()
    for o in outs[1:] + [xi]:
        assert torch.equal(o.view(torch.int16), outs[0].view(torch.int16))
    gsize = channels // groups * spatial
    flat = outs[0].view(-1)
    for q in (0, 1, 127, n * groups - 1):
        ref = oracle_groups(x, "bf16", channels, spatial, groups, g, b, wl.EPS, q, q + 1)
        check_groups(_decode(flat[q * gsize:(q + 1) * gsize], "bf16"), ref, gsize, "bf16",
                     "lagged group %d" % q)


@pytest.mark.parametrize("shape,dtype,param", [
    (LAGGED, "bf16", "fp32"),
    ((1, 128, 1024 * 1024, 32), "bf16", "fp32"),     # VAE out: 256 chunks per group
    ((8, 512, 16392, 32), "fp16", "bf16"),           # channel boundaries inside chunks
])
def test_lagged_waiters_that_reduce_chunks_themselves(shape, dtype, param):
    """With no polling allowed (the test entry point with 0 polls) every
    workgroup whose group is not complete at its first look reduces the
    missing chunks itself, racing their own workgroups; the first word
    published stands.  Out of place and in place, the bits equal the library
    call's."""
    n, channels, spatial, groups = shape
    x, g, b = _lagged_inputs(8300, dtype, param, shape=shape)
    xd, gd, bd = x.to(DEV), g.to(DEV), b.to(DEV)
    want = qkr.group_norm_silu(xd, gd, bd, groups)
    torch.cuda.synchronize()
    for _ in range(3):
        got = gn_hooks.group_norm_silu_polls(xd, gd, bd, groups, 0)
        xi = xd.clone()
        torch.cuda.synchronize()
        gn_hooks.group_norm_silu_polls(xi, gd, bd, groups, 0, out=xi)
        torch.cuda.synchronize()
        assert torch.equal(got.view(torch.int16), want.view(torch.int16))
        assert torch.equal(xi.view(torch.int16), want.view(torch.int16))


def test_lagged_graph_capture_replays_match_eager():
    """The clear kernel and the lagged kernel recorded into a graph: every
    replay, with the workspace overwritten and eager work between replays,
    equals the eager result."""
    n, channels, spatial, groups = LAGGED
    x, g, b = _lagged_inputs(8400)
    xd, gd, bd = x.to(DEV), g.to(DEV), b.to(DEV)
    eager = qkr.group_norm_silu(xd, gd, bd, groups)
    ws = torch.empty(qkr.group_norm_silu_workspace_size(n, channels, spatial, groups),
                     dtype=torch.uint8, device=DEV)
    out = torch.empty_like(xd)
    stream = torch.cuda.Stream()
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(stream):
        with torch.cuda.graph(graph, stream=stream):
            qkr.group_norm_silu(xd, gd, bd, groups, out=out, workspace=ws)
    torch.cuda.synchronize()
    for fill in (0x00, 0x7F, 0xFF):
        out.zero_()
        ws.fill_(fill)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), eager.view(torch.int16))


def test_lagged_calls_on_concurrent_streams():
    """Four lagged calls on four streams at once (own workspaces): each equals
    the same call run alone."""
    n, channels, spatial, groups = LAGGED
    cases = []
    for i in range(4):
        x, g, b = _lagged_inputs(8500 + i)
        xd, gd, bd = x.to(DEV), g.to(DEV), b.to(DEV)
        alone = qkr.group_norm_silu(xd, gd, bd, groups)
        torch.cuda.synchronize()
        cases.append((xd, gd, bd, alone, torch.cuda.Stream()))
    outs = []
    for xd, gd, bd, _, st in cases:
        with torch.cuda.stream(st):
            outs.append(qkr.group_norm_silu(xd, gd, bd, groups, stream=st))
    torch.cuda.synchronize()
    for (_, _, _, alone, _), out in zip(cases, outs):
        assert torch.equal(out.view(torch.int16), alone.view(torch.int16))



# ----------------------------------------------------------------------------- large and tiny finite values


def _groups_with_peaks(rng, n, channels, spatial, groups, peaks, chunk_peaks=None):
    """fp64 [n, channels, spatial]: each channel N(b_c, 1), each group rescaled
    so its largest |x| is one of `peaks` (cycling over the groups); with
    `chunk_peaks`, the group's elements are rescaled in runs of 16384 instead
    (chunks of different magnitude inside one group)."""
    raw = rng.standard_normal((n, channels, spatial)) + rng.standard_normal(channels)[None, :, None]
    flat = raw.reshape(n * groups, -1)
    flat /= np.abs(flat).max(axis=1, keepdims=True)
    peaks = np.asarray(peaks, dtype=np.float64)
    flat *= peaks[np.arange(n * groups) % len(peaks)][:, None]
    if chunk_peaks is not None:
        cp = np.asarray(chunk_peaks, dtype=np.float64)
        run_of = np.arange(flat.shape[1]) // 16384
        flat *= cp[run_of % len(cp)][None, :]
    return raw


def _gn_case(raw, dtype, param, seed):
    x = torch.from_numpy(raw.astype(np.float32)).to(wl.DTYPES[dtype])
    assert torch.isfinite(x.float()).all()
    rng = np.random.default_rng(seed)
    c = raw.shape[1]
    g = torch.from_numpy((1 + 0.1 * rng.standard_normal(c)).astype(np.float32))
    b = torch.from_numpy((0.1 * rng.standard_normal(c)).astype(np.float32))
    if param != "fp32":
        g, b = g.to(wl.DTYPES[param]), b.to(wl.DTYPES[param])
    return x, g, b


@pytest.mark.parametrize("shape,schedule", [
    ((2, 64, 64, 8), "one_read"),              # groups of 512: one chunk
    ((1, 64, 4096, 8), "two_pass"),            # 8 chunks of 4096 per group
    ((4, 96, 2048, 6), "two_pass"),            # 8 chunks of 4096 per group
    (LAGGED, "lagged"),                        # 16 chunks of 16384 per group
])
def test_large_finite_bf16_groups(shape, schedule):
    """bf16 groups whose fp32 chunk sums or squared deviations overflow
    (largest |x| 1e18, 1e30, 3e38) between O(1) groups, in each schedule;
    plus a constant group of 3e38 (zero variance) and a group of O(1) values
    with one element at 3.3e38.  Every group against the oracle."""
    n, channels, spatial, groups = shape
    assert qkr.group_norm_silu_schedule(n, channels, spatial, groups)[0] == schedule
    rng = np.random.default_rng(900 + spatial)
    raw = _groups_with_peaks(rng, n, channels, spatial, groups, [1.0, 1e18, 1e30, 3e38, 4.0])
    flat = raw.reshape(n * groups, -1)
    flat[1] = 3e38
    flat[2] = rng.standard_normal(flat.shape[1])
    flat[2, 77] = 3.3e38
    x, g, b = _gn_case(raw, "bf16", "fp32", 901)
    out = run(x, g, b, groups)
    gsize = channels // groups * spatial
    ref = oracle_groups(x, "bf16", channels, spatial, groups, g, b, wl.EPS)
    m = check_groups(_decode(out, "bf16"), ref, gsize, "bf16", "large groups %s" % (shape,))
    inplace = run(x, g, b, groups, inplace=True)
    assert torch.equal(inplace.view(torch.int16), out.view(torch.int16))
    print("large finite bf16 groups", shape, schedule, "max_abs", m)


@pytest.mark.parametrize("schedule_shape", [(1, 64, 4096, 2), LAGGED])
def test_groups_mixing_chunk_magnitudes(schedule_shape):
    """Groups whose chunks differ in magnitude (runs of 16384 elements at
    1, 1e30, 3e38 and 1e-3 of the group's peak): some chunk partials take the
    rescaled (mean, -sd) form and the group's combine goes rescaled too.
    Every group against the oracle; the lagged schedule's forced helpers give
    the same bits."""
    n, channels, spatial, groups = schedule_shape
    rng = np.random.default_rng(910)
    raw = _groups_with_peaks(rng, n, channels, spatial, groups, [1.0, 3e38],
                             chunk_peaks=[1.0, 1e-30, 1.0, 1e-8])
    x, g, b = _gn_case(raw, "bf16", "fp32", 911)
    out = run(x, g, b, groups)
    gsize = channels // groups * spatial
    ref = oracle_groups(x, "bf16", channels, spatial, groups, g, b, wl.EPS)
    m = check_groups(_decode(out, "bf16"), ref, gsize, "bf16", "mixed chunks")
    if qkr.group_norm_silu_schedule(n, channels, spatial, groups)[0] == "lagged":
        xd, gd, bd = x.to(DEV), g.to(DEV), b.to(DEV)
        helped = gn_hooks.group_norm_silu_polls(xd, gd, bd, groups, 0)
        torch.cuda.synchronize()
        assert torch.equal(helped.cpu().view(torch.int16), out.view(torch.int16))
    print("mixed chunk magnitudes", schedule_shape, "max_abs", m)


@pytest.mark.parametrize("eps", [1e-6, 1e-38, 1.4e-45])
@pytest.mark.parametrize("dtype,shape", [("bf16", (2, 64, 64, 8)), ("bf16", (1, 64, 4096, 8)),
                                         ("fp16", (1, 64, 4096, 8))])
def test_tiny_groups_and_tiny_eps(eps, dtype, shape):
    """Groups of tiny values (down to bf16 subnormals near 1e-40, fp16 ones
    near 1e-7) and an all-zero group, with eps down to the smallest fp32
    subnormal.  Every group against the oracle."""
    n, channels, spatial, groups = shape
    rng = np.random.default_rng(920)
    peaks = ([1.0, 1e-12, 1e-20, 1e-30, 1e-38, 1e-40] if dtype == "bf16"
             else [1.0, 1e-3, 1e-5, 3e-7])
    raw = _groups_with_peaks(rng, n, channels, spatial, groups, peaks)
    raw.reshape(n * groups, -1)[0] = 0.0
    x, g, b = _gn_case(raw, dtype, "fp32", 921)
    out = run(x, g, b, groups, eps=eps)
    gsize = channels // groups * spatial
    ref = oracle_groups(x, dtype, channels, spatial, groups, g, b, eps)
    m = check_groups(_decode(out, dtype), ref, gsize, dtype, "tiny groups eps %g" % eps)
    print("tiny groups", dtype, shape, "eps", eps, "max_abs", m)


@pytest.mark.parametrize("as_int", [False, True])
def test_binding_allocates_on_the_launch_stream(monkeypatch, as_int):
    """Called with a launch stream other than the current one (a torch
    stream, or its raw handle), the workspace and output the binding
    allocates belong to the launch stream: the caching allocator then reuses
    their memory only in that stream's order, never for work the current
    stream queues while the call may still run.  The launch stream is held
    back by a spin kernel, the current stream allocates and fills memory of
    the workspace's size right after the call, and the output still equals
    the same call on one stream."""
    n, channels, spatial, groups = LAGGED
    x, g, b = _lagged_inputs(8600)
    xd, gd, bd = x.to(DEV), g.to(DEV), b.to(DEV)
    want = qkr.group_norm_silu(xd, gd, bd, groups)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    seen = []
    real_empty, real_like = torch.empty, torch.empty_like

    def empty(*a, **kw):
        seen.append(torch.cuda.current_stream().cuda_stream)
        return real_empty(*a, **kw)

    def empty_like(*a, **kw):
        seen.append(torch.cuda.current_stream().cuda_stream)
        return real_like(*a, **kw)

    need = qkr.group_norm_silu_workspace_size(n, channels, spatial, groups)
    with torch.cuda.stream(side):
        torch.cuda._sleep(20_000_000)
    monkeypatch.setattr(torch, "empty", empty)
    monkeypatch.setattr(torch, "empty_like", empty_like)
    got = qkr.group_norm_silu(xd, gd, bd, groups, stream=side.cuda_stream if as_int else side)
    monkeypatch.undo()
    junk = [torch.full((need,), 0x7F, dtype=torch.uint8, device=DEV) for _ in range(4)]
    torch.cuda.synchronize()
    assert len(seen) == 2 and set(seen) == {side.cuda_stream}, seen
    assert torch.equal(got.view(torch.int16), want.view(torch.int16))
    del junk
