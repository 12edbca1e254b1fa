"""The group-norm entry point that allocates nothing, dit_group_norm_silu_noalloc,
through the C ABI on the GPU: its output equals dit_group_norm_silu's (given a
workspace) bit for bit, and the oracle's within the step's rounding model, on
two calls in a row on the same GPU (so on the same fixed scratch), the second
with a smaller input and another schedule.  A call beyond the scratch is
refused and writes nothing."""
import numpy as np
import pytest
import torch

import diffusion_transformer_qk_amd as qkr
import oracle
import workloads as wl
from diffusion_transformer_qk_amd import binding as b
from tests.gpu_common import decode as _decode

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")
FP32_NOISE = 8e-6


def _ulp_bf16(v):
    e = np.floor(np.log2(np.maximum(np.abs(v), 2.0 ** -126)))
    return 2.0 ** (e - 7)


def _with_workspace(x, y, g, bt, n, channels, spatial, groups, stream):
    need = qkr.group_norm_silu_workspace_size(n, channels, spatial, groups)
    ws = torch.empty(max(need, 16), dtype=torch.uint8, device=DEV)
    ws.fill_(0x5A)
    rc = qkr.dit_group_norm_silu_raw(x.data_ptr(), y.data_ptr(), n, channels, spatial, groups,
                                     g.data_ptr(), bt.data_ptr(), b.QKR_FP32, wl.EPS, b.QKR_BF16,
                                     ws.data_ptr(), ws.numel(), stream)
    torch.cuda.synchronize()
    assert rc == b.QKR_OK, qkr.strerror(rc)


def _noalloc(x, y, g, bt, n, channels, spatial, groups, stream):
    rc = qkr.dit_group_norm_silu_noalloc_raw(x.data_ptr(), y.data_ptr(), n, channels, spatial,
                                             groups, g.data_ptr(), bt.data_ptr(), b.QKR_FP32,
                                             wl.EPS, b.QKR_BF16, stream)
    return rc


# a larger call first (lagged single read, 64 KiB of scratch), then a smaller
# one (two passes, 512 B) over the scratch the first left behind
CASES = [((1, 128, 1024 * 1024, 32), "lagged", 65536),
         ((1, 64, 4096, 8), "two_pass", 512)]


def test_noalloc_matches_the_workspace_entry_point_on_two_calls():
    stream = torch.cuda.current_stream(DEV).cuda_stream
    for (n, channels, spatial, groups), sched, need in CASES:
        assert qkr.group_norm_silu_schedule(n, channels, spatial, groups)[0] == sched
        assert qkr.group_norm_silu_workspace_size(n, channels, spatial, groups) == need
        x_cpu, g_cpu, b_cpu = wl.gn_inputs(9700 + channels, n, channels, spatial, "bf16", "fp32")
        x, g, bt = x_cpu.to(DEV), g_cpu.to(DEV), b_cpu.to(DEV)
        want = torch.empty_like(x)
        _with_workspace(x, want, g, bt, n, channels, spatial, groups, stream)
        got = torch.full_like(x, 7.0)
        rc = _noalloc(x, got, g, bt, n, channels, spatial, groups, stream)
        torch.cuda.synchronize()
        assert rc == b.QKR_OK, qkr.strerror(rc)
        assert torch.equal(got.view(torch.int16), want.view(torch.int16)), sched
        # in place too
        xi = x.clone()
        rc = _noalloc(xi, xi, g, bt, n, channels, spatial, groups, stream)
        torch.cuda.synchronize()
        assert rc == b.QKR_OK
        assert torch.equal(xi.view(torch.int16), want.view(torch.int16)), sched + " in place"
        # the oracle on the first and last group
        gsize = channels // groups * spatial
        flat = got.view(-1)
        for q in (0, n * groups - 1):
            ref = oracle.group_norm_silu(wl.u16(x_cpu), "bf16", channels=channels,
                                         spatial=spatial, groups=groups, gamma=g_cpu.numpy(),
                                         beta=b_cpu.numpy(), param_dtype="fp32", eps=wl.EPS,
                                         group_begin=q, group_end=q + 1)
            dec = _decode(flat[q * gsize:(q + 1) * gsize], "bf16")
            bound = 0.5 * _ulp_bf16(ref) + FP32_NOISE * (1 + np.abs(ref).max())
            assert np.all(np.abs(dec - ref) <= bound), (sched, q)


def test_noalloc_refuses_a_call_beyond_its_scratch():
    """65 samples x 32 groups of 64 chunks need 1 MiB + 64 KiB of workspace:
    refused with QKR_ERR_SCRATCH, nothing written (the output keeps its
    fill).  A tiny y is enough: the call is refused before touching it."""
    n, channels, spatial, groups = 65, 512, 65536, 32
    assert qkr.group_norm_silu_workspace_size(n, channels, spatial, groups) > b.GN_NOALLOC_WORKSPACE_MAX
    x = torch.zeros(64, dtype=torch.bfloat16, device=DEV)
    y = torch.full((64,), 3.0, dtype=torch.bfloat16, device=DEV)
    g = torch.ones(channels, device=DEV)
    bt = torch.zeros(channels, device=DEV)
    # sizes are checked before the pointers are used; the fake extent of x
    # and y does not matter because nothing is launched
    rc = qkr.dit_group_norm_silu_noalloc_raw(x.data_ptr(), y.data_ptr() + (1 << 40), n, channels,
                                             spatial, groups, g.data_ptr(), bt.data_ptr(),
                                             b.QKR_FP32, wl.EPS, b.QKR_BF16, 0)
    torch.cuda.synchronize()
    assert rc == b.QKR_ERR_SCRATCH
    assert bool((y == 3.0).all())
