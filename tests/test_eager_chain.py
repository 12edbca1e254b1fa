"""The eager unfused chain that bench.py times beside the fused pass.

It is a comparison leg only ([FLUX PR] microbench against PyTorch eager
bf16).  These tests check that it computes the same function as the oracle,
so that the speedup compares like with like.  It rounds twice (after the
norm and after RoPE), so each output is within two half-ulps of the pair's
norm of the exact value:

    |eager - o| <= 2 * u * ||(o_a, o_b)||,   u = 2^-8 (bf16), 2^-11 (fp16)

(the norm's rounding moves each input of the 2x2 rotation by at most
u*|n|, the rotation keeps the pair norm, and the last rounding adds u*|o|),
plus fp32 noise and, for fp16, the subnormal quantum.
"""
import json
import types

import numpy as np
import pytest
import torch

import bench
import oracle
import workloads as wl

U = {"bf16": 2.0 ** -8, "fp16": 2.0 ** -11}


def pair_norm(o: np.ndarray, style: str) -> np.ndarray:
    """sqrt(o_a^2 + o_b^2) of each element's rotation pair, per element."""
    D = o.shape[-1]
    if style == "interleaved":
        p = o.reshape(o.shape[:-1] + (D // 2, 2))
        return np.repeat(np.sqrt(p[..., 0] ** 2 + p[..., 1] ** 2), 2, axis=-1)
    half = np.sqrt(o[..., :D // 2] ** 2 + o[..., D // 2:] ** 2)
    return np.concatenate([half, half], axis=-1)


def check_chain(got: torch.Tensor, ref: np.ndarray, dtype: str, style: str):
    g = got.float().cpu().numpy().astype(np.float64)
    bound = 2 * U[dtype] * pair_norm(ref, style) * (1 + 1e-4) + 2.0 ** -24
    err = np.abs(g - ref)
    assert np.all(err <= bound), "worst excess %.3g" % float((err - bound).max())
    return float(err.max())


def oracle_tensor(qkv_bits, dtype, H, D, gamma, cos, sin, style, col0):
    T = qkv_bits.shape[0]
    out = np.empty((T, H, D), dtype=np.float64)
    oracle.qknorm_rope(qkv_bits, dtype, row_stride=3 * H * D, col0=col0, heads=H, head_dim=D,
                       gamma=gamma, eps=wl.EPS, cos=cos, sin=sin, style=style, out=out)
    return out


@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
@pytest.mark.parametrize("style", ["interleaved", "rotate_half"])
def test_eager_chain_matches_the_oracle_on_cpu(oracle_lib, dtype, style):
    T, H, D = 150, 6, 128
    qkv = wl.fused_qkv(4401, T, H, D, dtype)
    qg, kg = wl.norm_weights(4401, D)
    tdt = wl.DTYPES[dtype]
    qg_t, kg_t = qg.to(tdt), kg.to(tdt)           # the norm module's weight, in the data dtype
    cos, sin = wl.rope_tables(np.arange(T) * 5, (D // 2,), D, style)
    before = qkv.clone()
    bits = wl.u16(qkv)
    for col0, g in ((0, qg_t), (H * D, kg_t)):
        x = qkv[:, col0:col0 + H * D].view(T, H, D)      # a strided view of the QKV buffer
        got = bench.eager_chain(x, g, cos, sin, wl.EPS, style)
        ref = oracle_tensor(bits, dtype, H, D, g.float().numpy(), cos.numpy(), sin.numpy(),
                            style, col0)
        check_chain(got, ref, dtype, style)
    assert torch.equal(qkv.view(torch.int16), before.view(torch.int16)), "input was modified"


def test_the_chain_bound_catches_a_wrong_rotation(oracle_lib):
    """A chain with the sine's sign flipped fails the same check."""
    T, H, D = 40, 3, 64
    qkv = wl.fused_qkv(4402, T, H, D, "bf16")
    qg, _ = wl.norm_weights(4402, D)
    g = qg.to(torch.bfloat16)
    cos, sin = wl.rope_tables(np.arange(T) * 9, (D // 2,), D, "interleaved")
    x = qkv[:, :H * D].view(T, H, D)
    ref = oracle_tensor(wl.u16(qkv), "bf16", H, D, g.float().numpy(), cos.numpy(), sin.numpy(),
                        "interleaved", 0)
    wrong = bench.eager_chain(x, g, cos, -sin, wl.EPS, "interleaved")
    with pytest.raises(AssertionError):
        check_chain(wrong, ref, "bf16", "interleaved")


@pytest.mark.gpu
@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
def test_eager_chain_on_the_gpu_matches_the_oracle(oracle_lib, dtype):
    """The FLUX workload's q and k, the shapes the comparison is timed on."""
    w = wl.WORKLOADS["flux"]
    T, H, D = w.tokens, w.heads, w.head_dim
    q_cpu, k_cpu = wl.separate_qk(w.seed, T, H, D, (dtype,))[dtype]
    qg, kg = wl.norm_weights(w.seed, D)
    tdt = wl.DTYPES[dtype]
    cos, sin = wl.workload_tables(w, "interleaved")
    dev = torch.device("cuda:0")
    for x_cpu, g in ((q_cpu, qg.to(tdt)), (k_cpu, kg.to(tdt))):
        got = bench.eager_chain(x_cpu.to(dev), g.to(dev), cos.to(dev), sin.to(dev), wl.EPS,
                                "interleaved")
        torch.cuda.synchronize()
        bits = wl.u16(x_cpu.reshape(T, H * D))
        out = np.empty((T, H, D), dtype=np.float64)
        oracle.qknorm_rope(bits, dtype, row_stride=H * D, col0=0, heads=H, head_dim=D,
                           gamma=g.float().numpy(), eps=wl.EPS, cos=cos.numpy(), sin=sin.numpy(),
                           style="interleaved", out=out)
        check_chain(got, out, dtype, "interleaved")


@pytest.mark.gpu
def test_eager_chain_bench_line(capsys):
    """The comparison leg runs end to end and reports the three FLUX shapes."""
    args = types.SimpleNamespace(workload="flux", style=None, dtype="bf16", steps=3, warmup=1)
    assert bench.bench_eager_chain(args) == 0
    line = json.loads(capsys.readouterr().out.strip().splitlines()[-1])
    assert [s["tokens"] for s in line["shapes"]] == [512, 4096, 4608]
    assert line["unit"] == "x" and line["value"] == line["shapes"][-1]["speedup"]
    for s in line["shapes"]:
        assert s["eager_us"] > 0 and s["fused_us"] > 0
