"""Seeded synthetic inputs for the fused DiT QK-norm + RoPE pass.

This module holds none of the pass's own arithmetic: it draws activations and
norm weights and builds RoPE cos/sin tables from token positions.  The HIP
path's tests and bench and the CPU oracle's tests all take their inputs from
here, so both sides see identical bits.

Shapes, distributions and position grids stand in for the activations of the
two models the source pages measure on (Wan A14B video, FLUX.2-dev images);
no model weights or datasets are involved.

Recipe (every workload):
  * root seed ``1000 + k`` for workload k = 1..5, split with
    ``numpy.random.SeedSequence.spawn`` into: per-token scale, activations
    (one child per block of ``ROWS_PER_BLOCK`` tokens, so the draw does not
    depend on the number of threads), q_gamma, k_gamma;
  * per-token scale ``s_t = exp(U[ln 0.1, ln 10])`` multiplies the whole
    activation row (Q, K and V alike) in fp32, then one RNE cast to bf16/fp16;
  * ``gamma = 1 + 0.1 N(0,1)`` in fp32, separately for Q and K;
  * cos/sin from integer positions: per axis a with n_a frequency pairs,
    ``freq_j = theta ** (-j / n_a)`` (j = 0..n_a-1), pair index axis-major,
    angle = pos * freq in fp64, cos/sin in fp64 rounded once to fp32; a bf16
    table is the RNE of that fp32 table.  Interleaved tables repeat each
    pair's value at dims (2i, 2i+1); rotate-half tables at (i, i + D/2).
"""
from __future__ import annotations

import math
import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field

import numpy as np
import torch

THETA = 10000.0
EPS = 1e-6
ROWS_PER_BLOCK = 512

DTYPES = {"bf16": torch.bfloat16, "fp16": torch.float16}


@dataclass(frozen=True)
class Workload:
    """One synthetic workload: tensor layout, sizes and RoPE position grid."""

    key: str
    seed: int
    layout: str              # "fused": one [T, 3*H*D] QKV buffer; "separate": q, k [T, H, D]
    tokens: int
    heads: int
    head_dim: int
    dtypes: tuple
    styles: tuple
    cos_layouts: tuple
    grid: tuple              # position grid (row-major), one entry per axis
    split: tuple             # frequency pairs per axis; sums to head_dim / 2
    text_tokens: int = 0     # leading tokens all at position 0 on every axis
    token_begin: int = 0     # first token of the grid's sequence this workload holds (a shard)
    note: str = field(default="", compare=False)


WORKLOADS = {
    "tiny": Workload(
        "tiny", 1001, "fused", 256, 24, 64, ("bf16",), ("interleaved",), ("shared",),
        (256,), (32,), note="1-D positions 0..255"),
    "mid": Workload(
        "mid", 1002, "fused", 4096, 24, 128, ("bf16",), ("rotate_half",),
        ("shared", "per_head"), (64, 64), (32, 32), note="2-D 64x64 grid"),
    "flux": Workload(
        "flux", 1003, "separate", 4608, 48, 128, ("fp16", "bf16"), ("interleaved",),
        ("shared",), (1, 64, 64), (22, 21, 21), text_tokens=512,
        note="512 text tokens at the origin, then a 64x64 image grid"),
    "headline": Workload(
        "headline", 1004, "fused", 32760, 40, 128, ("bf16",), ("interleaved",),
        ("shared",), (21, 30, 52), (22, 21, 21), note="Wan A14B 21x30x52 latent grid"),
    "large": Workload(
        "large", 1005, "fused", 75600, 40, 128, ("bf16",),
        ("interleaved", "rotate_half"), ("shared", "per_head"), (21, 45, 80), (22, 21, 21),
        note="21x45x80 latent grid"),
    # The headline's bytes with head_dim 256: 20 heads of 256 per tensor.
    "wide_heads": Workload(
        "wide_heads", 1008, "fused", 32760, 20, 256, ("bf16",), ("interleaved",),
        ("shared", "per_head"), (21, 30, 52), (43, 43, 42),
        note="Wan 21x30x52 grid, 20 heads of 256 (the headline's bytes at head_dim 256)"),
    # What one GPU of eight runs when the headline is sharded (the pass needs
    # no exchange): the last token shard, or one head shard of every token.
    "shard_tokens": Workload(
        "shard_tokens", 1006, "fused", 4095, 40, 128, ("bf16",), ("interleaved",),
        ("shared",), (21, 30, 52), (22, 21, 21), token_begin=7 * 4095,
        note="tokens 28665..32759 of the Wan 21x30x52 grid: the last of 8 token shards"),
    "shard_heads": Workload(
        "shard_heads", 1007, "fused", 32760, 5, 128, ("bf16",), ("interleaved",),
        ("shared",), (21, 30, 52), (22, 21, 21),
        note="Wan 21x30x52 grid, 5 of the 40 heads of Q, K and V: one of 8 head shards"),
}


def _threads() -> int:
    return max(1, min(16, os.cpu_count() or 1))


def grid_positions(grid: tuple, text_tokens: int = 0) -> np.ndarray:
    """Integer positions [text_tokens + prod(grid), len(grid)]: text tokens at
    the origin, then the grid row-major."""
    axes = [np.arange(n, dtype=np.int64) for n in grid]
    mesh = np.meshgrid(*axes, indexing="ij")
    grid_pos = np.stack([m.reshape(-1) for m in mesh], axis=1)
    text = np.zeros((text_tokens, len(grid)), dtype=np.int64)
    return np.concatenate([text, grid_pos], axis=0)


def positions(w: Workload) -> np.ndarray:
    """Integer positions [tokens, n_axes], row-major over ``w.grid``, from
    token ``w.token_begin`` of that sequence on."""
    pos = grid_positions(w.grid, w.text_tokens)[w.token_begin:w.token_begin + w.tokens]
    assert pos.shape[0] == w.tokens, (pos.shape, w.tokens)
    return pos


def rope_tables(pos: np.ndarray, split: tuple, head_dim: int, style: str,
                theta: float = THETA, dtype: str = "fp32"):
    """cos, sin tables [tokens, head_dim] as CPU torch tensors (fp32 or bf16)."""
    pos = np.asarray(pos, dtype=np.int64)
    if pos.ndim == 1:
        pos = pos[:, None]
    assert pos.shape[1] == len(split) and 2 * sum(split) == head_dim
    angles = []
    for a, n_a in enumerate(split):
        freq = theta ** (-np.arange(n_a, dtype=np.float64) / n_a)
        angles.append(pos[:, a:a + 1].astype(np.float64) * freq[None, :])
    ang = np.concatenate(angles, axis=1)                      # [T, D/2], fp64
    c_pair = np.cos(ang).astype(np.float32)
    s_pair = np.sin(ang).astype(np.float32)
    if style == "interleaved":
        cos = np.repeat(c_pair, 2, axis=1)
        sin = np.repeat(s_pair, 2, axis=1)
    elif style == "rotate_half":
        cos = np.concatenate([c_pair, c_pair], axis=1)
        sin = np.concatenate([s_pair, s_pair], axis=1)
    else:
        raise ValueError(style)
    cos_t = torch.from_numpy(np.ascontiguousarray(cos))
    sin_t = torch.from_numpy(np.ascontiguousarray(sin))
    if dtype == "bf16":
        cos_t, sin_t = cos_t.to(torch.bfloat16), sin_t.to(torch.bfloat16)
    elif dtype != "fp32":
        raise ValueError(dtype)
    return cos_t, sin_t


def expand_per_head(table: torch.Tensor, heads: int) -> torch.Tensor:
    """Materialise a shared [T, D] table as the per-head layout [T, heads, D]."""
    return table[:, None, :].expand(table.shape[0], heads, table.shape[1]).contiguous()


def _children(seed: int):
    root = np.random.SeedSequence(seed)
    return root.spawn(4)   # scale, activations, q_gamma, k_gamma


def token_scales(seed: int, tokens: int) -> np.ndarray:
    g = np.random.Generator(np.random.PCG64(_children(seed)[0]))
    return np.exp(g.uniform(math.log(0.1), math.log(10.0), size=tokens)).astype(np.float32)


def norm_weights(seed: int, head_dim: int):
    """(q_gamma, k_gamma), each fp32 [head_dim] = 1 + 0.1 N(0,1)."""
    kids = _children(seed)
    out = []
    for child in kids[2:4]:
        g = np.random.Generator(np.random.PCG64(child))
        gam = (1.0 + 0.1 * g.standard_normal(head_dim)).astype(np.float32)
        out.append(torch.from_numpy(gam))
    return tuple(out)


def _normal_rows(seed: int, tokens: int, width: int, scale: np.ndarray) -> np.ndarray:
    """fp32 [tokens, width] = N(0,1) * scale[t], drawn block by block."""
    out = np.empty((tokens, width), dtype=np.float32)
    n_blocks = -(-tokens // ROWS_PER_BLOCK) if tokens else 0
    blocks = _children(seed)[1].spawn(n_blocks) if n_blocks else []

    def work(b):
        lo = b * ROWS_PER_BLOCK
        hi = min(tokens, lo + ROWS_PER_BLOCK)
        g = np.random.Generator(np.random.PCG64(blocks[b]))
        g.standard_normal((hi - lo, width), dtype=np.float32, out=out[lo:hi])
        out[lo:hi] *= scale[lo:hi, None]

    with ThreadPoolExecutor(_threads()) as ex:
        list(ex.map(work, range(n_blocks)))
    return out


def _cast(a: np.ndarray, dtype: str) -> torch.Tensor:
    return torch.from_numpy(a).to(DTYPES[dtype])


def fused_qkv(seed: int, tokens: int, heads: int, head_dim: int, dtype: str) -> torch.Tensor:
    """Fused activation buffer [tokens, 3*heads*head_dim] (Q | K | V)."""
    s = token_scales(seed, tokens)
    return _cast(_normal_rows(seed, tokens, 3 * heads * head_dim, s), dtype)


def separate_qk(seed: int, tokens: int, heads: int, head_dim: int, dtypes=("bf16",)):
    """Per-tensor q and k [tokens, heads, head_dim] for each requested dtype.

    One fp32 draw [tokens, 2*heads*head_dim] (q then k per token) is cast to
    every dtype, so the fp16 and bf16 tensors hold the same underlying values.
    """
    s = token_scales(seed, tokens)
    raw = _normal_rows(seed, tokens, 2 * heads * head_dim, s)
    raw = raw.reshape(tokens, 2, heads, head_dim)
    out = {}
    for dt in dtypes:
        q = _cast(np.ascontiguousarray(raw[:, 0]), dt)
        k = _cast(np.ascontiguousarray(raw[:, 1]), dt)
        out[dt] = (q, k)
    return out


def workload_tables(w: Workload, style: str, dtype: str = "fp32"):
    return rope_tables(positions(w), w.split, w.head_dim, style, dtype=dtype)


def u16(t: torch.Tensor) -> np.ndarray:
    """The raw 16-bit pattern of a bf16/fp16 CPU tensor, as a numpy uint16 view."""
    return t.contiguous().view(torch.int16).numpy().view(np.uint16)


def algorithmic_bytes(tokens: int, heads: int, head_dim: int, n_tensors: int = 2,
                      x_bytes: int = 2, cos_layout: str = "shared", cos_bytes: int = 4) -> int:
    """Bytes the pass must move: Q/K read + written, cos and sin read once."""
    qk = tokens * n_tensors * heads * head_dim * x_bytes * 2
    rows = tokens * (heads if cos_layout == "per_head" else 1)
    return qk + rows * head_dim * cos_bytes * 2


# ----------------------------------------------------------------------------- AdaLN modulation
#
# Inputs for the fused layer norm + scale/shift (AdaLN) pass:
#   x[r, c]  = (N(0,1) + bias_c) * s_r, bias_c ~ N(0, 0.5) per channel, s_r the
#              per-token log-uniform[0.1, 10] scale, fp32 then one RNE cast;
#   scale, shift [batches, hidden] = 0.5 N(0,1) each, cast to their dtype.
# Seeds: SeedSequence(seed) spawned into token scale, activations (per block
# of rows), channel bias, scale, shift.


@dataclass(frozen=True)
class AdalnWorkload:
    key: str
    seed: int
    rows: int
    hidden: int
    batches: int
    dtypes: tuple
    note: str = field(default="", compare=False)

    @property
    def rows_per_batch(self) -> int:
        return self.rows // self.batches


ADALN_WORKLOADS = {
    "adaln_flux": AdalnWorkload("adaln_flux", 1101, 4608, 6144, 1, ("bf16", "fp16"),
                                note="FLUX.2-dev 1024x1024: 512 text + 4096 image tokens, hidden 48x128"),
    "adaln_wan": AdalnWorkload("adaln_wan", 1102, 32760, 5120, 1, ("bf16",),
                               note="Wan A14B 21x30x52 latent tokens, hidden 40x128"),
    "adaln_wan_cfg2": AdalnWorkload("adaln_wan_cfg2", 1103, 65520, 5120, 2, ("bf16",),
                                    note="two guidance branches of the Wan shape, one modulation row each"),
}


def _adaln_children(seed: int):
    return np.random.SeedSequence(seed).spawn(5)   # scale_t, activations, bias, scale, shift


def adaln_inputs(seed: int, rows: int, hidden: int, batches: int, dtype: str = "bf16",
                 mod_dtype: str = "fp32"):
    """(x [rows, hidden], scale [batches, hidden], shift [batches, hidden]) CPU tensors."""
    kids = _adaln_children(seed)
    g = np.random.Generator(np.random.PCG64(kids[0]))
    s = np.exp(g.uniform(math.log(0.1), math.log(10.0), size=rows)).astype(np.float32)
    gb = np.random.Generator(np.random.PCG64(kids[2]))
    bias = (0.5 * gb.standard_normal(hidden)).astype(np.float32)
    out = np.empty((rows, hidden), dtype=np.float32)
    n_blocks = -(-rows // ROWS_PER_BLOCK) if rows else 0
    blocks = kids[1].spawn(n_blocks) if n_blocks else []

    def work(b):
        lo = b * ROWS_PER_BLOCK
        hi = min(rows, lo + ROWS_PER_BLOCK)
        gg = np.random.Generator(np.random.PCG64(blocks[b]))
        gg.standard_normal((hi - lo, hidden), dtype=np.float32, out=out[lo:hi])
        out[lo:hi] += bias[None, :]
        out[lo:hi] *= s[lo:hi, None]

    with ThreadPoolExecutor(_threads()) as ex:
        list(ex.map(work, range(n_blocks)))
    x = _cast(out, dtype)
    mods = []
    for child in kids[3:5]:
        gm = np.random.Generator(np.random.PCG64(child))
        m = (0.5 * gm.standard_normal((batches, hidden))).astype(np.float32)
        t = torch.from_numpy(m)
        mods.append(t if mod_dtype == "fp32" else t.to(DTYPES[mod_dtype]))
    return x, mods[0], mods[1]


def adaln_bytes(rows: int, hidden: int, batches: int, x_bytes: int = 2, mod_bytes: int = 4) -> int:
    """Bytes the pass must move: x read, y written, scale and shift read once."""
    return rows * hidden * x_bytes * 2 + batches * hidden * mod_bytes * 2


# ----------------------------------------------------------------------------- group norm + SiLU
#
# Inputs for the VAE group norm + SiLU step: x [n, C, S] (S = H*W), each
# channel c = N(0,1) * a_c + b_c with a_c = exp(U[ln 0.2, ln 5]) and
# b_c = N(0, 1), fp32 then one RNE cast; gamma = 1 + 0.1 N(0,1),
# beta = 0.1 N(0,1) per channel.  Seeds: SeedSequence(seed) spawned into
# channel scale, channel offset, activations (per block of 2^20 elements),
# gamma, beta.


@dataclass(frozen=True)
class GroupNormWorkload:
    key: str
    seed: int
    n: int
    channels: int
    height: int
    width: int
    groups: int
    dtypes: tuple
    note: str = field(default="", compare=False)

    @property
    def spatial(self) -> int:
        return self.height * self.width


GN_WORKLOADS = {
    "gn_vae_mid": GroupNormWorkload("gn_vae_mid", 1201, 1, 512, 128, 128, 32, ("bf16",),
                                    note="VAE decoder mid block at 1/8 of 1024x1024"),
    "gn_vae_up": GroupNormWorkload("gn_vae_up", 1202, 1, 256, 512, 512, 32, ("bf16", "fp16"),
                                   note="VAE decoder up block at 1/2 resolution"),
    "gn_vae_out": GroupNormWorkload("gn_vae_out", 1203, 1, 128, 1024, 1024, 32, ("bf16",),
                                    note="VAE decoder last block at 1024x1024"),
}

GN_BLOCK = 1 << 20


def gn_inputs(seed: int, n: int, channels: int, spatial: int, dtype: str = "bf16",
              param_dtype: str = "fp32"):
    """(x [n, channels, spatial], gamma [channels], beta [channels]) CPU tensors."""
    kids = np.random.SeedSequence(seed).spawn(5)
    ga = np.random.Generator(np.random.PCG64(kids[0]))
    a = np.exp(ga.uniform(math.log(0.2), math.log(5.0), size=channels)).astype(np.float32)
    gb = np.random.Generator(np.random.PCG64(kids[1]))
    b = gb.standard_normal(channels).astype(np.float32)
    total = n * channels * spatial
    out = np.empty(total, dtype=np.float32)
    n_blocks = -(-total // GN_BLOCK) if total else 0
    blocks = kids[2].spawn(n_blocks) if n_blocks else []

    def work(k):
        lo, hi = k * GN_BLOCK, min(total, (k + 1) * GN_BLOCK)
        g = np.random.Generator(np.random.PCG64(blocks[k]))
        g.standard_normal(hi - lo, dtype=np.float32, out=out[lo:hi])

    with ThreadPoolExecutor(_threads()) as ex:
        list(ex.map(work, range(n_blocks)))
    v = out.reshape(n, channels, spatial)
    v *= a[None, :, None]
    v += b[None, :, None]
    x = _cast(v, dtype)
    params = []
    for child, base in ((kids[3], 1.0), (kids[4], 0.0)):
        g = np.random.Generator(np.random.PCG64(child))
        p = (base + 0.1 * g.standard_normal(channels)).astype(np.float32)
        t = torch.from_numpy(p)
        params.append(t if param_dtype == "fp32" else t.to(DTYPES[param_dtype]))
    return x, params[0], params[1]


def gn_bytes(n: int, channels: int, spatial: int, x_bytes: int = 2, param_bytes: int = 4) -> int:
    """Bytes the step must move: x read, y written, gamma and beta read once."""
    return n * channels * spatial * x_bytes * 2 + channels * param_bytes * 2
