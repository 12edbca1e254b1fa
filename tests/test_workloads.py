"""The synthetic input recipe: sizes, positions, tables, determinism."""
import numpy as np
import pytest
import torch

import workloads as wl


def test_algorithmic_bytes_of_each_workload():
    b = wl.algorithmic_bytes
    assert b(256, 24, 64) == 3_276_800
    assert b(4096, 24, 128) == 104_857_600
    assert b(4096, 24, 128, cos_layout="per_head") == 201_326_592
    assert b(4608, 48, 128) == 231_211_008
    assert b(32760, 40, 128) == 1_375_395_840
    assert b(75600, 40, 128) == 3_173_990_400
    assert b(75600, 40, 128, cos_layout="per_head") == 6_193_152_000
    # the headline's shards over 8 GPUs: by tokens, and by heads (the shared
    # row then serves 10 Q+K heads instead of 80)
    assert b(4095, 40, 128) == 1_375_395_840 // 8
    assert b(32760, 5, 128) == 32760 * 10 * 128 * 4 + 32760 * 128 * 8


@pytest.mark.parametrize("key", sorted(wl.WORKLOADS))
def test_positions_cover_the_grid(key):
    w = wl.WORKLOADS[key]
    pos = wl.positions(w)
    assert pos.shape == (w.tokens, len(w.grid))
    assert 2 * sum(w.split) == w.head_dim
    if w.token_begin:
        # a token shard: its slice of the whole grid's sequence
        full = wl.grid_positions(w.grid, w.text_tokens)
        assert np.array_equal(pos, full[w.token_begin:w.token_begin + w.tokens])
        assert w.token_begin + w.tokens <= full.shape[0]
        return
    assert np.all(pos[: w.text_tokens] == 0)
    img = pos[w.text_tokens:]
    for a, n in enumerate(w.grid):
        assert img[:, a].min() == 0 and img[:, a].max() == n - 1
    # row-major: the last axis varies fastest
    if len(w.grid) > 1 and w.grid[-1] > 1:
        assert img[1, -1] == 1 and img[1, 0] == 0


@pytest.mark.parametrize("style", ["interleaved", "rotate_half"])
def test_tables_repeat_each_pair(style):
    pos = np.stack(np.meshgrid(np.arange(3), np.arange(4), np.arange(5), indexing="ij"), -1)
    pos = pos.reshape(-1, 3)
    c, s = (t.numpy() for t in wl.rope_tables(pos, (22, 21, 21), 128, style))
    if style == "interleaved":
        assert np.array_equal(c[:, 0::2], c[:, 1::2]) and np.array_equal(s[:, 0::2], s[:, 1::2])
        first = c[:, 0::2]
    else:
        assert np.array_equal(c[:, :64], c[:, 64:]) and np.array_equal(s[:, :64], s[:, 64:])
        first = c[:, :64]
    # pair 0 of each axis has frequency 1: cos(pos)
    for a, start in enumerate((0, 22, 43)):
        assert np.allclose(first[:, start], np.cos(pos[:, a]), atol=1e-7)
    assert np.all(np.abs(c.astype(np.float64) ** 2 + s.astype(np.float64) ** 2 - 1) < 2.4e-7)


def test_bf16_table_is_rounded_fp32_table():
    c32, _ = wl.rope_tables(np.arange(50), (32,), 64, "interleaved")
    c16, _ = wl.rope_tables(np.arange(50), (32,), 64, "interleaved", dtype="bf16")
    assert c16.dtype == torch.bfloat16 and torch.equal(c32.to(torch.bfloat16), c16)


def test_draws_are_deterministic_and_thread_independent(monkeypatch):
    a = wl.fused_qkv(1234, 1100, 2, 64, "bf16")
    monkeypatch.setattr(wl, "_threads", lambda: 1)
    b = wl.fused_qkv(1234, 1100, 2, 64, "bf16")
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))
    c = wl.fused_qkv(1235, 1100, 2, 64, "bf16")
    assert not torch.equal(a.view(torch.int16), c.view(torch.int16))


def test_scale_and_weight_distributions():
    s = wl.token_scales(1004, 100000)
    assert s.min() >= 0.1 * (1 - 1e-6) and s.max() <= 10 * (1 + 1e-6)
    assert abs(np.mean(np.log(s))) < 0.03
    qg, kg = wl.norm_weights(1004, 128)
    assert qg.dtype == torch.float32 and not torch.equal(qg, kg)
    assert abs(float(qg.mean()) - 1) < 0.05


def test_separate_dtypes_share_values():
    out = wl.separate_qk(77, 30, 3, 64, ("fp16", "bf16"))
    q16, _ = out["fp16"]
    qb, _ = out["bf16"]
    assert q16.shape == (30, 3, 64)
    assert torch.allclose(q16.float(), qb.float(), rtol=1e-2, atol=1e-3)


def test_expand_per_head():
    c, _ = wl.rope_tables(np.arange(7), (32,), 64, "interleaved")
    e = wl.expand_per_head(c, 5)
    assert e.shape == (7, 5, 64) and e.is_contiguous()
    assert torch.equal(e[:, 3], c)
