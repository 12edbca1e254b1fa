"""GPU parity: the HIP path (through the C ABI) against the fp64 CPU oracle.

Bar: max |gpu - oracle| <= 1.6e-2 for bf16 outputs and <= 2e-3 for fp16,
comparing the decoded GPU output with the UNROUNDED fp64 oracle; on top of
that the GPU output must equal the oracle's round-to-nearest-even image on all
but a tiny fraction of elements (those where fp32 rounding sits at a rounding
midpoint), and never by more than one unit in the last place.  Shared and
per-head cos/sin layouts must agree bit for bit, V and every read-only input
must stay bit-identical, and nothing outside the tensors may be written.
"""
import numpy as np
import pytest
import torch

import diffusion_transformer_qk_amd as qkr
import oracle
import workloads as wl
from tests.gpu_common import decode as _decode, ulp as _ulp

pytestmark = pytest.mark.gpu

TOL = {"bf16": 1.6e-2, "fp16": 2e-3}
MISMATCH_FRAC = {"bf16": 1e-3, "fp16": 2e-3}
DEV = torch.device("cuda:0")
PAD = 4096          # canary elements on each side of a tensor
CANARY = 0x7E5A
FP32_NOISE = 8e-6   # fp32 math error, relative to the largest |o| of the head


def rounding_bound(ref: np.ndarray, dtype: str) -> np.ndarray:
    """Per-element error model: round to nearest (half an ulp of the exact
    value) plus fp32 arithmetic noise.  The noise term scales with the head's
    largest |o| because the two products of a rotated pair can cancel, leaving
    a tiny output with an absolute fp32 error of the terms' size."""
    scale = np.max(np.abs(ref), axis=-1, keepdims=True)
    return 0.5 * _ulp(ref, dtype) + FP32_NOISE * scale


def check_close(got: np.ndarray, ref: np.ndarray, dtype: str, what: str = "") -> float:
    """Assert the tolerance, the rounding model and the RNE agreement; return max_abs."""
    got = got.reshape(ref.shape)
    err = np.abs(got - ref)
    max_abs = float(err.max()) if err.size else 0.0
    assert max_abs <= TOL[dtype], "%s max_abs %.4g > %g (max|o| %.3g)" % (
        what, max_abs, TOL[dtype], np.abs(ref).max())
    over = err > rounding_bound(ref, dtype)
    assert not over.any(), "%s: %d elements outside the rounding model, worst %.3g" % (
        what, int(over.sum()), float((err - rounding_bound(ref, dtype)).max()))
    rne = oracle.round_to(ref, dtype)
    n_diff = int(np.count_nonzero(got != rne))
    assert n_diff <= max(2, MISMATCH_FRAC[dtype] * got.size), "%s: %d of %d differ from RNE" % (
        what, n_diff, got.size)
    return max_abs


def check_rounding_bound(got: np.ndarray, ref: np.ndarray, dtype: str, what=""):
    """For inputs whose outputs may exceed |o| = 8 (beyond the fixed tolerance)."""
    got = got.reshape(ref.shape)
    assert np.all(np.abs(got - ref) <= rounding_bound(ref, dtype)), what


def guarded(t_cpu: torch.Tensor):
    """Device copy of t inside a canary-filled buffer: (view, whole buffer)."""
    n = t_cpu.numel()
    buf = torch.full((n + 2 * PAD,), CANARY, dtype=torch.int16, device=DEV)
    view = buf[PAD:PAD + n].view(t_cpu.dtype).view(t_cpu.shape)
    view.copy_(t_cpu.to(DEV))
    return view, buf


def canaries_intact(buf: torch.Tensor) -> bool:
    return bool((buf[:PAD] == CANARY).all()) and bool((buf[-PAD:] == CANARY).all())


def dev(t):
    return t.to(DEV)


def tables(pos, split, d, style, dtype="fp32"):
    return wl.rope_tables(pos, split, d, style, dtype=dtype)


def table_np(t: torch.Tensor):
    return t.numpy() if t.dtype == torch.float32 else wl.u16(t)


def cos_dtype_name(t: torch.Tensor) -> str:
    return "fp32" if t.dtype == torch.float32 else "bf16"


def run_fused(qkv_cpu, qg, kg, cos, sin, style, layout="shared", eps=wl.EPS, stream=None):
    """Run the pass on a guarded device copy; check canaries; return CPU output."""
    x, buf = guarded(qkv_cpu)
    g = (dev(qg), dev(kg))
    c, s = dev(cos), dev(sin)
    keep = [t.clone() for t in (*g, c, s)]
    qkr.qknorm_rope_fused(x, q_gamma=g[0], k_gamma=g[1], cos=c, sin=s, eps=eps, style=style,
                          cos_layout=layout, stream=stream)
    torch.cuda.synchronize()
    assert canaries_intact(buf), "write outside the QKV buffer"
    for a, b in zip(keep, (*g, c, s)):
        assert torch.equal(a, b), "a read-only input changed"
    return x.cpu()


def oracle_fused(qkv_cpu, x_dtype, H, D, qg, kg, cos, sin, style, layout="shared",
                 t_begin=0, t_end=None):
    return oracle.fused_qk(wl.u16(qkv_cpu), x_dtype, heads=H, head_dim=D, q_gamma=qg.numpy(),
                           k_gamma=kg.numpy(), eps=wl.EPS, cos=table_np(cos), sin=table_np(sin),
                           cos_dtype=cos_dtype_name(cos), cos_layout=layout, style=style,
                           t_begin=t_begin, t_end=t_end)


def assert_v_untouched(out, inp, H, D):
    a = out.view(torch.int16).reshape(out.shape[0], -1)[:, 2 * H * D:]
    b = inp.view(torch.int16).reshape(inp.shape[0], -1)[:, 2 * H * D:]
    assert torch.equal(a, b), "V slice changed"


def figures(pairs, dtype):
    """(largest |o|, fraction of elements that differ from the oracle's
    round-to-nearest-even image) over (got, ref) pairs."""
    o = max(float(np.abs(r).max()) for _, r in pairs)
    diff = sum(int(np.count_nonzero(g.reshape(r.shape) != oracle.round_to(r, dtype)))
               for g, r in pairs)
    return o, diff / sum(r.size for _, r in pairs)


def compare_fused(out, qkv_cpu, x_dtype, H, D, qg, kg, cos, sin, style, layout="shared",
                  what=""):
    T = qkv_cpu.shape[0]
    q_ref, k_ref = oracle_fused(qkv_cpu, x_dtype, H, D, qg, kg, cos, sin, style, layout)
    got = _decode(out, x_dtype).reshape(T, 3, H, D)
    m1 = check_close(got[:, 0], q_ref, x_dtype, what + " Q")
    m2 = check_close(got[:, 1], k_ref, x_dtype, what + " K")
    assert_v_untouched(out, qkv_cpu, H, D)
    o, frac = figures([(got[:, 0], q_ref), (got[:, 1], k_ref)], x_dtype)
    print("%s: max_abs %.4g max|o| %.3g RNE-disagreement %.2e" % (what, max(m1, m2), o, frac))
    return max(m1, m2)


# ----------------------------------------------------------------------------- kernel resources


@pytest.mark.parametrize("head_dim", [64, 128, 256])
@pytest.mark.parametrize("layout", ["shared", "per_head"])
def test_kernels_do_not_spill(head_dim, layout):
    """Every instantiation (all unroll depths and block orders) has no scratch."""
    seen = set()
    for style in ("interleaved", "rotate_half"):
        for cd in (qkr.binding.QKR_FP32, qkr.binding.QKR_BF16):
            for xd in (qkr.binding.QKR_BF16, qkr.binding.QKR_FP16):
                for heads in (1, 10, 19, 24, 40, 48, 72, 100):
                    for tokens in (64, 100000):
                        info = qkr.kernel_info(head_dim, layout, cd, style, xd, heads=heads,
                                               tokens=tokens)
                        assert info["scratch_bytes"] == 0, info
                        # the per-head layout also holds each head's table rows:
                        # up to 10 heads' worth in flight, 2 waves per SIMD
                        limit = 256 if layout == "per_head" else 128
                        assert 0 < info["num_vgprs"] <= limit, info
                        seen.add((info["heads_in_flight"], info["die_runs"]))
    depths = (3, 6, 10) if layout == "per_head" else (3, 6, 10, 12)
    assert {(u, o) for u in depths for o in (0, 1)} <= seen, seen


def test_kernel_info_follows_the_tensors_passed():
    """The schedule kernel_info reports for each way of passing the tensors:
    two tokens per workgroup for fused QKV or a q, k pair, four for a single
    tensor; per-die token runs for one streamed buffer only; the residency
    cap for long grids of the shared layout with >= 6 KB in flight per wave."""
    args = (128, "shared", qkr.binding.QKR_FP32, "interleaved", qkr.binding.QKR_BF16)
    fused = qkr.kernel_info(*args, heads=40, tokens=100000, tensors="fused")
    pair = qkr.kernel_info(*args, heads=40, tokens=100000, tensors="pair")
    one = qkr.kernel_info(*args, heads=40, tokens=100000, tensors="one")
    assert (fused["tokens_per_block"], fused["die_runs"]) == (2, 1)
    assert (pair["tokens_per_block"], pair["die_runs"]) == (2, 0)
    assert (one["tokens_per_block"], one["die_runs"]) == (4, 1)
    assert fused["heads_in_flight"] == pair["heads_in_flight"] == one["heads_in_flight"] == 10
    small = qkr.kernel_info(*args, heads=40, tokens=1000, tensors="one")
    assert small["die_runs"] == 0
    # residency cap: long grids whose waves keep >= 6 KB of loads in flight
    for info in (fused, pair, one):
        assert (info["workgroups_per_cu"], info["dynamic_lds_bytes"]) == (2, 56 * 1024), info
    assert small["workgroups_per_cu"] == small["dynamic_lds_bytes"] == 0
    few_heads = qkr.kernel_info(*args, heads=5, tokens=100000, tensors="fused")
    assert few_heads["workgroups_per_cu"] == 0
    per_head = qkr.kernel_info(128, "per_head", qkr.binding.QKR_FP32, "interleaved",
                               qkr.binding.QKR_BF16, heads=40, tokens=100000, tensors="fused")
    assert per_head["workgroups_per_cu"] == 0
    assert qkr.kernel_info(*args, heads=24, tokens=8192, tensors="fused")["workgroups_per_cu"] == 2
    assert qkr.kernel_info(*args, heads=24, tokens=8190, tensors="fused")["workgroups_per_cu"] == 0


# ----------------------------------------------------------------------------- the five workloads


def test_tiny_workload():
    w = wl.WORKLOADS["tiny"]
    T, H, D = w.tokens, w.heads, w.head_dim
    qkv = wl.fused_qkv(w.seed, T, H, D, "bf16")
    qg, kg = wl.norm_weights(w.seed, D)
    cos, sin = wl.workload_tables(w, "interleaved")
    out = run_fused(qkv, qg, kg, cos, sin, "interleaved")
    m = compare_fused(out, qkv, "bf16", H, D, qg, kg, cos, sin, "interleaved", what="tiny")
    print("tiny max_abs", m)


def test_mid_workload_and_layout_parity():
    w = wl.WORKLOADS["mid"]
    T, H, D = w.tokens, w.heads, w.head_dim
    qkv = wl.fused_qkv(w.seed, T, H, D, "bf16")
    qg, kg = wl.norm_weights(w.seed, D)
    cos, sin = wl.workload_tables(w, "rotate_half")
    shared = run_fused(qkv, qg, kg, cos, sin, "rotate_half")
    m = compare_fused(shared, qkv, "bf16", H, D, qg, kg, cos, sin, "rotate_half", what="mid")
    print("mid max_abs", m)
    per_head = run_fused(qkv, qg, kg, wl.expand_per_head(cos, H), wl.expand_per_head(sin, H),
                         "rotate_half", layout="per_head")
    assert torch.equal(shared.view(torch.int16), per_head.view(torch.int16))


@pytest.mark.parametrize("x_dtype", ["fp16", "bf16"])
def test_flux_workload_separate_q_k(x_dtype):
    w = wl.WORKLOADS["flux"]
    T, H, D = w.tokens, w.heads, w.head_dim
    q, k = wl.separate_qk(w.seed, T, H, D, (x_dtype,))[x_dtype]
    qg, kg = wl.norm_weights(w.seed, D)
    cos, sin = wl.workload_tables(w, "interleaved")
    qd, qbuf = guarded(q)
    kd, kbuf = guarded(k)
    qkr.qknorm_rope_fused(q=qd, k=kd, q_gamma=dev(qg), k_gamma=dev(kg), cos=dev(cos),
                          sin=dev(sin), eps=wl.EPS, style="interleaved")
    torch.cuda.synchronize()
    assert canaries_intact(qbuf) and canaries_intact(kbuf)
    kw = dict(row_stride=H * D, col0=0, heads=H, head_dim=D, eps=wl.EPS, cos=cos.numpy(),
              sin=sin.numpy(), style="interleaved")
    q_ref = oracle.qknorm_rope(wl.u16(q), x_dtype, gamma=qg.numpy(), **kw)
    k_ref = oracle.qknorm_rope(wl.u16(k), x_dtype, gamma=kg.numpy(), **kw)
    mq = check_close(_decode(qd, x_dtype), q_ref, x_dtype, "flux q")
    mk = check_close(_decode(kd, x_dtype), k_ref, x_dtype, "flux k")
    o, frac = figures([(_decode(qd, x_dtype), q_ref), (_decode(kd, x_dtype), k_ref)], x_dtype)
    print("flux %s: max_abs %.4g max|o| %.3g RNE-disagreement %.2e" % (x_dtype, max(mq, mk), o,
                                                                     frac))
    # text tokens sit at position 0: their output is the norm alone
    print("flux", x_dtype, "max_abs", mq, mk)


@pytest.mark.parametrize("key", ["shard_tokens", "shard_heads"])
def test_headline_shards(key):
    """One GPU's share of the headline over 8 GPUs, in full against the oracle:
    the last token shard (tokens 28665..32759 with their own positions) and a
    5-head shard of all 32760 tokens; V untouched."""
    w = wl.WORKLOADS[key]
    T, H, D = w.tokens, w.heads, w.head_dim
    qkv = wl.fused_qkv(w.seed, T, H, D, "bf16")
    qg, kg = wl.norm_weights(w.seed, D)
    cos, sin = wl.workload_tables(w, "interleaved")
    out = run_fused(qkv, qg, kg, cos, sin, "interleaved")
    m = compare_fused(out, qkv, "bf16", H, D, qg, kg, cos, sin, "interleaved", what=key)
    print(key, "max_abs", m)


FULL_CHUNK = 2048    # tokens per oracle call when a whole large output is compared


def check_every_token(out, qkv, H, D, qg, kg, cos, sin, style, what, x_dtype="bf16",
                      layout="shared"):
    """Every Q and K element of a fused output against the oracle, in chunks
    of FULL_CHUNK tokens (four at a time on threads: the oracle call and
    numpy's array work release the interpreter lock).  Returns the largest
    |error|, the largest |o| and the fraction of elements that differ from
    the oracle's round-to-nearest-even image."""
    from concurrent.futures import ThreadPoolExecutor

    T = qkv.shape[0]
    got_all = out.view(T, 3, H, D)

    def one(a):
        b = min(T, a + FULL_CHUNK)
        q_ref, k_ref = oracle_fused(qkv, x_dtype, H, D, qg, kg, cos, sin, style, layout=layout,
                                    t_begin=a, t_end=b)
        got = _decode(got_all[a:b].contiguous(), x_dtype).reshape(b - a, 3, H, D)
        m = max(check_close(got[:, 0], q_ref, x_dtype, "%s Q[%d:%d]" % (what, a, b)),
                check_close(got[:, 1], k_ref, x_dtype, "%s K[%d:%d]" % (what, a, b)))
        o = max(float(np.abs(q_ref).max()), float(np.abs(k_ref).max()))
        diff = int(np.count_nonzero(got[:, 0] != oracle.round_to(q_ref, x_dtype)) +
                   np.count_nonzero(got[:, 1] != oracle.round_to(k_ref, x_dtype)))
        return m, o, diff

    with ThreadPoolExecutor(4) as ex:
        res = list(ex.map(one, range(0, T, FULL_CHUNK)))
    n = T * 2 * H * D
    return (max(r[0] for r in res), max(r[1] for r in res), sum(r[2] for r in res) / n)


def _sample_windows(T, rng, n=12, width=48):
    starts = sorted(set(rng.integers(0, T - width, n).tolist()))
    wins = [(0, width)] + [(s, s + width) for s in starts] + [(T - width - 3, T)]
    return wins


def _check_sampled(out, qkv, H, D, qg, kg, cos, sin, style, seed, what, x_dtype="bf16"):
    T = qkv.shape[0]
    rng = np.random.default_rng(seed)
    got_all = out.view(T, 3, H, D)
    worst = 0.0
    for a, b in _sample_windows(T, rng):
        q_ref, k_ref = oracle_fused(qkv, x_dtype, H, D, qg, kg, cos, sin, style, t_begin=a,
                                    t_end=b)
        got = _decode(got_all[a:b].contiguous(), x_dtype).reshape(b - a, 3, H, D)
        worst = max(worst, check_close(got[:, 0], q_ref, x_dtype, "%s Q[%d:%d]" % (what, a, b)),
                    check_close(got[:, 1], k_ref, x_dtype, "%s K[%d:%d]" % (what, a, b)))
    return worst


def test_headline_workload_every_token():
    """32760 x 3*40*128 bf16, the launch the bench times: every Q and K
    element of all 32760 tokens against the oracle, V bit-unchanged."""
    w = wl.WORKLOADS["headline"]
    T, H, D = w.tokens, w.heads, w.head_dim
    qkv = wl.fused_qkv(w.seed, T, H, D, "bf16")
    qg, kg = wl.norm_weights(w.seed, D)
    cos, sin = wl.workload_tables(w, "interleaved")
    out = run_fused(qkv, qg, kg, cos, sin, "interleaved")
    assert_v_untouched(out, qkv, H, D)
    m, o, frac = check_every_token(out, qkv, H, D, qg, kg, cos, sin, "interleaved", "headline")
    print("headline every token: max_abs %.4g max|o| %.3g RNE-disagreement %.2e" % (m, o, frac))


@pytest.mark.parametrize("layout", ["shared", "per_head"])
def test_repeated_calls_are_bit_identical(layout):
    """The headline launch run five times on fresh copies of one input gives
    the same bits every time: the cos/sin staging barrier and the
    per-die block order leave no run-to-run variation."""
    w = wl.WORKLOADS["headline"]
    T, H, D = w.tokens, w.heads, w.head_dim
    src = wl.fused_qkv(w.seed, T, H, D, "bf16").to(DEV)
    qg, kg = wl.norm_weights(w.seed, D)
    cos, sin = wl.workload_tables(w, "interleaved")
    c, s = dev(cos), dev(sin)
    if layout == "per_head":
        c, s = wl.expand_per_head(c, H), wl.expand_per_head(s, H)
    first = None
    for _ in range(5):
        x = src.clone()
        qkr.qknorm_rope_fused(x, q_gamma=dev(qg), k_gamma=dev(kg), cos=c, sin=s,
                              style="interleaved", cos_layout=layout)
        torch.cuda.synchronize()
        if first is None:
            first = x
        else:
            assert torch.equal(x.view(torch.int16), first.view(torch.int16))


@pytest.mark.parametrize("x_dtype,style,table", [("fp16", "interleaved", "fp32"),
                                                 ("bf16", "rotate_half", "bf16"),
                                                 ("fp16", "rotate_half", "bf16")])
def test_headline_shape_other_dtypes_and_styles(x_dtype, style, table):
    """The headline shape and launch configuration with fp16 data, rotate-half
    and bf16 cos/sin tables: every token against the oracle, V untouched."""
    w = wl.WORKLOADS["headline"]
    T, H, D = w.tokens, w.heads, w.head_dim
    qkv = wl.fused_qkv(w.seed + 7, T, H, D, x_dtype)
    qg, kg = wl.norm_weights(w.seed, D)
    cos, sin = wl.workload_tables(w, style, dtype=table)
    out = run_fused(qkv, qg, kg, cos, sin, style)
    assert_v_untouched(out, qkv, H, D)
    m, o, frac = check_every_token(out, qkv, H, D, qg, kg, cos, sin, style,
                                   "headline " + x_dtype, x_dtype=x_dtype)
    print("headline every token", x_dtype, style, table,
          "max_abs %.4g max|o| %.3g RNE-disagreement %.2e" % (m, o, frac))


@pytest.mark.slow
@pytest.mark.parametrize("style", ["interleaved", "rotate_half"])
def test_large_workload_every_token_and_layout_parity(style):
    """75600 x 3*40*128 bf16 in both styles: the shared row and the per-head
    control give the same bits, and every token of the output matches the
    oracle; V untouched."""
    w = wl.WORKLOADS["large"]
    T, H, D = w.tokens, w.heads, w.head_dim
    qkv = wl.fused_qkv(w.seed, T, H, D, "bf16")
    qg, kg = wl.norm_weights(w.seed, D)
    cos, sin = wl.workload_tables(w, style)
    x_in = dev(qkv)
    g = (dev(qg), dev(kg))
    c, s = dev(cos), dev(sin)
    a = x_in.clone()
    qkr.qknorm_rope_fused(a, q_gamma=g[0], k_gamma=g[1], cos=c, sin=s, style=style)
    cph, sph = wl.expand_per_head(c, H), wl.expand_per_head(s, H)
    b = x_in.clone()
    qkr.qknorm_rope_fused(b, q_gamma=g[0], k_gamma=g[1], cos=cph, sin=sph, style=style,
                          cos_layout="per_head")
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16)), "layouts differ"
    del b, cph, sph
    out = a.cpu()
    assert_v_untouched(out, qkv, H, D)
    m, o, frac = check_every_token(out, qkv, H, D, qg, kg, cos, sin, style, "large " + style)
    print("large every token", style, "max_abs %.4g max|o| %.3g RNE-disagreement %.2e"
          % (m, o, frac))


def test_byte_offsets_beyond_4gib():
    """[140000, 3*40*128] bf16 = 4.3 GB, in the headline's launch configuration:
    tokens on both sides of the 2^32-byte offset (token 139810 straddles it)
    against the oracle, and V untouched everywhere.  The activations repeat a
    2048-token block (the pass is per token, so each sampled token is a full
    case); cos/sin come from a 28 x 50 x 100 position grid."""
    T, H, D, B = 140000, 40, 128, 2048
    block = wl.fused_qkv(4242, B, H, D, "bf16")
    qg, kg = wl.norm_weights(4242, D)
    cos, sin = wl.rope_tables(wl.grid_positions((28, 50, 100)), (22, 21, 21), D, "interleaved")
    blk = block.to(DEV)
    x = torch.empty((T, 3 * H * D), dtype=torch.bfloat16, device=DEV)
    for i in range(0, T, B):
        x[i:i + B].copy_(blk[:min(B, T - i)])
    qkr.qknorm_rope_fused(x, q_gamma=dev(qg), k_gamma=dev(kg), cos=dev(cos), sin=dev(sin),
                          style="interleaved")
    torch.cuda.synchronize()
    info = qkr.kernel_info(D, "shared", qkr.binding.QKR_FP32, "interleaved",
                           qkr.binding.QKR_BF16, heads=H, tokens=T)
    assert info["die_runs"] == 1 and info["heads_in_flight"] == 10
    for i in range(0, T, B):
        n = min(B, T - i)
        assert torch.equal(x[i:i + n, 2 * H * D:], blk[:n, 2 * H * D:]), "V changed"
    samples = [0, 1, B - 1, B, 69905, 139809, 139810, 139811, T - 2, T - 1]
    assert max(samples) < T
    idx = torch.tensor(samples)
    rows = block[idx % B]
    q_ref, k_ref = oracle_fused(rows, "bf16", H, D, qg, kg, cos[idx], sin[idx], "interleaved")
    got = _decode(x[idx.to(DEV)], "bf16").reshape(len(samples), 3, H, D)
    m = max(check_close(got[:, 0], q_ref, "bf16", ">4GiB Q"),
            check_close(got[:, 1], k_ref, "bf16", ">4GiB K"))
    print("beyond 4 GiB max_abs", m)


@pytest.mark.parametrize("heads,head_dim", [(3, 128), (24, 128), (48, 128), (72, 64), (100, 64),
                                            (30, 256)])
def test_die_order_every_unroll(heads, head_dim):
    """8200 tokens = 4100 workgroups: the per-die token runs (with a ragged
    4100 % 8 remainder) for head counts that select each unroll depth."""
    T = 8200
    qkv = wl.fused_qkv(3000 + heads, T, heads, head_dim, "bf16")
    qg, kg = wl.norm_weights(3000 + heads, head_dim)
    cos, sin = tables(np.arange(T), (head_dim // 2,), head_dim, "rotate_half")
    info = qkr.kernel_info(head_dim, "shared", qkr.binding.QKR_FP32, "rotate_half",
                           qkr.binding.QKR_BF16, heads=heads, tokens=T)
    assert info["die_runs"] == 1
    out = run_fused(qkv, qg, kg, cos, sin, "rotate_half")
    assert_v_untouched(out, qkv, heads, head_dim)
    m = _check_sampled(out, qkv, heads, head_dim, qg, kg, cos, sin, "rotate_half", heads,
                       "die order U%d" % info["heads_in_flight"])
    print("die order heads", heads, "U", info["heads_in_flight"], "max_abs", m)


# ----------------------------------------------------------------------------- exact layout parity


@pytest.mark.parametrize("style", ["interleaved", "rotate_half"])
@pytest.mark.parametrize("heads,head_dim", [(24, 64), (24, 128), (40, 128), (16, 256)])
def test_shared_row_matches_expanded_bitwise(style, heads, head_dim):
    """Shared fp32 row vs the same row materialised per head: rtol = atol = 0."""
    T = 256
    qkv = wl.fused_qkv(2000 + heads + head_dim, T, heads, head_dim, "bf16")
    qg, kg = wl.norm_weights(2000 + heads, head_dim)
    cos, sin = tables(np.arange(T) * 5, (head_dim // 2,), head_dim, style)
    a = run_fused(qkv, qg, kg, cos, sin, style)
    b = run_fused(qkv, qg, kg, wl.expand_per_head(cos, heads), wl.expand_per_head(sin, heads),
                  style, layout="per_head")
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))
    assert_v_untouched(a, qkv, heads, head_dim)
    compare_fused(a, qkv, "bf16", heads, head_dim, qg, kg, cos, sin, style, what="parity")


@pytest.mark.parametrize("style", ["interleaved", "rotate_half"])
def test_bf16_tables_shared_vs_per_head(style):
    T, H, D = 133, 6, 128
    qkv = wl.fused_qkv(31, T, H, D, "fp16")
    qg, kg = wl.norm_weights(31, D)
    cos, sin = tables(np.arange(T), (D // 2,), D, style, dtype="bf16")
    a = run_fused(qkv, qg, kg, cos, sin, style)
    b = run_fused(qkv, qg, kg, wl.expand_per_head(cos, H), wl.expand_per_head(sin, H), style,
                  layout="per_head")
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))
    compare_fused(a, qkv, "fp16", H, D, qg, kg, cos, sin, style, what="bf16 tables")


def test_per_head_distinct_rows():
    """Per-head rows that are NOT a broadcast: row (t, h) must be used for head h."""
    T, H, D = 37, 5, 64
    rng = np.random.default_rng(5)
    qkv = wl.fused_qkv(32, T, H, D, "bf16")
    qg, kg = wl.norm_weights(32, D)
    ang = rng.uniform(0, 6.3, (T, H, D // 2))
    cos = torch.from_numpy(np.repeat(np.cos(ang), 2, axis=-1).astype(np.float32))
    sin = torch.from_numpy(np.repeat(np.sin(ang), 2, axis=-1).astype(np.float32))
    out = run_fused(qkv, qg, kg, cos, sin, "interleaved", layout="per_head")
    compare_fused(out, qkv, "bf16", H, D, qg, kg, cos, sin, "interleaved", layout="per_head",
                  what="per-head rows")


# ----------------------------------------------------------------------------- edge cases


@pytest.mark.parametrize("T,H,D", [(1, 1, 64), (1, 40, 128), (3, 5, 128), (5, 3, 64),
                                   (257, 7, 128), (130, 33, 64), (2, 9, 128), (65, 17, 64),
                                   (1, 1, 256), (67, 3, 256), (130, 25, 256)])
@pytest.mark.parametrize("style", ["interleaved", "rotate_half"])
def test_ragged_shapes(T, H, D, style):
    qkv = wl.fused_qkv(40 + T + H, T, H, D, "bf16")
    qg, kg = wl.norm_weights(41, D)
    cos, sin = tables(np.arange(T) * 11, (D // 2,), D, style)
    out = run_fused(qkv, qg, kg, cos, sin, style)
    compare_fused(out, qkv, "bf16", H, D, qg, kg, cos, sin, style, what="ragged")


@pytest.mark.parametrize("which", ["q", "k", "both"])
@pytest.mark.parametrize("T", [1, 6, 77])
def test_separate_single_tensor(which, T):
    H, D = 6, 128
    q, k = wl.separate_qk(50 + T, T, H, D, ("fp16",))["fp16"]
    qg, kg = wl.norm_weights(51, D)
    cos, sin = tables(np.arange(T), (D // 2,), D, "rotate_half")
    qd, qbuf = guarded(q)
    kd, kbuf = guarded(k)
    args = dict(cos=dev(cos), sin=dev(sin), style="rotate_half")
    if which in ("q", "both"):
        args.update(q=qd, q_gamma=dev(qg))
    if which in ("k", "both"):
        args.update(k=kd, k_gamma=dev(kg))
    qkr.qknorm_rope_fused(**args)
    torch.cuda.synchronize()
    assert canaries_intact(qbuf) and canaries_intact(kbuf)
    kw = dict(row_stride=H * D, col0=0, heads=H, head_dim=D, eps=wl.EPS, cos=cos.numpy(),
              sin=sin.numpy(), style="rotate_half")
    for name, t_in, t_dev, g in (("q", q, qd, qg), ("k", k, kd, kg)):
        if which in (name, "both"):
            ref = oracle.qknorm_rope(wl.u16(t_in), "fp16", gamma=g.numpy(), **kw)
            check_close(_decode(t_dev, "fp16"), ref, "fp16", name)
        else:
            assert torch.equal(t_dev.cpu().view(torch.int16), t_in.view(torch.int16))


def test_zero_tokens_changes_nothing():
    x = torch.zeros(0, 3 * 4 * 64, dtype=torch.bfloat16, device=DEV)
    g = torch.ones(64, device=DEV)
    c = torch.ones(0, 64, device=DEV)
    qkr.qknorm_rope_fused(x, q_gamma=g, k_gamma=g, cos=c, sin=c)
    torch.cuda.synchronize()


def test_max_heads():
    T, H, D = 2, 65536, 64
    qkv = wl.fused_qkv(60, T, H, D, "bf16")
    qg, kg = wl.norm_weights(60, D)
    cos, sin = tables(np.arange(T), (D // 2,), D, "interleaved")
    out = run_fused(qkv, qg, kg, cos, sin, "interleaved")
    compare_fused(out, qkv, "bf16", H, D, qg, kg, cos, sin, "interleaved", what="max heads")


def test_zero_heads_and_extreme_magnitudes():
    T, H, D = 9, 4, 128
    rng = np.random.default_rng(70)
    raw = rng.standard_normal((T, 3 * H * D)).astype(np.float32)
    raw[0, :H * D] = 0                      # every Q head of token 0 is zero
    raw[1, H * D:2 * H * D] = -0.0          # every K head of token 1 is -0
    raw[2] *= 8e3                           # large magnitudes (|x| < 65504 in fp16)
    raw[3] *= 1e-3
    raw[4, 5] = 900.0                       # one spike: |o| of that head reaches ~11
    for x_dtype in ("bf16", "fp16"):
        qkv = torch.from_numpy(raw).to(wl.DTYPES[x_dtype])
        qg, kg = wl.norm_weights(71, D)
        cos, sin = tables(np.arange(T) * 13, (D // 2,), D, "interleaved")
        out = run_fused(qkv, qg, kg, cos, sin, "interleaved")
        got = _decode(out, x_dtype).reshape(T, 3, H, D)
        assert np.all(got[0, 0] == 0) and np.all(got[1, 1] == 0)
        q_ref, k_ref = oracle_fused(qkv, x_dtype, H, D, qg, kg, cos, sin, "interleaved")
        check_rounding_bound(got[:, 0], q_ref, x_dtype, "extreme Q " + x_dtype)
        check_rounding_bound(got[:, 1], k_ref, x_dtype, "extreme K " + x_dtype)


def test_fp16_subnormal_inputs():
    T, H, D = 16, 3, 64
    rng = np.random.default_rng(80)
    raw = (rng.standard_normal((T, H, D)) * 3e-5).astype(np.float32)   # mostly subnormal fp16
    q = torch.from_numpy(raw).to(torch.float16)
    assert ((wl.u16(q) & 0x7C00) == 0).mean() > 0.5
    qg, _ = wl.norm_weights(81, D)
    cos, sin = tables(np.arange(T), (D // 2,), D, "interleaved")
    qd = dev(q)
    qkr.qknorm_rope_fused(q=qd, q_gamma=dev(qg), cos=dev(cos), sin=dev(sin), eps=1e-10)
    torch.cuda.synchronize()
    ref = oracle.qknorm_rope(wl.u16(q), "fp16", row_stride=H * D, col0=0, heads=H, head_dim=D,
                             gamma=qg.numpy(), eps=1e-10, cos=cos.numpy(), sin=sin.numpy())
    check_close(_decode(qd, "fp16"), ref, "fp16", "subnormal")


def test_side_stream():
    T, H, D = 300, 8, 128
    qkv = wl.fused_qkv(90, T, H, D, "bf16")
    qg, kg = wl.norm_weights(90, D)
    cos, sin = tables(np.arange(T), (D // 2,), D, "interleaved")
    st = torch.cuda.Stream()
    x = dev(qkv)
    g1, g2, c, s = dev(qg), dev(kg), dev(cos), dev(sin)
    torch.cuda.synchronize()
    with torch.cuda.stream(st):
        qkr.qknorm_rope_fused(x, q_gamma=g1, k_gamma=g2, cos=c, sin=s, stream=st)
    st.synchronize()
    compare_fused(x.cpu(), qkv, "bf16", H, D, qg, kg, cos, sin, "interleaved", what="stream")


def test_misaligned_pointer_is_rejected_and_nothing_changes():
    T, H, D = 8, 2, 64
    buf = torch.randn(T * 3 * H * D + 8, device=DEV).to(torch.bfloat16)
    before = buf.clone()
    x = buf[1:1 + T * 3 * H * D].view(T, 3 * H * D)          # 2-byte offset
    g = torch.ones(D, device=DEV)
    c = torch.ones(T, D, device=DEV)
    with pytest.raises(qkr.QkrError) as e:
        qkr.qknorm_rope_fused(x, q_gamma=g, k_gamma=g, cos=c, sin=c)
    assert e.value.status == qkr.binding.QKR_ERR_ALIGN
    torch.cuda.synchronize()
    assert torch.equal(buf.view(torch.int16), before.view(torch.int16))


# ----------------------------------------------------------------------------- capture and streams


@pytest.mark.parametrize("T,H", [(97, 6), (8200, 40)])
def test_graph_capture_replays_match_eager(T, H):
    """The call holds no allocation, copy or synchronisation, so it captures into a
    HIP graph; every replay must equal the same number of eager calls, bit for bit.
    8200 tokens of 40 heads is a long grid: its launch carries the residency
    reservation of dynamic LDS into the graph node."""
    D = 128
    info = qkr.kernel_info(D, heads=H, tokens=T)
    assert info["workgroups_per_cu"] == (2 if T == 8200 else 0), info
    qkv = wl.fused_qkv(100, T, H, D, "bf16")
    qg, kg = wl.norm_weights(100, D)
    cos, sin = tables(np.arange(T), (D // 2,), D, "interleaved")
    g1, g2, c, s = dev(qg), dev(kg), dev(cos), dev(sin)
    x_graph = dev(qkv)
    x_eager = dev(qkv)
    st = torch.cuda.Stream()
    graph = torch.cuda.CUDAGraph()
    torch.cuda.synchronize()
    with torch.cuda.graph(graph, stream=st):
        qkr.qknorm_rope_fused(x_graph, q_gamma=g1, k_gamma=g2, cos=c, sin=s)
    torch.cuda.synchronize()
    # capture does not execute: the buffer is still the input
    assert torch.equal(x_graph.view(torch.int16), x_eager.view(torch.int16))
    for replay in range(4):
        graph.replay()
        torch.cuda.synchronize()
        qkr.qknorm_rope_fused(x_eager, q_gamma=g1, k_gamma=g2, cos=c, sin=s)
        torch.cuda.synchronize()
        assert torch.equal(x_graph.view(torch.int16), x_eager.view(torch.int16)), replay
    # the first application matches the oracle (later ones re-normalise rotated data)
    once = dev(qkv)
    qkr.qknorm_rope_fused(once, q_gamma=g1, k_gamma=g2, cos=c, sin=s)
    torch.cuda.synchronize()
    compare_fused(once.cpu(), qkv, "bf16", H, D, qg, kg, cos, sin, "interleaved", what="graph")


def test_concurrent_streams_are_independent():
    """Calls on different streams over different buffers do not interfere."""
    T, H, D = 211, 8, 64
    streams = [torch.cuda.Stream() for _ in range(4)]
    cases = []
    for i, st in enumerate(streams):
        style = ("interleaved", "rotate_half")[i % 2]
        qkv = wl.fused_qkv(110 + i, T, H, D, "fp16")
        qg, kg = wl.norm_weights(110 + i, D)
        cos, sin = tables(np.arange(T) + 7 * i, (D // 2,), D, style)
        cases.append((qkv, qg, kg, cos, sin, style, dev(qkv), dev(qg), dev(kg), dev(cos), dev(sin)))
    torch.cuda.synchronize()
    for st, (_, _, _, _, _, style, x, g1, g2, c, s) in zip(streams, cases):
        with torch.cuda.stream(st):
            qkr.qknorm_rope_fused(x, q_gamma=g1, k_gamma=g2, cos=c, sin=s, style=style,
                                  stream=st)
    torch.cuda.synchronize()
    for qkv, qg, kg, cos, sin, style, x, *_ in cases:
        compare_fused(x.cpu(), qkv, "fp16", H, D, qg, kg, cos, sin, style, what="streams")


def _repeat_rows(block_dev: torch.Tensor, total: int) -> torch.Tensor:
    """[total, width] device tensor repeating the rows of block_dev."""
    b = block_dev.shape[0]
    out = torch.empty((total, block_dev.shape[1]), dtype=block_dev.dtype, device=DEV)
    n = total // b
    if n:
        out[:n * b].view(n, b, -1).copy_(block_dev.unsqueeze(0).expand(n, -1, -1))
    out[n * b:].copy_(block_dev[:total - n * b])
    return out


def test_maximum_tokens():
    """The largest call the library takes: tokens = 2^24 - 1, one 64-wide head,
    fused [16777215, 3*64] bf16 (6.4 GB) with 4.3 GB fp32 cos and sin tables,
    a grid of 2^23 workgroups in per-die runs.  Sampled tokens from both ends
    and the middle against the oracle; V untouched everywhere.  Activations and
    table rows repeat a 4096-token block (the pass is per token)."""
    T, H, D, B = (1 << 24) - 1, 1, 64, 4096
    block = wl.fused_qkv(4545, B, H, D, "bf16")
    qg, kg = wl.norm_weights(4545, D)
    cos, sin = tables(np.arange(B) * 7, (D // 2,), D, "interleaved")
    blk = block.to(DEV)
    x = _repeat_rows(blk, T)
    c, s = _repeat_rows(dev(cos), T), _repeat_rows(dev(sin), T)
    info = qkr.kernel_info(D, "shared", qkr.binding.QKR_FP32, "interleaved",
                           qkr.binding.QKR_BF16, heads=H, tokens=T)
    assert info["die_runs"] == 1 and info["tokens_per_block"] == 2
    qkr.qknorm_rope_fused(x, q_gamma=dev(qg), k_gamma=dev(kg), cos=c, sin=s, style="interleaved")
    torch.cuda.synchronize()
    del c, s
    n = T // B
    xb, bb = x.view(torch.int16), blk.view(torch.int16)
    v = xb[:n * B].view(n, B, -1)[:, :, 2 * H * D:]
    assert torch.equal(v, bb[:, 2 * H * D:].unsqueeze(0).expand(n, -1, -1)), "V changed"
    assert torch.equal(xb[n * B:, 2 * H * D:], bb[:T - n * B, 2 * H * D:]), "V changed"
    rng = np.random.default_rng(4546)
    samples = sorted({0, 1, B - 1, B, T // 2, T - B, T - 2, T - 1,
                      *rng.integers(0, T, 24).tolist()})
    assert max(samples) < T
    idx = torch.tensor(samples)
    rows = block[idx % B]
    q_ref, k_ref = oracle_fused(rows, "bf16", H, D, qg, kg, cos[idx % B], sin[idx % B],
                                "interleaved")
    got = _decode(x[idx.to(DEV)], "bf16").reshape(len(samples), 3, H, D)
    m = max(check_close(got[:, 0], q_ref, "bf16", "max tokens Q"),
            check_close(got[:, 1], k_ref, "bf16", "max tokens K"))
    print("maximum tokens max_abs", m)


# heads giving each unroll depth (head iterations in flight), per head_dim
SWEEP_HEADS = {128: {3: 5, 6: 20, 10: 40, 12: 48}, 64: {3: 9, 6: 44, 10: 72, 12: 100},
               256: {3: 5, 6: 11, 10: 19, 12: 30}}
CODES = {"bf16": qkr.binding.QKR_BF16, "fp16": qkr.binding.QKR_FP16, "fp32": qkr.binding.QKR_FP32}


@pytest.mark.parametrize("head_dim", [64, 128, 256])
@pytest.mark.parametrize("layout", ["shared", "per_head"])
@pytest.mark.parametrize("table", ["fp32", "bf16"])
@pytest.mark.parametrize("x_dtype", ["bf16", "fp16"])
def test_every_kernel_instantiation(head_dim, layout, table, x_dtype):
    """Every compiled kernel of one (head_dim, layout, table dtype, data dtype):
    both styles, each unroll depth and both block orders (203 tokens: hardware
    order; 8200 tokens = 4100 workgroups: per-die runs with a ragged
    remainder), against the oracle on sampled tokens, V checked on them too.
    Per-head tables hold a distinct row per (token, head).  Activations and
    tables repeat a 256-token block (the pass is per token)."""
    D, B = head_dim, 256
    depths = (3, 6, 10) if layout == "per_head" else (3, 6, 10, 12)
    hit = set()
    rng = np.random.default_rng(5000 + D)
    for style in ("interleaved", "rotate_half"):
        for depth in depths:
            H = SWEEP_HEADS[D][depth]
            block = wl.fused_qkv(5000 + H, B, H, D, x_dtype)
            qg, kg = wl.norm_weights(5000 + H, D)
            if layout == "shared":
                cos, sin = tables(np.arange(B) * 3 + 1, (D // 2,), D, style, dtype=table)
            else:
                c, s = tables(np.arange(B * H) + 1, (D // 2,), D, style, dtype=table)
                cos, sin = c.view(B, H, D), s.view(B, H, D)
            blk = block.to(DEV)
            for T in (203, 8200):
                info = qkr.kernel_info(D, layout, CODES[table], style, CODES[x_dtype], heads=H,
                                       tokens=T)
                hit.add((style, info["heads_in_flight"], info["die_runs"]))
                x = _repeat_rows(blk, T)
                cd = _repeat_rows(dev(cos).reshape(B, -1), T).view(T, *cos.shape[1:])
                sd = _repeat_rows(dev(sin).reshape(B, -1), T).view(T, *sin.shape[1:])
                qkr.qknorm_rope_fused(x, q_gamma=dev(qg), k_gamma=dev(kg), cos=cd, sin=sd,
                                      style=style, cos_layout=layout)
                torch.cuda.synchronize()
                idx = sorted(i for i in {0, 1, B - 1, B, T // 2, T - 2, T - 1,
                                         *rng.integers(0, T, 8).tolist()} if i < T)
                assert 0 <= idx[0] and idx[-1] < T     # checked here, before indexing on the GPU
                it = torch.tensor(idx)
                rows = block[it % B]
                q_ref, k_ref = oracle_fused(rows, x_dtype, H, D, qg, kg, cos[it % B],
                                            sin[it % B], style, layout)
                out = x[it.to(DEV)].cpu()
                got = _decode(out, x_dtype).reshape(len(idx), 3, H, D)
                what = "%s U%d order%d T%d" % (style, info["heads_in_flight"], info["die_runs"], T)
                check_close(got[:, 0], q_ref, x_dtype, what + " Q")
                check_close(got[:, 1], k_ref, x_dtype, what + " K")
                assert_v_untouched(out, rows, H, D)
    assert hit == {(st, u, o) for st in ("interleaved", "rotate_half") for u in depths
                   for o in (0, 1)}, hit


def _random_case(case, rng):
    """One seeded draw from the whole call space of the pass (the tensor mode
    cycles with the case number)."""
    D = int(rng.choice([64, 128, 256]))
    T = int(rng.choice([int(rng.integers(1, 300)), int(rng.integers(8190, 8400))]))
    H = int(rng.integers(1, 1 + {64: 60, 128: 40, 256: 24}[D]))
    return dict(
        mode=("fused", "pair", "q", "k")[case % 4], D=D, T=T, H=min(H, 12) if T > 4000 else H,
        style=str(rng.choice(["interleaved", "rotate_half"])),
        layout=str(rng.choice(["shared", "per_head"])),
        table=str(rng.choice(["fp32", "bf16"])), x_dtype=str(rng.choice(["bf16", "fp16"])))


@pytest.mark.parametrize("case", range(24))
def test_random_calls_across_the_api(case):
    """24 seeded draws over tensor mode (fused, q and k, q alone, k alone),
    head_dim, heads, tokens (small grids and grids past the per-die-runs
    threshold), style, cos/sin layout and dtype and data dtype: every output
    element against the oracle, tensors not passed bit-unchanged, canaries
    intact."""
    c = _random_case(case, np.random.default_rng(9000 + case))
    T, H, D, style, layout = c["T"], c["H"], c["D"], c["style"], c["layout"]
    xd = c["x_dtype"]
    seed = 9100 + case
    rows = T * (H if layout == "per_head" else 1)
    cos, sin = tables(np.arange(rows) * 3 + 1, (D // 2,), D, style, dtype=c["table"])
    if layout == "per_head":
        cos, sin = cos.view(T, H, D), sin.view(T, H, D)
    qg, kg = wl.norm_weights(seed, D)
    what = "case %d %s" % (case, c)
    if c["mode"] == "fused":
        qkv = wl.fused_qkv(seed, T, H, D, xd)
        out = run_fused(qkv, qg, kg, cos, sin, style, layout=layout)
        compare_fused(out, qkv, xd, H, D, qg, kg, cos, sin, style, layout=layout, what=what)
        return
    q, k = wl.separate_qk(seed, T, H, D, (xd,))[xd]
    qd, qbuf = guarded(q)
    kd, kbuf = guarded(k)
    args = dict(cos=dev(cos), sin=dev(sin), style=style, cos_layout=layout)
    if c["mode"] in ("pair", "q"):
        args.update(q=qd, q_gamma=dev(qg))
    if c["mode"] in ("pair", "k"):
        args.update(k=kd, k_gamma=dev(kg))
    qkr.qknorm_rope_fused(**args)
    torch.cuda.synchronize()
    assert canaries_intact(qbuf) and canaries_intact(kbuf), what
    kw = dict(row_stride=H * D, col0=0, heads=H, head_dim=D, eps=wl.EPS, cos=table_np(cos),
              sin=table_np(sin), cos_dtype=c["table"], cos_layout=layout, style=style)
    for name, t_in, t_dev, g in (("q", q, qd, qg), ("k", k, kd, kg)):
        if c["mode"] in (name, "pair"):
            ref = oracle.qknorm_rope(wl.u16(t_in), xd, gamma=g.numpy(), **kw)
            check_close(_decode(t_dev, xd), ref, xd, what + " " + name)
        else:
            assert torch.equal(t_dev.cpu().view(torch.int16), t_in.view(torch.int16)), what


# ----------------------------------------------------------------------------- large and tiny finite values


def _heads_with_peaks(rng, T, H, D, peaks):
    """fp64 [T, 3, H, D]: N(0,1) heads rescaled so that each head's largest |x|
    is one of `peaks`, cycling over token, tensor and head, so every token
    mixes heads of every magnitude in Q, K and V."""
    raw = rng.standard_normal((T, 3, H, D))
    raw /= np.abs(raw).max(axis=-1, keepdims=True)
    idx = (np.arange(T)[:, None, None] + np.arange(3)[None, :, None]
           + np.arange(H)[None, None, :]) % len(peaks)
    return raw * np.asarray(peaks, dtype=np.float64)[idx][..., None]


@pytest.mark.parametrize("head_dim", [64, 128, 256])
@pytest.mark.parametrize("style", ["interleaved", "rotate_half"])
def test_large_finite_bf16_heads(head_dim, style):
    """bf16 heads whose fp32 sum of squares overflows: largest |x| of 1e18,
    1e30 and 3e38 (the largest finite bf16 is 3.39e38), next to O(1) heads in
    the same token, plus heads that are O(1) but for one element at 3.3e38.
    Every element against the oracle within the rounding model (half an ulp
    plus fp32 noise); heads whose outputs stay below 8 also at the bf16
    tolerance (a spike head's normalised spike is about sqrt(D) * gamma, where
    half an ulp of bf16 exceeds the fixed tolerance).  The shared and
    per-head layouts stay bit-identical on them."""
    T, H, D = 41, 7, head_dim
    rng = np.random.default_rng(600 + D)
    raw = _heads_with_peaks(rng, T, H, D, [1.0, 1e18, 1e30, 3e38, 5.0])
    raw[::5, 1, 2] = rng.standard_normal(D)
    raw[::5, 1, 2, 3] = 3.3e38                       # a single spike in an O(1) head
    qkv = torch.from_numpy(raw.reshape(T, -1).astype(np.float32)).to(torch.bfloat16)
    assert torch.isfinite(qkv.float()).all()
    qg, kg = wl.norm_weights(601, D)
    cos, sin = tables(np.arange(T) * 7, (D // 2,), D, style)
    shared = run_fused(qkv, qg, kg, cos, sin, style)
    per_head = run_fused(qkv, qg, kg, wl.expand_per_head(cos, H), wl.expand_per_head(sin, H),
                         style, layout="per_head")
    assert torch.equal(shared.view(torch.int16), per_head.view(torch.int16))
    assert_v_untouched(shared, qkv, H, D)
    q_ref, k_ref = oracle_fused(qkv, "bf16", H, D, qg, kg, cos, sin, style)
    got = _decode(shared, "bf16").reshape(T, 3, H, D)
    m = 0.0
    for part, ref, name in ((got[:, 0], q_ref, "Q"), (got[:, 1], k_ref, "K")):
        check_rounding_bound(part, ref, "bf16", "large bf16 " + name)
        below8 = np.abs(ref).max(axis=-1) < 8
        assert below8.sum() > 0.9 * below8.size
        m = max(m, check_close(part[below8], ref[below8], "bf16", "large bf16 " + name))
    print("large finite bf16 heads D", D, style, "max_abs (heads below 8)", m)


@pytest.mark.parametrize("eps", [1e-6, 1e-38, 1.4e-45])
@pytest.mark.parametrize("x_dtype", ["bf16", "fp16"])
def test_tiny_heads_and_tiny_eps(eps, x_dtype):
    """Heads of tiny values (largest |x| from 1e-12 down to bf16 subnormals
    near 1e-40; fp16 down to its subnormals near 1e-7) with eps down to the
    smallest fp32 subnormal: where the fp32 sum of squares sinks into the
    subnormal range and eps does not swamp it, the head is summed again
    rescaled.  Every element against the oracle."""
    T, H, D = 37, 5, 128
    rng = np.random.default_rng(700)
    peaks = ([1.0, 1e-12, 1e-20, 1e-30, 1e-38, 1e-40] if x_dtype == "bf16"
             else [1.0, 1e-3, 1e-5, 3e-7, 5.0])
    raw = _heads_with_peaks(rng, T, H, D, peaks)
    raw[0, 0, 0] = 0.0                               # an all-zero head: exact zeros
    qkv = torch.from_numpy(raw.reshape(T, -1).astype(np.float32)).to(wl.DTYPES[x_dtype])
    qg, kg = wl.norm_weights(701, D)
    cos, sin = tables(np.arange(T) * 3, (D // 2,), D, "interleaved")
    out = run_fused(qkv, qg, kg, cos, sin, "interleaved", eps=eps)
    got = _decode(out, x_dtype).reshape(T, 3, H, D)
    assert np.all(got[0, 0, 0] == 0)
    q_ref, k_ref = oracle.fused_qk(wl.u16(qkv), x_dtype, heads=H, head_dim=D, q_gamma=qg.numpy(),
                                   k_gamma=kg.numpy(), eps=eps, cos=cos.numpy(), sin=sin.numpy(),
                                   style="interleaved")
    m = max(check_close(got[:, 0], q_ref, x_dtype, "tiny Q eps %g" % eps),
            check_close(got[:, 1], k_ref, x_dtype, "tiny K eps %g" % eps))
    assert_v_untouched(out, qkv, H, D)
    print("tiny heads", x_dtype, "eps", eps, "max_abs", m)


def test_large_heads_in_the_headline_launch():
    """The headline's launch configuration (32760 tokens, 40 heads, per-die
    runs, 10 head iterations in flight) with large-magnitude heads spread over
    the call: tokens whose heads mix 1e18 / 1e30 / 3e38 with O(1) ones, in
    every tenth token; oracle on those tokens and a few plain ones."""
    w = wl.WORKLOADS["headline"]
    T, H, D = w.tokens, w.heads, w.head_dim
    qkv = wl.fused_qkv(w.seed, T, H, D, "bf16")
    rng = np.random.default_rng(702)
    hot = np.arange(3, T, 10)
    block = _heads_with_peaks(rng, len(hot), H, D, [1.0, 1e18, 1e30, 3e38])
    qkv[torch.from_numpy(hot)] = torch.from_numpy(
        block.reshape(len(hot), -1).astype(np.float32)).to(torch.bfloat16)
    qg, kg = wl.norm_weights(w.seed, D)
    cos, sin = wl.workload_tables(w, "interleaved")
    out = run_fused(qkv, qg, kg, cos, sin, "interleaved")
    assert_v_untouched(out, qkv, H, D)
    idx = np.unique(np.concatenate([hot[:: max(1, len(hot) // 200)], [0, 1, 2, T - 1]]))
    assert idx.max() < T
    it = torch.from_numpy(idx)
    rows = qkv[it]
    q_ref, k_ref = oracle_fused(rows, "bf16", H, D, qg, kg, cos[it], sin[it], "interleaved")
    got = _decode(out[it], "bf16").reshape(len(idx), 3, H, D)
    m = max(check_close(got[:, 0], q_ref, "bf16", "headline large Q"),
            check_close(got[:, 1], k_ref, "bf16", "headline large K"))
    print("headline launch with large heads: max_abs", m, "tokens checked", len(idx))
