"""C-ABI checks that need no GPU: exports and argument validation.

Every call here is rejected (or is the tokens == 0 no-op) before the library
makes any HIP call, so nothing is launched.  Pointers are fake, aligned or
misaligned integers that are never dereferenced.
"""
import ctypes
import os
import re

import pytest

import diffusion_transformer_qk_amd as qkr
from diffusion_transformer_qk_amd import binding as b

INCLUDE = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include")

A = 0x10000          # a 16-byte aligned fake device address
MIS = 0x10008        # 8-byte aligned only


def declared_functions():
    names = set()
    for h in sorted(os.listdir(INCLUDE)):
        if h.endswith(".h"):
            with open(os.path.join(INCLUDE, h)) as f:
                text = re.sub(r"/\*.*?\*/", "", f.read(), flags=re.S)
            names |= set(re.findall(r"^\s*(?:int|int32_t|int64_t|const char\*)\s+(\w+)\s*\(", text,
                                    flags=re.M))
    return names


def test_every_declared_symbol_is_exported():
    lib = ctypes.CDLL(qkr.LIB_PATH)
    names = declared_functions()
    assert names == set(b.EXPORTS)
    for name in names:
        assert hasattr(lib, name), name


def test_version_and_strerror():
    assert qkr.version() == 2
    for code in (0, -1, -2, -3, -4, -5, -6, -7):
        assert qkr.strerror(code) != "unknown status"
    assert qkr.strerror(12345) == "unknown status"


def call(**over):
    args = dict(qkv=A, q=0, k=0, tokens=16, heads=40, head_dim=128, q_gamma=A, k_gamma=A,
                eps=1e-6, cos=A, sin=A, cos_layout=0, cos_dtype=b.QKR_FP32, style=0,
                dtype=b.QKR_BF16, stream=0)
    args.update(over)
    return qkr.qknorm_rope_fused_raw(**args)


@pytest.mark.parametrize("over,code", [
    (dict(head_dim=96), b.QKR_ERR_UNSUPPORTED),
    (dict(head_dim=512), b.QKR_ERR_UNSUPPORTED),
    (dict(head_dim=32), b.QKR_ERR_UNSUPPORTED),
    (dict(dtype=b.QKR_FP32), b.QKR_ERR_UNSUPPORTED),
    (dict(cos_dtype=b.QKR_FP16), b.QKR_ERR_UNSUPPORTED),
    (dict(dtype=7), b.QKR_ERR_ARG),
    (dict(cos_dtype=-1), b.QKR_ERR_ARG),
    (dict(style=2), b.QKR_ERR_ARG),
    (dict(cos_layout=5), b.QKR_ERR_ARG),
    (dict(eps=0.0), b.QKR_ERR_ARG),
    (dict(eps=-1e-6), b.QKR_ERR_ARG),
    (dict(eps=float("nan")), b.QKR_ERR_ARG),
    (dict(eps=float("inf")), b.QKR_ERR_ARG),
    (dict(tokens=-1), b.QKR_ERR_SHAPE),
    (dict(tokens=1 << 24), b.QKR_ERR_SHAPE),       # grid limit: 2^23 workgroups of 256
    (dict(tokens=1 << 31), b.QKR_ERR_SHAPE),
    (dict(heads=0), b.QKR_ERR_SHAPE),
    (dict(heads=65537), b.QKR_ERR_SHAPE),
    (dict(qkv=A, q=A), b.QKR_ERR_MODE),
    (dict(qkv=A, k=A), b.QKR_ERR_MODE),
    (dict(qkv=0), b.QKR_ERR_MODE),
    (dict(k_gamma=0), b.QKR_ERR_NULL),
    (dict(q_gamma=0), b.QKR_ERR_NULL),
    (dict(qkv=0, q=A, q_gamma=0), b.QKR_ERR_NULL),
    (dict(qkv=0, k=A, k_gamma=0), b.QKR_ERR_NULL),
    (dict(cos=0), b.QKR_ERR_NULL),
    (dict(sin=0), b.QKR_ERR_NULL),
    (dict(qkv=MIS), b.QKR_ERR_ALIGN),
    (dict(qkv=0, q=MIS), b.QKR_ERR_ALIGN),
    (dict(qkv=0, q=A, k=MIS), b.QKR_ERR_ALIGN),
    (dict(cos=MIS), b.QKR_ERR_ALIGN),
    (dict(sin=A + 4), b.QKR_ERR_ALIGN),
    (dict(q_gamma=A + 4), b.QKR_ERR_ALIGN),
    (dict(qkv=0, k=A, k_gamma=A + 12), b.QKR_ERR_ALIGN),
])
def test_rejects_before_any_hip_call(over, code):
    assert call(**over) == code


T16 = 16 * 3 * 40 * 128 * 2          # bytes of the default call's fused QKV buffer
Q16 = 16 * 40 * 128 * 2              # bytes of one separate [16, 40, 128] tensor
G = 0x4000000                        # far from every buffer of the default call
FAR = dict(cos=G, sin=G + 0x200000, q_gamma=G + 0x400000, k_gamma=G + 0x400000)


@pytest.mark.parametrize("over", [
    dict(cos=A + T16 - 16),                            # a table ends inside qkv
    dict(sin=A + 4096),
    dict(q_gamma=A + 1024),                            # a weight inside qkv (V region too)
    dict(k_gamma=A + T16 - 16),
    dict(qkv=0, q=A, k=A + Q16 - 16),                  # k starts inside q
    dict(qkv=0, q=A + Q16 - 16, k=A),                  # q starts inside k
    dict(qkv=0, q=A, k=A + Q16, cos=A + Q16 + 64),     # a table inside k
    dict(qkv=0, k=A, k_gamma=A + 256),                 # k's weight inside k
])
def test_written_buffer_overlapping_another_is_rejected(over):
    assert call(**{**FAR, **over}) == b.QKR_ERR_ARG


def test_adjacent_buffers_pass_validation():
    # adjacent, not overlapping: only the NULL table stops the call (nothing launched)
    assert call(**{**FAR, "qkv": 0, "q": A, "k": A + Q16, "cos": 0}) == b.QKR_ERR_NULL
    assert call(**{**FAR, "cos": A + T16, "sin": 0}) == b.QKR_ERR_NULL


def test_zero_tokens_is_a_no_op():
    # valid scalars: OK without looking at (or launching on) the pointers
    assert call(tokens=0, qkv=0, q_gamma=0, k_gamma=0, cos=0, sin=0) == b.QKR_OK
    # invalid scalars are still reported
    assert call(tokens=0, head_dim=32) == b.QKR_ERR_UNSUPPORTED


def test_kernel_info_rejects_bad_arguments_before_any_hip_call():
    lib = b.load_library()
    info = b.KernelInfo()
    ref = ctypes.byref(info)
    assert lib.qknorm_rope_kernel_info(128, 40, 100, 3, 0, b.QKR_FP32, 0, b.QKR_BF16, ref) \
        == b.QKR_ERR_ARG                                          # tensors out of range
    assert lib.qknorm_rope_kernel_info(128, 40, 100, -1, 0, b.QKR_FP32, 0, b.QKR_BF16, ref) \
        == b.QKR_ERR_ARG
    assert lib.qknorm_rope_kernel_info(128, 40, 100, 0, 0, b.QKR_FP32, 0, b.QKR_BF16, None) \
        == b.QKR_ERR_NULL
    assert lib.qknorm_rope_kernel_info(96, 40, 100, 1, 0, b.QKR_FP32, 0, b.QKR_BF16, ref) \
        == b.QKR_ERR_UNSUPPORTED
    assert lib.qknorm_rope_kernel_info(128, 40, 1 << 24, 2, 0, b.QKR_FP32, 0, b.QKR_BF16, ref) \
        == b.QKR_ERR_SHAPE


def test_separate_mode_skips_missing_tensor_gamma():
    # k absent: its gamma may be NULL; the call is then only rejected for the table
    assert call(qkv=0, q=A, k=0, k_gamma=0, cos=0) == b.QKR_ERR_NULL
    assert call(qkv=0, q=A, k=0, k_gamma=0, cos=MIS) == b.QKR_ERR_ALIGN


def test_python_binding_rejects_cpu_tensors():
    import torch
    x = torch.zeros(4, 3 * 2 * 64, dtype=torch.bfloat16)
    g = torch.ones(64)
    c = torch.ones(4, 64)
    with pytest.raises(ValueError):
        qkr.qknorm_rope_fused(x, q_gamma=g, k_gamma=g, cos=c, sin=c)
    with pytest.raises(ValueError):   # wrong table size
        qkr.qknorm_rope_fused(x, q_gamma=g, k_gamma=g, cos=c[:3], sin=c[:3])
    q = torch.zeros(4, 2, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="heads, head_dim"):   # heads disagree with the shape
        qkr.qknorm_rope_fused(q=q, q_gamma=g, cos=c, sin=c, heads=4)
    with pytest.raises(ValueError, match="heads, head_dim"):
        qkr.qknorm_rope_fused(q=q.view(4, 128), q_gamma=g, cos=c, sin=c, heads=2, head_dim=64)
    with pytest.raises(ValueError, match="style"):             # an unknown name, not a KeyError
        qkr.qknorm_rope_fused(x, q_gamma=g, k_gamma=g, cos=c, sin=c, style="neox")
    with pytest.raises(ValueError, match="cos_layout"):
        qkr.qknorm_rope_fused(x, q_gamma=g, k_gamma=g, cos=c, sin=c, cos_layout="expanded")


# ----------------------------------------------------------------------------- AdaLN entry point


def fss(**over):
    args = dict(x=A, y=A + 0x100000, rows=16, hidden=6144, rows_per_batch=16, scale=A,
                shift=A, mod_dtype=b.QKR_FP32, eps=1e-6, dtype=b.QKR_BF16, stream=0)
    args.update(over)
    return qkr.dit_fuse_scale_shift_raw(**args)


@pytest.mark.parametrize("over,code", [
    (dict(hidden=6), b.QKR_ERR_UNSUPPORTED),
    (dict(hidden=100), b.QKR_ERR_UNSUPPORTED),
    (dict(hidden=8200), b.QKR_ERR_UNSUPPORTED),
    (dict(dtype=b.QKR_FP32), b.QKR_ERR_UNSUPPORTED),
    (dict(dtype=9), b.QKR_ERR_ARG),
    (dict(mod_dtype=3), b.QKR_ERR_ARG),
    (dict(eps=0.0), b.QKR_ERR_ARG),
    (dict(eps=float("nan")), b.QKR_ERR_ARG),
    (dict(rows=-2), b.QKR_ERR_SHAPE),
    (dict(rows=1 << 24), b.QKR_ERR_SHAPE),
    (dict(rows=1 << 31), b.QKR_ERR_SHAPE),
    (dict(rows_per_batch=0), b.QKR_ERR_SHAPE),
    (dict(x=0), b.QKR_ERR_NULL),
    (dict(y=0), b.QKR_ERR_NULL),
    (dict(scale=0), b.QKR_ERR_NULL),
    (dict(shift=0), b.QKR_ERR_NULL),
    (dict(x=MIS), b.QKR_ERR_ALIGN),
    (dict(y=A + 0x100008), b.QKR_ERR_ALIGN),
    (dict(scale=A + 4), b.QKR_ERR_ALIGN),
    (dict(shift=MIS), b.QKR_ERR_ALIGN),
    (dict(y=A + 16 * 6144), b.QKR_ERR_ARG),        # y starts inside x
    (dict(x=A + 0x100000 + 1024 * 16, y=A + 0x100000), b.QKR_ERR_ARG),   # x inside y
    (dict(scale=A + 0x100000 + 64), b.QKR_ERR_ARG),  # modulation inside y
    (dict(x=A + 0x100000, y=A + 0x100000, shift=A + 0x100000 + 16 * 6144 * 2 - 16),
     b.QKR_ERR_ARG),                               # in place, shift inside the buffer
])
def test_fuse_scale_shift_rejects_before_any_hip_call(over, code):
    assert fss(**over) == code


def test_fuse_scale_shift_zero_rows_is_a_no_op():
    assert fss(rows=0, x=0, y=0, scale=0, shift=0) == b.QKR_OK
    assert fss(rows=0, hidden=12) == b.QKR_ERR_UNSUPPORTED


def test_fuse_scale_shift_binding_checks_shapes():
    import torch
    x = torch.zeros(6, 64, dtype=torch.bfloat16)
    s = torch.zeros(4, 64)
    with pytest.raises(ValueError):      # 6 rows do not split over 4 batches
        qkr.fuse_scale_shift(x, s, s)
    with pytest.raises(ValueError):      # hidden mismatch
        qkr.fuse_scale_shift(x, s[:, :32], s[:, :32])
    with pytest.raises(ValueError):      # CPU tensors are refused
        qkr.fuse_scale_shift(x, s[:2], s[:2])


# ----------------------------------------------------------------------------- group norm + SiLU


def gn(**over):
    args = dict(x=A, y=A + 0x1000000, n=2, channels=64, spatial=4096, groups=32, gamma=A, beta=A,
                param_dtype=b.QKR_FP32, eps=1e-6, dtype=b.QKR_BF16, workspace=0, workspace_bytes=0,
                stream=0)
    args.update(over)
    return qkr.dit_group_norm_silu_raw(**args)


def test_group_norm_workspace_size():
    """8 bytes per chunk; chunks of 16384 elements, or 8192 / 4096 when a call
    would otherwise run fewer than 2048 workgroups; nothing for one chunk."""
    ws = qkr.group_norm_silu_workspace_size
    assert ws(1, 128, 1024 * 1024, 32) == 32 * 256 * 8      # 8192 workgroups of 16384
    assert ws(1, 512, 128 * 128, 32) == 32 * 64 * 8         # 512 or 1024 would be too few: 4096
    assert ws(4, 256, 30000, 32) == 128 * 30 * 8            # 1920 at 16384, 3840 at 8192
    assert ws(4, 512, 16392, 32) == 128 * 17 * 8            # 2176 at 16384 (ragged)
    assert ws(2, 64, 4096, 32) == 0                         # 8192-element groups: one chunk
    assert ws(1, 6, 16384 * 2 + 8, 2) == 2 * 25 * 8         # 98328 elements in 4096s
    assert ws(1, 64, 12, 32) == b.QKR_ERR_UNSUPPORTED       # spatial not a multiple of 8
    assert ws(1, 60, 64, 32) == b.QKR_ERR_SHAPE             # groups do not divide channels
    assert ws(-1, 64, 64, 32) == b.QKR_ERR_SHAPE
    assert ws(1, 2, 1 << 31, 1) == b.QKR_ERR_UNSUPPORTED
    # one workgroup per chunk, and a grid holds fewer than 2^32 work-items of 256
    assert ws((1 << 24) - 1, 1, 8, 1) == 0                  # 2^24 - 1 one-chunk groups
    assert ws(1 << 22, 4, 8, 4) == b.QKR_ERR_SHAPE          # 2^24 one-chunk groups
    assert ws(1 << 10, 16, 16384 * 1024, 16) == b.QKR_ERR_SHAPE   # 2^14 pairs x 1024 chunks


@pytest.mark.parametrize("over,code", [
    (dict(dtype=b.QKR_FP32), b.QKR_ERR_UNSUPPORTED),
    (dict(dtype=5), b.QKR_ERR_ARG),
    (dict(param_dtype=-1), b.QKR_ERR_ARG),
    (dict(eps=0.0), b.QKR_ERR_ARG),
    (dict(groups=7), b.QKR_ERR_SHAPE),
    (dict(channels=0), b.QKR_ERR_SHAPE),
    (dict(spatial=100), b.QKR_ERR_UNSUPPORTED),
    (dict(n=-3), b.QKR_ERR_SHAPE),
    (dict(x=0), b.QKR_ERR_NULL),
    (dict(gamma=0), b.QKR_ERR_NULL),
    (dict(beta=MIS), b.QKR_ERR_ALIGN),
    (dict(y=A + 4096), b.QKR_ERR_ARG),                         # partial overlap
    (dict(spatial=65536), b.QKR_ERR_WORKSPACE),                # needs a workspace
    (dict(spatial=65536, workspace=A + 0x9000000, workspace_bytes=8), b.QKR_ERR_WORKSPACE),
    (dict(spatial=65536, workspace=MIS, workspace_bytes=1 << 20), b.QKR_ERR_WORKSPACE),
    (dict(gamma=A + 0x1000000 + 64), b.QKR_ERR_ARG),                   # gamma inside y
    (dict(x=A + 0x1000000, y=A + 0x1000000, beta=A + 0x1000000 + 4096), b.QKR_ERR_ARG),
    (dict(spatial=65536, workspace=A + 0x1000000 + 64, workspace_bytes=1 << 20),
     b.QKR_ERR_ARG),                                                   # workspace inside y
    (dict(spatial=65536, workspace=A, workspace_bytes=1 << 20), b.QKR_ERR_ARG),  # inside x
])
def test_group_norm_rejects_before_any_hip_call(over, code):
    assert gn(**over) == code


def test_group_norm_zero_samples_is_a_no_op():
    assert gn(n=0, x=0, y=0, gamma=0, beta=0) == b.QKR_OK


@pytest.mark.parametrize("n,channels,spatial,groups,want", [
    (2, 64, 512, 32, ("one_read", 16384)),             # a group fits one chunk
    (1, 128, 1024 * 1024, 32, ("lagged", 16384)),      # VAE out: 8,192 chunks of 256 per group
    (1, 256, 512 * 512, 32, ("lagged", 16384)),        # VAE up: 4,096 chunks
    (8, 512, 16384, 32, ("lagged", 16384)),            # exactly 4,096 chunks
    (4, 512, 16384, 32, ("two_pass", 16384)),          # 2,048 chunks: below the lagged threshold
    (1, 512, 128 * 128, 32, ("two_pass", 4096)),       # VAE mid: small chunks fill the chip
    (1, 64, 2048 * 2048, 32, ("two_pass", 16384)),     # 512 chunks per group: over 256
    (1, 32, 256 * 16384, 32, ("lagged", 16384)),       # exactly 256 chunks per group
    (1, 32, 257 * 16384, 32, ("two_pass", 16384)),     # 257 chunks per group
    (4096, 8, 2 * 16384, 4, ("lagged", 16384)),        # 16,384 groups of 4 chunks
    (1, 1365, 3 * 16384, 1365, ("two_pass", 16384)),   # 1,365 groups of 3 chunks: 4,095
    (1, 2048, 16392, 2048, ("lagged", 16384)),         # 2,048 groups of 2 chunks: 4,096
])
def test_group_norm_schedule_by_shape(n, channels, spatial, groups, want):
    assert qkr.group_norm_silu_schedule(n, channels, spatial, groups) == want


def test_group_norm_schedule_rejects_what_the_call_rejects():
    with pytest.raises(qkr.QkrError):
        qkr.group_norm_silu_schedule(1, 30, 64, 4)          # groups does not divide channels
    with pytest.raises(qkr.QkrError):
        qkr.group_norm_silu_schedule(1, 8, 12, 2)           # spatial not a multiple of 8
    lib = qkr.load_library()
    assert lib.dit_group_norm_silu_schedule(1, 8, 64, 2, None) == 0      # the size out-pointer is optional



def test_group_norm_test_hook_is_outside_the_public_headers():
    """dit_group_norm_silu_polls is exported for the tests only: declared in
    tests/c_abi/gn_test_hooks.h, not under include/, and it rejects a poll
    count outside 0..4096 before any HIP call."""
    from tests import gn_hooks

    assert "dit_group_norm_silu_polls" not in declared_functions()
    hooks = os.path.join(os.path.dirname(os.path.abspath(__file__)), "c_abi", "gn_test_hooks.h")
    with open(hooks) as f:
        assert "int dit_group_norm_silu_polls(" in f.read()
    for polls in (-1, gn_hooks.MAX_POLLS + 1):
        assert gn_hooks.polls_raw(A, A + (1 << 30), 1, 64, 64, 8, A, A, b.QKR_FP32, 1e-6,
                                  b.QKR_BF16, 0, 0, 0, polls) == b.QKR_ERR_ARG


def test_library_reads_no_environment():
    """The shipped library's behaviour depends on its arguments only: it
    imports no environment-reading function."""
    import subprocess

    out = subprocess.run(["nm", "-D", "--undefined-only", qkr.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    names = {line.split()[-1].split("@")[0] for line in out.splitlines() if line.strip()}
    assert not names & {"getenv", "secure_getenv", "__secure_getenv"}, names & {"getenv"}


def gn_noalloc(**over):
    args = dict(x=A, y=A + (1 << 36), n=1, channels=64, spatial=64, groups=8, gamma=A, beta=A,
                param_dtype=b.QKR_FP32, eps=1e-6, dtype=b.QKR_BF16, stream=0)
    args.update(over)
    return qkr.dit_group_norm_silu_noalloc_raw(**args)


@pytest.mark.parametrize("over,code", [
    (dict(n=65, channels=512, spatial=65536, groups=32), b.QKR_ERR_SCRATCH),
    (dict(dtype=b.QKR_FP32), b.QKR_ERR_UNSUPPORTED),
    (dict(param_dtype=7), b.QKR_ERR_ARG),
    (dict(eps=0.0), b.QKR_ERR_ARG),
    (dict(channels=63), b.QKR_ERR_SHAPE),
    (dict(spatial=12), b.QKR_ERR_UNSUPPORTED),
    (dict(x=0), b.QKR_ERR_NULL),
    (dict(y=MIS), b.QKR_ERR_ALIGN),
    (dict(n=0), b.QKR_OK),
])
def test_group_norm_noalloc_checks_before_any_hip_call(over, code):
    """The entry point without workspace rejects, before any HIP call, what
    dit_group_norm_silu rejects, and a call whose workspace would exceed the
    fixed scratch (65 x 32 groups of 64 chunks: 1 MiB + 64 KiB)."""
    assert gn_noalloc(**over) == code


def test_group_norm_noalloc_scratch_limit():
    """The largest workspace the fixed scratch takes is 1 MiB: 131,072 chunk
    words of 8 bytes, one more chunk is refused."""
    assert b.GN_NOALLOC_WORKSPACE_MAX == 1 << 20
    assert qkr.group_norm_silu_workspace_size(64, 512, 65536, 32) == 1 << 20
    assert qkr.group_norm_silu_workspace_size(65, 512, 65536, 32) > 1 << 20
    assert "scratch" in qkr.strerror(b.QKR_ERR_SCRATCH)
