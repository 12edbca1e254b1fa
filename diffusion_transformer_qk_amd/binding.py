"""ctypes binding of ``libqknorm_rope.so`` (argument marshalling only).

Every step runs in the HIP kernels behind the C ABI declared in
``include/qknorm_rope.h`` (fused QK-norm + RoPE), ``include/fuse_scale_shift.h``
(AdaLN modulation) and ``include/group_norm_silu.h`` (group norm + SiLU);
this module turns torch
tensors into device pointers, sizes and enum codes and raises on a non-zero
status.  There is no fallback: if the library is missing, loading fails
loudly.
"""
from __future__ import annotations

import contextlib
import ctypes
import os

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libqknorm_rope.so")

QKR_OK = 0
QKR_ERR_NULL, QKR_ERR_SHAPE, QKR_ERR_ALIGN = -1, -2, -3
QKR_ERR_UNSUPPORTED, QKR_ERR_MODE, QKR_ERR_HIP, QKR_ERR_ARG = -4, -5, -6, -7
QKR_ERR_WORKSPACE = -8
QKR_ERR_SCRATCH = -9
GN_NOALLOC_WORKSPACE_MAX = 1 << 20
QKR_BF16, QKR_FP16, QKR_FP32 = 0, 1, 2
QKR_COS_SHARED, QKR_COS_PER_HEAD = 0, 1
QKR_ROPE_INTERLEAVED, QKR_ROPE_ROTATE_HALF = 0, 1
QKR_TENSORS_FUSED, QKR_TENSORS_PAIR, QKR_TENSORS_ONE = 0, 1, 2

LAYOUTS = {"shared": QKR_COS_SHARED, "per_head": QKR_COS_PER_HEAD}
STYLES = {"interleaved": QKR_ROPE_INTERLEAVED, "rotate_half": QKR_ROPE_ROTATE_HALF}
TENSORS = {"fused": QKR_TENSORS_FUSED, "pair": QKR_TENSORS_PAIR, "one": QKR_TENSORS_ONE}
EXPORTS = ("qknorm_rope_fused", "qknorm_rope_strerror", "qknorm_rope_version",
           "qknorm_rope_kernel_info", "dit_fuse_scale_shift",
           "dit_group_norm_silu_workspace_size", "dit_group_norm_silu_schedule",
           "dit_group_norm_silu", "dit_group_norm_silu_noalloc")
MOD_DTYPES = {"bf16": QKR_BF16, "fp16": QKR_FP16, "fp32": QKR_FP32}


class QkrError(RuntimeError):
    """A non-zero status from the library."""

    def __init__(self, status: int, message: str):
        super().__init__("qknorm_rope: %s (status %d)" % (message, status))
        self.status = status


class KernelInfo(ctypes.Structure):
    _fields_ = [("num_vgprs", ctypes.c_int32), ("lds_bytes", ctypes.c_int32),
                ("scratch_bytes", ctypes.c_int32), ("block_threads", ctypes.c_int32),
                ("tokens_per_block", ctypes.c_int32), ("heads_in_flight", ctypes.c_int32),
                ("die_runs", ctypes.c_int32), ("dynamic_lds_bytes", ctypes.c_int32),
                ("workgroups_per_cu", ctypes.c_int32)]


_lib = None


def load_library(path: str = LIB_PATH):
    """Load the HIP library (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(
            "libqknorm_rope.so is not built (%s); run __graft_entry__.build() or "
            "python -m diffusion_transformer_qk_amd.build" % path)
    # torch first: it carries its own HIP runtime, and the library's HIP
    # dependency must resolve to that one.  Loaded the other way round, the
    # process holds two runtimes and the library's sees no device.
    try:
        import torch  # noqa: F401
    except ImportError:
        pass
    lib = ctypes.CDLL(path)
    vp, i64, i32, f32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_float
    lib.qknorm_rope_fused.argtypes = [vp, vp, vp, i64, i32, i32, vp, vp, f32, vp, vp,
                                      i32, i32, i32, i32, vp]
    lib.qknorm_rope_fused.restype = ctypes.c_int
    lib.qknorm_rope_strerror.argtypes = [ctypes.c_int]
    lib.qknorm_rope_strerror.restype = ctypes.c_char_p
    lib.qknorm_rope_version.argtypes = []
    lib.qknorm_rope_version.restype = ctypes.c_int
    lib.qknorm_rope_kernel_info.argtypes = [i32, i32, i64, i32, i32, i32, i32, i32,
                                            ctypes.POINTER(KernelInfo)]
    lib.qknorm_rope_kernel_info.restype = ctypes.c_int
    lib.dit_fuse_scale_shift.argtypes = [vp, vp, i64, i32, i64, vp, vp, i32, f32, i32, vp]
    lib.dit_fuse_scale_shift.restype = ctypes.c_int
    lib.dit_group_norm_silu_workspace_size.argtypes = [i64, i32, i64, i32]
    lib.dit_group_norm_silu_workspace_size.restype = i64
    lib.dit_group_norm_silu_schedule.argtypes = [i64, i32, i64, i32, ctypes.POINTER(i64)]
    lib.dit_group_norm_silu_schedule.restype = i32
    lib.dit_group_norm_silu.argtypes = [vp, vp, i64, i32, i64, i32, vp, vp, i32, f32, i32, vp, i64,
                                        vp]
    lib.dit_group_norm_silu.restype = ctypes.c_int
    lib.dit_group_norm_silu_noalloc.argtypes = [vp, vp, i64, i32, i64, i32, vp, vp, i32, f32,
                                                i32, vp]
    lib.dit_group_norm_silu_noalloc.restype = ctypes.c_int
    _lib = lib
    return lib


def strerror(status: int) -> str:
    return load_library().qknorm_rope_strerror(status).decode()


def version() -> int:
    return int(load_library().qknorm_rope_version())


def _check(status: int):
    if status != QKR_OK:
        raise QkrError(status, strerror(status))


def qknorm_rope_fused_raw(qkv: int, q: int, k: int, tokens: int, heads: int, head_dim: int,
                          q_gamma: int, k_gamma: int, eps: float, cos: int, sin: int,
                          cos_layout: int, cos_dtype: int, style: int, dtype: int,
                          stream: int) -> int:
    """The C entry point with integer pointers; returns the raw status."""
    lib = load_library()
    return int(lib.qknorm_rope_fused(qkv or None, q or None, k or None, tokens, heads, head_dim,
                                     q_gamma or None, k_gamma or None, eps, cos or None,
                                     sin or None, cos_layout, cos_dtype, style, dtype,
                                     stream or None))


def _torch():
    import torch
    return torch


def _x_code(t) -> int:
    torch = _torch()
    if t.dtype == torch.bfloat16:
        return QKR_BF16
    if t.dtype == torch.float16:
        return QKR_FP16
    raise ValueError("q/k/qkv must be bfloat16 or float16, got %s" % t.dtype)


def _table_code(t) -> int:
    torch = _torch()
    if t.dtype == torch.float32:
        return QKR_FP32
    if t.dtype == torch.bfloat16:
        return QKR_BF16
    raise ValueError("cos/sin must be float32 or bfloat16, got %s" % t.dtype)


def _ptr(t) -> int:
    if t is None:
        return 0
    if not t.is_contiguous():
        raise ValueError("tensors must be contiguous")
    if not t.is_cuda:
        raise ValueError("tensors must live on the GPU")
    return t.data_ptr()


def _call_context(ref, tensors, stream):
    """(device context, raw hipStream_t) for a call on ``ref``'s device.

    Every tensor given must live on that device; the call runs with it as the
    current device, so a NULL (default) stream means that device's.
    """
    torch = _torch()
    dev = ref.device
    for t in tensors:
        if t is not None and t.device != dev:
            raise ValueError("all tensors must be on one device (%s)" % dev)
    if stream is None:
        raw = torch.cuda.current_stream(dev).cuda_stream if ref.is_cuda else 0
    elif isinstance(stream, int):
        raw = stream
    else:
        raw = stream.cuda_stream
    # switching the current device costs a few µs per call: only when needed
    if ref.is_cuda and dev.index != torch.cuda.current_device():
        return torch.cuda.device(dev), raw
    return contextlib.nullcontext(), raw


def _launch_stream_context(ref, stream):
    """Context in which tensors the binding allocates for a call belong to the
    stream the call is launched on, so that the caching allocator hands their
    memory to other work only in that stream's order (memory allocated on the
    current stream and freed on return could be reused by the current stream
    while the launch stream still uses it)."""
    torch = _torch()
    if stream is None or not ref.is_cuda:
        return contextlib.nullcontext()
    if isinstance(stream, int):
        if stream == torch.cuda.current_stream(ref.device).cuda_stream:
            return contextlib.nullcontext()
        stream = torch.cuda.ExternalStream(stream, device=ref.device)
    return torch.cuda.stream(stream)


def qknorm_rope_fused(qkv=None, q=None, k=None, *, q_gamma=None, k_gamma=None,
                      cos=None, sin=None, eps: float = 1e-6, heads: int | None = None,
                      head_dim: int | None = None, cos_layout: str = "shared",
                      style: str = "interleaved", stream=None) -> None:
    """Apply the fused QK-norm + RoPE in place (see ``include/qknorm_rope.h``).

    Fused mode: ``qkv`` is [tokens, 3*heads*head_dim] (any leading shape whose
    last dimension is 3*heads*head_dim); ``head_dim`` defaults to the gamma
    length and ``heads`` to last_dim / (3*head_dim).
    Separate mode: ``q`` and/or ``k`` are [..., heads, head_dim].
    ``cos``/``sin``: [tokens, head_dim] ("shared") or [tokens, heads, head_dim]
    ("per_head"), float32 or bfloat16.  ``stream``: a torch stream or a raw
    hipStream_t integer; defaults to the current stream.
    """
    torch = _torch()
    if qkv is not None:
        ref = qkv
        gam = q_gamma if q_gamma is not None else k_gamma
        if head_dim is None:
            if gam is None:
                raise ValueError("head_dim is needed")
            head_dim = gam.numel()
        if heads is None:
            heads = qkv.shape[-1] // (3 * head_dim)
        if qkv.shape[-1] != 3 * heads * head_dim:
            raise ValueError("qkv last dimension must be 3*heads*head_dim")
        tokens = qkv.numel() // qkv.shape[-1] if qkv.numel() else 0
    else:
        ref = q if q is not None else k
        if ref is None:
            raise ValueError("pass qkv, or q and/or k")
        if ref.dim() < 2:
            raise ValueError("q/k must be [..., heads, head_dim]")
        head_dim = ref.shape[-1] if head_dim is None else head_dim
        heads = ref.shape[-2] if heads is None else heads
        if tuple(ref.shape[-2:]) != (heads, head_dim):
            raise ValueError("q/k must be [..., heads, head_dim] = [..., %d, %d]"
                             % (heads, head_dim))
        tokens = ref.numel() // (heads * head_dim) if ref.numel() else 0
        if q is not None and k is not None and (q.shape != k.shape or q.dtype != k.dtype):
            raise ValueError("q and k must have the same shape and dtype")
    if cos_layout not in LAYOUTS:
        raise ValueError("cos_layout must be one of %s" % sorted(LAYOUTS))
    if style not in STYLES:
        raise ValueError("style must be one of %s" % sorted(STYLES))
    if cos is None or sin is None:
        raise ValueError("cos and sin are required")
    if cos.dtype != sin.dtype or cos.shape != sin.shape:
        raise ValueError("cos and sin must match in shape and dtype")
    rows = tokens * (heads if cos_layout == "per_head" else 1)
    if cos.numel() != rows * head_dim:
        raise ValueError("cos/sin hold %d values, expected %d for the %s layout"
                         % (cos.numel(), rows * head_dim, cos_layout))
    for g in (q_gamma, k_gamma):
        if g is not None and (g.dtype != torch.float32 or g.numel() != head_dim):
            raise ValueError("gamma must be float32 [head_dim]")
    ctx, stream_ptr = _call_context(ref, (qkv, q, k, q_gamma, k_gamma, cos, sin), stream)
    with ctx:
        status = qknorm_rope_fused_raw(
            _ptr(qkv), _ptr(q), _ptr(k), tokens, heads, head_dim, _ptr(q_gamma), _ptr(k_gamma),
            float(eps), _ptr(cos), _ptr(sin), LAYOUTS[cos_layout], _table_code(cos),
            STYLES[style], _x_code(ref), stream_ptr)
    _check(status)


def kernel_info(head_dim: int = 128, cos_layout: str = "shared", cos_dtype: int = QKR_FP32,
                style: str = "interleaved", dtype: int = QKR_BF16, heads: int = 40,
                tokens: int = 32760, tensors: str = "fused") -> dict:
    """Registers, LDS, scratch and schedule of the kernel a call launches.

    ``tensors``: "fused" (one QKV buffer), "pair" (separate q and k) or "one"
    (q or k alone).
    """
    info = KernelInfo()
    _check(load_library().qknorm_rope_kernel_info(head_dim, heads, tokens, TENSORS[tensors],
                                                  LAYOUTS[cos_layout], cos_dtype, STYLES[style],
                                                  dtype, ctypes.byref(info)))
    return {name: getattr(info, name) for name, _ in KernelInfo._fields_}


def dit_fuse_scale_shift_raw(x: int, y: int, rows: int, hidden: int, rows_per_batch: int,
                             scale: int, shift: int, mod_dtype: int, eps: float, dtype: int,
                             stream: int) -> int:
    """The AdaLN C entry point with integer pointers; returns the raw status."""
    lib = load_library()
    return int(lib.dit_fuse_scale_shift(x or None, y or None, rows, hidden, rows_per_batch,
                                        scale or None, shift or None, mod_dtype, eps, dtype,
                                        stream or None))


def _mod_code(t) -> int:
    torch = _torch()
    codes = {torch.bfloat16: QKR_BF16, torch.float16: QKR_FP16, torch.float32: QKR_FP32}
    if t.dtype not in codes:
        raise ValueError("scale/shift must be bfloat16, float16 or float32, got %s" % t.dtype)
    return codes[t.dtype]


def fuse_scale_shift(x, scale, shift, *, out=None, eps: float = 1e-6,
                     rows_per_batch: int | None = None, stream=None):
    """AdaLN modulation (see ``include/fuse_scale_shift.h``); returns ``out``.

    ``x``: [..., hidden] bfloat16/float16; ``scale``/``shift``: [batches, hidden]
    (or [hidden] for one batch) of bfloat16, float16 or float32.  Row r of the
    flattened x uses modulation row r // rows_per_batch; by default the rows
    split evenly over the batches.  ``out`` defaults to a new tensor like x;
    pass ``out=x`` to modulate in place.
    """
    torch = _torch()
    hidden = x.shape[-1]
    rows = x.numel() // hidden if x.numel() else 0
    if scale.shape != shift.shape or scale.dtype != shift.dtype:
        raise ValueError("scale and shift must match in shape and dtype")
    if scale.shape[-1] != hidden:
        raise ValueError("scale/shift last dimension must equal hidden")
    batches = scale.numel() // hidden
    if rows_per_batch is None:
        if batches < 1 or rows % batches:
            raise ValueError("rows do not split evenly over the modulation batches")
        rows_per_batch = max(1, rows // batches)
    if rows and (rows - 1) // rows_per_batch >= batches:
        raise ValueError("scale/shift hold fewer batches than the rows need")
    if out is None:
        with _launch_stream_context(x, stream):
            out = torch.empty_like(x)
    elif out.shape != x.shape or out.dtype != x.dtype:
        raise ValueError("out must match x in shape and dtype")
    ctx, stream_ptr = _call_context(x, (out, scale, shift), stream)
    with ctx:
        status = dit_fuse_scale_shift_raw(_ptr(x), _ptr(out), rows, hidden, rows_per_batch,
                                          _ptr(scale), _ptr(shift), _mod_code(scale), float(eps),
                                          _x_code(x), stream_ptr)
    _check(status)
    return out


def group_norm_silu_workspace_size(n: int, channels: int, spatial: int, groups: int) -> int:
    """Workspace bytes the call needs (negative: a QKR_ERR_* code for bad sizes)."""
    return int(load_library().dit_group_norm_silu_workspace_size(n, channels, spatial, groups))


GN_SCHEDULES = {0: "one_read", 1: "lagged", 2: "two_pass"}


def group_norm_silu_schedule(n: int, channels: int, spatial: int, groups: int):
    """(schedule name, elements per chunk) the library would use for these
    sizes: "one_read", "lagged" or "two_pass" (see include/group_norm_silu.h)."""
    chunk = ctypes.c_int64(0)
    code = int(load_library().dit_group_norm_silu_schedule(n, channels, spatial, groups,
                                                           ctypes.byref(chunk)))
    if code < 0:
        raise QkrError(code, strerror(code))
    return GN_SCHEDULES[code], int(chunk.value)


def dit_group_norm_silu_raw(x: int, y: int, n: int, channels: int, spatial: int, groups: int,
                            gamma: int, beta: int, param_dtype: int, eps: float, dtype: int,
                            workspace: int, workspace_bytes: int, stream: int) -> int:
    """The group-norm C entry point with integer pointers; returns the raw status."""
    lib = load_library()
    return int(lib.dit_group_norm_silu(x or None, y or None, n, channels, spatial, groups,
                                       gamma or None, beta or None, param_dtype, eps, dtype,
                                       workspace or None, workspace_bytes, stream or None))


def dit_group_norm_silu_noalloc_raw(x: int, y: int, n: int, channels: int, spatial: int,
                                    groups: int, gamma: int, beta: int, param_dtype: int,
                                    eps: float, dtype: int, stream: int) -> int:
    """The group-norm entry point that allocates nothing (its workspace is the
    library's fixed per-GPU scratch), with integer pointers; returns the raw
    status."""
    lib = load_library()
    return int(lib.dit_group_norm_silu_noalloc(x or None, y or None, n, channels, spatial, groups,
                                               gamma or None, beta or None, param_dtype, eps,
                                               dtype, stream or None))


def group_norm_silu(x, gamma, beta, groups: int, *, out=None, eps: float = 1e-6,
                    workspace=None, stream=None):
    """Group norm + affine + SiLU (see ``include/group_norm_silu.h``); returns ``out``.

    ``x``: [n, channels, *spatial] bfloat16/float16 (spatial dims flattened,
    their product a multiple of 8).  ``gamma``/``beta``: [channels].
    ``workspace``: a device tensor of at least the queried size; when None and
    one is needed, a byte tensor is allocated here with torch (the library
    itself never allocates), on the launch stream, so its memory is not reused
    before the call's kernels are done with it.  ``out`` defaults to a new
    tensor (also on the launch stream); ``out=x`` works in place.
    """
    torch = _torch()
    if x.dim() < 3:
        raise ValueError("x must be [n, channels, *spatial]")
    n, channels = x.shape[0], x.shape[1]
    spatial = 1
    for d in x.shape[2:]:
        spatial *= d
    if gamma.shape != (channels,) or beta.shape != (channels,) or gamma.dtype != beta.dtype:
        raise ValueError("gamma and beta must be [channels] of one dtype")
    need = group_norm_silu_workspace_size(n, channels, spatial, groups) if x.numel() else 0
    if need < 0:
        raise QkrError(need, strerror(need))
    with _launch_stream_context(x, stream):
        if workspace is None and need > 0:
            workspace = torch.empty(need, dtype=torch.uint8, device=x.device)
        if out is None:
            out = torch.empty_like(x)
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    if out.shape != x.shape or out.dtype != x.dtype:
        raise ValueError("out must match x in shape and dtype")
    ctx, stream_ptr = _call_context(x, (out, gamma, beta, workspace), stream)
    with ctx:
        status = dit_group_norm_silu_raw(_ptr(x), _ptr(out), n, channels, spatial, groups,
                                         _ptr(gamma), _ptr(beta), _mod_code(gamma), float(eps),
                                         _x_code(x), _ptr(workspace), ws_bytes, stream_ptr)
    _check(status)
    return out
