"""ctypes access to the library's test-only entry point dit_group_norm_silu_polls
(declared in tests/c_abi/gn_test_hooks.h): dit_group_norm_silu with the
lagged schedule's polls per unpublished chunk word chosen by the test."""
import ctypes

from diffusion_transformer_qk_amd import binding as b

MAX_POLLS = 4096


def _fn():
    lib = b.load_library()
    fn = lib.dit_group_norm_silu_polls
    vp, i64, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32
    fn.argtypes = [vp, vp, i64, i32, i64, i32, vp, vp, i32, ctypes.c_float, i32, vp, i64, vp, i32]
    fn.restype = ctypes.c_int
    return fn


def polls_raw(x, y, n, channels, spatial, groups, gamma, beta, param_dtype, eps, dtype,
              workspace, workspace_bytes, stream, wait_polls) -> int:
    """The entry point with integer pointers; returns the raw status."""
    return int(_fn()(x or None, y or None, n, channels, spatial, groups, gamma or None,
                     beta or None, param_dtype, eps, dtype, workspace or None, workspace_bytes,
                     stream or None, wait_polls))


def group_norm_silu_polls(x, gamma, beta, groups, wait_polls, *, out=None, eps=1e-6):
    """b.group_norm_silu on the current stream, with `wait_polls` polls."""
    import torch

    n, channels = x.shape[0], x.shape[1]
    spatial = x[0, 0].numel()
    need = b.group_norm_silu_workspace_size(n, channels, spatial, groups)
    assert need >= 0
    ws = torch.empty(max(need, 16), dtype=torch.uint8, device=x.device)
    if out is None:
        out = torch.empty_like(x)
    stream = torch.cuda.current_stream(x.device).cuda_stream
    status = polls_raw(x.data_ptr(), out.data_ptr(), n, channels, spatial, groups,
                       gamma.data_ptr(), beta.data_ptr(), b._mod_code(gamma), float(eps),
                       b._x_code(x), ws.data_ptr(), ws.numel(), stream, wait_polls)
    if status != b.QKR_OK:
        raise b.QkrError(status, b.strerror(status))
    return out
