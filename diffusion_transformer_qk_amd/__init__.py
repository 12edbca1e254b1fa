"""Fused diffusion-transformer QK-norm + RoPE (with the AdaLN modulation and the
VAE group norm + SiLU steps) for AMD Instinct MI355X (gfx950).

The passes run in hand-written HIP kernels behind the C ABI of
``include/qknorm_rope.h``, ``include/fuse_scale_shift.h`` and
``include/group_norm_silu.h``
(``libqknorm_rope.so``); this package is the thin Python binding over it.
"""
from .binding import (  # noqa: F401
    EXPORTS, LIB_PATH, QkrError, dit_fuse_scale_shift_raw, dit_group_norm_silu_noalloc_raw,
    dit_group_norm_silu_raw,
    fuse_scale_shift, group_norm_silu, group_norm_silu_schedule,
    group_norm_silu_workspace_size, kernel_info,
    load_library, qknorm_rope_fused, qknorm_rope_fused_raw, strerror, version,
)

__all__ = ["qknorm_rope_fused", "qknorm_rope_fused_raw", "fuse_scale_shift",
           "dit_fuse_scale_shift_raw", "group_norm_silu", "group_norm_silu_schedule",
           "group_norm_silu_workspace_size",
           "dit_group_norm_silu_raw", "dit_group_norm_silu_noalloc_raw", "kernel_info",
           "load_library", "strerror", "version",
           "QkrError", "EXPORTS", "LIB_PATH"]
