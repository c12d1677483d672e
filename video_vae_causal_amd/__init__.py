"""libwvc: the causal video-VAE hot path (causal 3x3x3 Conv3D with a rolling
past-frame cache, channel RMS norm + SiLU, residual block, the encoder's
downsampling convs, tiled decoding, and an 8-bit E4M3 variant) for MI355X (gfx950).

The compute runs in hand-written HIP kernels behind the C ABI in
include/wvc.h; this package is the ctypes binding (``_lib``), the streaming
cache manager (``stream``), the seeded input generator (``inputs``) and the
FLOP/byte accounting (``accounting``).  Importing the package does not load
the library; the first call does, and raises if libwvc.so was not built.
"""
from ._lib import (  # noqa: F401
    WVC_BF16, WVC_E4M3, WVC_F32, WvcError, empty_cl, load, wvc_cache_reset,
    wvc_causal_conv3d_e4m3_fwd, wvc_causal_conv3d_fwd, wvc_conv3d_cache_frames,
    wvc_conv3d_pack_weights, wvc_get_counters, wvc_get_strict, wvc_last_error,
    wvc_quantize_e4m3, wvc_quantize_rows_e4m3, wvc_reset_counters, wvc_resblock_back,
    wvc_resblock_e4m3_fwd, wvc_resblock_front, wvc_resblock_fwd, wvc_rmsnorm_silu,
    wvc_rmsnorm_silu_conv3d_fwd, wvc_rmsnorm_silu_e4m3, wvc_set_strict, wvc_tile_blend,
    wvc_tile_blend_finish, wvc_tile_extract, wvc_upsample_nearest2x, wvc_version,
)

__all__ = [n for n in dir() if n.startswith("wvc_")] + ["WvcError", "empty_cl", "load"]
