"""ctypes binding of libwvc (include/wvc.h).

Argument marshalling only: every step of the path runs in the library's HIP
kernels.  PyTorch supplies device memory and the current HIP stream.  Tensors
use the logical NCTHW shapes with PyTorch's channels_last_3d memory format
(physical N,T,H,W,C), which is what the library expects; weights are
[C_out, C_in, kT, kH, kW] in channels_last_3d (physical C_out,kT,kH,kW,C_in).

There is no fallback: if libwvc.so is missing or fails to load, every entry
point raises.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libwvc.so")

WVC_OK, WVC_ERR_ARG, WVC_ERR_UNSUPPORTED, WVC_ERR_ALIAS, WVC_ERR_WORKSPACE, WVC_ERR_STRICT, \
    WVC_ERR_HIP = range(7)
WVC_F32, WVC_BF16, WVC_E4M3 = 0, 1, 2
WVC_WEIGHT_STANDARD, WVC_WEIGHT_PACKED = 0, 1
WVC_NOALLOC_SCRATCH_MIB = 48  # include/wvc.h: scratch array of the allocation-free conv call
ERROR_NAMES = {0: "WVC_OK", 1: "WVC_ERR_ARG", 2: "WVC_ERR_UNSUPPORTED", 3: "WVC_ERR_ALIAS",
               4: "WVC_ERR_WORKSPACE", 5: "WVC_ERR_STRICT", 6: "WVC_ERR_HIP"}

# Every symbol include/wvc.h declares.
EXPORTED = (
    "wvc_causal_conv3d_fwd", "wvc_causal_conv3d_workspace_bytes", "wvc_conv3d_cache_frames",
    "wvc_conv3d_packed_weight_bytes", "wvc_conv3d_pack_weights",
    "wvc_rmsnorm_silu", "wvc_resblock_fwd", "wvc_resblock_workspace_bytes",
    "wvc_resblock_front", "wvc_resblock_back", "wvc_cache_reset",
    "wvc_upsample_nearest2x", "wvc_set_strict", "wvc_get_strict", "wvc_get_counters",
    "wvc_reset_counters", "wvc_last_error", "wvc_version", "wvc_graph_capture_begin",
    "wvc_graph_capture_end", "wvc_graph_launch", "wvc_graph_destroy",
    "wvc_tile_extract", "wvc_tile_blend", "wvc_tile_blend_finish",
    "wvc_causal_conv3d_e4m3_fwd", "wvc_quantize_e4m3", "wvc_quantize_rows_e4m3",
    "wvc_rmsnorm_silu_e4m3", "wvc_rmsnorm_silu_conv3d_fwd", "wvc_resblock_e4m3_fwd",
    "wvc_resblock_e4m3_workspace_bytes", "wvc_conv3d_kernel_name", "wvc_causal_conv3d_fwd_noalloc",
    "wvc_causal_conv3d_norm_fwd", "wvc_causal_conv3d_norm_workspace_bytes",
    "wvc_causal_conv3d_e4m3_norm_fwd", "wvc_causal_conv3d_e4m3_norm_workspace_bytes",
)


class ConvDesc(ctypes.Structure):
    _fields_ = [(f, ctypes.c_int) for f in (
        "n", "c_in", "c_out", "t", "h", "w", "kt", "kh", "kw", "stride_t", "stride_h",
        "stride_w", "pad_h", "pad_w", "dil_t", "dil_h", "dil_w", "groups", "dtype",
        "weight_layout", "pad_h_extra", "pad_w_extra", "t_phase", "upsample_in", "cu_limit")]


class ResblockDesc(ctypes.Structure):
    _fields_ = [(f, ctypes.c_int) for f in ("n", "c_in", "c_out", "t", "h", "w", "dtype")] + \
        [("eps", ctypes.c_float), ("weights_packed", ctypes.c_int), ("cu_limit", ctypes.c_int)]


class ResblockParams(ctypes.Structure):
    _fields_ = [(f, ctypes.c_void_p) for f in (
        "gamma1", "beta1", "w1", "b1", "gamma2", "beta2", "w2", "b2", "w_short", "b_short")]


class ResblockE4M3Params(ctypes.Structure):
    _fields_ = [("gamma1", ctypes.c_void_p), ("beta1", ctypes.c_void_p), ("w1", ctypes.c_void_p),
                ("w1_scale", ctypes.c_void_p), ("b1", ctypes.c_void_p), ("gamma2", ctypes.c_void_p),
                ("beta2", ctypes.c_void_p), ("w2", ctypes.c_void_p), ("w2_scale", ctypes.c_void_p),
                ("b2", ctypes.c_void_p), ("s1", ctypes.c_float), ("s2", ctypes.c_float)]


class Counters(ctypes.Structure):
    _fields_ = [(f, ctypes.c_uint64) for f in ("fast_3x3x3", "fast_1x1x1", "generic", "rejected",
                                               "fast_strided")]


class WvcError(RuntimeError):
    def __init__(self, code: int, text: str):
        super().__init__(f"{ERROR_NAMES.get(code, code)}: {text}")
        self.code = code


_lib = None
# Device type every tensor argument must live on (the library takes device
# pointers only).
DEVICE_TYPE = "cuda"


def _on_device(t: torch.Tensor) -> bool:
    return t.device.type == DEVICE_TYPE


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libwvc.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise ImportError(f"{path} is missing: build it with __graft_entry__.build() "
                          "(hipcc, gfx950); there is no fallback path")
    lib = ctypes.CDLL(path)
    vp, sz, i, f = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int, ctypes.c_float
    dptr = ctypes.POINTER(ConvDesc)
    lib.wvc_causal_conv3d_fwd.argtypes = [dptr, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.wvc_causal_conv3d_fwd.restype = i
    lib.wvc_causal_conv3d_fwd_noalloc.argtypes = [dptr, vp, vp, vp, vp, vp, vp, vp, vp]
    lib.wvc_causal_conv3d_fwd_noalloc.restype = i
    lib.wvc_causal_conv3d_workspace_bytes.argtypes = [dptr]
    lib.wvc_causal_conv3d_workspace_bytes.restype = sz
    lib.wvc_causal_conv3d_norm_fwd.argtypes = [dptr, vp, vp, vp, vp, vp, vp, vp, vp, vp,
                                               ctypes.c_float, vp, vp, sz, vp]
    lib.wvc_causal_conv3d_norm_fwd.restype = i
    lib.wvc_causal_conv3d_norm_workspace_bytes.argtypes = [dptr]
    lib.wvc_causal_conv3d_norm_workspace_bytes.restype = sz
    lib.wvc_conv3d_kernel_name.argtypes = [dptr]
    lib.wvc_conv3d_kernel_name.restype = ctypes.c_char_p
    lib.wvc_conv3d_cache_frames.argtypes = [dptr]
    lib.wvc_conv3d_cache_frames.restype = i
    lib.wvc_conv3d_packed_weight_bytes.argtypes = [dptr]
    lib.wvc_conv3d_packed_weight_bytes.restype = sz
    lib.wvc_conv3d_pack_weights.argtypes = [dptr, vp, vp, vp]
    lib.wvc_conv3d_pack_weights.restype = i
    lib.wvc_rmsnorm_silu.argtypes = [vp, vp, vp, vp, i, i, i, i, i, i, f, i, vp]
    lib.wvc_rmsnorm_silu.restype = i
    lib.wvc_resblock_fwd.argtypes = [ctypes.POINTER(ResblockDesc), vp, vp,
                                     ctypes.POINTER(ResblockParams), vp, vp, vp, vp, vp, sz, vp]
    lib.wvc_resblock_fwd.restype = i
    lib.wvc_resblock_front.argtypes = [ctypes.POINTER(ResblockDesc), vp, vp,
                                       ctypes.POINTER(ResblockParams), vp, vp, vp, sz, vp]
    lib.wvc_resblock_front.restype = i
    lib.wvc_resblock_back.argtypes = [ctypes.POINTER(ResblockDesc), vp, vp, vp,
                                      ctypes.POINTER(ResblockParams), vp, vp, vp, sz, vp]
    lib.wvc_resblock_back.restype = i
    lib.wvc_resblock_workspace_bytes.argtypes = [ctypes.POINTER(ResblockDesc)]
    lib.wvc_resblock_workspace_bytes.restype = sz
    lib.wvc_cache_reset.argtypes = [vp, sz, vp]
    lib.wvc_cache_reset.restype = i
    lib.wvc_upsample_nearest2x.argtypes = [vp, vp, i, i, i, i, i, i, vp]
    lib.wvc_upsample_nearest2x.restype = i
    lib.wvc_set_strict.argtypes = [i]
    lib.wvc_set_strict.restype = None
    lib.wvc_get_strict.argtypes = []
    lib.wvc_get_strict.restype = i
    lib.wvc_get_counters.argtypes = [ctypes.POINTER(Counters)]
    lib.wvc_get_counters.restype = None
    lib.wvc_reset_counters.argtypes = []
    lib.wvc_reset_counters.restype = None
    lib.wvc_last_error.argtypes = []
    lib.wvc_last_error.restype = ctypes.c_char_p
    lib.wvc_version.argtypes = []
    lib.wvc_version.restype = ctypes.c_char_p
    lib.wvc_tile_extract.argtypes = [vp, vp] + [i] * 10 + [vp]
    lib.wvc_tile_extract.restype = i
    lib.wvc_tile_blend.argtypes = [vp, vp, vp] + [i] * 14 + [vp]
    lib.wvc_tile_blend.restype = i
    lib.wvc_tile_blend_finish.argtypes = [vp, vp, vp] + [i] * 6 + [vp]
    lib.wvc_tile_blend_finish.restype = i
    lib.wvc_graph_capture_begin.argtypes = [vp]
    lib.wvc_graph_capture_begin.restype = i
    lib.wvc_graph_capture_end.argtypes = [vp, ctypes.POINTER(vp)]
    lib.wvc_graph_capture_end.restype = i
    lib.wvc_graph_launch.argtypes = [vp, vp]
    lib.wvc_graph_launch.restype = i
    lib.wvc_graph_destroy.argtypes = [vp]
    lib.wvc_graph_destroy.restype = i
    lib.wvc_resblock_e4m3_fwd.argtypes = [ctypes.POINTER(ResblockDesc), vp, vp,
                                          ctypes.POINTER(ResblockE4M3Params), vp, vp, vp, vp, vp, sz, vp]
    lib.wvc_resblock_e4m3_fwd.restype = i
    lib.wvc_resblock_e4m3_workspace_bytes.argtypes = [ctypes.POINTER(ResblockDesc)]
    lib.wvc_resblock_e4m3_workspace_bytes.restype = sz
    lib.wvc_rmsnorm_silu_conv3d_fwd.argtypes = [dptr, vp, vp, vp, f, vp, vp, vp, vp, vp, sz, vp]
    lib.wvc_rmsnorm_silu_conv3d_fwd.restype = i
    lib.wvc_causal_conv3d_e4m3_fwd.argtypes = [dptr, vp, f, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.wvc_causal_conv3d_e4m3_fwd.restype = i
    lib.wvc_causal_conv3d_e4m3_norm_fwd.argtypes = [dptr, vp, f, vp, vp, vp, vp, vp, vp, vp, vp, vp, f,
                                                    f, vp, vp, sz, vp]
    lib.wvc_causal_conv3d_e4m3_norm_fwd.restype = i
    lib.wvc_causal_conv3d_e4m3_norm_workspace_bytes.argtypes = [dptr]
    lib.wvc_causal_conv3d_e4m3_norm_workspace_bytes.restype = sz
    i64 = ctypes.c_int64
    lib.wvc_quantize_e4m3.argtypes = [vp, i, i64, f, vp, vp]
    lib.wvc_quantize_e4m3.restype = i
    lib.wvc_quantize_rows_e4m3.argtypes = [vp, i, i64, i64, vp, vp, vp]
    lib.wvc_quantize_rows_e4m3.restype = i
    lib.wvc_rmsnorm_silu_e4m3.argtypes = [vp, vp, vp, vp, i, i, i, i, i, f, i, f, vp]
    lib.wvc_rmsnorm_silu_e4m3.restype = i
    _lib = lib
    return lib


def _check(rc: int):
    if rc != WVC_OK:
        raise WvcError(rc, load().wvc_last_error().decode())


def _memo(fn):
    """Memoise a pure function of hashable arguments (sizes the library
    derives from a descriptor, descriptors themselves): a streamed layer asks
    the same questions on every chunk, and the per-call host time decides
    whether the host keeps ahead of the GPU."""
    cache = {}

    def wrapper(*args):
        try:
            return cache[args]
        except KeyError:
            pass
        v = fn(*args)
        if len(cache) >= 4096:
            cache.clear()
        cache[args] = v
        return v

    wrapper.cache = cache
    return wrapper


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(t: Optional[torch.Tensor] = None):
    dev = t.device if t is not None and t.is_cuda else None
    return ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)


def _dtype_code(dt: torch.dtype) -> int:
    if dt == torch.bfloat16:
        return WVC_BF16
    if dt == torch.float32:
        return WVC_F32
    if dt == torch.uint8:  # E4M3 codes
        return WVC_E4M3
    raise TypeError(f"unsupported dtype {dt}: bfloat16, float32 or uint8 (E4M3 codes)")


def _need_cl(t: Optional[torch.Tensor], name: str, ndim: int = 5):
    if t is None:
        return
    if not _on_device(t):
        raise ValueError(f"{name} must be a device tensor")
    if t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims, got {tuple(t.shape)}")
    if ndim == 5 and not t.is_contiguous(memory_format=torch.channels_last_3d):
        raise ValueError(f"{name} must be channels_last_3d contiguous")


def _need_vec(t: Optional[torch.Tensor], name: str, c: int):
    if t is None:
        return
    if not _on_device(t) or t.dim() != 1 or t.shape[0] != c or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous device vector of {c} elements")


def _need_exact(t: Optional[torch.Tensor], name: str, shape, dtype: torch.dtype,
                device: torch.device):
    """A buffer the library reads or writes at a size derived from other
    arguments: it must have exactly that shape, dtype and device (the C ABI
    gets a bare pointer and trusts the size), channels-last when 5-d."""
    if t is None:
        return
    if t.shape != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(int(v) for v in shape)}, "
                         f"got {tuple(t.shape)}")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if t.device != device:
        raise ValueError(f"{name} must be on {device}, got {t.device}")
    _need_cl(t, name, len(shape))
    if len(shape) == 1 and not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _need_bytes(t: Optional[torch.Tensor], name: str, nbytes: int, device: torch.device):
    """A flat buffer (packed weights) of exactly ``nbytes`` bytes on ``device``."""
    if t is None:
        return
    if not _on_device(t) or t.device != device or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous tensor on {device}")
    got = t.numel() * t.element_size()
    if got != nbytes:
        raise ValueError(f"{name} holds {got} bytes, {nbytes} expected")


def empty_cl(shape: Sequence[int], dtype=torch.bfloat16, device="cuda") -> torch.Tensor:
    """Uninitialised [N,C,T,H,W] tensor in channels_last_3d memory."""
    return torch.empty(tuple(shape), dtype=dtype, device=device,
                       memory_format=torch.channels_last_3d)


def conv_desc(x_shape, w_shape, dtype: int, stride=(1, 1, 1), padding=(1, 1),
              dilation=(1, 1, 1), groups: int = 1,
              weight_layout: int = WVC_WEIGHT_STANDARD, pad_extra=(0, 0),
              t_phase: int = 0, upsample_in: int = 0, cu_limit: int = 0) -> ConvDesc:
    """Descriptor of a conv over x of shape ``x_shape``.  With upsample_in = 2
    the conv reads x through a nearest 2x upsample: its frame (d.h, d.w) is
    twice x's.  cu_limit > 0 plans the grid for that many CUs."""
    n, c, t, h, w = x_shape
    co, ci, kt, kh, kw = w_shape
    up = 2 if upsample_in == 2 else 1
    d = ConvDesc()
    d.n, d.c_in, d.c_out, d.t, d.h, d.w = n, ci, co, t, h * up, w * up
    d.upsample_in = upsample_in
    d.cu_limit = cu_limit
    d.kt, d.kh, d.kw = kt, kh, kw
    d.stride_t, d.stride_h, d.stride_w = stride
    d.pad_h, d.pad_w = padding
    d.dil_t, d.dil_h, d.dil_w = dilation
    d.groups = groups
    d.dtype = dtype
    d.weight_layout = weight_layout
    d.pad_h_extra, d.pad_w_extra = pad_extra
    d.t_phase = t_phase
    return d


@_memo
def _conv_desc_shared(x_shape, w_shape, dtype, stride, padding, dilation, groups, layout,
                      pad_extra, t_phase, upsample_in=0, cu_limit=0) -> ConvDesc:
    """conv_desc for the binding's own calls, one object per argument tuple
    (read only: the library never writes a descriptor)."""
    return conv_desc(x_shape, w_shape, dtype, stride, padding, dilation, groups, layout,
                     pad_extra, t_phase, upsample_in, cu_limit)


def conv_out_hw(h, w, k, stride, padding, dilation, pad_extra=(0, 0)):
    ho = (h + 2 * padding[0] + pad_extra[0] - dilation[1] * (k[1] - 1) - 1) // stride[1] + 1
    wo = (w + 2 * padding[1] + pad_extra[1] - dilation[2] * (k[2] - 1) - 1) // stride[2] + 1
    return ho, wo


def conv_out_frames(t: int, stride_t: int = 1, t_phase: int = 0) -> int:
    """Output frames of a t-frame chunk (see t_phase in include/wvc.h)."""
    first = (stride_t - t_phase) % stride_t
    return (t - 1 - first) // stride_t + 1 if first < t else 0


def wvc_conv3d_cache_frames(weight_shape, dilation=(1, 1, 1)) -> int:
    d = conv_desc((1, weight_shape[1], 1, 1, 1), weight_shape, WVC_BF16, dilation=dilation)
    return load().wvc_conv3d_cache_frames(ctypes.byref(d))


def wvc_conv3d_kernel_name(d: ConvDesc) -> str:
    """The kernel a conv call with descriptor ``d`` launches on this device."""
    return load().wvc_conv3d_kernel_name(ctypes.byref(d)).decode()


def wvc_causal_conv3d_workspace_bytes(d: ConvDesc) -> int:
    v = load().wvc_causal_conv3d_workspace_bytes(ctypes.byref(d))
    if v == ctypes.c_size_t(-1).value:
        raise WvcError(WVC_ERR_ARG, load().wvc_last_error().decode())
    return v


def wvc_conv3d_packed_weight_bytes(w_shape, dtype=torch.bfloat16, padding=(1, 1), stride=(1, 1, 1),
                                   pad_extra=(0, 0)) -> int:
    # the packed order depends on the channels and the kernel only; the
    # descriptor needs some frame the kernel fits in
    d = conv_desc((1, w_shape[1], 1, 16, 16), tuple(w_shape), _dtype_code(dtype), stride=stride,
                  padding=padding, pad_extra=pad_extra)
    v = load().wvc_conv3d_packed_weight_bytes(ctypes.byref(d))
    if v == ctypes.c_size_t(-1).value:
        raise WvcError(WVC_ERR_UNSUPPORTED, load().wvc_last_error().decode())
    return v


_packed_bytes_shared = _memo(wvc_conv3d_packed_weight_bytes)


@_memo
def _norm_ws_shared(x_shape, w_shape, code, padding, layout, device, upsample_in=0,
                    cu_limit=0) -> int:
    """wvc_causal_conv3d_norm_workspace_bytes of a unit-stride conv, asked once
    per shape and device (the size depends on the device's CU count)."""
    return wvc_causal_conv3d_norm_workspace_bytes(
        conv_desc(x_shape, w_shape, code, padding=padding, weight_layout=layout,
                  upsample_in=upsample_in, cu_limit=cu_limit))


def wvc_conv3d_pack_weights(weight: torch.Tensor, padding=(1, 1), stride=(1, 1, 1),
                            pad_extra=(0, 0)) -> torch.Tensor:
    """Weights [C_out, C_in, kT, kH, kW] (channels_last_3d) -> their packed MFMA
    fragment order (a flat uint8 device tensor), for calls with
    weight_layout=WVC_WEIGHT_PACKED (see wvc_conv3d_pack_weights in
    include/wvc.h)."""
    _need_cl(weight, "weight")
    shape = tuple(weight.shape)
    d = conv_desc((1, shape[1], 1, 16, 16), shape, _dtype_code(weight.dtype), stride=stride,
                  padding=padding, pad_extra=pad_extra)
    packed = torch.empty(wvc_conv3d_packed_weight_bytes(shape, weight.dtype, padding, stride,
                                                        pad_extra),
                         dtype=torch.uint8, device=weight.device)
    _check(load().wvc_conv3d_pack_weights(ctypes.byref(d), _ptr(weight), _ptr(packed),
                                          _stream(weight)))
    return packed


def wvc_causal_conv3d_fwd(x: torch.Tensor, weight: torch.Tensor, bias: Optional[torch.Tensor] = None,
                          cache_in: Optional[torch.Tensor] = None,
                          cache_out: Optional[torch.Tensor] = None,
                          residual: Optional[torch.Tensor] = None,
                          y: Optional[torch.Tensor] = None, stride=(1, 1, 1), padding=(1, 1),
                          dilation=(1, 1, 1), groups: int = 1,
                          workspace: Optional[torch.Tensor] = None,
                          packed_weight: Optional[torch.Tensor] = None, pad_extra=(0, 0),
                          t_phase: int = 0, upsample_in: int = 0, cu_limit: int = 0) -> torch.Tensor:
    """Causal Conv3D of one chunk (see wvc_causal_conv3d_fwd in include/wvc.h).
    ``weight`` gives the logical shape; when ``packed_weight`` (from
    wvc_conv3d_pack_weights) is given the call reads that instead.
    ``stride`` is (temporal, h, w); ``pad_extra`` adds zero rows below / columns
    right of the frame; ``t_phase`` is the number of sequence frames before this
    chunk modulo the temporal stride; ``upsample_in`` = 2 reads x and the
    caches (frames of h x w) through a nearest 2x upsample, so y has frames of
    2h x 2w; ``cu_limit`` > 0 plans the grid for that many CUs (see the
    descriptor in include/wvc.h).  Returns y (allocated if not given)."""
    lib = load()
    d, out_shape, wsrc = _conv_checks(x, weight, bias, cache_in, cache_out, residual, y, stride,
                                      padding, dilation, groups, packed_weight, pad_extra, t_phase,
                                      upsample_in, cu_limit)
    if y is None:
        y = empty_cl(out_shape, x.dtype, x.device)
    ws_bytes = 0
    if workspace is None:
        need = wvc_causal_conv3d_workspace_bytes(d)
        if need:  # contents on entry do not matter
            workspace = torch.empty(need, dtype=torch.uint8, device=x.device)
    if workspace is not None:
        ws_bytes = workspace.numel() * workspace.element_size()
    _check(lib.wvc_causal_conv3d_fwd(ctypes.byref(d), _ptr(x), _ptr(cache_in), _ptr(cache_out),
                                      _ptr(wsrc), _ptr(bias), _ptr(residual), _ptr(y),
                                      _ptr(workspace), ws_bytes, _stream(x)))
    return y


def wvc_causal_conv3d_norm_workspace_bytes(d: ConvDesc) -> int:
    v = load().wvc_causal_conv3d_norm_workspace_bytes(ctypes.byref(d))
    if v == ctypes.c_size_t(-1).value:
        raise WvcError(WVC_ERR_ARG, load().wvc_last_error().decode())
    return v


def wvc_causal_conv3d_norm_fwd(x: torch.Tensor, weight: torch.Tensor, gamma: torch.Tensor,
                               bias: Optional[torch.Tensor] = None,
                               beta: Optional[torch.Tensor] = None, eps: float = 1e-12,
                               cache_in: Optional[torch.Tensor] = None,
                               cache_out: Optional[torch.Tensor] = None,
                               residual: Optional[torch.Tensor] = None,
                               y: Optional[torch.Tensor] = None, h: Optional[torch.Tensor] = None,
                               padding=(1, 1), workspace: Optional[torch.Tensor] = None,
                               packed_weight: Optional[torch.Tensor] = None,
                               upsample_in: int = 0, cu_limit: int = 0) -> torch.Tensor:
    """Conv, then the RMS norm + SiLU of the layer it feeds (see
    wvc_causal_conv3d_norm_fwd in include/wvc.h): y = conv(x) + bias + residual
    (stored only when ``y`` is given), h = SiLU(norm(y)); ``upsample_in`` and
    ``cu_limit`` as for wvc_causal_conv3d_fwd.  Returns h (allocated if not
    given)."""
    d, out_shape, wsrc = _conv_checks(x, weight, bias, cache_in, cache_out, residual, y, (1, 1, 1),
                                      padding, (1, 1, 1), 1, packed_weight, (0, 0), 0, upsample_in,
                                      cu_limit)
    c_out = out_shape[1]
    _need_exact(gamma, "gamma", (c_out,), x.dtype, x.device)
    if gamma is None:
        raise ValueError("gamma must be given")
    _need_exact(beta, "beta", (c_out,), x.dtype, x.device)
    _need_exact(h, "h", out_shape, x.dtype, x.device)
    if h is None:
        h = empty_cl(out_shape, x.dtype, x.device)
    if workspace is None:
        need = _norm_ws_shared(tuple(x.shape), tuple(weight.shape), _dtype_code(x.dtype),
                               tuple(padding), d.weight_layout, x.device, upsample_in, cu_limit)
    if workspace is None and need:  # contents on entry do not matter
        workspace = torch.empty(need, dtype=torch.uint8, device=x.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(load().wvc_causal_conv3d_norm_fwd(ctypes.byref(d), _ptr(x), _ptr(cache_in),
                                             _ptr(cache_out), _ptr(wsrc), _ptr(bias), _ptr(residual),
                                             _ptr(y), _ptr(gamma), _ptr(beta), float(eps), _ptr(h),
                                             _ptr(workspace), ws_bytes, _stream(x)))
    return h


def wvc_causal_conv3d_fwd_noalloc(x: torch.Tensor, weight: torch.Tensor, y: torch.Tensor,
                                  bias: Optional[torch.Tensor] = None,
                                  cache_in: Optional[torch.Tensor] = None,
                                  cache_out: Optional[torch.Tensor] = None,
                                  residual: Optional[torch.Tensor] = None, stride=(1, 1, 1),
                                  padding=(1, 1), dilation=(1, 1, 1), groups: int = 1,
                                  packed_weight: Optional[torch.Tensor] = None, pad_extra=(0, 0),
                                  t_phase: int = 0) -> torch.Tensor:
    """wvc_causal_conv3d_fwd without a workspace: the library's fixed scratch
    array serves the kernels (see wvc_causal_conv3d_fwd_noalloc in
    include/wvc.h).  Allocates nothing, so ``y`` must be given."""
    if y is None:
        raise ValueError("y must be given: the allocation-free call allocates nothing")
    d, _, wsrc = _conv_checks(x, weight, bias, cache_in, cache_out, residual, y, stride, padding,
                              dilation, groups, packed_weight, pad_extra, t_phase)
    _check(load().wvc_causal_conv3d_fwd_noalloc(ctypes.byref(d), _ptr(x), _ptr(cache_in),
                                                _ptr(cache_out), _ptr(wsrc), _ptr(bias),
                                                _ptr(residual), _ptr(y), _stream(x)))
    return y


def _conv_checks(x, weight, bias, cache_in, cache_out, residual, y, stride, padding, dilation,
                 groups, packed_weight, pad_extra, t_phase, upsample_in=0, cu_limit=0):
    """Checks of a conv call's tensors against the descriptor built from x and
    the weight; returns (descriptor, output shape, weight pointer source)."""
    _need_cl(x, "x")
    _need_cl(weight, "weight")
    code = _dtype_code(x.dtype)
    n, c, t, h, w = x.shape
    if upsample_in not in (0, 2):
        raise WvcError(WVC_ERR_ARG, f"upsample_in {upsample_in} must be 0 or 2")
    if cu_limit < 0:
        raise WvcError(WVC_ERR_ARG, f"cu_limit {cu_limit} must be >= 0")
    up = 2 if upsample_in == 2 else 1   # the caches keep x's frame size
    _need_exact(weight, "weight", (weight.shape[0], c) + tuple(weight.shape[2:]), x.dtype, x.device)
    _need_exact(bias, "bias", (weight.shape[0],), x.dtype, x.device)
    ho, wo = conv_out_hw(h * up, w * up, weight.shape[2:], stride, padding, dilation, pad_extra)
    if ho < 1 or wo < 1:
        raise WvcError(WVC_ERR_ARG, "kernel larger than the padded frame")
    if stride[0] < 1 or not 0 <= t_phase < stride[0]:
        raise WvcError(WVC_ERR_ARG, "bad temporal stride or t_phase")
    to = conv_out_frames(t, stride[0], t_phase)
    out_shape = (n, weight.shape[0], to, ho, wo)
    frames = dilation[0] * (weight.shape[2] - 1)
    if frames > 0:  # (a conv with no temporal reach ignores the caches)
        for name, cc in (("cache_in", cache_in), ("cache_out", cache_out)):
            _need_exact(cc, name, (n, c, frames, h, w), x.dtype, x.device)
    _need_exact(residual, "residual", out_shape, x.dtype, x.device)
    _need_exact(y, "y", out_shape, x.dtype, x.device)
    layout = WVC_WEIGHT_STANDARD if packed_weight is None else WVC_WEIGHT_PACKED
    stride, padding, dilation, pad_extra = tuple(stride), tuple(padding), tuple(dilation), \
        tuple(pad_extra)
    d = _conv_desc_shared(tuple(x.shape), tuple(weight.shape), code, stride, padding, dilation,
                          groups, layout, pad_extra, t_phase, upsample_in, cu_limit)
    if packed_weight is not None:
        _need_bytes(packed_weight, "packed_weight",
                    _packed_bytes_shared(tuple(weight.shape), x.dtype, padding, stride, pad_extra),
                    x.device)
    wsrc = weight if packed_weight is None else packed_weight
    return d, out_shape, wsrc


def wvc_resblock_e4m3_workspace_bytes(d: ResblockDesc) -> int:
    v = load().wvc_resblock_e4m3_workspace_bytes(ctypes.byref(d))
    if v == ctypes.c_size_t(-1).value:
        raise WvcError(WVC_ERR_ARG, load().wvc_last_error().decode())
    return v


def wvc_resblock_e4m3_fwd(x: torch.Tensor, params: dict, s1: float, s2: float, cache1_in=None,
                          cache1_out=None, cache2_in=None, cache2_out=None,
                          y: Optional[torch.Tensor] = None, eps: float = 1e-12,
                          workspace: Optional[torch.Tensor] = None, packed: bool = False,
                          cu_limit: int = 0) -> torch.Tensor:
    """The residual block on the 8-bit path (see wvc_resblock_e4m3_fwd in
    include/wvc.h).  ``params`` holds gamma1, beta1, gamma2, beta2, b1, b2
    (bf16 vectors), w1, w2 (uint8 E4M3 codes, packed when ``packed``) and
    w1_scale, w2_scale (float32 [C]).  Caches are uint8 codes.  ``cu_limit``
    > 0 plans the convs' split-K grids for that many CUs."""
    lib = load()
    _need_cl(x, "x")
    n, c, t, h, w = x.shape
    if x.dtype != torch.bfloat16:
        raise TypeError("x must be bfloat16")
    _need_exact(y, "y", x.shape, torch.bfloat16, x.device)
    for name, cc in (("cache1_in", cache1_in), ("cache1_out", cache1_out), ("cache2_in", cache2_in),
                     ("cache2_out", cache2_out)):
        _need_exact(cc, name, (n, c, 2, h, w), torch.uint8, x.device)
    for k in ("gamma1", "gamma2", "beta1", "beta2", "b1", "b2"):
        _need_exact(params.get(k), k, (c,), torch.bfloat16, x.device)
    for k in ("w1_scale", "w2_scale"):
        _need_exact(params.get(k), k, (c,), torch.float32, x.device)
    wbytes = wvc_conv3d_packed_weight_bytes((c, c, 3, 3, 3), torch.uint8) if packed else c * c * 27
    for k in ("w1", "w2"):
        if params.get(k) is None or params[k].numel() * params[k].element_size() != wbytes \
                or params[k].dtype != torch.uint8 or params[k].device != x.device:
            raise ValueError(f"{k} must be {wbytes} bytes of E4M3 codes (uint8) on {x.device}")
    d = resblock_desc(tuple(x.shape), c, WVC_BF16, eps, weights_packed=packed, cu_limit=cu_limit)
    if y is None:
        y = empty_cl(x.shape, x.dtype, x.device)
    if workspace is None:
        workspace = torch.empty(max(1, wvc_resblock_e4m3_workspace_bytes(d)), dtype=torch.uint8,
                                device=x.device)
    pr = ResblockE4M3Params()
    for k in ("gamma1", "beta1", "w1", "w1_scale", "b1", "gamma2", "beta2", "w2", "w2_scale", "b2"):
        t = params.get(k)
        setattr(pr, k, None if t is None else t.data_ptr())
    pr.s1, pr.s2 = float(s1), float(s2)
    _check(lib.wvc_resblock_e4m3_fwd(ctypes.byref(d), _ptr(x), _ptr(y), ctypes.byref(pr),
                                      _ptr(cache1_in), _ptr(cache1_out), _ptr(cache2_in),
                                      _ptr(cache2_out), _ptr(workspace),
                                      workspace.numel() * workspace.element_size(), _stream(x)))
    return y


def wvc_rmsnorm_silu_conv3d_fwd(x: torch.Tensor, gamma: torch.Tensor, weight: torch.Tensor,
                                bias: Optional[torch.Tensor] = None,
                                beta: Optional[torch.Tensor] = None, eps: float = 1e-12,
                                residual: Optional[torch.Tensor] = None,
                                y: Optional[torch.Tensor] = None, stride=(1, 2, 2),
                                padding=(0, 0), pad_extra=(1, 1),
                                workspace: Optional[torch.Tensor] = None,
                                packed_weight: Optional[torch.Tensor] = None) -> torch.Tensor:
    """RMS norm + SiLU fused into the stride-2 spatial conv (see
    wvc_rmsnorm_silu_conv3d_fwd in include/wvc.h).  Returns y."""
    lib = load()
    _need_cl(x, "x")
    _need_cl(weight, "weight")
    n, c, t, h, w = x.shape
    _need_exact(weight, "weight", (weight.shape[0], c) + tuple(weight.shape[2:]), x.dtype, x.device)
    _need_exact(bias, "bias", (weight.shape[0],), x.dtype, x.device)
    _need_exact(gamma, "gamma", (c,), x.dtype, x.device)
    _need_exact(beta, "beta", (c,), x.dtype, x.device)
    ho, wo = conv_out_hw(h, w, weight.shape[2:], stride, padding, (1, 1, 1), pad_extra)
    if ho < 1 or wo < 1:
        raise WvcError(WVC_ERR_ARG, "kernel larger than the padded frame")
    out_shape = (n, weight.shape[0], t, ho, wo)
    _need_exact(residual, "residual", out_shape, x.dtype, x.device)
    _need_exact(y, "y", out_shape, x.dtype, x.device)
    layout = WVC_WEIGHT_STANDARD if packed_weight is None else WVC_WEIGHT_PACKED
    d = conv_desc(tuple(x.shape), tuple(weight.shape), _dtype_code(x.dtype), stride, padding,
                  weight_layout=layout, pad_extra=pad_extra)
    if packed_weight is not None:
        _need_bytes(packed_weight, "packed_weight",
                    wvc_conv3d_packed_weight_bytes(tuple(weight.shape), x.dtype, padding, stride,
                                                   pad_extra), x.device)
    if y is None:
        y = empty_cl(out_shape, x.dtype, x.device)
    ws_bytes = 0
    if workspace is None:
        need = wvc_causal_conv3d_workspace_bytes(d)
        if need:
            workspace = torch.empty(need, dtype=torch.uint8, device=x.device)
    if workspace is not None:
        ws_bytes = workspace.numel() * workspace.element_size()
    wsrc = weight if packed_weight is None else packed_weight
    _check(lib.wvc_rmsnorm_silu_conv3d_fwd(ctypes.byref(d), _ptr(x), _ptr(gamma), _ptr(beta),
                                            float(eps), _ptr(wsrc), _ptr(bias), _ptr(residual),
                                            _ptr(y), _ptr(workspace), ws_bytes, _stream(x)))
    return y


def wvc_causal_conv3d_e4m3_fwd(x: torch.Tensor, x_scale: float, weight: torch.Tensor,
                               w_scale: torch.Tensor, bias: Optional[torch.Tensor] = None,
                               cache_in: Optional[torch.Tensor] = None,
                               cache_out: Optional[torch.Tensor] = None,
                               residual: Optional[torch.Tensor] = None,
                               y: Optional[torch.Tensor] = None,
                               workspace: Optional[torch.Tensor] = None,
                               packed_weight: Optional[torch.Tensor] = None,
                               upsample_in: int = 0, cu_limit: int = 0) -> torch.Tensor:
    """Causal 3x3x3 conv of E4M3 operands (see wvc_causal_conv3d_e4m3_fwd in
    include/wvc.h).  x, caches and weight are uint8 tensors of E4M3 codes in
    channels_last_3d; w_scale is a float32 vector [C_out]; bias, residual and
    y are bfloat16.  ``upsample_in`` = 2 reads x and the caches through a
    nearest 2x upsample (y then has frames of twice x's); ``cu_limit`` > 0
    plans the split-K grid for that many CUs.  Returns y (allocated if not
    given)."""
    lib = load()
    _need_cl(x, "x")
    _need_cl(weight, "weight")
    if x.dtype != torch.uint8 or weight.dtype != torch.uint8 or w_scale.dtype != torch.float32:
        raise TypeError("x and weight must be uint8 (E4M3 codes), w_scale float32")
    n, c, t, h, w = x.shape
    if upsample_in not in (0, 2):
        raise WvcError(WVC_ERR_ARG, f"upsample_in {upsample_in} must be 0 or 2")
    up = 2 if upsample_in == 2 else 1   # the caches keep x's frame size
    co = weight.shape[0]
    _need_exact(weight, "weight", (co, c) + tuple(weight.shape[2:]), torch.uint8, x.device)
    _need_exact(bias, "bias", (co,), torch.bfloat16, x.device)
    _need_exact(w_scale, "w_scale", (co,), torch.float32, x.device)
    for name, cc in (("cache_in", cache_in), ("cache_out", cache_out)):
        _need_exact(cc, name, (n, c, 2, h, w), torch.uint8, x.device)
    for name, tt in (("residual", residual), ("y", y)):
        _need_exact(tt, name, (n, co, t, h * up, w * up), torch.bfloat16, x.device)
    layout = WVC_WEIGHT_STANDARD if packed_weight is None else WVC_WEIGHT_PACKED
    d = conv_desc(tuple(x.shape), tuple(weight.shape), WVC_E4M3, weight_layout=layout,
                  upsample_in=upsample_in, cu_limit=cu_limit)
    if packed_weight is not None:
        _need_bytes(packed_weight, "packed_weight",
                    wvc_conv3d_packed_weight_bytes(tuple(weight.shape), torch.uint8), x.device)
    wsrc = weight if packed_weight is None else packed_weight
    if y is None:
        y = empty_cl((n, co, t, h * up, w * up), torch.bfloat16, x.device)
    ws_bytes = 0
    if workspace is None:
        need = wvc_causal_conv3d_workspace_bytes(d)
        if need:
            workspace = torch.empty(need, dtype=torch.uint8, device=x.device)
    if workspace is not None:
        ws_bytes = workspace.numel() * workspace.element_size()
    _check(lib.wvc_causal_conv3d_e4m3_fwd(ctypes.byref(d), _ptr(x), float(x_scale), _ptr(cache_in),
                                           _ptr(cache_out), _ptr(wsrc), _ptr(w_scale), _ptr(bias),
                                           _ptr(residual), _ptr(y), _ptr(workspace), ws_bytes,
                                           _stream(x)))
    return y


def wvc_causal_conv3d_e4m3_norm_workspace_bytes(d: ConvDesc) -> int:
    v = load().wvc_causal_conv3d_e4m3_norm_workspace_bytes(ctypes.byref(d))
    if v == ctypes.c_size_t(-1).value:
        raise WvcError(WVC_ERR_ARG, load().wvc_last_error().decode())
    return v


def wvc_causal_conv3d_e4m3_norm_fwd(x: torch.Tensor, x_scale: float, weight: torch.Tensor,
                                    w_scale: torch.Tensor, gamma: torch.Tensor, q_scale: float,
                                    bias: Optional[torch.Tensor] = None,
                                    beta: Optional[torch.Tensor] = None, eps: float = 1e-12,
                                    cache_in: Optional[torch.Tensor] = None,
                                    cache_out: Optional[torch.Tensor] = None,
                                    residual: Optional[torch.Tensor] = None,
                                    y: Optional[torch.Tensor] = None,
                                    q: Optional[torch.Tensor] = None,
                                    workspace: Optional[torch.Tensor] = None,
                                    packed_weight: Optional[torch.Tensor] = None,
                                    upsample_in: int = 0, cu_limit: int = 0) -> torch.Tensor:
    """The 8-bit conv, then the RMS norm + SiLU of the layer it feeds stored as
    E4M3 codes at ``q_scale`` (see wvc_causal_conv3d_e4m3_norm_fwd in
    include/wvc.h): y = the 8-bit conv's bf16 output (stored only when ``y``
    is given), q = codes of SiLU(norm(y)).  Operands as for
    wvc_causal_conv3d_e4m3_fwd.  Returns q (uint8, allocated if not given)."""
    lib = load()
    _need_cl(x, "x")
    _need_cl(weight, "weight")
    if x.dtype != torch.uint8 or weight.dtype != torch.uint8 or w_scale.dtype != torch.float32:
        raise TypeError("x and weight must be uint8 (E4M3 codes), w_scale float32")
    n, c, t, h, w = x.shape
    if upsample_in not in (0, 2):
        raise WvcError(WVC_ERR_ARG, f"upsample_in {upsample_in} must be 0 or 2")
    up = 2 if upsample_in == 2 else 1
    co = weight.shape[0]
    out_shape = (n, co, t, h * up, w * up)
    _need_exact(weight, "weight", (co, c) + tuple(weight.shape[2:]), torch.uint8, x.device)
    for name, v in (("bias", bias), ("gamma", gamma), ("beta", beta)):
        _need_exact(v, name, (co,), torch.bfloat16, x.device)
    if gamma is None:
        raise ValueError("gamma must be given")
    _need_exact(w_scale, "w_scale", (co,), torch.float32, x.device)
    for name, cc in (("cache_in", cache_in), ("cache_out", cache_out)):
        _need_exact(cc, name, (n, c, 2, h, w), torch.uint8, x.device)
    for name, tt in (("residual", residual), ("y", y)):
        _need_exact(tt, name, out_shape, torch.bfloat16, x.device)
    _need_exact(q, "q", out_shape, torch.uint8, x.device)
    layout = WVC_WEIGHT_STANDARD if packed_weight is None else WVC_WEIGHT_PACKED
    d = conv_desc(tuple(x.shape), tuple(weight.shape), WVC_E4M3, weight_layout=layout,
                  upsample_in=upsample_in, cu_limit=cu_limit)
    if packed_weight is not None:
        _need_bytes(packed_weight, "packed_weight",
                    wvc_conv3d_packed_weight_bytes(tuple(weight.shape), torch.uint8), x.device)
    wsrc = weight if packed_weight is None else packed_weight
    if q is None:
        q = empty_cl(out_shape, torch.uint8, x.device)
    if workspace is None:
        workspace = torch.empty(max(1, wvc_causal_conv3d_e4m3_norm_workspace_bytes(d)), dtype=torch.uint8,
                                device=x.device)
    ws_bytes = workspace.numel() * workspace.element_size()
    _check(lib.wvc_causal_conv3d_e4m3_norm_fwd(ctypes.byref(d), _ptr(x), float(x_scale), _ptr(cache_in),
                                                _ptr(cache_out), _ptr(wsrc), _ptr(w_scale), _ptr(bias),
                                                _ptr(residual), _ptr(y), _ptr(gamma), _ptr(beta),
                                                float(eps), float(q_scale), _ptr(q), _ptr(workspace),
                                                ws_bytes, _stream(x)))
    return q


def wvc_quantize_e4m3(x: torch.Tensor, scale: float, q: Optional[torch.Tensor] = None) -> torch.Tensor:
    """E4M3 codes of fl32(x * fl32(1/scale)), same shape and strides as x (uint8)."""
    if not _on_device(x) or not x.is_contiguous(memory_format=torch.channels_last_3d if x.dim() == 5
                                            else torch.contiguous_format):
        raise ValueError("x must be a dense device tensor")
    if q is None:
        q = torch.empty_like(x, dtype=torch.uint8)
    _check(load().wvc_quantize_e4m3(_ptr(x), _dtype_code(x.dtype), x.numel(), float(scale), _ptr(q),
                                    _stream(x)))
    return q


def wvc_quantize_rows_e4m3(x: torch.Tensor, q: Optional[torch.Tensor] = None,
                           scale: Optional[torch.Tensor] = None):
    """Per-row absmax quantisation of a tensor viewed as [shape[0], rest] in its
    memory order (conv weights in channels_last_3d: one row per output
    channel).  Returns (codes uint8 like x, scales float32 [shape[0]])."""
    if not _on_device(x):
        raise ValueError("x must be a device tensor")
    mf = torch.channels_last_3d if x.dim() == 5 else torch.contiguous_format
    if not x.is_contiguous(memory_format=mf):
        raise ValueError("x must be dense (channels_last_3d for 5-d tensors)")
    rows = x.shape[0]
    if q is None:
        q = torch.empty_like(x, dtype=torch.uint8)
    if scale is None:
        scale = torch.empty(rows, dtype=torch.float32, device=x.device)
    _check(load().wvc_quantize_rows_e4m3(_ptr(x), _dtype_code(x.dtype), rows, x.numel() // max(rows, 1),
                                         _ptr(q), _ptr(scale), _stream(x)))
    return q, scale


def wvc_rmsnorm_silu_e4m3(x: torch.Tensor, gamma: torch.Tensor, scale: float,
                          beta: Optional[torch.Tensor] = None, q: Optional[torch.Tensor] = None,
                          eps: float = 1e-12, apply_silu: bool = True) -> torch.Tensor:
    """RMS norm (+ SiLU) of a bf16 tensor, stored as E4M3 codes of
    fl32(y * fl32(1/scale)) (see wvc_rmsnorm_silu_e4m3 in include/wvc.h)."""
    _need_cl(x, "x")
    n, c, t, h, w = x.shape
    if x.dtype != torch.bfloat16:
        raise TypeError("x must be bfloat16")
    _need_exact(q, "q", x.shape, torch.uint8, x.device)
    _need_exact(gamma, "gamma", (c,), torch.bfloat16, x.device)
    _need_exact(beta, "beta", (c,), torch.bfloat16, x.device)
    if q is None:
        q = empty_cl(x.shape, torch.uint8, x.device)
    _check(load().wvc_rmsnorm_silu_e4m3(_ptr(x), _ptr(gamma), _ptr(beta), _ptr(q), n, c, t, h, w,
                                        float(eps), int(bool(apply_silu)), float(scale), _stream(x)))
    return q


def wvc_rmsnorm_silu(x: torch.Tensor, gamma: torch.Tensor, beta: Optional[torch.Tensor] = None,
                     y: Optional[torch.Tensor] = None, eps: float = 1e-12,
                     apply_silu: bool = True) -> torch.Tensor:
    """Channel RMS norm (+ SiLU) (see wvc_rmsnorm_silu in include/wvc.h)."""
    lib = load()
    _need_cl(x, "x")
    n, c, t, h, w = x.shape
    _need_exact(y, "y", x.shape, x.dtype, x.device)
    _need_exact(gamma, "gamma", (c,), x.dtype, x.device)
    _need_exact(beta, "beta", (c,), x.dtype, x.device)
    if y is None:
        y = empty_cl(x.shape, x.dtype, x.device)
    _check(lib.wvc_rmsnorm_silu(_ptr(x), _ptr(gamma), _ptr(beta), _ptr(y), n, c, t, h, w,
                                _dtype_code(x.dtype), float(eps), int(bool(apply_silu)),
                                _stream(x)))
    return y


def resblock_desc(x_shape, c_out: int, dtype: int, eps: float = 1e-12,
                  weights_packed: bool = False, cu_limit: int = 0) -> ResblockDesc:
    d = ResblockDesc()
    d.cu_limit = cu_limit
    d.n, d.c_in, d.t, d.h, d.w = x_shape[0], x_shape[1], x_shape[2], x_shape[3], x_shape[4]
    d.c_out = c_out
    d.dtype = dtype
    d.eps = eps
    d.weights_packed = int(bool(weights_packed))
    return d


def wvc_resblock_workspace_bytes(d: ResblockDesc) -> int:
    v = load().wvc_resblock_workspace_bytes(ctypes.byref(d))
    if v == ctypes.c_size_t(-1).value:
        raise WvcError(WVC_ERR_ARG, load().wvc_last_error().decode())
    return v


# Parameter sets that passed _check_block_params, by (dict identities, x's
# shape, dtype, device) -> (fingerprint, C_out, ResblockParams).  A streamed
# block passes the same dicts on every chunk; the fingerprint (pointer, shape,
# strides and dtype of every tensor in them) shows they still hold what was
# checked, so the full check runs once per parameter set.
_BLOCK_CHECKED: dict = {}


def _block_fingerprint(params: dict, packed: Optional[dict]) -> tuple:
    fp = []
    for src in (params, packed):
        if src is None:
            fp.append(None)
            continue
        for k, t in src.items():
            fp.append((k, None) if t is None else (k, t.data_ptr(), t.shape, t.stride(), t.dtype))
    return tuple(fp)


def _block_params_struct(params: dict, packed: Optional[dict]) -> ResblockParams:
    merged = params if packed is None else dict(params, **packed)
    p = ResblockParams()
    for f, _ in ResblockParams._fields_:
        t = merged.get(f)
        setattr(p, f, None if t is None else t.data_ptr())
    return p


def _checked_block(x: torch.Tensor, params: dict, packed: Optional[dict]):
    """(C_out, ResblockParams) of a checked parameter set."""
    key = (id(params), id(packed), x.shape, x.dtype, x.device)
    fp = _block_fingerprint(params, packed)
    hit = _BLOCK_CHECKED.get(key)
    if hit is not None and hit[0] == fp:
        _need_cl(x, "x")
        return hit[1], hit[2]
    c_out = _check_block_params(x, params, packed)
    if len(_BLOCK_CHECKED) >= 256:
        _BLOCK_CHECKED.clear()
    p = _block_params_struct(params, packed)
    _BLOCK_CHECKED[key] = (fp, c_out, p)
    return c_out, p


@_memo
def _block_desc_ws(x_shape, c_out, code, eps, packed, device, cu_limit=0) -> tuple:
    """(ResblockDesc, workspace bytes) of a block call (the workspace size
    depends on the device's CU count through the split-K plan)."""
    d = resblock_desc(x_shape, c_out, code, eps, weights_packed=packed, cu_limit=cu_limit)
    return d, wvc_resblock_workspace_bytes(d)


def _check_block_params(x: torch.Tensor, params: dict, packed: Optional[dict]):
    """Shapes, dtypes and devices of a bf16/fp32 block's parameters (and of the
    packed weights when given) against x and w1."""
    _need_cl(x, "x")
    ci = x.shape[1]
    co = params["w1"].shape[0]
    dt, dev = x.dtype, x.device
    shapes = {"w1": (co, ci, 3, 3, 3), "w2": (co, co, 3, 3, 3), "gamma1": (ci,), "beta1": (ci,),
              "b1": (co,), "gamma2": (co,), "beta2": (co,), "b2": (co,),
              "w_short": (co, ci, 1, 1, 1), "b_short": (co,)}
    for k, shp in shapes.items():
        _need_exact(params.get(k), k, shp, dt, dev)
    if packed is not None:
        for k, pad in (("w1", (1, 1)), ("w2", (1, 1)), ("w_short", (0, 0))):
            if packed.get(k) is not None:
                _need_bytes(packed[k], f"packed {k}", _packed_bytes_shared(shapes[k], dt, pad), dev)
    return co


def wvc_resblock_fwd(x: torch.Tensor, params: dict, cache1_in=None, cache1_out=None,
                     cache2_in=None, cache2_out=None, y: Optional[torch.Tensor] = None,
                     eps: float = 1e-12, workspace: Optional[torch.Tensor] = None,
                     packed: Optional[dict] = None, cu_limit: int = 0) -> torch.Tensor:
    """Wan residual block on one chunk (see wvc_resblock_fwd in include/wvc.h).
    ``params``: gamma1, beta1, w1, b1, gamma2, beta2, w2, b2[, w_short, b_short].
    ``packed``: optional {w1, w2[, w_short]} from wvc_conv3d_pack_weights.
    ``cu_limit`` > 0 plans the convs' grids for that many CUs."""
    lib = load()
    c_out, p = _checked_block(x, params, packed)
    n, ci, t, h, w = x.shape
    for name, cc, ch in (("cache1_in", cache1_in, ci), ("cache1_out", cache1_out, ci),
                         ("cache2_in", cache2_in, c_out), ("cache2_out", cache2_out, c_out)):
        _need_exact(cc, name, (n, ch, 2, h, w), x.dtype, x.device)
    _need_exact(y, "y", (n, c_out, t, h, w), x.dtype, x.device)
    d, need = _block_desc_ws(tuple(x.shape), c_out, _dtype_code(x.dtype), float(eps),
                             packed is not None, x.device, int(cu_limit))
    if y is None:
        y = empty_cl((x.shape[0], c_out) + tuple(x.shape[2:]), x.dtype, x.device)
    if workspace is None and need:  # contents on entry do not matter
        workspace = torch.empty(need, dtype=torch.uint8, device=x.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib.wvc_resblock_fwd(ctypes.byref(d), _ptr(x), _ptr(y), ctypes.byref(p),
                                _ptr(cache1_in), _ptr(cache1_out), _ptr(cache2_in),
                                _ptr(cache2_out), _ptr(workspace), ws_bytes, _stream(x)))
    return y


def _block_call(x, params, packed, eps, workspace, outs, cu_limit=0):
    """Shared marshalling of the block halves: descriptor, params struct,
    workspace (allocated when not given) and its size."""
    c_out, p = _checked_block(x, params, packed)
    n, ci, t, h, w = x.shape
    want = {"cache1_in": (n, ci, 2, h, w), "cache1_out": (n, ci, 2, h, w),
            "cache2_in": (n, c_out, 2, h, w), "cache2_out": (n, c_out, 2, h, w),
            "h2": (n, c_out, t, h, w), "y": (n, c_out, t, h, w)}
    for name, tt in outs:
        _need_exact(tt, name, want[name], x.dtype, x.device)
    d, need = _block_desc_ws(tuple(x.shape), c_out, _dtype_code(x.dtype), float(eps),
                             packed is not None, x.device, int(cu_limit))
    if workspace is None and need:  # contents on entry do not matter
        workspace = torch.empty(need, dtype=torch.uint8, device=x.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    return d, p, c_out, workspace, ws_bytes


def wvc_resblock_front(x: torch.Tensor, params: dict, cache1_in=None, cache1_out=None,
                       h2: Optional[torch.Tensor] = None, eps: float = 1e-12,
                       workspace: Optional[torch.Tensor] = None,
                       packed: Optional[dict] = None, cu_limit: int = 0) -> torch.Tensor:
    """First half of the block, h2 = SiLU(norm2(conv1(SiLU(norm1(x)))))
    (see wvc_resblock_front in include/wvc.h)."""
    d, p, c_out, workspace, ws_bytes = _block_call(
        x, params, packed, eps, workspace,
        (("cache1_in", cache1_in), ("cache1_out", cache1_out), ("h2", h2)), cu_limit)
    if h2 is None:
        h2 = empty_cl((x.shape[0], c_out) + tuple(x.shape[2:]), x.dtype, x.device)
    _check(load().wvc_resblock_front(ctypes.byref(d), _ptr(x), _ptr(h2), ctypes.byref(p),
                                     _ptr(cache1_in), _ptr(cache1_out), _ptr(workspace),
                                     ws_bytes, _stream(x)))
    return h2


def wvc_resblock_back(h2: torch.Tensor, x: torch.Tensor, params: dict, cache2_in=None,
                      cache2_out=None, y: Optional[torch.Tensor] = None, eps: float = 1e-12,
                      workspace: Optional[torch.Tensor] = None,
                      packed: Optional[dict] = None, cu_limit: int = 0) -> torch.Tensor:
    """Second half of the block, y = conv2(h2) + shortcut(x) (see
    wvc_resblock_back in include/wvc.h)."""
    d, p, c_out, workspace, ws_bytes = _block_call(
        x, params, packed, eps, workspace,
        (("h2", h2), ("cache2_in", cache2_in), ("cache2_out", cache2_out), ("y", y)), cu_limit)
    if y is None:
        y = empty_cl((x.shape[0], c_out) + tuple(x.shape[2:]), x.dtype, x.device)
    _check(load().wvc_resblock_back(ctypes.byref(d), _ptr(h2), _ptr(x), _ptr(y), ctypes.byref(p),
                                    _ptr(cache2_in), _ptr(cache2_out), _ptr(workspace), ws_bytes,
                                    _stream(x)))
    return y


def wvc_cache_reset(cache: torch.Tensor):
    """Zero a cache in place (the zero causal padding of a fresh sequence)."""
    _check(load().wvc_cache_reset(_ptr(cache), cache.numel() * cache.element_size(),
                                  _stream(cache)))
    return cache


def wvc_upsample_nearest2x(x: torch.Tensor, y: Optional[torch.Tensor] = None) -> torch.Tensor:
    lib = load()
    _need_cl(x, "x")
    n, c, t, h, w = x.shape
    _need_exact(y, "y", (n, c, t, 2 * h, 2 * w), x.dtype, x.device)
    if y is None:
        y = empty_cl((n, c, t, 2 * h, 2 * w), x.dtype, x.device)
    _check(lib.wvc_upsample_nearest2x(_ptr(x), _ptr(y), n, c, t, h, w, _dtype_code(x.dtype),
                                      _stream(x)))
    return y


def wvc_set_strict(on: bool):
    load().wvc_set_strict(int(bool(on)))


def wvc_get_strict() -> bool:
    return bool(load().wvc_get_strict())


def wvc_get_counters() -> dict:
    c = Counters()
    load().wvc_get_counters(ctypes.byref(c))
    return {f: int(getattr(c, f)) for f, _ in Counters._fields_}


def wvc_reset_counters():
    load().wvc_reset_counters()


def wvc_last_error() -> str:
    return load().wvc_last_error().decode()


def wvc_version() -> str:
    return load().wvc_version().decode()


# ---------------------------------------------------------------------------
# Graphs (wvc_graph_* in include/wvc.h)
# ---------------------------------------------------------------------------

class Graph:
    """Handle of a captured HIP graph.  ``launch()`` enqueues one replay on
    the current stream; the handle is released by ``close()`` (or when it is
    garbage-collected), after the device has finished every replay."""

    def __init__(self, handle: ctypes.c_void_p, device: torch.device):
        self._h = handle
        self.device = device

    def launch(self, stream: Optional[torch.cuda.Stream] = None):
        wvc_graph_launch(self, stream)

    def close(self):
        if self._h is not None and self._h.value:
            torch.cuda.synchronize(self.device)
            _check(load().wvc_graph_destroy(self._h))
        self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def _stream_handle(stream: Optional[torch.cuda.Stream], device=None) -> ctypes.c_void_p:
    s = stream if stream is not None else torch.cuda.current_stream(device)
    return ctypes.c_void_p(s.cuda_stream)


def wvc_graph_capture_begin(stream: torch.cuda.Stream):
    """Start recording the library calls enqueued on ``stream`` (a created
    stream, not the null stream) from this thread."""
    _check(load().wvc_graph_capture_begin(_stream_handle(stream)))


def wvc_graph_capture_end(stream: torch.cuda.Stream) -> Graph:
    """End the recording on ``stream`` and instantiate it."""
    h = ctypes.c_void_p()
    _check(load().wvc_graph_capture_end(_stream_handle(stream), ctypes.byref(h)))
    return Graph(h, stream.device)


def wvc_graph_launch(graph: Graph, stream: Optional[torch.cuda.Stream] = None):
    """Enqueue one replay of ``graph`` on ``stream`` (default: current)."""
    if graph._h is None:
        raise ValueError("graph was destroyed")
    _check(load().wvc_graph_launch(graph._h, _stream_handle(stream, graph.device)))


def wvc_graph_destroy(graph: Graph):
    graph.close()


# ---------------------------------------------------------------------------
# Spatial tiling with overlap blending (wvc_tile_* in include/wvc.h)
# ---------------------------------------------------------------------------

def wvc_tile_extract(x: torch.Tensor, y0: int, x0: int, th: int, tw: int,
                     tile: Optional[torch.Tensor] = None) -> torch.Tensor:
    """tile = x[:, :, :, y0:y0+th, x0:x0+tw] as a channels-last tensor."""
    _need_cl(x, "x")
    n, c, t, h, w = x.shape
    _need_exact(tile, "tile", (n, c, t, th, tw), x.dtype, x.device)
    if tile is None:
        tile = empty_cl((n, c, t, th, tw), x.dtype, x.device)
    _check(load().wvc_tile_extract(_ptr(x), _ptr(tile), n, c, t, h, w, y0, x0, th, tw,
                                   _dtype_code(x.dtype), _stream(x)))
    return tile


def blend_accumulators(like: torch.Tensor, h: int, w: int):
    """Zeroed fp32 accumulator [N, C, T, h, w] (channels-last) and weight sum [h, w]."""
    n, c, t = like.shape[:3]
    acc = empty_cl((n, c, t, h, w), torch.float32, like.device)
    wsum = torch.empty((h, w), dtype=torch.float32, device=like.device)
    wvc_cache_reset(acc)
    _check(load().wvc_cache_reset(_ptr(wsum), wsum.numel() * 4, _stream(like)))
    return acc, wsum


def wvc_tile_blend(tile: torch.Tensor, acc: torch.Tensor, wsum: torch.Tensor, y0: int, x0: int,
                   ramps=(0, 0, 0, 0)):
    """acc += w * tile at (y0, x0), wsum += w; ramps = (top, bottom, left, right)."""
    _need_cl(tile, "tile")
    _need_cl(acc, "acc")
    n, c, t, th, tw = tile.shape
    h, w = acc.shape[3:]
    _need_exact(acc, "acc", (n, c, t, h, w), torch.float32, tile.device)
    _need_exact(wsum, "wsum", (h, w), torch.float32, tile.device)
    if not wsum.is_contiguous():
        raise ValueError("wsum must be contiguous")
    _check(load().wvc_tile_blend(_ptr(tile), _ptr(acc), _ptr(wsum), n, c, t, th, tw, h, w, y0, x0,
                                 *ramps, _dtype_code(tile.dtype), _stream(tile)))


def wvc_tile_blend_finish(acc: torch.Tensor, wsum: torch.Tensor, dtype=torch.bfloat16,
                          y: Optional[torch.Tensor] = None) -> torch.Tensor:
    """y = acc / wsum, rounded once to ``dtype``."""
    _need_cl(acc, "acc")
    n, c, t, h, w = acc.shape
    if acc.dtype != torch.float32:
        raise TypeError("acc must be float32")
    _need_exact(wsum, "wsum", (h, w), torch.float32, acc.device)
    if not wsum.is_contiguous():
        raise ValueError("wsum must be contiguous")
    if y is None:
        y = empty_cl((n, c, t, h, w), dtype, acc.device)
    _need_exact(y, "y", (n, c, t, h, w), y.dtype, acc.device)
    _check(load().wvc_tile_blend_finish(_ptr(acc), _ptr(wsum), _ptr(y), n, c, t, h, w,
                                        _dtype_code(y.dtype), _stream(acc)))
    return y
