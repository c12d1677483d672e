"""fp64 CPU oracle for the causal video-VAE hot path.

TEST INFRASTRUCTURE ONLY.  Only the test suite, ``__graft_entry__.smoke()`` and
the CPU-baseline leg of ``bench.py`` may import this package.  The product path
(``video_vae_causal_amd``) never imports, links or runs anything here, and this
package imports nothing from it: the two share no code.

Tensors are numpy float64 arrays in the pages' logical layout NCTHW
("Cosmos3 Wan VAE -- engine size vs runtime context memory", section 10.1).
The arithmetic lives in ``oracle.c`` (plain C, fp64); this module only marshals
arrays and composes the documented operations in the pages' order.

Pins (what each function is checked against) are listed in the test files
``tests/test_oracle_*.py``.  Nothing in this module is "parity unpinned".
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None

# The divisor clamp of the channel RMS norm.  The page names an L2 normalise
# with a max-clamp but prints no epsilon; 1e-12 is the documented default of
# the normalise call the page names.
DEFAULT_EPS = 1e-12
# Past frames a 3x3x3 causal conv with temporal dilation 1 keeps (the page's
# CACHE_T = 2, "Cosmos3 Wan VAE ...", section 8.5).
CACHE_T = 2


def build() -> str:
    """Compile oracle.c into liboracle.so with gcc (fp64, OpenMP)."""
    tmp = _LIB_PATH + ".tmp"
    subprocess.check_call(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11",
                           _SRC, "-o", tmp, "-lm"])
    os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
        build()
    lib = ctypes.CDLL(_LIB_PATH)
    dp = ctypes.POINTER(ctypes.c_double)
    i = ctypes.c_int
    lib.oracle_causal_conv3d.restype = ctypes.c_int
    lib.oracle_causal_conv3d.argtypes = [dp, i, i, i, i, i, dp, i, dp, i, i, i, i, dp,
                                         i, i, i, i, i, i, i, dp]
    lib.oracle_causal_conv3d_points.restype = ctypes.c_int
    lib.oracle_causal_conv3d_points.argtypes = [dp, i, i, i, i, i, dp, i, dp, i, i, i, i, dp,
                                                i, i, i, i, i, i, i,
                                                ctypes.POINTER(ctypes.c_int64), ctypes.c_long, dp]
    lib.oracle_rms_norm.restype = ctypes.c_int
    lib.oracle_rms_norm.argtypes = [dp, i, i, i, i, i, dp, dp, ctypes.c_double, dp]
    lib.oracle_silu.restype = None
    lib.oracle_silu.argtypes = [dp, ctypes.c_long, dp]
    lib.oracle_upsample_nearest2x.restype = None
    lib.oracle_upsample_nearest2x.argtypes = [dp, i, i, i, i, i, dp]
    lib.oracle_round_bf16.restype = None
    lib.oracle_round_bf16.argtypes = [dp, ctypes.c_long, dp]
    lib.oracle_conv_out_size.restype = ctypes.c_int
    lib.oracle_conv_out_size.argtypes = [i, i, i, i, i]
    lib.oracle_strided_out_frames.restype = ctypes.c_int
    lib.oracle_strided_out_frames.argtypes = [i, i, i]
    lib.oracle_strided_out_size.restype = ctypes.c_int
    lib.oracle_strided_out_size.argtypes = [i, i, i, i, i, i]
    u8p = ctypes.POINTER(ctypes.c_uint8)
    lib.oracle_e4m3_decode.restype = None
    lib.oracle_e4m3_decode.argtypes = [u8p, ctypes.c_long, dp]
    lib.oracle_e4m3_encode.restype = None
    lib.oracle_e4m3_encode.argtypes = [dp, ctypes.c_long, u8p]
    lib.oracle_causal_conv3d_strided.restype = ctypes.c_int
    lib.oracle_causal_conv3d_strided.argtypes = [dp, i, i, i, i, i, dp, i, dp, i, i, i, i, dp,
                                                 i, i, i, i, i, i, i, i, i, i, i, dp]
    _lib = lib
    return lib


def _f64(a) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(a, dtype=np.float64))


def _ptr(a: Optional[np.ndarray]):
    if a is None:
        return None
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def conv_out_size(n: int, k: int, stride: int, pad: int, dil: int) -> int:
    return int(_load().oracle_conv_out_size(n, k, stride, pad, dil))


def _conv_args(x, w, bias, cache, stride, pad, dil):
    x = _f64(x)
    w = _f64(w)
    if x.ndim != 5 or w.ndim != 5:
        raise ValueError("x must be [N,C,T,H,W] and w [Cout,Cin,kT,kH,kW]")
    N, C, T, H, W = x.shape
    Cout, Cin, kT, kH, kW = w.shape
    if Cin != C:
        raise ValueError("channel mismatch")
    sh, sw = stride
    ph, pw = pad
    dt, dh, dw = dil
    past = dt * (kT - 1)
    b = None if bias is None else _f64(bias).reshape(Cout)
    c = None
    if cache is not None:
        c = _f64(cache)
        if c.shape != (N, C, past, H, W):
            raise ValueError(f"cache must be {(N, C, past, H, W)}, got {c.shape}")
    return x, w, b, c, (N, C, T, H, W), (Cout, kT, kH, kW), (sh, sw, ph, pw, dt, dh, dw), past


def causal_conv3d(x, w, bias=None, cache=None, stride=(1, 1), pad=(1, 1),
                  dil=(1, 1, 1)) -> np.ndarray:
    """Causal Conv3D (temporal stride 1), fp64, whole chunk at once.

    "Cosmos3 Wan VAE ...", section 10.3: standard Conv3D sum with the temporal
    padding moved entirely to the past (dil_t*(kT-1) frames, zeros or the
    cache), symmetric spatial zero padding, bias added once after the sum.
    ``cache`` is [N, C_in, dil_t*(kT-1), H, W] (the past frames, oldest first)
    or None for zero causal padding.
    """
    x, w, b, c, (N, C, T, H, W), (Cout, kT, kH, kW), (sh, sw, ph, pw, dt, dh, dw), past = \
        _conv_args(x, w, bias, cache, stride, pad, dil)
    Ho = conv_out_size(H, kH, sh, ph, dh)
    Wo = conv_out_size(W, kW, sw, pw, dw)
    y = np.empty((N, Cout, T, Ho, Wo), dtype=np.float64)
    if N * T == 0:
        return y
    rc = _load().oracle_causal_conv3d(_ptr(x), N, C, T, H, W, _ptr(c), past if c is not None else 0,
                                      _ptr(w), Cout, kT, kH, kW, _ptr(b),
                                      sh, sw, ph, pw, dt, dh, dw, _ptr(y))
    if rc != 0:
        raise ValueError("oracle_causal_conv3d rejected its arguments")
    return y


def causal_conv3d_points(x, w, flat_idx, bias=None, cache=None, stride=(1, 1), pad=(1, 1),
                         dil=(1, 1, 1)) -> np.ndarray:
    """Same definition as :func:`causal_conv3d`, evaluated only at the given
    flat indices of the NCTHW output."""
    x, w, b, c, (N, C, T, H, W), (Cout, kT, kH, kW), (sh, sw, ph, pw, dt, dh, dw), past = \
        _conv_args(x, w, bias, cache, stride, pad, dil)
    idx = np.ascontiguousarray(np.asarray(flat_idx, dtype=np.int64).ravel())
    out = np.empty(idx.shape[0], dtype=np.float64)
    rc = _load().oracle_causal_conv3d_points(
        _ptr(x), N, C, T, H, W, _ptr(c), past if c is not None else 0,
        _ptr(w), Cout, kT, kH, kW, _ptr(b), sh, sw, ph, pw, dt, dh, dw,
        idx.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)), idx.shape[0], _ptr(out))
    if rc != 0:
        raise ValueError("oracle_causal_conv3d_points rejected its arguments")
    return out


def strided_out_frames(t: int, stride_t: int, t_phase: int = 0) -> int:
    """Output frames of a t-frame chunk under temporal stride ``stride_t``
    when ``t_phase`` sequence frames (mod stride_t) came before it."""
    return int(_load().oracle_strided_out_frames(t, stride_t, t_phase))


def causal_conv3d_strided(x, w, bias=None, cache=None, stride=(1, 1, 1), pad=(1, 1),
                          pad_extra=(0, 0), dil=(1, 1, 1), t_phase: int = 0) -> np.ndarray:
    """Causal Conv3D with temporal stride and trailing spatial zero padding,
    fp64 ("Cosmos3 Wan VAE ...", section 10.5, the downsample path; see
    oracle_causal_conv3d_strided in oracle.c for the definition).

    ``stride`` = (st, sh, sw); ``pad`` = symmetric (ph, pw); ``pad_extra`` =
    extra zero rows below / columns right of the frame; ``t_phase`` = number
    of sequence frames before this chunk, modulo st.  ``cache`` as for
    :func:`causal_conv3d`.
    """
    st, sh, sw = stride
    x, w, b, c, (N, C, T, H, W), (Cout, kT, kH, kW), (_, _, ph, pw, dt, dh, dw), past = \
        _conv_args(x, w, bias, cache, (sh, sw), pad, dil)
    eh, ew = pad_extra
    lib = _load()
    To = lib.oracle_strided_out_frames(T, st, t_phase)
    Ho = lib.oracle_strided_out_size(H, kH, sh, ph, eh, dh)
    Wo = lib.oracle_strided_out_size(W, kW, sw, pw, ew, dw)
    if To < 0:
        raise ValueError("bad temporal stride or phase")
    y = np.empty((N, Cout, To, Ho, Wo), dtype=np.float64)
    if N * To == 0:
        return y
    rc = lib.oracle_causal_conv3d_strided(_ptr(x), N, C, T, H, W, _ptr(c),
                                          past if c is not None else 0, _ptr(w), Cout, kT, kH, kW,
                                          _ptr(b), st, t_phase, sh, sw, ph, pw, eh, ew, dt, dh, dw,
                                          _ptr(y))
    if rc != 0:
        raise ValueError("oracle_causal_conv3d_strided rejected its arguments")
    return y


def downsample3d(x, p: dict, cache=None, t_phase: int = 0, temporal: bool = True,
                 pad=(0, 0), pad_extra=(1, 1), bf16: bool = False):
    """The downsample path of "Cosmos3 Wan VAE ...", section 10.5, on one
    chunk: per frame a zero pad and a 3x3 stride-2 conv (``p["w_s"]``,
    [C, C, 1, 3, 3], bias ``p["b_s"]``) halve H and W; then, when
    ``temporal``, the causal 3x1x1 conv with temporal stride 2 (``p["w_t"]``,
    [C, C, 3, 1, 1], bias ``p["b_t"]``) halves T, reading ``cache`` (the
    last 2 frames of its input before this chunk) and anchoring at phase
    ``t_phase``.  The zero pad is ``pad`` on every side plus ``pad_extra``
    below and to the right.  With ``bf16`` the intermediate is rounded to
    bf16, as it is stored.  Returns (y, next_cache)."""
    s = causal_conv3d_strided(x, p["w_s"], p.get("b_s"), stride=(1, 2, 2), pad=pad,
                              pad_extra=pad_extra)
    s = _maybe_round(s, bf16)
    if not temporal:
        return s, None
    y = causal_conv3d_strided(s, p["w_t"], p.get("b_t"), cache=cache, stride=(2, 1, 1),
                              pad=(0, 0), t_phase=t_phase)
    return _maybe_round(y, bf16), next_cache(cache, s)


def rms_norm(x, gamma, beta=None, eps: float = DEFAULT_EPS) -> np.ndarray:
    """Channel L2/RMS norm, "Cosmos3 Wan VAE ...", section 10.2:
    v / max(||v||_2, eps) * sqrt(C) * gamma + beta over dim C of NCTHW."""
    x = _f64(x)
    N, C, T, H, W = x.shape
    g = _f64(gamma).reshape(C)
    b = None if beta is None else _f64(beta).reshape(C)
    y = np.empty_like(x)
    if x.size == 0:
        return y
    rc = _load().oracle_rms_norm(_ptr(x), N, C, T, H, W, _ptr(g), _ptr(b), float(eps), _ptr(y))
    if rc != 0:
        raise ValueError("oracle_rms_norm rejected its arguments")
    return y


def silu(x) -> np.ndarray:
    """x * sigmoid(x), "Cosmos3 Wan VAE ...", section 10.4."""
    x = _f64(x)
    y = np.empty_like(x)
    _load().oracle_silu(_ptr(x), x.size, _ptr(y))
    return y


def upsample_nearest2x(x) -> np.ndarray:
    """Nearest 2x upsample in H and W, none in T (plainest reading)."""
    x = _f64(x)
    N, C, T, H, W = x.shape
    y = np.empty((N, C, T, 2 * H, 2 * W), dtype=np.float64)
    _load().oracle_upsample_nearest2x(_ptr(x), N, C, T, H, W, _ptr(y))
    return y


def round_bf16(x) -> np.ndarray:
    """Round to the nearest bfloat16 value (ties to even), returned as fp64."""
    x = _f64(x)
    y = np.empty_like(x)
    _load().oracle_round_bf16(_ptr(x), x.size, _ptr(y))
    return y


def next_cache(cache_in, x, frames: int = CACHE_T) -> np.ndarray:
    """The cache a causal conv leaves behind: the last ``frames`` frames of
    concat_T(cache_in, x) ("Cosmos3 Wan VAE ...", sections 8.5 and 10.3: the
    cached frames are concatenated in front of the chunk).  ``cache_in`` None
    means a fresh sequence (all-zero past)."""
    x = _f64(x)
    N, C, T, H, W = x.shape
    if cache_in is None:
        cache_in = np.zeros((N, C, frames, H, W))
    full = np.concatenate([_f64(cache_in), x], axis=2)
    return np.ascontiguousarray(full[:, :, full.shape[2] - frames:])


def _maybe_round(a, bf16: bool):
    return round_bf16(a) if bf16 else a


def norm_silu(x, gamma, beta=None, eps=DEFAULT_EPS, bf16: bool = False):
    """RMS norm then SiLU; in bf16 mode rounded once where the GPU stores it."""
    return _maybe_round(silu(rms_norm(x, gamma, beta, eps)), bf16)


def resblock(x, p: dict, cache1=None, cache2=None, bf16: bool = False, eps=DEFAULT_EPS):
    """Wan residual block, "Cosmos3 Wan VAE ...", section 10.4:
    norm1 -> SiLU -> conv1 (3x3x3 causal) -> norm2 -> SiLU -> Dropout (identity at
    inference) -> conv2 (3x3x3 causal), plus the shortcut (identity when
    C_in == C_out, else a 1x1x1 causal conv), added after conv2.

    ``p`` holds gamma1, beta1, w1, b1, gamma2, beta2, w2, b2 and optionally
    w_short, b_short.  ``cache1``/``cache2`` are the 2-frame caches of the two
    3x3x3 convs (their inputs, i.e. post norm+SiLU), None for a fresh sequence.
    In bf16 mode every stored tensor (norm outputs, conv1 output, block
    output) is rounded to bf16, as the GPU stores them.
    Returns (y, next_cache1, next_cache2).
    """
    h1 = norm_silu(x, p["gamma1"], p.get("beta1"), eps, bf16)
    a1 = _maybe_round(causal_conv3d(h1, p["w1"], p.get("b1"), cache=_zero_if_none(cache1, h1)), bf16)
    h2 = norm_silu(a1, p["gamma2"], p.get("beta2"), eps, bf16)
    if p.get("w_short") is not None:
        sc = _maybe_round(causal_conv3d(x, p["w_short"], p.get("b_short"), pad=(0, 0)), bf16)
    else:
        sc = _f64(x)
    a2 = causal_conv3d(h2, p["w2"], p.get("b2"), cache=_zero_if_none(cache2, h2))
    y = _maybe_round(a2 + sc, bf16)
    return y, next_cache(cache1, h1), next_cache(cache2, h2)


def _zero_if_none(cache, like):
    if cache is not None:
        return cache
    N, C, T, H, W = np.shape(like)
    return np.zeros((N, C, CACHE_T, H, W))


def decoder_stack(latent, p: dict, bf16: bool = False, eps=DEFAULT_EPS):
    """Decoder-shaped stack over a whole latent sequence (causal, so the whole
    sequence equals frame-by-frame streaming with per-layer caches):
    conv_in (3x3x3) -> resblock -> resblock -> nearest 2x spatial upsample ->
    conv_up (3x3x3) -> resblock -> resblock.

    ``p``: w_in, b_in, rb0..rb3 (resblock dicts), w_up, b_up.
    """
    h = _maybe_round(causal_conv3d(latent, p["w_in"], p.get("b_in")), bf16)
    for k in (0, 1):
        h, _, _ = resblock(h, p[f"rb{k}"], bf16=bf16, eps=eps)
    h = upsample_nearest2x(h)
    h = _maybe_round(causal_conv3d(h, p["w_up"], p.get("b_up")), bf16)
    for k in (2, 3):
        h, _, _ = resblock(h, p[f"rb{k}"], bf16=bf16, eps=eps)
    return h


def tile_origins(size: int, tile: int, stride: int) -> list:
    """Start offsets of overlapping tiles along one axis ("VSR Hover
    Comparison", the decoder-tiling paragraph: tile_size (60, 104) with
    tile_stride (30, 52) on the latent).  Reading (the page gives size and
    stride only): tiles start at 0, stride, 2*stride, ... while they fit, and
    one more tile is aligned to the far edge if the last one stops short of
    it; a frame no larger than the tile is one tile."""
    if size <= tile:
        return [0]
    starts = list(range(0, size - tile + 1, stride))
    if starts[-1] + tile < size:
        starts.append(size - tile)
    return starts


def ramp_weights(length: int, ramp_lo: int, ramp_hi: int) -> np.ndarray:
    """Per-pixel blend weight along one axis of a tile of ``length`` output
    pixels ("VSR Hover Comparison": tiles are fused with complementary linear
    ramp weights).  Over the ``ramp_lo`` pixels it shares with the previous
    tile the weight rises as (i + 1/2) / ramp_lo; over the ``ramp_hi`` pixels it
    shares with the next tile it falls as (length - i - 1/2) / ramp_hi;
    elsewhere it is 1.  Across one overlap the two tiles' weights sum to 1."""
    i = np.arange(length, dtype=np.float64)
    w = np.ones(length)
    if ramp_lo > 0:
        w = np.where(i < ramp_lo, (i + 0.5) / ramp_lo, w)
    if ramp_hi > 0:
        w = np.where(i >= length - ramp_hi, w * (length - i - 0.5) / ramp_hi, w)
    return w


def blend_tiles(tiles, origins, out_hw, scale: int = 1) -> np.ndarray:
    """Blend overlapping output tiles into one frame: each tile [N, C, T, h, w]
    at latent origin (y0, x0) covers output rows scale*y0 ... of ``out_hw``;
    its weight is the product of the row and column ramps over the overlaps
    with its neighbours (overlap lengths taken from the other origins); the
    result is sum(weight * tile) / sum(weight) per output pixel."""
    H, W = out_hw
    ys = sorted({o[0] for o in origins})
    xs = sorted({o[1] for o in origins})
    first = np.asarray(tiles[0])
    N, C, T = first.shape[:3]
    acc = np.zeros((N, C, T, H, W))
    wsum = np.zeros((H, W))
    for tile, (y0, x0) in zip(tiles, origins):
        tile = np.asarray(tile, dtype=np.float64)
        h, w = tile.shape[3:]
        oy, ox = scale * y0, scale * x0
        iy, ix = ys.index(y0), xs.index(x0)
        # overlaps (output pixels) with the neighbouring tiles on each side
        top = (scale * ys[iy - 1] + h) - oy if iy > 0 else 0
        bottom = (oy + h) - scale * ys[iy + 1] if iy + 1 < len(ys) else 0
        left = (scale * xs[ix - 1] + w) - ox if ix > 0 else 0
        right = (ox + w) - scale * xs[ix + 1] if ix + 1 < len(xs) else 0
        if min(top, bottom, left, right) < 0:
            raise ValueError("tiles leave a gap: the stride must not exceed the tile")
        wgt = np.outer(ramp_weights(h, top, bottom), ramp_weights(w, left, right))
        acc[:, :, :, oy:oy + h, ox:ox + w] += wgt * tile
        wsum[oy:oy + h, ox:ox + w] += wgt
    return acc / wsum


def tiled_decoder_stack(latent, p: dict, tile=(60, 104), stride=(30, 52), bf16: bool = False,
                        eps=DEFAULT_EPS):
    """Decode ``latent`` tile by tile ("VSR Hover Comparison": spatial tiles of
    the latent, each decoded on its own, fused with ramp weights): every tile
    goes through :func:`decoder_stack` over all frames from zero caches, and
    the 2x-upsampled outputs are blended with :func:`blend_tiles`.  With
    ``bf16`` each tile's output is rounded as stored and the blend result is
    rounded once."""
    latent = _f64(latent)
    N, C, T, H, W = latent.shape
    th, tw = min(tile[0], H), min(tile[1], W)
    origins = [(y, x) for y in tile_origins(H, th, stride[0]) for x in tile_origins(W, tw, stride[1])]
    outs = [decoder_stack(latent[:, :, :, y:y + th, x:x + tw], p, bf16=bf16, eps=eps)
            for y, x in origins]
    y = blend_tiles(outs, origins, (2 * H, 2 * W), scale=2)
    return _maybe_round(y, bf16)


# ---------------------------------------------------------------------------
# 8-bit (E4M3) quantised conv: "Cosmos3 Wan VAE ...", sections 7 and 9 (8-bit
# weights and activations as the byte reduction of the 16-bit engine), in the
# OCP OFP8 E4M3 format (codec in oracle.c).
# ---------------------------------------------------------------------------
E4M3_MAX = 448.0


def e4m3_decode(codes) -> np.ndarray:
    """E4M3 codes (uint8) -> their real values (fp64; NaN for the NaN codes)."""
    c = np.ascontiguousarray(np.asarray(codes, dtype=np.uint8))
    y = np.empty(c.shape, dtype=np.float64)
    _load().oracle_e4m3_decode(c.ctypes.data_as(ctypes.POINTER(ctypes.c_uint8)), c.size, _ptr(y))
    return y


def e4m3_encode(x) -> np.ndarray:
    """Nearest E4M3 code, ties to even, saturating at +-448 (uint8)."""
    x = _f64(x)
    c = np.empty(x.shape, dtype=np.uint8)
    _load().oracle_e4m3_encode(_ptr(x), x.size, c.ctypes.data_as(ctypes.POINTER(ctypes.c_uint8)))
    return c


def e4m3_scaled_input(x, scale) -> np.ndarray:
    """The value a quantiser rounds: x times the reciprocal of the scale, both
    the reciprocal and the product in fp32 (the pages fix no arithmetic for
    the quantiser; this reading makes the rounding decision reproducible)."""
    x32 = np.asarray(x, dtype=np.float32)
    r = np.float32(1.0) / np.asarray(scale, dtype=np.float32)
    return (x32 * r).astype(np.float64)


def quantize_e4m3(x, scale: float) -> np.ndarray:
    """Per-tensor quantisation: codes = E4M3(fl32(x * fl32(1/scale)))."""
    return e4m3_encode(e4m3_scaled_input(x, np.float32(scale)))


def quantize_rows_e4m3(w2d):
    """Per-row (per output channel) absmax quantisation of a [rows, cols]
    matrix: scale_r = fl32(amax_r / 448) (1 when the row is all zero), codes
    = E4M3(fl32(w * fl32(1/scale_r))).  Returns (codes uint8, scales fp32)."""
    w32 = np.asarray(w2d, dtype=np.float32)
    amax = np.max(np.abs(w32), axis=1)
    scale = (amax / np.float32(E4M3_MAX)).astype(np.float32)
    scale[amax == 0] = np.float32(1.0)
    return e4m3_encode(e4m3_scaled_input(w32, scale[:, None])), scale


def quantize_conv_weights_e4m3(w):
    """[C_out, C_in, kT, kH, kW] weights -> (codes of the same shape, scales
    [C_out]) with one scale per output channel over its C_in*kT*kH*kW taps."""
    w = np.asarray(w)
    codes, scale = quantize_rows_e4m3(w.reshape(w.shape[0], -1))
    return codes.reshape(w.shape), scale


def causal_conv3d_e4m3(xq, x_scale, wq, w_scale, bias=None, cache_q=None, residual=None):
    """Causal 3x3x3 conv of E4M3 operands: the codes are decoded exactly, the
    activations (chunk and cache) times the one per-tensor scale, the weights
    times the scale of their output channel; then the conv of section 10.3
    (``causal_conv3d``) in fp64, the bias once, and the residual after it."""
    x = e4m3_decode(xq) * float(x_scale)
    w = e4m3_decode(wq) * np.asarray(w_scale, dtype=np.float64)[:, None, None, None, None]
    cache = None if cache_q is None else e4m3_decode(cache_q) * float(x_scale)
    y = causal_conv3d(x, w, bias, cache)
    if residual is not None:
        y = y + _f64(residual)
    return y


def causal_conv3d_e4m3_points(xq, x_scale, wq, w_scale, flat_idx, bias=None, cache_q=None,
                              residual=None):
    """:func:`causal_conv3d_e4m3` evaluated only at the given flat indices of
    the NCTHW output."""
    x = e4m3_decode(xq) * float(x_scale)
    w = e4m3_decode(wq) * np.asarray(w_scale, dtype=np.float64)[:, None, None, None, None]
    cache = None if cache_q is None else e4m3_decode(cache_q) * float(x_scale)
    y = causal_conv3d_points(x, w, flat_idx, bias, cache)
    if residual is not None:
        y = y + _f64(residual).ravel()[np.asarray(flat_idx, dtype=np.int64).ravel()]
    return y


def norm_silu_e4m3(x, gamma, beta=None, scale: float = 1.0, eps=DEFAULT_EPS):
    """RMS norm + SiLU quantised to E4M3 with a per-tensor scale.  Returns
    (v, codes): v = norm_silu(x) / scale in fp64, the value the quantiser
    rounds, and its codes.  The GPU computes v in fp32, so a code may differ
    where v lies within fp32 error of a rounding boundary; the tests compare
    against v for that reason."""
    v = norm_silu(x, gamma, beta, eps) / float(scale)
    return v, e4m3_encode(v)


def resblock_e4m3(x, p: dict, s1: float, s2: float, eps=DEFAULT_EPS):
    """The residual block of section 10.4 on the 8-bit path, over a whole
    sequence from a fresh cache (identity shortcut): norm1 + SiLU quantised at
    activation scale s1, the E4M3 conv1 with per-output-channel weight scales,
    rounded to bf16 where it is stored; norm2 + SiLU quantised at s2, the E4M3
    conv2, plus the block input, rounded to bf16."""
    x = _f64(x)
    w1q, w1s = quantize_conv_weights_e4m3(p["w1"])
    w2q, w2s = quantize_conv_weights_e4m3(p["w2"])
    _, q1 = norm_silu_e4m3(x, p["gamma1"], p.get("beta1"), s1, eps)
    h = round_bf16(causal_conv3d_e4m3(q1, s1, w1q, w1s, p.get("b1")))
    _, q2 = norm_silu_e4m3(h, p["gamma2"], p.get("beta2"), s2, eps)
    return round_bf16(causal_conv3d_e4m3(q2, s2, w2q, w2s, p.get("b2"), None, x))


def decoder_stack_e4m3(latent, p: dict, scales: dict, eps=DEFAULT_EPS):
    """``decoder_stack`` on the 8-bit path, over the whole sequence: conv_in and
    conv_up read their input quantised at ``scales["in"]`` / ``scales["up"]``
    (``quantize_e4m3``) with per-output-channel weight scales, rounded to bf16
    where stored; the residual blocks are ``resblock_e4m3`` with
    ``scales["rb"][k]`` = (s1, s2)."""
    def conv8(x, w, b, s):
        wq, ws = quantize_conv_weights_e4m3(w)
        return round_bf16(causal_conv3d_e4m3(quantize_e4m3(x, s), s, wq, ws, b))

    h = conv8(_f64(latent), p["w_in"], p.get("b_in"), scales["in"])
    for k in (0, 1):
        h = resblock_e4m3(h, p[f"rb{k}"], *scales["rb"][k], eps=eps)
    h = upsample_nearest2x(h)
    h = conv8(h, p["w_up"], p.get("b_up"), scales["up"])
    for k in (2, 3):
        h = resblock_e4m3(h, p[f"rb{k}"], *scales["rb"][k], eps=eps)
    return h


def rel_l2(y, ref) -> float:
    """||y - ref||_2 / ||ref||_2 in fp64."""
    y = np.asarray(y, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    den = np.linalg.norm(ref.ravel())
    num = np.linalg.norm((y - ref).ravel())
    return float(num / den) if den > 0 else float(num)


def max_abs(y, ref) -> float:
    return float(np.max(np.abs(np.asarray(y, np.float64) - np.asarray(ref, np.float64)))) \
        if np.size(ref) else 0.0
