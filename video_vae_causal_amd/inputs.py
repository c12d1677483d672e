"""Seeded synthetic inputs for the causal video-VAE hot path.

This module is the only code that both the GPU path's tests/bench and the CPU
oracle consume.  It holds none of the method's arithmetic: it draws seeded
normal numbers, rounds them to the storage type, and describes workload shapes.

Generator: numpy's Philox4x64 counter-based bit generator, keyed per tensor by
(seed, crc32(tensor name)), drawing standard normals in float32; values for
bf16 workloads are then rounded to bfloat16 (round to nearest, ties to even)
so that the host copy holds exactly the values the device receives.

Distribution notation: ``N(0, s)`` is read as mean 0, standard deviation s.
Weights of a conv with C_in input channels and a kT x kH x kW kernel are drawn
with std 1/sqrt(C_in*kT*kH*kW); biases with std 0.1; norm scales gamma as
1 + 0.02 * N(0,1); norm shifts beta are absent (zero) unless asked for.
All arrays are in the logical NCTHW layout.
"""
from __future__ import annotations

import zlib
from dataclasses import dataclass, field
from typing import Dict, List, Optional, Tuple

import numpy as np


def _gen(seed: int, name: str) -> np.random.Generator:
    key = np.array([np.uint64(seed), np.uint64(zlib.crc32(name.encode()))], dtype=np.uint64)
    return np.random.Generator(np.random.Philox(key=key))


def normal(shape, seed: int, name: str, std: float = 1.0, mean: float = 0.0) -> np.ndarray:
    """float32 array of N(mean, std) values from the (seed, name) stream."""
    g = _gen(seed, name)
    a = g.standard_normal(size=tuple(shape), dtype=np.float32)
    if std != 1.0:
        a *= np.float32(std)
    if mean != 0.0:
        a += np.float32(mean)
    return a


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bit patterns (uint16), round to nearest even."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    r = (u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def quantize(a: np.ndarray, dtype: str) -> np.ndarray:
    """Return float32 values exactly representable in ``dtype`` ('bf16'|'f32')."""
    if dtype == "f32":
        return np.ascontiguousarray(a, dtype=np.float32)
    if dtype == "bf16":
        return bf16_bits_to_f32(f32_to_bf16_bits(a))
    raise ValueError(dtype)


def conv_weight(cout: int, cin: int, k: Tuple[int, int, int], seed: int, name: str,
                dtype: str) -> np.ndarray:
    std = 1.0 / np.sqrt(cin * k[0] * k[1] * k[2])
    return quantize(normal((cout, cin) + tuple(k), seed, name, std=std), dtype)


def conv_bias(cout: int, seed: int, name: str, dtype: str) -> np.ndarray:
    return quantize(normal((cout,), seed, name, std=0.1), dtype)


def norm_gamma(c: int, seed: int, name: str, dtype: str) -> np.ndarray:
    return quantize(normal((c,), seed, name, std=0.02, mean=1.0), dtype)


def norm_beta(c: int, seed: int, name: str, dtype: str) -> np.ndarray:
    return quantize(normal((c,), seed, name, std=0.1), dtype)


def resblock_params(c: int, seed: int, prefix: str, dtype: str, with_beta: bool = False) -> Dict:
    p = {
        "gamma1": norm_gamma(c, seed, prefix + ".gamma1", dtype),
        "w1": conv_weight(c, c, (3, 3, 3), seed, prefix + ".w1", dtype),
        "b1": conv_bias(c, seed, prefix + ".b1", dtype),
        "gamma2": norm_gamma(c, seed, prefix + ".gamma2", dtype),
        "w2": conv_weight(c, c, (3, 3, 3), seed, prefix + ".w2", dtype),
        "b2": conv_bias(c, seed, prefix + ".b2", dtype),
    }
    if with_beta:
        p["beta1"] = norm_beta(c, seed, prefix + ".beta1", dtype)
        p["beta2"] = norm_beta(c, seed, prefix + ".beta2", dtype)
    return p


# --------------------------------------------------------------------------
# The five workloads.  Shapes follow the pages' workloads: the Wan encoder on a
# 1x3x17x480x832 video (feature maps of 96 channels at 480x832 and 384
# channels at 240x416), decoder tiles of 60x104 latent pixels, and a 48-channel
# latent of 21 frames (81 video frames).
# --------------------------------------------------------------------------

@dataclass
class Workload:
    name: str
    seed: int
    dtype: str
    description: str
    shapes: Dict[str, Tuple[int, ...]] = field(default_factory=dict)


WORKLOADS: Dict[str, Workload] = {
    "tiny_conv_f32": Workload(
        "tiny_conv_f32", 1, "f32",
        "causal Conv3D 16->16, 3x3x3, x[1,16,5,32,32] fp32; whole sequence and 1-frame chunks",
        {"x": (1, 16, 5, 32, 32)}),
    "resblock_384_60x104": Workload(
        "resblock_384_60x104", 2, "bf16",
        "Wan residual block C=384, 5 latent frames fed one at a time, 60x104, bf16",
        {"x": (1, 384, 5, 60, 104)}),
    "layer_96_480x832": Workload(
        "layer_96_480x832", 3, "bf16",
        "RMSNorm+SiLU then causal Conv3D 96->96 on x[1,96,17,480,832], chunks 1+4+4+4+4",
        {"x": (1, 96, 17, 480, 832)}),
    "layer_384_240x416": Workload(
        "layer_384_240x416", 4, "bf16",
        "causal Conv3D 384->384 on x[1,384,17,240,416] whole and frame by frame, then 1x1x1 384->192",
        {"x": (1, 384, 17, 240, 416)}),
    "decoder_stack_48_30x52": Workload(
        "decoder_stack_48_30x52", 5, "bf16",
        "latent[1,48,21,30,52] -> conv_in 48->384 -> 2 resblocks -> up2x -> conv 384 -> 2 resblocks",
        {"latent": (1, 48, 21, 30, 52)}),
}


def tiny_conv_inputs(seed: int = 1, shape=(1, 16, 5, 32, 32), dtype: str = "f32") -> Dict:
    n, c, t, h, w = shape
    return {
        "x": quantize(normal(shape, seed, "x"), dtype),
        "w": conv_weight(c, c, (3, 3, 3), seed, "w", dtype),
        "b": conv_bias(c, seed, "b", dtype),
    }


def resblock_inputs(seed: int = 2, shape=(1, 384, 5, 60, 104), dtype: str = "bf16",
                    with_beta: bool = False) -> Dict:
    c = shape[1]
    return {"x": quantize(normal(shape, seed, "x"), dtype),
            "p": resblock_params(c, seed, "rb", dtype, with_beta)}


def layer96_inputs(seed: int = 3, shape=(1, 96, 17, 480, 832), dtype: str = "bf16") -> Dict:
    c = shape[1]
    return {"x": quantize(normal(shape, seed, "x"), dtype),
            "gamma": norm_gamma(c, seed, "gamma", dtype),
            "w": conv_weight(c, c, (3, 3, 3), seed, "w", dtype),
            "b": conv_bias(c, seed, "b", dtype)}


def layer384_inputs(seed: int = 4, shape=(1, 384, 17, 240, 416), cproj: int = 192,
                    dtype: str = "bf16") -> Dict:
    c = shape[1]
    return {"x": quantize(normal(shape, seed, "x"), dtype),
            "w": conv_weight(c, c, (3, 3, 3), seed, "w", dtype),
            "b": conv_bias(c, seed, "b", dtype),
            "wp": conv_weight(cproj, c, (1, 1, 1), seed, "wp", dtype),
            "bp": conv_bias(cproj, seed, "bp", dtype)}


def decoder_inputs(seed: int = 5, shape=(1, 48, 21, 30, 52), width: int = 384,
                   dtype: str = "bf16", with_latent_window=None) -> Dict:
    """Decoder-stack weights and a latent of ``shape``; with
    ``with_latent_window`` = (h, w) only the top-left h x w window of that
    latent is returned (the same values, without generating the rest)."""
    cl = shape[1]
    p = {"w_in": conv_weight(width, cl, (3, 3, 3), seed, "w_in", dtype),
         "b_in": conv_bias(width, seed, "b_in", dtype),
         "w_up": conv_weight(width, width, (3, 3, 3), seed, "w_up", dtype),
         "b_up": conv_bias(width, seed, "b_up", dtype)}
    for k in range(4):
        p[f"rb{k}"] = resblock_params(width, seed, f"rb{k}", dtype)
    lat = quantize(normal(shape, seed, "latent"), dtype)
    if with_latent_window is not None:
        lat = np.ascontiguousarray(lat[:, :, :, :with_latent_window[0], :with_latent_window[1]])
    return {"latent": lat, "p": p}


def downsample_inputs(seed: int = 6, shape=(1, 96, 17, 480, 832), dtype: str = "bf16",
                      with_x: bool = True) -> Dict:
    """The encoder's downsample path at the pages' L0 feature-map size: the
    96-channel 17x480x832 map, a 1x3x3 stride-2 conv (spatial), a 3x1x1
    temporal-stride-2 conv, and the RMS-norm gammas before and after."""
    c = shape[1]
    d = {"gamma1": norm_gamma(c, seed, "gamma1", dtype),
         "w_s": conv_weight(c, c, (1, 3, 3), seed, "w_s", dtype),
         "b_s": conv_bias(c, seed, "b_s", dtype),
         "w_t": conv_weight(c, c, (3, 1, 1), seed, "w_t", dtype),
         "b_t": conv_bias(c, seed, "b_t", dtype),
         "gamma2": norm_gamma(c, seed, "gamma2", dtype)}
    if with_x:
        d["x"] = quantize(normal(shape, seed, "x"), dtype)
    return d


def e4m3_codes(shape, seed: int, name: str, exp_lo: int = 1, exp_hi: int = 14) -> np.ndarray:
    """Random 8-bit E4M3 codes (uint8): uniform sign and 3-bit mantissa, the
    4-bit exponent field uniform in [exp_lo, exp_hi] (exp_hi <= 14 never
    draws the NaN codes).  No arithmetic: the bits are drawn directly."""
    g = _gen(seed, name)
    sign = g.integers(0, 2, size=tuple(shape), dtype=np.uint8) << np.uint8(7)
    expo = g.integers(exp_lo, exp_hi + 1, size=tuple(shape), dtype=np.uint8) << np.uint8(3)
    mant = g.integers(0, 8, size=tuple(shape), dtype=np.uint8)
    return (sign | expo | mant).astype(np.uint8)


def e4m3_conv_inputs(seed: int = 7, shape=(1, 384, 17, 240, 416), cout: int = 384,
                     with_cache: bool = True, with_residual: bool = False) -> Dict:
    """Operands of an 8-bit causal 3x3x3 conv: activation and cache codes, weight
    codes [C_out, C_in, 3, 3, 3], a per-tensor activation scale, per-output-
    channel weight scales (float32, uniform in [0.5, 1.5] * 2^-4 / sqrt(27 C_in)
    so that the outputs stay O(1)), bias N(0, 0.1) and residual N(0, 1) in bf16."""
    n, c, t, h, w = shape
    g = _gen(seed, "scales")
    d = {
        "x": e4m3_codes(shape, seed, "x", 1, 12),
        "w": e4m3_codes((cout, c, 3, 3, 3), seed, "w", 1, 14),
        "x_scale": float(np.float32(2.0 ** -6)),
        "w_scale": (g.uniform(0.5, 1.5, cout) * 2.0 ** -4 / np.sqrt(27 * c)).astype(np.float32),
        "b": quantize(normal((cout,), seed, "b", std=0.1), "bf16"),
    }
    if with_cache:
        d["cache"] = e4m3_codes((n, c, 2, h, w), seed, "cache", 1, 12)
    if with_residual:
        d["res"] = quantize(normal((n, cout, t, h, w), seed, "res"), "bf16")
    return d


def sample_indices(shape: Tuple[int, ...], count: int, seed: int,
                   include_frames: Optional[List[int]] = None) -> np.ndarray:
    """Flat NCTHW indices for point-sampled checks: ``count`` uniformly random
    outputs plus every spatial border position of a few random channels in the
    frames listed in ``include_frames`` (so edges and frame starts are always
    covered)."""
    n, c, t, h, w = shape
    g = _gen(seed, "sample_indices")
    idx = [g.integers(0, n * c * t * h * w, size=count, dtype=np.int64)]
    for f in include_frames or []:
        chans = g.integers(0, c, size=4)
        for ch in chans:
            hh, ww = np.meshgrid(np.arange(h), np.arange(w), indexing="ij")
            border = (hh == 0) | (hh == h - 1) | (ww == 0) | (ww == w - 1)
            flat = (((0 * c + ch) * t + f) * h + hh[border]) * w + ww[border]
            idx.append(flat.astype(np.int64))
    return np.unique(np.concatenate(idx))
