"""Work and byte accounting for the causal video-VAE hot path.

The conv is counted as the pages count it ("Cosmos3 Wan VAE -- engine size vs
runtime context memory", section 10.3, Conv3D as GEMM): M = B*T'*H'*W' output
positions, K = C_in*kT*kH*kW, N = C_out, FLOPs = 2*M*K*N, over every tap
including taps that land in the zero padding.

Algorithmic bytes are the compulsory HBM traffic of one launch: every input
element read once, every output element written once (bf16 = 2 B, fp32 = 4 B).
"""
from __future__ import annotations

from typing import Tuple

DTYPE_BYTES = {"bf16": 2, "f32": 4}


def conv_gemm_dims(n: int, t: int, h_out: int, w_out: int, c_in: int, c_out: int,
                   k: Tuple[int, int, int]) -> Tuple[int, int, int]:
    m = n * t * h_out * w_out
    kk = c_in * k[0] * k[1] * k[2]
    return m, kk, c_out


def conv_flops(n, t, h_out, w_out, c_in, c_out, k=(3, 3, 3)) -> int:
    m, kk, nn = conv_gemm_dims(n, t, h_out, w_out, c_in, c_out, k)
    return 2 * m * kk * nn


def tensor_bytes(shape, dtype: str = "bf16") -> int:
    e = 1
    for s in shape:
        e *= int(s)
    return e * DTYPE_BYTES[dtype]


def conv_launch_bytes(n, t, h, w, c_in, c_out, k=(3, 3, 3), dtype="bf16",
                      residual: bool = False, cache_frames: int = 2,
                      cache_out_frames: int = 0) -> int:
    """Compulsory bytes of one conv launch over a t-frame chunk: the chunk, the
    cache_frames past frames it reads, the weights and bias, the output chunk
    (and the residual when fused), and the cache_out_frames frames of the
    next cache it writes."""
    e = DTYPE_BYTES[dtype]
    plane_in = n * h * w * c_in
    plane_out = n * h * w * c_out
    b = (t + cache_frames) * plane_in * e
    b += c_out * c_in * k[0] * k[1] * k[2] * e + c_out * e
    b += t * plane_out * e
    if residual:
        b += t * plane_out * e
    b += cache_out_frames * plane_in * e
    return b


def norm_bytes(elements: int, dtype: str = "bf16", residual: bool = False) -> int:
    """Channel RMS norm (+SiLU): read x once, write y once (+ residual read)."""
    e = DTYPE_BYTES[dtype]
    return elements * e * (3 if residual else 2)


def latent_frames(video_frames: int, temporal_factor: int = 4) -> int:
    """Causal temporal compression: the first frame alone, then groups of
    ``temporal_factor`` frames ("diffusion inference workload anatomy", the
    two-compressions paragraph: 81 frames give 80/4 + 1 = 21 latent frames)."""
    return (video_frames - 1) // temporal_factor + 1
