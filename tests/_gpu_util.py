"""Helpers for the GPU parity tests: host<->device layout plumbing, the
tolerances, and point-sampled oracle evaluation.  Inputs always come from the
seeded generator; expected values always come from the oracle."""
from __future__ import annotations

import numpy as np
import torch

import oracle

# bf16: relative L2 <= 1e-2 and max-abs <= 2e-2 * max|ref|; fp32: relative L2 <= 1e-5.
BF16_REL_L2 = 1e-2
BF16_MAX_ABS_FRAC = 2e-2
F32_REL_L2 = 1e-5


def dev():
    return torch.device("cuda:0")


def to_dev(a: np.ndarray, dtype=torch.bfloat16) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(dev())
    t = t.to(dtype)
    if t.dim() == 5:
        t = t.contiguous(memory_format=torch.channels_last_3d)
    return t


def to_host(t: torch.Tensor) -> np.ndarray:
    return t.float().cpu().numpy().astype(np.float64)


def f64(a) -> np.ndarray:
    return np.asarray(a, dtype=np.float64)


def check_bf16(y, ref, what=""):
    rel = oracle.rel_l2(y, ref)
    mx = oracle.max_abs(y, ref)
    bound = BF16_MAX_ABS_FRAC * float(np.max(np.abs(ref)))
    print(f"[parity] {what} rel_l2={rel:.3e} max_abs={mx:.3e} (bound {bound:.3e})", flush=True)
    assert rel <= BF16_REL_L2, f"{what}: rel L2 {rel}"
    assert mx <= bound, f"{what}: max abs {mx} > {bound}"
    return rel


def check_f32(y, ref, what=""):
    rel = oracle.rel_l2(y, ref)
    print(f"[parity] {what} rel_l2={rel:.3e}", flush=True)
    assert rel <= F32_REL_L2, f"{what}: rel L2 {rel}"
    return rel


def frame_points(c, h, w, count, seed):
    """Random (channel, row, col) triples plus the full border of two channels."""
    g = np.random.default_rng(seed)
    co = g.integers(0, c, count)
    hh = g.integers(0, h, count)
    ww = g.integers(0, w, count)
    bh, bw = np.meshgrid(np.arange(h), np.arange(w), indexing="ij")
    border = (bh == 0) | (bh == h - 1) | (bw == 0) | (bw == w - 1)
    for ch in g.integers(0, c, 2):
        co = np.concatenate([co, np.full(border.sum(), ch)])
        hh = np.concatenate([hh, bh[border]])
        ww = np.concatenate([ww, bw[border]])
    return co, hh, ww


def oracle_conv_at_frame(x_window, w, b, co, hh, ww):
    """Oracle causal conv outputs at the LAST frame of ``x_window`` (which holds
    the frames the output reads: up to two past frames and the current one;
    fewer at the sequence start, where the causal zero padding applies)."""
    N, C, T, H, W = x_window.shape
    Cout = w.shape[0]
    t = T - 1
    flat = (((0 * Cout + co) * T + t) * H + hh) * W + ww
    return oracle.causal_conv3d_points(f64(x_window), f64(w), flat.astype(np.int64),
                                       None if b is None else f64(b))
