"""Pins for the oracle's channel RMS norm, SiLU, upsample and bf16 rounding.

RMS norm ("Cosmos3 Wan VAE -- engine size vs runtime context memory",
section 10.2): closed forms (unit RMS with gamma=1, beta=0; scale invariance;
constant vectors; the all-zero vector) and the library routine the page names
(torch.nn.functional.normalize over dim 1, fp64).  SiLU (same page, section
10.4): SiLU(0) = 0, SiLU(u) - SiLU(-u) = u, torch.nn.functional.silu in fp64.
Nearest 2x upsample: torch.nn.functional.interpolate.  bf16 rounding: torch's
float32 -> bfloat16 conversion and hand-worked tie cases of the format.
"""
import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
from video_vae_causal_amd import inputs

RNG = np.random.default_rng(99)


def test_rms_unit_rms_with_unit_gamma():
    C = 48
    x = RNG.standard_normal((2, C, 3, 4, 5))
    y = oracle.rms_norm(x, np.ones(C))
    np.testing.assert_allclose((y ** 2).sum(axis=1), C, rtol=1e-13)


def test_rms_scale_invariance():
    C = 16
    x = RNG.standard_normal((1, C, 2, 3, 3))
    g = 1 + 0.1 * RNG.standard_normal(C)
    b = RNG.standard_normal(C)
    np.testing.assert_allclose(oracle.rms_norm(3.7 * x, g, b), oracle.rms_norm(x, g, b), rtol=1e-13)


def test_rms_constant_and_zero_vectors():
    C = 12
    g = 1 + 0.1 * RNG.standard_normal(C)
    b = RNG.standard_normal(C)
    x = np.zeros((1, C, 1, 1, 3))
    x[:, :, :, :, 0] = 2.5
    x[:, :, :, :, 1] = -0.25
    y = oracle.rms_norm(x, g, b)
    np.testing.assert_allclose(y[0, :, 0, 0, 0], g + b, rtol=1e-13)
    np.testing.assert_allclose(y[0, :, 0, 0, 1], -g + b, rtol=1e-13)
    np.testing.assert_array_equal(y[0, :, 0, 0, 2], b)      # all-zero vector -> beta
    np.testing.assert_array_equal(oracle.rms_norm(x, g)[0, :, 0, 0, 2], 0.0)


def test_rms_matches_torch_normalize():
    C = 96
    x = RNG.standard_normal((1, C, 3, 5, 7))
    g = 1 + 0.02 * RNG.standard_normal(C)
    b = 0.1 * RNG.standard_normal(C)
    ref = F.normalize(torch.from_numpy(x), dim=1, eps=1e-12) * np.sqrt(C) \
        * torch.from_numpy(g)[None, :, None, None, None] + torch.from_numpy(b)[None, :, None, None, None]
    np.testing.assert_allclose(oracle.rms_norm(x, g, b), ref.numpy(), rtol=1e-13, atol=1e-14)


def test_silu_closed_forms_and_torch():
    u = np.concatenate([RNG.standard_normal(1000) * 5, [0.0, 40.0, -40.0, 1e-9]])
    s = oracle.silu(u)
    assert oracle.silu(np.array([0.0]))[0] == 0.0
    np.testing.assert_allclose(s - oracle.silu(-u), u, rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(s, F.silu(torch.from_numpy(u)).numpy(), rtol=1e-14, atol=1e-300)


def test_upsample_matches_interpolate():
    x = RNG.standard_normal((1, 3, 2, 4, 5))
    ref = F.interpolate(torch.from_numpy(x), scale_factor=(1, 2, 2), mode="nearest").numpy()
    np.testing.assert_array_equal(oracle.upsample_nearest2x(x), ref)


def test_round_bf16_matches_torch_on_float32_values():
    a = (RNG.standard_normal(100000) * np.exp(RNG.uniform(-30, 30, 100000))).astype(np.float32)
    ref = torch.from_numpy(a).to(torch.bfloat16).to(torch.float64).numpy()
    np.testing.assert_array_equal(oracle.round_bf16(a.astype(np.float64)), ref)


def test_round_bf16_ties_and_limits():
    e = 2.0 ** -8
    cases = {
        1.0 + e: 1.0,                       # halfway, even neighbour is 1.0
        1.0 + 3 * e: 1.0 + 4 * e,           # halfway, even neighbour above
        1.0 + e * 1.0001: 1.0 + 2 * e,      # just above halfway
        -(1.0 + 3 * e): -(1.0 + 4 * e),
        2.0 ** -133: 2.0 ** -133,           # smallest subnormal survives
        2.0 ** -134: 0.0,                   # half of it ties to zero
        3 * 2.0 ** -134: 2.0 ** -132,
        255 * 2.0 ** 120: 255 * 2.0 ** 120,  # largest finite
        3.4e38: np.inf,
        0.0: 0.0,
    }
    x = np.array(list(cases.keys()))
    np.testing.assert_array_equal(oracle.round_bf16(x), np.array(list(cases.values())))


def test_generator_bf16_matches_torch():
    a = inputs.normal((50000,), 7, "t", std=3.0)
    q = inputs.quantize(a, "bf16")
    ref = torch.from_numpy(a).to(torch.bfloat16).to(torch.float32).numpy()
    np.testing.assert_array_equal(q, ref)


def test_generator_is_seeded_and_streams_differ():
    a = inputs.normal((1000,), 3, "x")
    np.testing.assert_array_equal(a, inputs.normal((1000,), 3, "x"))
    assert not np.array_equal(a, inputs.normal((1000,), 3, "y"))
    assert not np.array_equal(a, inputs.normal((1000,), 4, "x"))
    assert abs(a.mean()) < 0.1 and abs(a.std() - 1) < 0.1
