"""Pins for the oracle's causal Conv3D (CPU only).

Each test checks the oracle against something other than itself:
  * a library routine the causal conv reduces to (torch.nn.functional.conv3d /
    conv2d in fp64 on an explicitly zero-padded input);
  * closed forms (impulse response, identity and shift kernels, constant input);
  * the invariants the pages state: the per-temporal-slice Conv2D sum equals
    the Conv3D with the bias added once ("cache-aware video decoder lowering",
    section on turning Conv3D into batched Conv2D), no future frame reaches an
    earlier output (same page), and chunked decoding with the cache equals one
    whole-sequence pass ("Cosmos3 Wan VAE -- engine size vs runtime context
    memory", section 10.3, causal padding);
  * a planted mistake (bias added per temporal slice) that the bias test must
    catch.
"""
import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle

RNG = np.random.default_rng(1234)


def rnd(*shape):
    return RNG.standard_normal(shape)


def torch_causal_reference(x, w, b, stride=(1, 1), pad=(1, 1), dil=(1, 1, 1), cache=None):
    """torch fp64 conv3d on the input padded explicitly: dil_t*(kT-1) past
    frames (zeros or the cache) in front, none behind, pad_h/pad_w zeros."""
    xt = torch.from_numpy(x)
    kT = w.shape[2]
    past = dil[0] * (kT - 1)
    N, C, T, H, W = x.shape
    if cache is None:
        front = torch.zeros((N, C, past, H, W), dtype=torch.float64)
    else:
        front = torch.from_numpy(cache)
    xt = torch.cat([front, xt], dim=2)
    xt = F.pad(xt, (pad[1], pad[1], pad[0], pad[0], 0, 0))
    y = F.conv3d(xt, torch.from_numpy(w), None if b is None else torch.from_numpy(b),
                 stride=(1,) + tuple(stride), dilation=tuple(dil))
    return y.numpy()


@pytest.mark.parametrize("k,stride,pad,dil", [
    ((3, 3, 3), (1, 1), (1, 1), (1, 1, 1)),
    ((3, 3, 3), (2, 2), (1, 1), (1, 1, 1)),
    ((3, 3, 3), (1, 2), (2, 0), (2, 2, 1)),
    ((1, 1, 1), (1, 1), (0, 0), (1, 1, 1)),
    ((2, 3, 1), (1, 1), (1, 0), (3, 1, 1)),
    ((3, 1, 3), (3, 1), (0, 2), (1, 1, 2)),
])
@pytest.mark.parametrize("with_bias", [True, False])
def test_matches_torch_conv3d_on_padded_input(k, stride, pad, dil, with_bias):
    x = rnd(2, 3, 6, 9, 11)
    w = rnd(4, 3, *k)
    b = rnd(4) if with_bias else None
    y = oracle.causal_conv3d(x, w, b, stride=stride, pad=pad, dil=dil)
    ref = torch_causal_reference(x, w, b, stride, pad, dil)
    assert y.shape == ref.shape
    np.testing.assert_allclose(y, ref, rtol=1e-12, atol=1e-12)


def test_matches_torch_with_cache():
    x = rnd(1, 3, 4, 7, 8)
    cache = rnd(1, 3, 2, 7, 8)
    w = rnd(5, 3, 3, 3, 3)
    b = rnd(5)
    y = oracle.causal_conv3d(x, w, b, cache=cache)
    ref = torch_causal_reference(x, w, b, cache=cache)
    np.testing.assert_allclose(y, ref, rtol=1e-12, atol=1e-12)


def test_impulse_response_closed_form():
    C, Co, T, H, W = 2, 3, 5, 6, 7
    w = rnd(Co, C, 3, 3, 3)
    b = rnd(Co)
    ci, t0, h0, w0 = 1, 2, 3, 0
    x = np.zeros((1, C, T, H, W))
    x[0, ci, t0, h0, w0] = 1.0
    y = oracle.causal_conv3d(x, w, b)
    expect = np.zeros((1, Co, T, H, W))
    for co in range(Co):
        for t in range(T):
            for h in range(H):
                for ww in range(W):
                    kt, kh, kw = t0 - t + 2, h0 - h + 1, w0 - ww + 1
                    if 0 <= kt < 3 and 0 <= kh < 3 and 0 <= kw < 3:
                        expect[0, co, t, h, ww] = w[co, ci, kt, kh, kw]
    np.testing.assert_allclose(y - b[None, :, None, None, None], expect, atol=1e-15)
    # kt = 2 multiplies the current frame: frames after t0+2 and before t0 see nothing
    assert np.all(y[:, :, :t0] == b[None, :, None, None, None])


def test_identity_and_shift_kernels():
    C, T, H, W = 3, 6, 5, 4
    x = rnd(2, C, T, H, W)
    b = rnd(C)
    ident = np.zeros((C, C, 3, 3, 3))
    shift = np.zeros((C, C, 3, 3, 3))
    for c in range(C):
        ident[c, c, 2, 1, 1] = 1.0   # current frame, centre tap
        shift[c, c, 0, 1, 1] = 1.0   # two frames back
    y = oracle.causal_conv3d(x, ident, b)
    np.testing.assert_array_equal(y, x + b[None, :, None, None, None])
    y = oracle.causal_conv3d(x, shift, b)
    bb = np.broadcast_to(b[None, :, None, None, None], (2, C, 2, H, W))
    np.testing.assert_array_equal(y[:, :, :2], bb)
    np.testing.assert_array_equal(y[:, :, 2:], x[:, :, :-2] + b[None, :, None, None, None])


def test_constant_input_closed_form():
    C, Co, T, H, W = 2, 2, 4, 5, 5
    w = rnd(Co, C, 3, 3, 3)
    b = rnd(Co)
    y = oracle.causal_conv3d(np.ones((1, C, T, H, W)), w, b)
    h, ww = 2, 2  # spatial interior
    for co in range(Co):
        assert np.isclose(y[0, co, 0, h, ww], b[co] + w[co, :, 2].sum(), rtol=1e-13)
        assert np.isclose(y[0, co, 1, h, ww], b[co] + w[co, :, 1:].sum(), rtol=1e-13)
        for t in range(2, T):
            assert np.isclose(y[0, co, t, h, ww], b[co] + w[co].sum(), rtol=1e-13)
        # corner (0,0): only kh, kw in {1,2} land inside the frame
        assert np.isclose(y[0, co, 3, 0, 0], b[co] + w[co, :, :, 1:, 1:].sum(), rtol=1e-13)


def _bias_per_slice_variant(x, w, b):
    """A planted mistake: the temporal-slice lowering with the bias added to
    every slice instead of once."""
    out = 0.0
    for kt in range(w.shape[2]):
        wk = np.zeros_like(w)
        wk[:, :, kt] = w[:, :, kt]
        out = out + oracle.causal_conv3d(x, wk, b)
    return out


def check_bias_once(conv, x_shape, w, b):
    y = conv(np.zeros(x_shape), w, b)
    return np.array_equal(y, np.broadcast_to(b[None, :, None, None, None], y.shape))


def test_bias_added_exactly_once_and_negative_control():
    w = rnd(3, 2, 3, 3, 3)
    b = rnd(3)
    shape = (1, 2, 4, 5, 6)
    assert check_bias_once(oracle.causal_conv3d, shape, w, b)
    # positive control: the same check rejects the planted mistake
    assert not check_bias_once(_bias_per_slice_variant, shape, w, b)


def test_temporal_slice_decomposition():
    """Conv3D == sum over kernel slices kt of a 2-D conv of frame t-2+kt with
    W[:, :, kt], bias once after the sum (torch conv2d per frame, fp64)."""
    x = rnd(1, 4, 6, 8, 9)
    w = rnd(5, 4, 3, 3, 3)
    b = rnd(5)
    y = oracle.causal_conv3d(x, w, b)
    N, C, T, H, W = x.shape
    ref = np.zeros_like(y)
    for t in range(T):
        acc = torch.zeros((1, 5, H, W), dtype=torch.float64)
        for kt in range(3):
            ts = t - 2 + kt
            if ts < 0:
                continue
            acc += F.conv2d(torch.from_numpy(x[:, :, ts]), torch.from_numpy(w[:, :, kt]), padding=1)
        ref[:, :, t] = (acc + torch.from_numpy(b)[None, :, None, None]).numpy()
    np.testing.assert_allclose(y, ref, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("t0", [0, 2, 5])
def test_causality_future_frames_do_not_reach_the_past(t0):
    x = rnd(1, 3, 7, 6, 6)
    w = rnd(3, 3, 3, 3, 3)
    b = rnd(3)
    y0 = oracle.causal_conv3d(x, w, b)
    x2 = x.copy()
    x2[:, :, t0] += rnd(1, 3, 6, 6)
    y1 = oracle.causal_conv3d(x2, w, b)
    np.testing.assert_array_equal(y1[:, :, :t0], y0[:, :, :t0])
    for t in range(t0, min(t0 + 3, 7)):
        assert not np.array_equal(y1[:, :, t], y0[:, :, t])
    np.testing.assert_array_equal(y1[:, :, t0 + 3:], y0[:, :, t0 + 3:])


def stream(x, w, b, sizes, **kw):
    outs = []
    cache = None
    t = 0
    for s in sizes:
        chunk = x[:, :, t:t + s]
        c = cache if cache is not None else np.zeros(x.shape[:2] + (2,) + x.shape[3:])
        outs.append(oracle.causal_conv3d(chunk, w, b, cache=c, **kw))
        cache = oracle.next_cache(cache, chunk)
        t += s
    return np.concatenate(outs, axis=2)


@pytest.mark.parametrize("sizes", [[1] * 7, [4, 3], [2, 2, 2, 1], [1, 4, 2], [7]])
def test_chunked_with_cache_equals_whole_sequence_bitwise(sizes):
    x = rnd(1, 3, 7, 5, 6)
    w = rnd(4, 3, 3, 3, 3)
    b = rnd(4)
    whole = oracle.causal_conv3d(x, w, b)
    np.testing.assert_array_equal(stream(x, w, b, sizes), whole)


def test_next_cache_rule():
    x = rnd(1, 2, 1, 3, 3)
    c = rnd(1, 2, 2, 3, 3)
    nc = oracle.next_cache(c, x)
    np.testing.assert_array_equal(nc[:, :, 0], c[:, :, 1])
    np.testing.assert_array_equal(nc[:, :, 1], x[:, :, 0])
    x3 = rnd(1, 2, 3, 3, 3)
    np.testing.assert_array_equal(oracle.next_cache(c, x3), x3[:, :, 1:])
    np.testing.assert_array_equal(oracle.next_cache(None, x)[:, :, 0], 0.0)


def test_points_equal_full_output_bitwise():
    x = rnd(2, 3, 4, 6, 7)
    w = rnd(5, 3, 3, 3, 3)
    b = rnd(5)
    cache = rnd(2, 3, 2, 6, 7)
    full = oracle.causal_conv3d(x, w, b, cache=cache)
    idx = np.arange(full.size)[::7]
    pts = oracle.causal_conv3d_points(x, w, idx, b, cache=cache)
    np.testing.assert_array_equal(pts, full.ravel()[idx])


def test_empty_and_degenerate_shapes():
    w = rnd(2, 2, 3, 3, 3)
    y = oracle.causal_conv3d(np.zeros((1, 2, 0, 4, 4)), w, None)
    assert y.shape == (1, 2, 0, 4, 4)
    # 1x1 spatial frame: only the centre taps touch data
    x = rnd(1, 2, 3, 1, 1)
    y = oracle.causal_conv3d(x, w, None)
    ref = torch_causal_reference(x, w, None)
    np.testing.assert_allclose(y, ref, rtol=1e-12, atol=1e-14)
