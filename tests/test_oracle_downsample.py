"""Pins of the oracle's strided causal conv and the downsample path.

"Cosmos3 Wan VAE -- engine size vs runtime context memory", section 10.5:
per frame a zero pad and a stride-2 Conv2d halve H and W, then a causal conv
with temporal stride 2 may halve T.  "diffusion inference workload anatomy
and cost ledger", the two-compressions paragraph: the causal video VAE encodes
the first frame alone and compresses time 4x, 81 frames -> 21 latent frames.

Each pin is independent of the oracle's own code: a library routine on an
explicitly padded input, numbers printed on the pages, closed forms and
invariants.
"""
import json
import os

import numpy as np
import pytest
import torch

import oracle

GOLDEN = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "page_accounting.json")))
rng = np.random.default_rng(1234)


def rnd(*shape):
    return rng.standard_normal(shape)


def torch_reference(x, w, b, stride, pad, pad_extra, dil):
    """F.conv3d (fp64) on x padded explicitly: dil_t*(kT-1) zero frames in
    front, pad + pad_extra zero rows/columns (trailing extra), no implicit
    padding in the conv."""
    kT = w.shape[2]
    ph, pw = pad
    eh, ew = pad_extra
    xt = torch.from_numpy(x)
    xt = torch.nn.functional.pad(xt, (pw, pw + ew, ph, ph + eh, dil[0] * (kT - 1), 0))
    y = torch.nn.functional.conv3d(xt, torch.from_numpy(w), None if b is None else torch.from_numpy(b),
                                   stride=stride, dilation=dil)
    return y.numpy()


@pytest.mark.parametrize("stride,pad,pad_extra,dil,k", [
    ((1, 2, 2), (0, 0), (1, 1), (1, 1, 1), (1, 3, 3)),   # the spatial downsample, trailing pad
    ((1, 2, 2), (1, 1), (0, 0), (1, 1, 1), (1, 3, 3)),   # the symmetric reading
    ((2, 1, 1), (0, 0), (0, 0), (1, 1, 1), (3, 1, 1)),   # the temporal downsample
    ((2, 2, 1), (1, 0), (1, 0), (1, 1, 2), (3, 3, 2)),   # everything at once
    ((3, 1, 2), (0, 1), (2, 1), (2, 1, 1), (2, 2, 3)),
])
def test_strided_conv_equals_library_conv_on_padded_input(stride, pad, pad_extra, dil, k):
    x = rnd(2, 3, 7, 9, 10)
    w = rnd(4, 3, *k)
    b = rnd(4)
    y = oracle.causal_conv3d_strided(x, w, b, stride=stride, pad=pad, pad_extra=pad_extra, dil=dil)
    ref = torch_reference(x, w, b, stride, pad, pad_extra, dil)
    assert y.shape == ref.shape
    assert np.abs(y - ref).max() <= 1e-12 * np.abs(ref).max()


def test_stride_one_is_the_pinned_causal_conv_bitwise():
    x, w, b, c = rnd(1, 3, 5, 6, 7), rnd(2, 3, 3, 3, 3), rnd(2), rnd(1, 3, 2, 6, 7)
    np.testing.assert_array_equal(oracle.causal_conv3d_strided(x, w, b, cache=c),
                                  oracle.causal_conv3d(x, w, b, cache=c))


def test_frame_counts_printed_on_the_pages():
    # two temporal-stride-2 causal convs: 81 -> 21 and 17 -> 5 latent frames
    for frames, latent in GOLDEN["latent_frames"]["pairs"]:
        t = frames
        for _ in range(2):
            t = oracle.strided_out_frames(t, 2, 0)
        assert t == latent
    # and the per-frame spatial downsample 480x832 -> 240x416, T unchanged
    g = GOLDEN["downsample_spatial"]
    t, h, w = g["in_thw"]
    for pad, ext in (((0, 0), (1, 1)), ((1, 1), (0, 0))):
        x = np.zeros((1, 1, 1, h, w))
        y = oracle.causal_conv3d_strided(x, np.zeros((1, 1, 1, 3, 3)), stride=(1, 2, 2), pad=pad,
                                         pad_extra=ext)
        assert (t,) + y.shape[3:] == tuple(g["out_thw"])


def test_first_output_frame_sees_only_the_first_input_frame():
    x, w = rnd(1, 2, 9, 4, 5), rnd(3, 2, 3, 1, 1)
    y = oracle.causal_conv3d_strided(x, w, stride=(2, 1, 1), pad=(0, 0))
    x2 = x.copy()
    x2[:, :, 1:] = rnd(1, 2, 8, 4, 5)
    y2 = oracle.causal_conv3d_strided(x2, w, stride=(2, 1, 1), pad=(0, 0))
    np.testing.assert_array_equal(y[:, :, 0], y2[:, :, 0])
    # output 0 is the last kernel slice applied to frame 0 alone
    ref = np.einsum("oi,nihw->nohw", w[:, :, 2, 0, 0], x[:, :, 0])
    assert np.abs(y[:, :, 0] - ref).max() <= 1e-13


@pytest.mark.parametrize("t0", [0, 3, 4, 8])
def test_causality_under_temporal_stride(t0):
    x, w = rnd(1, 2, 9, 3, 4), rnd(2, 2, 3, 3, 3)
    y = oracle.causal_conv3d_strided(x, w, stride=(2, 1, 1))
    x2 = x.copy()
    x2[:, :, t0] += 1.0
    y2 = oracle.causal_conv3d_strided(x2, w, stride=(2, 1, 1))
    for j in range(y.shape[2]):
        anchor = 2 * j
        if anchor < t0 or anchor - 2 > t0:
            np.testing.assert_array_equal(y[:, :, j], y2[:, :, j])
        else:
            assert not np.array_equal(y[:, :, j], y2[:, :, j])


def test_impulse_closed_form():
    """A unit impulse at (ci, t0, h0, w0) reaches output (co, j, ho, wo) with
    the single weight W[co, ci, kt, kh, kw] whose tap lands on it."""
    C, Co, T, H, W = 2, 3, 6, 7, 8
    w = rnd(Co, C, 3, 3, 3)
    ci, t0, h0, w0 = 1, 3, 4, 5
    x = np.zeros((1, C, T, H, W))
    x[0, ci, t0, h0, w0] = 1.0
    y = oracle.causal_conv3d_strided(x, w, stride=(2, 2, 2), pad=(0, 0), pad_extra=(1, 1))
    for j in range(y.shape[2]):
        for ho in range(y.shape[3]):
            for wo in range(y.shape[4]):
                kt, kh, kw = t0 - (2 * j - 2), h0 - 2 * ho, w0 - 2 * wo
                want = w[:, ci, kt, kh, kw] if 0 <= kt < 3 and 0 <= kh < 3 and 0 <= kw < 3 \
                    else np.zeros(Co)
                np.testing.assert_array_equal(y[0, :, j, ho, wo], want)


def test_bias_added_once():
    b = rnd(3)
    y = oracle.causal_conv3d_strided(np.zeros((1, 2, 5, 4, 6)), rnd(3, 2, 3, 3, 3), b,
                                     stride=(2, 2, 2), pad=(0, 0), pad_extra=(1, 1))
    np.testing.assert_array_equal(y, np.broadcast_to(b[None, :, None, None, None], y.shape))


@pytest.mark.parametrize("sizes", [[1, 4, 4], [2, 2, 2, 3], [3, 1, 5], [1] * 9, [9]])
def test_chunked_with_cache_and_phase_equals_whole_bitwise(sizes):
    """Chunks carry the last two input frames as the cache and the number of
    frames before them (mod 2) as the phase; their outputs concatenate to the
    whole-sequence output, bit for bit."""
    x, w, b = rnd(1, 3, sum(sizes), 4, 5), rnd(2, 3, 3, 1, 1), rnd(2)
    whole = oracle.causal_conv3d_strided(x, w, b, stride=(2, 1, 1), pad=(0, 0))
    outs, cache, g = [], None, 0
    for s in sizes:
        chunk = x[:, :, g:g + s]
        outs.append(oracle.causal_conv3d_strided(chunk, w, b, cache=cache, stride=(2, 1, 1),
                                                 pad=(0, 0), t_phase=g % 2))
        cache = oracle.next_cache(cache, chunk)
        g += s
    np.testing.assert_array_equal(np.concatenate(outs, axis=2), whole)


def test_downsample3d_composition_and_chunking():
    """The downsample path of section 10.5 on a 9-frame sequence: the spatial
    conv then the temporal one, whole vs 1+4+4 chunks threading the cache and
    the phase (bitwise); output shape halves T (ceil), H and W."""
    C = 4
    p = {"w_s": rnd(C, C, 1, 3, 3), "b_s": rnd(C), "w_t": rnd(C, C, 3, 1, 1), "b_t": rnd(C)}
    x = rnd(1, C, 9, 8, 10)
    whole, _ = oracle.downsample3d(x, p)
    assert whole.shape == (1, C, 5, 4, 5)
    outs, cache, g = [], None, 0
    for s in (1, 4, 4):
        y, cache = oracle.downsample3d(x[:, :, g:g + s], p, cache=cache, t_phase=g % 2)
        outs.append(y)
        g += s
    np.testing.assert_array_equal(np.concatenate(outs, axis=2), whole)
    s_only, _ = oracle.downsample3d(x, p, temporal=False)
    ref = torch_reference(x, p["w_s"], p["b_s"], (1, 2, 2), (0, 0), (1, 1), (1, 1, 1))
    assert np.abs(s_only - ref).max() <= 1e-12 * np.abs(ref).max()
