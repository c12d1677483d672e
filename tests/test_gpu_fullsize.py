"""Full-size GPU parity for the two single-layer workloads, on outputs the oracle
computes point by point, plus properties that hold at any size.

* 384-channel layer: causal Conv3D 3x3x3 on x[1,384,17,240,416] (bf16), whole
  sequence and frame by frame with the cache (must agree), then a 1x1x1
  384->192 projection of the conv output.
* 96-channel layer: fused RMS norm + SiLU, then causal Conv3D 3x3x3 on
  x[1,96,17,480,832] (bf16) in chunks of 1+4+4+4+4 frames with the cache.

Shapes follow the Wan encoder's feature maps on a 1x3x17x480x832 video
("Cosmos3 Wan VAE -- engine size vs runtime context memory", sections 3.1 and
10.1); the whole-sequence vs cached-chunk agreement is section 10.3's claim.
"""
import numpy as np
import pytest
import torch

import oracle
from video_vae_causal_amd import _lib as L
from video_vae_causal_amd import inputs
from _gpu_util import check_bf16, f64, frame_points, oracle_conv_at_frame, to_dev, to_host

pytestmark = [pytest.mark.gpu, pytest.mark.timeout(600)]


def cl(t):
    return t.contiguous(memory_format=torch.channels_last_3d)


def run_chunks(xd, wd, bd, sizes):
    n, c, t, h, w = xd.shape
    caches = [L.empty_cl((n, c, 2, h, w)) for _ in range(2)]
    L.wvc_cache_reset(caches[0])
    out = L.empty_cl((n, wd.shape[0], t, h, w))
    t0 = 0
    for i, s in enumerate(sizes):
        L.wvc_causal_conv3d_fwd(cl(xd[:, :, t0:t0 + s]), wd, bd, caches[i % 2], caches[(i + 1) % 2],
                                y=out[:, :, t0:t0 + s])
        t0 += s
    return out


def sampled_conv_check(x, wt, b, y_dev, frames, what, count=2000):
    for t in frames:
        co, hh, ww = frame_points(wt.shape[0], x.shape[3], x.shape[4], count, seed=100 + t)
        win = x[:, :, max(0, t - 2):t + 1]
        ref = oracle_conv_at_frame(win, wt, b, co, hh, ww)
        got = to_host(y_dev[0, :, t])[co, hh, ww]
        check_bf16(got, ref, f"{what} frame {t} ({len(co)} points)")


def test_layer_384_240x416():
    d = inputs.layer384_inputs()
    print("[case] layer 384 240x416 T=17: generated", flush=True)
    xd, wd, bd = to_dev(d["x"]), to_dev(d["w"]), to_dev(d["b"])
    y_whole = L.wvc_causal_conv3d_fwd(xd, wd, bd)
    torch.cuda.synchronize()
    print("[case] whole-sequence conv done", flush=True)
    sampled_conv_check(d["x"], d["w"], d["b"], y_whole, (0, 1, 8, 16), "conv384")

    y_frames = run_chunks(xd, wd, bd, [1] * 17)
    assert torch.equal(y_frames, run_chunks(xd, wd, bd, [1] * 17))
    for t in (0, 1, 16):
        check_bf16(to_host(y_frames[0, :, t]), to_host(y_whole[0, :, t]), f"frame {t}: 1-frame chunks vs whole")
    sampled_conv_check(d["x"], d["w"], d["b"], y_frames, (0, 1, 16), "conv384 frame-by-frame")

    # 1x1x1 projection 384 -> 192 of the conv output
    wp, bp = to_dev(d["wp"]), to_dev(d["bp"])
    proj = L.wvc_causal_conv3d_fwd(y_whole, wp, bp, padding=(0, 0))
    g = np.random.default_rng(7)
    pos = [(int(t), int(h), int(w)) for t, h, w in zip(g.integers(0, 17, 160), g.integers(0, 240, 160),
                                                        g.integers(0, 416, 160))]
    pos += [(0, 0, 0), (16, 239, 415), (3, 0, 415), (9, 239, 0)]
    conv_vals = np.empty((384, len(pos)))
    for i, (t, h, w) in enumerate(pos):
        win = d["x"][:, :, max(0, t - 2):t + 1]
        co = np.arange(384)
        conv_vals[:, i] = oracle_conv_at_frame(win, d["w"], d["b"], co, np.full(384, h), np.full(384, w))
    conv_b = oracle.round_bf16(conv_vals)       # the conv output is stored in bf16
    ref = oracle.causal_conv3d(conv_b[None, :, None, :, None], f64(d["wp"]), f64(d["bp"]), pad=(0, 0))
    ph = to_host(proj)
    got = np.stack([ph[0, :, t, h, w] for t, h, w in pos], axis=1)
    check_bf16(got, ref[0, :, 0, :, 0], "projection 384->192")


def test_layer_96_480x832_norm_then_conv():
    d = inputs.layer96_inputs()
    print("[case] layer 96 480x832 T=17: generated", flush=True)
    xd, gd, wd, bd = to_dev(d["x"]), to_dev(d["gamma"]), to_dev(d["w"]), to_dev(d["b"])
    h = L.wvc_rmsnorm_silu(xd, gd)
    torch.cuda.synchronize()

    # norm: sampled positions against the fp64 oracle
    g = np.random.default_rng(3)
    T, H, W = 17, 480, 832
    ts, hs, ws = g.integers(0, T, 4000), g.integers(0, H, 4000), g.integers(0, W, 4000)
    vecs = f64(d["x"][0][:, ts, hs, ws])                           # [96, P]
    ref = oracle.silu(oracle.rms_norm(vecs[None, :, None, :, None], f64(d["gamma"])))[0, :, 0, :, 0]
    hh = to_host(h)
    check_bf16(hh[0][:, ts, hs, ws], ref, "norm+silu 96ch (4000 positions)")

    y = run_chunks(h, wd, bd, [1, 4, 4, 4, 4])
    y_whole = L.wvc_causal_conv3d_fwd(h, wd, bd)
    y_other = run_chunks(h, wd, bd, [4, 4, 4, 4, 1])
    for t in (0, 4, 16):
        check_bf16(to_host(y[0, :, t]), to_host(y_whole[0, :, t]), f"frame {t}: 1+4+4+4+4 vs whole")
        check_bf16(to_host(y_other[0, :, t]), to_host(y_whole[0, :, t]), f"frame {t}: 4+4+4+4+1 vs whole")

    # conv on the normalised input: the oracle normalises (bf16-rounded, as
    # stored) the frames each sampled output reads, then convolves.
    for t in (0, 1, 4, 5, 16):
        t0 = max(0, t - 2)
        win = oracle.round_bf16(oracle.silu(oracle.rms_norm(f64(d["x"][:, :, t0:t + 1]),
                                                            f64(d["gamma"]))))
        co, rr, cc = frame_points(96, H, W, 2000, seed=200 + t)
        ref = oracle_conv_at_frame(win, d["w"], d["b"], co, rr, cc)
        got = to_host(y[0, :, t])[co, rr, cc]
        check_bf16(got, ref, f"conv96 after norm, frame {t}")
