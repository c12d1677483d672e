"""Full-size GPU parity for the two single-layer workloads: whole output frames
against the oracle, plus point samples the oracle computes one by one across
every frame, plus properties that hold at any size.

* 384-channel layer: causal Conv3D 3x3x3 on x[1,384,17,240,416] (bf16), whole
  sequence and frame by frame with the cache (must agree), then a 1x1x1
  384->192 projection of the conv output.
* 96-channel layer: fused RMS norm + SiLU, then causal Conv3D 3x3x3 on
  x[1,96,17,480,832] (bf16) in chunks of 1+4+4+4+4 frames with the cache.

Coverage of each conv: the oracle's whole output frames 0 (only zero causal
padding behind it), 1 (one real past frame) and 16 (the last, both past
frames real), and 4,000 random outputs in every one of the 17 frames (68,000)
plus the full spatial border of two channels per frame.

Shapes follow the Wan encoder's feature maps on a 1x3x17x480x832 video
("Cosmos3 Wan VAE -- engine size vs runtime context memory", sections 3.1 and
10.1); the whole-sequence vs cached-chunk agreement is section 10.3's claim.
Whole and chunked runs take the same kernel and tile plan here (no split of
K at these frame sizes), so they must agree bit for bit.
"""
import numpy as np
import pytest
import torch

import oracle
from video_vae_causal_amd import _lib as L
from video_vae_causal_amd import inputs
from _gpu_util import check_bf16, f64, frame_points, oracle_conv_at_frame, to_dev, to_host

pytestmark = [pytest.mark.gpu, pytest.mark.timeout(900)]

WHOLE_FRAMES = (0, 1, 16)
POINTS_PER_FRAME = 4000


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


def oracle_frame(x_in, w, b, t):
    """The oracle's whole output frame t: the chunk is frame t alone and the
    cache holds frames t-2 and t-1 (zeros before frame 0), the oracle's
    chunked mode, which equals its whole-sequence sum bit for bit."""
    n, c, _, h, wd = x_in.shape
    past = np.zeros((n, c, 2, h, wd))
    for k, s in enumerate((t - 2, t - 1)):
        if s >= 0:
            past[:, :, k] = x_in[:, :, s]
    return oracle.causal_conv3d(f64(x_in[:, :, t:t + 1]), f64(w), f64(b), cache=past)[0, :, 0]


def check_conv_full(x_in, w, b, y_dev, what):
    """Whole frames WHOLE_FRAMES and POINTS_PER_FRAME random outputs plus two
    channels' borders in every frame.  Returns the number of outputs compared."""
    compared = 0
    for t in WHOLE_FRAMES:
        ref = oracle_frame(x_in, w, b, t)
        check_bf16(to_host(y_dev[0, :, t]), ref, f"{what} whole frame {t}")
        compared += ref.size
    got_all, ref_all = [], []
    for t in range(x_in.shape[2]):
        co, hh, ww = frame_points(w.shape[0], x_in.shape[3], x_in.shape[4], POINTS_PER_FRAME,
                                  seed=100 + t)
        ref_all.append(oracle_conv_at_frame(x_in[:, :, max(0, t - 2):t + 1], w, b, co, hh, ww))
        got_all.append(to_host(y_dev[0, :, t])[co, hh, ww])
    got, ref = np.concatenate(got_all), np.concatenate(ref_all)
    check_bf16(got, ref, f"{what}: {got.size} sampled outputs over all {x_in.shape[2]} frames")
    return compared + got.size


def test_layer_384_240x416():
    d = inputs.layer384_inputs()
    print("[case] layer 384 240x416 T=17: generated", flush=True)
    xd, wd, bd = to_dev(d["x"]), to_dev(d["w"]), to_dev(d["b"])
    y_whole = L.wvc_causal_conv3d_fwd(xd, wd, bd)
    torch.cuda.synchronize()
    print("[case] whole-sequence conv done", flush=True)
    n = check_conv_full(d["x"], d["w"], d["b"], y_whole, "conv384")
    assert n >= 3 * 384 * 240 * 416 + 65536

    y_frames = run_chunks(xd, wd, bd, [1] * 17)
    assert torch.equal(y_frames, run_chunks(xd, wd, bd, [1] * 17))
    assert torch.equal(y_frames, y_whole), "1-frame chunks with the cache differ from the whole sequence"

    # 1x1x1 projection 384 -> 192 of the conv output
    wp, bp = to_dev(d["wp"]), to_dev(d["bp"])
    proj = L.wvc_causal_conv3d_fwd(y_whole, wp, bp, padding=(0, 0))
    g = np.random.default_rng(7)
    pos = [(int(t), int(h), int(w)) for t, h, w in zip(g.integers(0, 17, 400), g.integers(0, 240, 400),
                                                        g.integers(0, 416, 400))]
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
    check_bf16(got, ref[0, :, 0, :, 0], f"projection 384->192 ({len(pos)} positions x 192)")


def test_layer_96_480x832_norm_then_conv():
    d = inputs.layer96_inputs()
    print("[case] layer 96 480x832 T=17: generated", flush=True)
    xd, gd, wd, bd = to_dev(d["x"]), to_dev(d["gamma"]), to_dev(d["w"]), to_dev(d["b"])
    h = L.wvc_rmsnorm_silu(xd, gd)
    torch.cuda.synchronize()
    T, H, W = 17, 480, 832
    g64 = f64(d["gamma"])
    hh = to_host(h)

    def norm_ref(frames):
        return oracle.silu(oracle.rms_norm(f64(d["x"][:, :, frames]), g64))

    # norm: whole frames, then 65,536 random positions across the sequence
    for t in WHOLE_FRAMES:
        check_bf16(hh[:, :, t:t + 1], norm_ref(slice(t, t + 1)), f"norm+silu 96ch whole frame {t}")
    gr = np.random.default_rng(3)
    ts, hs, ws = gr.integers(0, T, 65536), gr.integers(0, H, 65536), gr.integers(0, W, 65536)
    vecs = f64(d["x"][0][:, ts, hs, ws])                           # [96, P]
    ref = oracle.silu(oracle.rms_norm(vecs[None, :, None, :, None], g64))[0, :, 0, :, 0]
    check_bf16(hh[0][:, ts, hs, ws], ref, "norm+silu 96ch (65,536 positions)")

    y = run_chunks(h, wd, bd, [1, 4, 4, 4, 4])
    y_whole = L.wvc_causal_conv3d_fwd(h, wd, bd)
    y_other = run_chunks(h, wd, bd, [4, 4, 4, 4, 1])
    assert torch.equal(y, y_whole), "1+4+4+4+4 chunks differ from the whole sequence"
    assert torch.equal(y_other, y_whole), "4+4+4+4+1 chunks differ from the whole sequence"

    # conv on the normalised input as the GPU stored it (bf16-rounded): the
    # oracle normalises the whole input, rounds it, then convolves
    x_n = np.empty(d["x"].shape, dtype=np.float32)   # bf16 values are exact in fp32
    for t in range(T):
        x_n[:, :, t:t + 1] = oracle.round_bf16(norm_ref(slice(t, t + 1)))
    n = check_conv_full(x_n, d["w"], d["b"], y, "conv96 after norm")
    assert n >= 3 * 96 * 480 * 832 + 65536
