"""GPU parity of the encoder's downsampling convs through the C ABI.

"Cosmos3 Wan VAE -- engine size vs runtime context memory", section 10.5:
per frame a zero pad and a stride-2 Conv2d halve H and W, then a causal conv
with temporal stride 2 halves T, with RMS norms around them.  Expected values
come from the oracle's strided causal conv (pinned in
tests/test_oracle_downsample.py), on the same seeded bf16 inputs.
"""
import numpy as np
import pytest
import torch

import oracle
from video_vae_causal_amd import _lib as L
from video_vae_causal_amd import inputs
from _gpu_util import check_bf16, f64, to_dev, to_host

pytestmark = pytest.mark.gpu


def bf(shape, seed, name):
    return inputs.quantize(inputs.normal(shape, seed, name), "bf16")


def strided_route_taken(expect_fast: bool):
    c = L.wvc_get_counters()
    if expect_fast:
        assert c["fast_strided"] == 1 and c["generic"] == 0, c
    else:
        assert c["generic"] == 1 and c["fast_strided"] == 0, c


@pytest.mark.parametrize("cin,cout,t,h,w,phase,cached,res,fast", [
    (96, 96, 5, 12, 20, 0, False, False, True),    # K = 288, 240 positions: 4 tiles (ragged)
    (96, 96, 4, 7, 9, 1, True, True, True),        # odd phase, cache, residual, 63 positions
    (64, 128, 6, 5, 70, 0, True, False, True),     # 350 positions, 4 waves x 2 blocks
    (160, 64, 3, 4, 4, 1, True, False, True),      # K = 480, the largest staged row
    (32, 48, 5, 3, 5, 0, True, False, True),       # one wave group of 3 blocks
    (40, 64, 5, 4, 6, 0, True, False, False),      # C_in % 32 != 0: direct route
    (96, 96, 1, 6, 6, 1, True, False, True),       # a chunk with no anchor: no output frame
])
def test_temporal_stride2_vs_oracle(cin, cout, t, h, w, phase, cached, res, fast):
    x = bf((1, cin, t, h, w), 51, "x")
    wt = inputs.conv_weight(cout, cin, (3, 1, 1), 51, "w", "bf16")
    b = inputs.conv_bias(cout, 51, "b", "bf16")
    cache = bf((1, cin, 2, h, w), 51, "c") if cached else None
    to = L.conv_out_frames(t, 2, phase)
    r = bf((1, cout, to, h, w), 51, "r") if res else None
    print(f"[case] temporal s2 {cin}->{cout} t={t} {h}x{w} phase={phase}", flush=True)
    cout_t = L.empty_cl((1, cin, 2, h, w))
    L.wvc_reset_counters()
    y = L.wvc_causal_conv3d_fwd(to_dev(x), to_dev(wt), to_dev(b), to_dev(cache) if cached else None,
                                cout_t, to_dev(r) if res else None, stride=(2, 1, 1), padding=(0, 0),
                                t_phase=phase)
    strided_route_taken(fast)
    ref = oracle.causal_conv3d_strided(f64(x), f64(wt), f64(b), cache=f64(cache) if cached else None,
                                       stride=(2, 1, 1), pad=(0, 0), t_phase=phase)
    if res:
        ref = ref + f64(r)
    assert tuple(y.shape) == ref.shape
    if to:
        check_bf16(to_host(y), ref, f"temporal stride 2 {cin}->{cout}")
    np.testing.assert_array_equal(to_host(cout_t), oracle.next_cache(f64(cache) if cached else None, f64(x)))


@pytest.mark.parametrize("cin,cout,h,w,pad,ext,fast", [
    (96, 96, 16, 30, (0, 0), (1, 1), True),     # the trailing-pad reading, 64-column runs, ragged
    (96, 96, 17, 131, (1, 1), (0, 0), True),    # symmetric reading, odd sizes, 2 runs
    (128, 64, 9, 40, (0, 0), (1, 1), True),     # 32-column runs (LDS), 4 waves x 1 block
    (192, 96, 8, 20, (0, 0), (1, 1), True),     # 32-column runs, 2 groups x 3 blocks
    (64, 48, 6, 10, (1, 0), (0, 1), True),      # mixed pads, one group of 3 blocks
    (48, 32, 6, 6, (0, 0), (1, 1), False),      # C_in % 32 != 0: direct route
])
def test_spatial_stride2_vs_oracle(cin, cout, h, w, pad, ext, fast):
    x = bf((2, cin, 2, h, w), 52, "x")
    wt = inputs.conv_weight(cout, cin, (1, 3, 3), 52, "w", "bf16")
    b = inputs.conv_bias(cout, 52, "b", "bf16")
    print(f"[case] spatial s2 {cin}->{cout} {h}x{w} pad={pad} ext={ext}", flush=True)
    L.wvc_reset_counters()
    y = L.wvc_causal_conv3d_fwd(to_dev(x), to_dev(wt), to_dev(b), stride=(1, 2, 2), padding=pad,
                                pad_extra=ext)
    strided_route_taken(fast)
    ref = oracle.causal_conv3d_strided(f64(x), f64(wt), f64(b), stride=(1, 2, 2), pad=pad, pad_extra=ext)
    assert tuple(y.shape) == ref.shape
    check_bf16(to_host(y), ref, f"spatial stride 2 {cin}->{cout}")


def test_temporal_chunks_with_phase_equal_whole_bitwise():
    """A 9-frame sequence fed 1+4+4 frames, threading the cache and the phase,
    equals the whole-sequence call bit for bit (same kernel, same sums)."""
    cin, h, w = 96, 10, 14
    x = to_dev(bf((1, cin, 9, h, w), 53, "x"))
    wt = to_dev(inputs.conv_weight(cin, cin, (3, 1, 1), 53, "w", "bf16"))
    b = to_dev(inputs.conv_bias(cin, 53, "b", "bf16"))
    whole = L.wvc_causal_conv3d_fwd(x, wt, b, stride=(2, 1, 1), padding=(0, 0))
    caches = [L.empty_cl((1, cin, 2, h, w)) for _ in range(2)]
    L.wvc_cache_reset(caches[0])
    outs, g, cur = [], 0, 0
    for s in (1, 4, 4):
        chunk = x[:, :, g:g + s].contiguous(memory_format=torch.channels_last_3d)
        outs.append(L.wvc_causal_conv3d_fwd(chunk, wt, b, caches[cur], caches[1 - cur], stride=(2, 1, 1),
                                            padding=(0, 0), t_phase=g % 2))
        cur ^= 1
        g += s
    assert torch.equal(torch.cat(outs, dim=2), whole)


def test_downsample3d_chain_vs_oracle():
    """Spatial conv then temporal conv (section 10.5) on a 9-frame 96-channel
    map, streamed 1+4+4 with the temporal conv's cache and phase, against the
    oracle's composition (bf16 where the GPU stores the intermediate)."""
    d = inputs.downsample_inputs(seed=54, shape=(1, 96, 9, 20, 36))
    p = {k: to_dev(v) for k, v in d.items()}
    x = p["x"]
    outs = []
    caches = [L.empty_cl((1, 96, 2, 10, 18)) for _ in range(2)]
    L.wvc_cache_reset(caches[0])
    g, cur = 0, 0
    for s in (1, 4, 4):
        chunk = x[:, :, g:g + s].contiguous(memory_format=torch.channels_last_3d)
        sp = L.wvc_causal_conv3d_fwd(chunk, p["w_s"], p["b_s"], stride=(1, 2, 2), padding=(0, 0),
                                     pad_extra=(1, 1))
        outs.append(L.wvc_causal_conv3d_fwd(sp, p["w_t"], p["b_t"], caches[cur], caches[1 - cur],
                                            stride=(2, 1, 1), padding=(0, 0), t_phase=g % 2))
        cur ^= 1
        g += s
    y = torch.cat(outs, dim=2)
    ref, _ = oracle.downsample3d(f64(d["x"]), {k: f64(v) for k, v in d.items()}, bf16=True)
    assert tuple(y.shape) == ref.shape == (1, 96, 5, 10, 18)
    check_bf16(to_host(y), ref, "downsample3d 96ch 9x20x36")


def test_downsample_full_size_sampled():
    """The L0 feature map of the pages (96 ch, 17x480x832): spatial stride-2
    conv to 17x240x416, then the temporal stride-2 conv to 9x240x416;
    sampled outputs of each against the oracle, evaluated only on the input
    values each sampled output reads (the oracle computes its own
    intermediate, rounded to bf16 where the GPU stores it)."""
    d = inputs.downsample_inputs()
    print("[case] downsample 96ch 17x480x832: generated", flush=True)
    x = to_dev(d["x"])
    sp = L.wvc_causal_conv3d_fwd(x, to_dev(d["w_s"]), to_dev(d["b_s"]), stride=(1, 2, 2),
                                 padding=(0, 0), pad_extra=(1, 1))
    y = L.wvc_causal_conv3d_fwd(sp, to_dev(d["w_t"]), to_dev(d["b_t"]), stride=(2, 1, 1), padding=(0, 0))
    torch.cuda.synchronize()
    assert tuple(sp.shape) == (1, 96, 17, 240, 416) and tuple(y.shape) == (1, 96, 9, 240, 416)
    g = np.random.default_rng(61)
    pts = [(int(t), int(h), int(w)) for t, h, w in zip(g.integers(0, 17, 96), g.integers(0, 240, 96),
                                                       g.integers(0, 416, 96))]
    pts += [(0, 0, 0), (16, 239, 415), (5, 239, 0), (9, 0, 415)]
    ws, bs = f64(d["w_s"]), f64(d["b_s"])

    def oracle_spatial(t, h, w):
        """The oracle's stride-2 conv output at (t, h, w), all channels: the
        3x3 window at (2h, 2w) with the trailing zero row and column."""
        win = np.zeros((1, 96, 1, 3, 3))
        rows = slice(2 * h, min(2 * h + 3, 480))
        cols = slice(2 * w, min(2 * w + 3, 832))
        win[:, :, 0, :rows.stop - rows.start, :cols.stop - cols.start] = d["x"][:, :, t, rows, cols]
        return oracle.causal_conv3d_strided(win, ws, bs, stride=(1, 1, 1), pad=(0, 0))[0, :, 0, 0, 0]

    spd = to_host(sp)
    got, ref = [], []
    for t, h, w in pts:
        ref.append(oracle_spatial(t, h, w))
        got.append(spd[0, :, t, h, w])
    check_bf16(np.stack(got, 1), np.stack(ref, 1), "spatial stride 2, full size (sampled)")
    wt_, bt = f64(d["w_t"]), f64(d["b_t"])
    yd = to_host(y)
    got, ref = [], []
    for t, h, w in pts:
        j = t % 9
        win = np.zeros((1, 96, 3, 1, 1))  # frames 2j-2 .. 2j of the intermediate, bf16 as stored
        for kt in range(3):
            f = 2 * j - 2 + kt
            if f >= 0:
                win[0, :, kt, 0, 0] = oracle.round_bf16(oracle_spatial(f, h, w))
        ref.append(oracle.causal_conv3d_strided(win, wt_, bt, stride=(1, 1, 1), pad=(0, 0))[0, :, 2, 0, 0])
        got.append(yd[0, :, j, h, w])
    check_bf16(np.stack(got, 1), np.stack(ref, 1), "temporal stride 2, full size (sampled)")

    # the same spatial conv with the first RMS norm + SiLU fused into it (the
    # bench's launch configuration), on the oracle's own bf16 norm output
    g1 = f64(d["gamma1"])
    spn = to_host(L.wvc_rmsnorm_silu_conv3d_fwd(x, to_dev(d["gamma1"]), to_dev(d["w_s"]), to_dev(d["b_s"])))
    got, ref = [], []
    for t, h, w in pts[:48] + pts[-4:]:
        win = np.zeros((1, 96, 1, 3, 3))
        rows = slice(2 * h, min(2 * h + 3, 480))
        cols = slice(2 * w, min(2 * w + 3, 832))
        xin = oracle.norm_silu(f64(d["x"][:, :, t:t + 1, rows, cols]), g1, bf16=True)
        win[:, :, :, :rows.stop - rows.start, :cols.stop - cols.start] = xin
        ref.append(oracle.causal_conv3d_strided(win, ws, bs, stride=(1, 1, 1), pad=(0, 0))[0, :, 0, 0, 0])
        got.append(spn[0, :, t, h, w])
    check_bf16(np.stack(got, 1), np.stack(ref, 1), "norm + spatial stride 2 fused, full size (sampled)")


@pytest.mark.parametrize("cin,cout,t,h,w,beta", [
    (96, 96, 2, 13, 150, False),   # the 96-channel path: ragged 64-column runs, odd rows
    (96, 96, 1, 8, 16, True),      # with beta: the zero padding must stay zero, not SiLU(beta)
    (64, 128, 2, 9, 70, True),     # the general channel count path
    (128, 64, 1, 6, 10, False),
])
def test_fused_norm_spatial_conv_vs_oracle(cin, cout, t, h, w, beta):
    # RMS norm + SiLU computed in the stride-2 conv's staging, against the
    # oracle's norm (rounded to bf16, where the unfused path stores it) then conv
    x = bf((1, cin, t, h, w), 61, "x") * 2.0
    g = inputs.norm_gamma(cin, 61, "g", "bf16")
    be = inputs.quantize(inputs.normal((cin,), 61, "be", std=0.3), "bf16") if beta else None
    wt = inputs.conv_weight(cout, cin, (1, 3, 3), 61, "w", "bf16")
    b = inputs.conv_bias(cout, 61, "b", "bf16")
    print(f"[case] fused norm + spatial s2 {cin}->{cout} t={t} {h}x{w} beta={beta}", flush=True)
    L.wvc_reset_counters()
    y = L.wvc_rmsnorm_silu_conv3d_fwd(to_dev(x), to_dev(g), to_dev(wt), to_dev(b),
                                      beta=to_dev(be) if beta else None)
    strided_route_taken(True)
    hn = oracle.norm_silu(f64(x), f64(g), f64(be) if beta else None, bf16=True)
    ref = oracle.causal_conv3d_strided(hn, f64(wt), f64(b), stride=(1, 2, 2), pad=(0, 0),
                                       pad_extra=(1, 1))
    assert tuple(y.shape) == ref.shape
    check_bf16(to_host(y), ref, f"fused norm + spatial conv {cin}->{cout}")
    # and it matches the unfused pair of kernels to within the last bit of
    # a few normalised inputs
    hd = L.wvc_rmsnorm_silu(to_dev(x), to_dev(g), to_dev(be) if beta else None)
    y2 = L.wvc_causal_conv3d_fwd(hd, to_dev(wt), to_dev(b), stride=(1, 2, 2), padding=(0, 0),
                                 pad_extra=(1, 1))
    rel = oracle.rel_l2(to_host(y), to_host(y2))
    print(f"[parity] fused vs unfused rel_l2={rel:.2e}", flush=True)
    assert rel < 2e-3


@pytest.mark.parametrize("fused", [False, True])
def test_spatial_stride2_larger_grid(fused):
    # a few thousand 64-column runs over 4 frames, ragged in both directions
    cin, cout, t, h, w = 96, 96, 4, 162, 258
    x = bf((1, cin, t, h, w), 71, "x")
    wt = inputs.conv_weight(cout, cin, (1, 3, 3), 71, "w", "bf16")
    b = inputs.conv_bias(cout, 71, "b", "bf16")
    g = inputs.norm_gamma(cin, 71, "g", "bf16")
    be = inputs.quantize(inputs.normal((cin,), 71, "be", std=0.3), "bf16")
    print(f"[case] spatial s2 larger grid {t}x{h}x{w} fused={fused}", flush=True)
    if fused:
        y = L.wvc_rmsnorm_silu_conv3d_fwd(to_dev(x), to_dev(g), to_dev(wt), to_dev(b), beta=to_dev(be))
        xin = oracle.norm_silu(f64(x), f64(g), f64(be), bf16=True)
    else:
        y = L.wvc_causal_conv3d_fwd(to_dev(x), to_dev(wt), to_dev(b), stride=(1, 2, 2), padding=(0, 0),
                                    pad_extra=(1, 1))
        xin = f64(x)
    ref = oracle.causal_conv3d_strided(xin, f64(wt), f64(b), stride=(1, 2, 2), pad=(0, 0), pad_extra=(1, 1))
    assert tuple(y.shape) == ref.shape
    check_bf16(to_host(y), ref, f"spatial s2 larger grid fused={fused}")


@pytest.mark.parametrize("fused", [False, True])
@pytest.mark.parametrize("n,t,h,w,pad,ext", [
    (2, 3, 161, 200, (1, 1), (0, 0)),   # symmetric pads, odd rows: runs that cross strip ends
    (1, 5, 96, 130, (0, 0), (1, 1)),    # 63-column strips, ragged last strip
])
def test_spatial_stride2_row_walk_96(n, t, h, w, pad, ext, fused):
    """The 96-channel spatial route walks down output rows of 63-column strips,
    several rows per workgroup with a 3-row ring in LDS: grids with more rows
    than CUs, so workgroups continue across rows and cross from one strip or
    frame to the next."""
    cin = cout = 96
    x = bf((n, cin, t, h, w), 81, "x")
    wt = inputs.conv_weight(cout, cin, (1, 3, 3), 81, "w", "bf16")
    b = inputs.conv_bias(cout, 81, "b", "bf16")
    g = inputs.norm_gamma(cin, 81, "g", "bf16")
    be = inputs.quantize(inputs.normal((cin,), 81, "be", std=0.3), "bf16")
    res = bf((n, cout, t, (h + 2 * pad[0] + ext[0] - 3) // 2 + 1, (w + 2 * pad[1] + ext[1] - 3) // 2 + 1),
             81, "res")
    print(f"[case] row walk {n}x{t}x{h}x{w} pad={pad} ext={ext} fused={fused}", flush=True)
    L.wvc_reset_counters()
    if fused:
        y = L.wvc_rmsnorm_silu_conv3d_fwd(to_dev(x), to_dev(g), to_dev(wt), to_dev(b), beta=to_dev(be),
                                          residual=to_dev(res), padding=pad, pad_extra=ext)
        xin = oracle.norm_silu(f64(x), f64(g), f64(be), bf16=True)
    else:
        y = L.wvc_causal_conv3d_fwd(to_dev(x), to_dev(wt), to_dev(b), residual=to_dev(res), stride=(1, 2, 2),
                                    padding=pad, pad_extra=ext)
        xin = f64(x)
    strided_route_taken(True)
    ref = oracle.causal_conv3d_strided(xin, f64(wt), f64(b), stride=(1, 2, 2), pad=pad, pad_extra=ext) + f64(res)
    assert tuple(y.shape) == ref.shape
    check_bf16(to_host(y), ref, f"row walk {n}x{t}x{h}x{w} fused={fused}")


def test_fused_norm_spatial_conv_empty_chunk():
    x = L.empty_cl((1, 96, 0, 8, 16))
    g = torch.ones(96, device="cuda", dtype=torch.bfloat16)
    wt = to_dev(inputs.conv_weight(96, 96, (1, 3, 3), 72, "w", "bf16"))
    print("[case] fused norm + spatial conv, empty chunk", flush=True)
    y = L.wvc_rmsnorm_silu_conv3d_fwd(x, g, wt)
    assert tuple(y.shape) == (1, 96, 0, 4, 8)
