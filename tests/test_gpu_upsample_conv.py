"""GPU parity of the conv that reads its input through the nearest 2x upsample
(descriptor field upsample_in = 2), through the C ABI.

Definitions: the decoder's nearest 2x spatial upsample followed by a causal
3x3x3 conv ("Cosmos3 Wan VAE -- engine size vs runtime context memory",
section 10.3 for the conv, its causal padding and the cache concatenated in
front of each chunk).  The expected values come from the oracle: its conv over
its upsample of x and of the cache.  The fused call must also be bitwise the
library's own two-call composition (upsample kernel, then the conv on the
upsampled frames and an upsampled cache), since the conv reads the same
values either way.
"""
import numpy as np
import pytest
import torch

import oracle
from video_vae_causal_amd import _lib as L
from video_vae_causal_amd import inputs
from _gpu_util import check_bf16, f64, to_dev, to_host

pytestmark = pytest.mark.gpu


def cl(t):
    return t.contiguous(memory_format=torch.channels_last_3d)


def case(cin, cout, t, h, w, seed):
    """x and cache at the stored (pre-upsample) size h x w."""
    x = inputs.quantize(inputs.normal((1, cin, t, h, w), seed, "x"), "bf16")
    wt = inputs.conv_weight(cout, cin, (3, 3, 3), seed, "w", "bf16")
    b = inputs.conv_bias(cout, seed, "b", "bf16")
    cache = inputs.quantize(inputs.normal((1, cin, 2, h, w), seed, "cache"), "bf16")
    return x, wt, b, cache


@pytest.mark.parametrize("cin,cout,t,h,w", [
    (64, 64, 3, 6, 10),       # 12x20 conv frame: ragged 16-wide tiles
    (48, 384, 2, 5, 7),       # partial channel block, three channel tiles, 10x14 frame
    (96, 96, 2, 9, 23),       # 16x16x32 MFMA tiles on an 18x46 frame
    (128, 128, 1, 16, 9),     # 32x32 MFMA on 8-wide tiles (32x18 frame)
    (384, 384, 1, 30, 52),    # the decoder's conv after the upsample: 60x104, split K
])
def test_upsampled_input_conv_vs_oracle(cin, cout, t, h, w):
    x, wt, b, cache = case(cin, cout, t, h, w, seed=cin + h + 7)
    print(f"[case] upsample-in conv cin={cin} cout={cout} t={t} {h}x{w} -> {2 * h}x{2 * w}", flush=True)
    xd, wd, bd, cd = to_dev(x), to_dev(wt), to_dev(b), to_dev(cache)
    cout_buf = L.empty_cl((1, cin, 2, h, w))
    L.wvc_reset_counters()
    y = L.wvc_causal_conv3d_fwd(xd, wd, bd, cache_in=cd, cache_out=cout_buf, upsample_in=2)
    assert tuple(y.shape) == (1, cout, t, 2 * h, 2 * w)
    assert L.wvc_get_counters()["fast_3x3x3"] == 1
    ref = oracle.causal_conv3d(oracle.upsample_nearest2x(f64(x)), f64(wt), f64(b),
                               cache=oracle.upsample_nearest2x(f64(cache)))
    check_bf16(to_host(y), ref, f"upsample-in conv {cin}->{cout} {2 * h}x{2 * w}")
    # the cache keeps the input frames before the upsample
    np.testing.assert_array_equal(to_host(cout_buf), oracle.next_cache(f64(cache), f64(x)))
    # bitwise the two-call composition
    up = L.wvc_upsample_nearest2x(xd)
    y2 = L.wvc_causal_conv3d_fwd(up, wd, bd, cache_in=L.wvc_upsample_nearest2x(cd))
    assert torch.equal(y, y2), "fused upsample read differs from upsample + conv"


def test_upsampled_input_chunks_equal_whole_sequence():
    """1-frame chunks with the (pre-upsample) cache equal the whole sequence
    from zero causal padding, bitwise; frame 0 alone matches the oracle."""
    cin, cout, t, h, w = 64, 128, 4, 7, 11
    x, wt, b, _ = case(cin, cout, t, h, w, seed=23)
    xd, wd, bd = to_dev(x), to_dev(wt), to_dev(b)
    print("[case] upsample-in conv chunked vs whole", flush=True)
    whole = L.wvc_causal_conv3d_fwd(xd, wd, bd, upsample_in=2)
    caches = [L.empty_cl((1, cin, 2, h, w)) for _ in range(2)]
    L.wvc_cache_reset(caches[0])
    outs = []
    for i in range(t):
        outs.append(L.wvc_causal_conv3d_fwd(cl(xd[:, :, i:i + 1]), wd, bd, caches[i % 2],
                                            caches[(i + 1) % 2], upsample_in=2))
    assert torch.equal(torch.cat(outs, dim=2), whole)
    ref = oracle.causal_conv3d(oracle.upsample_nearest2x(f64(x)), f64(wt), f64(b))
    check_bf16(to_host(whole), ref, "upsample-in conv whole sequence, zero past")


def test_upsampled_input_conv_norm_equals_composition():
    """wvc_causal_conv3d_norm_fwd reading through the upsample: y and h bitwise
    the upsample kernel, the conv + norm call on the upsampled frames; on the
    decoder's 30x52 -> 60x104 shape (split-K plan: the reduce runs in the norm)
    and on a small whole-K one, with a residual."""
    for cin, cout, h, w, seed in ((384, 384, 30, 52, 31), (64, 64, 6, 9, 32)):
        x, wt, b, cache = case(cin, cout, 1, h, w, seed)
        g = to_dev(inputs.norm_gamma(cout, seed, "g", "bf16"))
        be = to_dev(inputs.norm_beta(cout, seed, "be", "bf16"))
        res = to_dev(inputs.quantize(inputs.normal((1, cout, 1, 2 * h, 2 * w), seed, "r"), "bf16"))
        xd, wd, bd, cd = to_dev(x), to_dev(wt), to_dev(b), to_dev(cache)
        print(f"[case] upsample-in conv + norm {cin}->{cout} {2 * h}x{2 * w}", flush=True)
        y1 = L.empty_cl((1, cout, 1, 2 * h, 2 * w))
        c1 = L.empty_cl((1, cin, 2, h, w))
        h1 = L.wvc_causal_conv3d_norm_fwd(xd, wd, g, bd, be, 1e-12, cd, c1, res, y1, upsample_in=2)
        y2 = L.empty_cl((1, cout, 1, 2 * h, 2 * w))
        c2 = L.empty_cl((1, cin, 2, 2 * h, 2 * w))
        h2 = L.wvc_causal_conv3d_norm_fwd(L.wvc_upsample_nearest2x(xd), wd, g, bd, be, 1e-12,
                                          L.wvc_upsample_nearest2x(cd), c2, res, y2)
        assert torch.equal(y1, y2) and torch.equal(h1, h2)
        assert torch.equal(L.wvc_upsample_nearest2x(c1), c2)
        ref = oracle.causal_conv3d(oracle.upsample_nearest2x(f64(x)), f64(wt), f64(b),
                                   cache=oracle.upsample_nearest2x(f64(cache))) + to_host(res)
        check_bf16(to_host(y1), ref, f"upsample-in conv + residual {cin}->{cout}")


def test_upsampled_input_e4m3_conv():
    """The 8-bit conv reading E4M3 codes through the upsample (the decoder's
    8-bit conv_up): bitwise the 8-bit conv over the codes of the upsampled
    frames (the quantiser is elementwise, so those are the upsampled codes),
    and within the 8-bit conv's bar of the oracle's conv of the decoded,
    upsampled codes."""
    from test_gpu_fp8 import check_e4m3_conv
    cin, cout, t, h, w, seed = 128, 128, 2, 15, 26, 44
    xs = 6.0 / 448
    x = inputs.quantize(inputs.normal((1, cin, t, h, w), seed, "x"), "bf16")
    cache = inputs.quantize(inputs.normal((1, cin, 2, h, w), seed, "cache"), "bf16")
    wt = inputs.conv_weight(cout, cin, (3, 3, 3), seed, "w", "bf16")
    b = inputs.conv_bias(cout, seed, "b", "bf16")
    print(f"[case] upsample-in E4M3 conv {cin}->{cout} t={t} {h}x{w} -> {2 * h}x{2 * w}", flush=True)
    xd, cd, bd = to_dev(x), to_dev(cache), to_dev(b)
    xq, cq = L.wvc_quantize_e4m3(xd, xs), L.wvc_quantize_e4m3(cd, xs)
    wq, wsc = L.wvc_quantize_rows_e4m3(to_dev(wt))
    c_next = L.empty_cl((1, cin, 2, h, w), torch.uint8)
    y = L.wvc_causal_conv3d_e4m3_fwd(xq, xs, wq, wsc, bd, cq, c_next, upsample_in=2)
    assert tuple(y.shape) == (1, cout, t, 2 * h, 2 * w)
    assert torch.equal(c_next, xq)    # t = 2: the cache is the chunk's codes, before the upsample
    y2 = L.wvc_causal_conv3d_e4m3_fwd(L.wvc_quantize_e4m3(L.wvc_upsample_nearest2x(xd), xs), xs, wq,
                                      wsc, bd, L.wvc_quantize_e4m3(L.wvc_upsample_nearest2x(cd), xs))
    assert torch.equal(y, y2), "fused upsample read differs from the upsampled codes"

    def codes(tq):
        return tq.cpu().numpy()

    def up_codes(c):
        return oracle.upsample_nearest2x(c.astype(np.float64)).astype(np.uint8)

    ref = oracle.causal_conv3d_e4m3(up_codes(codes(xq)), xs, codes(wq), wsc.cpu().numpy(), f64(b),
                                    cache_q=up_codes(codes(cq)))
    check_e4m3_conv(to_host(y), ref, "upsample-in E4M3 conv")
