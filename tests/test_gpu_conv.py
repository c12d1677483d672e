"""GPU parity of the causal conv (both MFMA routes and the direct route)
against the fp64 oracle, through the C ABI.

Definitions: "Cosmos3 Wan VAE -- engine size vs runtime context memory",
section 10.3 (conv, causal padding, cache concatenation) and "cache-aware video
decoder lowering" (bias once, stride/padding/dilation honoured, causal order,
route counters and strict mode).
"""
import numpy as np
import pytest
import torch

import oracle
from video_vae_causal_amd import _lib as L
from video_vae_causal_amd import inputs
from _gpu_util import check_bf16, check_f32, f64, to_dev, to_host

pytestmark = pytest.mark.gpu


def cl(t):
    return t.contiguous(memory_format=torch.channels_last_3d)


def conv_case(cin, cout, t, h, w, seed, k=(3, 3, 3), dtype="bf16"):
    x = inputs.quantize(inputs.normal((1, cin, t, h, w), seed, "x"), dtype)
    wt = inputs.conv_weight(cout, cin, k, seed, "w", dtype)
    b = inputs.conv_bias(cout, seed, "b", dtype)
    cache = inputs.quantize(inputs.normal((1, cin, 2, h, w), seed, "cache"), dtype)
    return x, wt, b, cache


@pytest.mark.parametrize("cin,cout,t,h,w", [
    (64, 64, 3, 20, 37),     # ragged tiles in both directions
    (48, 384, 2, 9, 13),     # partial 32-channel block, 3 channel tiles
    (96, 96, 2, 17, 33),     # 96-channel tile variant
    (32, 128, 1, 8, 8),
    (32, 32, 2, 1, 70),      # one-row frames
    (384, 384, 1, 30, 52),   # decoder low-res frame
    # the host's tile choice (fewest ragged positions, 8-wide tiles charged 25 %)
    # gives each MFMA shape x tile width its own LDS maps:
    (96, 96, 2, 14, 45),     # 16x16x32 MFMA on 16-wide tiles, ragged both ways
    (64, 64, 2, 31, 17),     # 16x16x32 MFMA on 8-wide tiles
    (128, 128, 2, 31, 17),   # 32x32x16 MFMA on 8-wide tiles
    (128, 128, 2, 14, 45),   # 32x32x16 MFMA on 16-wide tiles (rotated second rows)
])
def test_conv3x3x3_bf16_vs_oracle(cin, cout, t, h, w):
    x, wt, b, cache = conv_case(cin, cout, t, h, w, seed=cin + cout + h)
    print(f"[case] conv3 cin={cin} cout={cout} t={t} {h}x{w}", flush=True)
    L.wvc_reset_counters()
    y = L.wvc_causal_conv3d_fwd(to_dev(x), to_dev(wt), to_dev(b), cache_in=to_dev(cache))
    ref = oracle.causal_conv3d(f64(x), f64(wt), f64(b), cache=f64(cache))
    check_bf16(to_host(y), ref, f"conv3 {cin}->{cout} {h}x{w}")
    assert L.wvc_get_counters()["fast_3x3x3"] == 1


@pytest.mark.parametrize("cin,cout,t,h,w,tw", [
    (96, 192, 3, 100, 150, 32),  # two channel tiles, ragged rows and columns; 9 stages (odd)
    (64, 64, 4, 128, 200, 16),   # 6 stages (even)
    (96, 96, 8, 2048, 8, 8),     # 8-wide tiles (one per row band), 512 tiles
    (64, 64, 8, 2048, 8, 8),
    (32, 96, 4, 128, 256, 32),   # 3 stages: only the odd last stage
    (48, 64, 3, 130, 260, 32),   # a half-filled channel block (channels past C_in read zero)
])
def test_conv3x3x3_two_waves_per_simd_vs_oracle(cin, cout, t, h, w, tw):
    """Whole-K grids of 16x16 MFMA tiles run two workgroups per CU, two waves
    per SIMD: two weight row sets that alternate while the kernel rows cycle
    through three (two stages per loop iteration, then an odd last stage), and
    the B fragments in a 3-slot ring.  The library names the kernel it
    launches; the case must reach that kernel at the expected tile width."""
    x, wt, b, cache = conv_case(cin, cout, t, h, w, seed=cin + cout + h + 1)
    d = L.conv_desc(x.shape, wt.shape, L.WVC_BF16)
    name = L.wvc_conv3d_kernel_name(d)
    print(f"[case] conv3 two waves per SIMD cin={cin} cout={cout} t={t} {h}x{w}: {name}", flush=True)
    assert name.startswith("igemm_occ2_kernel<") and name.endswith(f", 2, {tw}>"), name
    y = L.wvc_causal_conv3d_fwd(to_dev(x), to_dev(wt), to_dev(b), cache_in=to_dev(cache))
    ref = oracle.causal_conv3d(f64(x), f64(wt), f64(b), cache=f64(cache))
    check_bf16(to_host(y), ref, f"conv3 two waves per SIMD {cin}->{cout} {h}x{w}")


def test_split_k_workspace_reused_across_shapes():
    """Small frames take the split-K path (fp32 partials in the workspace, then
    a reduce kernel).  One workspace, filled with NaN bit patterns first (its
    contents on entry must not matter), serves several calls of different
    shapes in a row; every call must match the oracle and repeat bitwise."""
    shapes = [(384, 384, 1, 30, 52), (96, 96, 1, 17, 23), (384, 384, 1, 60, 104), (48, 384, 1, 30, 52)]
    cases = [conv_case(ci, co, t, h, w, seed=200 + i) for i, (ci, co, t, h, w) in enumerate(shapes)]
    need = max(L.wvc_causal_conv3d_workspace_bytes(L.conv_desc(c[0].shape, c[1].shape, L.WVC_BF16))
               for c in cases)
    assert need > 0, "expected at least one split-K plan"
    ws = torch.full((need,), 0xFF, dtype=torch.uint8, device="cuda")
    for rep in range(2):
        for (ci, co, t, h, w), (x, wt, b, cache) in zip(shapes, cases):
            print(f"[case] split-K rep={rep} {ci}->{co} {h}x{w}", flush=True)
            args = (to_dev(x), to_dev(wt), to_dev(b), to_dev(cache))
            y = L.wvc_causal_conv3d_fwd(*args, workspace=ws)
            y2 = L.wvc_causal_conv3d_fwd(*args, workspace=ws)
            assert torch.equal(y, y2)
            ref = oracle.causal_conv3d(f64(x), f64(wt), f64(b), cache=f64(cache))
            check_bf16(to_host(y), ref, f"split-K {ci}->{co} {h}x{w}")


@pytest.mark.parametrize("cin,cout,t,h,w", [(384, 384, 2, 12, 40), (48, 384, 1, 9, 13),
                                             (96, 96, 2, 17, 33), (64, 64, 1, 10, 10)])
def test_packed_weights_equal_standard_layout_bitwise(cin, cout, t, h, w):
    """A call with weights packed once by wvc_conv3d_pack_weights runs the same
    kernel on the same numbers as a call that packs them itself: bitwise."""
    x, wt, b, cache = conv_case(cin, cout, t, h, w, seed=300 + cin)
    xd, wd, bd, cd = to_dev(x), to_dev(wt), to_dev(b), to_dev(cache)
    packed = L.wvc_conv3d_pack_weights(wd)
    assert packed.numel() == L.wvc_conv3d_packed_weight_bytes(tuple(wd.shape))
    y_std = L.wvc_causal_conv3d_fwd(xd, wd, bd, cd)
    y_pk = L.wvc_causal_conv3d_fwd(xd, wd, bd, cd, packed_weight=packed)
    assert torch.equal(y_std, y_pk)
    check_bf16(to_host(y_pk), oracle.causal_conv3d(f64(x), f64(wt), f64(b), cache=f64(cache)),
               f"packed weights {cin}->{cout}")


def test_conv_residual_and_no_bias():
    x, wt, b, cache = conv_case(64, 64, 2, 11, 19, seed=7)
    res = inputs.quantize(inputs.normal((1, 64, 2, 11, 19), 7, "res"), "bf16")
    y = L.wvc_causal_conv3d_fwd(to_dev(x), to_dev(wt), None, residual=to_dev(res))
    ref = oracle.causal_conv3d(f64(x), f64(wt), None) + f64(res)
    check_bf16(to_host(y), ref, "conv3 + residual, no bias")


def test_conv3x3x3_two_waves_residual_no_bias_cache_out():
    """The two-wave kernel's other epilogue and staging paths: a residual, no
    bias, and the cache of the last two input frames written by its staging
    (the chunk's last output frame), with and without a cache coming in."""
    for cached in (True, False):
        x, wt, _, cache = conv_case(96, 96, 4, 96, 160, seed=61 + cached)
        res = inputs.quantize(inputs.normal((1, 96, 4, 96, 160), 61, "res"), "bf16")
        d = L.conv_desc(x.shape, wt.shape, L.WVC_BF16)
        name = L.wvc_conv3d_kernel_name(d)
        print(f"[case] two waves, residual, no bias, cache_out, cached={cached}: {name}", flush=True)
        assert name.startswith("igemm_occ2_kernel<"), name
        cout = L.empty_cl((1, 96, 2, 96, 160))
        y = L.wvc_causal_conv3d_fwd(to_dev(x), to_dev(wt), None, to_dev(cache) if cached else None, cout,
                                    residual=to_dev(res))
        ref = oracle.causal_conv3d(f64(x), f64(wt), None, cache=f64(cache) if cached else None) + f64(res)
        check_bf16(to_host(y), ref, f"two waves + residual, no bias, cached={cached}")
        np.testing.assert_array_equal(to_host(cout), oracle.next_cache(f64(cache) if cached else None, f64(x)))


def test_cache_out_is_last_two_frames_exactly():
    for t in (1, 2, 4):
        x, wt, b, cache = conv_case(32, 32, t, 6, 10, seed=20 + t)
        cin, cout = to_dev(cache), L.empty_cl((1, 32, 2, 6, 10))
        L.wvc_causal_conv3d_fwd(to_dev(x), to_dev(wt), to_dev(b), cache_in=cin, cache_out=cout)
        expect = oracle.next_cache(f64(cache), f64(x))
        np.testing.assert_array_equal(to_host(cout), expect)
    # no cache_in: the past is zero
    x, wt, b, _ = conv_case(32, 32, 1, 6, 10, seed=30)
    cout = L.empty_cl((1, 32, 2, 6, 10))
    L.wvc_causal_conv3d_fwd(to_dev(x), to_dev(wt), to_dev(b), cache_out=cout)
    np.testing.assert_array_equal(to_host(cout), oracle.next_cache(None, f64(x)))


def test_tiny_f32_config_whole_and_frame_chunks():
    """fp32 causal conv 16->16 on [1,16,5,32,32] (direct route): whole sequence
    and 1-frame chunks with the cache, rel L2 <= 1e-5; chunked == whole bitwise."""
    d = inputs.tiny_conv_inputs(seed=1)
    ref = oracle.causal_conv3d(f64(d["x"]), f64(d["w"]), f64(d["b"]))
    xd, wd, bd = (to_dev(d[k], torch.float32) for k in ("x", "w", "b"))
    L.wvc_reset_counters()
    whole = L.wvc_causal_conv3d_fwd(xd, wd, bd)
    check_f32(to_host(whole), ref, "tiny fp32 whole")
    caches = [L.empty_cl((1, 16, 2, 32, 32), torch.float32) for _ in range(2)]
    L.wvc_cache_reset(caches[0])
    outs = []
    for t in range(5):
        outs.append(L.wvc_causal_conv3d_fwd(cl(xd[:, :, t:t + 1]), wd, bd, caches[t % 2],
                                            caches[(t + 1) % 2]))
    chunked = torch.cat(outs, dim=2)
    check_f32(to_host(chunked), ref, "tiny fp32 1-frame chunks")
    assert torch.equal(chunked, whole)
    assert L.wvc_get_counters()["generic"] == 6


@pytest.mark.parametrize("k,stride,pad,dil", [
    ((3, 3, 3), (1, 2, 2), (1, 1), (1, 1, 1)),
    ((3, 3, 3), (1, 1, 1), (2, 2), (2, 2, 2)),
    ((2, 5, 3), (1, 1, 2), (2, 0), (1, 1, 3)),
    ((3, 3, 3), (1, 1, 1), (1, 1), (1, 1, 1)),
])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_direct_route_stride_pad_dilation(k, stride, pad, dil, dtype):
    cin, cout = 12, 10          # channel counts the MFMA routes do not take
    x = inputs.quantize(inputs.normal((2, cin, 4, 13, 15), 3, "x"), dtype)
    wt = inputs.conv_weight(cout, cin, k, 3, "w", dtype)
    b = inputs.conv_bias(cout, 3, "b", dtype)
    past = dil[0] * (k[0] - 1)
    cache = inputs.quantize(inputs.normal((2, cin, past, 13, 15), 3, "c"), dtype)
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    y = L.wvc_causal_conv3d_fwd(to_dev(x, tdt), to_dev(wt, tdt), to_dev(b, tdt),
                                cache_in=to_dev(cache, tdt) if past else None,
                                stride=stride, padding=pad, dilation=dil)
    ref = oracle.causal_conv3d(f64(x), f64(wt), f64(b), cache=f64(cache) if past else None,
                               stride=stride[1:], pad=pad, dil=dil)
    (check_bf16 if dtype == "bf16" else check_f32)(to_host(y), ref, f"direct {k} {stride} {pad} {dil}")


@pytest.mark.parametrize("cin,cout,t,h,w", [(64, 64, 2, 11, 19),      # one launch, no split
                                             (384, 384, 1, 30, 52),   # split-K + reduce
                                             (96, 96, 3, 5, 9),
                                             (96, 96, 4, 120, 160)])  # whole K, 16x16 tiles: two workgroups per CU
def test_conv3x3x3_batch2_with_cache_out(cin, cout, t, h, w):
    """N = 2: both batch items through the MFMA route in one call, each with
    its own cache frames in and out."""
    n = 2
    x = inputs.quantize(inputs.normal((n, cin, t, h, w), 77, "x"), "bf16")
    wt = inputs.conv_weight(cout, cin, (3, 3, 3), 77, "w", "bf16")
    b = inputs.conv_bias(cout, 77, "b", "bf16")
    cache = inputs.quantize(inputs.normal((n, cin, 2, h, w), 77, "cache"), "bf16")
    print(f"[case] conv3 batch2 {cin}->{cout} t={t} {h}x{w}", flush=True)
    L.wvc_reset_counters()
    cout_t = L.empty_cl((n, cin, 2, h, w))
    y = L.wvc_causal_conv3d_fwd(to_dev(x), to_dev(wt), to_dev(b), cache_in=to_dev(cache),
                                cache_out=cout_t)
    ref = oracle.causal_conv3d(f64(x), f64(wt), f64(b), cache=f64(cache))
    check_bf16(to_host(y), ref, f"conv3 batch2 {cin}->{cout}")
    np.testing.assert_array_equal(to_host(cout_t), oracle.next_cache(f64(cache), f64(x)))
    assert L.wvc_get_counters()["fast_3x3x3"] == 1


@pytest.mark.parametrize("cin,cout,h,w", [(64, 32, 9, 13), (384, 192, 12, 40), (48, 96, 5, 7)])
def test_conv1x1x1_projection(cin, cout, h, w):
    x = inputs.quantize(inputs.normal((1, cin, 2, h, w), 9, "x"), "bf16")
    wt = inputs.conv_weight(cout, cin, (1, 1, 1), 9, "w", "bf16")
    b = inputs.conv_bias(cout, 9, "b", "bf16")
    L.wvc_reset_counters()
    y = L.wvc_causal_conv3d_fwd(to_dev(x), to_dev(wt), to_dev(b), padding=(0, 0))
    ref = oracle.causal_conv3d(f64(x), f64(wt), f64(b), pad=(0, 0))
    check_bf16(to_host(y), ref, f"conv1x1 {cin}->{cout}")
    assert L.wvc_get_counters()["fast_1x1x1"] == 1


@pytest.mark.parametrize("n,cin,cout,t,h,w", [(2, 40, 64, 2, 3, 7),     # C_in not a multiple of 32
                                               (1, 384, 192, 1, 30, 52),  # 1560 positions: ragged last tile
                                               (1, 256, 256, 3, 5, 5),
                                               (2, 96, 32, 1, 1, 63)])
def test_conv1x1x1_projection_edges_with_residual(n, cin, cout, t, h, w):
    """The 1x1x1 route (one 64-position tile per workgroup, all output
    channels): zero-padded channel blocks, a ragged last tile, two batch items
    and a fused residual."""
    x = inputs.quantize(inputs.normal((n, cin, t, h, w), 19, "x"), "bf16")
    wt = inputs.conv_weight(cout, cin, (1, 1, 1), 19, "w", "bf16")
    b = inputs.conv_bias(cout, 19, "b", "bf16")
    res = inputs.quantize(inputs.normal((n, cout, t, h, w), 19, "r"), "bf16")
    print(f"[case] conv1x1 n={n} {cin}->{cout} t={t} {h}x{w}", flush=True)
    L.wvc_reset_counters()
    y = L.wvc_causal_conv3d_fwd(to_dev(x), to_dev(wt), to_dev(b), residual=to_dev(res), padding=(0, 0))
    ref = oracle.causal_conv3d(f64(x), f64(wt), f64(b), pad=(0, 0)) + f64(res)
    check_bf16(to_host(y), ref, f"conv1x1 {cin}->{cout} + residual")
    assert L.wvc_get_counters()["fast_1x1x1"] == 1


@pytest.mark.parametrize("cin,cout,with_bias", [(384, 192, True), (96, 64, False), (256, 128, True),
                                                (320, 176, True)])
def test_conv1x1x1_projection_persistent_vs_oracle(cin, cout, with_bias):
    """Enough 64-position tiles (66049 positions, a 1-position last tile) for
    the persistent variant that keeps the weights in registers and loops over
    tiles: one to three 16-channel blocks per wave, fewer than 12 K-steps and
    an unused block (176 channels), no bias; every output against the oracle,
    with a fused residual."""
    shape = (1, cin, 1, 257, 257)
    x = inputs.quantize(inputs.normal(shape, 23, "x"), "bf16")
    wt = inputs.conv_weight(cout, cin, (1, 1, 1), 23, "w", "bf16")
    b = inputs.conv_bias(cout, 23, "b", "bf16") if with_bias else None
    res = inputs.quantize(inputs.normal((1, cout, 1, 257, 257), 23, "r"), "bf16")
    print(f"[case] conv1x1 persistent {cin}->{cout} 257x257 bias={with_bias}", flush=True)
    y = L.wvc_causal_conv3d_fwd(to_dev(x), to_dev(wt), to_dev(b) if with_bias else None,
                                residual=to_dev(res), padding=(0, 0))
    ref = oracle.causal_conv3d(f64(x), f64(wt), f64(b) if with_bias else None, pad=(0, 0)) + f64(res)
    check_bf16(to_host(y), ref, f"conv1x1 persistent {cin}->{cout}")
    y2 = L.wvc_causal_conv3d_fwd(to_dev(x), to_dev(wt), to_dev(b) if with_bias else None,
                                 residual=to_dev(res), padding=(0, 0))
    assert torch.equal(y, y2), "persistent projection is not run-to-run deterministic"


@pytest.mark.parametrize("sizes", [[1, 1, 1, 1, 1], [2, 3], [4, 1], [1, 4]])
def test_chunked_equals_whole(sizes):
    """Chunks with the rolling cache give the whole-sequence result.  Launches
    of different chunk lengths may split K differently (a different fp32
    summation grouping), so the bar is the bf16 parity bar against the whole
    pass and against the oracle; a repeated chunked run is bitwise equal."""
    x, wt, b, _ = conv_case(64, 128, 5, 14, 22, seed=41)
    xd, wd, bd = to_dev(x), to_dev(wt), to_dev(b)
    whole = L.wvc_causal_conv3d_fwd(xd, wd, bd)

    def chunked():
        caches = [L.empty_cl((1, 64, 2, 14, 22)) for _ in range(2)]
        L.wvc_cache_reset(caches[0])
        outs, t0 = [], 0
        for i, s in enumerate(sizes):
            outs.append(L.wvc_causal_conv3d_fwd(cl(xd[:, :, t0:t0 + s]), wd, bd, caches[i % 2],
                                                caches[(i + 1) % 2]))
            t0 += s
        return torch.cat(outs, dim=2)

    a = chunked()
    assert torch.equal(a, chunked())
    check_bf16(to_host(a), to_host(whole), f"chunks {sizes} vs whole")
    check_bf16(to_host(a), oracle.causal_conv3d(f64(x), f64(wt), f64(b)), f"chunks {sizes} vs oracle")


@pytest.mark.parametrize("t0", [0, 2, 4])
def test_causality_bitwise(t0):
    x, wt, b, _ = conv_case(32, 64, 6, 10, 18, seed=50)
    y0 = L.wvc_causal_conv3d_fwd(to_dev(x), to_dev(wt), to_dev(b))
    x2 = x.copy()
    x2[:, :, t0] = inputs.quantize(inputs.normal((1, 32, 10, 18), 51, "p"), "bf16")
    y1 = L.wvc_causal_conv3d_fwd(to_dev(x2), to_dev(wt), to_dev(b))
    assert torch.equal(y1[:, :, :t0], y0[:, :, :t0])
    for t in range(t0, min(t0 + 3, 6)):
        assert not torch.equal(y1[:, :, t], y0[:, :, t])
    assert torch.equal(y1[:, :, t0 + 3:], y0[:, :, t0 + 3:])


def test_bias_added_exactly_once():
    for cin, cout, dtype in ((64, 128, "bf16"), (12, 10, "f32")):
        _, wt, b, _ = conv_case(cin, cout, 2, 7, 9, seed=60, dtype=dtype)
        tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
        x = torch.zeros((1, cin, 3, 7, 9), dtype=tdt, device="cuda").contiguous(
            memory_format=torch.channels_last_3d)
        y = L.wvc_causal_conv3d_fwd(x, to_dev(wt, tdt), to_dev(b, tdt))
        expect = np.broadcast_to(f64(b)[None, :, None, None, None], y.shape)
        np.testing.assert_array_equal(to_host(y), expect)


def test_determinism_bitwise():
    x, wt, b, cache = conv_case(96, 96, 3, 25, 31, seed=70)
    args = (to_dev(x), to_dev(wt), to_dev(b), to_dev(cache))
    y0 = L.wvc_causal_conv3d_fwd(*args)
    y1 = L.wvc_causal_conv3d_fwd(*args)
    assert torch.equal(y0, y1)


def test_output_canaries_untouched():
    """Outputs are written into the front of a larger buffer whose tail holds a
    sentinel; the tail must be untouched (no out-of-bounds stores)."""
    cin, cout, t, h, w = 64, 128, 2, 9, 21
    x, wt, b, _ = conv_case(cin, cout, t, h, w, seed=80)
    numel = t * h * w * cout
    flat = torch.full((numel + 4096,), 0x7FC1, dtype=torch.int16, device="cuda")
    y = flat[:numel].view(torch.bfloat16).view(1, t, h, w, cout).permute(0, 4, 1, 2, 3)
    assert y.is_contiguous(memory_format=torch.channels_last_3d)
    L.wvc_causal_conv3d_fwd(to_dev(x), to_dev(wt), to_dev(b), y=y)
    assert torch.all(flat[numel:] == 0x7FC1)
    ref = oracle.causal_conv3d(f64(x), f64(wt), f64(b))
    check_bf16(to_host(y), ref, "canary run")


def test_strict_mode_allows_fast_route_and_refuses_generic():
    x, wt, b, _ = conv_case(32, 32, 1, 6, 6, seed=90)
    L.wvc_set_strict(True)
    try:
        L.wvc_causal_conv3d_fwd(to_dev(x), to_dev(wt), to_dev(b))
        with pytest.raises(L.WvcError) as e:
            L.wvc_causal_conv3d_fwd(to_dev(x, torch.float32), to_dev(wt, torch.float32))
        assert e.value.code == L.WVC_ERR_STRICT
    finally:
        L.wvc_set_strict(False)


def test_conv_planned_for_fewer_cus_vs_oracle():
    """cu_limit = 160: the 384-channel 30x52 frame splits K 6 ways instead of
    9 (144 workgroups instead of 216, leaving CUs to another stream's work);
    the result stays within the bf16 bar of the oracle and within rounding of
    the full-device plan, which adds the same products in another grouping."""
    x, wt, b, cache = conv_case(384, 384, 1, 30, 52, seed=61)
    print("[case] conv 384 30x52 planned for 160 CUs", flush=True)
    xd, wd, bd, cd = to_dev(x), to_dev(wt), to_dev(b), to_dev(cache)
    y6 = L.wvc_causal_conv3d_fwd(xd, wd, bd, cache_in=cd, cu_limit=160)
    y9 = L.wvc_causal_conv3d_fwd(xd, wd, bd, cache_in=cd)
    ref = oracle.causal_conv3d(f64(x), f64(wt), f64(b), cache=f64(cache))
    check_bf16(to_host(y6), ref, "conv 384 30x52, 160 CUs")
    check_bf16(to_host(y6), to_host(y9), "conv 384 30x52, 160 CUs vs all CUs")
