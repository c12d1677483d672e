"""C-ABI tests that need no GPU: the library loads, exports every symbol the
header declares, and rejects bad calls with the documented status code before
enqueueing anything (so fake, never-dereferenced pointers are safe here).

Route guard semantics follow "cache-aware video decoder lowering" (section on
turning Conv3D into batched Conv2D): the fast path covers unit temporal stride
and one group; counters record each call's route; strict mode stops on an
unexpected fallback.
"""
import ctypes
import os
import re

import pytest

from video_vae_causal_amd import _lib as L

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "wvc.h")

# Fake device addresses: validation compares them but never dereferences them.
X, CIN, COUT, W, B, Y, WS = (0x10000000 + i * 0x01000000 for i in range(7))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(L.LIB_PATH):
        pytest.skip("libwvc.so not built")
    return L.load()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(wvc_[a-z0-9_]+)\s*\(", text)))


def test_header_and_binding_agree():
    assert sorted(L.EXPORTED) == declared_functions()


def test_library_exports_every_declared_symbol(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name
    assert L.wvc_version().startswith("libwvc")


def desc(**kw):
    base = dict(x_shape=(1, 16, 2, 8, 8), w_shape=(16, 16, 3, 3, 3), dtype=L.WVC_BF16)
    base.update(kw)
    return L.conv_desc(base["x_shape"], base["w_shape"], base["dtype"],
                       base.get("stride", (1, 1, 1)), base.get("padding", (1, 1)),
                       base.get("dilation", (1, 1, 1)), base.get("groups", 1))


def call(lib, d, x=X, cin=CIN, cout=COUT, w=W, b=B, res=None, y=Y, ws=None, wsb=0):
    return lib.wvc_causal_conv3d_fwd(ctypes.byref(d) if d is not None else None, x, cin, cout, w,
                                     b, res, y, ws, wsb, None)


def test_unsupported_guard_and_rejected_counter(lib):
    L.wvc_reset_counters()
    assert call(lib, desc(groups=2)) == L.WVC_ERR_UNSUPPORTED
    assert "group" in L.wvc_last_error()
    assert call(lib, desc(dtype=7)) == L.WVC_ERR_UNSUPPORTED
    c = L.wvc_get_counters()
    assert c["rejected"] == 2 and c["fast_3x3x3"] == c["generic"] == c["fast_strided"] == 0


def test_temporal_stride_and_phase_validation(lib):
    """Temporal stride is legal (the encoder's downsample); its phase must lie
    in [0, stride_t) and trailing pads must be >= 0."""
    d = desc(stride=(2, 1, 1), w_shape=(16, 16, 3, 1, 1), padding=(0, 0))
    assert L.wvc_causal_conv3d_workspace_bytes(d) >= 0
    d.t_phase = 2
    assert call(lib, d) == L.WVC_ERR_ARG and "t_phase" in L.wvc_last_error()
    d.t_phase = -1
    assert call(lib, d) == L.WVC_ERR_ARG
    assert call(lib, desc(stride=(0, 1, 1))) == L.WVC_ERR_ARG
    e = desc(stride=(1, 2, 2), w_shape=(16, 16, 1, 3, 3), padding=(0, 0))
    e.pad_h_extra = -1
    assert call(lib, e) == L.WVC_ERR_ARG
    # output frames: anchors first = (s - phase) % s, first + s, ... inside the chunk
    assert [L.conv_out_frames(t, 2, ph) for t, ph in ((1, 0), (1, 1), (4, 1), (5, 0), (9, 0))] == \
        [1, 0, 2, 3, 5]
    # y is sized for t_out frames: a 1-frame chunk at odd phase writes nothing,
    # so even a y of zero bytes passes the size checks (argument errors only here)
    f = desc(x_shape=(1, 16, 1, 8, 8), stride=(2, 1, 1), w_shape=(16, 16, 3, 1, 1), padding=(0, 0))
    f.t_phase = 1
    assert L.wvc_causal_conv3d_workspace_bytes(f) >= 0


def test_bad_arguments(lib):
    assert call(lib, None) == L.WVC_ERR_ARG
    assert call(lib, desc(x_shape=(0, 16, 2, 8, 8))) == L.WVC_ERR_ARG
    assert call(lib, desc(x_shape=(1, 16, -1, 8, 8))) == L.WVC_ERR_ARG
    assert call(lib, desc(padding=(-1, 1))) == L.WVC_ERR_ARG
    assert call(lib, desc(dilation=(0, 1, 1))) == L.WVC_ERR_ARG
    assert call(lib, desc(x_shape=(1, 16, 2, 1, 1), padding=(0, 0))) == L.WVC_ERR_ARG
    assert call(lib, desc(), w=None) == L.WVC_ERR_ARG
    assert call(lib, desc(), x=None) == L.WVC_ERR_ARG
    assert call(lib, desc(), ws=None, wsb=64) == L.WVC_ERR_ARG
    assert L.wvc_last_error()


def test_aliasing_of_written_buffers(lib):
    assert call(lib, desc(), y=X) == L.WVC_ERR_ALIAS                 # in place
    assert "'y'" in L.wvc_last_error()
    assert call(lib, desc(), cout=CIN) == L.WVC_ERR_ALIAS            # cache not ping-ponged
    assert call(lib, desc(), y=X + 64) == L.WVC_ERR_ALIAS            # partial overlap
    assert call(lib, desc(), ws=W, wsb=16) == L.WVC_ERR_ALIAS         # workspace on weights
    assert call(lib, desc(), cout=Y + 2048) == L.WVC_ERR_ALIAS       # cache_out inside y


def test_read_only_buffers_may_overlap_until_a_launch(lib):
    """residual == x is legal; with strict mode on, an fp32 call (generic route)
    is refused before any launch, proving validation passed the aliasing."""
    L.wvc_set_strict(True)
    try:
        d = desc(dtype=L.WVC_F32)
        assert call(lib, d, res=X) != L.WVC_ERR_ALIAS
        assert call(lib, d, res=X) == L.WVC_ERR_STRICT
    finally:
        L.wvc_set_strict(False)


def test_strict_mode_refuses_generic_route(lib):
    L.wvc_reset_counters()
    L.wvc_set_strict(True)
    try:
        assert L.wvc_get_strict()
        assert call(lib, desc(dtype=L.WVC_F32)) == L.WVC_ERR_STRICT
        assert call(lib, desc(stride=(1, 2, 2))) == L.WVC_ERR_STRICT
        assert call(lib, desc(w_shape=(16, 16, 3, 5, 5), padding=(2, 2))) == L.WVC_ERR_STRICT
        # misaligned pointers fall to the generic route as well
        assert call(lib, desc(), x=X + 2) == L.WVC_ERR_STRICT
        assert "strict" in L.wvc_last_error()
        assert L.wvc_get_counters()["rejected"] == 4
    finally:
        L.wvc_set_strict(False)
    assert not L.wvc_get_strict()


def test_cache_frames_and_workspace_queries(lib):
    assert lib.wvc_conv3d_cache_frames(ctypes.byref(desc())) == 2
    assert lib.wvc_conv3d_cache_frames(ctypes.byref(desc(w_shape=(16, 16, 1, 1, 1)))) == 0
    assert lib.wvc_conv3d_cache_frames(ctypes.byref(desc(dilation=(3, 1, 1)))) == 6
    assert lib.wvc_conv3d_cache_frames(None) == -1
    L.wvc_reset_counters()
    assert L.wvc_causal_conv3d_workspace_bytes(desc()) == 0
    with pytest.raises(L.WvcError):
        L.wvc_causal_conv3d_workspace_bytes(desc(groups=2))
    assert L.wvc_get_counters()["rejected"] == 0   # a size query is not a call
    # the strided MFMA routes pack standard-layout weights into the workspace
    t = desc(x_shape=(1, 32, 3, 8, 8), w_shape=(32, 32, 3, 1, 1), stride=(2, 1, 1), padding=(0, 0))
    assert L.wvc_causal_conv3d_workspace_bytes(t) >= 32 * 32 * 3 * 2


def test_packed_weight_layout_validation(lib):
    L.wvc_reset_counters()
    d = desc(dtype=L.WVC_F32)
    assert lib.wvc_conv3d_packed_weight_bytes(ctypes.byref(d)) == ctypes.c_size_t(-1).value
    assert lib.wvc_conv3d_pack_weights(ctypes.byref(d), W, WS, None) == L.WVC_ERR_UNSUPPORTED
    d = desc(dtype=L.WVC_F32)
    d.weight_layout = L.WVC_WEIGHT_PACKED
    assert call(lib, d) == L.WVC_ERR_UNSUPPORTED
    d = desc(x_shape=(1, 32, 2, 8, 8), w_shape=(32, 32, 3, 3, 3))
    d.weight_layout = 7
    assert call(lib, d) == L.WVC_ERR_ARG
    # 384 -> 384 3x3x3: 384 * 27 * 384 * 2 bytes, channels padded to 32
    d = desc(x_shape=(1, 384, 1, 8, 8), w_shape=(384, 384, 3, 3, 3))
    assert lib.wvc_conv3d_packed_weight_bytes(ctypes.byref(d)) == 384 * 27 * 384 * 2
    d = desc(x_shape=(1, 48, 1, 8, 8), w_shape=(384, 48, 3, 3, 3))
    assert lib.wvc_conv3d_packed_weight_bytes(ctypes.byref(d)) == 384 * 27 * 64 * 2
    assert lib.wvc_conv3d_pack_weights(ctypes.byref(d), W, W + 64, None) == L.WVC_ERR_ALIAS
    assert lib.wvc_conv3d_pack_weights(ctypes.byref(d), W, None, None) == L.WVC_ERR_ARG
    # a packed call whose tensors are not 16-byte aligned cannot fall back
    d = desc(x_shape=(1, 32, 2, 8, 8), w_shape=(32, 32, 3, 3, 3))
    d.weight_layout = L.WVC_WEIGHT_PACKED
    assert call(lib, d, x=X + 2) == L.WVC_ERR_ARG


def rb_desc(c_in=16, c_out=16, t=1, eps=1e-12):
    return L.resblock_desc((1, c_in, t, 8, 8), c_out, L.WVC_BF16, eps)


def test_resblock_validation(lib):
    d = rb_desc()
    need = L.wvc_resblock_workspace_bytes(d)
    assert need >= 3 * 8 * 8 * 16 * 2
    assert L.wvc_resblock_workspace_bytes(rb_desc(c_out=32)) > need   # shortcut output too
    p = L.ResblockParams()
    p.gamma1, p.w1, p.gamma2, p.w2 = 0x50000000, 0x51000000, 0x52000000, 0x53000000

    def rcall(d, x=X, y=Y, params=p, ws=WS, wsb=None, c1i=None, c1o=None):
        return lib.wvc_resblock_fwd(ctypes.byref(d), x, y, ctypes.byref(params) if params else None,
                                    c1i, c1o, None, None, ws, need if wsb is None else wsb, None)

    assert rcall(d, wsb=need - 1) == L.WVC_ERR_WORKSPACE
    assert rcall(d, params=None) == L.WVC_ERR_ARG
    assert rcall(rb_desc(eps=0.0)) == L.WVC_ERR_ARG
    assert rcall(rb_desc(c_out=32)) == L.WVC_ERR_ARG       # C_in != C_out needs w_short
    assert rcall(d, y=X) == L.WVC_ERR_ALIAS
    assert rcall(d, ws=Y) == L.WVC_ERR_ALIAS
    assert rcall(d, c1i=CIN, c1o=CIN) == L.WVC_ERR_ALIAS
    q = L.ResblockParams()
    q.gamma1 = 0x50000000
    assert rcall(d, params=q) == L.WVC_ERR_ARG


def test_resblock_halves_validation(lib):
    d = rb_desc()
    need = L.wvc_resblock_workspace_bytes(d)
    p = L.ResblockParams()
    p.gamma1, p.w1, p.gamma2, p.w2 = 0x50000000, 0x51000000, 0x52000000, 0x53000000
    H2 = 0x60000000

    def front(d=d, x=X, h2=H2, params=p, ws=WS, wsb=need, c1i=None, c1o=None):
        return lib.wvc_resblock_front(ctypes.byref(d), x, h2, ctypes.byref(params) if params else None,
                                      c1i, c1o, ws, wsb, None)

    def back(d=d, h2=H2, x=X, y=Y, params=p, ws=WS, wsb=need, c2i=None, c2o=None):
        return lib.wvc_resblock_back(ctypes.byref(d), h2, x, y, ctypes.byref(params) if params else None,
                                     c2i, c2o, ws, wsb, None)

    assert front(params=None) == L.WVC_ERR_ARG and back(params=None) == L.WVC_ERR_ARG
    assert front(wsb=need - 1) == L.WVC_ERR_WORKSPACE and back(wsb=need - 1) == L.WVC_ERR_WORKSPACE
    assert front(h2=None) == L.WVC_ERR_ARG and back(h2=None) == L.WVC_ERR_ARG
    assert front(h2=X) == L.WVC_ERR_ALIAS           # h2 is written: may not overlap x
    assert back(y=H2) == L.WVC_ERR_ALIAS            # y may not overlap h2
    assert back(ws=H2) == L.WVC_ERR_ALIAS
    assert front(c1i=CIN, c1o=CIN) == L.WVC_ERR_ALIAS
    assert back(c2i=CIN, c2o=CIN) == L.WVC_ERR_ALIAS
    assert back(d=rb_desc(c_out=32)) == L.WVC_ERR_ARG   # the shortcut conv is the back half's
    q = L.ResblockParams()
    q.w2 = 0x53000000
    assert front(params=q) == L.WVC_ERR_ARG         # the front half needs gamma1, w1, gamma2
    r = L.ResblockParams()
    r.gamma1, r.w1, r.gamma2 = 0x50000000, 0x51000000, 0x52000000
    assert back(params=r) == L.WVC_ERR_ARG          # the back half needs w2


def test_norm_and_upsample_validation(lib):
    assert lib.wvc_rmsnorm_silu(X, B, None, Y, 1, 0, 1, 4, 4, L.WVC_BF16, 1e-12, 1, None) == L.WVC_ERR_ARG
    assert lib.wvc_rmsnorm_silu(X, B, None, Y, 1, 8, 1, 4, 4, L.WVC_BF16, 0.0, 1, None) == L.WVC_ERR_ARG
    assert lib.wvc_rmsnorm_silu(X, None, None, Y, 1, 8, 1, 4, 4, L.WVC_BF16, 1e-12, 1, None) == L.WVC_ERR_ARG
    assert lib.wvc_rmsnorm_silu(X, B, None, X, 1, 8, 1, 4, 4, L.WVC_BF16, 1e-12, 1, None) == L.WVC_ERR_ALIAS
    assert lib.wvc_rmsnorm_silu(X, B, None, Y, 1, 8, 1, 4, 4, 9, 1e-12, 1, None) == L.WVC_ERR_UNSUPPORTED
    assert lib.wvc_upsample_nearest2x(X, X + 16, 1, 8, 1, 4, 4, L.WVC_BF16, None) == L.WVC_ERR_ALIAS
    assert lib.wvc_upsample_nearest2x(X, Y, 1, 8, 1, 0, 4, L.WVC_BF16, None) == L.WVC_ERR_ARG
    assert lib.wvc_cache_reset(None, 64, None) == L.WVC_ERR_ARG
    assert lib.wvc_cache_reset(X + 2, 64, None) == L.WVC_ERR_ARG
    assert lib.wvc_cache_reset(X, 6, None) == L.WVC_ERR_ARG
    assert lib.wvc_cache_reset(X, 0, None) == L.WVC_OK


def test_binding_refuses_host_tensors(lib):
    import torch
    x = torch.zeros((1, 16, 1, 4, 4), dtype=torch.bfloat16)
    w = torch.zeros((16, 16, 3, 3, 3), dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        L.wvc_causal_conv3d_fwd(x, w)


def test_graph_calls_reject_bad_arguments_without_touching_the_gpu(lib):
    # the null stream cannot be captured; NULL handles are argument errors
    assert lib.wvc_graph_capture_begin(None) == L.WVC_ERR_ARG
    assert "null stream" in L.wvc_last_error()
    h = ctypes.c_void_p(0x1234)
    assert lib.wvc_graph_capture_end(None, ctypes.byref(h)) == L.WVC_ERR_ARG
    assert h.value is None                      # *graph is cleared on failure
    assert lib.wvc_graph_capture_end(ctypes.c_void_p(0x1000), None) == L.WVC_ERR_ARG
    assert lib.wvc_graph_launch(None, None) == L.WVC_ERR_ARG
    assert lib.wvc_graph_destroy(None) == L.WVC_OK


def test_tiling_validation(lib):
    A, WS_, T = 0x70000000, 0x78000000, 0x7c000000
    # window outside the frame, bad dtype, aliasing
    assert lib.wvc_tile_extract(X, Y, 1, 8, 1, 16, 16, 10, 0, 8, 8, L.WVC_BF16, None) == L.WVC_ERR_ARG
    assert lib.wvc_tile_extract(X, Y, 1, 8, 1, 16, 16, 0, 0, 8, 8, 9, None) == L.WVC_ERR_UNSUPPORTED
    assert lib.wvc_tile_extract(X, X, 1, 8, 1, 16, 16, 0, 0, 8, 8, L.WVC_BF16, None) == L.WVC_ERR_ALIAS
    # blend: C % 4, ramps beyond the tile, tile outside the output, aliasing acc/wsum
    assert lib.wvc_tile_blend(T, A, WS_, 1, 6, 1, 8, 8, 16, 16, 0, 0, 0, 0, 0, 0, L.WVC_BF16, None) == L.WVC_ERR_ARG
    assert lib.wvc_tile_blend(T, A, WS_, 1, 8, 1, 8, 8, 16, 16, 0, 0, 9, 0, 0, 0, L.WVC_BF16, None) == L.WVC_ERR_ARG
    assert lib.wvc_tile_blend(T, A, WS_, 1, 8, 1, 8, 8, 16, 16, 12, 0, 0, 0, 0, 0, L.WVC_BF16, None) == L.WVC_ERR_ARG
    assert lib.wvc_tile_blend(T, A, A + 64, 1, 8, 1, 8, 8, 16, 16, 0, 0, 0, 0, 0, 0, L.WVC_BF16, None) == L.WVC_ERR_ALIAS
    assert lib.wvc_tile_blend_finish(A, WS_, A, 1, 8, 1, 16, 16, L.WVC_BF16, None) == L.WVC_ERR_ALIAS
    assert lib.wvc_tile_blend_finish(A, WS_, Y, 1, 6, 1, 16, 16, L.WVC_BF16, None) == L.WVC_ERR_ARG
    assert stream_origins() == [[0, 30, 60], [0, 52, 104], [0]]


def stream_origins():
    from video_vae_causal_amd import stream
    return [stream.tile_origins(120, 60, 30), stream.tile_origins(208, 104, 52), stream.tile_origins(40, 60, 30)]


def e4m3_call(lib, d, x=X, xs=1.0, cin=CIN, cout=COUT, w=W, ws_scale=WS + 0x100000, b=B, res=None,
              y=Y, ws=None, wsb=0):
    return lib.wvc_causal_conv3d_e4m3_fwd(ctypes.byref(d) if d is not None else None, x, xs, cin,
                                          cout, w, ws_scale, b, res, y, ws, wsb, None)


def test_e4m3_conv_validation(lib):
    ok = desc(x_shape=(1, 32, 2, 8, 8), w_shape=(32, 32, 3, 3, 3), dtype=L.WVC_E4M3)
    need = lib.wvc_causal_conv3d_workspace_bytes(ctypes.byref(ok))
    assert need != ctypes.c_size_t(-1).value and need > 0  # packs the weights
    # packed sizes: one 64-byte slice per (output channel, tap, 64-channel unit)
    assert lib.wvc_conv3d_packed_weight_bytes(ctypes.byref(ok)) == 32 * 27 * 64
    wide = desc(x_shape=(1, 96, 2, 8, 8), w_shape=(128, 96, 3, 3, 3), dtype=L.WVC_E4M3)
    assert lib.wvc_conv3d_packed_weight_bytes(ctypes.byref(wide)) == 128 * 27 * 2 * 64
    # the bf16 entry point refuses 8-bit descriptors
    assert call(lib, ok) == L.WVC_ERR_UNSUPPORTED
    assert "e4m3" in L.wvc_last_error()
    # the 8-bit entry point needs an 8-bit descriptor
    assert e4m3_call(lib, desc()) == L.WVC_ERR_ARG
    assert e4m3_call(lib, None) == L.WVC_ERR_ARG
    # 3x3x3 / stride 1 / pad 1 / C_in % 16 / C_out % 32 only: no generic 8-bit route
    for bad in (desc(x_shape=(1, 32, 2, 8, 8), w_shape=(32, 32, 1, 1, 1), padding=(0, 0), dtype=L.WVC_E4M3),
                desc(x_shape=(1, 24, 2, 8, 8), w_shape=(32, 24, 3, 3, 3), dtype=L.WVC_E4M3),
                desc(x_shape=(1, 32, 2, 8, 8), w_shape=(48, 32, 3, 3, 3), dtype=L.WVC_E4M3),
                desc(x_shape=(1, 32, 2, 8, 8), w_shape=(32, 32, 3, 3, 3), dilation=(1, 2, 2),
                     dtype=L.WVC_E4M3),
                desc(x_shape=(1, 32, 2, 8, 8), w_shape=(32, 32, 3, 3, 3), stride=(1, 2, 2),
                     dtype=L.WVC_E4M3)):
        assert e4m3_call(lib, bad) == L.WVC_ERR_UNSUPPORTED
    # scales
    assert e4m3_call(lib, ok, ws_scale=None, ws=WS, wsb=need) == L.WVC_ERR_ARG
    assert e4m3_call(lib, ok, ws_scale=WS + 4, ws=WS, wsb=need) == L.WVC_ERR_ARG  # unaligned
    for xs in (0.0, -1.0, float("inf"), float("nan")):
        assert e4m3_call(lib, ok, xs=xs, ws=WS, wsb=need) == L.WVC_ERR_ARG
    # workspace too small, unaligned tensors, aliasing of y with the scales
    assert e4m3_call(lib, ok, ws=WS, wsb=need - 1) == L.WVC_ERR_WORKSPACE
    assert e4m3_call(lib, ok, x=X + 8, ws=WS, wsb=need) == L.WVC_ERR_ARG
    assert e4m3_call(lib, ok, ws_scale=Y, ws=WS, wsb=need) == L.WVC_ERR_ALIAS
    # the block entry points stay 16/32-bit
    rd = L.resblock_desc((1, 32, 2, 8, 8), 32, L.WVC_E4M3)
    assert lib.wvc_resblock_workspace_bytes(ctypes.byref(rd)) == ctypes.c_size_t(-1).value


def test_e4m3_quantiser_and_norm_validation(lib):
    assert lib.wvc_quantize_e4m3(X, L.WVC_E4M3, 16, 1.0, Y, None) == L.WVC_ERR_UNSUPPORTED
    assert lib.wvc_quantize_e4m3(X, L.WVC_BF16, -1, 1.0, Y, None) == L.WVC_ERR_ARG
    for sc in (0.0, -2.0, float("inf"), float("nan")):
        assert lib.wvc_quantize_e4m3(X, L.WVC_BF16, 16, sc, Y, None) == L.WVC_ERR_ARG
    assert lib.wvc_quantize_e4m3(X, L.WVC_BF16, 16, 1.0, None, None) == L.WVC_ERR_ARG
    assert lib.wvc_quantize_e4m3(X, L.WVC_BF16, 64, 1.0, X + 64, None) == L.WVC_ERR_ALIAS
    assert lib.wvc_quantize_e4m3(None, L.WVC_BF16, 0, 1.0, None, None) == L.WVC_OK  # empty
    assert lib.wvc_quantize_rows_e4m3(X, L.WVC_F32, 4, 0, Y, W, None) == L.WVC_ERR_ARG
    assert lib.wvc_quantize_rows_e4m3(X, L.WVC_F32, 4, 8, Y, None, None) == L.WVC_ERR_ARG
    assert lib.wvc_quantize_rows_e4m3(X, L.WVC_F32, 4, 8, Y, Y + 8, None) == L.WVC_ERR_ALIAS
    assert lib.wvc_quantize_rows_e4m3(X, 7, 4, 8, Y, W, None) == L.WVC_ERR_UNSUPPORTED
    args = dict(n=1, c=16, t=1, h=4, w=4)
    norm = lambda **kw: lib.wvc_rmsnorm_silu_e4m3(
        kw.get("x", X), kw.get("g", W), None, kw.get("q", Y), args["n"], args["c"], args["t"],
        args["h"], args["w"], kw.get("eps", 1e-12), 1, kw.get("scale", 1.0), None)
    assert norm(eps=0.0) == L.WVC_ERR_ARG
    assert norm(scale=0.0) == L.WVC_ERR_ARG
    assert norm(g=None) == L.WVC_ERR_ARG
    assert norm(q=X + 16) == L.WVC_ERR_ALIAS


def test_fused_norm_conv_validation(lib):
    sp = L.conv_desc((1, 96, 2, 16, 16), (96, 96, 1, 3, 3), L.WVC_BF16, stride=(1, 2, 2),
                     padding=(0, 0), pad_extra=(1, 1))
    need = lib.wvc_causal_conv3d_workspace_bytes(ctypes.byref(sp))
    G, BE = W + 0x200000, W + 0x300000
    f = lambda d, **kw: lib.wvc_rmsnorm_silu_conv3d_fwd(
        ctypes.byref(d), kw.get("x", X), kw.get("g", G), kw.get("be", BE), kw.get("eps", 1e-12), W, B,
        None, kw.get("y", Y), WS, need, None)
    # only the stride-2 spatial route has a fused form
    assert f(desc()) == L.WVC_ERR_UNSUPPORTED
    assert f(sp, g=None) == L.WVC_ERR_ARG
    assert f(sp, eps=0.0) == L.WVC_ERR_ARG
    assert f(sp, g=G + 8) == L.WVC_ERR_ARG        # unaligned gamma
    assert f(sp, y=G) == L.WVC_ERR_ALIAS          # y over gamma
    assert need > 0  # standard-layout weights are packed into the workspace
    assert lib.wvc_rmsnorm_silu_conv3d_fwd(ctypes.byref(sp), X, G, None, 1e-12, W, B, None, Y, WS,
                                           need - 1, None) == L.WVC_ERR_WORKSPACE


def test_resblock_e4m3_validation(lib):
    rd = L.resblock_desc((1, 32, 2, 8, 8), 32, L.WVC_BF16)
    need = lib.wvc_resblock_e4m3_workspace_bytes(ctypes.byref(rd))
    assert need != ctypes.c_size_t(-1).value and need > 0
    bad = L.resblock_desc((1, 32, 2, 8, 8), 64, L.WVC_BF16)   # projection shortcut
    assert lib.wvc_resblock_e4m3_workspace_bytes(ctypes.byref(bad)) == ctypes.c_size_t(-1).value
    f32 = L.resblock_desc((1, 32, 2, 8, 8), 32, L.WVC_F32)
    assert lib.wvc_resblock_e4m3_workspace_bytes(ctypes.byref(f32)) == ctypes.c_size_t(-1).value
    odd = L.resblock_desc((1, 24, 2, 8, 8), 24, L.WVC_BF16)   # C % 16 != 0: no 8-bit conv
    assert lib.wvc_resblock_e4m3_workspace_bytes(ctypes.byref(odd)) == ctypes.c_size_t(-1).value

    def params(**kw):
        pr = L.ResblockE4M3Params()
        base = dict(gamma1=W + 0x100000, gamma2=W + 0x110000, w1=W, w2=W + 0x200000,
                    w1_scale=W + 0x300000, w2_scale=W + 0x310000, s1=0.01, s2=0.01)
        base.update(kw)
        for k, v in base.items():
            setattr(pr, k, v)
        return pr

    call = lambda pr, wsb=need, y=Y: lib.wvc_resblock_e4m3_fwd(
        ctypes.byref(rd), X, y, ctypes.byref(pr), None, None, None, None, WS, wsb, None)
    assert call(params(w1_scale=None)) == L.WVC_ERR_ARG
    assert call(params(gamma2=None)) == L.WVC_ERR_ARG
    assert call(params(s1=0.0)) == L.WVC_ERR_ARG
    assert call(params(s2=float("inf"))) == L.WVC_ERR_ARG
    assert call(params(), wsb=need - 1) == L.WVC_ERR_WORKSPACE
    assert call(params(), y=X) == L.WVC_ERR_ALIAS
    assert lib.wvc_resblock_e4m3_fwd(ctypes.byref(rd), X, Y, None, None, None, None, None, WS, need,
                                     None) == L.WVC_ERR_ARG


# ---------------------------------------------------------------------------
# Binding-side size checks.  The C ABI sizes every buffer from the descriptor
# it builds from x and the weight, so a buffer of another size must be refused
# by the binding before any launch.  Here the binding's device check points at
# the CPU, so host tensors stand in for device ones; every call below must
# raise before reaching the stream query (which would need a GPU).
# ---------------------------------------------------------------------------

@pytest.fixture
def host_binding(lib, monkeypatch):
    import torch
    monkeypatch.setattr(L, "DEVICE_TYPE", "cpu")

    def no_launch(*a, **k):
        raise AssertionError("reached a launch: the mismatch was not caught by the binding")
    monkeypatch.setattr(L, "_stream", no_launch)
    return torch


def cl_host(torch, shape, dtype=None):
    return torch.zeros(shape, dtype=dtype or torch.bfloat16).contiguous(
        memory_format=torch.channels_last_3d)


def test_conv_binding_refuses_mismatched_buffers(host_binding):
    torch = host_binding
    x = cl_host(torch, (1, 16, 2, 8, 12))
    w = cl_host(torch, (32, 16, 3, 3, 3))
    b = torch.zeros(32, dtype=torch.bfloat16)
    cache = cl_host(torch, (1, 16, 2, 8, 12))
    y = cl_host(torch, (1, 32, 2, 8, 12))
    bad = [
        dict(cache_in=cl_host(torch, (1, 16, 2, 4, 12))),          # cache of another resolution
        dict(cache_out=cl_host(torch, (1, 16, 1, 8, 12))),         # one cache frame
        dict(cache_in=cl_host(torch, (1, 16, 2, 8, 12), torch.float32)),  # other dtype
        dict(y=cl_host(torch, (1, 32, 1, 8, 12))),                 # fewer frames
        dict(y=cl_host(torch, (1, 16, 2, 8, 12))),                 # C_in instead of C_out
        dict(residual=cl_host(torch, (1, 32, 2, 8, 11))),
        dict(bias=torch.zeros(16, dtype=torch.bfloat16)),
        dict(packed_weight=torch.zeros(100, dtype=torch.uint8)),   # wrong packed size
    ]
    for kw in bad:
        args = dict(bias=b, cache_in=cache, cache_out=cl_host(torch, (1, 16, 2, 8, 12)), y=y)
        args.update(kw)
        with pytest.raises((ValueError, TypeError)):
            L.wvc_causal_conv3d_fwd(x, w, **args)
    with pytest.raises((ValueError, TypeError)):   # weight C_in != x's channels
        L.wvc_causal_conv3d_fwd(x, cl_host(torch, (32, 8, 3, 3, 3)), y=y)
    # a well-formed call passes every check and stops at the (stubbed) launch
    with pytest.raises(AssertionError, match="reached a launch"):
        L.wvc_causal_conv3d_fwd(x, w, b, cache, cl_host(torch, (1, 16, 2, 8, 12)), y=y)


def test_block_binding_refuses_mismatched_buffers(host_binding):
    torch = host_binding
    c = 32
    x = cl_host(torch, (1, c, 1, 6, 10))
    vec = lambda n: torch.zeros(n, dtype=torch.bfloat16)
    p = {"gamma1": vec(c), "w1": cl_host(torch, (c, c, 3, 3, 3)), "b1": vec(c), "gamma2": vec(c),
         "w2": cl_host(torch, (c, c, 3, 3, 3)), "b2": vec(c)}
    good = lambda: cl_host(torch, (1, c, 2, 6, 10))
    for kw in (dict(cache1_in=cl_host(torch, (1, c, 2, 3, 10))),
               dict(cache2_out=cl_host(torch, (1, c, 2, 6, 5))),
               dict(y=cl_host(torch, (1, c, 2, 6, 10)))):
        args = dict(cache1_in=good(), cache1_out=good(), cache2_in=good(), cache2_out=good())
        args.update(kw)
        with pytest.raises((ValueError, TypeError)):
            L.wvc_resblock_fwd(x, p, **args)
    with pytest.raises((ValueError, TypeError)):
        L.wvc_resblock_fwd(x, dict(p, gamma2=vec(c - 8)))
    with pytest.raises((ValueError, TypeError)):
        L.wvc_resblock_fwd(x, p, packed={"w1": torch.zeros(64, dtype=torch.uint8),
                                         "w2": torch.zeros(64, dtype=torch.uint8)})
    with pytest.raises((ValueError, TypeError)):
        L.wvc_resblock_front(x, p, h2=cl_host(torch, (1, c, 1, 6, 9)))
    with pytest.raises((ValueError, TypeError)):
        L.wvc_resblock_back(x, x, p, cache2_in=cl_host(torch, (1, c, 2, 6, 9)))


def test_block_parameter_check_is_redone_when_the_set_changes(host_binding):
    """A block's parameter set is checked in full once; later calls with the
    same dict only compare its fingerprint, so a tensor swapped into the dict
    (another shape, dtype or layout) is caught on the next call."""
    torch = host_binding
    c = 32
    x = cl_host(torch, (1, c, 1, 6, 10))
    vec = lambda n, dt=torch.bfloat16: torch.zeros(n, dtype=dt)
    p = {"gamma1": vec(c), "w1": cl_host(torch, (c, c, 3, 3, 3)), "b1": vec(c), "gamma2": vec(c),
         "w2": cl_host(torch, (c, c, 3, 3, 3)), "b2": vec(c)}
    for _ in range(2):  # checked in full, then by fingerprint: both reach the launch
        with pytest.raises(AssertionError, match="reached a launch"):
            L.wvc_resblock_fwd(x, p)
    for k, bad in (("w2", cl_host(torch, (c, c // 2, 3, 3, 3))),
                   ("b1", vec(c, torch.float32)),
                   ("w1", torch.zeros((c, c, 3, 3, 3), dtype=torch.bfloat16))):  # not channels-last
        good = p[k]
        p[k] = bad
        with pytest.raises((ValueError, TypeError)):
            L.wvc_resblock_fwd(x, p)
        p[k] = good
    with pytest.raises(AssertionError, match="reached a launch"):
        L.wvc_resblock_fwd(x, p)


def test_conv_norm_binding_refuses_mismatched_buffers(host_binding):
    """wvc_causal_conv3d_norm_fwd: the conv's buffers are checked as for the
    conv call, and gamma, beta and h against C_out and the output shape."""
    torch = host_binding
    x = cl_host(torch, (1, 16, 2, 8, 12))
    w = cl_host(torch, (32, 16, 3, 3, 3))
    g = torch.zeros(32, dtype=torch.bfloat16)
    h_ok = cl_host(torch, (1, 32, 2, 8, 12))
    bad = [
        dict(gamma=torch.zeros(16, dtype=torch.bfloat16)),           # C_in instead of C_out
        dict(beta=torch.zeros(31, dtype=torch.bfloat16)),
        dict(gamma=torch.zeros(32, dtype=torch.float32)),             # other dtype
        dict(h=cl_host(torch, (1, 32, 1, 8, 12))),                    # fewer frames
        dict(h=torch.zeros((1, 32, 2, 8, 12), dtype=torch.bfloat16)),  # not channels-last
        dict(y=cl_host(torch, (1, 16, 2, 8, 12))),                    # C_in instead of C_out
        dict(cache_in=cl_host(torch, (1, 16, 2, 4, 12))),
        dict(residual=cl_host(torch, (1, 32, 2, 8, 11))),
    ]
    for kw in bad:
        args = dict(gamma=g, h=h_ok)
        args.update(kw)
        gamma = args.pop("gamma")
        with pytest.raises((ValueError, TypeError)):
            L.wvc_causal_conv3d_norm_fwd(x, w, gamma, **args)
    with pytest.raises(AssertionError, match="reached a launch"):
        L.wvc_causal_conv3d_norm_fwd(x, w, g, h=h_ok, workspace=torch.zeros(1 << 20, dtype=torch.uint8))


def test_conv_norm_c_abi_argument_errors(lib):
    """The C entry point's own refusals, before anything is enqueued (no GPU):
    a dtype it does not cover, C_out outside its range, eps <= 0, a missing
    gamma or h, and a workspace smaller than its size query."""
    import ctypes
    ok = 1 << 12
    d = L.conv_desc((1, 16, 2, 8, 12), (32, 16, 3, 3, 3), L.WVC_BF16)
    need = L.wvc_causal_conv3d_norm_workspace_bytes(d)
    assert need >= L.wvc_causal_conv3d_workspace_bytes(d)
    p = ctypes.c_void_p
    fake = lambda k: p(ok * k)   # distinct, 4 KiB-aligned, never dereferenced

    def call(desc, gamma=fake(7), eps=1e-12, h=fake(9), ws_bytes=None):
        return lib.wvc_causal_conv3d_norm_fwd(ctypes.byref(desc), fake(1), None, None, fake(3), None,
                                              None, None, gamma, None, ctypes.c_float(eps), h,
                                              fake(100), need if ws_bytes is None else ws_bytes, None)
    d32 = L.conv_desc((1, 16, 2, 8, 12), (32, 16, 3, 3, 3), L.WVC_F32)
    assert call(d32) == L.WVC_ERR_UNSUPPORTED
    d20 = L.conv_desc((1, 16, 2, 8, 12), (20, 16, 3, 3, 3), L.WVC_BF16)
    assert call(d20) == L.WVC_ERR_UNSUPPORTED
    assert call(d, eps=0.0) == L.WVC_ERR_ARG
    assert call(d, gamma=None) == L.WVC_ERR_ARG
    assert call(d, h=None) == L.WVC_ERR_ARG
    assert call(d, ws_bytes=need - 1) == L.WVC_ERR_WORKSPACE


def test_norm_upsample_e4m3_bindings_refuse_mismatched_buffers(host_binding):
    torch = host_binding
    x = cl_host(torch, (1, 32, 2, 6, 10))
    g = torch.zeros(32, dtype=torch.bfloat16)
    with pytest.raises((ValueError, TypeError)):
        L.wvc_rmsnorm_silu(x, g, y=cl_host(torch, (1, 32, 1, 6, 10)))
    with pytest.raises((ValueError, TypeError)):
        L.wvc_rmsnorm_silu(x, torch.zeros(16, dtype=torch.bfloat16))
    with pytest.raises((ValueError, TypeError)):
        L.wvc_rmsnorm_silu_e4m3(x, g, 0.1, q=cl_host(torch, (1, 32, 2, 6, 10)))  # bf16, not codes
    with pytest.raises((ValueError, TypeError)):
        L.wvc_upsample_nearest2x(x, y=cl_host(torch, (1, 32, 2, 12, 10)))
    q = cl_host(torch, (1, 32, 2, 6, 10), torch.uint8)
    wq = cl_host(torch, (32, 32, 3, 3, 3), torch.uint8)
    ws = torch.ones(32)
    with pytest.raises((ValueError, TypeError)):
        L.wvc_causal_conv3d_e4m3_fwd(q, 0.1, wq, ws, cache_in=cl_host(torch, (1, 32, 2, 6, 5), torch.uint8))
    with pytest.raises((ValueError, TypeError)):
        L.wvc_causal_conv3d_e4m3_fwd(q, 0.1, wq, ws, y=cl_host(torch, (1, 32, 2, 6, 10), torch.uint8))


def test_noalloc_scratch_size_and_validation(lib):
    """The allocation-free conv call: its scratch limit as the header states it,
    and argument errors (including a need beyond the scratch) reported before
    the scratch is even looked up (no GPU involved)."""
    text = open(HEADER).read()
    m = re.search(r"#define\s+WVC_NOALLOC_SCRATCH_MIB\s+(\d+)", text)
    assert m and int(m.group(1)) == L.WVC_NOALLOC_SCRATCH_MIB
    L.wvc_reset_counters()
    f = lib.wvc_causal_conv3d_fwd_noalloc
    assert f(None, X, CIN, COUT, W, B, None, Y, None) == L.WVC_ERR_ARG
    assert f(ctypes.byref(desc(groups=2)), X, CIN, COUT, W, B, None, Y, None) == L.WVC_ERR_UNSUPPORTED
    big = desc(x_shape=(1, 384, 2, 60, 104), w_shape=(384, 384, 3, 3, 3))
    assert L.wvc_causal_conv3d_workspace_bytes(big) > L.WVC_NOALLOC_SCRATCH_MIB << 20
    assert f(ctypes.byref(big), X, CIN, COUT, W, B, None, Y, None) == L.WVC_ERR_WORKSPACE
    assert "scratch" in L.wvc_last_error()
    assert L.wvc_get_counters()["fast_3x3x3"] == 0


def test_upsampled_input_validation(lib):
    """upsample_in = 2: the conv reads x and the caches (h/2 x w/2 frames)
    through a nearest 2x upsample, so the conv frame h x w must be even, and
    only the MFMA 3x3x3 route (bf16 or E4M3) reads that way; any other value
    is an argument error."""
    w32 = (32, 16, 3, 3, 3)
    d = desc(x_shape=(1, 16, 2, 8, 12), w_shape=w32)
    d.upsample_in = 2
    assert L.wvc_causal_conv3d_workspace_bytes(d) >= 0
    assert L.wvc_causal_conv3d_norm_workspace_bytes(d) >= 0
    for v in (1, 3, -2):
        d.upsample_in = v
        assert call(lib, d) == L.WVC_ERR_ARG and "upsample_in" in L.wvc_last_error()
    for shape in ((1, 16, 2, 7, 12), (1, 16, 2, 8, 9)):
        odd = desc(x_shape=shape, w_shape=w32)
        odd.upsample_in = 2
        assert call(lib, odd) == L.WVC_ERR_ARG and "even" in L.wvc_last_error()
    L.wvc_reset_counters()
    others = [desc(w_shape=(32, 16, 1, 1, 1), padding=(0, 0)),        # projection route
              desc(w_shape=w32, dtype=L.WVC_F32),                     # direct route
              desc(x_shape=(1, 12, 2, 8, 8), w_shape=(32, 12, 3, 3, 3))]  # C_in % 8 != 0
    for o in others:
        o.upsample_in = 2
        assert call(lib, o) == L.WVC_ERR_UNSUPPORTED and "upsample_in" in L.wvc_last_error()
    assert L.wvc_get_counters()["rejected"] == len(others)
    e8 = desc(w_shape=w32, dtype=L.WVC_E4M3)   # the 8-bit conv reads through it too
    e8.upsample_in = 2
    assert L.wvc_causal_conv3d_workspace_bytes(e8) >= 0
    # x ends at h/2 * w/2 positions per frame: a y 16 bytes before that end
    # overlaps it
    u = desc(x_shape=(1, 16, 2, 8, 8), w_shape=w32)
    u.upsample_in = 2
    need = L.wvc_causal_conv3d_workspace_bytes(u)
    x_bytes = 1 * 16 * 2 * 4 * 4 * 2
    assert call(lib, u, y=X + x_bytes - 16, ws=WS, wsb=need) == L.WVC_ERR_ALIAS
    assert "'y'" in L.wvc_last_error()


def test_upsampled_input_binding_shapes(host_binding):
    """The binding sizes x and the caches at the stored frame and y at twice
    it, and refuses the other sizes before any launch."""
    torch = host_binding
    x = cl_host(torch, (1, 16, 2, 4, 6))
    w = cl_host(torch, (32, 16, 3, 3, 3))
    small = lambda: cl_host(torch, (1, 16, 2, 4, 6))
    y = cl_host(torch, (1, 32, 2, 8, 12))
    bad = [dict(cache_in=cl_host(torch, (1, 16, 2, 8, 12))),   # cache at the upsampled size
           dict(y=cl_host(torch, (1, 32, 2, 4, 6))),             # y at the stored size
           dict(upsample_in=3)]
    for kw in bad:
        args = dict(cache_in=small(), cache_out=small(), y=y, upsample_in=2)
        args.update(kw)
        with pytest.raises((ValueError, TypeError, L.WvcError)):
            L.wvc_causal_conv3d_fwd(x, w, **args)
    with pytest.raises(AssertionError, match="reached a launch"):
        L.wvc_causal_conv3d_fwd(x, w, None, small(), small(), y=y, upsample_in=2)


def test_cu_limit_plans_the_split_for_fewer_cus(lib):
    """cu_limit > 0 plans a small grid's split-K for that many CUs: the
    384-channel 30x52 frame (24 tiles of 128 channels x 256 positions, 36
    K units) splits K 9 ways on 256 CUs (216 workgroups) and 6 ways on 160
    (144 workgroups), which the partial-sum workspace shows; < 0 is refused,
    for the conv and for the block descriptor."""
    def ws(cu):
        d = L.conv_desc((1, 384, 1, 30, 52), (384, 384, 3, 3, 3), L.WVC_BF16,
                        weight_layout=L.WVC_WEIGHT_PACKED, cu_limit=cu)
        return L.wvc_causal_conv3d_workspace_bytes(d)
    part = 1560 * 384 * 4
    align = lambda v: (v + 255) // 256 * 256
    assert ws(0) == align(9 * part) and ws(256) == align(9 * part)
    assert ws(160) == align(6 * part)
    bad = L.conv_desc((1, 384, 1, 30, 52), (384, 384, 3, 3, 3), L.WVC_BF16, cu_limit=-1)
    assert call(lib, bad) == L.WVC_ERR_ARG and "cu_limit" in L.wvc_last_error()
    rd = L.resblock_desc((1, 64, 1, 8, 8), 64, L.WVC_BF16)
    assert L.wvc_resblock_workspace_bytes(rd) > 0
    rd.cu_limit = -1
    assert lib.wvc_resblock_workspace_bytes(ctypes.byref(rd)) == ctypes.c_size_t(-1).value


def test_e4m3_conv_norm_workspace_query():
    """The 8-bit conv + norm call's workspace is the 8-bit conv's plus room
    for y, and the query refuses a bf16 descriptor (no GPU needed)."""
    from video_vae_causal_amd import _lib as L
    d8 = L.conv_desc((1, 384, 1, 30, 52), (384, 384, 3, 3, 3), L.WVC_E4M3,
                     weight_layout=L.WVC_WEIGHT_PACKED)
    conv = L.wvc_causal_conv3d_workspace_bytes(d8)
    y_bytes = 1 * 384 * 1 * 30 * 52 * 2

    def align(v):
        return (v + 255) // 256 * 256
    assert L.wvc_causal_conv3d_e4m3_norm_workspace_bytes(d8) == align(conv) + align(y_bytes)
    dbf = L.conv_desc((1, 384, 1, 30, 52), (384, 384, 3, 3, 3), L.WVC_BF16)
    with pytest.raises(L.WvcError, match="WVC_E4M3"):
        L.wvc_causal_conv3d_e4m3_norm_workspace_bytes(dbf)
