"""GPU tests of the conv followed by the next layer's RMS norm + SiLU in one
library call (wvc_causal_conv3d_norm_fwd), and of the decoder stack composed
from such calls.

Definitions: "Cosmos3 Wan VAE -- engine size vs runtime context memory",
sections 10.3 (causal conv, residual block) and 10.2 / 10.4 (RMS norm, SiLU).
The call must store exactly what the conv call followed by the norm call
stores (bitwise; on split-K plans the reduce runs inside the norm kernel),
and the oracle bounds it like any conv + norm pair.
"""
import numpy as np
import pytest
import torch

import oracle
from video_vae_causal_amd import _lib as L
from video_vae_causal_amd import inputs, stream
from _gpu_util import check_bf16, f64, to_dev, to_host

pytestmark = pytest.mark.gpu


def _case(cin, cout, t, h, w, seed):
    x = inputs.quantize(inputs.normal((1, cin, t, h, w), seed, "x"), "bf16")
    cache = inputs.quantize(inputs.normal((1, cin, 2, h, w), seed, "cache"), "bf16")
    wt = inputs.conv_weight(cout, cin, (3, 3, 3), seed, "w", "bf16")
    b = inputs.conv_bias(cout, seed, "b", "bf16")
    res = inputs.quantize(inputs.normal((1, cout, t, h, w), seed, "res"), "bf16")
    g = inputs.norm_gamma(cout, seed, "g", "bf16")
    bt = inputs.norm_beta(cout, seed, "bt", "bf16")
    return x, cache, wt, b, res, g, bt


# 384 channels at 60x104 and 30x52 split K (one frame); 3 frames at 60x104 and
# 96 channels do not; 48 -> 384 is the decoder's conv_in
@pytest.mark.parametrize("cin,cout,t,h,w", [(384, 384, 1, 60, 104), (384, 384, 1, 30, 52),
                                            (384, 384, 3, 60, 104), (96, 96, 2, 9, 17),
                                            (48, 384, 1, 30, 52)])
@pytest.mark.parametrize("with_res,with_y,with_beta", [(True, True, True), (False, False, False),
                                                       (True, False, True)])
def test_conv_norm_equals_conv_then_norm_bitwise(cin, cout, t, h, w, with_res, with_y, with_beta):
    x, cache, wt, b, res, g, bt = _case(cin, cout, t, h, w, seed=cin + cout + t + h)
    xd, cd, wd, bd, rd, gd = to_dev(x), to_dev(cache), to_dev(wt), to_dev(b), to_dev(res), to_dev(g)
    btd = to_dev(bt) if with_beta else None
    rdv = rd if with_res else None
    packed = L.wvc_conv3d_pack_weights(wd)
    print(f"[case] conv+norm {cin}->{cout} t={t} {h}x{w} res={with_res} y={with_y} beta={with_beta} "
          f"kernel {L.wvc_conv3d_kernel_name(L.conv_desc(tuple(xd.shape), tuple(wd.shape), L.WVC_BF16))}",
          flush=True)
    co_a, co_b = L.empty_cl((1, cin, 2, h, w)), L.empty_cl((1, cin, 2, h, w))
    y_sep = L.wvc_causal_conv3d_fwd(xd, wd, bd, cd, co_a, residual=rdv, packed_weight=packed)
    h_sep = L.wvc_rmsnorm_silu(y_sep, gd, btd)
    y_f = L.empty_cl(tuple(y_sep.shape)) if with_y else None
    h_f = L.wvc_causal_conv3d_norm_fwd(xd, wd, gd, bd, btd, cache_in=cd, cache_out=co_b, residual=rdv,
                                       y=y_f, packed_weight=packed)
    torch.cuda.synchronize()
    assert torch.equal(h_f, h_sep)
    if with_y:
        assert torch.equal(y_f, y_sep)
    assert torch.equal(co_a, co_b)


def test_conv_norm_vs_oracle():
    """One split-K case against the oracle's conv, rounded to bf16 where the
    library stores y, then its norm + SiLU."""
    x, cache, wt, b, res, g, bt = _case(384, 384, 1, 30, 52, seed=77)
    h = L.wvc_causal_conv3d_norm_fwd(to_dev(x), to_dev(wt), to_dev(g), to_dev(b), to_dev(bt),
                                     cache_in=to_dev(cache), residual=to_dev(res))
    y_ref = oracle.round_bf16(oracle.causal_conv3d(f64(x), f64(wt), f64(b), cache=f64(cache)) + f64(res))
    ref = oracle.silu(oracle.rms_norm(y_ref, f64(g), f64(bt)))
    check_bf16(to_host(h), ref, "conv + norm 384 30x52 vs oracle")


def test_conv_norm_rejects_what_it_does_not_cover():
    x = to_dev(inputs.quantize(inputs.normal((1, 32, 1, 8, 8), 3, "x"), "bf16"))
    w = to_dev(inputs.conv_weight(20, 32, (3, 3, 3), 3, "w", "bf16"))   # C_out % 8 != 0
    g = to_dev(inputs.norm_gamma(20, 3, "g", "bf16"))
    with pytest.raises(L.WvcError):
        L.wvc_causal_conv3d_norm_fwd(x, w, g)
    torch.cuda.synchronize()


def _stack(d):
    return {k: ({kk: to_dev(vv) for kk, vv in v.items()} if isinstance(v, dict) else to_dev(v))
            for k, v in d["p"].items()}


@pytest.mark.parametrize("shape,width", [((1, 16, 4, 6, 9), 64), ((1, 48, 3, 30, 52), 384)])
def test_decoder_stack_fused_equals_layerwise_bitwise(shape, width):
    """The decoder stack composed from conv + norm calls against the same
    stack layer by layer (each block's own norm1, separate split-K reduces),
    frame by frame through the caches: every output frame bitwise equal."""
    d = inputs.decoder_inputs(seed=19, shape=shape, width=width)
    pd = _stack(d)
    lat = to_dev(d["latent"])
    print(f"[case] decoder stack fused vs layerwise {shape} width {width}", flush=True)
    fused = stream.DecoderStack(pd)
    layer = stream.DecoderStack(pd)
    layer._fusable = lambda: False
    assert fused._fusable()
    y_f = fused.run(lat, chunk_frames=1)
    y_l = layer.run(lat, chunk_frames=1)
    torch.cuda.synchronize()
    assert torch.equal(y_f, y_l)


def test_conv_norm_empty_chunk_only_rolls_the_cache():
    """A chunk of no frames: nothing to convolve or normalise, and cache_out
    is cache_in (the last two frames of cache || empty chunk)."""
    c, h, w = 64, 10, 14
    cache = to_dev(inputs.quantize(inputs.normal((1, c, 2, h, w), 5, "cache"), "bf16"))
    x = L.empty_cl((1, c, 0, h, w))
    wt = to_dev(inputs.conv_weight(c, c, (3, 3, 3), 5, "w", "bf16"))
    g = to_dev(inputs.norm_gamma(c, 5, "g", "bf16"))
    cout = L.empty_cl((1, c, 2, h, w))
    cout.fill_(float("nan"))
    print("[case] conv+norm empty chunk", flush=True)
    hh = L.wvc_causal_conv3d_norm_fwd(x, wt, g, cache_in=cache, cache_out=cout)
    torch.cuda.synchronize()
    assert tuple(hh.shape) == (1, c, 0, h, w)
    assert torch.equal(cout, cache)
