"""Pins the FLOP/byte accounting against the pages' worked numbers
(tests/golden/page_accounting.json, each entry cited there)."""
import json
import os

from video_vae_causal_amd import accounting as acc

GOLDEN = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "page_accounting.json")))


def close_to_printed(value, printed, digits=2):
    # "approx" figures are printed to 2 significant digits
    from math import floor, log10
    scale = 10 ** (floor(log10(abs(printed))) - digits + 1)
    return abs(value - printed) <= scale


def test_l0_conv_gemm_dims_and_bytes():
    g = GOLDEN["l0_conv_gemm"]
    n, c, t, h, w = g["shape"]
    m, k, nn = acc.conv_gemm_dims(n, t, h, w, c, g["c_out"], tuple(g["k"]))
    assert close_to_printed(m, g["M_approx"]) and close_to_printed(k, g["K_approx"]) and nn == g["N"]
    assert close_to_printed(acc.tensor_bytes(g["shape"]), g["feature_map_bytes_approx"])
    assert close_to_printed(acc.tensor_bytes((96, 96, 3, 3, 3)), g["weight_bytes_approx"], digits=1)
    flops = acc.conv_flops(n, t, h, w, c, g["c_out"])
    assert flops == 2 * m * k * nn
    # the printed total is 10x below the product of the printed factors
    assert close_to_printed(flops / 10, g["printed_flops"])


def test_encode_io_volumes():
    g = GOLDEN["encode_io"]
    assert close_to_printed(acc.tensor_bytes(g["video_shape"]) / 1e6, g["video_bytes_approx_MB"])
    assert close_to_printed(acc.tensor_bytes(g["latent_shape"]) / 1e6, g["latent_bytes_approx_MB"], digits=1)


def test_latent_frame_rule():
    for frames, latent in GOLDEN["latent_frames"]["pairs"]:
        assert acc.latent_frames(frames) == latent


def test_workload_flops():
    # 384-channel 3x3x3 conv at 240x416 x 17 frames and per 60x104 frame
    assert acc.conv_flops(1, 17, 240, 416, 384, 384) == 13_514_802_462_720
    assert acc.conv_flops(1, 1, 60, 104, 384, 384) == 49_686_773_760
    assert acc.conv_flops(1, 17, 480, 832, 96, 96) == 3_378_700_615_680


def test_conv_launch_bytes():
    # 384-channel 60x104 frame with its 2 cached frames: 3 input frames, the
    # 384x384x27 weights and bias, 1 output frame, 2 cache-out frames
    plane = 60 * 104 * 384 * 2
    wb = 384 * 384 * 27 * 2 + 384 * 2
    assert acc.conv_launch_bytes(1, 1, 60, 104, 384, 384) == 3 * plane + wb + plane
    assert acc.conv_launch_bytes(1, 1, 60, 104, 384, 384, cache_out_frames=2) == 5 * plane + wb + plane
    assert acc.conv_launch_bytes(1, 1, 60, 104, 384, 384, residual=True) == 3 * plane + wb + 2 * plane
    # the whole 17-frame sequence from zero padding: no cache read
    p4 = 240 * 416 * 384 * 2
    assert acc.conv_launch_bytes(1, 17, 240, 416, 384, 384, cache_frames=0, cache_out_frames=2) == \
        17 * p4 + wb + 17 * p4 + 2 * p4
