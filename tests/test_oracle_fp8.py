"""Pins for the oracle's 8-bit (E4M3) quantisation and quantised conv (CPU only).

The format is OCP OFP8 E4M3, taken for the quantised Conv3D direction of
"Cosmos3 Wan VAE -- engine size vs runtime context memory" (sections 7 and 9).
Each test checks the oracle against something other than itself:
  * torch's float8_e4m3fn dtype (an independent implementation of the format):
    every code decodes to torch's value, and in-range values encode to torch's
    round-to-nearest-even cast;
  * closed forms of the format (largest finite, smallest subnormal and normal,
    1.0, the NaN code) and hand-worked ties;
  * brute force: a per-row quantised code is the nearest of all 256 codes;
  * the quantised conv equals torch's fp64 conv3d of the dequantised operands,
    with the weight scale on the output-channel axis (a scale applied per
    input channel fails it).
"""
import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle

RNG = np.random.default_rng(808)
ALL = np.arange(256, dtype=np.uint8)


def torch_decode(codes):
    return torch.from_numpy(np.asarray(codes, dtype=np.uint8)).view(torch.float8_e4m3fn).double().numpy()


def torch_encode(values):
    t = torch.from_numpy(np.asarray(values, dtype=np.float32)).to(torch.float8_e4m3fn)
    return t.view(torch.uint8).numpy()


def test_decode_every_code_matches_torch():
    d = oracle.e4m3_decode(ALL)
    t = torch_decode(ALL)
    assert np.array_equal(np.isnan(d), np.isnan(t))
    ok = ~np.isnan(d)
    assert np.array_equal(d[ok], t[ok])
    assert np.array_equal(np.signbit(d[ok]), np.signbit(t[ok]))
    # exactly two NaN codes (0x7F, 0xFF), no infinities
    assert np.flatnonzero(np.isnan(d)).tolist() == [0x7F, 0xFF]
    assert not np.isinf(d).any()


def test_closed_form_values():
    d = oracle.e4m3_decode(np.array([0x7E, 0x01, 0x07, 0x08, 0x38, 0x40, 0xC0, 0x00, 0x80], np.uint8))
    assert d.tolist()[:7] == [448.0, 2.0 ** -9, 7 * 2.0 ** -9, 2.0 ** -6, 1.0, 2.0, -2.0]
    assert d[7] == 0.0 and d[8] == 0.0 and np.signbit(d[8]) and not np.signbit(d[7])
    assert oracle.E4M3_MAX == 448.0


def test_encode_roundtrips_every_code():
    d = oracle.e4m3_decode(ALL)
    ok = ~np.isnan(d)
    assert np.array_equal(oracle.e4m3_encode(d[ok]), ALL[ok])


def test_encode_matches_torch_on_all_bf16_in_range():
    # every bf16 bit pattern with |v| <= 448, as fp32
    bits = np.arange(1 << 16, dtype=np.uint32) << 16
    v = bits.view(np.float32)
    v = v[np.isfinite(v) & (np.abs(v) <= 448.0)]
    assert np.array_equal(oracle.e4m3_encode(v.astype(np.float64)), torch_encode(v))


def test_encode_matches_torch_on_random_fp32():
    v = (RNG.standard_normal(200000) * np.exp(RNG.uniform(-12, 6, 200000))).astype(np.float32)
    v = v[np.abs(v) <= 448.0]
    assert np.array_equal(oracle.e4m3_encode(v.astype(np.float64)), torch_encode(v))


def test_ties_to_even_and_saturation():
    enc = lambda x: int(oracle.e4m3_encode(np.array([x]))[0])
    assert enc(1.0625) == 0x38          # halfway 1.0 / 1.125 -> even mantissa 0
    assert enc(1.1875) == 0x3A          # halfway 1.125 / 1.25 -> 1.25 (m = 2)
    assert enc(2.0 ** -10) == 0x00      # halfway 0 / smallest subnormal -> 0
    assert enc(3 * 2.0 ** -10) == 0x02  # halfway 1 / 2 subnormal steps -> 2
    assert enc(15 * 2.0 ** -10) == 0x08  # halfway 7*2^-9 / 2^-6 -> smallest normal
    assert enc(240.0 + 8.0) == 0x78     # halfway 240 / 256 -> 256 (exponent carry)
    assert enc(-0.0) == 0x80
    for big in (448.0, 449.0, 464.0, 480.0, 1e6, np.inf):
        assert enc(big) == 0x7E and enc(-big) == 0xFE
    assert enc(np.nan) == 0x7F


def test_quantize_rows_nearest_code_brute_force():
    w = RNG.standard_normal((6, 50)) * np.array([1e-3, 0.1, 1.0, 30.0, 1e3, 0.0])[:, None]
    w = w.astype(np.float32)
    codes, scale = oracle.quantize_rows_e4m3(w)
    assert scale.dtype == np.float32 and scale[5] == 1.0 and not (codes[5] & 0x7F).any()  # signed zeros
    table = oracle.e4m3_decode(ALL)
    finite = np.flatnonzero(~np.isnan(table))
    for r in range(5):
        t = w[r].astype(np.float64) * float(np.float32(1.0) / scale[r])
        dist = np.abs(table[finite][None, :] - t[:, None])
        best = dist.min(axis=1)
        got = np.abs(table[codes[r]] - t)
        assert np.array_equal(got, best)
        # the row maximum lands on the largest code
        assert np.max(np.abs(table[codes[r]])) == 448.0
        # dequantised values stay within half a grid step (1/16 relative) of w
        deq = table[codes[r]] * float(scale[r])
        big = np.abs(w[r]) > 2.0 ** -6 * float(scale[r])
        assert np.all(np.abs(deq - w[r])[big] <= np.abs(w[r])[big] / 16 * (1 + 1e-6))


def test_quantize_per_tensor_power_of_two_scale_is_exact_scaling():
    x = RNG.standard_normal(1000).astype(np.float32)
    q1 = oracle.quantize_e4m3(x, 1.0)
    q4 = oracle.quantize_e4m3(x * 4, 4.0)
    assert np.array_equal(q1, q4)
    assert np.array_equal(q1, oracle.e4m3_encode(x.astype(np.float64)))


def _conv_case(cin=8, cout=12, T=3, H=5, W=6, seed=3):
    rng = np.random.default_rng(seed)
    xq = rng.integers(0, 256, (1, cin, T, H, W)).astype(np.uint8)
    cq = rng.integers(0, 256, (1, cin, 2, H, W)).astype(np.uint8)
    wq = rng.integers(0, 256, (cout, cin, 3, 3, 3)).astype(np.uint8)
    for a in (xq, cq, wq):
        a[(a & 0x7F) == 0x7F] = 0x3C  # no NaN codes
    ws = (0.01 + rng.random(cout)).astype(np.float32)
    b = rng.standard_normal(cout)
    r = rng.standard_normal((1, cout, T, H, W))
    return xq, cq, wq, ws, b, r


def test_conv_e4m3_equals_torch_conv_of_dequantised_operands():
    xq, cq, wq, ws, b, r = _conv_case()
    xs = 0.37
    y = oracle.causal_conv3d_e4m3(xq, xs, wq, ws, b, cq, r)
    x = torch_decode(xq) * xs
    c = torch_decode(cq) * xs
    w = torch_decode(wq) * ws.astype(np.float64)[:, None, None, None, None]
    full = torch.from_numpy(np.concatenate([c, x], axis=2))
    ref = F.conv3d(F.pad(full, (1, 1, 1, 1, 0, 0)), torch.from_numpy(w), torch.from_numpy(b)).numpy() + r
    assert np.allclose(y, ref, rtol=1e-12, atol=1e-9)
    # a scale applied along the input-channel axis instead is a different result
    w_wrong = torch_decode(wq) * np.resize(ws, wq.shape[1])[None, :, None, None, None]
    wrong = F.conv3d(F.pad(full, (1, 1, 1, 1, 0, 0)), torch.from_numpy(w_wrong), torch.from_numpy(b)).numpy() + r
    assert not np.allclose(y, wrong, rtol=1e-6, atol=1e-6)


def test_conv_e4m3_without_cache_is_zero_past():
    xq, cq, wq, ws, b, _ = _conv_case(seed=4)
    y0 = oracle.causal_conv3d_e4m3(xq, 1.0, wq, ws, b)
    yz = oracle.causal_conv3d_e4m3(xq, 1.0, wq, ws, b, np.zeros_like(cq))
    assert np.array_equal(y0, yz)


def test_norm_silu_e4m3_is_scaled_norm_silu():
    rng = np.random.default_rng(5)
    x = rng.standard_normal((1, 16, 2, 3, 4))
    g = 1 + 0.1 * rng.standard_normal(16)
    v, codes = oracle.norm_silu_e4m3(x, g, None, scale=0.03125)
    ref = F.silu(torch.from_numpy(F.normalize(torch.from_numpy(x), dim=1).numpy() * 4.0 * g[None, :, None, None, None])).numpy()
    assert np.allclose(v * 0.03125, ref, rtol=1e-12, atol=1e-14)
    assert np.array_equal(codes, oracle.e4m3_encode(v))


def _torch_q(v, s):
    """codes of v / s (torch's float8 cast after explicit saturation), decoded
    back to multiples of s"""
    t = torch.clamp(v / s, -448.0, 448.0).to(torch.float8_e4m3fn)
    return t.double() * s


def _torch_wq(w):
    w = torch.from_numpy(w) if isinstance(w, np.ndarray) else w
    sc = (w.abs().amax(dim=(1, 2, 3, 4)).float() / 448.0).double()
    codes = (w.float() * (1.0 / sc.float())[:, None, None, None, None]).to(torch.float8_e4m3fn)
    return codes.double() * sc[:, None, None, None, None]


def _torch_conv(v, w, b):
    return F.conv3d(F.pad(v, (1, 1, 1, 1, 2, 0)), w, torch.from_numpy(b))


def _torch_block8(x, p, s1, s2):
    c = x.shape[1]

    def norm_silu(v, g):
        u = F.normalize(v, dim=1, eps=1e-12) * np.sqrt(c) * torch.from_numpy(g)[None, :, None, None, None]
        return F.silu(u)

    h = _torch_conv(_torch_q(norm_silu(x, p["gamma1"]), s1), _torch_wq(p["w1"]), p["b1"])
    h = h.to(torch.bfloat16).double()
    y = _torch_conv(_torch_q(norm_silu(h, p["gamma2"]), s2), _torch_wq(p["w2"]), p["b2"]) + x
    return y.to(torch.bfloat16).double()


def _rand_block(rng, c):
    p = {"gamma1": 1 + 0.05 * rng.standard_normal(c), "gamma2": 1 + 0.05 * rng.standard_normal(c),
         "w1": rng.standard_normal((c, c, 3, 3, 3)) / np.sqrt(27 * c),
         "w2": rng.standard_normal((c, c, 3, 3, 3)) / np.sqrt(27 * c),
         "b1": 0.1 * rng.standard_normal(c), "b2": 0.1 * rng.standard_normal(c)}
    return {k: torch.from_numpy(v).to(torch.bfloat16).double().numpy() for k, v in p.items()}


def test_decoder_stack_e4m3_equals_torch_recomposition():
    rng = np.random.default_rng(10)
    cl, c = 8, 16
    lat = torch.from_numpy(rng.standard_normal((1, cl, 2, 3, 4))).to(torch.bfloat16).double()
    bf = lambda a: torch.from_numpy(a).to(torch.bfloat16).double().numpy()
    p = {"w_in": bf(rng.standard_normal((c, cl, 3, 3, 3)) / np.sqrt(27 * cl)), "b_in": bf(0.1 * rng.standard_normal(c)),
         "w_up": bf(rng.standard_normal((c, c, 3, 3, 3)) / np.sqrt(27 * c)), "b_up": bf(0.1 * rng.standard_normal(c))}
    for k in range(4):
        p[f"rb{k}"] = _rand_block(rng, c)
    scales = {"in": 6.0 / 448, "up": 8.0 / 448, "rb": [(6.0 / 448, 5.0 / 448)] * 4}
    y = oracle.decoder_stack_e4m3(lat.numpy(), p, scales)

    def conv8(v, w, b, s):
        # the quantiser multiplies by fl32(1/s) in fp32 (exact for bf16 inputs)
        v32 = (v.float() * (1.0 / torch.tensor(s, dtype=torch.float32))).double()
        q = torch.clamp(v32, -448.0, 448.0).to(torch.float8_e4m3fn).double() * s
        return _torch_conv(q, _torch_wq(w), b).to(torch.bfloat16).double()

    h = conv8(lat, p["w_in"], p["b_in"], scales["in"])
    for k in (0, 1):
        h = _torch_block8(h, p[f"rb{k}"], *scales["rb"][k])
    h = F.interpolate(h, scale_factor=(1, 2, 2), mode="nearest")
    h = conv8(h, p["w_up"], p["b_up"], scales["up"])
    for k in (2, 3):
        h = _torch_block8(h, p[f"rb{k}"], *scales["rb"][k])
    assert y.shape == tuple(h.shape)
    assert oracle.rel_l2(y, h.numpy()) < 2e-3


def test_resblock_e4m3_equals_torch_recomposition():
    # the 8-bit block rebuilt from torch ops: F.normalize-based norm, torch's
    # float8_e4m3fn cast (after explicit saturation), torch conv3d, bf16 casts
    rng = np.random.default_rng(9)
    c, shape = 16, (1, 16, 3, 5, 6)
    x = torch.from_numpy(rng.standard_normal(shape)).to(torch.bfloat16).double()
    p = {"gamma1": 1 + 0.05 * rng.standard_normal(c), "gamma2": 1 + 0.05 * rng.standard_normal(c),
         "w1": rng.standard_normal((c, c, 3, 3, 3)) / np.sqrt(27 * c),
         "w2": rng.standard_normal((c, c, 3, 3, 3)) / np.sqrt(27 * c),
         "b1": 0.1 * rng.standard_normal(c), "b2": 0.1 * rng.standard_normal(c)}
    p = {k: torch.from_numpy(v).to(torch.bfloat16).double().numpy() for k, v in p.items()}
    s1, s2 = 5.0 / 448, 3.0 / 448
    y = oracle.resblock_e4m3(x.numpy(), p, s1, s2)

    def q(v, s):  # codes of v / s, decoded back to multiples of s
        t = torch.clamp(v / s, -448.0, 448.0).to(torch.float8_e4m3fn)
        return t.double() * s

    def wq(w):
        w = torch.from_numpy(w)
        sc = (w.abs().amax(dim=(1, 2, 3, 4)).float() / 448.0).double()
        codes = (w.float() * (1.0 / sc.float())[:, None, None, None, None]).to(torch.float8_e4m3fn)
        return codes.double() * sc[:, None, None, None, None]

    def norm_silu(v, g):
        u = F.normalize(v, dim=1, eps=1e-12) * np.sqrt(c) * torch.from_numpy(g)[None, :, None, None, None]
        return F.silu(u)

    def conv(v, w, b):
        v = F.pad(v, (1, 1, 1, 1, 2, 0))
        return F.conv3d(v, w, torch.from_numpy(b))

    h = conv(q(norm_silu(x, p["gamma1"]), s1), wq(p["w1"]), p["b1"]).to(torch.bfloat16).double()
    ref = (conv(q(norm_silu(h, p["gamma2"]), s2), wq(p["w2"]), p["b2"]) + x).to(torch.bfloat16).double()
    assert np.allclose(y, ref.numpy(), rtol=1e-2, atol=1e-2)
    assert oracle.rel_l2(y, ref.numpy()) < 1e-3
