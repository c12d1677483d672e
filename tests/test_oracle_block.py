"""Pins for the oracle's residual block and decoder stack (CPU only).

The block and the stack are compositions of pinned parts (conv, norm, SiLU,
upsample).  What is checked here is the composition itself:
  * the block's order (norm -> SiLU -> conv, twice, residual after conv2) against
    an explicit torch fp64 composition of the library routines
    ("Cosmos3 Wan VAE -- engine size vs runtime context memory", section 10.4);
  * streaming frame by frame with per-layer 2-frame caches equals one
    whole-sequence pass, bitwise (same page, section 10.3, causal padding);
  * checkpoint/resume: copying every cache out and back in mid-stream changes
    nothing, bitwise;
  * the bf16-boundary mode rounds exactly the stored tensors.
"""
import numpy as np
import torch
import torch.nn.functional as F

import oracle
from video_vae_causal_amd import inputs

RNG = np.random.default_rng(5)


def _t(a):
    return torch.from_numpy(np.asarray(a, dtype=np.float64))


def torch_block(x, p):
    def norm_silu(v, g):
        C = v.shape[1]
        return F.silu(F.normalize(v, dim=1, eps=1e-12) * C ** 0.5 * g[None, :, None, None, None])

    def conv(v, w, b):
        vp = F.pad(v, (1, 1, 1, 1, 2, 0))
        return F.conv3d(vp, w, b)

    xt = _t(x)
    h1 = norm_silu(xt, _t(p["gamma1"]))
    a1 = conv(h1, _t(p["w1"]), _t(p["b1"]))
    h2 = norm_silu(a1, _t(p["gamma2"]))
    return (conv(h2, _t(p["w2"]), _t(p["b2"])) + xt).numpy()


def small_block(c=8, seed=11):
    p = inputs.resblock_params(c, seed, "rb", "f32")
    return {k: v.astype(np.float64) for k, v in p.items()}


def test_block_matches_torch_composition():
    p = small_block()
    x = RNG.standard_normal((1, 8, 4, 5, 6))
    y, _, _ = oracle.resblock(x, p)
    np.testing.assert_allclose(y, torch_block(x, p), rtol=1e-11, atol=1e-11)


def stream_block(x, p, bf16=False, checkpoint_at=None):
    c1 = c2 = None
    outs = []
    for t in range(x.shape[2]):
        y, c1, c2 = oracle.resblock(x[:, :, t:t + 1], p, c1, c2, bf16=bf16)
        outs.append(y)
        if checkpoint_at == t:
            # move the resumable state out and back (a fresh copy each)
            c1, c2 = np.array(c1, copy=True), np.array(c2, copy=True)
    return np.concatenate(outs, axis=2)


def test_block_streaming_equals_whole_bitwise():
    p = small_block()
    x = RNG.standard_normal((1, 8, 5, 4, 7))
    whole, _, _ = oracle.resblock(x, p)
    np.testing.assert_array_equal(stream_block(x, p), whole)
    np.testing.assert_array_equal(stream_block(x, p, checkpoint_at=2), whole)


def test_block_bf16_mode_streaming_equals_whole_and_rounds_outputs():
    p = small_block()
    x = oracle.round_bf16(RNG.standard_normal((1, 8, 3, 4, 5)))
    whole, c1, c2 = oracle.resblock(x, p, bf16=True)
    np.testing.assert_array_equal(stream_block(x, p, bf16=True), whole)
    np.testing.assert_array_equal(oracle.round_bf16(whole), whole)
    np.testing.assert_array_equal(oracle.round_bf16(c1), c1)
    exact, _, _ = oracle.resblock(x, p)
    assert 0 < oracle.rel_l2(whole, exact) < 1e-2


def small_stack(cl=4, width=8, seed=3):
    d = inputs.decoder_inputs(seed, (1, cl, 4, 3, 5), width=width, dtype="f32")
    p = d["p"]
    p = {k: ({kk: vv.astype(np.float64) for kk, vv in v.items()} if isinstance(v, dict)
             else v.astype(np.float64)) for k, v in p.items()}
    return d["latent"].astype(np.float64), p


def stream_stack(latent, p, bf16=False):
    caches = {}
    outs = []
    r = (lambda a: oracle.round_bf16(a)) if bf16 else (lambda a: a)
    for t in range(latent.shape[2]):
        x = latent[:, :, t:t + 1]
        c = caches.get("in", np.zeros(x.shape[:2] + (2,) + x.shape[3:]))
        h = r(oracle.causal_conv3d(x, p["w_in"], p["b_in"], cache=c))
        caches["in"] = oracle.next_cache(c, x)
        for k in (0, 1):
            h, caches[f"rb{k}a"], caches[f"rb{k}b"] = oracle.resblock(
                h, p[f"rb{k}"], caches.get(f"rb{k}a"), caches.get(f"rb{k}b"), bf16=bf16)
        h = oracle.upsample_nearest2x(h)
        c = caches.get("up", np.zeros(h.shape[:2] + (2,) + h.shape[3:]))
        hn = r(oracle.causal_conv3d(h, p["w_up"], p["b_up"], cache=c))
        caches["up"] = oracle.next_cache(c, h)
        h = hn
        for k in (2, 3):
            h, caches[f"rb{k}a"], caches[f"rb{k}b"] = oracle.resblock(
                h, p[f"rb{k}"], caches.get(f"rb{k}a"), caches.get(f"rb{k}b"), bf16=bf16)
        outs.append(h)
    return np.concatenate(outs, axis=2)


def test_stack_streaming_equals_whole_bitwise():
    latent, p = small_stack()
    whole = oracle.decoder_stack(latent, p)
    assert whole.shape == (1, 8, 4, 6, 10)
    np.testing.assert_array_equal(stream_stack(latent, p), whole)
    latent_b = oracle.round_bf16(latent)
    np.testing.assert_array_equal(stream_stack(latent_b, p, bf16=True),
                                  oracle.decoder_stack(latent_b, p, bf16=True))


def test_stack_layer_order_against_torch():
    latent, p = small_stack()

    def conv(v, w, b):
        return F.conv3d(F.pad(v, (1, 1, 1, 1, 2, 0)), _t(w), _t(b))

    h = conv(_t(latent), p["w_in"], p["b_in"]).numpy()
    h = torch_block(torch_block(h, p["rb0"]), p["rb1"])
    h = F.interpolate(_t(h), scale_factor=(1, 2, 2), mode="nearest")
    h = conv(h, p["w_up"], p["b_up"]).numpy()
    h = torch_block(torch_block(h, p["rb2"]), p["rb3"])
    np.testing.assert_allclose(oracle.decoder_stack(latent, p), h, rtol=1e-10, atol=1e-10)


def test_block_with_projection_shortcut():
    """C_in != C_out: the shortcut is a 1x1x1 causal conv (section 10.4)."""
    cin, cout = 6, 4
    p = {"gamma1": np.ones(cin), "w1": RNG.standard_normal((cout, cin, 3, 3, 3)) * 0.1,
         "b1": np.zeros(cout), "gamma2": np.ones(cout),
         "w2": RNG.standard_normal((cout, cout, 3, 3, 3)) * 0.1, "b2": np.zeros(cout),
         "w_short": RNG.standard_normal((cout, cin, 1, 1, 1)), "b_short": RNG.standard_normal(cout)}
    x = RNG.standard_normal((1, cin, 2, 3, 4))
    y, _, _ = oracle.resblock(x, p)
    sc = np.einsum("oc,ncthw->nothw", p["w_short"][:, :, 0, 0, 0], x) + p["b_short"][None, :, None, None, None]
    q = dict(p)
    del q["w_short"], q["b_short"]
    # main path alone: same block with the shortcut replaced by zero input contribution
    h1 = oracle.silu(oracle.rms_norm(x, p["gamma1"]))
    a1 = oracle.causal_conv3d(h1, p["w1"], p["b1"])
    h2 = oracle.silu(oracle.rms_norm(a1, p["gamma2"]))
    main = oracle.causal_conv3d(h2, p["w2"], p["b2"])
    np.testing.assert_allclose(y, main + sc, rtol=1e-12, atol=1e-12)
