"""GPU parity of the fused RMS norm + SiLU, the upsample, the residual block
and the decoder-shaped stack against the oracle, through the C ABI.

Definitions: "Cosmos3 Wan VAE -- engine size vs runtime context memory",
sections 10.2 (RMS norm), 10.4 (SiLU, residual block), 10.3 and 8.5 (cache).
Single ops are compared with the pure fp64 oracle; blocks and stacks with the
oracle that rounds to bf16 where the GPU stores a tensor (the distance to the
pure fp64 chain is printed as well).
"""
import numpy as np
import pytest
import torch

import oracle
from video_vae_causal_amd import _lib as L
from video_vae_causal_amd import inputs, stream
from _gpu_util import check_bf16, check_f32, f64, to_dev, to_host

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("c", [384, 96, 48, 16, 24, 20, 8, 1152])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("beta,silu", [(False, True), (True, True), (True, False)])
def test_rmsnorm_silu_vs_oracle(c, dtype, beta, silu):
    shape = (2, c, 3, 7, 11)
    x = inputs.quantize(inputs.normal(shape, c, "x", std=2.0), dtype)
    g = inputs.norm_gamma(c, c, "g", dtype)
    bt = inputs.norm_beta(c, c, "b", dtype) if beta else None
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    y = L.wvc_rmsnorm_silu(to_dev(x, tdt), to_dev(g, tdt), None if bt is None else to_dev(bt, tdt),
                           apply_silu=silu)
    ref = oracle.rms_norm(f64(x), f64(g), None if bt is None else f64(bt))
    if silu:
        ref = oracle.silu(ref)
    if dtype == "bf16":
        check_bf16(to_host(y), ref, f"norm c={c}")
    else:
        check_f32(to_host(y), ref, f"norm c={c}")


@pytest.mark.parametrize("c,h,w,dtype", [(16, 1031, 1019, "bf16"), (96, 420, 421, "bf16"),
                                         (384, 211, 211, "bf16"), (1152, 121, 123, "bf16"),
                                         (96, 297, 297, "f32")])
def test_rmsnorm_silu_large_vs_oracle(c, h, w, dtype):
    """Tensors of over two million 16-byte chunks (the launch for large
    tensors: two chunks per thread, non-temporal accesses) whose position
    count leaves a ragged last workgroup."""
    shape = (1, c, 1, h, w)
    x = inputs.quantize(inputs.normal(shape, c + 7, "x", std=1.5), dtype)
    g = inputs.norm_gamma(c, c + 7, "g", dtype)
    bt = inputs.norm_beta(c, c + 7, "b", dtype)
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    print(f"[case] norm large c={c} {h}x{w} {dtype}", flush=True)
    y = L.wvc_rmsnorm_silu(to_dev(x, tdt), to_dev(g, tdt), to_dev(bt, tdt))
    ref = oracle.silu(oracle.rms_norm(f64(x), f64(g), f64(bt)))
    if dtype == "bf16":
        check_bf16(to_host(y), ref, f"norm large c={c}")
    else:
        check_f32(to_host(y), ref, f"norm large c={c}")


def test_rmsnorm_zero_vector_gives_beta():
    c = 96
    x = torch.zeros((1, c, 1, 2, 3), dtype=torch.bfloat16, device="cuda").contiguous(
        memory_format=torch.channels_last_3d)
    g = to_dev(inputs.norm_gamma(c, 1, "g", "bf16"))
    b = inputs.norm_beta(c, 1, "b", "bf16")
    y = L.wvc_rmsnorm_silu(x, g, to_dev(b), apply_silu=False)
    np.testing.assert_array_equal(to_host(y), np.broadcast_to(f64(b)[None, :, None, None, None], y.shape))


@pytest.mark.parametrize("c", [384, 20])
def test_upsample_nearest2x(c):
    x = inputs.quantize(inputs.normal((1, c, 2, 5, 7), 2, "x"), "bf16")
    y = L.wvc_upsample_nearest2x(to_dev(x))
    np.testing.assert_array_equal(to_host(y), oracle.upsample_nearest2x(f64(x)))


def block_params_dev(p):
    return {k: to_dev(v) for k, v in p.items()}


def block_params_f64(p):
    return {k: f64(v) for k, v in p.items()}


def run_block_stream(x_dev, pd, sizes):
    rb = stream.ResBlock(pd)
    return stream.run_chunked(rb, x_dev, sizes), rb


@pytest.mark.parametrize("c,t,h,w,beta", [(64, 3, 10, 12, False), (96, 2, 9, 17, True)])
def test_resblock_small_vs_oracle(c, t, h, w, beta):
    r = inputs.resblock_inputs(seed=c + h, shape=(1, c, t, h, w), with_beta=beta)
    y, _ = run_block_stream(to_dev(r["x"]), block_params_dev(r["p"]), [1] * t)
    ref, _, _ = oracle.resblock(f64(r["x"]), block_params_f64(r["p"]), bf16=True)
    check_bf16(to_host(y), ref, f"resblock c={c}")


def test_resblock_projection_shortcut():
    cin, cout = 48, 64
    x = inputs.quantize(inputs.normal((1, cin, 2, 6, 9), 5, "x"), "bf16")
    p = {"gamma1": inputs.norm_gamma(cin, 5, "g1", "bf16"),
         "w1": inputs.conv_weight(cout, cin, (3, 3, 3), 5, "w1", "bf16"),
         "b1": inputs.conv_bias(cout, 5, "b1", "bf16"),
         "gamma2": inputs.norm_gamma(cout, 5, "g2", "bf16"),
         "w2": inputs.conv_weight(cout, cout, (3, 3, 3), 5, "w2", "bf16"),
         "b2": inputs.conv_bias(cout, 5, "b2", "bf16"),
         "w_short": inputs.conv_weight(cout, cin, (1, 1, 1), 5, "ws", "bf16"),
         "b_short": inputs.conv_bias(cout, 5, "bs", "bf16")}
    y, _ = run_block_stream(to_dev(x), block_params_dev(p), [1, 1])
    ref, _, _ = oracle.resblock(f64(x), block_params_f64(p), bf16=True)
    check_bf16(to_host(y), ref, "resblock 48->64 with 1x1x1 shortcut")


def test_resblock_384_60x104_five_frames_one_at_a_time():
    """Wan-style block, C=384, 5 latent frames of 60x104 fed one frame at a
    time with the 2-frame caches, bf16 in/out, fp32 accumulation."""
    r = inputs.resblock_inputs(seed=2)
    print("[case] resblock 384 60x104 T=5 streamed", flush=True)
    xd = to_dev(r["x"])
    y, _ = run_block_stream(xd, block_params_dev(r["p"]), [1] * 5)
    yh = to_host(y)
    ref, _, _ = oracle.resblock(f64(r["x"]), block_params_f64(r["p"]), bf16=True)
    check_bf16(yh, ref, "resblock 384 (bf16-boundary oracle)")
    exact, _, _ = oracle.resblock(f64(r["x"]), block_params_f64(r["p"]), bf16=False)
    print(f"[parity] resblock 384 distance to pure fp64 chain: rel_l2={oracle.rel_l2(yh, exact):.3e}",
          flush=True)
    # whole sequence at once agrees with the frame-by-frame stream (the two
    # launch shapes may split K differently, so the bar is the parity bar)
    yw, _ = run_block_stream(xd, block_params_dev(r["p"]), [5])
    check_bf16(to_host(yw), yh, "resblock 384 whole vs streamed")


def test_resblock_mixed_chunk_lengths_share_one_workspace():
    """Chunks of different lengths through one block (one workspace): at 384
    channels and 30x52 a 4-frame chunk runs unsplit while a 1-frame chunk
    splits K, so the split-K scratch and the chunk-length-dependent
    intermediates share the workspace in different proportions from call to
    call.  Regression test for a workspace layout that let them collide."""
    r = inputs.resblock_inputs(seed=31, shape=(1, 384, 8, 30, 52))
    xd = to_dev(r["x"])
    ref, _, _ = oracle.resblock(f64(r["x"]), block_params_f64(r["p"]), bf16=True)
    for sizes in ([4, 1, 2, 1], [1, 4, 1, 2], [1, 1, 4, 2]):
        y, _ = run_block_stream(xd, block_params_dev(r["p"]), sizes)
        check_bf16(to_host(y), ref, f"resblock 384 30x52 chunks {sizes}")


def test_resblock_packed_and_standard_weights_agree_bitwise():
    r = inputs.resblock_inputs(seed=41, shape=(1, 96, 2, 9, 17))
    xd, pd = to_dev(r["x"]), block_params_dev(r["p"])
    packed = {k: L.wvc_conv3d_pack_weights(pd[k]) for k in ("w1", "w2")}
    y_std = L.wvc_resblock_fwd(xd, pd)
    y_pk = L.wvc_resblock_fwd(xd, pd, packed=packed)
    assert torch.equal(y_std, y_pk)


@pytest.mark.parametrize("c,t,h,w", [(384, 1, 60, 104), (384, 1, 30, 52), (96, 2, 9, 17),
                                     (384, 3, 60, 104)])
def test_resblock_equals_its_abi_composition_bitwise(c, t, h, w):
    """wvc_resblock_fwd against the same block spelled out as single ABI calls
    (norm, conv with cache, norm, conv with residual).  On split-K frames the
    block fuses conv1's partial-sum reduction into norm2; that must give the
    very bits the separate reduce + norm give."""
    r = inputs.resblock_inputs(seed=c + h + t, shape=(1, c, t, h, w))
    xd, pd = to_dev(r["x"]), block_params_dev(r["p"])
    n = 1
    caches = [L.empty_cl((n, c, 2, h, w)) for _ in range(4)]
    for cc in caches:
        L.wvc_cache_reset(cc)
    print(f"[case] resblock composition c={c} t={t} {h}x{w}", flush=True)
    y_blk = L.wvc_resblock_fwd(xd, pd, caches[0], caches[1], caches[2], caches[3])
    h1 = L.wvc_rmsnorm_silu(xd, pd["gamma1"])
    c1o, c2o = L.empty_cl((n, c, 2, h, w)), L.empty_cl((n, c, 2, h, w))
    a1 = L.wvc_causal_conv3d_fwd(h1, pd["w1"], pd["b1"], caches[0], c1o)
    h2 = L.wvc_rmsnorm_silu(a1, pd["gamma2"])
    y_sep = L.wvc_causal_conv3d_fwd(h2, pd["w2"], pd["b2"], caches[2], c2o, residual=xd)
    assert torch.equal(y_blk, y_sep)
    assert torch.equal(caches[1], c1o) and torch.equal(caches[3], c2o)


def test_resblock_checkpoint_resume_bitwise():
    r = inputs.resblock_inputs(seed=9, shape=(1, 64, 4, 8, 12))
    xd, pd = to_dev(r["x"]), block_params_dev(r["p"])
    full, _ = run_block_stream(xd, pd, [1, 1, 1, 1])
    rb = stream.ResBlock(pd)
    rb.start(1, 8, 12)
    s = stream.Stream([rb])
    outs = [rb(xd[:, :, t:t + 1].contiguous(memory_format=torch.channels_last_3d)) for t in range(2)]
    saved = s.state()
    rb.start(1, 8, 12)                # a fresh stream ...
    s.load_state(saved)              # ... resumed from the checkpoint
    outs += [rb(xd[:, :, t:t + 1].contiguous(memory_format=torch.channels_last_3d)) for t in (2, 3)]
    assert torch.equal(torch.cat(outs, dim=2), full)


def stack_dev(p):
    return {k: (block_params_dev(v) if isinstance(v, dict) else to_dev(v)) for k, v in p.items()}


def stack_f64(p):
    return {k: (block_params_f64(v) if isinstance(v, dict) else f64(v)) for k, v in p.items()}


def test_decoder_stack_small_vs_oracle():
    d = inputs.decoder_inputs(seed=15, shape=(1, 16, 3, 6, 9), width=64)
    out = stream.DecoderStack(stack_dev(d["p"])).run(to_dev(d["latent"]), chunk_frames=1)
    ref = oracle.decoder_stack(f64(d["latent"]), stack_f64(d["p"]), bf16=True)
    check_bf16(to_host(out), ref, "decoder stack small")


def test_decoder_stack_checkpoint_resume_bitwise():
    """The decoder stack's whole resumable state is its ten caches (conv_up's
    at the frame size before the upsample it reads through): a stack resumed
    from a checkpoint taken after frame 2 continues bitwise as the
    uninterrupted stream ("Cosmos3 Wan VAE", section 8.5: the cache carries
    the past frames from chunk to chunk)."""
    d = inputs.decoder_inputs(seed=16, shape=(1, 16, 5, 6, 9), width=64)
    pd, lat = stack_dev(d["p"]), to_dev(d["latent"])
    n, _, t, h, w = lat.shape
    frames = [lat[:, :, i:i + 1].contiguous(memory_format=torch.channels_last_3d) for i in range(t)]
    print("[case] decoder stack checkpoint after frame 2, resume", flush=True)
    whole = stream.DecoderStack(pd)
    whole.start(n, h, w)
    full = [whole.chunk(f).clone() for f in frames]
    first = stream.DecoderStack(pd)
    first.start(n, h, w)
    for f in frames[:3]:
        first.chunk(f)
    saved = first.state()
    assert len(saved) == 10
    assert tuple(first.conv_up.caches()[0].shape[3:]) == (h, w)
    resumed = stream.DecoderStack(pd)
    resumed.start(n, h, w)
    resumed.load_state(saved)
    for f, ref in zip(frames[3:], full[3:]):
        assert torch.equal(resumed.chunk(f), ref)


@pytest.mark.timeout(900)
def test_decoder_stack_full_21_frames_vs_oracle():
    """The decoder-shaped stack at its real widths (48-ch latent, 384 ch, 30x52
    -> 60x104), all 21 latent frames streamed one frame at a time, every
    output against the oracle's stack (bf16 at the points where the GPU stores
    a tensor).  Frames 2-20 are the steady state in which both cached frames
    of all ten convs are real frames; 81 video frames compress to these 21
    latent frames ("diffusion inference workload anatomy", two-compressions
    paragraph), and streaming them must equal the whole sequence ("Cosmos3 Wan
    VAE", section 10.3)."""
    d = inputs.decoder_inputs(seed=5)
    print("[case] decoder stack 48->384 30x52 T=21 vs oracle", flush=True)
    out = stream.DecoderStack(stack_dev(d["p"])).run(to_dev(d["latent"]), chunk_frames=1)
    got = to_host(out)
    ref = oracle.decoder_stack(f64(d["latent"]), stack_f64(d["p"]), bf16=True)
    check_bf16(got, ref, "decoder stack 384, all 21 frames")
    check_bf16(got[:, :, :2], ref[:, :, :2], "decoder stack 384, frames 0-1")
    check_bf16(got[:, :, 2:], ref[:, :, 2:], "decoder stack 384, frames 2-20")
    check_bf16(got[:, :, 20:], ref[:, :, 20:], "decoder stack 384, frame 20")
    ref64 = oracle.decoder_stack(f64(d["latent"][:, :, :3]), stack_f64(d["p"]), bf16=False)
    print(f"[parity] decoder stack frames 0-2, distance from the pure fp64 chain: "
          f"{oracle.rel_l2(got[:, :, :3], ref64):.3e}", flush=True)


def test_decoder_stack_21_frames_chunking_invariant():
    """All 21 latent frames: frame-by-frame streaming, 4-frame chunks and one
    whole-sequence pass agree (parity bar: chunk lengths may change the split-K
    grouping), and two runs of the same chunking are bitwise equal."""
    d = inputs.decoder_inputs(seed=5)
    pd = stack_dev(d["p"])
    lat = to_dev(d["latent"])
    print("[case] decoder stack T=21 chunk invariance", flush=True)
    a = stream.DecoderStack(pd).run(lat, chunk_frames=1)
    b = stream.DecoderStack(pd).run(lat, chunk_frames=4)
    c = stream.DecoderStack(pd).run(lat, chunk_frames=21)
    a2 = stream.DecoderStack(pd).run(lat, chunk_frames=1)
    assert torch.equal(a, a2)
    assert torch.isfinite(a.float()).all()
    check_bf16(to_host(b), to_host(a), "decoder 4-frame chunks vs frame by frame")
    check_bf16(to_host(c), to_host(a), "decoder whole vs frame by frame")


def test_layers_restart_when_the_frame_size_changes():
    """A layer called on a chunk of another batch or frame size starts a new
    sequence (fresh caches of the new size) instead of writing full-size cache
    frames into the old buffers: its output equals a fresh layer's, bitwise."""
    r = inputs.resblock_inputs(seed=44, shape=(1, 64, 2, 12, 20))
    pd = block_params_dev(r["p"])
    small = to_dev(inputs.resblock_inputs(seed=45, shape=(1, 64, 2, 6, 10))["x"])
    big = to_dev(r["x"])
    for make, call in ((lambda: stream.ResBlock(pd), lambda l, x: l(x)),
                       (lambda: stream.CausalConv3d(pd["w1"], pd["b1"]), lambda l, x: l(x))):
        layer = make()
        call(layer, big)                  # caches sized 12x20 ...
        got = call(layer, small)          # ... then a 6x10 chunk, no start()
        want = call(make(), small)
        assert torch.equal(got, want)
