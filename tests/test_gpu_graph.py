"""HIP-graph replay of the streamed path (wvc_graph_* through the C ABI).

The Cosmos3 page ("Cosmos3 Wan VAE -- engine size vs runtime context
memory") counts its decoder's launches per iteration in section 8.5 and lists
graph capture against their overhead in section 8.7.  A replay runs the
launches of the recorded library calls on the buffers they named, so every
replay must equal the eager run bitwise; the eager path itself is checked
against the oracle elsewhere, and one test here checks a replayed stack
against the oracle directly.  Each test replays several times with eager work
and synchronisations between the replays and checks every replay.
"""
import pytest
import torch

import oracle
from video_vae_causal_amd import _lib as L
from video_vae_causal_amd import inputs, stream
from _gpu_util import check_bf16, f64, to_dev, to_host
from test_gpu_norm_block import block_params_dev, stack_dev, stack_f64

pytestmark = pytest.mark.gpu


def cl(t):
    return t.contiguous(memory_format=torch.channels_last_3d)


def test_resblock_step_graph_replays_equal_eager():
    """The default bench step: one C=384 residual block, five 60x104 latent
    frames fed one at a time from reset caches, recorded as one graph."""
    r = inputs.resblock_inputs(seed=2)
    n, c, t, h, w = r["x"].shape
    x = to_dev(r["x"])
    frames = [cl(x[:, :, i:i + 1]) for i in range(t)]
    out = L.empty_cl(x.shape)
    outs = [out[:, :, i:i + 1] for i in range(t)]
    rb = stream.ResBlock(block_params_dev(r["p"]))
    rb.start(n, h, w)

    def step():
        rb.reset()
        for i in range(t):
            rb(frames[i], y=outs[i])

    print("[case] resblock 384 60x104 step graph", flush=True)
    step()
    torch.cuda.synchronize()
    ref = out.clone()
    g = stream.capture(step)
    for k in range(3):
        out.fill_(float("nan"))
        g.launch()
        torch.cuda.synchronize()
        assert torch.equal(out, ref), f"replay {k} differs from the eager step"
        step()                          # eager work between replays
        torch.cuda.synchronize()
        assert torch.equal(out, ref)
    g.close()


def run_frame_graph(fg, lat, eager_frames=()):
    """Stream lat frame by frame through fg; frames listed in eager_frames run
    eagerly on the same stack instead of replaying."""
    fg.reset()
    outs = []
    for i in range(lat.shape[2]):
        xi = cl(lat[:, :, i:i + 1])
        if i in eager_frames:
            outs.append(fg.stack.chunk(xi).clone())
            fg.parity ^= 1              # an eager chunk flips the caches like a replay
        else:
            fg.x.copy_(xi)
            outs.append(fg().clone())
        torch.cuda.synchronize()
    return torch.cat(outs, dim=2)


def test_frame_graph_small_decoder_vs_oracle_and_eager():
    d = inputs.decoder_inputs(seed=15, shape=(1, 16, 3, 6, 9), width=64)
    pd, lat = stack_dev(d["p"]), to_dev(d["latent"])
    eager = stream.DecoderStack(pd).run(lat, chunk_frames=1)
    fg = stream.FrameGraph(stream.DecoderStack(pd), (1, 16, 1, 6, 9))
    for seq in range(2):
        got = run_frame_graph(fg, lat)
        assert torch.equal(got, eager), f"sequence {seq}: graph replay differs from eager"
    ref = oracle.decoder_stack(f64(d["latent"]), stack_f64(d["p"]), bf16=True)
    check_bf16(to_host(got), ref, "decoder stack small, graph replay")
    fg.close()


def test_frame_graph_decoder_21_frames_equals_eager_with_interleaved_eager_chunks():
    """The decoder-shaped stack at full width (48-ch latent, 384 ch, 30x52 ->
    60x104), 21 latent frames: replayed per frame, then again with some
    frames run eagerly in between (the stack's ping-pong state must follow
    the replays)."""
    d = inputs.decoder_inputs(seed=5)
    pd, lat = stack_dev(d["p"]), to_dev(d["latent"])
    print("[case] decoder stack 21 frames, frame graphs", flush=True)
    eager = stream.DecoderStack(pd).run(lat, chunk_frames=1)
    fg = stream.FrameGraph(stream.DecoderStack(pd), (1, 48, 1, 30, 52))
    assert torch.equal(run_frame_graph(fg, lat), eager)
    assert torch.equal(run_frame_graph(fg, lat, eager_frames=(0, 5, 6, 20)), eager)
    fg.close()


def test_frame_graph_single_conv_layer_with_checkpoint():
    """One cached 3x3x3 conv layer replayed per frame; the caches saved after
    two replayed frames resume a fresh stream bitwise."""
    x = inputs.quantize(inputs.normal((1, 64, 4, 9, 13), 31, "x"), "bf16")
    wt = inputs.conv_weight(64, 64, (3, 3, 3), 31, "w", "bf16")
    b = inputs.conv_bias(64, 31, "b", "bf16")
    xd = to_dev(x)
    conv = stream.CausalConv3d(to_dev(wt), to_dev(b))
    eager = stream.run_chunked(conv, xd, [1, 1, 1, 1])
    ref = oracle.causal_conv3d(f64(x), f64(wt), f64(b))
    check_bf16(to_host(eager), ref, "conv 64ch eager")

    fg = stream.FrameGraph(stream.CausalConv3d(to_dev(wt), to_dev(b)), (1, 64, 1, 9, 13))
    fg.reset()
    outs = []
    for i in range(2):
        fg.x.copy_(cl(xd[:, :, i:i + 1]))
        outs.append(fg().clone())
    saved = stream.Stream([fg.stack]).state()
    fg.reset()                                   # a fresh sequence ...
    stream.Stream([fg.stack]).load_state(saved)  # ... resumed from the checkpoint
    fg.parity = fg.stack.cache.cur               # the replay parity follows the restored state
    for i in range(2, 4):
        fg.x.copy_(cl(xd[:, :, i:i + 1]))
        outs.append(fg().clone())
    torch.cuda.synchronize()
    assert torch.equal(torch.cat(outs, dim=2), eager)
    fg.close()
