"""The two-stream pipeline with each chunk's two parts replayed as HIP graphs
(stream.PipelineGraph).

The replays make the calls the eager pipeline makes (the eager pipeline in
turn makes the sequential loop's calls), on fixed per-buffer-set input and
output chunks that the host fills and drains with copies; so every
comparison here is bitwise against the sequential chunk loop, which the
stack tests hold to the oracle.  Definitions: "Cosmos3 Wan VAE -- engine size
vs runtime context memory", sections 8.5 (per-layer cache) and 10.4
(residual block).  Every test replays several times with eager work and
synchronisations in between; the bound mode (recordings that read and write
the caller's tensors, no copies) is held to the same comparisons.
"""
import pytest
import torch

from video_vae_causal_amd import _lib as L
from video_vae_causal_amd import inputs, stream
from _gpu_util import check_bf16, to_dev, to_host
from test_gpu_norm_block import block_params_dev, stack_dev

pytestmark = pytest.mark.gpu


def cl(t):
    return t.contiguous(memory_format=torch.channels_last_3d)


def run_passes(stack, pipe, frames, outs, out, seq, what, reps=3, between=None):
    for rep in range(reps):
        out.fill_(float("nan"))
        stack.reset()
        pipe.run(frames, outs)
        torch.cuda.synchronize()
        assert torch.equal(out, seq), f"{what}: replay pass {rep} differs from the sequential loop"
        if between is not None:
            between()
            torch.cuda.synchronize()


@pytest.mark.parametrize("t,slots,bind", [(7, 3, False), (5, 2, False), (2, 3, False), (7, 3, True),
                                          (5, 2, True)])
def test_small_decoder_graph_pipeline_equals_sequential(t, slots, bind):
    d = inputs.decoder_inputs(seed=17, shape=(1, 16, t, 6, 9), width=64)
    pd, lat = stack_dev(d["p"]), to_dev(d["latent"])
    print(f"[case] graph-replayed pipeline, small decoder t={t} slots={slots} bind={bind}", flush=True)
    seq = stream.DecoderStack(pd).run(lat, chunk_frames=1)
    stack = stream.DecoderStack(pd)
    frames = [cl(lat[:, :, i:i + 1]) for i in range(t)]
    out = L.empty_cl(seq.shape)
    outs = [out[:, :, i:i + 1] for i in range(t)]
    pipe = stream.PipelineGraph(stack, frames[0].shape, slots=slots, bind=bind)
    try:
        other_ref = stream.DecoderStack(pd).run(lat, chunk_frames=t)

        def eager_between():      # another stack's eager work between replays
            check_bf16(to_host(stream.DecoderStack(pd).run(lat, chunk_frames=t)), to_host(other_ref),
                       "eager whole-sequence pass between replays")
        run_passes(stack, pipe, frames, outs, out, seq, "small decoder", between=eager_between)
        # an eager chunk first moves the cache parity: the replays continue from it
        if t > 1:
            out.fill_(float("nan"))
            stack.reset()
            stack.chunk(frames[0], out=outs[0])
            pipe.run(frames[1:], outs[1:])
            torch.cuda.synchronize()
            assert torch.equal(out, seq), "replays after an eager chunk differ"
            # and a sequence continued over two run() calls
            out.fill_(float("nan"))
            stack.reset()
            pipe.run(frames[:1], outs[:1])
            pipe.run(frames[1:], outs[1:])
            torch.cuda.synchronize()
            assert torch.equal(out, seq), "a sequence split over two run() calls differs"
        if bind:
            # every (recording, chunk, output) triple met so far has its pair
            # of graphs; a repeated pass records nothing new
            n = len(pipe._bound)
            run_passes(stack, pipe, frames, outs, out, seq, "bound, repeated", reps=1)
            assert len(pipe._bound) == n
    finally:
        torch.cuda.synchronize()
        pipe.close()


@pytest.mark.parametrize("bind", [False, True])
def test_decoder_21_frames_graph_pipeline_equals_sequential(bind):
    """Full-width decoder stack (48-ch latent, 384 ch, 30x52 -> 60x104), 21
    latent frames, the shape the decoder measurement streams."""
    d = inputs.decoder_inputs(seed=5)
    pd, lat = stack_dev(d["p"]), to_dev(d["latent"])
    t = lat.shape[2]
    print(f"[case] graph-replayed pipeline, decoder 21 frames, bind={bind}", flush=True)
    seq = stream.DecoderStack(pd).run(lat, chunk_frames=1)
    stack = stream.DecoderStack(pd)
    frames = [cl(lat[:, :, i:i + 1]) for i in range(t)]
    out = L.empty_cl(seq.shape)
    outs = [out[:, :, i:i + 1] for i in range(t)]
    pipe = stream.PipelineGraph(stack, frames[0].shape, bind=bind)
    try:
        run_passes(stack, pipe, frames, outs, out, seq, "decoder 21 frames", reps=2)
    finally:
        torch.cuda.synchronize()
        pipe.close()


@pytest.mark.parametrize("bind", [False, True])
def test_e4m3_decoder_graph_pipeline_equals_sequential(bind):
    from test_gpu_fp8 import DEC8_SCALES
    d = inputs.decoder_inputs(seed=27, shape=(1, 48, 5, 10, 16), width=128)
    pd, lat = stack_dev(d["p"]), to_dev(d["latent"])
    t = lat.shape[2]
    print("[case] graph-replayed pipeline, 8-bit decoder", flush=True)
    frames = [cl(lat[:, :, i:i + 1]) for i in range(t)]
    ref_stack = stream.DecoderStackE4M3(pd, DEC8_SCALES)
    ref_stack.start(1, 10, 16)
    seq = torch.cat([ref_stack.chunk(f).clone() for f in frames], dim=2)
    stack = stream.DecoderStackE4M3(pd, DEC8_SCALES)
    out = L.empty_cl(seq.shape)
    outs = [out[:, :, i:i + 1] for i in range(t)]
    pipe = stream.PipelineGraph(stack, frames[0].shape, bind=bind)
    try:
        run_passes(stack, pipe, frames, outs, out, seq, "8-bit decoder")
    finally:
        torch.cuda.synchronize()
        pipe.close()


def test_resblock_halves_graph_pipeline_equals_sequential():
    """The 384-channel block at 60x104, five frames, cut between its halves."""
    r = inputs.resblock_inputs(seed=2)
    n, c, t, h, w = r["x"].shape
    x, p = to_dev(r["x"]), block_params_dev(r["p"])
    frames = [cl(x[:, :, i:i + 1]) for i in range(t)]
    print("[case] graph-replayed pipeline, resblock 384 60x104 x5", flush=True)
    rb = stream.ResBlock(p)
    rb.start(n, h, w)
    seq = torch.cat([rb(f) for f in frames], dim=2)
    out = L.empty_cl(x.shape)
    outs = [out[:, :, i:i + 1] for i in range(t)]
    pipe = stream.PipelineGraph(rb, frames[0].shape)
    try:
        run_passes(rb, pipe, frames, outs, out, seq, "resblock halves", reps=2)
    finally:
        torch.cuda.synchronize()
        pipe.close()


def test_graph_pipeline_refuses_to_be_recorded(monkeypatch):
    d = inputs.decoder_inputs(seed=16, shape=(1, 16, 2, 6, 9), width=64)
    stack = stream.DecoderStack(stack_dev(d["p"]))
    lat = to_dev(d["latent"])
    frames = [cl(lat[:, :, i:i + 1]) for i in range(2)]
    out = L.empty_cl((1, 64, 2, 12, 18))
    outs = [out[:, :, i:i + 1] for i in range(2)]
    pipe = stream.PipelineGraph(stack, frames[0].shape)
    torch.cuda.synchronize()
    monkeypatch.setattr(torch.cuda, "is_current_stream_capturing", lambda: True)
    try:
        with pytest.raises(RuntimeError, match="cannot itself be recorded"):
            pipe.run(frames, outs)
    finally:
        monkeypatch.undo()
        pipe.close()


def test_bound_recordings_are_released_oldest_first():
    """With room for 4 bound pairs: passes over two different output tensors
    release each other's recordings and re-record them, every pass bitwise
    the sequential loop; a pass needing more pairs than the limit is refused
    before it records or replays anything."""
    d = inputs.decoder_inputs(seed=18, shape=(1, 16, 3, 6, 9), width=64)
    pd, lat = stack_dev(d["p"]), to_dev(d["latent"])
    t = lat.shape[2]
    print("[case] bound recordings, release and refusal", flush=True)
    seq = stream.DecoderStack(pd).run(lat, chunk_frames=1)
    stack = stream.DecoderStack(pd)
    frames = [cl(lat[:, :, i:i + 1]) for i in range(t)]
    pipe = stream.PipelineGraph(stack, frames[0].shape, bind=True)
    pipe.MAX_BOUND = 4
    try:
        outs_ab = [L.empty_cl(seq.shape) for _ in range(2)]
        for rep in range(4):
            out = outs_ab[rep % 2]
            out.fill_(float("nan"))
            stack.reset()
            pipe.run(frames, [out[:, :, i:i + 1] for i in range(t)])
            torch.cuda.synchronize()
            assert torch.equal(out, seq), f"pass {rep} differs from the sequential loop"
            assert len(pipe._bound) <= 4
        long_lat = to_dev(inputs.decoder_inputs(seed=18, shape=(1, 16, 5, 6, 9), width=64)["latent"])
        long_frames = [cl(long_lat[:, :, i:i + 1]) for i in range(5)]
        long_out = L.empty_cl((1, 64, 5, 12, 18))
        stack.reset()
        with pytest.raises(ValueError, match="exceeds"):
            pipe.run(long_frames, [long_out[:, :, i:i + 1] for i in range(5)])
    finally:
        torch.cuda.synchronize()
        pipe.close()
