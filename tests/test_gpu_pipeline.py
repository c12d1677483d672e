"""The residual block in two halves and the two-stream chunk pipeline.

Definitions: "Cosmos3 Wan VAE -- engine size vs runtime context memory",
section 10.4 (residual block) and 8.5 (per-layer cache).  The halves run the
same kernels as the whole-block call, and the pipeline runs the same calls as
the sequential chunk loop, only on two streams with events between them; so
every comparison here is bitwise.  The sequential path is checked against the
oracle in the block and stack tests; one test here checks the pipeline
against the oracle directly.
"""
import pytest
import torch

import oracle
from video_vae_causal_amd import _lib as L
from video_vae_causal_amd import inputs, stream
from _gpu_util import check_bf16, f64, to_dev, to_host
from test_gpu_norm_block import block_params_dev, block_params_f64, stack_dev, stack_f64

pytestmark = pytest.mark.gpu


def cl(t):
    return t.contiguous(memory_format=torch.channels_last_3d)


def block_params(cin, cout, seed, beta):
    """Block parameters with a 1x1x1 shortcut when cin != cout."""
    if cin == cout:
        return inputs.resblock_params(cin, seed, "rb", "bf16", beta)
    g = lambda tag: f"rb.{tag}"
    p = {"gamma1": inputs.norm_gamma(cin, seed, g("g1"), "bf16"),
         "w1": inputs.conv_weight(cout, cin, (3, 3, 3), seed, g("w1"), "bf16"),
         "b1": inputs.conv_bias(cout, seed, g("b1"), "bf16"),
         "gamma2": inputs.norm_gamma(cout, seed, g("g2"), "bf16"),
         "w2": inputs.conv_weight(cout, cout, (3, 3, 3), seed, g("w2"), "bf16"),
         "b2": inputs.conv_bias(cout, seed, g("b2"), "bf16"),
         "w_short": inputs.conv_weight(cout, cin, (1, 1, 1), seed, g("ws"), "bf16"),
         "b_short": inputs.conv_bias(cout, seed, g("bs"), "bf16")}
    if beta:
        p["beta1"] = inputs.norm_beta(cin, seed, g("be1"), "bf16")
        p["beta2"] = inputs.norm_beta(cout, seed, g("be2"), "bf16")
    return p


@pytest.mark.parametrize("cin,cout,t,h,w,beta", [(64, 64, 3, 9, 13, True), (48, 96, 2, 7, 11, False),
                                                  (384, 384, 1, 60, 104, False)])
def test_front_then_back_equals_whole_block_bitwise(cin, cout, t, h, w, beta):
    xh = inputs.quantize(inputs.normal((1, cin, t, h, w), 41, "x"), "bf16")
    x = to_dev(xh)
    p = block_params_dev(block_params(cin, cout, 41, beta))
    print(f"[case] block halves {cin}->{cout} t={t} {h}x{w}", flush=True)
    c1 = [L.empty_cl((1, cin, 2, h, w)) for _ in range(2)]
    c2 = [L.empty_cl((1, cout, 2, h, w)) for _ in range(2)]
    for c in c1 + c2:
        L.wvc_cache_reset(c)
    y_whole = L.wvc_resblock_fwd(x, p, c1[0], c1[1], c2[0], c2[1])
    c1b = [L.empty_cl((1, cin, 2, h, w)) for _ in range(2)]
    c2b = [L.empty_cl((1, cout, 2, h, w)) for _ in range(2)]
    for c in c1b + c2b:
        L.wvc_cache_reset(c)
    h2 = L.wvc_resblock_front(x, p, c1b[0], c1b[1])
    y_split = L.wvc_resblock_back(h2, x, p, c2b[0], c2b[1])
    assert torch.equal(y_whole, y_split)
    assert torch.equal(c1[1], c1b[1]) and torch.equal(c2[1], c2b[1])
    if h * w < 1000:
        pf = block_params_f64(block_params(cin, cout, 41, beta))
        ref, _, _ = oracle.resblock(f64(xh), pf, bf16=True)
        check_bf16(to_host(y_split), ref, f"block halves {cin}->{cout}")


def test_pipelined_resblock_five_frames_equals_sequential():
    """The default bench workload: C = 384 at 60x104, five latent frames one
    at a time, sequential vs two-stream pipeline, twice each."""
    r = inputs.resblock_inputs(seed=2)
    n, c, t, h, w = r["x"].shape
    x, p = to_dev(r["x"]), block_params_dev(r["p"])
    frames = [cl(x[:, :, i:i + 1]) for i in range(t)]
    print("[case] pipelined resblock 384 60x104 x5", flush=True)
    rb = stream.ResBlock(p)
    rb.start(n, h, w)
    seq = torch.cat([rb(f) for f in frames], dim=2)
    out = L.empty_cl(x.shape)
    outs = [out[:, :, i:i + 1] for i in range(t)]
    pipe = stream.Pipeline(rb)
    for rep in range(2):
        out.fill_(float("nan"))
        rb.reset()
        pipe.run(frames, outs)
        torch.cuda.synchronize()
        assert torch.equal(out, seq), f"pass {rep}: pipeline differs from the sequential frames"


def test_pipelined_small_decoder_vs_oracle():
    d = inputs.decoder_inputs(seed=15, shape=(1, 16, 4, 6, 9), width=64)
    stack = stream.DecoderStack(stack_dev(d["p"]))
    lat = to_dev(d["latent"])
    stack.start(1, 6, 9)
    out = L.empty_cl((1, 64, 4, 12, 18))
    stream.Pipeline(stack).run([cl(lat[:, :, i:i + 1]) for i in range(4)],
                               [out[:, :, i:i + 1] for i in range(4)])
    torch.cuda.synchronize()
    ref = oracle.decoder_stack(f64(d["latent"]), stack_f64(d["p"]), bf16=True)
    check_bf16(to_host(out), ref, "decoder stack small, pipelined")
    assert torch.equal(out, stream.DecoderStack(stack_dev(d["p"])).run(lat, chunk_frames=1))


def test_pipelined_decoder_21_frames_equals_sequential():
    """Full-width decoder stack (48-ch latent, 384 ch, 30x52 -> 60x104), 21
    latent frames: the pipelined pass equals the sequential one, twice."""
    d = inputs.decoder_inputs(seed=5)
    pd, lat = stack_dev(d["p"]), to_dev(d["latent"])
    t = lat.shape[2]
    print("[case] pipelined decoder 21 frames", flush=True)
    seq = stream.DecoderStack(pd).run(lat, chunk_frames=1)
    stack = stream.DecoderStack(pd)
    stack.start(1, 30, 52)
    frames = [cl(lat[:, :, i:i + 1]) for i in range(t)]
    out = L.empty_cl(seq.shape)
    outs = [out[:, :, i:i + 1] for i in range(t)]
    pipe = stream.Pipeline(stack)
    for rep in range(2):
        out.fill_(float("nan"))
        stack.reset()
        pipe.run(frames, outs)
        torch.cuda.synchronize()
        assert torch.equal(out, seq), f"pass {rep}: pipeline differs from the sequential frames"


@pytest.mark.skip(reason="ending a HIP stream capture that recorded the two-stream fork/join "
                         "crashed the host process (segmentation fault inside hipStreamEndCapture), "
                         "also with fork and join events that outlive the capture; the cause is not "
                         "known, so Pipeline.run raises under capture and this case stays off the GPU")
def test_pipelined_decoder_recorded_into_a_graph_equals_sequential():
    """The two-stream pipeline recorded into one HIP graph: its fork and join
    use events that outlive the capture (no temporary events are destroyed
    while they are recorded into it).  Every replay, with eager work and
    synchronisations in between, equals the sequential chunk loop bitwise."""
    d = inputs.decoder_inputs(seed=16, shape=(1, 16, 4, 6, 9), width=64)
    pd, lat = stack_dev(d["p"]), to_dev(d["latent"])
    t = lat.shape[2]
    seq = stream.DecoderStack(pd).run(lat, chunk_frames=1)
    stack = stream.DecoderStack(pd)
    stack.start(1, 6, 9)
    frames = [cl(lat[:, :, i:i + 1]) for i in range(t)]
    out = L.empty_cl(seq.shape)
    outs = [out[:, :, i:i + 1] for i in range(t)]
    pipe = stream.Pipeline(stack)
    pipe.run(frames, outs)              # eager pass: sizes every buffer set
    torch.cuda.synchronize()
    assert torch.equal(out, seq)
    stack.reset()                       # the recording starts a fresh sequence
    print("[case] pipeline recorded into a graph", flush=True)
    graph = stream.capture(lambda: pipe.run(frames, outs))
    try:
        for rep in range(3):
            out.fill_(float("nan"))
            graph.launch()
            torch.cuda.synchronize()
            assert torch.equal(out, seq), f"replay {rep} differs from the sequential loop"
            other = stream.DecoderStack(pd).run(lat, chunk_frames=2)   # eager work in between
            torch.cuda.synchronize()
            check_bf16(to_host(other), to_host(seq), "eager 2-frame chunks between replays")
    finally:
        torch.cuda.synchronize()
        graph.close()


def test_pipeline_refuses_to_be_recorded(monkeypatch):
    """Until the capture crash above is understood, a pipelined pass refuses
    to run on a capturing stream, before it enqueues anything (the capture
    state is simulated here: no capture is started)."""
    d = inputs.decoder_inputs(seed=16, shape=(1, 16, 2, 6, 9), width=64)
    stack = stream.DecoderStack(stack_dev(d["p"]))
    lat = to_dev(d["latent"])
    stack.start(1, 6, 9)
    out = L.empty_cl((1, 64, 2, 12, 18))
    frames = [cl(lat[:, :, i:i + 1]) for i in range(2)]
    outs = [out[:, :, i:i + 1] for i in range(2)]
    pipe = stream.Pipeline(stack)
    torch.cuda.synchronize()
    monkeypatch.setattr(torch.cuda, "is_current_stream_capturing", lambda: True)
    with pytest.raises(RuntimeError, match="cannot be recorded"):
        pipe.run(frames, outs)
