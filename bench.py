"""Benchmark of the causal video-VAE hot path on one MI355X.

python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--no-cpu-baseline]

A step is one pass of the whole hot path over one batch of synthetic input:

  layer_384_240x416 (default): causal conv 3x3x3 384->384 over
      x[1,384,17,240,416] (whole sequence, writing the 2-frame cache a next
      chunk would read), then the 1x1x1 384->192 projection.  The default
      line also carries, measured in the same run: the decoder-shaped stack
      streamed one latent frame at a time (ms per decoded latent frame), and
      the fused RMS norm + SiLU over the 96-channel 17x480x832 map (GB/s and
      its fraction of HBM bandwidth).
  resblock_384_60x104: the Wan residual block, C=384, 60x104, 5
      latent frames fed one frame at a time through the 2-frame caches (caches
      reset at the start of each step): per frame RMSNorm+SiLU -> causal conv
      3x3x3 -> RMSNorm+SiLU -> causal conv 3x3x3 + residual, plus the cache
      updates.
  resblock_384_60x104_e4m3: the default workload on the 8-bit path: the
      norms store E4M3 codes, both convs run on codes (weights with one scale
      per output channel), outputs and residual bf16.
  layer_384_240x416_e4m3: the same layer with the 3x3x3 conv on 8-bit E4M3
      codes (activations with one scale, weights with one scale per output
      channel; fp32 accumulation, bf16 output), the projection in bf16.
  layer_96_480x832: RMSNorm+SiLU then causal conv 3x3x3 96->96 over
      x[1,96,17,480,832] in chunks 1+4+4+4+4 with the cache.
  decoder_stack_48_30x52: latent[1,48,21,30,52] -> conv_in -> 2 resblocks ->
      up 2x -> conv -> 2 resblocks, streamed one latent frame at a time.

Prints one JSON line.  ``value`` is the conv throughput of the whole step
(conv FLOPs counted as 2*M*K*N over all taps, divided by the step time) in
TFLOP/s; ``ms_per_latent_frame`` is the step time per latent frame.  The
``roofline`` object covers the dominant kernel (the 3x3x3 conv, or the norm
where stated), timed live with HIP events on the stream it runs on; the
``cpu_baseline`` object times the fp64 CPU oracle on a bounded sample (with
all host threads and with one), and compares the GPU's output of the timed
step with the oracle's on that sample (``parity``).
Inputs are seeded synthetic tensors already resident in HBM when timing starts.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

MFMA_BF16_PEAK_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
MFMA_FP8_PEAK_TFLOPS = 5000.0    # MI355X dense fp8 MFMA
HBM_PEAK_GBS = 8000.0            # MI355X HBM3E
METRIC = "causal Conv3D bf16 TFLOP/s (% MFMA peak) + ms per decoded latent frame"


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="layer_384_240x416",
                    choices=sorted(["resblock_384_60x104", "layer_384_240x416", "layer_96_480x832",
                                    "layer_384_240x416_e4m3", "resblock_384_60x104_e4m3",
                                    "decoder_stack_48_30x52_e4m3",
                                    "decoder_stack_48_30x52", "downsample_96_480x832",
                                    "decoder_tiled_192x336"]))
    ap.add_argument("--tiling", choices=sorted(TILINGS), default="page",
                    help="decoder_tiled_192x336: the page's (60,104)/(30,52) tiles, a reduced "
                         "overlap (stride (52,96)), or no tiling")
    ap.add_argument("--fuse-norm", choices=("on", "off"), default="on",
                    help="downsample_96_480x832: compute the first RMS norm + SiLU inside the "
                         "stride-2 conv (on) or as its own kernel (off)")
    ap.add_argument("--kernel-timing", choices=("graph", "eager"), default="graph",
                    help="time the dominant kernel from a replayed HIP graph of its launches, or "
                         "from eager launches (for profiler runs that collect counters)")
    ap.add_argument("--kernel-reps", type=int, default=50,
                    help="launches of the dominant kernel timed for the roofline")
    ap.add_argument("--warmup-seconds", type=float, default=0.5,
                    help="keep warming up (untimed) until this much wall time has passed "
                         "after the --warmup steps")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extras", action="store_true",
                    help="layer_384_240x416: leave out the decoder-stack and norm measurements "
                         "the default line carries")
    ap.add_argument("--pipeline", choices=("auto", "on", "off"), default="auto",
                    help="streamed workloads: split each frame's layers over two streams so that "
                         "the second part of frame i runs next to the first part of frame i+1 "
                         "(auto: on for the decoder stack, where it is faster; off for the single "
                         "residual block, where it is not)")
    ap.add_argument("--graph", choices=("auto", "on", "off"), default="auto",
                    help="replay recorded HIP graphs instead of enqueuing the launches one by one: "
                         "the whole step as one graph (after the eager warm-up), or with the "
                         "two-stream pipeline each frame's two parts as graphs (auto: on for the "
                         "8-bit decoder stack, whose eager launches the host cannot issue as fast "
                         "as the GPU runs them; off elsewhere)")
    ap.add_argument("--traffic-json", default=os.path.join(ROOT, "profiles", "traffic.json"),
                    help="measured HBM bytes per launch (from rocprofv3 --pmc), if present")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run 5 plain device copies of MIB MiB (bf16) and exit: the known-size "
                         "kernel that scales rocprofv3's FETCH_SIZE / WRITE_SIZE counters")
    ap.add_argument("--operands", choices=("random", "zero"), default="random",
                    help="zero: layer_384_240x416 and layer_96_480x832 only, with all-zero input and weights -- a diagnostic "
                         "that keeps every instruction, address and wait of the conv and removes the "
                         "operands' bit toggling, to separate the chip's clock response from the "
                         "schedule; its numbers are not the metric")
    ap.add_argument("--library-gemm", default="", metavar="M,N,K",
                    help="only time the vendor library's dense GEMM of this shape (bf16 through "
                         "torch.matmul in both operand orders, E4M3 through torch._scaled_mm) on "
                         "operands already laid out as matrices, print one JSON line and exit")
    return ap.parse_args()


PIPELINE = False  # set from --pipeline in main()
PIPE_GRAPH = False  # --pipeline on with --graph on: each chunk's two parts replayed as graphs
OPERANDS = "random"  # set from --operands in main()
PIPELINED = ("resblock_384_60x104", "decoder_stack_48_30x52", "decoder_stack_48_30x52_e4m3")
PIPELINE_AUTO = ("decoder_stack_48_30x52", "decoder_stack_48_30x52_e4m3")  # where it measured faster
GRAPH_AUTO = ("decoder_stack_48_30x52_e4m3",)  # where graph replay measured faster


def make_pipe(stack, chunk_shape):
    """The two-stream pipeline over ``stack``: eager launches, or with
    PIPE_GRAPH each chunk's two parts replayed as recorded graphs, bound to
    the step's own chunk and output tensors (no copies)."""
    from video_vae_causal_amd import stream
    if PIPE_GRAPH:
        return stream.PipelineGraph(stack, tuple(chunk_shape), bind=True)
    return stream.Pipeline(stack)


def cl(t):
    import torch
    return t.contiguous(memory_format=torch.channels_last_3d)


def to_dev(a, dtype=None):
    import torch
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to("cuda")
    t = t.to(dtype or torch.bfloat16)
    return cl(t) if t.dim() == 5 else t


def steady_cache(shape, name, e4m3_scale=None):
    """A 2-frame cache of past activations (seeded normals, like the kernel's
    input chunk): the state a streamed conv sees from its third chunk on.  A
    zeroed cache (the first chunk) feeds the MFMAs zeros on two of the three
    temporal taps, which draws less power, so the chip holds a higher clock
    and the launch runs faster than in the steady state."""
    import torch
    from video_vae_causal_amd import _lib as L, inputs
    v = to_dev(inputs.quantize(inputs.normal(tuple(shape), 6, name), "bf16"))
    if e4m3_scale is None:
        return v
    q = L.empty_cl(tuple(shape), torch.uint8)
    L.wvc_quantize_e4m3(v, e4m3_scale, q=q)
    return q


def conv_workspace(x, w, padding=(1, 1), packed=False):
    """Conv workspace allocated once, outside any timed region."""
    import torch
    from video_vae_causal_amd import _lib as L
    d = L.conv_desc(tuple(x.shape), tuple(w.shape), L.WVC_BF16, padding=padding,
                    weight_layout=L.WVC_WEIGHT_PACKED if packed else L.WVC_WEIGHT_STANDARD)
    need = L.wvc_causal_conv3d_workspace_bytes(d)
    return torch.empty(need, dtype=torch.uint8, device="cuda") if need else None


def conv_kernel_name(x, w, padding=(1, 1)):
    """The kernel the library launches for a conv of x by w (packed weights)."""
    from video_vae_causal_amd import _lib as L
    return L.wvc_conv3d_kernel_name(L.conv_desc(tuple(x.shape), tuple(w.shape), L.WVC_BF16,
                                                padding=padding, weight_layout=L.WVC_WEIGHT_PACKED))


def time_region(fn, steps, warmup, warmup_s=0.0):
    """Warm up (``warmup`` calls, and more until ``warmup_s`` seconds have
    passed: the GPU clock takes ~0.1 s of load to reach its steady state), then
    time exactly ``steps`` calls between two events on the current stream,
    synchronised on both sides.  Returns (ms per call, wall s)."""
    import torch
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    w0 = time.perf_counter()
    k = 0
    while time.perf_counter() - w0 < warmup_s:
        fn()
        k += 1
        if k % 8 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    w0 = time.perf_counter()
    start.record()
    for _ in range(steps):
        fn()
    end.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - w0
    return start.elapsed_time(end) / steps, wall


def kernel_ms(fn, reps, warmup_s, use_graph=True):
    """Average duration of one launch of ``fn``'s kernels, with HIP events on
    the current stream around replays of a HIP graph that records ``reps``
    calls of ``fn`` back to back: replays carry no host launch overhead, which
    for a kernel of a few tens of microseconds can exceed the kernel itself.
    Falls back to timing eager calls if the calls cannot be recorded."""
    import torch
    from video_vae_causal_amd import stream
    if not use_graph:
        ms, _ = time_region(fn, reps, 3, warmup_s)
        return ms, "eager launches"
    try:
        fn()
        torch.cuda.synchronize()
        graph = stream.capture(lambda: [fn() for _ in range(reps)])
    except Exception as e:  # noqa: BLE001 -- report and time eagerly instead
        ms, _ = time_region(fn, reps, 3, warmup_s)
        return ms, f"eager launches ({type(e).__name__} while recording)"
    try:
        ms, _ = time_region(graph.launch, 5, 2, warmup_s)
    finally:
        torch.cuda.synchronize()
        graph.close()
    return ms / reps, f"HIP graph of {reps} launches, replayed 5 times"


# ---------------------------------------------------------------------------
# Workloads: each returns (step_fn, info) where info describes FLOPs, frames,
# the dominant kernel and how to time it alone.
# ---------------------------------------------------------------------------

def wl_resblock():
    import torch
    from video_vae_causal_amd import _lib as L, accounting as acc, inputs, stream
    r = inputs.resblock_inputs(seed=2)
    n, c, t, h, w = r["x"].shape
    x = to_dev(r["x"])
    p = {k: to_dev(v) for k, v in r["p"].items()}
    frames = [cl(x[:, :, i:i + 1]) for i in range(t)]
    out = L.empty_cl(x.shape)
    outs = [out[:, :, i:i + 1] for i in range(t)]
    rb = stream.ResBlock(p)
    rb.start(n, h, w)

    pipe = make_pipe(rb, frames[0].shape) if PIPELINE else None

    def step():
        rb.reset()
        if pipe is not None:
            pipe.run(frames, outs)
        else:
            for i in range(t):
                rb(frames[i], y=outs[i])

    conv_flops = 2 * t * acc.conv_flops(n, 1, h, w, c, c)
    # dominant kernel alone: the 3x3x3 conv of one 60x104 frame with its cache
    # in and out, as the block's convs run
    cache = steady_cache((n, c, 2, h, w), "kernel_cache")
    cache_o = L.empty_cl((n, c, 2, h, w))
    ky = L.empty_cl((n, c, 1, h, w))
    kws = conv_workspace(frames[0], p["w1"], packed=True)
    w1p = L.wvc_conv3d_pack_weights(p["w1"])

    def kernel():
        L.wvc_causal_conv3d_fwd(frames[0], p["w1"], p["b1"], cache, cache_o, None, ky, workspace=kws,
                                packed_weight=w1p)

    info = dict(workload="resblock_384_60x104", conv_flops=conv_flops, latent_frames=t,
                config={"workload": "resblock_384_60x104", "channels": c, "frames": t,
                        "height": h, "width": w, "chunk_frames": 1, "cache_frames": 2,
                        "batch": n},
                kernel=kernel, kernel_name=conv_kernel_name(frames[0], p["w1"]),
                kernel_units=acc.conv_flops(n, 1, h, w, c, c), kernel_bound="mfma",
                kernel_bytes=acc.conv_launch_bytes(n, 1, h, w, c, c, cache_out_frames=2))
    return step, info


def wl_resblock_e4m3():
    import torch
    from video_vae_causal_amd import _lib as L, accounting as acc, inputs, stream
    r = inputs.resblock_inputs(seed=2)
    n, c, t, h, w = r["x"].shape
    x = to_dev(r["x"])
    p = {k: to_dev(v) for k, v in r["p"].items()}
    frames = [cl(x[:, :, i:i + 1]) for i in range(t)]
    out = L.empty_cl(x.shape)
    outs = [out[:, :, i:i + 1] for i in range(t)]
    # activation scales: a fixed calibration for these synthetic activations
    # (SiLU of unit-RMS values stays below 5)
    rb = stream.ResBlockE4M3(p, 5.0 / 448, 5.0 / 448)
    rb.start(n, h, w)

    def step():
        rb.reset()
        for i in range(t):
            rb(frames[i], y=outs[i])

    conv_flops = 2 * t * acc.conv_flops(n, 1, h, w, c, c)
    qx = L.empty_cl((n, c, 1, h, w), torch.uint8)
    L.wvc_quantize_e4m3(frames[0], 5.0 / 448, q=qx)
    cache = steady_cache((n, c, 2, h, w), "kernel_cache", 5.0 / 448)
    ky = L.empty_cl((n, c, 1, h, w))
    wq, wsc, wqp = rb.w["w1"]
    d8 = L.conv_desc(tuple(qx.shape), tuple(wq.shape), L.WVC_E4M3, weight_layout=L.WVC_WEIGHT_PACKED)
    need = L.wvc_causal_conv3d_workspace_bytes(d8)
    kws = torch.empty(need, dtype=torch.uint8, device="cuda") if need else None

    def kernel():
        L.wvc_causal_conv3d_e4m3_fwd(qx, 5.0 / 448, wq, wsc, p["b1"], cache, None, None, ky,
                                     workspace=kws, packed_weight=wqp)

    info = dict(workload="resblock_384_60x104_e4m3", conv_flops=conv_flops, latent_frames=t,
                config={"workload": "resblock_384_60x104_e4m3", "channels": c, "frames": t,
                        "height": h, "width": w, "chunk_frames": 1, "cache_frames": 2,
                        "batch": n, "conv_operands": "e4m3", "activation_scales": [5.0 / 448] * 2},
                kernel=kernel,
                kernel_name="igemm_kernel<3, 128, 32, 2, true, 16, true> + splitk_reduce_kernel",
                kernel_units=acc.conv_flops(n, 1, h, w, c, c), kernel_bound="mfma",
                kernel_peak=MFMA_FP8_PEAK_TFLOPS,
                kernel_bytes=n * h * w * c * 3 + c * c * 27 + c * 6 + n * h * w * c * 2,
                dtype="e4m3 x e4m3 -> f32 (convs); norms, residual and outputs bf16")
    return step, info


def wl_layer384():
    import torch
    from video_vae_causal_amd import _lib as L, accounting as acc, inputs
    d = inputs.layer384_inputs()
    n, c, t, h, w = d["x"].shape
    x, wt, b = to_dev(d["x"]), to_dev(d["w"]), to_dev(d["b"])
    wp, bp = to_dev(d["wp"]), to_dev(d["bp"])
    y = L.empty_cl((n, c, t, h, w))
    proj = L.empty_cl((n, wp.shape[0], t, h, w))
    # the cache a following chunk would read: the last 2 input frames, written
    # by the conv's own staging pass
    cache_out = L.empty_cl((n, c, 2, h, w))

    ws3 = conv_workspace(x, wt, packed=True)
    ws1 = conv_workspace(y, wp, padding=(0, 0), packed=True)
    if OPERANDS == "zero":
        for a in (x, wt, b, wp, bp):
            a.zero_()
    wtp = L.wvc_conv3d_pack_weights(wt)
    wpp = L.wvc_conv3d_pack_weights(wp, padding=(0, 0))

    def kernel():
        L.wvc_causal_conv3d_fwd(x, wt, b, cache_out=cache_out, y=y, workspace=ws3, packed_weight=wtp)

    def step():
        kernel()
        L.wvc_causal_conv3d_fwd(y, wp, bp, y=proj, padding=(0, 0), workspace=ws1, packed_weight=wpp)

    f3 = acc.conv_flops(n, t, h, w, c, c)
    f1 = acc.conv_flops(n, t, h, w, c, wp.shape[0], (1, 1, 1))
    kname = L.wvc_conv3d_kernel_name(L.conv_desc(tuple(x.shape), tuple(wt.shape), L.WVC_BF16,
                                                 weight_layout=L.WVC_WEIGHT_PACKED))

    def gpu_outputs():
        """The timed step's outputs, for the oracle comparison of the CPU leg."""
        return {"y": y, "proj": proj}

    info = dict(workload="layer_384_240x416", conv_flops=f3 + f1, latent_frames=t,
                config={"workload": "layer_384_240x416", "channels": c, "frames": t,
                        "height": h, "width": w, "chunk_frames": t, "projection_out": int(wp.shape[0]),
                        "batch": n, "cache_out": True,
                        **({"operands": "zero (diagnostic)"} if OPERANDS == "zero" else {})},
                kernel=kernel, kernel_name=kname, kernel_units=f3, kernel_reps=10,
                kernel_bound="mfma",
                kernel_bytes=acc.conv_launch_bytes(n, t, h, w, c, c, cache_frames=0, cache_out_frames=2),
                host=d, gpu_outputs=gpu_outputs)
    return step, info


def wl_layer384_e4m3():
    import torch
    from video_vae_causal_amd import _lib as L, accounting as acc, inputs
    shape = (1, 384, 17, 240, 416)
    n, c, t, h, w = shape
    d = inputs.e4m3_conv_inputs(seed=7, shape=shape, cout=c, with_cache=False)
    x = cl(torch.from_numpy(d["x"]).to("cuda"))
    wq = cl(torch.from_numpy(d["w"]).to("cuda"))
    ws = torch.from_numpy(d["w_scale"]).to("cuda")
    b = to_dev(d["b"])
    wp = to_dev(inputs.conv_weight(192, c, (1, 1, 1), 7, "wp", "bf16"))
    bp = to_dev(inputs.conv_bias(192, 7, "bp", "bf16"))
    y = L.empty_cl((n, c, t, h, w))
    proj = L.empty_cl((n, 192, t, h, w))
    d8 = L.conv_desc(shape, tuple(wq.shape), L.WVC_E4M3, weight_layout=L.WVC_WEIGHT_PACKED)
    need = L.wvc_causal_conv3d_workspace_bytes(d8)
    ws3 = torch.empty(need, dtype=torch.uint8, device="cuda") if need else None
    ws1 = conv_workspace(y, wp, padding=(0, 0), packed=True)
    wqp = L.wvc_conv3d_pack_weights(wq)
    wpp = L.wvc_conv3d_pack_weights(wp, padding=(0, 0))
    # the norm that writes these codes in a block, timed on a bf16 activation
    # of the same shape
    xn = to_dev(inputs.quantize(inputs.normal(shape, 7, "xn"), "bf16"))
    gn = to_dev(inputs.norm_gamma(c, 7, "gn", "bf16"))
    qn = L.empty_cl(shape, torch.uint8)
    del d

    def conv():
        L.wvc_causal_conv3d_e4m3_fwd(x, 2.0 ** -6, wq, ws, b, y=y, workspace=ws3, packed_weight=wqp)

    def step():
        conv()
        L.wvc_causal_conv3d_fwd(y, wp, bp, y=proj, padding=(0, 0), workspace=ws1, packed_weight=wpp)

    def norm_kernel():
        L.wvc_rmsnorm_silu_e4m3(xn, gn, 4.0 / 448, q=qn)

    f3 = acc.conv_flops(n, t, h, w, c, c)
    f1 = acc.conv_flops(n, t, h, w, c, 192, (1, 1, 1))
    elems = n * c * t * h * w
    # compulsory bytes: input codes and weight codes (1 byte), bias and the
    # per-channel scales, the bf16 output
    k_bytes = elems * 1 + c * c * 27 * 1 + c * 2 + c * 4 + elems * 2
    info = dict(workload="layer_384_240x416_e4m3", conv_flops=f3 + f1, latent_frames=t,
                config={"workload": "layer_384_240x416_e4m3", "channels": c, "frames": t,
                        "height": h, "width": w, "chunk_frames": t, "projection_out": 192,
                        "batch": n, "conv_operands": "e4m3", "projection": "bf16"},
                kernel=conv, kernel_name="igemm_kernel<3, 128, 32, 2, false, 32, true>",
                kernel_units=f3, kernel_bound="mfma", kernel_peak=MFMA_FP8_PEAK_TFLOPS,
                kernel_bytes=k_bytes, dtype="e4m3 x e4m3 -> f32 (conv), bf16 (projection)",
                norm_kernel=norm_kernel, norm_kernel_name="rmsnorm_flat_kernel<true, 4, true, false, true>",
                norm_bytes=elems * 3)
    return step, info


def wl_layer96():
    import torch
    from video_vae_causal_amd import _lib as L, accounting as acc, inputs
    d = inputs.layer96_inputs()
    n, c, t, h, w = d["x"].shape
    x, g, wt, b = to_dev(d["x"]), to_dev(d["gamma"]), to_dev(d["w"]), to_dev(d["b"])
    hbuf = L.empty_cl(x.shape)
    y = L.empty_cl(x.shape)
    caches = [L.empty_cl((n, c, 2, h, w)) for _ in range(2)]
    sizes = [1, 4, 4, 4, 4]
    starts = np.cumsum([0] + sizes[:-1])
    hs = [cl(hbuf[:, :, s:s + k]) for s, k in zip(starts, sizes)]
    ys = [y[:, :, s:s + k] for s, k in zip(starts, sizes)]

    wss = [conv_workspace(hs[i], wt, packed=True) for i in range(len(sizes))]
    if OPERANDS == "zero":
        for a in (x, g, wt, b, hbuf):
            a.zero_()
    wtp = L.wvc_conv3d_pack_weights(wt)

    def step():
        L.wvc_rmsnorm_silu(x, g, y=hbuf)
        L.wvc_cache_reset(caches[0])
        for i in range(len(sizes)):
            L.wvc_causal_conv3d_fwd(hs[i], wt, b, caches[i % 2], caches[(i + 1) % 2], y=ys[i],
                                    workspace=wss[i], packed_weight=wtp)

    conv_flops = acc.conv_flops(n, t, h, w, c, c)

    def kernel():
        L.wvc_causal_conv3d_fwd(hs[1], wt, b, caches[0], None, None, ys[1], workspace=wss[1],
                                packed_weight=wtp)

    def norm_kernel():
        L.wvc_rmsnorm_silu(x, g, y=hbuf)

    info = dict(workload="layer_96_480x832", conv_flops=conv_flops, latent_frames=t,
                config={"workload": "layer_96_480x832", "channels": c, "frames": t,
                        "height": h, "width": w, "chunks": sizes, "batch": n,
                        **({"operands": "zero (diagnostic)"} if OPERANDS == "zero" else {})},
                kernel=kernel, kernel_name=conv_kernel_name(hs[1], wt),
                kernel_units=acc.conv_flops(n, 4, h, w, c, c), kernel_bound="mfma",
                kernel_bytes=acc.conv_launch_bytes(n, 4, h, w, c, c),
                norm_kernel=norm_kernel, norm_kernel_name="rmsnorm_flat_kernel<true, 2, true, false, false>",
                norm_bytes=acc.norm_bytes(n * c * t * h * w))
    return step, info


def wl_decoder():
    import torch
    from video_vae_causal_amd import _lib as L, accounting as acc, inputs, stream
    d = inputs.decoder_inputs(seed=5)
    n, cl_, t, h, w = d["latent"].shape
    width = d["p"]["w_in"].shape[0]
    lat = to_dev(d["latent"])
    p = {k: ({kk: to_dev(vv) for kk, vv in v.items()} if isinstance(v, dict) else to_dev(v))
         for k, v in d["p"].items()}
    frames = [cl(lat[:, :, i:i + 1]) for i in range(t)]
    stack = stream.DecoderStack(p)
    stack.start(n, h, w)
    out = L.empty_cl((n, width, t, 2 * h, 2 * w))
    outs = [out[:, :, i:i + 1] for i in range(t)]

    pipe = make_pipe(stack, frames[0].shape) if PIPELINE else None

    def step():
        stack.reset()
        if pipe is not None:
            pipe.run(frames, outs)
        else:
            for i in range(t):
                stack.chunk(frames[i], out=outs[i])

    per_frame = (acc.conv_flops(n, 1, h, w, cl_, width) + 4 * acc.conv_flops(n, 1, h, w, width, width)
                 + 5 * acc.conv_flops(n, 1, 2 * h, 2 * w, width, width))
    cache = steady_cache((n, width, 2, 2 * h, 2 * w), "kernel_cache")
    cache_o = L.empty_cl((n, width, 2, 2 * h, 2 * w))
    kx = to_dev(inputs.quantize(inputs.normal((n, width, 1, 2 * h, 2 * w), 5, "kernel_x"), "bf16"))
    ky = L.empty_cl((n, width, 1, 2 * h, 2 * w))

    kws = conv_workspace(kx, p["w_up"], packed=True)
    wup = L.wvc_conv3d_pack_weights(p["w_up"])

    def kernel():
        L.wvc_causal_conv3d_fwd(kx, p["w_up"], p["b_up"], cache, cache_o, None, ky, workspace=kws,
                                packed_weight=wup)

    info = dict(workload="decoder_stack_48_30x52", conv_flops=per_frame * t, latent_frames=t,
                config={"workload": "decoder_stack_48_30x52", "latent_channels": cl_, "channels": width,
                        "frames": t, "height": h, "width": w, "chunk_frames": 1, "batch": n},
                kernel=kernel, kernel_name=conv_kernel_name(kx, p["w_up"]),
                kernel_units=acc.conv_flops(n, 1, 2 * h, 2 * w, width, width), kernel_bound="mfma",
                kernel_bytes=acc.conv_launch_bytes(n, 1, 2 * h, 2 * w, width, width, cache_out_frames=2),
                host=d, stack=stack, frames_dev=frames, outs=outs)
    return step, info


def wl_decoder_e4m3():
    """The decoder stack on the 8-bit path: conv_in and conv_up quantise their
    inputs (activation scales 6/448 and 8/448), the residual blocks are the
    8-bit block (norm outputs at 6/448); streamed a latent frame at a time,
    two-stream pipeline as for the bf16 stack."""
    import torch
    from video_vae_causal_amd import _lib as L, accounting as acc, inputs, stream
    d = inputs.decoder_inputs(seed=5)
    n, cl_, t, h, w = d["latent"].shape
    width = d["p"]["w_in"].shape[0]
    lat = to_dev(d["latent"])
    p = {k: ({kk: to_dev(vv) for kk, vv in v.items()} if isinstance(v, dict) else to_dev(v))
         for k, v in d["p"].items()}
    frames = [cl(lat[:, :, i:i + 1]) for i in range(t)]
    scales = {"in": 6.0 / 448, "up": 8.0 / 448, "rb": [(6.0 / 448, 6.0 / 448)] * 4}
    stack = stream.DecoderStackE4M3(p, scales)
    stack.start(n, h, w)
    out = L.empty_cl((n, width, t, 2 * h, 2 * w))
    outs = [out[:, :, i:i + 1] for i in range(t)]
    pipe = make_pipe(stack, frames[0].shape) if PIPELINE else None

    def step():
        stack.reset()
        if pipe is not None:
            pipe.run(frames, outs)
        else:
            for i in range(t):
                stack.chunk(frames[i], out=outs[i])

    per_frame = (acc.conv_flops(n, 1, h, w, cl_, width) + 4 * acc.conv_flops(n, 1, h, w, width, width)
                 + 5 * acc.conv_flops(n, 1, 2 * h, 2 * w, width, width))
    kx = L.empty_cl((n, width, 1, 2 * h, 2 * w), torch.uint8)
    L.wvc_quantize_e4m3(to_dev(inputs.quantize(inputs.normal((n, width, 1, 2 * h, 2 * w), 5, "kernel_x"),
                                               "bf16")), 8.0 / 448, q=kx)
    cache = steady_cache((n, width, 2, 2 * h, 2 * w), "kernel_cache", 8.0 / 448)
    ky = L.empty_cl((n, width, 1, 2 * h, 2 * w))
    cu = stack.conv_up
    d8 = L.conv_desc(tuple(kx.shape), tuple(cu.wq.shape), L.WVC_E4M3, weight_layout=L.WVC_WEIGHT_PACKED)
    need = L.wvc_causal_conv3d_workspace_bytes(d8)
    kws = torch.empty(need, dtype=torch.uint8, device="cuda") if need else None

    def kernel():
        L.wvc_causal_conv3d_e4m3_fwd(kx, 8.0 / 448, cu.wq, cu.wsc, p["b_up"], cache, None, None, ky,
                                     workspace=kws, packed_weight=cu.packed)

    info = dict(workload="decoder_stack_48_30x52_e4m3", conv_flops=per_frame * t, latent_frames=t,
                config={"workload": "decoder_stack_48_30x52_e4m3", "latent_channels": cl_,
                        "channels": width, "frames": t, "height": h, "width": w, "chunk_frames": 1,
                        "batch": n, "conv_operands": "e4m3", "activation_scales": scales},
                kernel=kernel,
                kernel_name="igemm_kernel<3, 128, 32, 2, true, 16, true> + splitk_reduce_kernel",
                kernel_units=acc.conv_flops(n, 1, 2 * h, 2 * w, width, width), kernel_bound="mfma",
                kernel_peak=MFMA_FP8_PEAK_TFLOPS,
                kernel_bytes=n * 4 * h * w * width * 3 + width * width * 27 + width * 6
                + n * 4 * h * w * width * 2,
                dtype="e4m3 x e4m3 -> f32 (convs); norms, upsample and activations bf16")
    return step, info


def wl_downsample():
    """The encoder's downsample path ("Cosmos3 Wan VAE", section 10.5) on the
    pages' L0 map: RMS norm + SiLU, the 1x3x3 stride-2 conv (480x832 ->
    240x416, one trailing zero row and column), the 3x1x1 temporal-stride-2
    conv (17 -> 9 frames, its cache and phase carried across chunks), RMS norm
    + SiLU; chunks of 1+4+4+4+4 frames.  With --fuse-norm on (the default) the
    first norm runs inside the stride-2 conv's staging."""
    import torch
    from video_vae_causal_amd import _lib as L, accounting as acc, inputs
    d = inputs.downsample_inputs()
    n, c, t, h, w = d["x"].shape
    x = to_dev(d["x"])
    p = {k: to_dev(v) for k, v in d.items() if k != "x"}
    ho, wo = h // 2, w // 2
    sizes = [1, 4, 4, 4, 4]
    starts = [int(v) for v in np.cumsum([0] + sizes[:-1])]
    phases = [g % 2 for g in starts]
    touts = [L.conv_out_frames(k, 2, ph) for k, ph in zip(sizes, phases)]
    ostarts = [int(v) for v in np.cumsum([0] + touts[:-1])]
    h1 = L.empty_cl(x.shape)
    sbuf = L.empty_cl((n, c, t, ho, wo))
    y = L.empty_cl((n, c, sum(touts), ho, wo))
    out = L.empty_cl(y.shape)
    caches = [L.empty_cl((n, c, 2, ho, wo)) for _ in range(2)]
    hs = [cl(h1[:, :, s:s + k]) for s, k in zip(starts, sizes)]
    xs = [cl(x[:, :, s:s + k]) for s, k in zip(starts, sizes)]
    ss = [cl(sbuf[:, :, s:s + k]) for s, k in zip(starts, sizes)]
    ys = [y[:, :, s:s + k] for s, k in zip(ostarts, touts)]
    sp_kw = dict(stride=(1, 2, 2), padding=(0, 0), pad_extra=(1, 1))
    tm_kw = dict(stride=(2, 1, 1), padding=(0, 0))
    wsp = L.wvc_conv3d_pack_weights(p["w_s"], **sp_kw)
    wtp = L.wvc_conv3d_pack_weights(p["w_t"], **tm_kw)

    def spatial(i):
        if FUSE_NORM:
            L.wvc_rmsnorm_silu_conv3d_fwd(xs[i], p["gamma1"], p["w_s"], p["b_s"], y=ss[i],
                                          packed_weight=wsp)
        else:
            L.wvc_causal_conv3d_fwd(hs[i], p["w_s"], p["b_s"], y=ss[i], packed_weight=wsp, **sp_kw)

    def step():
        if not FUSE_NORM:
            L.wvc_rmsnorm_silu(x, p["gamma1"], y=h1)
        L.wvc_cache_reset(caches[0])
        for i in range(len(sizes)):
            spatial(i)
            L.wvc_causal_conv3d_fwd(ss[i], p["w_t"], p["b_t"], caches[i % 2], caches[(i + 1) % 2],
                                    y=ys[i], packed_weight=wtp, t_phase=phases[i], **tm_kw)
        L.wvc_rmsnorm_silu(y, p["gamma2"], y=out)

    f_sp = 2 * 9 * c * c * t * ho * wo
    f_tm = 2 * 3 * c * c * sum(touts) * ho * wo

    def kernel():
        spatial(1)

    k_bytes = 2 * c * (4 * h * w + 4 * ho * wo) + 2 * 9 * c * c
    info = dict(workload="downsample_96_480x832", conv_flops=f_sp + f_tm, latent_frames=t,
                config={"workload": "downsample_96_480x832", "channels": c, "frames": t,
                        "height": h, "width": w, "out_frames": sum(touts), "out_height": ho,
                        "out_width": wo, "chunks": sizes, "batch": n, "fused_norm": FUSE_NORM},
                kernel=kernel,
                kernel_name=(L.wvc_conv3d_kernel_name(L.conv_desc(tuple(xs[1].shape), tuple(p["w_s"].shape),
                                                                  L.WVC_BF16, **{k: v for k, v in sp_kw.items()}))
                             .replace("<false>", "<true>" if FUSE_NORM else "<false>")),
                kernel_units=k_bytes, kernel_bound="hbm", kernel_bytes=k_bytes,
                kernel_flops=2 * 9 * c * c * 4 * ho * wo)
    return step, info


FUSE_NORM = True  # set from --fuse-norm in main()
TILINGS = {"page": ((60, 104), (30, 52)), "reduced": ((60, 104), (52, 96)), "untiled": (None, None)}
TILING = "page"  # set from --tiling in main()


def wl_tiled():
    """Tiled decode ("VSR Hover Comparison", decoder tiling): the decoder-shaped
    stack on a 192x336 latent (a 2688x1536 video's latent at 8x), 3 frames,
    in (60, 104) latent tiles at the page's stride (30, 52) -- 50 % overlap --
    or a reduced stride, or untiled; tiles blended with linear ramps."""
    import torch
    from video_vae_causal_amd import _lib as L, accounting as acc, inputs, stream
    d = inputs.decoder_inputs(seed=8, shape=(1, 48, 3, 192, 336))
    n, cl_, t, h, w = d["latent"].shape
    width = d["p"]["w_in"].shape[0]
    lat = to_dev(d["latent"])
    p = {k: ({kk: to_dev(vv) for kk, vv in v.items()} if isinstance(v, dict) else to_dev(v))
         for k, v in d["p"].items()}
    stack = stream.DecoderStack(p)
    tile, stride = TILINGS[TILING]
    if tile is None:
        def step():
            stack.run(lat, chunk_frames=1)
        tiles, th, tw = 1, h, w
    else:
        td = stream.TiledDecode(stack, tile=tile, stride=stride)
        th, tw, ys, xs = td.origins(h, w)
        tiles = len(ys) * len(xs)

        def step():
            td.run(lat, chunk_frames=1)

    def per_frame(hh, ww):
        return (acc.conv_flops(n, 1, hh, ww, cl_, width) + 4 * acc.conv_flops(n, 1, hh, ww, width, width)
                + 5 * acc.conv_flops(n, 1, 2 * hh, 2 * ww, width, width))

    # the dominant kernel: the 3x3x3 conv on one decoded tile frame at 2x
    kx = cl(torch.randn((n, width, 1, 2 * th, 2 * tw), device="cuda").to(torch.bfloat16))
    ky = L.empty_cl(kx.shape)
    cache = steady_cache((n, width, 2, 2 * th, 2 * tw), "kernel_cache")
    kws = conv_workspace(kx, p["w_up"], packed=True)
    wup = L.wvc_conv3d_pack_weights(p["w_up"])

    def kernel():
        L.wvc_causal_conv3d_fwd(kx, p["w_up"], p["b_up"], cache, None, None, ky, workspace=kws,
                                packed_weight=wup)

    info = dict(workload="decoder_tiled_192x336", conv_flops=tiles * t * per_frame(th, tw),
                latent_frames=t,
                config={"workload": "decoder_tiled_192x336", "latent_channels": cl_, "channels": width,
                        "frames": t, "height": h, "width": w, "tiling": TILING,
                        "tile": list(tile) if tile else None, "stride": list(stride) if stride else None,
                        "tiles": tiles, "decoded_latent_px_per_px": round(tiles * th * tw / (h * w), 3),
                        "chunk_frames": 1, "batch": n},
                kernel=kernel,
                kernel_name=conv_kernel_name(kx, p["w_up"]),
                kernel_units=acc.conv_flops(n, 1, 2 * th, 2 * tw, width, width), kernel_bound="mfma",
                kernel_bytes=acc.conv_launch_bytes(n, 1, 2 * th, 2 * tw, width, width))
    return step, info


WORKLOADS = {"resblock_384_60x104": wl_resblock, "layer_384_240x416": wl_layer384,
             "layer_384_240x416_e4m3": wl_layer384_e4m3, "resblock_384_60x104_e4m3": wl_resblock_e4m3,
             "decoder_stack_48_30x52_e4m3": wl_decoder_e4m3,
             "layer_96_480x832": wl_layer96, "decoder_stack_48_30x52": wl_decoder,
             "downsample_96_480x832": wl_downsample, "decoder_tiled_192x336": wl_tiled}


# ---------------------------------------------------------------------------
# Measurements the default line carries besides its own workload.
# ---------------------------------------------------------------------------

def extra_decoder(args):
    """ms per decoded latent frame: the decoder-shaped stack (48-ch latent
    [1,48,21,30,52] -> 384 ch, 30x52 -> 60x104) streamed one latent frame at a
    time through its ten 2-frame caches, two-stream pipeline on; plus a
    sequential pass with events around every frame, for frame 0 (zero
    caches) and the steady state of frames 2-20 (both cached frames real)."""
    import torch
    global PIPELINE
    saved, PIPELINE = PIPELINE, True
    try:
        step, info = wl_decoder()
    finally:
        PIPELINE = saved
    ms, _ = time_region(step, args.steps, args.warmup, args.warmup_seconds)
    stack, frames_dev = info["stack"], info["frames_dev"]
    n_fr = info["latent_frames"]
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(n_fr + 1)]
    per = []
    for _ in range(3):
        stack.reset()
        ev[0].record()
        for i in range(n_fr):
            stack.chunk(frames_dev[i], out=info["outs"][i])
            ev[i + 1].record()
        torch.cuda.synchronize()
        per.append([ev[i].elapsed_time(ev[i + 1]) for i in range(n_fr)])
    per = np.median(np.array(per), axis=0)
    tflops = info["conv_flops"] / (ms * 1e-3) / 1e12
    return {"ms_per_decoded_latent_frame": round(ms / n_fr, 4),
            "decoder_stack": {"workload": "decoder_stack_48_30x52", "latent_frames": n_fr,
                              "ms_per_step": round(ms, 4), "conv_tflops": round(tflops, 1),
                              "pct_mfma_peak": round(100 * tflops / MFMA_BF16_PEAK_TFLOPS, 2),
                              "two_stream_pipeline": True,
                              "sequential_ms_frame0": round(float(per[0]), 4),
                              "sequential_ms_per_frame_2_to_20": round(float(per[2:].mean()), 4),
                              "sequential_ms_per_frame": round(float(per.sum()) / n_fr, 4),
                              "dominant_kernel": info["kernel_name"]}}


def extra_norm96(args):
    """The fused RMS norm + SiLU over the 96-channel encoder map
    x[1,96,17,480,832] (bf16 in and out): its HBM roofline."""
    from video_vae_causal_amd import _lib as L, accounting as acc, inputs
    shape = (1, 96, 17, 480, 832)
    x = to_dev(inputs.quantize(inputs.normal(shape, 3, "x"), "bf16"))
    g = to_dev(inputs.norm_gamma(96, 3, "gamma", "bf16"))
    y = L.empty_cl(shape)

    def norm_kernel():
        L.wvc_rmsnorm_silu(x, g, y=y)

    n_ms, n_timing = kernel_ms(norm_kernel, 20, min(args.warmup_seconds, 0.2),
                               args.kernel_timing == "graph")
    nbytes = acc.norm_bytes(int(np.prod(shape)))
    gbs = nbytes / (n_ms * 1e-3) / 1e9
    name = "rmsnorm_flat_kernel<true, 2, true, false, false>"
    return {"roofline_norm": {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS,
                              "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4),
                              "traffic": measured_traffic(args.traffic_json, "layer_96_480x832/norm", name),
                              "kernel": name, "kernel_ms": round(n_ms, 5), "timing": n_timing,
                              "bytes_per_launch": nbytes,
                              "workload": "rmsnorm_silu_96_480x832 (x[1,96,17,480,832] bf16)"}}


# ---------------------------------------------------------------------------
# CPU baseline: the fp64 oracle on a bounded sample of the same workload.
# ---------------------------------------------------------------------------

def cpu_time_loop(run, min_s: float = 10.0):
    """Run the sample once, then again until ``min_s`` seconds of CPU work
    have passed; returns (seconds, runs)."""
    t0 = time.perf_counter()
    runs = 0
    while True:
        run()
        runs += 1
        dt = time.perf_counter() - t0
        if dt >= min_s:
            return dt, runs


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def omp_threads(k: int):
    """Set the OpenMP thread count of later parallel regions started from this
    thread (the oracle's library is built with OpenMP)."""
    import ctypes
    ctypes.CDLL("libgomp.so.1").omp_set_num_threads(int(k))


def layer384_baseline(info, threads):
    """The 384-channel layer's leg: the oracle on output frames 2-4, rows
    0-119 of the 3x3x3 conv (its cache = input frames 0-1, so every tap is a
    real frame), timed on all host threads; the same conv on 2 rows of one
    frame with one thread; then the GPU's output of the timed step compared
    with the oracle's on that sample (rows 0-118, whose 3x3 window lies inside
    the cropped rows) and the projection of frame 2 likewise."""
    import oracle
    from video_vae_causal_amd import accounting as acc
    d = info["host"]
    rows = 120
    w64, b64 = d["w"].astype(np.float64), d["b"].astype(np.float64)
    xs = d["x"][:, :, 2:5, :rows].astype(np.float64)
    past = d["x"][:, :, 0:2, :rows].astype(np.float64)
    n, c, f, h, w = xs.shape
    flops = acc.conv_flops(n, f, h, w, c, c)
    out = {}
    run = lambda: out.__setitem__("y", oracle.causal_conv3d(xs, w64, b64, cache=past))
    dt, runs = cpu_time_loop(run)
    res = {"value": flops * runs / dt / 1e12, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
           "cpu_model": cpu_model(),
           "sample": f"3x3x3 conv output frames 2-4 x rows 0-{rows - 1} x {w} x {c} channels "
                     f"(cache = input frames 0-1), run {runs}x",
           "seconds": round(dt, 3), "flops": flops * runs}
    # one thread, a smaller sample of the same conv: frame 2, rows 0-1
    x1, p1 = xs[:, :, 0:1, :2], past[:, :, :, :2]
    f1 = acc.conv_flops(n, 1, 2, w, c, c)
    omp_threads(1)
    try:
        dt1, runs1 = cpu_time_loop(lambda: oracle.causal_conv3d(x1, w64, b64, cache=p1), min_s=5.0)
    finally:
        omp_threads(threads)
    res["single_thread"] = {"value": f1 * runs1 / dt1 / 1e12, "unit": "TFLOP/s", "cores": 1,
                            "sample": f"conv output frame 2, rows 0-1 x {w} x {c} channels, run {runs1}x",
                            "seconds": round(dt1, 3), "flops": f1 * runs1}
    # parity of the benched run on the sample
    g = info["gpu_outputs"]()
    ref = out["y"][:, :, :, :rows - 1]
    got = g["y"][:, :, 2:5, :rows - 1].float().cpu().numpy().astype(np.float64)
    parity = {"conv": parity_entry(got, ref, "bf16 conv vs fp64 oracle, frames 2-4, rows 0-118, all "
                                             "416 columns and 384 channels")}
    conv_b = oracle.round_bf16(ref[:, :, 0:1])          # the conv output as stored (bf16)
    pref = oracle.causal_conv3d(conv_b, d["wp"].astype(np.float64), d["bp"].astype(np.float64), pad=(0, 0))
    pgot = g["proj"][:, :, 2:3, :rows - 1].float().cpu().numpy().astype(np.float64)
    parity["projection"] = parity_entry(pgot, pref, "1x1x1 384->192 of the bf16 conv output, frame 2, "
                                                    "rows 0-118 (oracle fed the oracle's rounded conv)")
    res["parity"] = parity
    return res


def parity_entry(got, ref, what):
    import oracle
    rel = oracle.rel_l2(got, ref)
    mx = oracle.max_abs(got, ref)
    bound = 2e-2 * float(np.max(np.abs(ref)))
    return {"compared": int(ref.size), "rel_l2": float(f"{rel:.4g}"), "max_abs": float(f"{mx:.4g}"),
            "max_abs_bound": float(f"{bound:.4g}"), "rel_l2_bound": 1e-2,
            "pass": bool(rel <= 1e-2 and mx <= bound), "what": what}


def cpu_baseline(workload: str, info=None):
    import oracle
    from video_vae_causal_amd import accounting as acc, inputs
    threads = int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))
    if workload == "layer_384_240x416" and info is not None and "host" in info:
        return layer384_baseline(info, threads)

    def f64_params(p):
        return {k: ({kk: vv.astype(np.float64) for kk, vv in v.items()} if isinstance(v, dict)
                    else v.astype(np.float64)) for k, v in p.items()}

    if workload in ("decoder_stack_48_30x52", "decoder_tiled_192x336"):
        if workload == "decoder_stack_48_30x52":
            d = inputs.decoder_inputs(seed=5)
            sample = "latent frames 0-1 of 21 through the whole stack (bf16-boundary oracle)"
        else:
            d = inputs.decoder_inputs(seed=8, shape=(1, 48, 3, 192, 336), with_latent_window=(30, 52))
            sample = "latent frames 0-1, the 30x52 top-left window, through the whole stack"
        lat = d["latent"][:, :, :2].astype(np.float64)
        p = f64_params(d["p"])
        n, cl_, t, h, w = lat.shape
        width = p["w_in"].shape[0]
        flops = (acc.conv_flops(n, t, h, w, cl_, width) + 4 * acc.conv_flops(n, t, h, w, width, width)
                 + 5 * acc.conv_flops(n, t, 2 * h, 2 * w, width, width))
        run = lambda: oracle.decoder_stack(lat, p, bf16=True)
    elif workload == "resblock_384_60x104":
        r = inputs.resblock_inputs(seed=2)
        x = r["x"].astype(np.float64)
        p = f64_params(r["p"])
        n, c, t, h, w = x.shape
        flops = 2 * acc.conv_flops(n, t, h, w, c, c)
        run = lambda: oracle.resblock(x, p, bf16=True)
        sample = "the whole 5-frame step through the block (bf16-boundary oracle)"
    elif workload == "downsample_96_480x832":
        d = inputs.downsample_inputs()
        xs = d["x"][:, :, :4].astype(np.float64)   # frames 0..3 (one 4-frame chunk)
        n, c, f, h, w = xs.shape
        flops = 2 * 9 * c * c * f * (h // 2) * (w // 2)
        ws_, bs_, g_ = d["w_s"].astype(np.float64), d["b_s"].astype(np.float64), d["gamma1"].astype(np.float64)
        run = lambda: oracle.causal_conv3d_strided(oracle.norm_silu(xs, g_, bf16=True), ws_, bs_,
                                                   stride=(1, 2, 2), pad=(0, 0), pad_extra=(1, 1))
        sample = "frames 0-3 (one 4-frame chunk): norm + SiLU, then the stride-2 spatial conv"
    elif workload == "decoder_stack_48_30x52_e4m3":
        d = inputs.decoder_inputs(seed=5)
        lat = d["latent"][:, :, :2].astype(np.float64)
        p = f64_params(d["p"])
        n, cl_, t, h, w = lat.shape
        width = p["w_in"].shape[0]
        flops = (acc.conv_flops(n, t, h, w, cl_, width) + 4 * acc.conv_flops(n, t, h, w, width, width)
                 + 5 * acc.conv_flops(n, t, 2 * h, 2 * w, width, width))
        sc = {"in": 6.0 / 448, "up": 8.0 / 448, "rb": [(6.0 / 448, 6.0 / 448)] * 4}
        run = lambda: oracle.decoder_stack_e4m3(lat, p, sc)
        sample = "latent frames 0-1 of 21 through the whole 8-bit stack"
    elif workload == "resblock_384_60x104_e4m3":
        r = inputs.resblock_inputs(seed=2)
        x = r["x"].astype(np.float64)
        p = f64_params(r["p"])
        n, c, t, h, w = x.shape
        flops = 2 * acc.conv_flops(n, t, h, w, c, c)
        run = lambda: oracle.resblock_e4m3(x, p, 5.0 / 448, 5.0 / 448)
        sample = "the whole 5-frame step through the 8-bit block"
    elif workload == "layer_384_240x416_e4m3":
        rows = 120
        d = inputs.e4m3_conv_inputs(seed=7, shape=(1, 384, 3, rows, 416), cout=384, with_cache=False)
        n, c, f, h, w = d["x"].shape
        flops = acc.conv_flops(n, f, h, w, c, c)
        b64 = d["b"].astype(np.float64)
        run = lambda: oracle.causal_conv3d_e4m3(d["x"], d["x_scale"], d["w"], d["w_scale"], b64)
        sample = f"3 frames x {rows} rows x 416 of the 8-bit 3x3x3 conv (decode + fp64 conv)"
    else:
        d = inputs.layer384_inputs() if workload == "layer_384_240x416" else inputs.layer96_inputs()
        c = d["x"].shape[1]
        frames, rows = (3, 120) if c == 384 else (4, 480)
        xs = d["x"][:, :, :frames, :rows].astype(np.float64)
        n, c, _, h, w = xs.shape
        past = np.zeros((n, c, 2, rows, w))
        flops = acc.conv_flops(n, frames, rows, w, c, c)
        w64, b64 = d["w"].astype(np.float64), d["b"].astype(np.float64)
        run = lambda: oracle.causal_conv3d(xs, w64, b64, cache=past)
        sample = f"frames 0-{frames - 1}, rows 0-{rows - 1} of the 3x3x3 conv"
    dt, runs = cpu_time_loop(run)
    return {"value": flops * runs / dt / 1e12, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "cpu_model": cpu_model(),
            "sample": sample + f", run {runs}x", "seconds": round(dt, 3), "flops": flops * runs}


def measured_traffic(path: str, key: str, kernel_name: str):
    """HBM bytes per launch of ``kernel_name`` from rocprofv3 FETCH_SIZE and
    WRITE_SIZE runs (scaled by the counters' reading for a copy of known size),
    or None when there is no record or the kernel's source changed since."""
    import hashlib
    try:
        entry = json.load(open(path)).get(key)
    except (OSError, ValueError):
        return None
    if not entry or entry.get("kernel") != kernel_name:
        return None
    try:
        src = open(os.path.join(ROOT, entry["source"]), "rb").read()
    except (OSError, KeyError):
        return None
    if hashlib.sha256(src).hexdigest() != entry.get("source_sha256"):
        return None
    return entry.get("bytes_per_launch")


def copy_calibration(mib: int):
    """Five launches of torch's contiguous copy over ``mib`` MiB: each reads and
    writes exactly that many bytes, so the counters' readings for it give the
    scale of FETCH_SIZE and WRITE_SIZE."""
    import torch
    n = mib * (1 << 20) // 2
    a = torch.ones(n, dtype=torch.bfloat16, device="cuda")
    b = torch.empty_like(a)
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    for _ in range(5):
        b.copy_(a)
    end.record()
    torch.cuda.synchronize()
    ms = start.elapsed_time(end) / 5
    print(json.dumps({"copy_bytes_read": 2 * n, "copy_bytes_written": 2 * n, "ms": round(ms, 4),
                      "GBs_read_plus_write": round(4 * n / ms / 1e6, 1)}), flush=True)


def library_gemm(spec: str):
    """The vendor library's GEMM (hipBLASLt under torch) on the conv's contraction
    shape, M = C_out, K = 27 * C_in, N = output positions, with both operands
    already materialised: a reference point for the implicit-GEMM conv, which
    builds its B operand from the halo on the fly."""
    import torch
    m, n, k = (int(v) for v in spec.split(","))
    a = torch.randn(m, k, device="cuda", dtype=torch.bfloat16)
    b = torch.randn(k, n, device="cuda", dtype=torch.bfloat16)
    bt = torch.randn(n, k, device="cuda", dtype=torch.bfloat16)
    c = torch.empty(m, n, device="cuda", dtype=torch.bfloat16)
    ct = torch.empty(n, m, device="cuda", dtype=torch.bfloat16)

    def timed(fn, reps=20):
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        start.record()
        for _ in range(reps):
            fn()
        end.record()
        torch.cuda.synchronize()
        return start.elapsed_time(end) / reps

    flops = 2.0 * m * n * k
    out = {"library_gemm": [m, n, k], "flops": flops}
    for key, fn in (("bf16_w_x", lambda: torch.matmul(a, b, out=c)),
                    ("bf16_xt_wt", lambda: torch.matmul(bt, a.t(), out=ct))):
        ms = timed(fn)
        out[key] = {"ms": round(ms, 4), "tflops": round(flops / ms / 1e9, 1)}
    a8, bt8 = a.to(torch.float8_e4m3fn), bt.to(torch.float8_e4m3fn)
    one = torch.ones((), device="cuda")
    ms = timed(lambda: torch._scaled_mm(bt8, a8.t(), scale_a=one, scale_b=one,
                                        out_dtype=torch.bfloat16))
    out["e4m3_xt_wt"] = {"ms": round(ms, 4), "tflops": round(flops / ms / 1e9, 1)}
    print(json.dumps(out), flush=True)


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on exactly one GPU; --gpus {args.gpus} is not supported "
              "(the library runs on one GPU and has no multi-GPU sharding)", file=sys.stderr)
        sys.exit(2)
    if args.operands == "zero":
        if args.workload not in ("layer_384_240x416", "layer_96_480x832"):
            print("--operands zero is a diagnostic of the layer_384_240x416 and layer_96_480x832 "
                  "workloads only", file=sys.stderr)
            sys.exit(2)
        args.no_cpu_baseline = True  # the oracle's sample is random data
    if args.pipeline == "auto":
        args.pipeline = "on" if args.workload in PIPELINE_AUTO else "off"
    if args.graph == "auto":
        args.graph = "on" if args.workload in GRAPH_AUTO else "off"
    import torch
    if args.copy_calibration:
        copy_calibration(args.copy_calibration)
        return
    if args.library_gemm:
        library_gemm(args.library_gemm)
        return
    from video_vae_causal_amd import _lib as L
    L.load()
    torch.cuda.set_device(0)

    global PIPELINE, PIPE_GRAPH, TILING, FUSE_NORM, OPERANDS
    OPERANDS = args.operands
    PIPELINE = args.pipeline == "on"
    # two streams are not recorded into one graph: with the pipeline, --graph
    # records each chunk's two parts (stream.PipelineGraph) instead of the step
    PIPE_GRAPH = PIPELINE and args.graph == "on" and args.workload in PIPELINED
    FUSE_NORM = args.fuse_norm == "on"
    TILING = args.tiling
    step, info = WORKLOADS[args.workload]()
    timed = step
    if args.graph == "on" and not PIPE_GRAPH:
        # The eager warm-up sizes every workspace and buffer; the graph then
        # records one whole step (cache resets included) and each timed call
        # replays it.
        from video_vae_causal_amd import stream
        for _ in range(max(1, args.warmup)):
            step()
        torch.cuda.synchronize()
        graph = stream.capture(step)
        timed = graph.launch
    ms_step, wall = time_region(timed, args.steps, args.warmup, args.warmup_seconds)
    value = info["conv_flops"] / (ms_step * 1e-3) / 1e12

    # dominant kernel, timed alone with events on the stream it is launched on
    k_ms, k_timing = kernel_ms(info["kernel"], info.get("kernel_reps", args.kernel_reps),
                               min(args.warmup_seconds, 0.2), args.kernel_timing == "graph")
    traffic = measured_traffic(args.traffic_json, args.workload, info["kernel_name"])
    if info["kernel_bound"] == "hbm":
        achieved = info["kernel_bytes"] / (k_ms * 1e-3) / 1e9
        peak, unit = HBM_PEAK_GBS, "GB/s"
        flops = info["kernel_flops"]
    else:
        achieved = info["kernel_units"] / (k_ms * 1e-3) / 1e12
        peak, unit = info.get("kernel_peak", MFMA_BF16_PEAK_TFLOPS), "TFLOP/s"
        flops = info["kernel_units"]
    roofline = {"bound": info["kernel_bound"], "achieved": round(achieved, 2),
                "peak": peak, "unit": unit,
                "frac": round(achieved / peak, 4), "traffic": traffic,
                "kernel": info["kernel_name"], "kernel_ms": round(k_ms, 5), "timing": k_timing,
                "flops_per_launch": flops,
                "mfma_frac": round(flops / (k_ms * 1e-3) / 1e12 / info.get("kernel_peak", MFMA_BF16_PEAK_TFLOPS), 4),
                "algorithmic_bytes_per_launch": info["kernel_bytes"]}

    line = {
        "metric": METRIC, "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "warmup_s": args.warmup_seconds,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": info.get("dtype", "bf16"),
        "data": ("synthetic (seeded Philox normals, random-init weights)" if args.operands == "random"
                 else "all-zero input and weights (diagnostic, not the metric)"),
        "config": dict(info["config"], hip_graph=args.graph == "on",
                       two_stream_pipeline=PIPELINE and args.workload in PIPELINED),
        "pct_mfma_peak": round(100 * value / info.get("kernel_peak", MFMA_BF16_PEAK_TFLOPS), 2),
        "ms_per_latent_frame": round(ms_step / info["latent_frames"], 4),
        "conv_flops_per_step": info["conv_flops"],
        "wall_s_timed": round(wall, 3),
        "roofline": roofline,
    }
    if "norm_kernel" in info:
        n_ms, n_timing = kernel_ms(info["norm_kernel"], 20, min(args.warmup_seconds, 0.2),
                                   args.kernel_timing == "graph")
        gbs = info["norm_bytes"] / (n_ms * 1e-3) / 1e9
        line["roofline_norm"] = {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS,
                                 "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4),
                                 "traffic": measured_traffic(args.traffic_json, args.workload + "/norm",
                                                             info["norm_kernel_name"]),
                                 "kernel": info["norm_kernel_name"],
                                 "kernel_ms": round(n_ms, 5), "timing": n_timing,
                                 "bytes_per_launch": info["norm_bytes"]}
    if args.workload == "layer_384_240x416" and not args.no_extras and args.operands == "random":
        line.update(extra_decoder(args))
        line.update(extra_norm96(args))
    if not args.no_cpu_baseline:
        cb = cpu_baseline(args.workload, info)
        parity = cb.pop("parity", None)
        line["cpu_baseline"] = cb
        if parity is not None:
            line["parity"] = parity
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
