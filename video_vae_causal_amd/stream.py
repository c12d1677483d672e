"""Streaming driver: per-layer rolling caches and chunked decoding.

A causal conv only looks back, so a long latent sequence can be decoded chunk
by chunk (one frame, or k frames) as long as every conv keeps the last two
frames of its input and puts them in front of the next chunk ("Cosmos3 Wan VAE
-- engine size vs runtime context memory", sections 8.5 and 10.3; frame-by-
frame decoding with a shared cache is how the pages keep VAE decode memory
bounded: "diffusion inference workload anatomy", VAE-decode peak paragraph).

Each layer owns two cache buffers and ping-pongs them: chunk i reads cache
``cur`` and the library writes the next cache into the other one.  Resetting a
stream zero-fills the caches, which is exactly zero causal padding before
frame 0.  The caches are the whole resumable state of a stream:
``state()``/``load_state()`` copy them out and back (checkpoint/resume).

A chunk of a stack is a few dozen short launches.  ``capture`` records them
into a HIP graph (the launch-overhead remedy of the Cosmos3 page's section
8.7); ``FrameGraph`` replays one chunk per call with the stack's ping-pong
state kept in step.

Host orchestration only; every tensor operation is a libwvc call.
"""
from __future__ import annotations

from typing import Callable, Dict, List, Optional, Sequence

import torch

from . import _lib as L

CACHE_T = 2


def _try_pack(weight: torch.Tensor, padding) -> Optional[torch.Tensor]:
    """Pack a layer's weights once for the MFMA routes; None when the layer
    takes the direct route (no packed form exists)."""
    try:
        return L.wvc_conv3d_pack_weights(weight, padding)
    except L.WvcError:
        return None


def _cached_buf(bufs: Dict[str, torch.Tensor], name: str, shape, like: torch.Tensor) -> torch.Tensor:
    b = bufs.get(name)
    if b is None or tuple(b.shape) != tuple(shape) or b.dtype != like.dtype:
        b = L.empty_cl(shape, like.dtype, like.device)
        bufs[name] = b
    return b


class _PingPong:
    """A layer's cache pair.  After ``reset()`` the cache is *fresh*: the next
    chunk passes ``cache_in = NULL``, which the library reads as zero causal
    padding, so a new sequence costs no fill.  ``materialize()`` writes those
    zeros into the buffer for callers that need the buffer itself (a graph
    that records buffer addresses, a checkpoint)."""

    def __init__(self, shape, dtype, device):
        self.buf = [L.empty_cl(shape, dtype, device), L.empty_cl(shape, dtype, device)]
        self.cur = 0
        self.reset()

    def reset(self):
        self.cur = 0
        self.fresh = True

    def materialize(self):
        if self.fresh:
            # Only the buffer the next chunk reads must be zero; the other is
            # entirely rewritten as that chunk's cache_out.
            L.wvc_cache_reset(self.buf[self.cur])
            self.fresh = False

    @property
    def cin(self):
        return None if self.fresh else self.buf[self.cur]

    @property
    def cout(self):
        return self.buf[1 - self.cur]

    def flip(self):
        self.cur ^= 1
        self.fresh = False


class CausalConv3d:
    """A causal 3x3x3 conv layer with its rolling 2-frame cache."""

    def __init__(self, weight: torch.Tensor, bias: Optional[torch.Tensor]):
        self.weight = weight
        self.bias = bias
        self.frames = L.wvc_conv3d_cache_frames(tuple(weight.shape))
        self.cache: Optional[_PingPong] = None
        self.ws: Optional[torch.Tensor] = None
        self.padding = (1, 1) if weight.shape[3] == 3 else (0, 0)
        self.packed = _try_pack(weight, self.padding)

    def start(self, n: int, h: int, w: int):
        c = self.weight.shape[1]
        if self.frames:
            shape = (n, c, self.frames, h, w)
            if self.cache is None or tuple(self.cache.buf[0].shape) != shape:
                self.cache = _PingPong(shape, self.weight.dtype, self.weight.device)
            else:
                self.cache.reset()

    def __call__(self, x: torch.Tensor, y: Optional[torch.Tensor] = None,
                 residual: Optional[torch.Tensor] = None) -> torch.Tensor:
        if self.cache is None and self.frames:
            self.start(x.shape[0], x.shape[3], x.shape[4])
        cin = self.cache.cin if self.frames else None
        cout = self.cache.cout if self.frames else None
        layout = L.WVC_WEIGHT_PACKED if self.packed is not None else L.WVC_WEIGHT_STANDARD
        d = L.conv_desc(tuple(x.shape), tuple(self.weight.shape), L._dtype_code(x.dtype),
                        padding=self.padding, weight_layout=layout)
        need = L.wvc_causal_conv3d_workspace_bytes(d)
        if need and (self.ws is None or self.ws.numel() < need):
            self.ws = torch.empty(need, dtype=torch.uint8, device=x.device)
        y = L.wvc_causal_conv3d_fwd(x, self.weight, self.bias, cin, cout, residual, y,
                                    padding=self.padding, workspace=self.ws if need else None,
                                    packed_weight=self.packed)
        if self.frames:
            self.cache.flip()
        return y

    def caches(self) -> List[torch.Tensor]:
        if self.cache is None:
            return []
        self.cache.materialize()
        return [self.cache.cin]

    def reset(self):
        """Zero the caches in place (a new sequence), keeping their buffers."""
        if self.cache is not None:
            self.cache.reset()

    def pingpongs(self) -> List[_PingPong]:
        return [self.cache] if self.cache is not None else []

    def stages(self, x: torch.Tensor, y: torch.Tensor, buf) -> List[Callable[[], object]]:
        return [lambda: self(x, y=y)]


class ResBlock:
    """Wan residual block with the two caches of its 3x3x3 convs."""

    def __init__(self, params: Dict[str, torch.Tensor], eps: float = 1e-12):
        self.p = params
        self.eps = eps
        self.c1: Optional[_PingPong] = None
        self.c2: Optional[_PingPong] = None
        self.ws: Optional[torch.Tensor] = None
        packed = {"w1": _try_pack(params["w1"], (1, 1)), "w2": _try_pack(params["w2"], (1, 1))}
        if params.get("w_short") is not None:
            packed["w_short"] = _try_pack(params["w_short"], (0, 0))
        self.packed = packed if all(v is not None for v in packed.values()) else None

    def start(self, n: int, h: int, w: int):
        cin = self.p["w1"].shape[1]
        cout = self.p["w1"].shape[0]
        dt, dev = self.p["w1"].dtype, self.p["w1"].device
        s1, s2 = (n, cin, CACHE_T, h, w), (n, cout, CACHE_T, h, w)
        if self.c1 is not None and tuple(self.c1.buf[0].shape) == s1 and \
                tuple(self.c2.buf[0].shape) == s2:
            self.reset()
            return
        self.c1 = _PingPong(s1, dt, dev)
        self.c2 = _PingPong(s2, dt, dev)

    def reset(self):
        """Zero the caches in place (a new sequence), keeping their buffers."""
        if self.c1 is not None:
            self.c1.reset()
            self.c2.reset()

    def pingpongs(self) -> List[_PingPong]:
        return [self.c1, self.c2] if self.c1 is not None else []

    def __call__(self, x: torch.Tensor, y: Optional[torch.Tensor] = None) -> torch.Tensor:
        if self.c1 is None:
            self.start(x.shape[0], x.shape[3], x.shape[4])
        d = L.resblock_desc(tuple(x.shape), self.p["w1"].shape[0], L._dtype_code(x.dtype), self.eps,
                            weights_packed=self.packed is not None)
        need = L.wvc_resblock_workspace_bytes(d)
        if self.ws is None or self.ws.numel() < need:
            self.ws = torch.empty(need, dtype=torch.uint8, device=x.device)
        y = L.wvc_resblock_fwd(x, self.p, self.c1.cin, self.c1.cout, self.c2.cin, self.c2.cout,
                               y=y, eps=self.eps, workspace=self.ws, packed=self.packed)
        self.c1.flip()
        self.c2.flip()
        return y

    def caches(self) -> List[torch.Tensor]:
        if self.c1 is None:
            return []
        self.c1.materialize()
        self.c2.materialize()
        return [self.c1.cin, self.c2.cin]

    def _half_ws(self, name: str, x: torch.Tensor) -> torch.Tensor:
        d = L.resblock_desc(tuple(x.shape), self.p["w1"].shape[0], L._dtype_code(x.dtype), self.eps,
                            weights_packed=self.packed is not None)
        need = L.wvc_resblock_workspace_bytes(d)
        ws = self.__dict__.get(name)
        if ws is None or ws.numel() < need:
            ws = torch.empty(need, dtype=torch.uint8, device=x.device)
            setattr(self, name, ws)
        return ws

    def front(self, x: torch.Tensor, h2: torch.Tensor) -> torch.Tensor:
        """First half (norm1, conv1, norm2) into h2; advances cache1."""
        if self.c1 is None:
            self.start(x.shape[0], x.shape[3], x.shape[4])
        L.wvc_resblock_front(x, self.p, self.c1.cin, self.c1.cout, h2=h2, eps=self.eps,
                             workspace=self._half_ws("ws_front", x), packed=self.packed)
        self.c1.flip()
        return h2

    def back(self, h2: torch.Tensor, x: torch.Tensor, y: torch.Tensor) -> torch.Tensor:
        """Second half (conv2 + shortcut) into y; advances cache2."""
        L.wvc_resblock_back(h2, x, self.p, self.c2.cin, self.c2.cout, y=y, eps=self.eps,
                            workspace=self._half_ws("ws_back", x), packed=self.packed)
        self.c2.flip()
        return y

    def stages(self, x: torch.Tensor, y: torch.Tensor, buf) -> List[Callable[[], object]]:
        """The chunk as two stages (front, back); ``buf(name, shape, like)``
        supplies the intermediate h2."""
        shape = (x.shape[0], self.p["w1"].shape[0]) + tuple(x.shape[2:])
        h2 = buf("h2", shape, x)
        return [lambda: self.front(x, h2), lambda: self.back(h2, x, y)]


class CausalConv3dE4M3:
    """A causal 3x3x3 conv on the 8-bit path whose input is not a norm output
    (the decoder's conv_in and conv_up): the bf16 chunk is quantised at the
    activation scale ``scale`` (``wvc_quantize_e4m3``), then the 8-bit conv
    runs on the codes with its code cache; the output is bf16."""

    def __init__(self, weight: torch.Tensor, bias: Optional[torch.Tensor], scale: float):
        self.weight, self.bias, self.scale = weight, bias, float(scale)
        self.wq, self.wsc = L.wvc_quantize_rows_e4m3(weight)
        self.packed = L.wvc_conv3d_pack_weights(self.wq)
        self.cache: Optional[_PingPong] = None
        self.bufs: Dict[str, torch.Tensor] = {}
        self.ws: Optional[torch.Tensor] = None

    def start(self, n: int, h: int, w: int):
        shape = (n, self.weight.shape[1], CACHE_T, h, w)
        if self.cache is None or tuple(self.cache.buf[0].shape) != shape:
            self.cache = _PingPong(shape, torch.uint8, self.weight.device)
        else:
            self.cache.reset()

    def reset(self):
        if self.cache is not None:
            self.cache.reset()

    def pingpongs(self) -> List[_PingPong]:
        return [self.cache] if self.cache is not None else []

    def caches(self) -> List[torch.Tensor]:
        if self.cache is None:
            return []
        self.cache.materialize()
        return [self.cache.cin]

    def __call__(self, x: torch.Tensor, y: Optional[torch.Tensor] = None) -> torch.Tensor:
        if self.cache is None:
            self.start(x.shape[0], x.shape[3], x.shape[4])
        q = _cached_buf(self.bufs, "q", x.shape, x.new_empty(0, dtype=torch.uint8))
        L.wvc_quantize_e4m3(x, self.scale, q=q)
        d = L.conv_desc(tuple(q.shape), tuple(self.wq.shape), L.WVC_E4M3, weight_layout=L.WVC_WEIGHT_PACKED)
        need = L.wvc_causal_conv3d_workspace_bytes(d)
        if need and (self.ws is None or self.ws.numel() < need):
            self.ws = torch.empty(need, dtype=torch.uint8, device=x.device)
        y = L.wvc_causal_conv3d_e4m3_fwd(q, self.scale, self.wq, self.wsc, self.bias, self.cache.cin,
                                         self.cache.cout, None, y, workspace=self.ws if need else None,
                                         packed_weight=self.packed)
        self.cache.flip()
        return y

    def stages(self, x: torch.Tensor, y: torch.Tensor, buf) -> List[Callable[[], object]]:
        return [lambda: self(x, y=y)]


class ResBlockE4M3:
    """The residual block on the 8-bit path (identity shortcut, C_in == C_out),
    one ``wvc_resblock_e4m3_fwd`` call per chunk: norm1 + SiLU stored as E4M3
    codes at activation scale s1, the 8-bit conv1, norm2 + SiLU as codes at s2
    (fed straight from conv1's split-K partial sums), the 8-bit conv2 plus the
    block input.  The weights are quantised once on the GPU, one scale per
    output channel, and packed; the caches hold codes.  The activation scales
    are the caller's calibration constants."""

    def __init__(self, params: Dict[str, torch.Tensor], s1: float, s2: float, eps: float = 1e-12):
        if params["w1"].shape[0] != params["w1"].shape[1] or params.get("w_short") is not None:
            raise ValueError("ResBlockE4M3 covers the identity-shortcut block (C_in == C_out)")
        self.p, self.s1, self.s2, self.eps = params, float(s1), float(s2), eps
        self.w = {}
        for k in ("w1", "w2"):
            q, sc = L.wvc_quantize_rows_e4m3(params[k])
            self.w[k] = (q, sc, L.wvc_conv3d_pack_weights(q))
        self.q8 = {"gamma1": params["gamma1"], "beta1": params.get("beta1"),
                   "gamma2": params["gamma2"], "beta2": params.get("beta2"),
                   "b1": params.get("b1"), "b2": params.get("b2"),
                   "w1": self.w["w1"][2], "w1_scale": self.w["w1"][1],
                   "w2": self.w["w2"][2], "w2_scale": self.w["w2"][1]}
        self.c1: Optional[_PingPong] = None
        self.c2: Optional[_PingPong] = None
        self.ws: Optional[torch.Tensor] = None

    def start(self, n: int, h: int, w: int):
        c = self.p["w1"].shape[0]
        shape = (n, c, CACHE_T, h, w)
        if self.c1 is not None and tuple(self.c1.buf[0].shape) == shape:
            self.reset()
            return
        dev = self.p["w1"].device
        self.c1 = _PingPong(shape, torch.uint8, dev)
        self.c2 = _PingPong(shape, torch.uint8, dev)

    def reset(self):
        if self.c1 is not None:
            self.c1.reset()
            self.c2.reset()

    def pingpongs(self) -> List[_PingPong]:
        return [self.c1, self.c2] if self.c1 is not None else []

    def caches(self) -> List[torch.Tensor]:
        if self.c1 is None:
            return []
        self.c1.materialize()
        self.c2.materialize()
        return [self.c1.cin, self.c2.cin]

    def __call__(self, x: torch.Tensor, y: Optional[torch.Tensor] = None) -> torch.Tensor:
        if self.c1 is None:
            self.start(x.shape[0], x.shape[3], x.shape[4])
        d = L.resblock_desc(tuple(x.shape), x.shape[1], L.WVC_BF16, self.eps, weights_packed=True)
        need = L.wvc_resblock_e4m3_workspace_bytes(d)
        if self.ws is None or self.ws.numel() < need:
            self.ws = torch.empty(max(1, need), dtype=torch.uint8, device=x.device)
        y = L.wvc_resblock_e4m3_fwd(x, self.q8, self.s1, self.s2, self.c1.cin, self.c1.cout,
                                    self.c2.cin, self.c2.cout, y=y, eps=self.eps, workspace=self.ws,
                                    packed=True)
        self.c1.flip()
        self.c2.flip()
        return y

    def stages(self, x: torch.Tensor, y: torch.Tensor, buf) -> List[Callable[[], object]]:
        return [lambda: self(x, y=y)]


class Stream:
    """Runs a sequence of layers over a latent sequence chunk by chunk."""

    def __init__(self, layers: Sequence):
        self.layers = list(layers)

    def _cache_layers(self):
        return [l for l in self.layers if hasattr(l, "caches")]

    def state(self) -> List[torch.Tensor]:
        """Copies of every cache (the complete resumable state)."""
        return [c.clone() for l in self._cache_layers() for c in l.caches()]

    def load_state(self, saved: List[torch.Tensor]):
        it = iter(saved)
        for l in self._cache_layers():
            for c in l.caches():
                c.copy_(next(it))

    def reset(self):
        """Zero every cache in place (a new sequence)."""
        for l in self._cache_layers():
            l.reset()

    def pingpongs(self) -> List[_PingPong]:
        return [pp for l in self._cache_layers() for pp in l.pingpongs()]


class DecoderStack(Stream):
    """Decoder-shaped stack: conv_in (C_lat -> C) -> 2 resblocks -> nearest 2x
    upsample -> conv_up (C -> C) -> 2 resblocks, streamed chunk by chunk with one
    2-frame cache per 3x3x3 conv (10 caches for 4 resblocks)."""

    # Pipeline cut: conv_in, both low-resolution blocks and the upsample on
    # one stream; conv_up and the two full-resolution blocks on the other.
    # The low-resolution convs fill fewer workgroups than there are CUs, and
    # the other stream's convs use the rest.
    PIPELINE_SPLIT = 6

    def __init__(self, p: Dict, eps: float = 1e-12):
        self.conv_in = CausalConv3d(p["w_in"], p.get("b_in"))
        self.rbs = [ResBlock(p[f"rb{k}"], eps) for k in range(4)]
        self.conv_up = CausalConv3d(p["w_up"], p.get("b_up"))
        super().__init__([self.conv_in] + self.rbs[:2] + [self.conv_up] + self.rbs[2:])

    def start(self, n: int, h: int, w: int):
        self.conv_in.start(n, h, w)
        for rb in self.rbs[:2]:
            rb.start(n, h, w)
        self.conv_up.start(n, 2 * h, 2 * w)
        for rb in self.rbs[2:]:
            rb.start(n, 2 * h, 2 * w)

    def _buf(self, name: str, shape, like: torch.Tensor) -> torch.Tensor:
        """Intermediate activation buffer, reused from chunk to chunk (so a
        recorded graph names the same memory every time)."""
        return _cached_buf(self.__dict__.setdefault("_bufs", {}), name, shape, like)

    def stages(self, x: torch.Tensor, out: torch.Tensor, buf) -> List[Callable[[], object]]:
        """The chunk as a list of stages (each a few library calls); the
        intermediates come from ``buf(name, shape, like)``."""
        n, _, t, h, w = x.shape
        c = self.conv_in.weight.shape[0]
        lo, hi = (n, c, t, h, w), (n, c, t, 2 * h, 2 * w)
        a_in, a0, a1 = buf("in", lo, x), buf("rb0", lo, x), buf("rb1", lo, x)
        up, a_up, a2 = buf("up", hi, x), buf("conv_up", hi, x), buf("rb2", hi, x)

        def sub(k):
            return lambda name, shape, like: buf(f"rb{k}.{name}", shape, like)

        st = self.conv_in.stages(x, a_in, buf)
        st += self.rbs[0].stages(a_in, a0, sub(0))
        st += self.rbs[1].stages(a0, a1, sub(1))
        st.append(lambda: L.wvc_upsample_nearest2x(a1, y=up))
        st += self.conv_up.stages(up, a_up, buf)
        st += self.rbs[2].stages(a_up, a2, sub(2))
        st += self.rbs[3].stages(a2, out, sub(3))
        return st

    def chunk(self, x: torch.Tensor, out: Optional[torch.Tensor] = None) -> torch.Tensor:
        if out is None:
            n, _, t, h, w = x.shape
            out = L.empty_cl((n, self.conv_up.weight.shape[0], t, 2 * h, 2 * w), x.dtype, x.device)
        for stage in self.stages(x, out, self._buf):
            stage()
        return out

    def run(self, latent: torch.Tensor, chunk_frames: int = 1) -> torch.Tensor:
        n, c, t, h, w = latent.shape
        self.start(n, h, w)
        width = self.conv_up.weight.shape[0]
        out = L.empty_cl((n, width, t, 2 * h, 2 * w), latent.dtype, latent.device)
        for t0 in range(0, t, chunk_frames):
            t1 = min(t, t0 + chunk_frames)
            x = latent[:, :, t0:t1]
            if not x.is_contiguous(memory_format=torch.channels_last_3d):
                x = x.contiguous(memory_format=torch.channels_last_3d)
            y = self.chunk(x)
            out[:, :, t0:t1].copy_(y)
        return out


class DecoderStackE4M3(DecoderStack):
    """The decoder-shaped stack on the 8-bit path: conv_in and conv_up quantise
    their bf16 inputs at the activation scales ``scales["in"]`` and
    ``scales["up"]``; each residual block k quantises its two norm outputs at
    ``scales["rb"][k]`` = (s1, s2).  Activations between layers stay bf16."""

    # conv_in, rb0, rb1 and the upsample on one stream; the rest on the other
    PIPELINE_SPLIT = 4

    def __init__(self, p: Dict, scales: Dict, eps: float = 1e-12):
        self.conv_in = CausalConv3dE4M3(p["w_in"], p.get("b_in"), scales["in"])
        self.rbs = [ResBlockE4M3(p[f"rb{k}"], *scales["rb"][k], eps) for k in range(4)]
        self.conv_up = CausalConv3dE4M3(p["w_up"], p.get("b_up"), scales["up"])
        Stream.__init__(self, [self.conv_in] + self.rbs[:2] + [self.conv_up] + self.rbs[2:])


def run_chunked(layer, x: torch.Tensor, sizes: Sequence[int]) -> torch.Tensor:
    """Run one cached layer (CausalConv3d or ResBlock) over ``x`` in chunks of
    the given frame counts, from a fresh (zero) cache."""
    n, c, t, h, w = x.shape
    assert sum(sizes) == t
    layer.start(n, h, w)
    outs = []
    t0 = 0
    for s in sizes:
        chunk = x[:, :, t0:t0 + s].contiguous(memory_format=torch.channels_last_3d)
        outs.append(layer(chunk))
        t0 += s
    return torch.cat(outs, dim=2).contiguous(memory_format=torch.channels_last_3d)


def capture(fn: Callable[[], object], device=None) -> L.Graph:
    """Record the library calls that ``fn()`` enqueues into a HIP graph.

    ``fn`` runs once on a side stream under capture: its calls are recorded,
    not run, so it must only make library calls on buffers that already exist
    (run it eagerly once first, so that every workspace and intermediate is
    allocated).  Python state that ``fn`` changes (e.g. the cache parity) is
    changed as if it had run."""
    dev = torch.device("cuda", torch.cuda.current_device()) if device is None else torch.device(device)
    side = torch.cuda.Stream(dev)
    side.wait_stream(torch.cuda.current_stream(dev))
    with torch.cuda.stream(side):
        L.wvc_graph_capture_begin(side)
        try:
            fn()
        except BaseException:
            try:
                L.wvc_graph_capture_end(side).close()
            except Exception:
                pass
            raise
        graph = L.wvc_graph_capture_end(side)
    torch.cuda.current_stream(dev).wait_stream(side)
    return graph


class FrameGraph:
    """One chunk of a streamed stack (``DecoderStack``, ``ResBlock`` or
    ``CausalConv3d``) replayed as a HIP graph.

    Chunk i reads the caches chunk i-1 wrote, so even and odd chunks name the
    two buffers of every ping-pong the other way round: two graphs are
    recorded, one per parity.  ``x`` and ``y`` are the static input and output
    chunk buffers they read and write: fill ``x``, call, read ``y`` before the
    next call.  ``reset()`` starts a new sequence."""

    def __init__(self, stack, x_shape: Sequence[int], dtype=torch.bfloat16, device="cuda"):
        n, c, t, h, w = x_shape
        self.stack = stack
        self._run = stack.chunk if hasattr(stack, "chunk") else \
            (lambda x, out=None: stack(x, y=out))
        self.x = L.empty_cl(tuple(x_shape), dtype, device)
        L.wvc_cache_reset(self.x)
        stack.start(n, h, w)
        y = self._run(self.x)          # eager pass: sizes every workspace and buffer
        self.y = L.empty_cl(tuple(y.shape), dtype, device)
        self._pps = stack.pingpongs()
        self.reset()   # the recorded calls must name the cache buffers, not NULL
        self.graphs = [capture(lambda: self._run(self.x, out=self.y), device) for _ in range(2)]
        # each recording flipped every cache once, so the parity is back to 0
        self.parity = 0

    def reset(self):
        self.stack.reset()
        for pp in self._pps:
            pp.materialize()
        self.parity = 0

    def __call__(self) -> torch.Tensor:
        self.graphs[self.parity].launch()
        for pp in self._pps:        # the stack's ping-pong state follows the replay
            pp.flip()
        self.parity ^= 1
        return self.y

    def close(self):
        for g in self.graphs:
            g.close()



class Pipeline:
    """Streams a stack over a sequence of chunks on two HIP streams.

    A chunk is a list of stages (``stack.stages``).  Stages [0, split) of every
    chunk run in order on stream A, stages [split, n) on stream B; B starts a
    chunk once A has finished that chunk's first part (one event per chunk).
    A stage touches the caches and workspace of its own layer only, and a
    layer's stages all sit on one side of the split (a residual block may be
    cut between its halves: they use different caches and workspaces), so
    each stream runs its layers in chunk order exactly as the sequential loop
    does, and the second part of chunk i runs next to the first part of chunk
    i+1 (for a residual block: conv2 of frame i next to conv1 of frame i+1).
    The intermediates live in ``slots`` buffer sets used round robin; A waits
    before reusing a set until B is done with the chunk that used it last.
    Every call is the one ``stack.chunk`` makes, so the outputs are bitwise
    equal to the sequential loop.
    """

    def __init__(self, stack, split: Optional[int] = None, slots: int = 3, device=None):
        self.stack = stack
        self.split = split if split is not None else getattr(stack, "PIPELINE_SPLIT", 1)
        self.slots = slots
        dev = torch.device("cuda", torch.cuda.current_device()) if device is None else torch.device(device)
        self.device = dev
        self.streams = [torch.cuda.Stream(dev), torch.cuda.Stream(dev)]
        self._bufs = [{} for _ in range(slots)]
        self._ev_a = [torch.cuda.Event() for _ in range(slots)]
        self._ev_b = [torch.cuda.Event() for _ in range(slots)]

    def _buf(self, slot: int):
        bufs = self._bufs[slot]

        def get(name, shape, like):
            b = bufs.get(name)
            if b is None or tuple(b.shape) != tuple(shape) or b.dtype != like.dtype:
                b = _cached_buf(bufs, name, shape, like)
                for s in self.streams:
                    b.record_stream(s)
            return b
        return get

    def run(self, chunks: Sequence[torch.Tensor], outs: Sequence[torch.Tensor]):
        """Run every chunk in order (chunks[i] -> outs[i]) from the stack's
        current cache state.  The work goes to the two streams; the current
        stream waits for all of it before this returns."""
        if torch.cuda.is_current_stream_capturing():
            # Recording a two-stream fork/join into a graph crashed the HIP
            # runtime inside end-capture; graphs record single-stream work.
            raise RuntimeError("Pipeline.run cannot be recorded into a graph; record the "
                               "sequential chunk loop (or FrameGraph) instead")
        main = torch.cuda.current_stream(self.device)
        sa, sb = self.streams
        sa.wait_stream(main)
        sb.wait_stream(main)
        for i, (x, y) in enumerate(zip(chunks, outs)):
            slot = i % self.slots
            stages = self.stack.stages(x, y, self._buf(slot))
            if not 0 < self.split < len(stages):
                raise ValueError(f"split {self.split} must cut the {len(stages)} stages in two")
            with torch.cuda.stream(sa):
                if i >= self.slots:
                    sa.wait_event(self._ev_b[slot])   # B is done with this buffer set
                for stage in stages[:self.split]:
                    stage()
                self._ev_a[slot].record(sa)
            with torch.cuda.stream(sb):
                sb.wait_event(self._ev_a[slot])
                for stage in stages[self.split:]:
                    stage()
                self._ev_b[slot].record(sb)
            x.record_stream(sa)
            x.record_stream(sb)
            y.record_stream(sb)
        main.wait_stream(sa)
        main.wait_stream(sb)


def tile_origins(size: int, tile: int, stride: int) -> List[int]:
    """Tile starts along one axis: 0, stride, 2*stride, ... while the tile
    fits, plus one tile aligned to the far edge if the last stops short; a
    frame no larger than the tile is one tile."""
    if size <= tile:
        return [0]
    if not 0 < stride <= tile:
        raise ValueError("the stride must lie in (0, tile]: larger strides leave gaps")
    starts = list(range(0, size - tile + 1, stride))
    if starts[-1] + tile < size:
        starts.append(size - tile)
    return starts


class TiledDecode:
    """Decode a latent in overlapping spatial tiles and blend them ("VSR
    Hover Comparison", decoder tiling: (60, 104) tiles at stride (30, 52) of
    the latent, fused with complementary linear ramps).

    Each tile is cut out of the latent (wvc_tile_extract), decoded through
    ``stack`` over all frames from zero caches, and blended into an fp32
    accumulator (wvc_tile_blend) with ramps over its overlaps with its
    neighbours; wvc_tile_blend_finish divides by the weight sum and rounds
    once.  ``scale`` is the stack's spatial upsampling factor (2 for the
    decoder stack).  Smaller overlaps decode fewer latent pixels; the page
    measures that trade."""

    def __init__(self, stack, tile=(60, 104), stride=(30, 52), scale: int = 2):
        self.stack = stack
        self.tile = tuple(tile)
        self.stride = tuple(stride)
        self.scale = scale

    def origins(self, h: int, w: int):
        th, tw = min(self.tile[0], h), min(self.tile[1], w)
        return th, tw, tile_origins(h, th, self.stride[0]), tile_origins(w, tw, self.stride[1])

    def run(self, latent: torch.Tensor, chunk_frames: int = 1) -> torch.Tensor:
        n, c, t, h, w = latent.shape
        th, tw, ys, xs = self.origins(h, w)
        s = self.scale
        acc = wsum = None
        for iy, y0 in enumerate(ys):
            for ix, x0 in enumerate(xs):
                tile = L.wvc_tile_extract(latent, y0, x0, th, tw)
                out = self.stack.run(tile, chunk_frames=chunk_frames)
                if acc is None:
                    acc, wsum = L.blend_accumulators(out, s * h, s * w)
                oh, ow = out.shape[3:]
                top = s * (ys[iy - 1] + th - y0) if iy > 0 else 0
                bottom = s * (y0 + th - ys[iy + 1]) if iy + 1 < len(ys) else 0
                left = s * (xs[ix - 1] + tw - x0) if ix > 0 else 0
                right = s * (x0 + tw - xs[ix + 1]) if ix + 1 < len(xs) else 0
                L.wvc_tile_blend(out, acc, wsum, s * y0, s * x0, (top, bottom, left, right))
        return L.wvc_tile_blend_finish(acc, wsum, latent.dtype)
