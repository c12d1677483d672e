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


def _norm_workspace(ws: Optional[torch.Tensor], x: torch.Tensor, weight: torch.Tensor, padding,
                    packed: Optional[torch.Tensor], upsample_in: int = 0,
                    cu_limit: int = 0) -> torch.Tensor:
    """A workspace for wvc_causal_conv3d_norm_fwd on chunks of x's shape:
    ``ws`` when it is large enough, else a new one."""
    layout = L.WVC_WEIGHT_PACKED if packed is not None else L.WVC_WEIGHT_STANDARD
    need = L._norm_ws_shared(tuple(x.shape), tuple(weight.shape), L._dtype_code(x.dtype),
                             tuple(padding), layout, x.device, upsample_in, cu_limit)
    if ws is None or ws.numel() < need:
        ws = torch.empty(max(need, 1), dtype=torch.uint8, device=x.device)
    return ws


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

    def fits(self, shape) -> bool:
        return tuple(self.buf[0].shape) == tuple(shape)


def _fits(pp: Optional[_PingPong], shape) -> bool:
    """Whether a layer's cache pair serves a chunk of this batch and frame
    size.  A chunk of another size cannot continue the stream: the layer
    starts a new sequence (fresh caches of the new size) instead of letting
    the library write full-size cache frames into a smaller buffer."""
    return pp is not None and pp.fits(shape)


class CausalConv3d:
    """A causal 3x3x3 conv layer with its rolling 2-frame cache.  With
    ``upsample_in`` = 2 the layer is the decoder's nearest 2x upsample and the
    conv after it in one call: it takes chunks of h x w frames, caches them at
    that size and returns frames of 2h x 2w."""

    def __init__(self, weight: torch.Tensor, bias: Optional[torch.Tensor], upsample_in: int = 0):
        self.weight = weight
        self.bias = bias
        self.upsample_in = upsample_in
        self.cu_limit = 0   # > 0: plan the conv's grid for that many CUs (see set_cu_limit)
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
        n, c, _, h, w = x.shape
        if self.frames and not _fits(self.cache, (n, c, self.frames, h, w)):
            self.start(n, h, w)
        cin = self.cache.cin if self.frames else None
        cout = self.cache.cout if self.frames else None
        need = self._ws_need(x)
        if need and (self.ws is None or self.ws.numel() < need):
            self.ws = torch.empty(need, dtype=torch.uint8, device=x.device)
        y = L.wvc_causal_conv3d_fwd(x, self.weight, self.bias, cin, cout, residual, y,
                                    padding=self.padding, workspace=self.ws if need else None,
                                    packed_weight=self.packed, upsample_in=self.upsample_in,
                                    cu_limit=self.cu_limit)
        if self.frames:
            self.cache.flip()
        return y

    def norm_into(self, x: torch.Tensor, y: Optional[torch.Tensor], gamma: torch.Tensor,
                  beta: Optional[torch.Tensor], eps: float, h: torch.Tensor,
                  residual: Optional[torch.Tensor] = None) -> torch.Tensor:
        """The conv into y (skipped when None) and the RMS norm + SiLU of the
        layer it feeds into h, as one library call (wvc_causal_conv3d_norm_fwd:
        a split-K conv's reduce runs inside the norm kernel)."""
        n, c, _, hh, ww = x.shape
        if self.frames and not _fits(self.cache, (n, c, self.frames, hh, ww)):
            self.start(n, hh, ww)
        cin = self.cache.cin if self.frames else None
        cout = self.cache.cout if self.frames else None
        self.nws = _norm_workspace(self.__dict__.get("nws"), x, self.weight, self.padding, self.packed,
                                   self.upsample_in, self.cu_limit)
        L.wvc_causal_conv3d_norm_fwd(x, self.weight, gamma, self.bias, beta, eps, cin, cout, residual,
                                     y, h, padding=self.padding, workspace=self.nws,
                                     packed_weight=self.packed, upsample_in=self.upsample_in,
                                     cu_limit=self.cu_limit)
        if self.frames:
            self.cache.flip()
        return h

    def _ws_need(self, x: torch.Tensor) -> int:
        """Workspace bytes of a chunk of x's shape (asked once per shape)."""
        key = (x.shape, x.dtype, x.device, self.cu_limit)
        need = self.__dict__.setdefault("_needs", {}).get(key)
        if need is None:
            layout = L.WVC_WEIGHT_PACKED if self.packed is not None else L.WVC_WEIGHT_STANDARD
            d = L.conv_desc(tuple(x.shape), tuple(self.weight.shape), L._dtype_code(x.dtype),
                            padding=self.padding, weight_layout=layout, upsample_in=self.upsample_in,
                            cu_limit=self.cu_limit)
            need = self._needs[key] = L.wvc_causal_conv3d_workspace_bytes(d)
        return need

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
        self.cu_limit = 0   # > 0: plan the convs' grids for that many CUs
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

    def _ensure(self, x: torch.Tensor):
        n, c, _, h, w = x.shape
        if not _fits(self.c1, (n, c, CACHE_T, h, w)):
            self.start(n, h, w)

    def _ws_need(self, x: torch.Tensor) -> int:
        """Workspace bytes of a chunk of x's shape (asked once per shape)."""
        key = (x.shape, x.dtype, x.device, self.cu_limit)
        need = self.__dict__.setdefault("_needs", {}).get(key)
        if need is None:
            d = L.resblock_desc(tuple(x.shape), self.p["w1"].shape[0], L._dtype_code(x.dtype),
                                self.eps, weights_packed=self.packed is not None,
                                cu_limit=self.cu_limit)
            need = self._needs[key] = L.wvc_resblock_workspace_bytes(d)
        return need

    def __call__(self, x: torch.Tensor, y: Optional[torch.Tensor] = None) -> torch.Tensor:
        self._ensure(x)
        need = self._ws_need(x)
        if self.ws is None or self.ws.numel() < need:
            self.ws = torch.empty(need, dtype=torch.uint8, device=x.device)
        y = L.wvc_resblock_fwd(x, self.p, self.c1.cin, self.c1.cout, self.c2.cin, self.c2.cout,
                               y=y, eps=self.eps, workspace=self.ws, packed=self.packed,
                               cu_limit=self.cu_limit)
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
        need = self._ws_need(x)
        ws = self.__dict__.get(name)
        if ws is None or ws.numel() < need:
            ws = torch.empty(need, dtype=torch.uint8, device=x.device)
            setattr(self, name, ws)
        return ws

    def front(self, x: torch.Tensor, h2: torch.Tensor) -> torch.Tensor:
        """First half (norm1, conv1, norm2) into h2; advances cache1."""
        self._ensure(x)
        L.wvc_resblock_front(x, self.p, self.c1.cin, self.c1.cout, h2=h2, eps=self.eps,
                             workspace=self._half_ws("ws_front", x), packed=self.packed,
                             cu_limit=self.cu_limit)
        self.c1.flip()
        return h2

    def back(self, h2: torch.Tensor, x: torch.Tensor, y: torch.Tensor) -> torch.Tensor:
        """Second half (conv2 + shortcut) into y; advances cache2."""
        n, _, _, h, w = x.shape
        if not _fits(self.c2, (n, self.p["w1"].shape[0], CACHE_T, h, w)):
            raise ValueError("back() of a chunk whose front() ran at another size")
        L.wvc_resblock_back(h2, x, self.p, self.c2.cin, self.c2.cout, y=y, eps=self.eps,
                            workspace=self._half_ws("ws_back", x), packed=self.packed,
                            cu_limit=self.cu_limit)
        self.c2.flip()
        return y

    def front_from_h1(self, h1: torch.Tensor, h2: torch.Tensor) -> torch.Tensor:
        """First half given h1 = SiLU(norm1(x)), computed by the layer before
        (wvc_causal_conv3d_norm_fwd): conv1 + norm2 into h2; advances cache1."""
        self._ensure(h1)
        p, pk = self.p, self.packed
        self.ws_f1 = _norm_workspace(self.__dict__.get("ws_f1"), h1, p["w1"], (1, 1),
                                     None if pk is None else pk["w1"], cu_limit=self.cu_limit)
        L.wvc_causal_conv3d_norm_fwd(h1, p["w1"], p["gamma2"], p.get("b1"), p.get("beta2"), self.eps,
                                     self.c1.cin, self.c1.cout, None, None, h2, workspace=self.ws_f1,
                                     packed_weight=None if pk is None else pk["w1"],
                                     cu_limit=self.cu_limit)
        self.c1.flip()
        return h2

    def back_norm(self, h2: torch.Tensor, x: torch.Tensor, y: torch.Tensor, gamma: torch.Tensor,
                  beta: Optional[torch.Tensor], eps: float, h_next: torch.Tensor) -> torch.Tensor:
        """Second half of an identity-shortcut block, y = conv2(h2) + x, and the
        next block's norm1 + SiLU of y into h_next, in one library call;
        advances cache2."""
        if self.p.get("w_short") is not None:
            raise ValueError("back_norm covers the identity-shortcut block")
        n, _, _, hh, ww = x.shape
        if not _fits(self.c2, (n, self.p["w1"].shape[0], CACHE_T, hh, ww)):
            raise ValueError("back_norm() of a chunk whose front ran at another size")
        p, pk = self.p, self.packed
        self.ws_b1 = _norm_workspace(self.__dict__.get("ws_b1"), h2, p["w2"], (1, 1),
                                     None if pk is None else pk["w2"], cu_limit=self.cu_limit)
        L.wvc_causal_conv3d_norm_fwd(h2, p["w2"], gamma, p.get("b2"), beta, eps, self.c2.cin,
                                     self.c2.cout, x, y, h_next, workspace=self.ws_b1,
                                     packed_weight=None if pk is None else pk["w2"],
                                     cu_limit=self.cu_limit)
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
    runs on the codes with its code cache; the output is bf16.  With
    ``upsample_in`` = 2 the conv reads the codes through the nearest 2x
    upsample (the quantiser is elementwise, so quantising before the upsample
    gives the same codes), and the chunk and cache keep the small frame."""

    def __init__(self, weight: torch.Tensor, bias: Optional[torch.Tensor], scale: float,
                 upsample_in: int = 0):
        self.weight, self.bias, self.scale = weight, bias, float(scale)
        self.upsample_in = upsample_in
        self.cu_limit = 0   # > 0: plan the conv's grid for that many CUs
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
        n, c, _, h, w = x.shape
        if not _fits(self.cache, (n, c, CACHE_T, h, w)):
            self.start(n, h, w)
        q = _cached_buf(self.bufs, "q", x.shape, x.new_empty(0, dtype=torch.uint8))
        L.wvc_quantize_e4m3(x, self.scale, q=q)
        d = L.conv_desc(tuple(q.shape), tuple(self.wq.shape), L.WVC_E4M3, weight_layout=L.WVC_WEIGHT_PACKED,
                        upsample_in=self.upsample_in, cu_limit=self.cu_limit)
        need = L.wvc_causal_conv3d_workspace_bytes(d)
        if need and (self.ws is None or self.ws.numel() < need):
            self.ws = torch.empty(need, dtype=torch.uint8, device=x.device)
        y = L.wvc_causal_conv3d_e4m3_fwd(q, self.scale, self.wq, self.wsc, self.bias, self.cache.cin,
                                         self.cache.cout, None, y, workspace=self.ws if need else None,
                                         packed_weight=self.packed, upsample_in=self.upsample_in,
                                         cu_limit=self.cu_limit)
        self.cache.flip()
        return y

    def norm_into(self, x: torch.Tensor, y: Optional[torch.Tensor], gamma: torch.Tensor,
                  beta: Optional[torch.Tensor], eps: float, q_scale: float, q: torch.Tensor) -> torch.Tensor:
        """This conv on the chunk, then the next layer's norm + SiLU stored as
        codes at ``q_scale`` in ``q`` (one wvc_causal_conv3d_e4m3_norm_fwd
        call after the quantiser); the conv's bf16 output goes to ``y`` when
        given (a block's shortcut needs it)."""
        n, c, _, h, w = x.shape
        if not _fits(self.cache, (n, c, CACHE_T, h, w)):
            self.start(n, h, w)
        qx = _cached_buf(self.bufs, "q", x.shape, x.new_empty(0, dtype=torch.uint8))
        L.wvc_quantize_e4m3(x, self.scale, q=qx)
        d = L.conv_desc(tuple(qx.shape), tuple(self.wq.shape), L.WVC_E4M3, weight_layout=L.WVC_WEIGHT_PACKED,
                        upsample_in=self.upsample_in, cu_limit=self.cu_limit)
        need = L.wvc_causal_conv3d_e4m3_norm_workspace_bytes(d)
        ws = self.__dict__.get("ws_n")
        if ws is None or ws.numel() < need:
            ws = self.ws_n = torch.empty(max(1, need), dtype=torch.uint8, device=x.device)
        L.wvc_causal_conv3d_e4m3_norm_fwd(qx, self.scale, self.wq, self.wsc, gamma, q_scale, self.bias, beta,
                                          eps, self.cache.cin, self.cache.cout, None, y, q, workspace=ws,
                                          packed_weight=self.packed, upsample_in=self.upsample_in,
                                          cu_limit=self.cu_limit)
        self.cache.flip()
        return q

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
        self.cu_limit = 0   # > 0: plan the convs' grids for that many CUs

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
        n, c, _, h, w = x.shape
        if not _fits(self.c1, (n, c, CACHE_T, h, w)):
            self.start(n, h, w)
        d = L.resblock_desc(tuple(x.shape), x.shape[1], L.WVC_BF16, self.eps, weights_packed=True,
                            cu_limit=self.cu_limit)
        need = L.wvc_resblock_e4m3_workspace_bytes(d)
        if self.ws is None or self.ws.numel() < need:
            self.ws = torch.empty(max(1, need), dtype=torch.uint8, device=x.device)
        y = L.wvc_resblock_e4m3_fwd(x, self.q8, self.s1, self.s2, self.c1.cin, self.c1.cout,
                                    self.c2.cin, self.c2.cout, y=y, eps=self.eps, workspace=self.ws,
                                    packed=True, cu_limit=self.cu_limit)
        self.c1.flip()
        self.c2.flip()
        return y

    def _ws8(self, name: str, q: torch.Tensor, norm: bool) -> torch.Tensor:
        d = L.conv_desc(tuple(q.shape), tuple(self.w["w1"][0].shape), L.WVC_E4M3,
                        weight_layout=L.WVC_WEIGHT_PACKED, cu_limit=self.cu_limit)
        need = (L.wvc_causal_conv3d_e4m3_norm_workspace_bytes(d) if norm
                else L.wvc_causal_conv3d_workspace_bytes(d))
        ws = self.__dict__.get(name)
        if ws is None or ws.numel() < need:
            ws = torch.empty(max(1, need), dtype=torch.uint8, device=q.device)
            setattr(self, name, ws)
        return ws

    def front_from_q1(self, q1: torch.Tensor, q2: torch.Tensor) -> torch.Tensor:
        """The block's first half from the codes of norm1(x) (at scale s1),
        which the previous layer's conv + norm call wrote: conv1, then norm2 +
        SiLU as codes at s2 in ``q2``; the calls the block call makes after
        its norm1."""
        n, c, _, h, w = q1.shape
        if not _fits(self.c1, (n, c, CACHE_T, h, w)):
            self.start(n, h, w)
        wq, sc, pk = self.w["w1"]
        L.wvc_causal_conv3d_e4m3_norm_fwd(q1, self.s1, wq, sc, self.p["gamma2"], self.s2, self.p.get("b1"),
                                          self.p.get("beta2"), self.eps, self.c1.cin, self.c1.cout, q=q2,
                                          workspace=self._ws8("ws_f8", q1, True), packed_weight=pk,
                                          cu_limit=self.cu_limit)
        self.c1.flip()
        return q2

    def back(self, q2: torch.Tensor, x: torch.Tensor, y: torch.Tensor) -> torch.Tensor:
        """conv2 on the codes of norm2 plus the shortcut x into y."""
        wq, sc, pk = self.w["w2"]
        L.wvc_causal_conv3d_e4m3_fwd(q2, self.s2, wq, sc, self.p.get("b2"), self.c2.cin, self.c2.cout, x, y,
                                     workspace=self._ws8("ws_b8", q2, False), packed_weight=pk,
                                     cu_limit=self.cu_limit)
        self.c2.flip()
        return y

    def back_norm(self, q2: torch.Tensor, x: torch.Tensor, y: torch.Tensor, gamma: torch.Tensor,
                  beta: Optional[torch.Tensor], eps: float, q_scale: float, q_next: torch.Tensor) -> torch.Tensor:
        """conv2 plus the shortcut into y, and the next block's norm1 + SiLU
        as codes at ``q_scale`` in ``q_next``, in one conv + norm call."""
        wq, sc, pk = self.w["w2"]
        L.wvc_causal_conv3d_e4m3_norm_fwd(q2, self.s2, wq, sc, gamma, q_scale, self.p.get("b2"), beta, eps,
                                          self.c2.cin, self.c2.cout, x, y, q_next,
                                          workspace=self._ws8("ws_bn8", q2, True), packed_weight=pk,
                                          cu_limit=self.cu_limit)
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
    2-frame cache per 3x3x3 conv (10 caches for 4 resblocks).  The upsample is
    read inside conv_up (upsample_in = 2): the upsampled frames never reach
    memory, and conv_up caches its input frames before the upsample."""

    # Pipeline cut: conv_in and both low-resolution blocks on one stream;
    # conv_up (reading through the upsample) and the two full-resolution
    # blocks on the other.  The low-resolution convs fill fewer workgroups
    # than there are CUs, and the other stream's convs use the rest.
    PIPELINE_SPLIT = 5

    def __init__(self, p: Dict, eps: float = 1e-12):
        self.conv_in = CausalConv3d(p["w_in"], p.get("b_in"))
        self.rbs = [ResBlock(p[f"rb{k}"], eps) for k in range(4)]
        self.conv_up = CausalConv3d(p["w_up"], p.get("b_up"), upsample_in=2)
        super().__init__([self.conv_in] + self.rbs[:2] + [self.conv_up] + self.rbs[2:])

    def _up_fused(self) -> bool:
        """Whether conv_up reads its input through the upsample itself."""
        return getattr(self.conv_up, "upsample_in", 0) == 2

    # The low-resolution convs plan their grids for this share of the CUs
    # (their split-K count drops), which leaves CUs to the other stream's
    # full-resolution convs when the stack runs in the two-stream pipeline.
    # Sequential runs use the same plans, so both give the same bits.
    LOW_RES_CU_SHARE = (5, 8)

    def set_cu_limit(self, cus: int):
        """Plan the low-resolution layers' grids for ``cus`` CUs (0: all)."""
        for layer in [self.conv_in] + self.rbs[:2]:
            if hasattr(layer, "cu_limit"):
                layer.cu_limit = cus

    def start(self, n: int, h: int, w: int):
        num, den = self.LOW_RES_CU_SHARE
        dev = self.conv_in.weight.device
        if dev.type == "cuda":
            self.set_cu_limit(torch.cuda.get_device_properties(dev).multi_processor_count * num // den)
        self.conv_in.start(n, h, w)
        for rb in self.rbs[:2]:
            rb.start(n, h, w)
        if self._up_fused():
            self.conv_up.start(n, h, w)   # its cache holds frames before the upsample
        else:
            self.conv_up.start(n, 2 * h, 2 * w)
        for rb in self.rbs[2:]:
            rb.start(n, 2 * h, 2 * w)

    def _buf(self, name: str, shape, like: torch.Tensor) -> torch.Tensor:
        """Intermediate activation buffer, reused from chunk to chunk (so a
        recorded graph names the same memory every time)."""
        return _cached_buf(self.__dict__.setdefault("_bufs", {}), name, shape, like)

    def _fusable(self) -> bool:
        """Every block has an identity shortcut and bf16 parameters, so each
        conv can hand its output straight to the next norm
        (wvc_causal_conv3d_norm_fwd)."""
        c = self.conv_in.weight.shape[0] if isinstance(self.conv_in, CausalConv3d) else 0
        return all(isinstance(rb, ResBlock) and rb.p.get("w_short") is None and
                   rb.p["w1"].dtype == torch.bfloat16 for rb in self.rbs) and \
            isinstance(self.conv_in, CausalConv3d) and isinstance(self.conv_up, CausalConv3d) and \
            c % 8 == 0 and c <= 2048  # the conv + norm call's channel range

    def stages(self, x: torch.Tensor, out: torch.Tensor, buf) -> List[Callable[[], object]]:
        """The chunk as a list of stages (each a few library calls); the
        intermediates come from ``buf(name, shape, like)``.

        Each conv that feeds a norm computes that norm too: conv_in and conv_up
        the first block's norm1, a block's conv1 its norm2, the first block's
        conv2 (plus its input) the second block's norm1.  The stages are those
        of the layer-by-layer composition, bitwise, with four norm kernels and
        four split-K reduces fewer per chunk."""
        if not self._fusable():
            return self._stages_layerwise(x, out, buf)
        n, _, t, h, w = x.shape
        c = self.conv_in.weight.shape[0]
        lo, hi = (n, c, t, h, w), (n, c, t, 2 * h, 2 * w)
        a_in, a0, a1 = buf("in", lo, x), buf("rb0", lo, x), buf("rb1", lo, x)
        a_up, a2 = buf("conv_up", hi, x), buf("rb2", hi, x)
        h1 = [buf(f"rb{k}.h1", lo if k < 2 else hi, x) for k in range(4)]
        h2 = [buf(f"rb{k}.h2", lo if k < 2 else hi, x) for k in range(4)]
        rb = self.rbs

        def norm1(k):
            return rb[k].p["gamma1"], rb[k].p.get("beta1"), rb[k].eps

        return [
            lambda: self.conv_in.norm_into(x, a_in, *norm1(0), h1[0]),
            lambda: rb[0].front_from_h1(h1[0], h2[0]),
            lambda: rb[0].back_norm(h2[0], a_in, a0, *norm1(1), h1[1]),
            lambda: rb[1].front_from_h1(h1[1], h2[1]),
            lambda: rb[1].back(h2[1], a0, a1),
            lambda: self.conv_up.norm_into(a1, a_up, *norm1(2), h1[2]),
            lambda: rb[2].front_from_h1(h1[2], h2[2]),
            lambda: rb[2].back_norm(h2[2], a_up, a2, *norm1(3), h1[3]),
            lambda: rb[3].front_from_h1(h1[3], h2[3]),
            lambda: rb[3].back(h2[3], a2, out),
        ]

    def _stages_layerwise(self, x: torch.Tensor, out: torch.Tensor, buf) -> List[Callable[[], object]]:
        """The chunk layer by layer: each layer's own calls (its norm1 inside
        the block call)."""
        n, _, t, h, w = x.shape
        c = self.conv_in.weight.shape[0]
        lo, hi = (n, c, t, h, w), (n, c, t, 2 * h, 2 * w)
        a_in, a0, a1 = buf("in", lo, x), buf("rb0", lo, x), buf("rb1", lo, x)
        a_up, a2 = buf("conv_up", hi, x), buf("rb2", hi, x)

        def sub(k):
            return lambda name, shape, like: buf(f"rb{k}.{name}", shape, like)

        st = self.conv_in.stages(x, a_in, buf)
        st += self.rbs[0].stages(a_in, a0, sub(0))
        st += self.rbs[1].stages(a0, a1, sub(1))
        if self._up_fused():
            st += self.conv_up.stages(a1, a_up, buf)
        else:
            up = buf("up", hi, x)
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

    # The 8-bit convs are shorter, and with each norm folded into the conv
    # before it the low-resolution stream gives up more of the GPU: 3/8 of
    # the CUs measured fastest (2/8 to 5/8 swept), against 5/8 for bf16.
    LOW_RES_CU_SHARE = (3, 8)

    def __init__(self, p: Dict, scales: Dict, eps: float = 1e-12):
        self.conv_in = CausalConv3dE4M3(p["w_in"], p.get("b_in"), scales["in"])
        self.rbs = [ResBlockE4M3(p[f"rb{k}"], *scales["rb"][k], eps) for k in range(4)]
        self.conv_up = CausalConv3dE4M3(p["w_up"], p.get("b_up"), scales["up"], upsample_in=2)
        Stream.__init__(self, [self.conv_in] + self.rbs[:2] + [self.conv_up] + self.rbs[2:])

    @property
    def PIPELINE_SPLIT(self) -> int:
        """The pipeline's cut, before conv_up: conv_in and the first two
        blocks on one stream (5 fused stages, or 3 layers), the rest on the
        other."""
        return 5 if self._fusable() else 3

    def _fusable(self) -> bool:
        """Every conv that feeds a norm can compute that norm too
        (wvc_causal_conv3d_e4m3_norm_fwd): the channel count fits the call."""
        c = self.conv_in.weight.shape[0]
        return c % 8 == 0 and c <= 2048 and all(isinstance(rb, ResBlockE4M3) for rb in self.rbs)

    def stages(self, x: torch.Tensor, out: torch.Tensor, buf) -> List[Callable[[], object]]:
        """The chunk as 10 stages.  Each conv that feeds a block's norm
        computes that norm too and stores it as the block's codes: conv_in
        and conv_up the next block's norm1, a block's conv1 its norm2, the
        first block's conv2 (plus its input) the second block's norm1.  The
        calls are those of the layer-by-layer composition with the norm folded
        into the conv before it, bitwise the same codes and outputs, with four
        norm kernels and four split-K reduces fewer per chunk."""
        if not self._fusable():
            return self._stages_layerwise(x, out, buf)
        n, _, t, h, w = x.shape
        c = self.conv_in.weight.shape[0]
        lo, hi = (n, c, t, h, w), (n, c, t, 2 * h, 2 * w)
        u8 = x.new_empty(0, dtype=torch.uint8)
        a_in, a0, a1 = buf("in", lo, x), buf("rb0", lo, x), buf("rb1", lo, x)
        a_up, a2 = buf("conv_up", hi, x), buf("rb2", hi, x)
        q1 = [buf(f"rb{k}.q1", lo if k < 2 else hi, u8) for k in range(4)]
        q2 = [buf(f"rb{k}.q2", lo if k < 2 else hi, u8) for k in range(4)]
        rb = self.rbs

        def norm1(k):
            return rb[k].p["gamma1"], rb[k].p.get("beta1"), rb[k].eps, rb[k].s1

        return [
            lambda: self.conv_in.norm_into(x, a_in, *norm1(0), q1[0]),
            lambda: rb[0].front_from_q1(q1[0], q2[0]),
            lambda: rb[0].back_norm(q2[0], a_in, a0, *norm1(1), q1[1]),
            lambda: rb[1].front_from_q1(q1[1], q2[1]),
            lambda: rb[1].back(q2[1], a0, a1),
            lambda: self.conv_up.norm_into(a1, a_up, *norm1(2), q1[2]),
            lambda: rb[2].front_from_q1(q1[2], q2[2]),
            lambda: rb[2].back_norm(q2[2], a_up, a2, *norm1(3), q1[3]),
            lambda: rb[3].front_from_q1(q1[3], q2[3]),
            lambda: rb[3].back(q2[3], a2, out),
        ]


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
        # Every event the pipeline records lives as long as the pipeline (the
        # fork and join use these instead of wait_stream's temporary events).
        self._ev_a = [torch.cuda.Event() for _ in range(slots)]
        self._ev_b = [torch.cuda.Event() for _ in range(slots)]
        self._ev_fork = torch.cuda.Event()
        self._ev_join = [torch.cuda.Event(), torch.cuda.Event()]

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
            # Ending a capture that recorded this two-stream fork/join crashed
            # the HIP runtime (a host segmentation fault inside end-capture),
            # also with every event outliving the capture; graphs record
            # single-stream work only.
            raise RuntimeError("Pipeline.run cannot be recorded into a graph; record the "
                               "sequential chunk loop (or FrameGraph) instead")
        main = torch.cuda.current_stream(self.device)
        sa, sb = self.streams
        self._ev_fork.record(main)
        sa.wait_event(self._ev_fork)
        sb.wait_event(self._ev_fork)
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
        for ev, st in zip(self._ev_join, (sa, sb)):
            ev.record(st)
            main.wait_event(ev)



class PipelineGraph:
    """The two-stream pipeline of ``Pipeline`` with each chunk's two parts
    replayed as HIP graphs, so the host enqueues two graph launches, two
    copies and four event operations per chunk instead of every library call.

    Each part is recorded alone on one stream (a recording holds no
    dependency between streams); the replays go to streams A and B with the
    events of ``Pipeline.run`` between them.  A recording names fixed
    buffers: buffer set k has its own input chunk ``x[k]`` and output chunk
    ``y[k]``, and ``run`` copies each chunk into ``x[k]`` on A before the
    first part and ``y[k]`` into the caller's output on B after the second.
    Chunk i reads the caches chunk i-1 wrote, so the two buffers of every
    ping-pong swap roles from chunk to chunk; with ``slots`` buffer sets the
    (buffer set, cache parity) pairs repeat every lcm(slots, 2) chunks, and
    that many chunks are recorded.  The replays make the calls the eager
    pipeline makes, on the same buffers' contents, so the outputs are bitwise
    those of ``Pipeline.run`` and of the sequential loop.

    The stack's ping-pong state follows the replays (as for ``FrameGraph``),
    so eager chunks, checkpoints and replays can be mixed; ``reset()`` starts
    a new sequence.

    With ``bind=True`` the recordings read the caller's chunk and write the
    caller's output tensor themselves, with no copies: a pair of graphs is
    recorded the first time a (recording, chunk tensor, output tensor)
    combination is run and replayed after that.  This suits callers that pass
    the same tensors on every pass (a preallocated sequence); at most
    ``MAX_BOUND`` pairs are kept, the oldest released first (never one the
    pass in hand needs; a pass needing more is refused).  The tensors
    must stay unchanged and alive until the pass has finished."""

    MAX_BOUND = 512

    def __init__(self, stack, x_shape: Sequence[int], split: Optional[int] = None, slots: int = 3,
                 dtype=torch.bfloat16, device=None, bind: bool = False):
        dev = torch.device("cuda", torch.cuda.current_device()) if device is None else torch.device(device)
        self.stack, self.device, self.slots, self.bind = stack, dev, slots, bind
        self._bound: Dict[tuple, tuple] = {}
        self.split = split if split is not None else getattr(stack, "PIPELINE_SPLIT", 1)
        self.period = slots if slots % 2 == 0 else 2 * slots
        n, c, t, h, w = x_shape
        run1 = stack.chunk if hasattr(stack, "chunk") else (lambda x, out=None: stack(x, y=out))
        self.x = [L.empty_cl(tuple(x_shape), dtype, dev) for _ in range(slots)]
        for xb in self.x:
            L.wvc_cache_reset(xb)
        stack.start(n, h, w)
        y0 = run1(self.x[0])             # an eager chunk gives the output shape
        self.y = [L.empty_cl(tuple(y0.shape), y0.dtype, dev) for _ in range(slots)]
        self._bufs = [{} for _ in range(slots)]
        self._pps = stack.pingpongs()
        # an eager pass over one period sizes every buffer and workspace
        for r in range(self.period):
            stages = self._stages(r)
            if not 0 < self.split < len(stages):
                raise ValueError(f"split {self.split} must cut the {len(stages)} stages in two")
            for stage in stages:
                stage()
        self._materialize()
        self.graphs = []
        for r in range(self.period):
            stages = self._stages(r)
            ga = capture(lambda: [st() for st in stages[:self.split]], dev)
            gb = capture(lambda: [st() for st in stages[self.split:]], dev)
            self.graphs.append((ga, gb))
        # every layer flipped its caches once per recorded chunk, an even
        # number of times: the parity is back where the recording started
        self.streams = [torch.cuda.Stream(dev), torch.cuda.Stream(dev)]
        self._ev_a = [torch.cuda.Event() for _ in range(slots)]
        self._ev_b = [torch.cuda.Event() for _ in range(slots)]
        self._ev_fork = torch.cuda.Event()
        self._ev_join = [torch.cuda.Event(), torch.cuda.Event()]
        self.reset()

    def _stages(self, r: int, x=None, y=None):
        k = r % self.slots
        bufs = self._bufs[k]
        return self.stack.stages(self.x[k] if x is None else x, self.y[k] if y is None else y,
                                 lambda name, shape, like: _cached_buf(bufs, name, shape, like))

    @staticmethod
    def _key(r: int, x: torch.Tensor, y: torch.Tensor) -> tuple:
        return (r, x.data_ptr(), tuple(x.shape), x.stride(), x.dtype,
                y.data_ptr(), tuple(y.shape), y.stride(), y.dtype)

    def _record_bound(self, todo: List[tuple], needed: set):
        """Record the graph pairs of (r, chunk, output) triples that have none:
        each at cache parity r % 2, then the stack's cache state as it was.
        Pairs the pass in hand needs (``needed``) are never released."""
        if len(needed) > self.MAX_BOUND:
            raise ValueError(f"a pass over {len(needed)} distinct chunk/output pairs exceeds the "
                             f"{self.MAX_BOUND} bound recordings kept; use bind=False")
        saved = [(pp.cur, pp.fresh) for pp in self._pps]
        try:
            for r, x, y in todo:
                if tuple(x.shape) != tuple(self.x[0].shape) or tuple(y.shape) != tuple(self.y[0].shape):
                    raise ValueError(f"chunk {tuple(x.shape)} / output {tuple(y.shape)} differ from the "
                                     f"recorded {tuple(self.x[0].shape)} / {tuple(self.y[0].shape)}")
                for pp in self._pps:
                    pp.cur, pp.fresh = r % 2, False
                stages = self._stages(r, x, y)
                ga = capture(lambda: [st() for st in stages[:self.split]], self.device)
                gb = capture(lambda: [st() for st in stages[self.split:]], self.device)
                while len(self._bound) >= self.MAX_BOUND:
                    oldest = next(k for k in self._bound if k not in needed)
                    old = self._bound.pop(oldest)
                    old[0].close()
                    old[1].close()
                self._bound[self._key(r, x, y)] = (ga, gb)
        finally:
            for pp, (cur, fresh) in zip(self._pps, saved):
                pp.cur, pp.fresh = cur, fresh

    def _materialize(self):
        """Recorded calls name both buffers of every ping-pong: a fresh cache
        is written as zeros instead of passed as NULL."""
        self.stack.reset()
        for pp in self._pps:
            pp.materialize()

    def reset(self):
        """A new sequence: zero caches, recording 0 next."""
        self._materialize()
        self.next = 0

    def run(self, chunks: Sequence[torch.Tensor], outs: Sequence[torch.Tensor]):
        """Run every chunk in order (chunks[i] -> outs[i]) from the stack's
        current cache state; the current stream waits for all of it before
        this returns.  Each chunk must have the recorded shape and each
        output the shape of the stack's output chunk."""
        if torch.cuda.is_current_stream_capturing():
            raise RuntimeError("PipelineGraph.run replays graphs on two streams and cannot itself "
                               "be recorded into a graph")
        for pp in self._pps:
            pp.materialize()    # eager chunks since reset() may have left a fresh cache
        r = self.next
        if self._pps and r % 2 != self._pps[0].cur:
            r = (r + 1) % self.period    # eager chunks moved the parity
        if self.bind:
            rs = [(r + i) % self.period for i in range(len(chunks))]
            keys = [self._key(ri, x, y) for ri, x, y in zip(rs, chunks, outs)]
            todo = [(ri, x, y) for ri, x, y, k in zip(rs, chunks, outs, keys) if k not in self._bound]
            if todo:
                self._record_bound(todo, set(keys))
        main = torch.cuda.current_stream(self.device)
        sa, sb = self.streams
        self._ev_fork.record(main)
        sa.wait_event(self._ev_fork)
        sb.wait_event(self._ev_fork)
        for i, (x, y) in enumerate(zip(chunks, outs)):
            k = r % self.slots
            ga, gb = self._bound[self._key(r, x, y)] if self.bind else self.graphs[r]
            with torch.cuda.stream(sa):
                if i >= self.slots:
                    sa.wait_event(self._ev_b[k])   # B is done with this buffer set
                if not self.bind:
                    self.x[k].copy_(x)
                ga.launch(sa)
                self._ev_a[k].record(sa)
            with torch.cuda.stream(sb):
                sb.wait_event(self._ev_a[k])
                gb.launch(sb)
                if not self.bind:
                    y.copy_(self.y[k])
                self._ev_b[k].record(sb)
            x.record_stream(sa)
            y.record_stream(sb)
            for pp in self._pps:
                pp.flip()
            r = (r + 1) % self.period
        self.next = r
        for ev, st in zip(self._ev_join, (sa, sb)):
            ev.record(st)
            main.wait_event(ev)

    def close(self):
        for ga, gb in self.graphs + list(self._bound.values()):
            ga.close()
            gb.close()
        self._bound.clear()


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
