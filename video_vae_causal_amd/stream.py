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

Host orchestration only; every tensor operation is a libwvc call.
"""
from __future__ import annotations

from typing import Dict, List, Optional, Sequence

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


class _PingPong:
    def __init__(self, shape, dtype, device):
        self.buf = [L.empty_cl(shape, dtype, device), L.empty_cl(shape, dtype, device)]
        self.cur = 0
        self.reset()

    def reset(self):
        # Only the buffer the next chunk reads must be zero (zero causal
        # padding); the other one is entirely rewritten as that chunk's cache_out.
        L.wvc_cache_reset(self.buf[0])
        self.cur = 0

    @property
    def cin(self):
        return self.buf[self.cur]

    @property
    def cout(self):
        return self.buf[1 - self.cur]

    def flip(self):
        self.cur ^= 1


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
        return [self.cache.cin] if self.cache is not None else []


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
        self.c1 = _PingPong((n, cin, CACHE_T, h, w), dt, dev)
        self.c2 = _PingPong((n, cout, CACHE_T, h, w), dt, dev)

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
        return [self.c1.cin, self.c2.cin] if self.c1 is not None else []


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


class DecoderStack(Stream):
    """Decoder-shaped stack: conv_in (C_lat -> C) -> 2 resblocks -> nearest 2x
    upsample -> conv_up (C -> C) -> 2 resblocks, streamed chunk by chunk with one
    2-frame cache per 3x3x3 conv (10 caches for 4 resblocks)."""

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

    def chunk(self, x: torch.Tensor, out: Optional[torch.Tensor] = None) -> torch.Tensor:
        h = self.conv_in(x)
        h = self.rbs[0](h)
        h = self.rbs[1](h)
        h = L.wvc_upsample_nearest2x(h)
        h = self.conv_up(h)
        h = self.rbs[2](h)
        return self.rbs[3](h, y=out)

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
