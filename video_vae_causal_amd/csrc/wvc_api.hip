// wvc_api.hip -- the C ABI of libwvc (declared in include/wvc.h): argument
// validation, route selection, aliasing checks, route counters, strict mode
// and per-thread error text.  Every argument error is reported before any
// work is enqueued.
#include <atomic>
#include <cmath>
#include <mutex>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>

#include <new>

#include "wvc.h"
#include "wvc_internal.h"

namespace {

thread_local char g_err[512] = "";
std::atomic<int> g_strict{-1};
std::atomic<uint64_t> g_fast3{0}, g_fast1{0}, g_generic{0}, g_rejected{0}, g_strided{0};

int fail(int code, const char *fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof(g_err), fmt, ap);
    va_end(ap);
    return code;
}

int strict_on() {
    int s = g_strict.load();
    if (s < 0) {
        const char *e = std::getenv("WVC_STRICT");
        int want = (e && std::atoi(e) != 0) ? 1 : 0;
        int expected = -1;
        g_strict.compare_exchange_strong(expected, want);
        s = g_strict.load();
    }
    return s;
}

int elem_bytes(int dtype) { return dtype == WVC_F32 ? 4 : dtype == WVC_BF16 ? 2 : 0; }

struct Buf {
    const void *p;
    size_t bytes;
    bool written;
    const char *name;
};

// Every written buffer must be disjoint from every other buffer of the call.
int check_aliasing(const Buf *b, int nb) {
    for (int i = 0; i < nb; ++i) {
        if (!b[i].written || !b[i].p || b[i].bytes == 0) continue;
        const uintptr_t lo = (uintptr_t)b[i].p, hi = lo + b[i].bytes;
        for (int j = 0; j < nb; ++j) {
            if (j == i || !b[j].p || b[j].bytes == 0) continue;
            const uintptr_t lo2 = (uintptr_t)b[j].p, hi2 = lo2 + b[j].bytes;
            if (lo < hi2 && lo2 < hi)
                return fail(WVC_ERR_ALIAS, "written buffer '%s' overlaps buffer '%s'", b[i].name,
                            b[j].name);
        }
    }
    return WVC_OK;
}

bool mul_ok(size_t a, size_t b, size_t *out) {
    if (a != 0 && b > (SIZE_MAX >> 2) / a) return false;
    *out = a * b;
    return true;
}

int out_size(int in, int k, int s, int p, int d) {
    const long span = (long)d * (k - 1) + 1;
    if ((long)in + 2L * p < span) return 0;
    return (int)(((long)in + 2L * p - span) / s + 1);
}

bool aligned(const void *p, uintptr_t a) { return ((uintptr_t)p % a) == 0; }

struct ConvPlan {
    wvc::ConvCall call;
    wvc::ConvRoute route;
    size_t x_bytes, cache_bytes, w_bytes, b_bytes, y_bytes;
};

bool strided_route(wvc::ConvRoute r) {
    return r == wvc::ConvRoute::FastTemporal || r == wvc::ConvRoute::FastSpatial2;
}

size_t route_ws_bytes(const ConvPlan &pl, bool packed) {
    if (pl.route == wvc::ConvRoute::Generic) return 0;
    if (strided_route(pl.route)) return wvc::strided_workspace_bytes(pl.call, packed);
    return wvc::igemm_workspace_bytes(pl.call, pl.route, packed);
}

size_t route_packed_bytes(const ConvPlan &pl) {
    return strided_route(pl.route) ? wvc::strided_packed_weight_bytes(pl.call)
                                   : wvc::igemm_packed_weight_bytes(pl.call);
}

// Validates the descriptor (not the pointers) and fills the sizes.
int plan_conv(const wvc_conv3d_desc *d, ConvPlan *pl, bool count = true) {
    if (!d) return fail(WVC_ERR_ARG, "conv descriptor is NULL");
    if (d->groups != 1) {
        if (count) g_rejected++;
        return fail(WVC_ERR_UNSUPPORTED, "groups=%d: only one group is supported", d->groups);
    }
    // E4M3 calls: 1-byte codes in x, cache and weight; bf16 bias, residual, y.
    const bool e4m3 = d->dtype == WVC_E4M3;
    const int e = e4m3 ? 1 : elem_bytes(d->dtype);
    const int eo = e4m3 ? 2 : e;
    if (!e) {
        if (count) g_rejected++;
        return fail(WVC_ERR_UNSUPPORTED, "dtype %d is not WVC_F32, WVC_BF16 or WVC_E4M3", d->dtype);
    }
    if (d->n < 1 || d->c_in < 1 || d->c_out < 1 || d->t < 0 || d->h < 1 || d->w < 1)
        return fail(WVC_ERR_ARG, "bad shape n=%d c_in=%d c_out=%d t=%d h=%d w=%d", d->n, d->c_in,
                    d->c_out, d->t, d->h, d->w);
    if (d->weight_layout != WVC_WEIGHT_STANDARD && d->weight_layout != WVC_WEIGHT_PACKED)
        return fail(WVC_ERR_ARG, "weight_layout %d is neither standard nor packed", d->weight_layout);
    if (d->kt < 1 || d->kh < 1 || d->kw < 1 || d->stride_h < 1 || d->stride_w < 1 ||
        d->pad_h < 0 || d->pad_w < 0 || d->dil_t < 1 || d->dil_h < 1 || d->dil_w < 1 ||
        d->stride_t < 1 || d->stride_t > 64 || d->pad_h_extra < 0 || d->pad_w_extra < 0 ||
        d->pad_h_extra > 64 || d->pad_w_extra > 64)
        return fail(WVC_ERR_ARG, "bad kernel/stride/pad/dilation");
    if (d->t_phase < 0 || d->t_phase >= d->stride_t)
        return fail(WVC_ERR_ARG, "t_phase %d must lie in [0, stride_t = %d)", d->t_phase, d->stride_t);
    if (d->upsample_in != 0 && d->upsample_in != 2)
        return fail(WVC_ERR_ARG, "upsample_in %d must be 0 or 2", d->upsample_in);
    if (d->cu_limit < 0) return fail(WVC_ERR_ARG, "cu_limit %d must be >= 0", d->cu_limit);
    // Upsampled input: x and the caches hold h/2 x w/2 frames.
    const int up = d->upsample_in == 2 ? 2 : 1;
    if (up == 2 && (d->h % 2 != 0 || d->w % 2 != 0))
        return fail(WVC_ERR_ARG, "upsample_in needs an even h and w (got %d x %d)", d->h, d->w);
    // One-sided padding extends the padded frame at its far end only.
    const int ho = out_size(d->h + d->pad_h_extra, d->kh, d->stride_h, d->pad_h, d->dil_h);
    const int wo = out_size(d->w + d->pad_w_extra, d->kw, d->stride_w, d->pad_w, d->dil_w);
    if (ho < 1 || wo < 1) return fail(WVC_ERR_ARG, "kernel larger than the padded frame");
    // Output frames: anchors first, first + stride_t, ... inside the chunk.
    const int first = (d->stride_t - d->t_phase) % d->stride_t;
    const int to = first < d->t ? (d->t - 1 - first) / d->stride_t + 1 : 0;
    const long frames = (long)d->dil_t * (d->kt - 1);
    if (frames > 1024) return fail(WVC_ERR_ARG, "temporal receptive field too large");

    wvc::ConvCall &c = pl->call;
    std::memset(&c, 0, sizeof(c));
    c.n = d->n; c.cin = d->c_in; c.cout = d->c_out; c.t = d->t; c.h = d->h; c.w = d->w;
    c.ho = ho; c.wo = wo;
    c.kt = d->kt; c.kh = d->kh; c.kw = d->kw;
    c.sh = d->stride_h; c.sw = d->stride_w; c.ph = d->pad_h; c.pw = d->pad_w;
    c.dt = d->dil_t; c.dh = d->dil_h; c.dw = d->dil_w;
    c.frames = (int)frames;
    c.dtype = d->dtype;
    c.st = d->stride_t;
    c.t0 = first;
    c.to = to;
    c.eh = d->pad_h_extra;
    c.ew = d->pad_w_extra;
    c.up = up;
    c.cu_limit = d->cu_limit;

    size_t plane_in, plane_out, v;
    bool ok = mul_ok((size_t)(d->h / up), (size_t)(d->w / up), &plane_in) &&
              mul_ok(plane_in, d->c_in, &plane_in);
    ok = ok && mul_ok((size_t)ho, (size_t)wo, &plane_out) && mul_ok(plane_out, d->c_out, &plane_out);
    ok = ok && mul_ok(plane_in, (size_t)d->n * d->t, &v) && mul_ok(v, e, &pl->x_bytes);
    ok = ok && mul_ok(plane_in, (size_t)d->n * frames, &v) && mul_ok(v, e, &pl->cache_bytes);
    ok = ok && mul_ok((size_t)d->c_out * d->c_in, (size_t)d->kt * d->kh * d->kw, &v) &&
         mul_ok(v, e, &pl->w_bytes);
    ok = ok && mul_ok(plane_out, (size_t)d->n * to, &v) && mul_ok(v, eo, &pl->y_bytes);
    if (!ok) return fail(WVC_ERR_ARG, "tensor size overflows");
    pl->b_bytes = (size_t)d->c_out * eo;

    const bool chan_ok = d->c_in % 8 == 0 && d->c_out % 32 == 0;
    const bool unit = d->stride_h == 1 && d->stride_w == 1 && d->stride_t == 1 &&
                      d->pad_h_extra == 0 && d->pad_w_extra == 0;
    const bool dil1 = d->dil_t == 1 && d->dil_h == 1 && d->dil_w == 1;
    if (d->dtype == WVC_BF16 && chan_ok && unit && d->kt == 3 && d->kh == 3 && d->kw == 3 &&
        d->pad_h == 1 && d->pad_w == 1 && dil1)
        pl->route = wvc::ConvRoute::Fast3x3x3;
    else if (d->dtype == WVC_BF16 && chan_ok && unit && d->kt == 1 && d->kh == 1 && d->kw == 1 &&
             d->pad_h == 0 && d->pad_w == 0)
        pl->route = wvc::ConvRoute::Fast1x1x1;
    else if (d->dtype == WVC_BF16 && wvc::strided_supports(c))
        pl->route = d->kt > 1 ? wvc::ConvRoute::FastTemporal : wvc::ConvRoute::FastSpatial2;
    else
        pl->route = wvc::ConvRoute::Generic;
    if ((pl->route == wvc::ConvRoute::Fast3x3x3 || pl->route == wvc::ConvRoute::Fast1x1x1) &&
        !wvc::igemm_supports(c))
        pl->route = wvc::ConvRoute::Generic;
    if (e4m3) {
        // The 8-bit conv exists on the MFMA 3x3x3 route only.
        const bool fits = d->c_in % 16 == 0 && d->c_out % 32 == 0 && unit && d->kt == 3 &&
                          d->kh == 3 && d->kw == 3 && d->pad_h == 1 && d->pad_w == 1 && dil1 &&
                          wvc::igemm_supports(c);
        if (!fits) {
            if (count) g_rejected++;
            return fail(WVC_ERR_UNSUPPORTED,
                        "E4M3 convs must be 3x3x3, stride 1, pad 1, dilation 1, C_in %% 16 == 0, "
                        "C_out %% 32 == 0");
        }
        pl->route = wvc::ConvRoute::Fast3x3x3;
    }
    if (up == 2 && pl->route != wvc::ConvRoute::Fast3x3x3) {
        if (count) g_rejected++;
        return fail(WVC_ERR_UNSUPPORTED,
                    "upsample_in is read by the MFMA 3x3x3 route only (bf16 or E4M3; 3x3x3, stride 1, "
                    "pad 1, dilation 1, C_in %% 8 == 0, C_out %% 32 == 0)");
    }
    if (d->weight_layout == WVC_WEIGHT_PACKED) {
        if (pl->route == wvc::ConvRoute::Generic) {
            if (count) g_rejected++;
            return fail(WVC_ERR_UNSUPPORTED, "packed weights exist only for the MFMA routes");
        }
        pl->w_bytes = route_packed_bytes(*pl);
    }
    return WVC_OK;
}

bool ws_ok(const void *ws, size_t bytes) { return ws || bytes == 0; }

int hip_status(hipError_t err, const char *what) {
    if (err == hipSuccess) return WVC_OK;
    return fail(WVC_ERR_HIP, "%s: %s", what, hipGetErrorString(err));
}

// Validated conv call shared by wvc_causal_conv3d_fwd and wvc_resblock_fwd.
// With `defer` given, a split-K MFMA conv leaves its partial sums for the
// caller instead of reducing them into y (defer->S > 1 then; see
// launch_conv_igemm).
int conv_fwd(const wvc_conv3d_desc *d, const void *x, const void *cache_in, void *cache_out,
             const void *weight, const void *bias, const void *residual, void *y, void *ws,
             size_t ws_bytes, hipStream_t s, wvc::ConvPartials *defer = nullptr,
             float x_scale = 1.f, const float *w_scale = nullptr) {
    if (defer) *defer = wvc::ConvPartials{};
    ConvPlan pl;
    int rc = plan_conv(d, &pl);
    if (rc) return rc;
    const bool e4m3 = d->dtype == WVC_E4M3;
    if (!weight) return fail(WVC_ERR_ARG, "weight is NULL");
    if (e4m3) {
        if (!w_scale || !aligned(w_scale, 16))
            return fail(WVC_ERR_ARG, "w_scale must be a 16-byte aligned device array of C_out floats");
        if (!(x_scale > 0.f) || !(x_scale < INFINITY))
            return fail(WVC_ERR_ARG, "x_scale must be finite and > 0");
    }
    // y is needed only when the chunk has output frames (a strided chunk may
    // have none: its frames only feed the cache).
    if (d->t > 0 && (!x || (pl.call.to > 0 && !y))) return fail(WVC_ERR_ARG, "x or y is NULL");
    if (pl.call.frames == 0) {
        cache_in = nullptr;
        cache_out = nullptr;
    }
    if (!ws && ws_bytes) return fail(WVC_ERR_ARG, "workspace is NULL but workspace_bytes > 0");

    // Fast routes read 16-byte vectors; anything not aligned takes the generic route.
    const bool packed = d->weight_layout == WVC_WEIGHT_PACKED;
    if (pl.route != wvc::ConvRoute::Generic) {
        const bool al = aligned(x, 16) && aligned(cache_in, 16) && aligned(weight, 16) &&
                        aligned(y, 16) && aligned(residual, 16) && aligned(bias, 8);
        if (!al) {
            if (packed || e4m3 || pl.call.up == 2)
                return fail(WVC_ERR_ARG, "%s need 16-byte aligned tensors",
                            e4m3 ? "E4M3 convs" : packed ? "packed weights" : "upsampled-input convs");
            pl.route = wvc::ConvRoute::Generic;
        }
    }
    size_t need = route_ws_bytes(pl, packed);
    if (ws_bytes < need)
        return fail(WVC_ERR_WORKSPACE, "workspace of %zu bytes, %zu needed", ws_bytes, need);

    const Buf bufs[] = {
        {x, pl.x_bytes, false, "x"},
        {cache_in, pl.cache_bytes, false, "cache_in"},
        {cache_out, pl.cache_bytes, true, "cache_out"},
        {weight, pl.w_bytes, false, "weight"},
        {bias, pl.b_bytes, false, "bias"},
        {residual, pl.y_bytes, false, "residual"},
        {y, pl.y_bytes, true, "y"},
        {ws, ws_bytes, true, "workspace"},
        {w_scale, e4m3 ? (size_t)d->c_out * 4 : 0, false, "w_scale"},
    };
    rc = check_aliasing(bufs, 9);
    if (rc) return rc;

    if (pl.route == wvc::ConvRoute::Generic && strict_on()) {
        g_rejected++;
        return fail(WVC_ERR_STRICT, "strict mode: call would take the generic direct route");
    }

    wvc::ConvCall &c = pl.call;
    c.x = x;
    c.cache_in = cache_in;
    c.weight = weight;
    c.bias = bias;
    c.residual = residual;
    c.y = y;
    c.xscale = x_scale;
    c.wscale = e4m3 ? w_scale : nullptr;
    hipError_t err = hipSuccess;
    bool cache_done = false;
    if (d->t > 0) {
        if (pl.route == wvc::ConvRoute::Generic) {
            err = wvc::launch_conv_direct(c, s);
        } else if (strided_route(pl.route)) {
            err = wvc::launch_conv_strided(c, pl.route, packed, ws, ws_bytes, s);
        } else {
            err = wvc::launch_conv_igemm(c, pl.route, packed, ws, ws_bytes, cache_out, s, defer);
            cache_done = pl.route == wvc::ConvRoute::Fast3x3x3;  // written by the conv itself
        }
        if (err != hipSuccess) return hip_status(err, "conv launch");
    }
    if (cache_out && !cache_done) {
        const size_t frame_elems = (size_t)(d->h / c.up) * (d->w / c.up) * d->c_in;
        err = wvc::launch_cache_update(x, cache_in, cache_out, d->n, d->t, c.frames, frame_elems,
                                       e4m3 ? 1 : elem_bytes(d->dtype), s);
        if (err != hipSuccess) return hip_status(err, "cache update launch");
    }
    if (pl.route == wvc::ConvRoute::Fast3x3x3)
        g_fast3++;
    else if (pl.route == wvc::ConvRoute::Fast1x1x1)
        g_fast1++;
    else if (strided_route(pl.route))
        g_strided++;
    else
        g_generic++;
    return WVC_OK;
}

int norm_fwd(const void *x, const void *gamma, const void *beta, void *y, int n, int c, int t,
             int h, int w, int dtype, float eps, int apply_silu, hipStream_t s) {
    const int e = elem_bytes(dtype);
    if (!e) return fail(WVC_ERR_UNSUPPORTED, "dtype %d is neither WVC_F32 nor WVC_BF16", dtype);
    if (n < 1 || c < 1 || t < 0 || h < 1 || w < 1)
        return fail(WVC_ERR_ARG, "bad shape n=%d c=%d t=%d h=%d w=%d", n, c, t, h, w);
    if (!(eps > 0.f)) return fail(WVC_ERR_ARG, "eps must be > 0");
    if (!gamma) return fail(WVC_ERR_ARG, "gamma is NULL");
    const long positions = (long)n * t * h * w;
    if (positions > 0 && (!x || !y)) return fail(WVC_ERR_ARG, "x or y is NULL");
    const size_t bytes = (size_t)positions * c * e;
    const Buf bufs[] = {{x, bytes, false, "x"},
                        {y, bytes, true, "y"},
                        {gamma, (size_t)c * e, false, "gamma"},
                        {beta, (size_t)c * e, false, "beta"}};
    int rc = check_aliasing(bufs, 4);
    if (rc) return rc;
    return hip_status(wvc::launch_rmsnorm_silu(x, gamma, beta, y, positions, c, dtype, eps,
                                               apply_silu, s),
                      "rmsnorm launch");
}

size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }

struct BlockLayout {
    size_t h1, a1, h2, sc, conv, conv_bytes, total;
};

int plan_block(const wvc_resblock_desc *d, BlockLayout *L) {
    if (!d) return fail(WVC_ERR_ARG, "resblock descriptor is NULL");
    const int e = elem_bytes(d->dtype);
    if (!e) return fail(WVC_ERR_UNSUPPORTED, "dtype %d is neither WVC_F32 nor WVC_BF16", d->dtype);
    if (d->n < 1 || d->c_in < 1 || d->c_out < 1 || d->t < 0 || d->h < 1 || d->w < 1)
        return fail(WVC_ERR_ARG, "bad resblock shape");
    if (!(d->eps > 0.f)) return fail(WVC_ERR_ARG, "eps must be > 0");
    if (d->weights_packed != 0 && d->weights_packed != 1)
        return fail(WVC_ERR_ARG, "weights_packed must be 0 or 1");
    if (d->cu_limit < 0) return fail(WVC_ERR_ARG, "cu_limit %d must be >= 0", d->cu_limit);
    const size_t pos = (size_t)d->n * d->t * d->h * d->w;
    // The convs' scratch (split-K partials, packed weights) comes first, sized
    // for the largest of the block's convs; the intermediates follow.
    wvc_conv3d_desc c{};
    c.n = d->n; c.c_in = d->c_in; c.c_out = d->c_out; c.t = d->t; c.h = d->h; c.w = d->w;
    c.kt = c.kh = c.kw = 3;
    c.stride_t = c.stride_h = c.stride_w = 1;
    c.pad_h = c.pad_w = 1;
    c.dil_t = c.dil_h = c.dil_w = 1;
    c.groups = 1;
    c.dtype = d->dtype;
    c.weight_layout = d->weights_packed ? WVC_WEIGHT_PACKED : WVC_WEIGHT_STANDARD;
    c.cu_limit = d->cu_limit;
    size_t need = 0;
    for (int k = 0; k < 3; ++k) {
        if (k == 1) c.c_in = d->c_out;
        if (k == 2) {  // the 1x1x1 shortcut, when there is one
            if (d->c_in == d->c_out) break;
            c.c_in = d->c_in;
            c.kt = c.kh = c.kw = 1;
            c.pad_h = c.pad_w = 0;
        }
        ConvPlan pl;
        if (plan_conv(&c, &pl, false) == WVC_OK && pl.route != wvc::ConvRoute::Generic) {
            const size_t b = wvc::igemm_workspace_bytes(pl.call, pl.route, d->weights_packed != 0);
            if (b > need) need = b;
        }
    }
    L->conv = 0;
    L->conv_bytes = align256(need);
    L->h1 = L->conv_bytes;
    L->a1 = L->h1 + align256(pos * d->c_in * e);
    L->h2 = L->a1 + align256(pos * d->c_out * e);
    L->sc = L->h2 + align256(pos * d->c_out * e);
    L->total = L->sc + (d->c_in != d->c_out ? align256(pos * d->c_out * e) : 0);
    return WVC_OK;
}

// ---- scratch of the allocation-free conv entry point
//
// One fixed device array per GPU, in place of a caller workspace.  In host
// code `scratch` names a host-side stand-in, never the device memory: its
// device address is looked up once per device (hipGetSymbolAddress, with that
// device current) and only that address is handed to kernels.
constexpr size_t NOALLOC_SCRATCH_BYTES = (size_t)WVC_NOALLOC_SCRATCH_MIB << 20;
static __device__ __align__(256) unsigned char scratch[NOALLOC_SCRATCH_BYTES];

constexpr int SCRATCH_DEVICES = 64;
struct ScratchSlot {
    std::once_flag once;
    void *ptr = nullptr;
    hipError_t err = hipSuccess;
};
ScratchSlot g_scratch[SCRATCH_DEVICES];

// Device address of the current device's scratch array.
int scratch_address(void **out) {
    int dev = -1;
    const hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_status(e, "hipGetDevice");
    if (dev < 0 || dev >= SCRATCH_DEVICES)
        return fail(WVC_ERR_ARG, "device %d: the scratch table covers devices 0-%d", dev,
                    SCRATCH_DEVICES - 1);
    ScratchSlot &slot = g_scratch[dev];
    std::call_once(slot.once, [&slot] {
        void *p = nullptr;
        slot.err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (slot.err == hipSuccess && p == nullptr) slot.err = hipErrorInvalidSymbol;
        slot.ptr = slot.err == hipSuccess ? p : nullptr;
    });
    if (slot.err != hipSuccess) return hip_status(slot.err, "scratch symbol address");
    *out = slot.ptr;
    return WVC_OK;
}

}  // namespace

extern "C" {

int wvc_causal_conv3d_fwd_noalloc(const wvc_conv3d_desc *d, const void *x, const void *cache_in,
                                  void *cache_out, const void *weight, const void *bias,
                                  const void *residual, void *y, void *stream) {
    if (d && d->dtype == WVC_E4M3) {
        g_rejected++;
        return fail(WVC_ERR_UNSUPPORTED, "E4M3 convs take wvc_causal_conv3d_e4m3_fwd (they need scales)");
    }
    ConvPlan pl;
    const int rc = plan_conv(d, &pl, /*count=*/false);  // conv_fwd counts the call
    if (rc) return rc;
    const size_t need = route_ws_bytes(pl, d->weight_layout == WVC_WEIGHT_PACKED);
    if (need > NOALLOC_SCRATCH_BYTES)
        return fail(WVC_ERR_WORKSPACE,
                    "the call needs %zu bytes of scratch; the allocation-free entry point has %zu "
                    "(take wvc_causal_conv3d_fwd with a workspace)", need, NOALLOC_SCRATCH_BYTES);
    void *ws = nullptr;
    if (need > 0) {
        const int r2 = scratch_address(&ws);
        if (r2) return r2;
    }
    return conv_fwd(d, x, cache_in, cache_out, weight, bias, residual, y, ws, need,
                    static_cast<hipStream_t>(stream));
}

int wvc_causal_conv3d_fwd(const wvc_conv3d_desc *d, const void *x, const void *cache_in,
                          void *cache_out, const void *weight, const void *bias,
                          const void *residual, void *y, void *workspace, size_t workspace_bytes,
                          void *stream) {
    if (d && d->dtype == WVC_E4M3) {
        g_rejected++;
        return fail(WVC_ERR_UNSUPPORTED, "E4M3 convs take wvc_causal_conv3d_e4m3_fwd (they need scales)");
    }
    return conv_fwd(d, x, cache_in, cache_out, weight, bias, residual, y, workspace,
                    workspace_bytes, static_cast<hipStream_t>(stream));
}

int wvc_rmsnorm_silu_conv3d_fwd(const wvc_conv3d_desc *d, const void *x, const void *gamma,
                                const void *beta, float eps, const void *weight, const void *bias,
                                const void *residual, void *y, void *workspace,
                                size_t workspace_bytes, void *stream) {
    ConvPlan pl;
    int rc = plan_conv(d, &pl);
    if (rc) return rc;
    if (pl.route != wvc::ConvRoute::FastSpatial2) {
        g_rejected++;
        return fail(WVC_ERR_UNSUPPORTED,
                    "the fused norm + conv exists for the bf16 1x3x3 stride-(1,2,2) route only");
    }
    if (!weight) return fail(WVC_ERR_ARG, "weight is NULL");
    if (!gamma) return fail(WVC_ERR_ARG, "gamma is NULL");
    if (!(eps > 0.f)) return fail(WVC_ERR_ARG, "eps must be > 0");
    if (d->t > 0 && (!x || !y)) return fail(WVC_ERR_ARG, "x or y is NULL");
    if (!ws_ok(workspace, workspace_bytes)) return fail(WVC_ERR_ARG, "workspace is NULL but workspace_bytes > 0");
    const bool packed = d->weight_layout == WVC_WEIGHT_PACKED;
    if (!(aligned(x, 16) && aligned(weight, 16) && aligned(y, 16) && aligned(residual, 16) &&
          aligned(bias, 8) && aligned(gamma, 16) && aligned(beta, 16)))
        return fail(WVC_ERR_ARG, "the fused norm + conv needs 16-byte aligned tensors");
    const size_t need = route_ws_bytes(pl, packed);
    if (workspace_bytes < need)
        return fail(WVC_ERR_WORKSPACE, "workspace of %zu bytes, %zu needed", workspace_bytes, need);
    const Buf bufs[] = {
        {x, pl.x_bytes, false, "x"},
        {weight, pl.w_bytes, false, "weight"},
        {bias, pl.b_bytes, false, "bias"},
        {residual, pl.y_bytes, false, "residual"},
        {gamma, (size_t)d->c_in * 2, false, "gamma"},
        {beta, (size_t)d->c_in * 2, false, "beta"},
        {y, pl.y_bytes, true, "y"},
        {workspace, workspace_bytes, true, "workspace"},
    };
    rc = check_aliasing(bufs, 8);
    if (rc) return rc;
    wvc::ConvCall &c = pl.call;
    c.x = x;
    c.weight = weight;
    c.bias = bias;
    c.residual = residual;
    c.y = y;
    c.norm_gamma = gamma;
    c.norm_beta = beta;
    c.norm_eps = eps;
    if (d->t > 0 && pl.call.to > 0) {
        const hipError_t err = wvc::launch_conv_strided(c, pl.route, packed, workspace, workspace_bytes,
                                                        static_cast<hipStream_t>(stream));
        if (err != hipSuccess) return hip_status(err, "fused norm + conv launch");
    }
    g_strided++;
    return WVC_OK;
}

int wvc_causal_conv3d_e4m3_fwd(const wvc_conv3d_desc *d, const void *x, float x_scale,
                               const void *cache_in, void *cache_out, const void *weight,
                               const float *w_scale, const void *bias, const void *residual,
                               void *y, void *workspace, size_t workspace_bytes, void *stream) {
    if (!d) return fail(WVC_ERR_ARG, "conv descriptor is NULL");
    if (d->dtype != WVC_E4M3)
        return fail(WVC_ERR_ARG, "wvc_causal_conv3d_e4m3_fwd needs d->dtype == WVC_E4M3");
    return conv_fwd(d, x, cache_in, cache_out, weight, bias, residual, y, workspace,
                    workspace_bytes, static_cast<hipStream_t>(stream), nullptr, x_scale, w_scale);
}

size_t wvc_causal_conv3d_workspace_bytes(const wvc_conv3d_desc *d) {
    ConvPlan pl;
    if (plan_conv(d, &pl, /*count=*/false)) return (size_t)-1;  // a size query is not a call
    return route_ws_bytes(pl, d->weight_layout == WVC_WEIGHT_PACKED);
}

// ---- conv, then the next layer's RMS norm + SiLU
//
// Workspace: [the conv's workspace][room for y when the caller passes none].
size_t wvc_causal_conv3d_norm_workspace_bytes(const wvc_conv3d_desc *d) {
    ConvPlan pl;
    if (plan_conv(d, &pl, /*count=*/false)) return (size_t)-1;
    return align256(route_ws_bytes(pl, d->weight_layout == WVC_WEIGHT_PACKED)) + align256(pl.y_bytes);
}

int wvc_causal_conv3d_norm_fwd(const wvc_conv3d_desc *d, const void *x, const void *cache_in,
                               void *cache_out, const void *weight, const void *bias,
                               const void *residual, void *y, const void *gamma, const void *beta,
                               float eps, void *h, void *workspace, size_t workspace_bytes,
                               void *stream) {
    ConvPlan pl;
    int rc = plan_conv(d, &pl, /*count=*/false);  // conv_fwd below counts the call
    if (rc) return rc;
    if (d->dtype != WVC_BF16) {
        g_rejected++;
        return fail(WVC_ERR_UNSUPPORTED, "the conv + norm call exists for WVC_BF16 only");
    }
    if (d->c_out % 8 != 0 || d->c_out > 2048) {
        g_rejected++;
        return fail(WVC_ERR_UNSUPPORTED, "the conv + norm call needs C_out %% 8 == 0 and C_out <= 2048");
    }
    if (!gamma) return fail(WVC_ERR_ARG, "gamma is NULL");
    if (!(eps > 0.f)) return fail(WVC_ERR_ARG, "eps must be > 0");
    const long positions = (long)d->n * pl.call.to * pl.call.ho * pl.call.wo;
    if (d->t > 0 && positions > 0 && !h) return fail(WVC_ERR_ARG, "h is NULL");
    if (!ws_ok(workspace, workspace_bytes)) return fail(WVC_ERR_ARG, "workspace is NULL but workspace_bytes > 0");
    const size_t conv_need = align256(route_ws_bytes(pl, d->weight_layout == WVC_WEIGHT_PACKED));
    const size_t need = conv_need + align256(pl.y_bytes);
    if (workspace_bytes < need)
        return fail(WVC_ERR_WORKSPACE, "workspace of %zu bytes, %zu needed", workspace_bytes, need);
    const Buf bufs[] = {
        {x, pl.x_bytes, false, "x"},
        {cache_in, pl.cache_bytes, false, "cache_in"},
        {cache_out, pl.cache_bytes, true, "cache_out"},
        {residual, pl.y_bytes, false, "residual"},
        {y, pl.y_bytes, true, "y"},
        {gamma, (size_t)d->c_out * 2, false, "gamma"},
        {beta, (size_t)d->c_out * 2, false, "beta"},
        {h, pl.y_bytes, true, "h"},
        {workspace, workspace_bytes, true, "workspace"},
    };
    rc = check_aliasing(bufs, 9);
    if (rc) return rc;
    hipStream_t s = static_cast<hipStream_t>(stream);
    char *ws = static_cast<char *>(workspace);
    void *yy = y ? y : ws + conv_need;
    // On a split-K plan the reduce is fused into the norm: the norm kernel adds
    // the partial sums in split order, the bias and the residual, rounds y
    // once (storing it when y is given) and normalises that rounded value.
    const bool fuse = aligned(gamma, 16) && aligned(beta, 16) && aligned(bias, 16) &&
                      aligned(residual, 16) && aligned(y, 16) && aligned(h, 16);
    wvc::ConvPartials parts;
    if ((rc = conv_fwd(d, x, cache_in, cache_out, weight, bias, residual, yy, ws, conv_need, s,
                       fuse ? &parts : nullptr)))
        return rc;
    if (parts.S > 1)
        return hip_status(wvc::launch_rmsnorm_silu_from_partials(parts, bias, gamma, beta, h, positions,
                                                                 d->c_out, eps, 1, s, nullptr, 1.f, 0.f,
                                                                 residual, y),
                          "norm launch");
    if (d->t == 0 || positions == 0) return WVC_OK;
    return norm_fwd(yy, gamma, beta, h, d->n, d->c_out, pl.call.to, pl.call.ho, pl.call.wo, d->dtype,
                    eps, 1, s);
}

// ---- the 8-bit conv, then the next layer's RMS norm + SiLU stored as codes
//
// Workspace: [the conv's workspace][room for y when the caller passes none].
size_t wvc_causal_conv3d_e4m3_norm_workspace_bytes(const wvc_conv3d_desc *d) {
    if (d && d->dtype != WVC_E4M3) {
        fail(WVC_ERR_ARG, "the 8-bit conv + norm call needs d->dtype == WVC_E4M3");
        return (size_t)-1;
    }
    return wvc_causal_conv3d_norm_workspace_bytes(d);
}

int wvc_causal_conv3d_e4m3_norm_fwd(const wvc_conv3d_desc *d, const void *x, float x_scale,
                                    const void *cache_in, void *cache_out, const void *weight,
                                    const float *w_scale, const void *bias, const void *residual,
                                    void *y, const void *gamma, const void *beta, float eps,
                                    float q_scale, void *q, void *workspace,
                                    size_t workspace_bytes, void *stream) {
    if (!d) return fail(WVC_ERR_ARG, "conv descriptor is NULL");
    if (d->dtype != WVC_E4M3)
        return fail(WVC_ERR_ARG, "wvc_causal_conv3d_e4m3_norm_fwd needs d->dtype == WVC_E4M3");
    ConvPlan pl;
    int rc = plan_conv(d, &pl, /*count=*/false);  // conv_fwd below counts the call
    if (rc) return rc;
    if (d->c_out % 8 != 0 || d->c_out > 2048) {
        g_rejected++;
        return fail(WVC_ERR_UNSUPPORTED, "the conv + norm call needs C_out %% 8 == 0 and C_out <= 2048");
    }
    if (!gamma) return fail(WVC_ERR_ARG, "gamma is NULL");
    if (!(eps > 0.f)) return fail(WVC_ERR_ARG, "eps must be > 0");
    if (!(q_scale > 0.f) || !(q_scale < INFINITY))
        return fail(WVC_ERR_ARG, "q_scale must be finite and > 0");
    const long positions = (long)d->n * pl.call.to * pl.call.ho * pl.call.wo;
    if (d->t > 0 && positions > 0 && !q) return fail(WVC_ERR_ARG, "q is NULL");
    if (!ws_ok(workspace, workspace_bytes)) return fail(WVC_ERR_ARG, "workspace is NULL but workspace_bytes > 0");
    const size_t conv_need = align256(route_ws_bytes(pl, d->weight_layout == WVC_WEIGHT_PACKED));
    const size_t need = conv_need + align256(pl.y_bytes);
    if (workspace_bytes < need)
        return fail(WVC_ERR_WORKSPACE, "workspace of %zu bytes, %zu needed", workspace_bytes, need);
    const Buf bufs[] = {
        {x, pl.x_bytes, false, "x"},
        {cache_in, pl.cache_bytes, false, "cache_in"},
        {cache_out, pl.cache_bytes, true, "cache_out"},
        {residual, pl.y_bytes, false, "residual"},
        {y, pl.y_bytes, true, "y"},
        {gamma, (size_t)d->c_out * 2, false, "gamma"},
        {beta, (size_t)d->c_out * 2, false, "beta"},
        {q, pl.y_bytes / 2, true, "q"},
        {workspace, workspace_bytes, true, "workspace"},
    };
    rc = check_aliasing(bufs, 9);
    if (rc) return rc;
    hipStream_t s = static_cast<hipStream_t>(stream);
    char *ws = static_cast<char *>(workspace);
    void *yy = y ? y : ws + conv_need;
    // On a split-K plan the reduce is fused into the norm, as in the bf16
    // call; the norm kernel also applies the two scales in the reduce's order.
    const bool fuse = aligned(gamma, 16) && aligned(beta, 16) && aligned(bias, 16) &&
                      aligned(residual, 16) && aligned(y, 16) && aligned(w_scale, 16) &&
                      aligned(q, 16);
    wvc::ConvPartials parts;
    if ((rc = conv_fwd(d, x, cache_in, cache_out, weight, bias, residual, yy, ws, conv_need, s,
                       fuse ? &parts : nullptr, x_scale, w_scale)))
        return rc;
    if (parts.S > 1)
        return hip_status(wvc::launch_rmsnorm_silu_from_partials(parts, bias, gamma, beta, q, positions,
                                                                 d->c_out, eps, 1, s, w_scale, x_scale,
                                                                 1.f / q_scale, residual, y),
                          "norm launch");
    if (d->t == 0 || positions == 0) return WVC_OK;
    return hip_status(wvc::launch_rmsnorm_silu_e4m3(yy, gamma, beta, q, positions, d->c_out, eps, 1,
                                                    1.f / q_scale, s),
                      "norm launch");
}

size_t wvc_conv3d_packed_weight_bytes(const wvc_conv3d_desc *d) {
    ConvPlan pl;
    if (plan_conv(d, &pl, /*count=*/false)) return (size_t)-1;
    if (pl.route == wvc::ConvRoute::Generic) {
        fail(WVC_ERR_UNSUPPORTED, "packed weights exist only for the MFMA routes");
        return (size_t)-1;
    }
    return route_packed_bytes(pl);
}

int wvc_conv3d_pack_weights(const wvc_conv3d_desc *d, const void *weight, void *packed,
                            void *stream) {
    ConvPlan pl;
    int rc = plan_conv(d, &pl, /*count=*/false);
    if (rc) return rc;
    if (pl.route == wvc::ConvRoute::Generic)
        return fail(WVC_ERR_UNSUPPORTED, "packed weights exist only for the MFMA routes");
    if (!weight || !packed) return fail(WVC_ERR_ARG, "weight or packed is NULL");
    if (!aligned(weight, 2) || !aligned(packed, 16))
        return fail(WVC_ERR_ARG, "packed weights need a 16-byte aligned buffer");
    const size_t std_bytes =
        (size_t)d->c_out * d->c_in * d->kt * d->kh * d->kw * (d->dtype == WVC_E4M3 ? 1 : 2);
    const Buf bufs[] = {{weight, std_bytes, false, "weight"},
                        {packed, route_packed_bytes(pl), true, "packed"}};
    rc = check_aliasing(bufs, 2);
    if (rc) return rc;
    hipStream_t s = static_cast<hipStream_t>(stream);
    return hip_status(strided_route(pl.route) ? wvc::launch_strided_pack(pl.call, weight, packed, s)
                                              : wvc::launch_pack_weights(pl.call, weight, packed, s),
                      "weight packing launch");
}

int wvc_quantize_e4m3(const void *x, int dtype, int64_t count, float scale, void *q, void *stream) {
    if (dtype != WVC_BF16 && dtype != WVC_F32)
        return fail(WVC_ERR_UNSUPPORTED, "the quantiser reads WVC_BF16 or WVC_F32, not dtype %d", dtype);
    if (count < 0) return fail(WVC_ERR_ARG, "count < 0");
    if (!(scale > 0.f) || !(scale < INFINITY)) return fail(WVC_ERR_ARG, "scale must be finite and > 0");
    if (count > 0 && (!x || !q)) return fail(WVC_ERR_ARG, "x or q is NULL");
    const Buf bufs[] = {{x, (size_t)count * elem_bytes(dtype), false, "x"}, {q, (size_t)count, true, "q"}};
    int rc = check_aliasing(bufs, 2);
    if (rc) return rc;
    const float qr = 1.f / scale;  // fp32, IEEE
    return hip_status(wvc::launch_quantize_e4m3(x, dtype == WVC_BF16, (long)count, qr, q,
                                                static_cast<hipStream_t>(stream)),
                      "quantiser launch");
}

int wvc_quantize_rows_e4m3(const void *x, int dtype, int64_t rows, int64_t cols, void *q,
                           float *scale, void *stream) {
    if (dtype != WVC_BF16 && dtype != WVC_F32)
        return fail(WVC_ERR_UNSUPPORTED, "the quantiser reads WVC_BF16 or WVC_F32, not dtype %d", dtype);
    if (rows < 0 || cols < 1 || rows > 0x7fffffff) return fail(WVC_ERR_ARG, "bad rows/cols");
    size_t count;
    if (!mul_ok((size_t)rows, (size_t)cols, &count)) return fail(WVC_ERR_ARG, "tensor size overflows");
    if (rows > 0 && (!x || !q || !scale)) return fail(WVC_ERR_ARG, "x, q or scale is NULL");
    const Buf bufs[] = {{x, count * elem_bytes(dtype), false, "x"},
                        {q, count, true, "q"},
                        {scale, (size_t)rows * 4, true, "scale"}};
    int rc = check_aliasing(bufs, 3);
    if (rc) return rc;
    return hip_status(wvc::launch_quantize_rows_e4m3(x, dtype == WVC_BF16, (long)rows, (long)cols, q,
                                                     scale, static_cast<hipStream_t>(stream)),
                      "row quantiser launch");
}

int wvc_rmsnorm_silu_e4m3(const void *x, const void *gamma, const void *beta, void *q, int n, int c,
                          int t, int h, int w, float eps, int apply_silu, float scale, void *stream) {
    if (n < 1 || c < 1 || t < 0 || h < 1 || w < 1)
        return fail(WVC_ERR_ARG, "bad shape n=%d c=%d t=%d h=%d w=%d", n, c, t, h, w);
    if (!(eps > 0.f)) return fail(WVC_ERR_ARG, "eps must be > 0");
    if (!(scale > 0.f) || !(scale < INFINITY)) return fail(WVC_ERR_ARG, "scale must be finite and > 0");
    if (!gamma) return fail(WVC_ERR_ARG, "gamma is NULL");
    const long positions = (long)n * t * h * w;
    if (positions > 0 && (!x || !q)) return fail(WVC_ERR_ARG, "x or q is NULL");
    const size_t elems = (size_t)positions * c;
    const Buf bufs[] = {{x, elems * 2, false, "x"},
                        {q, elems, true, "q"},
                        {gamma, (size_t)c * 2, false, "gamma"},
                        {beta, (size_t)c * 2, false, "beta"}};
    int rc = check_aliasing(bufs, 4);
    if (rc) return rc;
    return hip_status(wvc::launch_rmsnorm_silu_e4m3(x, gamma, beta, q, positions, c, eps, apply_silu,
                                                    1.f / scale, static_cast<hipStream_t>(stream)),
                      "rmsnorm e4m3 launch");
}

const char *wvc_conv3d_kernel_name(const wvc_conv3d_desc *d) {
    thread_local char name[160];
    name[0] = 0;
    ConvPlan pl;
    if (plan_conv(d, &pl, /*count=*/false)) return name;  // a query is not a call
    switch (pl.route) {
        case wvc::ConvRoute::Generic: snprintf(name, sizeof(name), "direct_conv_kernel"); break;
        case wvc::ConvRoute::FastTemporal:
        case wvc::ConvRoute::FastSpatial2:
            snprintf(name, sizeof(name), "%s", wvc::strided_kernel_name(pl.call, false));
            break;
        default: wvc::igemm_kernel_name(pl.call, pl.route, name, sizeof(name)); break;
    }
    return name;
}

int wvc_conv3d_cache_frames(const wvc_conv3d_desc *d) {
    if (!d || d->kt < 1 || d->dil_t < 1) return -1;
    return d->dil_t * (d->kt - 1);
}

int wvc_rmsnorm_silu(const void *x, const void *gamma, const void *beta, void *y, int n, int c,
                     int t, int h, int w, int dtype, float eps, int apply_silu, void *stream) {
    return norm_fwd(x, gamma, beta, y, n, c, t, h, w, dtype, eps, apply_silu,
                    static_cast<hipStream_t>(stream));
}

size_t wvc_resblock_workspace_bytes(const wvc_resblock_desc *d) {
    BlockLayout L;
    if (plan_block(d, &L)) return (size_t)-1;
    return L.total;
}

namespace {

// Checks shared by the block entry points: the descriptor, the parameters the
// given half uses, the workspace size; fills the two conv descriptors.
int check_block(const wvc_resblock_desc *d, const wvc_resblock_params *p, bool front, bool back,
                size_t workspace_bytes, const void *workspace, BlockLayout *L,
                wvc_conv3d_desc *c1, wvc_conv3d_desc *c2) {
    int rc = plan_block(d, L);
    if (rc) return rc;
    if (!p) return fail(WVC_ERR_ARG, "params is NULL");
    if (front && (!p->gamma1 || !p->w1 || !p->gamma2))
        return fail(WVC_ERR_ARG, "gamma1, w1 and gamma2 are required");
    if (back && !p->w2) return fail(WVC_ERR_ARG, "w2 is required");
    const bool proj = d->c_in != d->c_out;
    if (back && proj && !p->w_short) return fail(WVC_ERR_ARG, "C_in != C_out needs w_short");
    if (back && !proj && p->w_short) return fail(WVC_ERR_ARG, "w_short given but C_in == C_out");
    if (workspace_bytes < L->total || (!workspace && L->total))
        return fail(WVC_ERR_WORKSPACE, "workspace of %zu bytes, %zu needed", workspace_bytes,
                    L->total);
    *c1 = wvc_conv3d_desc{};
    c1->n = d->n; c1->c_in = d->c_in; c1->c_out = d->c_out; c1->t = d->t; c1->h = d->h; c1->w = d->w;
    c1->kt = c1->kh = c1->kw = 3;
    c1->stride_t = c1->stride_h = c1->stride_w = 1;
    c1->pad_h = c1->pad_w = 1;
    c1->dil_t = c1->dil_h = c1->dil_w = 1;
    c1->groups = 1;
    c1->dtype = d->dtype;
    c1->weight_layout = d->weights_packed ? WVC_WEIGHT_PACKED : WVC_WEIGHT_STANDARD;
    c1->cu_limit = d->cu_limit;
    *c2 = *c1;
    c2->c_in = d->c_out;
    // Validate the convs (and strict mode) before enqueueing anything.
    ConvPlan pl1, pl2;
    if (front && (rc = plan_conv(c1, &pl1))) return rc;
    if (back && (rc = plan_conv(c2, &pl2))) return rc;
    if (strict_on() && ((front && pl1.route == wvc::ConvRoute::Generic) ||
                        (back && pl2.route == wvc::ConvRoute::Generic))) {
        g_rejected++;
        return fail(WVC_ERR_STRICT, "strict mode: a block conv would take the generic route");
    }
    return WVC_OK;
}

// h2 = SiLU(norm2(conv1(SiLU(norm1(x)) | cache1))).
int block_front(const wvc_resblock_desc *d, const wvc_conv3d_desc &c1, const BlockLayout &L,
                const void *x, void *h2, const wvc_resblock_params *p, const void *cache1_in,
                void *cache1_out, char *ws, hipStream_t s) {
    const size_t pos = (size_t)d->n * d->t * d->h * d->w;
    void *h1 = ws + L.h1, *a1 = ws + L.a1;
    int rc;
    if ((rc = norm_fwd(x, p->gamma1, p->beta1, h1, d->n, d->c_in, d->t, d->h, d->w, d->dtype,
                       d->eps, 1, s)))
        return rc;
    void *cws = ws + L.conv;
    // On a split-K plan conv1's reduce is fused into norm2: the norm kernel
    // adds the partial sums and the bias and rounds to bf16 itself (the value
    // a1 would hold), so a1 is never written.
    // (Only where the vector norm applies: bf16, 16-byte aligned parameters.)
    const bool fuse = d->dtype == WVC_BF16 && d->c_out % 8 == 0 && d->c_out <= 2048 &&
                      aligned(p->gamma2, 16) &&
                      aligned(p->beta2, 16) && aligned(p->b1, 16) && aligned(h2, 16);
    wvc::ConvPartials parts;
    if ((rc = conv_fwd(&c1, h1, cache1_in, cache1_out, p->w1, p->b1, nullptr, a1, cws, L.conv_bytes,
                       s, fuse ? &parts : nullptr)))
        return rc;
    if (parts.S > 1) {
        const hipError_t err = wvc::launch_rmsnorm_silu_from_partials(
            parts, p->b1, p->gamma2, p->beta2, h2, (long)pos, d->c_out, d->eps, 1, s);
        if (err != hipSuccess) return hip_status(err, "norm launch");
        return WVC_OK;
    }
    return norm_fwd(a1, p->gamma2, p->beta2, h2, d->n, d->c_out, d->t, d->h, d->w, d->dtype, d->eps,
                    1, s);
}

// y = conv2(h2 | cache2) + shortcut(x).
int block_back(const wvc_resblock_desc *d, const wvc_conv3d_desc &c1, const wvc_conv3d_desc &c2,
               const BlockLayout &L, const void *h2, const void *x, void *y,
               const wvc_resblock_params *p, const void *cache2_in, void *cache2_out, char *ws,
               hipStream_t s) {
    void *cws = ws + L.conv;
    const void *shortcut = x;
    if (d->c_in != d->c_out) {
        wvc_conv3d_desc cs = c1;
        cs.kt = cs.kh = cs.kw = 1;
        cs.pad_h = cs.pad_w = 0;
        void *sc = ws + L.sc;
        const int rc = conv_fwd(&cs, x, nullptr, nullptr, p->w_short, p->b_short, nullptr, sc, cws,
                                L.conv_bytes, s);
        if (rc) return rc;
        shortcut = sc;
    }
    return conv_fwd(&c2, h2, cache2_in, cache2_out, p->w2, p->b2, shortcut, y, cws, L.conv_bytes, s);
}

// ---- the 8-bit residual block
struct Block8Layout {
    size_t conv_bytes, q, h, total;
};

int plan_block8(const wvc_resblock_desc *d, Block8Layout *L, wvc_conv3d_desc *c, ConvPlan *pl,
                bool count) {
    if (!d) return fail(WVC_ERR_ARG, "resblock descriptor is NULL");
    if (d->dtype != WVC_BF16)
        return fail(WVC_ERR_UNSUPPORTED, "the 8-bit block reads and writes bf16 (dtype WVC_BF16)");
    if (d->n < 1 || d->c_in < 1 || d->c_out < 1 || d->t < 0 || d->h < 1 || d->w < 1)
        return fail(WVC_ERR_ARG, "bad resblock shape");
    if (d->c_in != d->c_out)
        return fail(WVC_ERR_UNSUPPORTED, "the 8-bit block has the identity shortcut (C_in == C_out)");
    if (!(d->eps > 0.f)) return fail(WVC_ERR_ARG, "eps must be > 0");
    if (d->weights_packed != 0 && d->weights_packed != 1)
        return fail(WVC_ERR_ARG, "weights_packed must be 0 or 1");
    *c = wvc_conv3d_desc{};
    c->n = d->n; c->c_in = d->c_in; c->c_out = d->c_out; c->t = d->t; c->h = d->h; c->w = d->w;
    c->kt = c->kh = c->kw = 3;
    c->stride_t = c->stride_h = c->stride_w = 1;
    c->pad_h = c->pad_w = 1;
    c->dil_t = c->dil_h = c->dil_w = 1;
    c->groups = 1;
    c->dtype = WVC_E4M3;
    c->weight_layout = d->weights_packed ? WVC_WEIGHT_PACKED : WVC_WEIGHT_STANDARD;
    c->cu_limit = d->cu_limit;
    const int rc = plan_conv(c, pl, count);
    if (rc) return rc;
    const size_t pos = (size_t)d->n * d->t * d->h * d->w;
    L->conv_bytes = align256(route_ws_bytes(*pl, d->weights_packed != 0));
    L->q = L->conv_bytes;                                  // codes of a norm output
    L->h = L->q + align256(pos * d->c_in);                 // conv1 output, when not fused
    L->total = L->h + align256(pos * d->c_out * 2);
    return WVC_OK;
}

}  // namespace

size_t wvc_resblock_e4m3_workspace_bytes(const wvc_resblock_desc *d) {
    Block8Layout L;
    wvc_conv3d_desc c;
    ConvPlan pl;
    if (plan_block8(d, &L, &c, &pl, false)) return (size_t)-1;
    return L.total;
}

int wvc_resblock_e4m3_fwd(const wvc_resblock_desc *d, const void *x, void *y,
                          const wvc_resblock_e4m3_params *p, const void *cache1_in,
                          void *cache1_out, const void *cache2_in, void *cache2_out,
                          void *workspace, size_t workspace_bytes, void *stream) {
    Block8Layout L;
    wvc_conv3d_desc c;
    ConvPlan pl;
    int rc = plan_block8(d, &L, &c, &pl, true);
    if (rc) return rc;
    if (!p) return fail(WVC_ERR_ARG, "params is NULL");
    if (!p->gamma1 || !p->gamma2 || !p->w1 || !p->w2 || !p->w1_scale || !p->w2_scale)
        return fail(WVC_ERR_ARG, "gamma1, gamma2, w1, w2, w1_scale and w2_scale are required");
    if (!(p->s1 > 0.f) || !(p->s1 < INFINITY) || !(p->s2 > 0.f) || !(p->s2 < INFINITY))
        return fail(WVC_ERR_ARG, "activation scales must be finite and > 0");
    if (d->t > 0 && (!x || !y)) return fail(WVC_ERR_ARG, "x or y is NULL");
    if (workspace_bytes < L.total || (!workspace && L.total))
        return fail(WVC_ERR_WORKSPACE, "workspace of %zu bytes, %zu needed", workspace_bytes, L.total);
    const size_t pos = (size_t)d->n * d->t * d->h * d->w;
    const size_t plane = (size_t)d->n * 2 * d->h * d->w * d->c_in;
    const Buf bufs[] = {
        {x, pos * d->c_in * 2, false, "x"},
        {y, pos * d->c_out * 2, true, "y"},
        {cache1_in, plane, false, "cache1_in"},
        {cache1_out, plane, true, "cache1_out"},
        {cache2_in, plane, false, "cache2_in"},
        {cache2_out, plane, true, "cache2_out"},
        {workspace, workspace_bytes, true, "workspace"},
    };
    if ((rc = check_aliasing(bufs, 7))) return rc;
    if (d->t == 0) {  // no frames: the caches pass through
        wvc::ConvPartials none;
        if ((rc = conv_fwd(&c, x, cache1_in, cache1_out, p->w1, p->b1, nullptr, nullptr, workspace,
                           L.conv_bytes, static_cast<hipStream_t>(stream), &none, p->s1, p->w1_scale)))
            return rc;
        return conv_fwd(&c, x, cache2_in, cache2_out, p->w2, p->b2, nullptr, nullptr, workspace,
                        L.conv_bytes, static_cast<hipStream_t>(stream), &none, p->s2, p->w2_scale);
    }
    hipStream_t s = static_cast<hipStream_t>(stream);
    char *ws = static_cast<char *>(workspace);
    void *q = ws + L.q, *h = ws + L.h;
    hipError_t err = wvc::launch_rmsnorm_silu_e4m3(x, p->gamma1, p->beta1, q, (long)pos, d->c_in,
                                                   d->eps, 1, 1.f / p->s1, s);
    if (err != hipSuccess) return hip_status(err, "norm launch");
    // conv1's split-K partial sums go straight into norm2 (scales, bias, one
    // bf16 rounding, the norm, the codes), where the vector norm applies
    const bool fuse = d->c_out % 8 == 0 && d->c_out <= 2048 && aligned(p->gamma2, 16) &&
                      aligned(p->beta2, 16) && aligned(p->b1, 16) && aligned(p->w1_scale, 16) &&
                      aligned(q, 16);
    wvc::ConvPartials parts;
    if ((rc = conv_fwd(&c, q, cache1_in, cache1_out, p->w1, p->b1, nullptr, h, ws, L.conv_bytes, s,
                       fuse ? &parts : nullptr, p->s1, p->w1_scale)))
        return rc;
    if (parts.S > 1)
        err = wvc::launch_rmsnorm_silu_from_partials(parts, p->b1, p->gamma2, p->beta2, q, (long)pos,
                                                     d->c_out, d->eps, 1, s, p->w1_scale, p->s1,
                                                     1.f / p->s2);
    else
        err = wvc::launch_rmsnorm_silu_e4m3(h, p->gamma2, p->beta2, q, (long)pos, d->c_out, d->eps, 1,
                                            1.f / p->s2, s);
    if (err != hipSuccess) return hip_status(err, "norm launch");
    return conv_fwd(&c, q, cache2_in, cache2_out, p->w2, p->b2, x, y, ws, L.conv_bytes, s, nullptr,
                    p->s2, p->w2_scale);
}

int wvc_resblock_fwd(const wvc_resblock_desc *d, const void *x, void *y,
                     const wvc_resblock_params *p, const void *cache1_in, void *cache1_out,
                     const void *cache2_in, void *cache2_out, void *workspace,
                     size_t workspace_bytes, void *stream) {
    BlockLayout L;
    wvc_conv3d_desc c1, c2;
    int rc = check_block(d, p, true, true, workspace_bytes, workspace, &L, &c1, &c2);
    if (rc) return rc;
    if (d->t > 0 && (!x || !y)) return fail(WVC_ERR_ARG, "x or y is NULL");
    const int e = elem_bytes(d->dtype);
    const size_t pos = (size_t)d->n * d->t * d->h * d->w;
    const size_t plane_in = (size_t)d->n * 2 * d->h * d->w;
    const Buf bufs[] = {
        {x, pos * d->c_in * e, false, "x"},
        {y, pos * d->c_out * e, true, "y"},
        {cache1_in, plane_in * d->c_in * e, false, "cache1_in"},
        {cache1_out, plane_in * d->c_in * e, true, "cache1_out"},
        {cache2_in, plane_in * d->c_out * e, false, "cache2_in"},
        {cache2_out, plane_in * d->c_out * e, true, "cache2_out"},
        {workspace, workspace_bytes, true, "workspace"},
    };
    if ((rc = check_aliasing(bufs, 7))) return rc;
    hipStream_t s = static_cast<hipStream_t>(stream);
    char *ws = static_cast<char *>(workspace);
    void *h2 = ws + L.h2;
    if ((rc = block_front(d, c1, L, x, h2, p, cache1_in, cache1_out, ws, s))) return rc;
    return block_back(d, c1, c2, L, h2, x, y, p, cache2_in, cache2_out, ws, s);
}

int wvc_resblock_front(const wvc_resblock_desc *d, const void *x, void *h2,
                       const wvc_resblock_params *p, const void *cache1_in, void *cache1_out,
                       void *workspace, size_t workspace_bytes, void *stream) {
    BlockLayout L;
    wvc_conv3d_desc c1, c2;
    int rc = check_block(d, p, true, false, workspace_bytes, workspace, &L, &c1, &c2);
    if (rc) return rc;
    if (d->t > 0 && (!x || !h2)) return fail(WVC_ERR_ARG, "x or h2 is NULL");
    const int e = elem_bytes(d->dtype);
    const size_t pos = (size_t)d->n * d->t * d->h * d->w;
    const size_t plane_in = (size_t)d->n * 2 * d->h * d->w;
    const Buf bufs[] = {
        {x, pos * d->c_in * e, false, "x"},
        {h2, pos * d->c_out * e, true, "h2"},
        {cache1_in, plane_in * d->c_in * e, false, "cache1_in"},
        {cache1_out, plane_in * d->c_in * e, true, "cache1_out"},
        {workspace, workspace_bytes, true, "workspace"},
    };
    if ((rc = check_aliasing(bufs, 5))) return rc;
    return block_front(d, c1, L, x, h2, p, cache1_in, cache1_out, static_cast<char *>(workspace),
                       static_cast<hipStream_t>(stream));
}

int wvc_resblock_back(const wvc_resblock_desc *d, const void *h2, const void *x, void *y,
                      const wvc_resblock_params *p, const void *cache2_in, void *cache2_out,
                      void *workspace, size_t workspace_bytes, void *stream) {
    BlockLayout L;
    wvc_conv3d_desc c1, c2;
    int rc = check_block(d, p, false, true, workspace_bytes, workspace, &L, &c1, &c2);
    if (rc) return rc;
    if (d->t > 0 && (!x || !h2 || !y)) return fail(WVC_ERR_ARG, "h2, x or y is NULL");
    const int e = elem_bytes(d->dtype);
    const size_t pos = (size_t)d->n * d->t * d->h * d->w;
    const size_t plane_out = (size_t)d->n * 2 * d->h * d->w;
    const Buf bufs[] = {
        {h2, pos * d->c_out * e, false, "h2"},
        {x, pos * d->c_in * e, false, "x"},
        {y, pos * d->c_out * e, true, "y"},
        {cache2_in, plane_out * d->c_out * e, false, "cache2_in"},
        {cache2_out, plane_out * d->c_out * e, true, "cache2_out"},
        {workspace, workspace_bytes, true, "workspace"},
    };
    if ((rc = check_aliasing(bufs, 6))) return rc;
    return block_back(d, c1, c2, L, h2, x, y, p, cache2_in, cache2_out,
                      static_cast<char *>(workspace), static_cast<hipStream_t>(stream));
}

int wvc_cache_reset(void *cache, size_t bytes, void *stream) {
    if (bytes == 0) return WVC_OK;
    if (!cache) return fail(WVC_ERR_ARG, "cache is NULL");
    if (bytes % 4 != 0 || !aligned(cache, 4))
        return fail(WVC_ERR_ARG, "cache reset needs 4-byte aligned pointer and size");
    return hip_status(wvc::launch_fill_zero(cache, bytes, static_cast<hipStream_t>(stream)),
                      "cache reset launch");
}

int wvc_upsample_nearest2x(const void *x, void *y, int n, int c, int t, int h, int w, int dtype,
                           void *stream) {
    const int e = elem_bytes(dtype);
    if (!e) return fail(WVC_ERR_UNSUPPORTED, "dtype %d is neither WVC_F32 nor WVC_BF16", dtype);
    if (n < 1 || c < 1 || t < 0 || h < 1 || w < 1) return fail(WVC_ERR_ARG, "bad upsample shape");
    const long planes = (long)n * t;
    if (planes > 0 && (!x || !y)) return fail(WVC_ERR_ARG, "x or y is NULL");
    const size_t in_bytes = (size_t)planes * h * w * c * e;
    const Buf bufs[] = {{x, in_bytes, false, "x"}, {y, in_bytes * 4, true, "y"}};
    int rc = check_aliasing(bufs, 2);
    if (rc) return rc;
    return hip_status(
        wvc::launch_upsample2x(x, y, planes, h, w, c, e, static_cast<hipStream_t>(stream)),
        "upsample launch");
}

int wvc_tile_extract(const void *x, void *tile, int n, int c, int t, int h, int w, int y0, int x0,
                     int th, int tw, int dtype, void *stream) {
    const int e = elem_bytes(dtype);
    if (!e) return fail(WVC_ERR_UNSUPPORTED, "dtype %d is neither WVC_F32 nor WVC_BF16", dtype);
    if (n < 1 || c < 1 || t < 0 || h < 1 || w < 1 || th < 1 || tw < 1 || y0 < 0 || x0 < 0 ||
        y0 + th > h || x0 + tw > w)
        return fail(WVC_ERR_ARG, "tile window %dx%d at (%d, %d) outside the %dx%d frame", th, tw, y0,
                    x0, h, w);
    const long planes = (long)n * t;
    if (planes > 0 && (!x || !tile)) return fail(WVC_ERR_ARG, "x or tile is NULL");
    const Buf bufs[] = {{x, (size_t)planes * h * w * c * e, false, "x"},
                        {tile, (size_t)planes * th * tw * c * e, true, "tile"}};
    int rc = check_aliasing(bufs, 2);
    if (rc) return rc;
    return hip_status(wvc::launch_tile_extract(x, tile, planes, h, w, y0, x0, th, tw, c, e,
                                               static_cast<hipStream_t>(stream)),
                      "tile extract launch");
}

int wvc_tile_blend(const void *tile, float *acc, float *wsum, int n, int c, int t, int th, int tw,
                   int h, int w, int y0, int x0, int ramp_top, int ramp_bottom, int ramp_left,
                   int ramp_right, int dtype, void *stream) {
    const int e = elem_bytes(dtype);
    if (!e) return fail(WVC_ERR_UNSUPPORTED, "dtype %d is neither WVC_F32 nor WVC_BF16", dtype);
    if (n < 1 || c < 1 || c % 4 != 0 || t < 0 || h < 1 || w < 1 || th < 1 || tw < 1 || y0 < 0 ||
        x0 < 0 || y0 + th > h || x0 + tw > w)
        return fail(WVC_ERR_ARG, "bad tile blend shape (C %% 4 == 0, tile inside the frame)");
    if (ramp_top < 0 || ramp_bottom < 0 || ramp_left < 0 || ramp_right < 0 || ramp_top > th ||
        ramp_bottom > th || ramp_left > tw || ramp_right > tw)
        return fail(WVC_ERR_ARG, "ramps must lie in [0, tile size]");
    const long planes = (long)n * t;
    if (planes > 0 && (!tile || !acc || !wsum)) return fail(WVC_ERR_ARG, "tile, acc or wsum is NULL");
    if (!aligned(tile, 8) || !aligned(acc, 16) || !aligned(wsum, 4))
        return fail(WVC_ERR_ARG, "tile blend needs 8-byte aligned tile, 16-byte aligned acc");
    const Buf bufs[] = {{tile, (size_t)planes * th * tw * c * e, false, "tile"},
                        {acc, (size_t)planes * h * w * c * 4, true, "acc"},
                        {wsum, (size_t)h * w * 4, true, "wsum"}};
    int rc = check_aliasing(bufs, 3);
    if (rc) return rc;
    return hip_status(wvc::launch_tile_blend(tile, acc, wsum, planes, c, th, tw, h, w, y0, x0, ramp_top,
                                             ramp_bottom, ramp_left, ramp_right, dtype == WVC_BF16,
                                             static_cast<hipStream_t>(stream)),
                      "tile blend launch");
}

int wvc_tile_blend_finish(const float *acc, const float *wsum, void *y, int n, int c, int t, int h,
                          int w, int dtype, void *stream) {
    const int e = elem_bytes(dtype);
    if (!e) return fail(WVC_ERR_UNSUPPORTED, "dtype %d is neither WVC_F32 nor WVC_BF16", dtype);
    if (n < 1 || c < 1 || c % 4 != 0 || t < 0 || h < 1 || w < 1)
        return fail(WVC_ERR_ARG, "bad tile finish shape (C %% 4 == 0)");
    const long planes = (long)n * t;
    if (planes > 0 && (!acc || !wsum || !y)) return fail(WVC_ERR_ARG, "acc, wsum or y is NULL");
    if (!aligned(acc, 16) || !aligned(y, 8)) return fail(WVC_ERR_ARG, "misaligned acc or y");
    const Buf bufs[] = {{acc, (size_t)planes * h * w * c * 4, false, "acc"},
                        {wsum, (size_t)h * w * 4, false, "wsum"},
                        {y, (size_t)planes * h * w * c * e, true, "y"}};
    int rc = check_aliasing(bufs, 3);
    if (rc) return rc;
    return hip_status(wvc::launch_tile_finish(acc, wsum, y, planes, c, (long)h * w, dtype == WVC_BF16,
                                              static_cast<hipStream_t>(stream)),
                      "tile finish launch");
}

struct wvc_graph {
    hipGraph_t graph;
    hipGraphExec_t exec;
};

int wvc_graph_capture_begin(void *stream) {
    if (!stream) return fail(WVC_ERR_ARG, "the null stream cannot be captured; pass a created stream");
    return hip_status(hipStreamBeginCapture(static_cast<hipStream_t>(stream),
                                            hipStreamCaptureModeThreadLocal),
                      "begin capture");
}

int wvc_graph_capture_end(void *stream, wvc_graph **graph) {
    if (!graph) return fail(WVC_ERR_ARG, "graph is NULL");
    *graph = nullptr;
    if (!stream) return fail(WVC_ERR_ARG, "stream is NULL");
    hipGraph_t g = nullptr;
    hipError_t err = hipStreamEndCapture(static_cast<hipStream_t>(stream), &g);
    if (err != hipSuccess) {
        if (g) (void)hipGraphDestroy(g);
        return hip_status(err, "end capture");
    }
    if (!g) return fail(WVC_ERR_HIP, "end capture returned no graph");
    hipGraphExec_t exec = nullptr;
    hipGraphNode_t err_node = nullptr;
    char log[256] = "";
    err = hipGraphInstantiate(&exec, g, &err_node, log, sizeof(log));
    if (err != hipSuccess) {
        (void)hipGraphDestroy(g);
        return fail(WVC_ERR_HIP, "graph instantiate: %s %s", hipGetErrorString(err), log);
    }
    wvc_graph *h = new (std::nothrow) wvc_graph{g, exec};
    if (!h) {
        (void)hipGraphExecDestroy(exec);
        (void)hipGraphDestroy(g);
        return fail(WVC_ERR_HIP, "out of host memory for the graph handle");
    }
    *graph = h;
    return WVC_OK;
}

int wvc_graph_launch(const wvc_graph *graph, void *stream) {
    if (!graph) return fail(WVC_ERR_ARG, "graph is NULL");
    return hip_status(hipGraphLaunch(graph->exec, static_cast<hipStream_t>(stream)), "graph launch");
}

int wvc_graph_destroy(wvc_graph *graph) {
    if (!graph) return WVC_OK;
    const hipError_t e1 = hipGraphExecDestroy(graph->exec);
    const hipError_t e2 = hipGraphDestroy(graph->graph);
    delete graph;
    if (e1 != hipSuccess) return hip_status(e1, "graph exec destroy");
    return hip_status(e2, "graph destroy");
}

void wvc_set_strict(int on) { g_strict.store(on ? 1 : 0); }
int wvc_get_strict(void) { return strict_on(); }

void wvc_get_counters(wvc_counters *out) {
    if (!out) return;
    out->fast_3x3x3 = g_fast3.load();
    out->fast_1x1x1 = g_fast1.load();
    out->generic = g_generic.load();
    out->rejected = g_rejected.load();
    out->fast_strided = g_strided.load();
}

void wvc_reset_counters(void) {
    g_fast3 = 0;
    g_fast1 = 0;
    g_generic = 0;
    g_rejected = 0;
    g_strided = 0;
}

const char *wvc_last_error(void) { return g_err; }

const char *wvc_version(void) { return "libwvc 0.1 (gfx950)"; }

}  // extern "C"
