// conv_direct.hip -- direct causal convolution for every legal descriptor the
// MFMA routes do not cover (fp32, other kernel sizes, spatial stride, padding
// and dilation, temporal dilation).
//
// Definition ("Cosmos3 Wan VAE -- engine size vs runtime context memory",
// section 10.3): y[n,t,ho,wo,co] = sum over kt, kh, kw, ci of
// W[co,kt,kh,kw,ci] * X'[n, t-(kT-1-kt)*dil_t, ho*s_h-p_h+kh*dil_h,
// wo*s_w-p_w+kw*dil_w, ci] (t the chunk frame output t is anchored at: t
// itself for temporal stride 1, t0 + j*s_t under a temporal stride, [P1]
// 10.5), then + bias once ("cache-aware video decoder
// lowering": stride, padding and dilation honoured, bias after the sum).
// Frames before the chunk come from the cache (or are zero); positions outside
// the frame are zero.  One thread per output element, channel fastest so that
// output stores are coalesced; accumulation in fp32.
#include "wvc_internal.h"
#include "wvc.h"

namespace wvc {
namespace {

template <typename T>
__device__ __forceinline__ float ld(const T *p);
template <>
__device__ __forceinline__ float ld<float>(const float *p) { return *p; }
template <>
__device__ __forceinline__ float ld<uint16_t>(const uint16_t *p) { return bf16_to_f32(*p); }

template <typename T>
__device__ __forceinline__ void st(T *p, float v);
template <>
__device__ __forceinline__ void st<float>(float *p, float v) { *p = v; }
template <>
__device__ __forceinline__ void st<uint16_t>(uint16_t *p, float v) { *p = f32_to_bf16(v); }

template <typename T>
__global__ void __launch_bounds__(256) direct_kernel(ConvCall c) {
    const long total = (long)c.n * c.to * c.ho * c.wo * c.cout;
    const long idx = (long)blockIdx.x * 256 + threadIdx.x;
    if (idx >= total) return;
    long r = idx;
    const int co = (int)(r % c.cout);
    r /= c.cout;
    const int wo = (int)(r % c.wo);
    r /= c.wo;
    const int ho = (int)(r % c.ho);
    r /= c.ho;
    const int j = (int)(r % c.to);
    const int n = (int)(r / c.to);
    const int t = c.t0 + j * c.st;  // the chunk frame output j is anchored at

    const T *x = static_cast<const T *>(c.x);
    const T *cache = static_cast<const T *>(c.cache_in);
    const T *w = static_cast<const T *>(c.weight);
    const size_t frame = (size_t)c.h * c.w * c.cin;
    float acc = 0.f;
    for (int kt = 0; kt < c.kt; ++kt) {
        const int ts = t - (c.kt - 1 - kt) * c.dt;
        const T *fp;
        if (ts >= 0)
            fp = x + (size_t)(n * c.t + ts) * frame;
        else if (cache)
            fp = cache + (size_t)(n * c.frames + c.frames + ts) * frame;
        else
            continue;
        for (int kh = 0; kh < c.kh; ++kh) {
            const int hs = ho * c.sh - c.ph + kh * c.dh;
            if (hs < 0 || hs >= c.h) continue;
            for (int kw = 0; kw < c.kw; ++kw) {
                const int ws = wo * c.sw - c.pw + kw * c.dw;
                if (ws < 0 || ws >= c.w) continue;
                const T *xp = fp + ((size_t)hs * c.w + ws) * c.cin;
                const T *wp = w + ((((size_t)co * c.kt + kt) * c.kh + kh) * c.kw + kw) * c.cin;
                for (int ci = 0; ci < c.cin; ++ci) acc = fmaf(ld(wp + ci), ld(xp + ci), acc);
            }
        }
    }
    if (c.bias) acc += ld(static_cast<const T *>(c.bias) + co);
    const size_t o = (size_t)idx;
    if (c.residual) acc += ld(static_cast<const T *>(c.residual) + o);
    st(static_cast<T *>(c.y) + o, acc);
}

}  // namespace

hipError_t launch_conv_direct(const ConvCall &c, hipStream_t s) {
    const long total = (long)c.n * c.to * c.ho * c.wo * c.cout;
    if (total <= 0) return hipSuccess;
    const long blocks = (total + 255) / 256;
    if (blocks > 0x7fffffffL) return hipErrorInvalidValue;
    if (c.dtype == WVC_F32)
        hipLaunchKernelGGL(direct_kernel<float>, dim3((unsigned)blocks), dim3(256), 0, s, c);
    else
        hipLaunchKernelGGL(direct_kernel<uint16_t>, dim3((unsigned)blocks), dim3(256), 0, s, c);
    return hipGetLastError();
}

}  // namespace wvc
