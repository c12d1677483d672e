// rmsnorm.hip -- fused channel RMS norm + SiLU, channels-last.
//
// Definition ("Cosmos3 Wan VAE -- engine size vs runtime context memory",
// section 10.2, and section 10.4 for SiLU): for one position (n,t,h,w) with
// channel vector v,  u_c = v_c / max(||v||_2, eps) * sqrt(C) * gamma_c + beta_c,
// y_c = u_c * sigmoid(u_c).  fp32 inside, one rounding at the store.
//
// Bandwidth-bound: every element is read once and written once.  With the
// channels-last layout one position's C channels are contiguous, so a group of
// LPP lanes owns a position and the C/VEC 16-byte chunks are spread over the
// group as chunk j + LPP*i (i < CH): for every i the group reads one
// contiguous run, and consecutive groups read consecutive positions, so each
// load instruction of a wave covers 64/LPP adjacent positions.  The sum of
// squares is reduced across the group with lane shuffles (no LDS).  gamma and
// beta are loaded once per thread: a lane sees the same channels at every
// position it handles.
#include "wvc_internal.h"
#include "wvc.h"

namespace wvc {
namespace {

constexpr int MAX_CH = 8;

template <bool BF16>
struct Vec;
template <>
struct Vec<true> {
    static constexpr int N = 8;
    __device__ static void unpack(uint4 v, float *o) {
        const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            o[2 * k] = bf16_to_f32(w[k] & 0xffffu);
            o[2 * k + 1] = bf16_to_f32(w[k] >> 16);
        }
    }
    __device__ static uint4 pack(const float *o) {
        uint32_t w[4];
#pragma unroll
        for (int k = 0; k < 4; ++k)
            w[k] = (uint32_t)f32_to_bf16(o[2 * k]) | ((uint32_t)f32_to_bf16(o[2 * k + 1]) << 16);
        return make_uint4(w[0], w[1], w[2], w[3]);
    }
};
template <>
struct Vec<false> {
    static constexpr int N = 4;
    __device__ static void unpack(uint4 v, float *o) {
        o[0] = __uint_as_float(v.x);
        o[1] = __uint_as_float(v.y);
        o[2] = __uint_as_float(v.z);
        o[3] = __uint_as_float(v.w);
    }
    __device__ static uint4 pack(const float *o) {
        return make_uint4(__float_as_uint(o[0]), __float_as_uint(o[1]), __float_as_uint(o[2]),
                          __float_as_uint(o[3]));
    }
};

template <bool BF16>
__device__ __forceinline__ float silu(float u) {
    // u * sigmoid(u) = u / (1 + e^-u); bf16 output tolerates the fast exp.
    if (BF16) return u / (1.f + __expf(-u));
    return u / (1.f + expf(-u));
}

template <bool BF16, int LPP>
__global__ void __launch_bounds__(256) rmsnorm_vec_kernel(const uint4 *__restrict__ x,
                                                          const uint4 *__restrict__ gamma,
                                                          const uint4 *__restrict__ beta,
                                                          uint4 *__restrict__ y, long positions,
                                                          int chunks, int ch, float scale,
                                                          float eps, int apply_silu) {
    using V = Vec<BF16>;
    const long gid = (long)blockIdx.x * 256 + threadIdx.x;
    const long pos = gid / LPP;
    const int j = (int)(gid % LPP);
    // Every lane of a group takes part in the shuffles, so no early return
    // before the reduction; lanes past the end load nothing.
    const bool live = pos < positions;

    uint4 raw[MAX_CH];
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < MAX_CH; ++i) {
        if (i < ch && live) {
            raw[i] = x[pos * chunks + j + LPP * i];
            float f[V::N];
            V::unpack(raw[i], f);
#pragma unroll
            for (int k = 0; k < V::N; ++k) s = fmaf(f[k], f[k], s);
        }
    }
#pragma unroll
    for (int off = LPP / 2; off > 0; off >>= 1) s += __shfl_xor(s, off, 64);
    if (!live) return;
    const float r = scale / fmaxf(sqrtf(s), eps);
#pragma unroll
    for (int i = 0; i < MAX_CH; ++i) {
        if (i < ch) {
            const int chunk = j + LPP * i;
            float f[V::N], g[V::N], b[V::N];
            V::unpack(raw[i], f);
            V::unpack(gamma[chunk], g);
            if (beta)
                V::unpack(beta[chunk], b);
            else
#pragma unroll
                for (int k = 0; k < V::N; ++k) b[k] = 0.f;
#pragma unroll
            for (int k = 0; k < V::N; ++k) {
                const float u = f[k] * r * g[k] + b[k];
                f[k] = apply_silu ? silu<BF16>(u) : u;
            }
            y[pos * chunks + chunk] = V::pack(f);
        }
    }
}

// Any C: one thread per position, scalar loop (used when C is not a multiple
// of the 16-byte vector or needs more than MAX_CH chunks per lane).
template <bool BF16>
__global__ void __launch_bounds__(256) rmsnorm_scalar_kernel(const void *xv, const void *gv,
                                                             const void *bv, void *yv,
                                                             long positions, int c, float scale,
                                                             float eps, int apply_silu) {
    const long pos = (long)blockIdx.x * 256 + threadIdx.x;
    if (pos >= positions) return;
    auto load = [](const void *p, long i) -> float {
        return BF16 ? bf16_to_f32(static_cast<const uint16_t *>(p)[i])
                    : static_cast<const float *>(p)[i];
    };
    float s = 0.f;
    for (int k = 0; k < c; ++k) {
        const float v = load(xv, pos * c + k);
        s = fmaf(v, v, s);
    }
    const float r = scale / fmaxf(sqrtf(s), eps);
    for (int k = 0; k < c; ++k) {
        float u = load(xv, pos * c + k) * r * load(gv, k) + (bv ? load(bv, k) : 0.f);
        if (apply_silu) u = silu<BF16>(u);
        if (BF16)
            static_cast<uint16_t *>(yv)[pos * c + k] = f32_to_bf16(u);
        else
            static_cast<float *>(yv)[pos * c + k] = u;
    }
}

template <bool BF16, int LPP>
hipError_t launch_vec(const void *x, const void *g, const void *b, void *y, long positions,
                      int chunks, int ch, float scale, float eps, int silu_on, hipStream_t s) {
    const long threads = positions * LPP;
    const long blocks = (threads + 255) / 256;
    if (blocks > 0x7fffffffL) return hipErrorInvalidValue;
    hipLaunchKernelGGL((rmsnorm_vec_kernel<BF16, LPP>), dim3((unsigned)blocks), dim3(256), 0, s,
                       static_cast<const uint4 *>(x), static_cast<const uint4 *>(g),
                       static_cast<const uint4 *>(b), static_cast<uint4 *>(y), positions, chunks,
                       ch, scale, eps, silu_on);
    return hipGetLastError();
}

template <bool BF16>
hipError_t dispatch(const void *x, const void *g, const void *b, void *y, long positions, int c,
                    float eps, int silu_on, hipStream_t s) {
    const float scale = sqrtf((float)c);
    constexpr int VN = Vec<BF16>::N;
    const bool aligned = ((uintptr_t)x % 16 == 0) && ((uintptr_t)y % 16 == 0) &&
                         ((uintptr_t)g % 16 == 0) && ((uintptr_t)b % 16 == 0);
    if (c % VN == 0 && aligned) {
        const int chunks = c / VN;
        int lpp = 1;
        while (lpp < 16 && chunks % (lpp * 2) == 0) lpp *= 2;
        const int ch = chunks / lpp;
        if (ch <= MAX_CH) {
            switch (lpp) {
                case 1: return launch_vec<BF16, 1>(x, g, b, y, positions, chunks, ch, scale, eps, silu_on, s);
                case 2: return launch_vec<BF16, 2>(x, g, b, y, positions, chunks, ch, scale, eps, silu_on, s);
                case 4: return launch_vec<BF16, 4>(x, g, b, y, positions, chunks, ch, scale, eps, silu_on, s);
                case 8: return launch_vec<BF16, 8>(x, g, b, y, positions, chunks, ch, scale, eps, silu_on, s);
                default: return launch_vec<BF16, 16>(x, g, b, y, positions, chunks, ch, scale, eps, silu_on, s);
            }
        }
    }
    const long blocks = (positions + 255) / 256;
    if (blocks > 0x7fffffffL) return hipErrorInvalidValue;
    hipLaunchKernelGGL(rmsnorm_scalar_kernel<BF16>, dim3((unsigned)blocks), dim3(256), 0, s, x, g,
                       b, y, positions, c, scale, eps, silu_on);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_rmsnorm_silu(const void *x, const void *gamma, const void *beta, void *y,
                               long positions, int c, int dtype, float eps, int apply_silu,
                               hipStream_t s) {
    if (positions <= 0) return hipSuccess;
    if (dtype == WVC_BF16)
        return dispatch<true>(x, gamma, beta, y, positions, c, eps, apply_silu, s);
    return dispatch<false>(x, gamma, beta, y, positions, c, eps, apply_silu, s);
}

}  // namespace wvc
