// rmsnorm.hip -- fused channel RMS norm + SiLU, channels-last.
//
// Definition ("Cosmos3 Wan VAE -- engine size vs runtime context memory",
// section 10.2, and section 10.4 for SiLU): for one position (n,t,h,w) with
// channel vector v,  u_c = v_c / max(||v||_2, eps) * sqrt(C) * gamma_c + beta_c,
// y_c = u_c * sigmoid(u_c).  fp32 inside, one rounding at the store.
//
// Bandwidth-bound: every element is read once and written once.  With the
// channels-last layout one position's C channels are contiguous, so a run of
// whole positions is one contiguous block of memory; the kernel below streams
// such blocks with fully coalesced 16-byte accesses and does the per-position
// reduction in LDS.
#include "wvc_internal.h"
#include "wvc.h"

namespace wvc {
namespace {

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
    // gfx950's v_cvt_pk_bf16_f32 (pack2_bf16): the store-side rounding is
    // most of this kernel's ALU work otherwise.
    __device__ static uint4 pack(const float *o) {
        return make_uint4(pack2_bf16(o[0], o[1]), pack2_bf16(o[2], o[3]), pack2_bf16(o[4], o[5]),
                          pack2_bf16(o[6], o[7]));
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
    // u * sigmoid(u) = u / (1 + e^-u).  For a bf16 result the hardware exp2
    // and reciprocal (about 1 ulp of fp32 each) are far inside the final
    // rounding; the fp32 path keeps the accurate exp and division.
    if (BF16) return u * __builtin_amdgcn_rcpf(1.f + __expf(-u));
    return u / (1.f + expf(-u));
}

// Flat layout: a workgroup owns P whole positions, i.e. P*cpp consecutive
// 16-byte chunks (cpp = chunks per position), and thread t takes chunks
// t + 256k (k < K).  Every load and store instruction of a wave then covers
// one contiguous 1 KiB run, whatever C is, so each cache line is read and
// written whole by one instruction.  Per-position sums of squares go through
// LDS: each chunk's partial sum is stored, R lanes per position add them up
// (shuffles inside the R-lane group), and the reciprocal scale comes back
// through LDS.  gamma and beta are staged in LDS once per workgroup.
constexpr int FLAT_MAX_CPP = 256;

// Non-temporal 16-byte accesses for tensors far larger than the caches: the
// data is touched once, so it should not push other lines out of L2 / MALL.
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint4 ld_stream(const uint4 *p) {
    const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(p));
    return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ void st_stream(uint4 *p, uint4 v) {
    __builtin_nontemporal_store(u32x4{v.x, v.y, v.z, v.w}, reinterpret_cast<u32x4 *>(p));
}

// Source of a conv's split-K partial sums for the fused variant.
struct Partials {
    const float *part;  // [S][positions * C] fp32
    size_t stride;      // elements of one split
    int S;
    const uint4 *bias;  // [C] bf16, or nullptr
    const float4 *wscale = nullptr;  // 8-bit conv: [C] weight scales (sum *= xscale * wscale)
    float xscale = 1.f;
    const uint4 *res = nullptr;  // [positions * C] bf16 residual added after the bias, or nullptr
    uint4 *xstore = nullptr;     // where the rounded x is also stored, or nullptr
};

// FROM_PARTS: the input chunk is not read from x but built from partial sums,
// x = round_bf16(sum over splits in order + bias + residual), bit for bit
// what the split-K reduce kernel stores (bf16 only); pp.xstore receives that
// x as well when given.
// OUT8: the result is stored as E4M3 codes of fl32(y * qr), 8 bytes per chunk
// of 8 channels (bf16 input only): the quantised conv's input written by the
// norm itself, half the bytes of a bf16 store.
template <bool BF16, int K, bool STREAM, bool FROM_PARTS = false, bool OUT8 = false>
__global__ void __launch_bounds__(256) rmsnorm_flat_kernel(const uint4 *__restrict__ x,
                                                           const uint4 *__restrict__ gamma,
                                                           const uint4 *__restrict__ beta,
                                                           uint4 *__restrict__ y, long positions,
                                                           int cpp, int P, int R, float scale,
                                                           float eps, int apply_silu,
                                                           Partials pp = Partials{}, float qr = 1.f) {
    static_assert(!OUT8 || BF16, "E4M3 output from bf16 input only");
    using V = Vec<BF16>;
    __shared__ float part[256 * K];
    __shared__ float rinv[256 * K];
    __shared__ uint4 g_s[FLAT_MAX_CPP];
    __shared__ uint4 b_s[FLAT_MAX_CPP];
    __shared__ uint4 cb_s[FROM_PARTS ? FLAT_MAX_CPP : 1];  // the conv's bias
    __shared__ float4 sc_s[FROM_PARTS ? 2 * FLAT_MAX_CPP : 1];  // x_scale * w_scale (8-bit conv)
    const int tid = threadIdx.x;
    const long pos0 = (long)blockIdx.x * P;
    const long left = positions - pos0;
    const int np = left < P ? (int)left : P;
    const int nchunks = np * cpp;
    const uint4 *xb = FROM_PARTS ? nullptr : x + pos0 * cpp;
    uint4 *yb = y + pos0 * cpp;

    for (int c = tid; c < cpp; c += 256) {
        g_s[c] = gamma[c];
        b_s[c] = beta ? beta[c] : make_uint4(0u, 0u, 0u, 0u);
        if constexpr (FROM_PARTS) {
            cb_s[c] = pp.bias ? pp.bias[c] : make_uint4(0u, 0u, 0u, 0u);
            if (pp.wscale) {
                const float4 a = pp.wscale[2 * c], b = pp.wscale[2 * c + 1];
                sc_s[2 * c] = make_float4(pp.xscale * a.x, pp.xscale * a.y, pp.xscale * a.z, pp.xscale * a.w);
                sc_s[2 * c + 1] = make_float4(pp.xscale * b.x, pp.xscale * b.y, pp.xscale * b.z, pp.xscale * b.w);
            }
        }
    }
    uint4 raw[K];
    if constexpr (FROM_PARTS) {
        __syncthreads();  // cb_s
#pragma unroll
        for (int k = 0; k < K; ++k) {
            const int f = tid + 256 * k;
            raw[k] = make_uint4(0u, 0u, 0u, 0u);
            if (f < nchunks) {
                const size_t e0 = (size_t)(pos0 * cpp + f) * 8;
                float v[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) v[e] = 0.f;
                // splits in order, four splits' loads in flight before their adds
                for (int sp0 = 0; sp0 < pp.S; sp0 += 4) {
                    float4 a[4], b[4];
#pragma unroll
                    for (int u = 0; u < 4; ++u)
                        if (sp0 + u < pp.S) {
                            a[u] = *reinterpret_cast<const float4 *>(pp.part + (sp0 + u) * pp.stride + e0);
                            b[u] = *reinterpret_cast<const float4 *>(pp.part + (sp0 + u) * pp.stride + e0 + 4);
                        }
#pragma unroll
                    for (int u = 0; u < 4; ++u)
                        if (sp0 + u < pp.S) {
                            v[0] += a[u].x; v[1] += a[u].y; v[2] += a[u].z; v[3] += a[u].w;
                            v[4] += b[u].x; v[5] += b[u].y; v[6] += b[u].z; v[7] += b[u].w;
                        }
                }
                if (pp.wscale) {  // the split-K reduce's order: the sum, times the scales
                    const float4 a = sc_s[2 * (f % cpp)], b = sc_s[2 * (f % cpp) + 1];
                    v[0] *= a.x; v[1] *= a.y; v[2] *= a.z; v[3] *= a.w;
                    v[4] *= b.x; v[5] *= b.y; v[6] *= b.z; v[7] *= b.w;
                }
                if (pp.bias) {
                    float bb[8];
                    V::unpack(cb_s[f % cpp], bb);
#pragma unroll
                    for (int e = 0; e < 8; ++e) v[e] += bb[e];
                }
                if (pp.res) {
                    float rr[8];
                    V::unpack(pp.res[pos0 * cpp + f], rr);
#pragma unroll
                    for (int e = 0; e < 8; ++e) v[e] += rr[e];
                }
                raw[k] = V::pack(v);
                if (pp.xstore) pp.xstore[pos0 * cpp + f] = raw[k];
            }
        }
    } else {
#pragma unroll
        for (int k = 0; k < K; ++k) {
            const int f = tid + 256 * k;
            raw[k] = make_uint4(0u, 0u, 0u, 0u);
            if (f < nchunks) raw[k] = STREAM ? ld_stream(xb + f) : xb[f];
        }
    }
    float v[K][V::N];  // unpacked once, used by both passes
#pragma unroll
    for (int k = 0; k < K; ++k) {
        const int f = tid + 256 * k;
        V::unpack(raw[k], v[k]);
        if (f < nchunks) {
            float s = 0.f;
#pragma unroll
            for (int e = 0; e < V::N; ++e) s = fmaf(v[k][e], v[k][e], s);
            part[f] = s;
        }
    }
    __syncthreads();
    // R lanes (a power of two dividing 64) per position; every lane of a group
    // runs the same number of iterations, so the shuffles always pair live lanes.
    for (int pp = tid / R; pp < np; pp += 256 / R) {
        const int sub = tid % R;
        float s = 0.f;
        for (int c = sub; c < cpp; c += R) s += part[pp * cpp + c];
        for (int off = R / 2; off > 0; off >>= 1) s += __shfl_xor(s, off, 64);
        if (sub == 0) rinv[pp] = scale / fmaxf(sqrtf(s), eps);
    }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < K; ++k) {
        const int f = tid + 256 * k;
        if (f < nchunks) {
            const int pp = f / cpp, c = f - pp * cpp;
            const float r = rinv[pp];
            float g[V::N], b[V::N], o[V::N];
            V::unpack(g_s[c], g);
            V::unpack(b_s[c], b);
#pragma unroll
            for (int e = 0; e < V::N; ++e) {
                const float u = fmaf(v[k][e] * r, g[e], b[e]);
                o[e] = apply_silu ? silu<BF16>(u) : u;
            }
            if constexpr (OUT8) {
                const uint2 c8 = make_uint2(pack4_e4m3(o[0] * qr, o[1] * qr, o[2] * qr, o[3] * qr),
                                            pack4_e4m3(o[4] * qr, o[5] * qr, o[6] * qr, o[7] * qr));
                uint2 *q8 = reinterpret_cast<uint2 *>(y) + pos0 * cpp + f;
                if (STREAM)
                    __builtin_nontemporal_store(u32x2{c8.x, c8.y}, reinterpret_cast<u32x2 *>(q8));
                else
                    *q8 = c8;
            } else if (STREAM) {
                st_stream(yb + f, V::pack(o));
            } else {
                yb[f] = V::pack(o);
            }
        }
    }
}

// Any C: one thread per position, scalar loop (used when C is not a multiple
// of the 16-byte vector, unaligned tensors, or more than FLAT_MAX_CPP chunks).
template <bool BF16, bool OUT8 = false>
__global__ void __launch_bounds__(256) rmsnorm_scalar_kernel(const void *xv, const void *gv,
                                                             const void *bv, void *yv,
                                                             long positions, int c, float scale,
                                                             float eps, int apply_silu,
                                                             float qr = 1.f) {
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
        if (OUT8)
            static_cast<uint8_t *>(yv)[pos * c + k] = to_e4m3(u * qr);
        else if (BF16)
            static_cast<uint16_t *>(yv)[pos * c + k] = f32_to_bf16(u);
        else
            static_cast<float *>(yv)[pos * c + k] = u;
    }
}

int num_cus_norm() {
    static int cached = 0;
    if (!cached) {
        int dev = 0, cus = 0;
        if (hipGetDevice(&dev) == hipSuccess &&
            hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess &&
            cus > 0)
            cached = cus;
        else
            cached = 256;
    }
    return cached;
}

template <bool BF16, int K, bool STREAM>
hipError_t launch_flat(const void *x, const void *g, const void *b, void *y, long positions,
                       int cpp, float scale, float eps, int silu_on, hipStream_t s) {
    const int P = 256 * K / cpp;  // whole positions per workgroup (cpp <= 256 * K)
    int R = 1;                     // reducer lanes per position: power of two, <= 64
    while (R < 64 && 2 * R * P <= 256 && 2 * R <= cpp) R *= 2;
    const long blocks = (positions + P - 1) / P;
    if (blocks > 0x7fffffffL) return hipErrorInvalidValue;
    hipLaunchKernelGGL((rmsnorm_flat_kernel<BF16, K, STREAM>), dim3((unsigned)blocks), dim3(256), 0, s,
                       static_cast<const uint4 *>(x), static_cast<const uint4 *>(g),
                       static_cast<const uint4 *>(b), static_cast<uint4 *>(y), positions, cpp, P,
                       R, scale, eps, silu_on);
    return hipGetLastError();
}

template <bool BF16>
hipError_t dispatch(const void *x, const void *g, const void *b, void *y, long positions, int c,
                    float eps, int silu_on, hipStream_t s) {
    const float scale = sqrtf((float)c);
    constexpr int VN = Vec<BF16>::N;
    const bool aligned = ((uintptr_t)x % 16 == 0) && ((uintptr_t)y % 16 == 0) &&
                         ((uintptr_t)g % 16 == 0) && ((uintptr_t)b % 16 == 0);
    if (c % VN == 0 && aligned && c / VN <= FLAT_MAX_CPP) {
        const int cpp = c / VN;
        // Large tensors (far beyond L2): two chunks per thread, non-temporal
        // accesses.  Small ones (one frame of a streamed block, read again by
        // the next conv while it is still in L2): one chunk per thread, so the
        // grid still covers every CU several times, and ordinary stores.
        const long chunks = positions * cpp;
        if (chunks >= 8L * 1024 * num_cus_norm())
            return launch_flat<BF16, 2, true>(x, g, b, y, positions, cpp, scale, eps, silu_on, s);
        return launch_flat<BF16, 1, false>(x, g, b, y, positions, cpp, scale, eps, silu_on, s);
    }
    const long blocks = (positions + 255) / 256;
    if (blocks > 0x7fffffffL) return hipErrorInvalidValue;
    hipLaunchKernelGGL(rmsnorm_scalar_kernel<BF16>, dim3((unsigned)blocks), dim3(256), 0, s, x, g,
                       b, y, positions, c, scale, eps, silu_on);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_rmsnorm_silu_from_partials(const ConvPartials &pp, const void *bias,
                                             const void *gamma, const void *beta, void *y,
                                             long positions, int c, float eps, int apply_silu,
                                             hipStream_t s, const float *wscale, float xscale,
                                             float out_qr, const void *residual, void *xstore) {
    if (positions <= 0) return hipSuccess;
    const int cpp = c / 8;
    if (c % 8 != 0 || cpp > FLAT_MAX_CPP || pp.S < 1) return hipErrorInvalidValue;
    const int P = 256 / cpp;
    int R = 1;
    while (R < 64 && 2 * R * P <= 256 && 2 * R <= cpp) R *= 2;
    const long blocks = (positions + P - 1) / P;
    if (blocks > 0x7fffffffL) return hipErrorInvalidValue;
    const Partials q{pp.part, pp.stride, pp.S, static_cast<const uint4 *>(bias),
                     reinterpret_cast<const float4 *>(wscale), xscale,
                     static_cast<const uint4 *>(residual), static_cast<uint4 *>(xstore)};
    if (out_qr > 0.f)  // 8-bit output: codes of fl32(y * out_qr)
        hipLaunchKernelGGL((rmsnorm_flat_kernel<true, 1, false, true, true>), dim3((unsigned)blocks),
                           dim3(256), 0, s, nullptr, static_cast<const uint4 *>(gamma),
                           static_cast<const uint4 *>(beta), static_cast<uint4 *>(y), positions, cpp, P,
                           R, sqrtf((float)c), eps, apply_silu, q, out_qr);
    else
        hipLaunchKernelGGL((rmsnorm_flat_kernel<true, 1, false, true>), dim3((unsigned)blocks), dim3(256),
                           0, s, nullptr, static_cast<const uint4 *>(gamma),
                           static_cast<const uint4 *>(beta), static_cast<uint4 *>(y), positions, cpp, P,
                           R, sqrtf((float)c), eps, apply_silu, q);
    return hipGetLastError();
}

hipError_t launch_rmsnorm_silu_e4m3(const void *x, const void *gamma, const void *beta, void *q,
                                    long positions, int c, float eps, int apply_silu, float qr,
                                    hipStream_t s) {
    if (positions <= 0) return hipSuccess;
    const float scale = sqrtf((float)c);
    const bool aligned = ((uintptr_t)x % 16 == 0) && ((uintptr_t)q % 8 == 0) &&
                         ((uintptr_t)gamma % 16 == 0) && ((uintptr_t)beta % 16 == 0);
    if (c % 8 == 0 && aligned && c / 8 <= FLAT_MAX_CPP) {
        const int cpp = c / 8;
        const long chunks = positions * cpp;
        // Large tensors: four chunks per thread (more reads in flight per
        // thread; with half the write bytes of the bf16 store the read stream
        // sets the pace), non-temporal accesses.
        const bool big = chunks >= 8L * 1024 * num_cus_norm();
        const int K = big ? 4 : 1;
        const int P = 256 * K / cpp;
        int R = 1;
        while (R < 64 && 2 * R * P <= 256 && 2 * R <= cpp) R *= 2;
        const long blocks = (positions + P - 1) / P;
        if (blocks > 0x7fffffffL) return hipErrorInvalidValue;
        if (big)
            hipLaunchKernelGGL((rmsnorm_flat_kernel<true, 4, true, false, true>), dim3((unsigned)blocks),
                               dim3(256), 0, s, static_cast<const uint4 *>(x),
                               static_cast<const uint4 *>(gamma), static_cast<const uint4 *>(beta),
                               static_cast<uint4 *>(q), positions, cpp, P, R, scale, eps, apply_silu,
                               Partials{}, qr);
        else
            hipLaunchKernelGGL((rmsnorm_flat_kernel<true, 1, false, false, true>), dim3((unsigned)blocks),
                               dim3(256), 0, s, static_cast<const uint4 *>(x),
                               static_cast<const uint4 *>(gamma), static_cast<const uint4 *>(beta),
                               static_cast<uint4 *>(q), positions, cpp, P, R, scale, eps, apply_silu,
                               Partials{}, qr);
        return hipGetLastError();
    }
    const long blocks = (positions + 255) / 256;
    if (blocks > 0x7fffffffL) return hipErrorInvalidValue;
    hipLaunchKernelGGL((rmsnorm_scalar_kernel<true, true>), dim3((unsigned)blocks), dim3(256), 0, s, x,
                       gamma, beta, q, positions, c, scale, eps, apply_silu, qr);
    return hipGetLastError();
}

hipError_t launch_rmsnorm_silu(const void *x, const void *gamma, const void *beta, void *y,
                               long positions, int c, int dtype, float eps, int apply_silu,
                               hipStream_t s) {
    if (positions <= 0) return hipSuccess;
    if (dtype == WVC_BF16)
        return dispatch<true>(x, gamma, beta, y, positions, c, eps, apply_silu, s);
    return dispatch<false>(x, gamma, beta, y, positions, c, eps, apply_silu, s);
}

}  // namespace wvc
