// conv_proj.hip -- 1x1x1 channel projection (stride 1, no padding) on bf16
// MFMA: y[p, co] = b[co] + sum_ci W[co, ci] * x[p, ci] for every position p of
// the chunk ("Cosmos3 Wan VAE -- engine size vs runtime context memory",
// section 10.3 with a one-tap kernel; the block's shortcut conv of section
// 10.4).
//
// With a single tap there is no halo and the positions of a chunk are one
// contiguous channels-last run, so the conv is a plain GEMM
// [P x C_in] x [C_in x C_out] with arithmetic intensity ~C_out/3 FLOP/B: at
// C_out = 192 it is bound by HBM, not by the matrix cores.  The kernel is laid
// out for that:
//   * a workgroup owns 64 consecutive positions and every output channel, so
//     each input byte is read from HBM exactly once;
//   * its input tile (64 x C_in bf16) is staged in LDS with fully coalesced
//     16-byte loads, rows padded by 16 bytes so that the 16 lanes of an MFMA
//     operand read land in distinct banks;
//   * the weights (C_out x C_in, a few hundred KB, L2-resident) stream from L2
//     as 16x16x32 MFMA A fragments, two K-steps ahead;
//   * registers and LDS are sized for three workgroups per CU, so one
//     workgroup's HBM loads overlap another's MFMAs and stores.
// Waves split the output channels: wave w owns the 16-row blocks w, w+4, ...
#include <type_traits>

#include "wvc_internal.h"
#include "wvc.h"

namespace wvc {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr int PT = 64;  // positions per workgroup

__device__ __forceinline__ bf16x8 as_bf16x8(uint4 v) { return __builtin_bit_cast(bf16x8, v); }

__device__ __forceinline__ uint4 wload(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0);
    return make_uint4(v.x, v.y, v.z, v.w);
}

// FCO: 16-row output blocks per wave (ceil(C_out / 64)).
template <int FCO>
__global__ void __launch_bounds__(256) proj_kernel(const uint16_t *__restrict__ x,
                                                   const uint16_t *__restrict__ wp,
                                                   const uint16_t *__restrict__ bias,
                                                   const uint16_t *__restrict__ res,
                                                   uint16_t *__restrict__ y, long P, int cin,
                                                   int cout, uint32_t w_bytes) {
    extern __shared__ uint4 xs[];  // [PT][pitch16] 16-byte entries
    const int nb = (cin + 31) / 32;      // K-steps of 32 channels
    const int pitch16 = nb * 4 + 1;      // entries per position row (+1: bank offset)
    const int nblk = cout / 16;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lr = lane & 15, lg = lane >> 4;
    const long p0 = (long)blockIdx.x * PT;
    const int np = (int)(P - p0 < PT ? P - p0 : PT);

    // Stage the input tile: chunk q of the contiguous run (8 channels each)
    // goes to row q / (cin/8), entry q % (cin/8); the padding channels up to
    // nb*32 and the rows past np are zero.
    const int c8 = cin / 8;
    const uint4 *xg = reinterpret_cast<const uint4 *>(x + p0 * cin);
    for (int q = tid; q < PT * nb * 4; q += 256) {
        const int r = q / (nb * 4), e = q - r * (nb * 4);
        uint4 v = make_uint4(0u, 0u, 0u, 0u);
        if (r < np && e < c8) v = xg[(long)r * c8 + e];
        xs[r * pitch16 + e] = v;
    }

    // Weights: packed [K-step][16-row block][lane] 1 KiB fragments.
    const __amdgpu_buffer_rsrc_t wr =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t *>(wp), (short)0, (int)w_bytes, 0x00020000);
    bf16x8 A[3][FCO];
    auto load_a = [&](int set, int ks) {
#pragma unroll
        for (int f = 0; f < FCO; ++f) {
            const int blk = wave + 4 * f;
            const int bc = blk < nblk ? blk : 0;  // surplus blocks read block 0, never used
            const uint32_t off = (uint32_t)((ks * nblk + bc) * 1024 + lane * 16);
            if (set == 0) A[0][f] = as_bf16x8(wload(wr, off));
            else if (set == 1) A[1][f] = as_bf16x8(wload(wr, off));
            else A[2][f] = as_bf16x8(wload(wr, off));
        }
    };
    load_a(0, 0);
    load_a(1, nb > 1 ? 1 : 0);

    f32x4 acc[FCO][4];
#pragma unroll
    for (int f = 0; f < FCO; ++f)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[f][j] = f32x4{0.f, 0.f, 0.f, 0.f};
    __syncthreads();

    // B fragment of position block j at K-step ks: row j*16 + lr, channels
    // ks*32 + lg*8 .. +7.
    auto kstep = [&](auto set_tag, int ks) {
        constexpr int SET = decltype(set_tag)::value;
        load_a((SET + 2) % 3, ks + 2 < nb ? ks + 2 : nb - 1);
        bf16x8 B[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) B[j] = as_bf16x8(xs[(j * 16 + lr) * pitch16 + ks * 4 + lg]);
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int f = 0; f < FCO; ++f)
                acc[f][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A[SET][f], B[j], acc[f][j], 0, 0, 0);
    };
    for (int ks = 0; ks < nb; ks += 3) {
        kstep(std::integral_constant<int, 0>{}, ks);
        if (ks + 1 < nb) kstep(std::integral_constant<int, 1>{}, ks + 1);
        if (ks + 2 < nb) kstep(std::integral_constant<int, 2>{}, ks + 2);
    }

    // Epilogue: accumulator element e of tile (f, j) is channel
    // blk*16 + lg*4 + e at position j*16 + lr; + bias, + residual, one rounding.
#pragma unroll
    for (int f = 0; f < FCO; ++f) {
        const int blk = wave + 4 * f;
        if (blk >= nblk) continue;
        const int co = blk * 16 + lg * 4;
        float bv[4] = {0.f, 0.f, 0.f, 0.f};
        if (bias) {
            const uint2 bb = *reinterpret_cast<const uint2 *>(bias + co);
            bv[0] = bf16_to_f32(bb.x & 0xffffu);
            bv[1] = bf16_to_f32(bb.x >> 16);
            bv[2] = bf16_to_f32(bb.y & 0xffffu);
            bv[3] = bf16_to_f32(bb.y >> 16);
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int r = j * 16 + lr;
            if (r >= np) continue;
            const size_t o = (size_t)(p0 + r) * cout + co;
            float v[4] = {acc[f][j][0], acc[f][j][1], acc[f][j][2], acc[f][j][3]};
            if (bias)
#pragma unroll
                for (int e = 0; e < 4; ++e) v[e] += bv[e];
            if (res) {
                const uint2 rr = *reinterpret_cast<const uint2 *>(res + o);
                v[0] += bf16_to_f32(rr.x & 0xffffu);
                v[1] += bf16_to_f32(rr.x >> 16);
                v[2] += bf16_to_f32(rr.y & 0xffffu);
                v[3] += bf16_to_f32(rr.y >> 16);
            }
            *reinterpret_cast<uint2 *>(y + o) = make_uint2(pack2_bf16(v[0], v[1]), pack2_bf16(v[2], v[3]));
        }
    }
}

}  // namespace

bool proj_supports(const ConvCall &c) {
    return c.kt == 1 && c.kh == 1 && c.kw == 1 && c.cout % 16 == 0 && c.cout <= 256 &&
           c.cin % 8 == 0 && ((size_t)PT * ((c.cin + 31) / 32 * 4 + 1) * 16) <= 64 * 1024;
}

hipError_t launch_conv_proj(const ConvCall &c, const void *packed, size_t packed_bytes,
                            hipStream_t s) {
    const long P = (long)c.n * c.t * c.h * c.w;
    if (P <= 0) return hipSuccess;
    const long blocks = (P + PT - 1) / PT;
    if (blocks > 0x7fffffffL) return hipErrorInvalidValue;
    const int nb = (c.cin + 31) / 32;
    const size_t lds = (size_t)PT * (nb * 4 + 1) * 16;
    const int fco = (c.cout / 16 + 3) / 4;
    const auto *x = static_cast<const uint16_t *>(c.x);
    const auto *w = static_cast<const uint16_t *>(packed);
    const auto *b = static_cast<const uint16_t *>(c.bias);
    const auto *r = static_cast<const uint16_t *>(c.residual);
    auto *y = static_cast<uint16_t *>(c.y);
    const uint32_t wb = (uint32_t)packed_bytes;
    switch (fco) {
        case 1: hipLaunchKernelGGL(proj_kernel<1>, dim3((unsigned)blocks), dim3(256), lds, s, x, w, b, r, y, P, c.cin, c.cout, wb); break;
        case 2: hipLaunchKernelGGL(proj_kernel<2>, dim3((unsigned)blocks), dim3(256), lds, s, x, w, b, r, y, P, c.cin, c.cout, wb); break;
        case 3: hipLaunchKernelGGL(proj_kernel<3>, dim3((unsigned)blocks), dim3(256), lds, s, x, w, b, r, y, P, c.cin, c.cout, wb); break;
        default: hipLaunchKernelGGL(proj_kernel<4>, dim3((unsigned)blocks), dim3(256), lds, s, x, w, b, r, y, P, c.cin, c.cout, wb); break;
    }
    return hipGetLastError();
}

}  // namespace wvc
