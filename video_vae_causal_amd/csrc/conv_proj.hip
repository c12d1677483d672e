// conv_proj.hip -- 1x1x1 channel projection (stride 1, no padding) on bf16
// MFMA: y[p, co] = b[co] + sum_ci W[co, ci] * x[p, ci] for every position p of
// the chunk ("Cosmos3 Wan VAE -- engine size vs runtime context memory",
// section 10.3 with a one-tap kernel; the block's shortcut conv of section
// 10.4).
//
// With a single tap there is no halo and the positions of a chunk are one
// contiguous channels-last run, so the conv is a plain GEMM
// [P x C_in] x [C_in x C_out] with arithmetic intensity ~C_out/3 FLOP/B: at
// C_out = 192 it is bound by HBM, not by the matrix cores.  Two kernels:
//
// proj_persist_kernel (C_in % 32 == 0, C_in <= 384, C_out <= 192, and at
// least four tiles per CU): one 8-wave workgroup per CU keeps its slice of
// the weights in registers for the whole launch and loops over 64-position
// tiles, staging each through one of two LDS buffers while the next tile's
// loads are in flight; a wave owns a quarter of the output channels for half
// of the tile's positions, so the LDS reads per tile are twice the tile, not
// one tile per wave.
//
// proj_kernel (every other shape) is laid out as follows:
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

constexpr int PT = 64;    // positions per workgroup
constexpr int MAXQ = 16;  // staging chunks per thread: PT * 4 * nb / 256 = nb <= 16

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
    // All of a thread's loads are issued before its first LDS store, so the
    // tile costs one HBM round trip, not one per chunk.
    const int c8 = cin / 8;
    const uint4 *xg = reinterpret_cast<const uint4 *>(x + p0 * cin);
    const int nq = PT * nb * 4;  // <= 256 * MAXQ (proj_supports bounds nb)
    uint4 v[MAXQ];
#pragma unroll
    for (int k = 0; k < MAXQ; ++k) {
        const int q = tid + 256 * k;
        const int r = q / (nb * 4), e = q - r * (nb * 4);
        v[k] = make_uint4(0u, 0u, 0u, 0u);
        if (q < nq && r < np && e < c8) v[k] = xg[(long)r * c8 + e];
    }
#pragma unroll
    for (int k = 0; k < MAXQ; ++k) {
        const int q = tid + 256 * k;
        const int r = q / (nb * 4), e = q - r * (nb * 4);
        if (q < nq) xs[r * pitch16 + e] = v[k];
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

// Persistent variant, one workgroup of 8 waves per CU, for C_in % 32 == 0,
// C_in <= 384 and C_out <= 192.  Wave w owns the output blocks (w & 3) + 4f
// for the half (w >> 2) of the 64 positions, so each wave reads only its half
// of the LDS tile.  Its weight fragments (NB K-steps x FCO blocks) are loaded
// into registers once; the workgroup then loops over tiles g, g + grid, ...
// Per tile: the tile's staged chunks go to one of two LDS buffers, one
// barrier, the next tile's loads are issued, then the MFMAs and stores of
// this tile run while those loads are in flight.  The bias is kept as fp32 in
// LDS so that no global load in the epilogue waits behind the prefetch.
template <int FCO, int MAXNB>
__global__ void __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2)))
proj_persist_kernel(const uint16_t *__restrict__ x, const uint16_t *__restrict__ wp,
                    const uint16_t *__restrict__ bias, const uint16_t *__restrict__ res,
                    uint16_t *__restrict__ y, long P, int cin, int cout, uint32_t w_bytes) {
    constexpr int MAXC = MAXNB / 2;  // 16-byte chunks per thread: 64 * nb * 4 / 512
    extern __shared__ uint4 xs[];    // [2][PT][pitch16], then C_out fp32 bias
    const int nb = cin / 32;
    const int c8 = cin / 8;
    const int pitch16 = c8 + 1;
    const int buf16 = PT * pitch16;
    const int nblk = cout / 16;
    const int nq = PT * c8;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int cg = wave & 3, ph = wave >> 2;
    const int lr = lane & 15, lg = lane >> 4;
    const long ntiles = (P + PT - 1) / PT;

    const __amdgpu_buffer_rsrc_t wr =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t *>(wp), (short)0, (int)w_bytes, 0x00020000);
    bf16x8 A[MAXNB][FCO];
#pragma unroll
    for (int ks = 0; ks < MAXNB; ++ks)
#pragma unroll
        for (int f = 0; f < FCO; ++f) {
            const int blk = cg + 4 * f;
            const int bc = blk < nblk ? blk : 0;  // surplus blocks read block 0, never stored
            const int kc = ks < nb ? ks : 0;
            A[ks][f] = as_bf16x8(wload(wr, (uint32_t)((kc * nblk + bc) * 1024 + lane * 16)));
        }
    float *bias_s = reinterpret_cast<float *>(xs + 2 * buf16);
    for (int i = tid; i < cout; i += 512) bias_s[i] = bias ? bf16_to_f32(bias[i]) : 0.f;

    // A tile is one contiguous run of np * c8 chunks; chunk q goes to LDS
    // entry q + q / c8 (one pad entry per row).  Buffer loads bounded to the
    // tile's bytes return zero for the rows past the last position.
    const float inv_c8 = 1.0f / (float)c8;  // q / c8 exactly: q < 2^12, c8 <= 48
    uint4 v[MAXC];
    auto load_tile = [&](long tile) {
        const long p0 = tile * PT;
        const long left = P - p0;
        const int np = tile < ntiles ? (int)(left < PT ? left : PT) : 0;
        const __amdgpu_buffer_rsrc_t xr = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<uint16_t *>(x + (tile < ntiles ? p0 : 0) * cin), (short)0, np * cin * 2,
            0x00020000);
#pragma unroll
        for (int k = 0; k < MAXC; ++k) {
            const u32x4 t4 = __builtin_amdgcn_raw_buffer_load_b128(xr, tid * 16, k * 8192, 0);
            v[k] = make_uint4(t4.x, t4.y, t4.z, t4.w);
        }
    };
    auto store_tile = [&](int b) {
#pragma unroll
        for (int k = 0; k < MAXC; ++k) {
            const int q = tid + 512 * k;
            const int r = (int)(((float)q + 0.5f) * inv_c8);
            if (q < nq) xs[b * buf16 + q + r] = v[k];
        }
    };
    auto compute = [&](long tile, int b) {
        const long p0 = tile * PT;
        const int np = (int)(P - p0 < PT ? P - p0 : PT);
        f32x4 acc[FCO][2];
#pragma unroll
        for (int f = 0; f < FCO; ++f)
#pragma unroll
            for (int j = 0; j < 2; ++j) acc[f][j] = f32x4{0.f, 0.f, 0.f, 0.f};
        // B fragment j: row ph*32 + j*16 + lr, channels ks*32 + lg*8 .. +7.
        const uint4 *xb = xs + b * buf16 + (ph * 32 + lr) * pitch16 + lg;
#pragma unroll
        for (int ks = 0; ks < MAXNB; ++ks) {
            if (ks < nb) {
                bf16x8 B[2];
#pragma unroll
                for (int j = 0; j < 2; ++j) B[j] = as_bf16x8(xb[j * 16 * pitch16 + ks * 4]);
#pragma unroll
                for (int j = 0; j < 2; ++j)
#pragma unroll
                    for (int f = 0; f < FCO; ++f)
                        acc[f][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A[ks][f], B[j], acc[f][j], 0, 0, 0);
            }
        }
        // Element e of tile (f, j): channel blk*16 + lg*4 + e, position
        // ph*32 + j*16 + lr; + bias, + residual, one rounding.
#pragma unroll
        for (int f = 0; f < FCO; ++f) {
            const int blk = cg + 4 * f;
            if (blk >= nblk) continue;
            const int co = blk * 16 + lg * 4;
            const float4 bq = *reinterpret_cast<const float4 *>(bias_s + co);
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                const int r = ph * 32 + j * 16 + lr;
                if (r >= np) continue;
                const size_t o = (size_t)(p0 + r) * cout + co;
                float vv[4] = {acc[f][j][0] + bq.x, acc[f][j][1] + bq.y, acc[f][j][2] + bq.z,
                               acc[f][j][3] + bq.w};
                if (res) {
                    const uint2 rr = *reinterpret_cast<const uint2 *>(res + o);
                    vv[0] += bf16_to_f32(rr.x & 0xffffu);
                    vv[1] += bf16_to_f32(rr.x >> 16);
                    vv[2] += bf16_to_f32(rr.y & 0xffffu);
                    vv[3] += bf16_to_f32(rr.y >> 16);
                }
                *reinterpret_cast<uint2 *>(y + o) =
                    make_uint2(pack2_bf16(vv[0], vv[1]), pack2_bf16(vv[2], vv[3]));
            }
        }
    };

    // Buffer b is written only after the barrier that follows the last reads
    // of it (the compute two tiles back), so one barrier per tile suffices.
    const long G = gridDim.x;
    int b = 0;
    long tile = blockIdx.x;
    load_tile(tile);
    for (; tile < ntiles; tile += G) {
        store_tile(b);
        __syncthreads();
        load_tile(tile + G);
        compute(tile, b);
        b ^= 1;
    }
}

int num_cus_proj() {
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

}  // namespace

bool proj_supports(const ConvCall &c) {
    return c.dtype != WVC_E4M3 && c.kt == 1 && c.kh == 1 && c.kw == 1 && c.cout % 16 == 0 && c.cout <= 256 &&
           c.cin % 8 == 0 && (c.cin + 31) / 32 <= MAXQ &&
           ((size_t)PT * ((c.cin + 31) / 32 * 4 + 1) * 16) <= 64 * 1024;
}

const char *proj_kernel_name(const ConvCall &c) {
    const long P = (long)c.n * c.t * c.h * c.w;
    const long blocks = (P + PT - 1) / PT;
    const int nb = (c.cin + 31) / 32;
    const int fco = (c.cout / 16 + 3) / 4;
    if (c.cin % 32 == 0 && nb <= 12 && fco <= 3 && blocks >= 4L * num_cus_proj()) {
        static const char *names[] = {"proj_persist_kernel<1, 12>", "proj_persist_kernel<2, 12>",
                                      "proj_persist_kernel<3, 12>"};
        return names[fco < 1 ? 0 : fco - 1];
    }
    static const char *names[] = {"proj_kernel<1>", "proj_kernel<2>", "proj_kernel<3>", "proj_kernel<4>"};
    return names[fco < 1 ? 0 : (fco > 4 ? 3 : fco - 1)];
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
    // Persistent variant: C_in a multiple of 32 with at most 12 K-steps (the
    // waves' weight fragments fit in registers), C_out <= 192, and several
    // tiles per CU.
    if (c.cin % 32 == 0 && nb <= 12 && fco <= 3 && blocks >= 4L * num_cus_proj()) {
        const unsigned grid = (unsigned)num_cus_proj();
        const size_t lds2 = 2 * lds + (size_t)c.cout * 4;
        switch (fco) {
            case 1: hipLaunchKernelGGL((proj_persist_kernel<1, 12>), dim3(grid), dim3(512), lds2, s, x, w, b, r, y, P, c.cin, c.cout, wb); break;
            case 2: hipLaunchKernelGGL((proj_persist_kernel<2, 12>), dim3(grid), dim3(512), lds2, s, x, w, b, r, y, P, c.cin, c.cout, wb); break;
            default: hipLaunchKernelGGL((proj_persist_kernel<3, 12>), dim3(grid), dim3(512), lds2, s, x, w, b, r, y, P, c.cin, c.cout, wb); break;
        }
        return hipGetLastError();
    }
    switch (fco) {
        case 1: hipLaunchKernelGGL(proj_kernel<1>, dim3((unsigned)blocks), dim3(256), lds, s, x, w, b, r, y, P, c.cin, c.cout, wb); break;
        case 2: hipLaunchKernelGGL(proj_kernel<2>, dim3((unsigned)blocks), dim3(256), lds, s, x, w, b, r, y, P, c.cin, c.cout, wb); break;
        case 3: hipLaunchKernelGGL(proj_kernel<3>, dim3((unsigned)blocks), dim3(256), lds, s, x, w, b, r, y, P, c.cin, c.cout, wb); break;
        default: hipLaunchKernelGGL(proj_kernel<4>, dim3((unsigned)blocks), dim3(256), lds, s, x, w, b, r, y, P, c.cin, c.cout, wb); break;
    }
    return hipGetLastError();
}

}  // namespace wvc
