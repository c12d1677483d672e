// quant.hip -- quantisers to 8-bit floats (OCP E4M3) for the 8-bit conv path.
//
// The quantised Conv3D of "Cosmos3 Wan VAE -- engine size vs runtime context
// memory" (sections 7 and 9: 8-bit weights and activations as the byte
// reduction of the 16-bit engine) needs its operands as codes: weights once,
// with one scale per output channel (the absmax of the channel maps to 448),
// and activations with one scale per tensor.  Both are streaming passes over
// HBM; the activations of a block normally come out of the fused norm + SiLU
// kernel already quantised (rmsnorm.hip), so the per-tensor quantiser here is
// for conv inputs that no norm produces.
#include "wvc_internal.h"
#include "wvc.h"

namespace wvc {
namespace {

template <bool BF16>
__device__ __forceinline__ float load_elem(const void *x, long i) {
    if (BF16) return bf16_to_f32(static_cast<const uint16_t *>(x)[i]);
    return static_cast<const float *>(x)[i];
}

// Eight elements per thread: one 16-byte (bf16) or two 16-byte (fp32) loads
// and one 8-byte store when VEC; element by element otherwise.
template <bool BF16, bool VEC>
__global__ void __launch_bounds__(256) quantize_kernel(const void *__restrict__ x,
                                                       uint8_t *__restrict__ q, long count,
                                                       float qr) {
    const long groups = (count + 7) / 8;
    for (long gi = (long)blockIdx.x * 256 + threadIdx.x; gi < groups; gi += (long)gridDim.x * 256) {
        const long e0 = gi * 8;
        if (VEC && e0 + 8 <= count) {
            float v[8];
            if (BF16) {
                const uint4 u = static_cast<const uint4 *>(x)[gi];
                const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    v[2 * k] = bf16_to_f32(w[k] & 0xffffu);
                    v[2 * k + 1] = bf16_to_f32(w[k] >> 16);
                }
            } else {
                const float4 a = static_cast<const float4 *>(x)[2 * gi];
                const float4 b = static_cast<const float4 *>(x)[2 * gi + 1];
                v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
                v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
            }
            reinterpret_cast<uint2 *>(q)[gi] = make_uint2(
                pack4_e4m3(v[0] * qr, v[1] * qr, v[2] * qr, v[3] * qr),
                pack4_e4m3(v[4] * qr, v[5] * qr, v[6] * qr, v[7] * qr));
        } else {
            for (long e = e0; e < count && e < e0 + 8; ++e) q[e] = to_e4m3(load_elem<BF16>(x, e) * qr);
        }
    }
}

// One workgroup per row: the row's absmax (a max, so the order of the
// reduction does not matter), its scale, then the codes.
template <bool BF16>
__global__ void __launch_bounds__(256) quantize_rows_kernel(const void *__restrict__ x,
                                                            uint8_t *__restrict__ q,
                                                            float *__restrict__ scale, long cols) {
    __shared__ float wmax[4];
    const long base = (long)blockIdx.x * cols;
    const int tid = threadIdx.x;
    float m = 0.f;
    for (long c = tid; c < cols; c += 256) m = fmaxf(m, fabsf(load_elem<BF16>(x, base + c)));
    for (int off = 32; off > 0; off >>= 1) m = fmaxf(m, __shfl_xor(m, off, 64));
    if ((tid & 63) == 0) wmax[tid >> 6] = m;
    __syncthreads();
    const float amax = fmaxf(fmaxf(wmax[0], wmax[1]), fmaxf(wmax[2], wmax[3]));
    // IEEE fp32 divisions (hipcc's default), as the per-row rule states
    const float sc = amax > 0.f ? amax / E4M3_MAX : 1.f;
    const float r = 1.f / sc;
    if (tid == 0) scale[blockIdx.x] = sc;
    for (long c = tid; c < cols; c += 256) q[base + c] = to_e4m3(load_elem<BF16>(x, base + c) * r);
}

unsigned grid_for(long work) {
    long b = (work + 255) / 256;
    if (b > 65536) b = 65536;
    return (unsigned)(b < 1 ? 1 : b);
}

}  // namespace

hipError_t launch_quantize_e4m3(const void *x, bool bf16, long count, float qr, void *q,
                                hipStream_t s) {
    if (count <= 0) return hipSuccess;
    const bool vec = (uintptr_t)x % 16 == 0 && (uintptr_t)q % 8 == 0;
    const dim3 grid(grid_for((count + 7) / 8));
    uint8_t *qb = static_cast<uint8_t *>(q);
    if (bf16) {
        if (vec)
            hipLaunchKernelGGL((quantize_kernel<true, true>), grid, dim3(256), 0, s, x, qb, count, qr);
        else
            hipLaunchKernelGGL((quantize_kernel<true, false>), grid, dim3(256), 0, s, x, qb, count, qr);
    } else {
        if (vec)
            hipLaunchKernelGGL((quantize_kernel<false, true>), grid, dim3(256), 0, s, x, qb, count, qr);
        else
            hipLaunchKernelGGL((quantize_kernel<false, false>), grid, dim3(256), 0, s, x, qb, count, qr);
    }
    return hipGetLastError();
}

hipError_t launch_quantize_rows_e4m3(const void *x, bool bf16, long rows, long cols, void *q,
                                     float *scale, hipStream_t s) {
    if (rows <= 0) return hipSuccess;
    if (rows > 0x7fffffffL) return hipErrorInvalidValue;
    if (bf16)
        hipLaunchKernelGGL(quantize_rows_kernel<true>, dim3((unsigned)rows), dim3(256), 0, s, x,
                           static_cast<uint8_t *>(q), scale, cols);
    else
        hipLaunchKernelGGL(quantize_rows_kernel<false>, dim3((unsigned)rows), dim3(256), 0, s, x,
                           static_cast<uint8_t *>(q), scale, cols);
    return hipGetLastError();
}

}  // namespace wvc
