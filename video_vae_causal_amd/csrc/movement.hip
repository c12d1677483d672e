// movement.hip -- the data-movement kernels of the path: the rolling cache
// update, the nearest 2x upsample and the zero fill that resets a cache.
#include "wvc_internal.h"
#include "wvc.h"

namespace wvc {
namespace {

// cache_out frame f (of F) is logical frame t - F + f of concat_T(cache_in, x):
// the last F frames of the cached past followed by the chunk ("Cosmos3 Wan
// VAE -- engine size vs runtime context memory", sections 8.5 and 10.3).
template <typename U>
__global__ void __launch_bounds__(256) cache_update_kernel(const U *__restrict__ x,
                                                           const U *__restrict__ cache_in,
                                                           U *__restrict__ out, int n, int t,
                                                           int frames, long frame_units) {
    const long total = (long)n * frames * frame_units;
    for (long i = (long)blockIdx.x * 256 + threadIdx.x; i < total; i += (long)gridDim.x * 256) {
        const long off = i % frame_units;
        const long nf = i / frame_units;
        const int f = (int)(nf % frames);
        const int b = (int)(nf / frames);
        const int lf = t - frames + f;
        U v{};
        if (lf >= 0)
            v = x[((long)b * t + lf) * frame_units + off];
        else if (cache_in)
            v = cache_in[((long)b * frames + frames + lf) * frame_units + off];
        out[i] = v;
    }
}

// y[.., 2h+i, 2w+j, :] = x[.., h, w, :]; U is the copy unit (16 B when the
// channel row allows it).
template <typename U>
__global__ void __launch_bounds__(256) upsample2x_kernel(const U *__restrict__ x, U *__restrict__ y,
                                                         long planes, int h, int w, int cu) {
    const int ho = 2 * h, wo = 2 * w;
    const long total = planes * ho * wo * cu;
    for (long i = (long)blockIdx.x * 256 + threadIdx.x; i < total; i += (long)gridDim.x * 256) {
        const int k = (int)(i % cu);
        long r = i / cu;
        const int xo = (int)(r % wo);
        r /= wo;
        const int yo = (int)(r % ho);
        const long pl = r / ho;
        y[i] = x[((pl * h + yo / 2) * w + xo / 2) * cu + k];
    }
}

__global__ void __launch_bounds__(256) fill_zero_kernel(uint4 *p, long n16, uint32_t *tail,
                                                        int ntail) {
    for (long i = (long)blockIdx.x * 256 + threadIdx.x; i < n16; i += (long)gridDim.x * 256)
        p[i] = make_uint4(0u, 0u, 0u, 0u);
    if (blockIdx.x == 0 && (int)threadIdx.x < ntail) tail[threadIdx.x] = 0u;
}

unsigned grid_for(long work) {
    long blocks = (work + 255) / 256;
    if (blocks > 65536) blocks = 65536;
    if (blocks < 1) blocks = 1;
    return (unsigned)blocks;
}

}  // namespace

hipError_t launch_cache_update(const void *x, const void *cache_in, void *cache_out, int n, int t,
                               int frames, size_t frame_elems, int elem_bytes, hipStream_t s) {
    const size_t frame_bytes = frame_elems * (size_t)elem_bytes;
    const long total_bytes = (long)n * frames * (long)frame_bytes;
    if (total_bytes <= 0) return hipSuccess;
    const bool a16 = frame_bytes % 16 == 0 && (uintptr_t)x % 16 == 0 &&
                     (uintptr_t)cache_in % 16 == 0 && (uintptr_t)cache_out % 16 == 0;
    if (a16) {
        const long units = (long)(frame_bytes / 16);
        hipLaunchKernelGGL(cache_update_kernel<uint4>, dim3(grid_for(n * frames * units)), dim3(256),
                           0, s, static_cast<const uint4 *>(x), static_cast<const uint4 *>(cache_in),
                           static_cast<uint4 *>(cache_out), n, t, frames, units);
    } else {
        const long units = (long)(frame_bytes / 2);
        hipLaunchKernelGGL(cache_update_kernel<uint16_t>, dim3(grid_for(n * frames * units)),
                           dim3(256), 0, s, static_cast<const uint16_t *>(x),
                           static_cast<const uint16_t *>(cache_in),
                           static_cast<uint16_t *>(cache_out), n, t, frames, units);
    }
    return hipGetLastError();
}

hipError_t launch_upsample2x(const void *x, void *y, long planes, int h, int w, int c,
                             int elem_bytes, hipStream_t s) {
    const long row_bytes = (long)c * elem_bytes;
    if (planes <= 0) return hipSuccess;
    if (row_bytes % 16 == 0 && (uintptr_t)x % 16 == 0 && (uintptr_t)y % 16 == 0) {
        const int cu = (int)(row_bytes / 16);
        hipLaunchKernelGGL(upsample2x_kernel<uint4>, dim3(grid_for(planes * 4 * h * w * cu)),
                           dim3(256), 0, s, static_cast<const uint4 *>(x), static_cast<uint4 *>(y),
                           planes, h, w, cu);
    } else {
        const int cu = (int)(row_bytes / 2);
        hipLaunchKernelGGL(upsample2x_kernel<uint16_t>, dim3(grid_for(planes * 4 * h * w * cu)),
                           dim3(256), 0, s, static_cast<const uint16_t *>(x),
                           static_cast<uint16_t *>(y), planes, h, w, cu);
    }
    return hipGetLastError();
}

hipError_t launch_fill_zero(void *p, size_t bytes, hipStream_t s) {
    if (bytes == 0) return hipSuccess;
    // Split into an aligned 16-byte body and a 4-byte tail (bytes % 4 == 0).
    char *base = static_cast<char *>(p);
    const uintptr_t a = (uintptr_t)base;
    size_t head = (16 - (a % 16)) % 16;
    if (head > bytes) head = bytes;
    // head bytes are written through the tail path below as 4-byte words.
    if (head % 4 != 0) return hipErrorInvalidValue;
    const size_t body = ((bytes - head) / 16) * 16;
    const size_t rest = bytes - head - body;
    // Head and rest together are at most 12 + 12 bytes: clear them with a
    // second tiny launch each so one kernel handles one contiguous tail.
    if (body)
        hipLaunchKernelGGL(fill_zero_kernel, dim3(grid_for((long)(body / 16))), dim3(256), 0, s,
                           reinterpret_cast<uint4 *>(base + head), (long)(body / 16),
                           reinterpret_cast<uint32_t *>(base + head + body), (int)(rest / 4));
    else if (rest)
        hipLaunchKernelGGL(fill_zero_kernel, dim3(1), dim3(256), 0, s, nullptr, 0L,
                           reinterpret_cast<uint32_t *>(base + head), (int)(rest / 4));
    if (head)
        hipLaunchKernelGGL(fill_zero_kernel, dim3(1), dim3(256), 0, s, nullptr, 0L,
                           reinterpret_cast<uint32_t *>(base), (int)(head / 4));
    return hipGetLastError();
}

}  // namespace wvc
