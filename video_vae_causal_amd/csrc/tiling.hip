// tiling.hip -- spatial tiling of a decode with overlap blending ("VSR Hover
// Comparison", the decoder-tiling paragraph: the latent is decoded in
// overlapping spatial tiles, (60, 104) at stride (30, 52) there, and the
// decoded tiles are fused with complementary linear-ramp weights).
//
//   tile_extract: tile[n, t, i, j, :] = x[n, t, y0 + i, x0 + j, :]
//   tile_blend:   acc[n, t, y0 + i, x0 + j, :] += w(i, j) * tile[n, t, i, j, :]
//                 wsum[y0 + i, x0 + j] += w(i, j)
//   tile_finish:  y = acc / wsum, rounded once to the output dtype.
// w(i, j) = wy(i) * wx(j); along an axis of a tile of length L the weight is
// (i + 1/2) / lo over the lo pixels shared with the previous tile, times
// (L - i - 1/2) / hi over the hi pixels shared with the next one, else 1; two
// tiles' weights across one overlap add to 1.
//
// All three are HBM-bound streaming kernels over channels-last data: a thread
// handles 4 consecutive channels (one 8-byte bf16 or 16-byte fp32 unit).
#include "wvc_internal.h"
#include "wvc.h"

namespace wvc {
namespace {

unsigned grid_of(long work) {
    long blocks = (work + 255) / 256;
    if (blocks > 65536) blocks = 65536;
    return (unsigned)(blocks < 1 ? 1 : blocks);
}

template <typename U>
__global__ void __launch_bounds__(256) tile_extract_kernel(const U *__restrict__ x, U *__restrict__ y,
                                                           long planes, int h, int w, int y0, int x0,
                                                           int th, int tw, int cu) {
    const long total = planes * th * tw * cu;
    for (long i = (long)blockIdx.x * 256 + threadIdx.x; i < total; i += (long)gridDim.x * 256) {
        const int k = (int)(i % cu);
        long r = i / cu;
        const int jj = (int)(r % tw);
        r /= tw;
        const int ii = (int)(r % th);
        const long pl = r / th;
        y[i] = x[((pl * h + y0 + ii) * w + x0 + jj) * cu + k];
    }
}

__device__ __forceinline__ float ramp(int i, int len, int lo, int hi) {
    float v = 1.0f;
    if (i < lo) v = ((float)i + 0.5f) / (float)lo;
    if (i >= len - hi) v *= ((float)(len - i) - 0.5f) / (float)hi;
    return v;
}

template <bool BF16>
__global__ void __launch_bounds__(256) tile_blend_kernel(const void *__restrict__ tile,
                                                         float *__restrict__ acc,
                                                         float *__restrict__ wsum, long planes,
                                                         int c4, int th, int tw, int h, int w, int y0,
                                                         int x0, int rt, int rb, int rl, int rr) {
    const long total = planes * th * tw * c4;
    for (long i = (long)blockIdx.x * 256 + threadIdx.x; i < total; i += (long)gridDim.x * 256) {
        const int k = (int)(i % c4);
        long r = i / c4;
        const int jj = (int)(r % tw);
        r /= tw;
        const int ii = (int)(r % th);
        const long pl = r / th;
        const float wt = ramp(ii, th, rt, rb) * ramp(jj, tw, rl, rr);
        float v[4];
        if (BF16) {
            const uint2 u = static_cast<const uint2 *>(tile)[i];
            v[0] = bf16_to_f32(u.x & 0xffffu);
            v[1] = bf16_to_f32(u.x >> 16);
            v[2] = bf16_to_f32(u.y & 0xffffu);
            v[3] = bf16_to_f32(u.y >> 16);
        } else {
            const float4 u = static_cast<const float4 *>(tile)[i];
            v[0] = u.x; v[1] = u.y; v[2] = u.z; v[3] = u.w;
        }
        const long pos = (long)(y0 + ii) * w + x0 + jj;
        float4 *a = reinterpret_cast<float4 *>(acc) + (pl * h * w + pos) * c4 + k;
        float4 o = *a;
        o.x = fmaf(wt, v[0], o.x);
        o.y = fmaf(wt, v[1], o.y);
        o.z = fmaf(wt, v[2], o.z);
        o.w = fmaf(wt, v[3], o.w);
        *a = o;
        if (pl == 0 && k == 0) wsum[pos] += wt;
    }
}

template <bool BF16>
__global__ void __launch_bounds__(256) tile_finish_kernel(const float *__restrict__ acc,
                                                          const float *__restrict__ wsum,
                                                          void *__restrict__ y, long planes, int c4,
                                                          long hw) {
    const long total = planes * hw * c4;
    for (long i = (long)blockIdx.x * 256 + threadIdx.x; i < total; i += (long)gridDim.x * 256) {
        const long pos = (i / c4) % hw;
        const float inv = 1.0f / wsum[pos];
        const float4 a = reinterpret_cast<const float4 *>(acc)[i];
        if (BF16)
            static_cast<uint2 *>(y)[i] = make_uint2(pack2_bf16(a.x * inv, a.y * inv), pack2_bf16(a.z * inv, a.w * inv));
        else
            static_cast<float4 *>(y)[i] = make_float4(a.x * inv, a.y * inv, a.z * inv, a.w * inv);
    }
}

}  // namespace

hipError_t launch_tile_extract(const void *x, void *y, long planes, int h, int w, int y0, int x0,
                               int th, int tw, int c, int elem, hipStream_t s) {
    const long row = (long)c * elem;
    const long work = planes * th * tw;
    if (work <= 0) return hipSuccess;
    if (row % 16 == 0)
        hipLaunchKernelGGL(tile_extract_kernel<uint4>, dim3(grid_of(work * (row / 16))), dim3(256), 0, s,
                           static_cast<const uint4 *>(x), static_cast<uint4 *>(y), planes, h, w, y0, x0,
                           th, tw, (int)(row / 16));
    else
        hipLaunchKernelGGL(tile_extract_kernel<uint16_t>, dim3(grid_of(work * (row / 2))), dim3(256), 0,
                           s, static_cast<const uint16_t *>(x), static_cast<uint16_t *>(y), planes, h, w,
                           y0, x0, th, tw, (int)(row / 2));
    return hipGetLastError();
}

hipError_t launch_tile_blend(const void *tile, float *acc, float *wsum, long planes, int c, int th,
                             int tw, int h, int w, int y0, int x0, int rt, int rb, int rl, int rr,
                             bool bf16, hipStream_t s) {
    const long work = planes * th * tw * (c / 4);
    if (work <= 0) return hipSuccess;
    if (bf16)
        hipLaunchKernelGGL(tile_blend_kernel<true>, dim3(grid_of(work)), dim3(256), 0, s, tile, acc, wsum,
                           planes, c / 4, th, tw, h, w, y0, x0, rt, rb, rl, rr);
    else
        hipLaunchKernelGGL(tile_blend_kernel<false>, dim3(grid_of(work)), dim3(256), 0, s, tile, acc,
                           wsum, planes, c / 4, th, tw, h, w, y0, x0, rt, rb, rl, rr);
    return hipGetLastError();
}

hipError_t launch_tile_finish(const float *acc, const float *wsum, void *y, long planes, int c,
                              long hw, bool bf16, hipStream_t s) {
    const long work = planes * hw * (c / 4);
    if (work <= 0) return hipSuccess;
    if (bf16)
        hipLaunchKernelGGL(tile_finish_kernel<true>, dim3(grid_of(work)), dim3(256), 0, s, acc, wsum, y,
                           planes, c / 4, hw);
    else
        hipLaunchKernelGGL(tile_finish_kernel<false>, dim3(grid_of(work)), dim3(256), 0, s, acc, wsum, y,
                           planes, c / 4, hw);
    return hipGetLastError();
}

}  // namespace wvc
