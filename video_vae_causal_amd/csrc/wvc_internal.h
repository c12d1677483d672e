// wvc_internal.h -- declarations shared by libwvc's own translation units.
// Nothing here is part of the C ABI (that is include/wvc.h).
#pragma once

#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>

namespace wvc {

// ---------------------------------------------------------------------------
// bf16 storage helpers (bf16 is carried as raw 16-bit patterns in memory).
// ---------------------------------------------------------------------------
__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
    return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// float -> bf16, round to nearest, ties to even; NaN stays a quiet NaN.
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return static_cast<uint16_t>((u >> 16) | 0x40u);
    u += 0x7fffu + ((u >> 16) & 1u);
    return static_cast<uint16_t>(u >> 16);
}

// Two floats -> two bf16 (lo in the low half), round to nearest even, with
// gfx950's v_cvt_pk_bf16_f32.  It agrees with f32_to_bf16 on every input
// except some of magnitude below 2^-126 (the smallest normal binade and the
// subnormals), which the kernels here never produce from non-degenerate data.
typedef float wvc_f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 wvc_bf16x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack2_bf16(float lo, float hi) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(wvc_f32x2{lo, hi}, wvc_bf16x2));
}

// ---------------------------------------------------------------------------
// OCP E4M3 (8-bit float: bias 7, no infinities, largest finite 448) codes.
// v_cvt_pk_fp8_f32 rounds to nearest even; the inputs are clamped to +-448
// first so that out-of-range values saturate.  Codes for NaN inputs are
// unspecified.
// ---------------------------------------------------------------------------
constexpr float E4M3_MAX = 448.f;
__device__ __forceinline__ float e4m3_clamp(float v) {
    return __builtin_amdgcn_fmed3f(v, -E4M3_MAX, E4M3_MAX);
}
// 4 floats -> 4 codes in one word (v[0] in the low byte).
__device__ __forceinline__ uint32_t pack4_e4m3(float a, float b, float c, float d) {
    int w = __builtin_amdgcn_cvt_pk_fp8_f32(e4m3_clamp(a), e4m3_clamp(b), 0, false);
    w = __builtin_amdgcn_cvt_pk_fp8_f32(e4m3_clamp(c), e4m3_clamp(d), w, true);
    return (uint32_t)w;
}
__device__ __forceinline__ uint8_t to_e4m3(float a) {
    return (uint8_t)(__builtin_amdgcn_cvt_pk_fp8_f32(e4m3_clamp(a), 0.f, 0, false) & 0xff);
}

// ---------------------------------------------------------------------------
// Conv launch description (already validated by the API layer).
// Tensor layouts are channels-last, see include/wvc.h.
// ---------------------------------------------------------------------------
struct ConvCall {
    const void *x;         // [N][T][H][W][Cin]
    const void *cache_in;  // [N][F][H][W][Cin] or nullptr (zeros)
    const void *weight;    // [Cout][kT][kH][kW][Cin]
    const void *bias;      // [Cout] or nullptr
    const void *residual;  // [N][T][Ho][Wo][Cout] or nullptr
    void *y;               // [N][T][Ho][Wo][Cout]
    int n, cin, cout, t, h, w, ho, wo;
    int kt, kh, kw, sh, sw, ph, pw, dt, dh, dw;
    int frames;            // F = dt*(kt-1)
    int dtype;             // WVC_F32 / WVC_BF16 / WVC_E4M3
    int st, t0, to;        // temporal stride, first anchor frame, output frames
    int eh, ew;            // extra zero rows below / columns right of the frame
    int up;                // 2: x and the caches hold h/2 x w/2 frames, read through a
                           // nearest 2x upsample (MFMA 3x3x3 route only); else 1
    int cu_limit;          // > 0: plan the split-K grid for this many CUs
    // WVC_E4M3 calls: x, cache and weight hold E4M3 codes; bias, residual and
    // y are bf16; the sum is multiplied by xscale * wscale[co].
    float xscale;
    const float *wscale;   // [Cout], 16-byte aligned
    // Spatial stride-2 route only: the conv's input is RMS norm + SiLU of x
    // with these gamma [Cin] (bf16) / beta [Cin] or nullptr, computed in the
    // conv's staging (nullptr gamma: x is the input itself).
    const void *norm_gamma;
    const void *norm_beta;
    float norm_eps;
};

enum class ConvRoute { Fast3x3x3, Fast1x1x1, FastTemporal, FastSpatial2, Generic };

// MFMA routes of the encoder's downsampling convs ("Cosmos3 Wan VAE", section
// 10.5), conv_strided.hip: FastTemporal (3x1x1, temporal stride 2, no spatial
// padding) and FastSpatial2 (1x3x3, spatial stride 2).  Their packed weights
// are the conv as one [C_out x K] GEMM operand, K = kT*kH*kW*C_in in the
// standard weight order, in 16x16x32 MFMA A-fragment order.
bool strided_supports(const ConvCall &c);
size_t strided_workspace_bytes(const ConvCall &c, bool packed_given);
size_t strided_packed_weight_bytes(const ConvCall &c);
// Name of the kernel launch_conv_strided launches (norm: the fused-norm form).
const char *strided_kernel_name(const ConvCall &c, bool norm);
hipError_t launch_strided_pack(const ConvCall &c, const void *w, void *packed, hipStream_t s);
hipError_t launch_conv_strided(const ConvCall &c, ConvRoute r, bool packed_given, void *ws,
                               size_t ws_bytes, hipStream_t s);

// MFMA implicit-GEMM route (bf16; the 3x3x3 conv also in E4M3).  Weights are read in the packed
// fragment order written by launch_pack_weights; a call that brings
// standard-layout weights packs them into its workspace first.  The workspace
// holds split-K partial sums and packed weights; its contents on entry do not
// matter.  The 3x3x3 route also writes cache_out (may be nullptr) when t > 0.
size_t igemm_workspace_bytes(const ConvCall &c, ConvRoute r, bool packed_given);
size_t igemm_packed_weight_bytes(const ConvCall &c);
bool igemm_supports(const ConvCall &c);
hipError_t launch_pack_weights(const ConvCall &c, const void *w, void *packed, hipStream_t s);
// Split-K partial sums left for a consumer (see launch_conv_igemm).
struct ConvPartials {
    const float *part = nullptr;  // [S][N][T][H][W][Cout] fp32
    size_t stride = 0;            // elements of one split
    int S = 0;                    // 0: the conv wrote y itself
};
// With `defer` given and a split-K plan, the reduce kernel is not launched:
// *defer describes the partials (the caller's consumer adds them in split
// order, then the bias, and rounds once).  Otherwise defer->S is 0 and y holds
// the output.
hipError_t launch_conv_igemm(const ConvCall &c, ConvRoute r, bool packed_given, void *ws,
                             size_t ws_bytes, void *cache_out, hipStream_t s,
                             ConvPartials *defer = nullptr);
// 1x1x1 projection kernel (conv_proj.hip), used by launch_conv_igemm for the
// 1x1x1 route when proj_supports(c): C_out <= 256, C_in <= 480.  `packed` holds
// the weights in the 16-row fragment order for a single channel tile.
bool proj_supports(const ConvCall &c);
const char *proj_kernel_name(const ConvCall &c);
// Name of the kernel(s) launch_conv_igemm launches for this call on the
// current device (snprintf semantics into buf).
int igemm_kernel_name(const ConvCall &c, ConvRoute r, char *buf, size_t n);
hipError_t launch_conv_proj(const ConvCall &c, const void *packed, size_t packed_bytes,
                            hipStream_t s);
// Direct-convolution route (any stride/pad/dilation, fp32 or bf16).
hipError_t launch_conv_direct(const ConvCall &c, hipStream_t s);

// cache_out = last F frames of concat_T(cache_in, x) (cache_in nullptr = zeros).
hipError_t launch_cache_update(const void *x, const void *cache_in, void *cache_out, int n,
                               int t, int frames, size_t frame_elems, int elem_bytes,
                               hipStream_t s);

hipError_t launch_rmsnorm_silu(const void *x, const void *gamma, const void *beta, void *y,
                               long positions, int c, int dtype, float eps, int apply_silu,
                               hipStream_t s);
// RMS norm + SiLU whose bf16 input is itself produced on the fly from split-K
// partial sums: x = round_bf16(sum_s part[s] (* xscale * wscale[c] for an
// 8-bit conv) + bias + residual), exactly what the reduce kernel would store
// (and stores to xstore when given), then the norm of launch_rmsnorm_silu,
// stored as bf16 or, with out_qr > 0, as E4M3 codes of fl32(y * out_qr).
// bf16 only.
hipError_t launch_rmsnorm_silu_from_partials(const ConvPartials &pp, const void *bias,
                                             const void *gamma, const void *beta, void *y,
                                             long positions, int c, float eps, int apply_silu,
                                             hipStream_t s, const float *wscale = nullptr,
                                             float xscale = 1.f, float out_qr = 0.f,
                                             const void *residual = nullptr,
                                             void *xstore = nullptr);

// RMS norm + SiLU of a bf16 tensor, stored as E4M3 codes of fl32(u * qr)
// (qr: the reciprocal of the activation scale).
hipError_t launch_rmsnorm_silu_e4m3(const void *x, const void *gamma, const void *beta, void *q,
                                    long positions, int c, float eps, int apply_silu, float qr,
                                    hipStream_t s);
// E4M3 quantisers (quant.hip).  Per tensor: q = E4M3(fl32(x * qr)).  Per row
// of a [rows, cols] matrix: scale_r = fl32(amax_r / 448) (1 for an all-zero
// row), q = E4M3(fl32(x * fl32(1 / scale_r))).  x is bf16 or fp32.
hipError_t launch_quantize_e4m3(const void *x, bool bf16, long count, float qr, void *q,
                                hipStream_t s);
hipError_t launch_quantize_rows_e4m3(const void *x, bool bf16, long rows, long cols, void *q,
                                     float *scale, hipStream_t s);

hipError_t launch_upsample2x(const void *x, void *y, long planes, int h, int w, int c,
                             int elem_bytes, hipStream_t s);

hipError_t launch_fill_zero(void *p, size_t bytes, hipStream_t s);

// Spatial tiling with overlap blending (tiling.hip).
hipError_t launch_tile_extract(const void *x, void *y, long planes, int h, int w, int y0, int x0,
                               int th, int tw, int c, int elem, hipStream_t s);
hipError_t launch_tile_blend(const void *tile, float *acc, float *wsum, long planes, int c, int th,
                             int tw, int h, int w, int y0, int x0, int rt, int rb, int rl, int rr,
                             bool bf16, hipStream_t s);
hipError_t launch_tile_finish(const float *acc, const float *wsum, void *y, long planes, int c,
                              long hw, bool bf16, hipStream_t s);

}  // namespace wvc
