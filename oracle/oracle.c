/*
 * oracle.c -- plain fp64 CPU oracle for the causal video-VAE hot path.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the slow, obviously-correct
 * definition that the GPU library is checked against.  Only the test suite,
 * the smoke check and the CPU-baseline leg of the benchmark may load it; the
 * product path never does.  It shares no code, header, table or helper with
 * the HIP library (video_vae_causal_amd/csrc), and includes nothing from it.
 *
 * Layout: every tensor here uses the pages' logical layout NCTHW
 * ([batch, channel, time, height, width], row-major), as stated in
 * "Cosmos3 Wan VAE -- engine size vs runtime context memory", section 10.1.
 * Weights are [C_out, C_in, kT, kH, kW] (same page, section 10.3).
 *
 * Every floating-point value is a double; nothing is rounded unless a caller
 * asks for bf16 rounding explicitly (oracle_round_bf16).
 *
 * Built with: gcc -O2 -fopenmp -shared -fPIC oracle.c -o liboracle.so -lm
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>

/* ------------------------------------------------------------------------ */
/* Causal 3-D convolution                                                   */
/* ------------------------------------------------------------------------ */
/*
 * Definition ("Cosmos3 Wan VAE ...", section 10.3, the standard Conv3D sum and
 * the causal padding paragraph):
 *
 *   y[n,co,t,h,w] = ( sum over ci, kt, kh, kw of
 *                       W[co,ci,kt,kh,kw] * X'[n, ci, ts, hs, ws] ) + b[co]
 *
 *   ts = t - (kT-1-kt)*dil_t          (past-only temporal padding: the pad
 *                                      tuple puts 2*T_pad frames before frame 0
 *                                      and none after, so the last kernel
 *                                      slice kt = kT-1 sees the current frame)
 *   hs = h*stride_h - pad_h + kh*dil_h (symmetric zero padding in space)
 *   ws = w*stride_w - pad_w + kw*dil_w
 *
 * X' is the logical input: frames ts >= 0 come from x; frames ts < 0 come from
 * the past-frame cache when one is given (the cache frames are concatenated in
 * front of x along T before padding, same section), else they are zeros.
 * Spatial positions outside [0,H) x [0,W) read zero.
 *
 * The bias is added once, after the whole sum (the temporal-slice lowering in
 * "cache-aware video decoder lowering", section on turning Conv3D into batched
 * Conv2D, stresses the bias is added exactly once after summation).
 *
 * The temporal stride is 1 (t_out = t); that is the only temporal stride this
 * path defines.
 *
 * Sum order for each output element: ci outermost, then kt, kh, kw.  The loop
 * below walks whole output planes for speed, but every output element still
 * receives its terms in exactly that order, one multiply-add at a time.
 *
 * cache: [N, C_in, cache_frames, H, W] or NULL.  cache_frames must equal
 * dil_t*(kT-1) when cache is non-NULL; frame f of the cache stands for
 * logical frame f - cache_frames.
 * bias: [C_out] or NULL (no bias).
 * y: [N, C_out, T, Ho, Wo], Ho = (H + 2 pad_h - dil_h (kH-1) - 1)/stride_h + 1.
 * Returns 0, or -1 on an inconsistent argument.
 */
static long floordiv(long a, long b) { /* b > 0 */
    long q = a / b;
    if ((a % b != 0) && (a < 0)) q -= 1;
    return q;
}

static void valid_out_range(int in_size, int out_size, int stride, int pad,
                            int offset_k, int *lo, int *hi) {
    /* output indices o with 0 <= o*stride - pad + offset_k <= in_size-1 */
    long a = (long)pad - offset_k;           /* need o*stride >= a */
    long b = (long)in_size - 1 + pad - offset_k; /* need o*stride <= b */
    long l = -floordiv(-a, stride);          /* ceil(a/stride) */
    long h = floordiv(b, stride) + 1;
    if (l < 0) l = 0;
    if (h > out_size) h = out_size;
    if (h < l) h = l;
    *lo = (int)l;
    *hi = (int)h;
}

int oracle_conv_out_size(int in_size, int k, int stride, int pad, int dil) {
    int span = dil * (k - 1) + 1;
    if (in_size + 2 * pad < span) return 0;
    return (in_size + 2 * pad - span) / stride + 1;
}

int oracle_causal_conv3d(const double *x, int N, int Cin, int T, int H, int W,
                         const double *cache, int cache_frames,
                         const double *wt, int Cout, int kT, int kH, int kW,
                         const double *bias,
                         int stride_h, int stride_w, int pad_h, int pad_w,
                         int dil_t, int dil_h, int dil_w,
                         double *y) {
    if (N < 0 || Cin <= 0 || Cout <= 0 || T < 0 || H <= 0 || W <= 0) return -1;
    if (kT <= 0 || kH <= 0 || kW <= 0 || stride_h <= 0 || stride_w <= 0) return -1;
    if (dil_t <= 0 || dil_h <= 0 || dil_w <= 0 || pad_h < 0 || pad_w < 0) return -1;
    const int past = dil_t * (kT - 1);
    if (cache && cache_frames != past) return -1;
    const int Ho = oracle_conv_out_size(H, kH, stride_h, pad_h, dil_h);
    const int Wo = oracle_conv_out_size(W, kW, stride_w, pad_w, dil_w);
    if (Ho <= 0 || Wo <= 0) return -1;
    const size_t plane_in = (size_t)H * W;
    const size_t plane_out = (size_t)Ho * Wo;
    const long jobs = (long)N * Cout * T;

#pragma omp parallel for schedule(dynamic, 1)
    for (long job = 0; job < jobs; ++job) {
        const int t = (int)(job % T);
        const int co = (int)((job / T) % Cout);
        const int n = (int)(job / ((long)T * Cout));
        double *acc = y + (((size_t)n * Cout + co) * T + t) * plane_out;
        for (size_t i = 0; i < plane_out; ++i) acc[i] = 0.0;

        for (int ci = 0; ci < Cin; ++ci) {
            for (int kt = 0; kt < kT; ++kt) {
                const int ts = t - (kT - 1 - kt) * dil_t;
                const double *frame;
                if (ts >= 0) {
                    frame = x + (((size_t)n * Cin + ci) * T + ts) * plane_in;
                } else if (cache) {
                    frame = cache + (((size_t)n * Cin + ci) * cache_frames +
                                     (size_t)(cache_frames + ts)) * plane_in;
                } else {
                    continue; /* zero causal padding: contributes nothing */
                }
                for (int kh = 0; kh < kH; ++kh) {
                    int ho_lo, ho_hi;
                    valid_out_range(H, Ho, stride_h, pad_h, kh * dil_h, &ho_lo, &ho_hi);
                    for (int kw = 0; kw < kW; ++kw) {
                        int wo_lo, wo_hi;
                        valid_out_range(W, Wo, stride_w, pad_w, kw * dil_w, &wo_lo, &wo_hi);
                        const double wv =
                            wt[((((size_t)co * Cin + ci) * kT + kt) * kH + kh) * kW + kw];
                        for (int ho = ho_lo; ho < ho_hi; ++ho) {
                            const int hs = ho * stride_h - pad_h + kh * dil_h;
                            const double *row = frame + (size_t)hs * W;
                            double *orow = acc + (size_t)ho * Wo;
                            for (int wo = wo_lo; wo < wo_hi; ++wo) {
                                const int ws = wo * stride_w - pad_w + kw * dil_w;
                                orow[wo] += wv * row[ws];
                            }
                        }
                    }
                }
            }
        }
        if (bias) {
            const double b = bias[co];
            for (size_t i = 0; i < plane_out; ++i) acc[i] = acc[i] + b;
        }
    }
    return 0;
}

/*
 * Point-sampled form of the same definition: evaluates y at the flat NCTHW
 * output indices idx[0..npts), each one as an independent 7-loop sum in the
 * order ci, kt, kh, kw, then + bias.  Used where the whole output is too large
 * to compute on the host.
 */
int oracle_causal_conv3d_points(const double *x, int N, int Cin, int T, int H, int W,
                                const double *cache, int cache_frames,
                                const double *wt, int Cout, int kT, int kH, int kW,
                                const double *bias,
                                int stride_h, int stride_w, int pad_h, int pad_w,
                                int dil_t, int dil_h, int dil_w,
                                const int64_t *idx, long npts, double *out) {
    const int past = dil_t * (kT - 1);
    if (cache && cache_frames != past) return -1;
    const int Ho = oracle_conv_out_size(H, kH, stride_h, pad_h, dil_h);
    const int Wo = oracle_conv_out_size(W, kW, stride_w, pad_w, dil_w);
    if (Ho <= 0 || Wo <= 0) return -1;
    const int64_t total = (int64_t)N * Cout * T * Ho * Wo;
    for (long p = 0; p < npts; ++p)
        if (idx[p] < 0 || idx[p] >= total) return -1;

#pragma omp parallel for schedule(dynamic, 64)
    for (long p = 0; p < npts; ++p) {
        int64_t r = idx[p];
        const int wo = (int)(r % Wo); r /= Wo;
        const int ho = (int)(r % Ho); r /= Ho;
        const int t = (int)(r % T); r /= T;
        const int co = (int)(r % Cout); r /= Cout;
        const int n = (int)r;
        double acc = 0.0;
        for (int ci = 0; ci < Cin; ++ci)
            for (int kt = 0; kt < kT; ++kt) {
                const int ts = t - (kT - 1 - kt) * dil_t;
                const double *frame;
                if (ts >= 0)
                    frame = x + (((size_t)n * Cin + ci) * T + ts) * (size_t)H * W;
                else if (cache)
                    frame = cache + (((size_t)n * Cin + ci) * cache_frames +
                                     (size_t)(cache_frames + ts)) * (size_t)H * W;
                else
                    continue;
                for (int kh = 0; kh < kH; ++kh) {
                    const int hs = ho * stride_h - pad_h + kh * dil_h;
                    if (hs < 0 || hs >= H) continue;
                    for (int kw = 0; kw < kW; ++kw) {
                        const int ws = wo * stride_w - pad_w + kw * dil_w;
                        if (ws < 0 || ws >= W) continue;
                        acc += wt[((((size_t)co * Cin + ci) * kT + kt) * kH + kh) * kW + kw] *
                               frame[(size_t)hs * W + ws];
                    }
                }
            }
        out[p] = bias ? acc + bias[co] : acc;
    }
    return 0;
}

/* ------------------------------------------------------------------------ */
/* Strided causal convolution (the encoder's downsampling convs)            */
/* ------------------------------------------------------------------------ */
/*
 * "Cosmos3 Wan VAE ...", section 10.5 (the downsample path): per frame a zero
 * pad and a stride-2 Conv2d halve H and W; then a CausalConv3d with temporal
 * stride 2 may halve T.  This is the same causal sum as oracle_causal_conv3d
 * with two generalisations:
 *
 *   - temporal stride st >= 1.  Output frame j of a chunk is anchored at input
 *     frame a_j = first + j*st of the chunk, and reads frames
 *     a_j - (kT-1-kt)*dil_t (past-only padding, so output j never sees a
 *     frame after a_j).  first = (st - t_phase % st) % st, where t_phase is
 *     the number of sequence frames before this chunk, modulo st: the anchors
 *     of a whole sequence are frames 0, st, 2st, ..., and a chunk that starts
 *     at sequence frame g anchors at the first of those that is >= g.  So a
 *     T-frame sequence gives ceil(T/st) output frames, and frame 0 alone
 *     produces output 0 ("diffusion inference workload anatomy", token
 *     ledger: the causal video VAE encodes the first frame on its own and
 *     compresses the rest 4x in time, 81 frames -> 21 latents).
 *   - trailing spatial zero padding: ext_h extra zero rows below the frame and
 *     ext_w extra zero columns right of it, on top of the symmetric pad.
 *     Ho = (H + 2 pad_h + ext_h - dil_h (kH-1) - 1)/stride_h + 1.
 *
 *   y[n,co,j,ho,wo] = sum over ci, kt, kh, kw (in that order) of
 *       W[co,ci,kt,kh,kw] * X'[n, ci, a_j - (kT-1-kt)*dil_t,
 *                             ho*stride_h - pad_h + kh*dil_h,
 *                             wo*stride_w - pad_w + kw*dil_w]
 *     + b[co]
 *
 * X' as above: frames < 0 of the chunk come from the cache (frame f of the
 * cache stands for chunk frame f - cache_frames) or are zero; positions
 * outside [0,H) x [0,W) are zero.
 * y: [N, C_out, T_out, Ho, Wo] with T_out = the number of anchors in [0, T).
 * Each output element is one plain sum, evaluated on its own.
 * Returns 0, or -1 on an inconsistent argument.
 */
int oracle_strided_out_frames(int T, int stride_t, int t_phase) {
    if (stride_t <= 0 || t_phase < 0 || T < 0) return -1;
    const int first = (stride_t - t_phase % stride_t) % stride_t;
    return first < T ? (T - 1 - first) / stride_t + 1 : 0;
}

int oracle_strided_out_size(int in_size, int k, int stride, int pad, int ext, int dil) {
    const int span = dil * (k - 1) + 1;
    if (in_size + 2 * pad + ext < span) return 0;
    return (in_size + 2 * pad + ext - span) / stride + 1;
}

int oracle_causal_conv3d_strided(const double *x, int N, int Cin, int T, int H, int W,
                                 const double *cache, int cache_frames,
                                 const double *wt, int Cout, int kT, int kH, int kW,
                                 const double *bias, int stride_t, int t_phase,
                                 int stride_h, int stride_w, int pad_h, int pad_w,
                                 int ext_h, int ext_w, int dil_t, int dil_h, int dil_w,
                                 double *y) {
    if (N < 0 || Cin <= 0 || Cout <= 0 || T < 0 || H <= 0 || W <= 0) return -1;
    if (kT <= 0 || kH <= 0 || kW <= 0 || stride_h <= 0 || stride_w <= 0) return -1;
    if (stride_t <= 0 || t_phase < 0 || t_phase >= stride_t) return -1;
    if (dil_t <= 0 || dil_h <= 0 || dil_w <= 0 || pad_h < 0 || pad_w < 0) return -1;
    if (ext_h < 0 || ext_w < 0) return -1;
    const int past = dil_t * (kT - 1);
    if (cache && cache_frames != past) return -1;
    const int To = oracle_strided_out_frames(T, stride_t, t_phase);
    const int Ho = oracle_strided_out_size(H, kH, stride_h, pad_h, ext_h, dil_h);
    const int Wo = oracle_strided_out_size(W, kW, stride_w, pad_w, ext_w, dil_w);
    if (Ho <= 0 || Wo <= 0) return -1;
    const int first = (stride_t - t_phase % stride_t) % stride_t;
    const long total = (long)N * Cout * To * Ho * Wo;

#pragma omp parallel for schedule(static)
    for (long idx = 0; idx < total; ++idx) {
        long r = idx;
        const int wo = (int)(r % Wo); r /= Wo;
        const int ho = (int)(r % Ho); r /= Ho;
        const int j = (int)(r % To); r /= To;
        const int co = (int)(r % Cout); r /= Cout;
        const int n = (int)r;
        const int anchor = first + j * stride_t;
        double acc = 0.0;
        for (int ci = 0; ci < Cin; ++ci)
            for (int kt = 0; kt < kT; ++kt) {
                const int ts = anchor - (kT - 1 - kt) * dil_t;
                const double *frame;
                if (ts >= 0)
                    frame = x + (((size_t)n * Cin + ci) * T + ts) * (size_t)H * W;
                else if (cache && cache_frames + ts >= 0)
                    frame = cache + (((size_t)n * Cin + ci) * cache_frames +
                                     (size_t)(cache_frames + ts)) * (size_t)H * W;
                else
                    continue;
                for (int kh = 0; kh < kH; ++kh) {
                    const int hs = ho * stride_h - pad_h + kh * dil_h;
                    if (hs < 0 || hs >= H) continue;
                    for (int kw = 0; kw < kW; ++kw) {
                        const int ws = wo * stride_w - pad_w + kw * dil_w;
                        if (ws < 0 || ws >= W) continue;
                        acc += wt[((((size_t)co * Cin + ci) * kT + kt) * kH + kh) * kW + kw] *
                               frame[(size_t)hs * W + ws];
                    }
                }
            }
        y[idx] = bias ? acc + bias[co] : acc;
    }
    return 0;
}

/* ------------------------------------------------------------------------ */
/* RMS norm over channels                                                   */
/* ------------------------------------------------------------------------ */
/*
 * "Cosmos3 Wan VAE ...", section 10.2 (WanRMS_norm): for every fixed
 * (n, t, h, w), v = x[n, :, t, h, w] is divided by its L2 norm over the C
 * channels (an L2 normalise, no mean subtraction), then multiplied by sqrt(C)
 * and by gamma[c], and beta[c] is added.  The divisor is clamped from below by
 * eps (the fused kernel the same section names takes a max before dividing).
 *
 *   s   = sum_c v_c^2                  (channel order)
 *   d   = max(sqrt(s), eps)
 *   y_c = v_c / d * sqrt(C) * gamma_c + beta_c
 *
 * beta may be NULL (treated as zero).
 */
int oracle_rms_norm(const double *x, int N, int C, int T, int H, int W,
                    const double *gamma, const double *beta, double eps,
                    double *y) {
    if (N < 0 || C <= 0 || T < 0 || H <= 0 || W <= 0 || !gamma) return -1;
    const size_t plane = (size_t)T * H * W;
    const double scale = sqrt((double)C);
    const long jobs = (long)N * (long)plane;
#pragma omp parallel for schedule(static)
    for (long j = 0; j < jobs; ++j) {
        const size_t n = (size_t)(j / (long)plane);
        const size_t pos = (size_t)(j % (long)plane);
        const double *v = x + n * C * plane + pos;
        double *o = y + n * C * plane + pos;
        double s = 0.0;
        for (int c = 0; c < C; ++c) s += v[(size_t)c * plane] * v[(size_t)c * plane];
        double d = sqrt(s);
        if (d < eps) d = eps;
        for (int c = 0; c < C; ++c) {
            double u = v[(size_t)c * plane] / d * scale * gamma[c];
            if (beta) u = u + beta[c];
            o[(size_t)c * plane] = u;
        }
    }
    return 0;
}

/*
 * SiLU, "Cosmos3 Wan VAE ...", section 10.4: x * sigmoid(x) = x / (1 + e^-x).
 */
void oracle_silu(const double *x, long count, double *y) {
#pragma omp parallel for schedule(static)
    for (long i = 0; i < count; ++i) y[i] = x[i] / (1.0 + exp(-x[i]));
}

/*
 * Nearest-neighbour 2x spatial upsample, per frame, no temporal change:
 * y[n,c,t,2h+i,2w+j] = x[n,c,t,h,w] for i, j in {0,1}.  The pages give no
 * operator detail for the decoder's upsampler; this is the plainest reading.
 */
void oracle_upsample_nearest2x(const double *x, int N, int C, int T, int H, int W,
                               double *y) {
    const long planes = (long)N * C * T;
    const int Ho = 2 * H, Wo = 2 * W;
#pragma omp parallel for schedule(static)
    for (long p = 0; p < planes; ++p) {
        const double *src = x + (size_t)p * H * W;
        double *dst = y + (size_t)p * Ho * Wo;
        for (int ho = 0; ho < Ho; ++ho)
            for (int wo = 0; wo < Wo; ++wo)
                dst[(size_t)ho * Wo + wo] = src[(size_t)(ho / 2) * W + wo / 2];
    }
}

/* ------------------------------------------------------------------------ */
/* bf16 rounding (only for the "round where the GPU stores" oracle mode)     */
/* ------------------------------------------------------------------------ */
/*
 * Rounds each value to the nearest bfloat16 (1 sign bit, 8 exponent bits,
 * 7 stored fraction bits), ties to even, straight from double.  Written from
 * the format's definition: a normal bf16 value is (1.f) * 2^E with E in
 * [-126, 127] and an 8-bit significand, so its spacing is 2^(E-7); below
 * 2^-126 the spacing stays 2^-133 (subnormals).  Results above the largest
 * finite bf16 become infinity.  rint() rounds half to even in the default
 * rounding mode.
 */
void oracle_round_bf16(const double *x, long count, double *y) {
    const double max_finite = ldexp(255.0, 120); /* (2 - 2^-7) * 2^127 */
    for (long i = 0; i < count; ++i) {
        const double v = x[i];
        if (v == 0.0 || isnan(v) || isinf(v)) {
            y[i] = v;
            continue;
        }
        int e;
        frexp(v, &e); /* v = m * 2^e, 0.5 <= |m| < 1, so E = e - 1 */
        int qexp = (e - 1) - 7;
        if (qexp < -133) qexp = -133;
        const double q = ldexp(1.0, qexp);
        double r = rint(v / q) * q;
        if (fabs(r) > max_finite) r = copysign(INFINITY, v);
        y[i] = r;
    }
}

/* ------------------------------------------------------------------------ */
/* 8-bit floating point, E4M3                                               */
/* ------------------------------------------------------------------------ */
/*
 * The quantised Conv3D of "Cosmos3 Wan VAE -- engine size vs runtime context
 * memory" (sections 7 and 9: 8-bit weights and activations halve the bytes
 * of the 16-bit engine) is taken here in the 8-bit float format the MI355X
 * matrix cores read: E4M3 as defined by the OCP 8-bit Floating Point
 * specification (OFP8).  A code is s.eeee.mmm with exponent bias 7:
 *   e == 0          : (-1)^s * m * 2^-9            (zero and subnormals)
 *   1 <= e <= 15    : (-1)^s * (1 + m/8) * 2^(e-7)  (normals)
 *   e == 15, m == 7 : NaN (the format has no infinities)
 * so the largest finite magnitude is 1.75 * 2^8 = 448.
 */
double oracle_e4m3_decode_one(unsigned code) {
    const int s = (code >> 7) & 1, e = (code >> 3) & 15, m = code & 7;
    double v;
    if (e == 15 && m == 7) return NAN;
    if (e == 0)
        v = ldexp((double)m, -9);
    else
        v = ldexp(1.0 + m / 8.0, e - 7);
    return s ? -v : v;
}

void oracle_e4m3_decode(const uint8_t *codes, long count, double *y) {
    for (long i = 0; i < count; ++i) y[i] = oracle_e4m3_decode_one(codes[i]);
}

/*
 * Encoding of a real value: round to the nearest E4M3 value, ties to the even
 * code (the OFP8 round-to-nearest-even mode), and saturate: magnitudes beyond
 * 448 become 448 with the value's sign (OFP8's saturating conversion).  NaN
 * becomes the NaN code 0x7F.  A value v with 2^E <= |v| < 2^(E+1) sits on a
 * grid of spacing 2^(E-3); below 2^-6 the spacing stays 2^-9.  rint() rounds
 * half to even in the default rounding mode.
 */
void oracle_e4m3_encode(const double *x, long count, uint8_t *codes) {
    for (long i = 0; i < count; ++i) {
        const double v = x[i];
        if (isnan(v)) {
            codes[i] = 0x7F;
            continue;
        }
        const unsigned sign = signbit(v) ? 0x80u : 0u;
        const double a = fabs(v);
        unsigned mag;
        if (a >= 448.0) {
            mag = 0x7E;
        } else if (a < ldexp(1.0, -6)) {
            /* subnormal grid: m * 2^-9, m in 0..8 (8 is the smallest normal) */
            mag = (unsigned)rint(ldexp(a, 9));
        } else {
            int e2;
            frexp(a, &e2); /* a = f * 2^e2, 0.5 <= f < 1: E = e2 - 1 */
            int E = e2 - 1;
            unsigned m = (unsigned)rint(ldexp(a, 3 - E)) - 8u; /* 8..16 -> 0..8 */
            if (m == 8) {
                m = 0;
                E += 1;
            }
            mag = (unsigned)(E + 7) << 3 | m;
            if (mag > 0x7E) mag = 0x7E;
        }
        codes[i] = (uint8_t)(sign | mag);
    }
}
