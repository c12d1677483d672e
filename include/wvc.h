/*
 * wvc.h -- C ABI of libwvc: the causal video-VAE hot path on MI355X (gfx950).
 *
 * The library computes the causal 3-D convolution of the Wan video VAE with
 * its rolling past-frame cache, the channel RMS norm + SiLU around it, and the
 * residual block that chains them.  Sources of each definition are named at
 * every entry point:
 *   [P1] "Cosmos3 Wan VAE -- engine size vs runtime context memory"
 *        (devpress.csdn.net), sections 8.5, 10.1-10.4.
 *   [P3] "cache-aware video decoder lowering" (rit.work), section on turning
 *        Conv3D into batched Conv2D.
 *   [P5] "VSR Hover Comparison" (vsr-hover-compare.pages.dev), the
 *        decoder-tiling paragraph.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * Pointers.  Every tensor pointer is a DEVICE pointer owned by the caller.
 *   The library never allocates device memory, frees it, or keeps a pointer
 *   past the call (a captured graph keeps the pointers it recorded; see the
 *   graph calls at the end).
 * Streams.  `stream` is a hipStream_t passed as void* (NULL = the null
 *   stream).  Every call only enqueues work on that stream and returns; the
 *   library never synchronises.  Results are ready when the stream is.
 * Layout.  Activations are logically [N, C, T, H, W] (the pages' NCTHW,
 *   [P1] 10.1) and stored channels-last: physical [N][T][H][W][C], C fastest
 *   (PyTorch's channels_last_3d).  Conv weights are logically
 *   [C_out, C_in, kT, kH, kW] ([P1] 10.3) stored [C_out][kT][kH][kW][C_in].
 *   Bias, gamma, beta are [C].  All tensors of one call share one dtype.
 * Caches.  A past-frame cache of a causal conv is [N, C_in, F, H, W]
 *   (physical [N][F][H][W][C_in]) with F = wvc_conv3d_cache_frames() (2 for
 *   the 3x3x3 conv: the page's CACHE_T = 2, [P1] 8.5).  Frame 0 is the oldest.
 *   An all-zero cache is exactly the zero causal padding before frame 0.
 * Errors.  Every function returning int returns WVC_OK (0) or one WVC_ERR_*.
 *   Argument errors are detected before anything is enqueued, so a failed call
 *   has no side effect.  wvc_last_error() gives text for the calling thread's
 *   last failure.  No C++ exception crosses this boundary.
 * Threads.  Calls on different streams or threads are independent; the route
 *   counters and the strict flag are process-wide.
 */
#ifndef WVC_H
#define WVC_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
    WVC_OK = 0,
    WVC_ERR_ARG = 1,         /* null / negative / inconsistent argument        */
    WVC_ERR_UNSUPPORTED = 2, /* groups != 1, a dtype no route covers, an E4M3 or
                                fused call outside its one route, packed weights
                                for the direct route                          */
    WVC_ERR_ALIAS = 3,       /* a written buffer overlaps another buffer       */
    WVC_ERR_WORKSPACE = 4,   /* workspace missing or too small                 */
    WVC_ERR_STRICT = 5,      /* strict mode on and the call needs the generic route */
    WVC_ERR_HIP = 6          /* the HIP runtime reported an error at launch    */
};

enum { WVC_F32 = 0, WVC_BF16 = 1, WVC_E4M3 = 2 /* OCP 8-bit float, see the E4M3 calls */ };

/* Weight layouts: the standard [C_out][kT][kH][kW][C_in] one, or the packed
 * MFMA fragment order written by wvc_conv3d_pack_weights (fast routes only). */
enum { WVC_WEIGHT_STANDARD = 0, WVC_WEIGHT_PACKED = 1 };

/* Descriptor of one causal Conv3D call over a chunk of `t` frames. */
typedef struct wvc_conv3d_desc {
    int n, c_in, c_out, t, h, w; /* batch, channels, frames in this chunk, spatial  */
    int kt, kh, kw;              /* kernel extent                                   */
    int stride_t;                /* >= 1; see t_phase                               */
    int stride_h, stride_w;
    int pad_h, pad_w;            /* symmetric zero padding; temporal pad is causal  */
    int dil_t, dil_h, dil_w;
    int groups;                  /* must be 1                                       */
    int dtype;                   /* WVC_F32, WVC_BF16, or WVC_E4M3 (8-bit calls)    */
    int weight_layout;           /* WVC_WEIGHT_STANDARD or WVC_WEIGHT_PACKED        */
    int pad_h_extra, pad_w_extra;/* extra zero rows below / columns right of the
                                    frame (the downsample's one-sided zero pad,
                                    [P1] 10.5); 0 for the symmetric case        */
    int t_phase;                 /* sequence frames before this chunk, modulo
                                    stride_t (0 when stride_t == 1)             */
    int upsample_in;             /* 0, or 2: the conv's input is x (and the
                                    cache) seen through a nearest 2x spatial
                                    upsample; h, w are then the upsampled
                                    frame's, x and the caches hold h/2 x w/2
                                    frames (see wvc_causal_conv3d_fwd)          */
    int cu_limit;                /* 0, or the number of CUs to plan the grid for:
                                    a call that shares the GPU with work on
                                    another stream leaves the other CUs to it.
                                    Only the split-K choice of the MFMA 3x3x3
                                    route reads it (a different split count
                                    adds the partial sums in another grouping,
                                    so results may differ in the last bit);
                                    < 0 is WVC_ERR_ARG                        */
} wvc_conv3d_desc;

/* Route counters ([P3]: counters show which route every call took). */
typedef struct wvc_counters {
    uint64_t fast_3x3x3; /* MFMA implicit-GEMM 3x3x3 route       */
    uint64_t fast_1x1x1; /* MFMA 1x1x1 channel-projection route  */
    uint64_t generic;    /* direct-convolution route             */
    uint64_t rejected;   /* calls refused with WVC_ERR_UNSUPPORTED or WVC_ERR_STRICT */
    uint64_t fast_strided; /* MFMA routes of the downsampling convs ([P1] 10.5) */
} wvc_counters;

/*
 * Causal 3-D convolution of one chunk, with an explicit cache in and out.
 * Implements [P1] 10.3: y = b + sum_{ci,kt,kh,kw} W * X', where X' is the
 * chunk with the F cached past frames concatenated in front along T ([P1] 8.5,
 * 10.3), then zero padded pad_h/pad_w in space; no future frame is read, so
 * kernel slice kt = kT-1 multiplies the current frame and slice kt multiplies
 * frame t - (kT-1-kt)*dil_t.  The bias is added once after the sum over all
 * slices, and stride, padding and dilation are honoured as given ([P3]).
 * The output has h_out = (h + 2 pad_h + pad_h_extra - dil_h (kh-1) - 1)/stride_h + 1
 * rows (w_out likewise) and t_out frames.  With stride_t == 1, t_out = t.
 * With stride_t = s > 1 (the encoder's temporal downsample, [P1] 10.5) output
 * frame j is anchored at chunk frame a_j = first + j*s, first =
 * (s - t_phase) % s, and reads frames a_j - (kT-1-kt)*dil_t: the anchors of a
 * whole sequence are its frames 0, s, 2s, ..., so T frames give ceil(T/s)
 * outputs and the first frame alone gives the first ("diffusion inference
 * workload anatomy", two-compressions paragraph: 81 frames -> 21 latents
 * over two such stages).  t_out = the number of anchors in [0, t).  A caller
 * streaming chunks passes t_phase = (frames already fed) % s; the cache
 * carries the last F input frames as for stride 1.
 *
 *   x         [N, C_in, t, H, W]          read
 *   cache_in  [N, C_in, F, H, W] or NULL  read; NULL = zero causal padding
 *                                          (start of a sequence)
 *   cache_out [N, C_in, F, H, W] or NULL  written: the last F frames of
 *                                          concat_T(cache_in, x); NULL = skip
 *   weight    [C_out, C_in, kT, kH, kW]   read (or its packed form when
 *                                          d->weight_layout is WVC_WEIGHT_PACKED)
 *   bias      [C_out] or NULL             read
 *   residual  [N, C_out, t_out, h_out, w_out] or NULL; added after the bias
 *                                          (fused residual of the block)
 *   y         [N, C_out, t_out, h_out, w_out] written
 *   workspace / workspace_bytes: scratch of at least
 *             wvc_causal_conv3d_workspace_bytes(d) bytes (may be NULL if 0).
 *             It holds split-K partial sums (and the packed weights when
 *             standard-layout weights come in); its contents on entry do not
 *             matter.  Calls that share a workspace must not overlap in time
 *             (use one stream, or one workspace per stream).
 *
 * Routes: bf16 3x3x3 / stride 1 / pad 1 / dilation 1 with C_in % 8 == 0,
 * C_out % 32 == 0 and 16-byte aligned tensors takes the MFMA implicit-GEMM
 * kernel (which also writes cache_out, in the same pass); bf16 1x1x1 /
 * stride 1 / pad 0 with the same channel rules takes the MFMA projection
 * kernel; the downsampling convs of [P1] 10.5 (bf16, same channel rules,
 * dilation 1) take MFMA routes of their own, counted as fast_strided: the
 * per-frame 1x3x3 stride (1,2,2) conv, and the 3x1x1 stride (2,1,1) conv
 * without spatial padding; every
 * other legal call takes the direct-convolution route (counted as generic,
 * refused with WVC_ERR_STRICT in strict mode).  groups != 1 is
 * WVC_ERR_UNSUPPORTED ([P3]: its fast path covers 5-D tensors, unit temporal
 * stride and one group; this library adds the strided routes the encoder
 * needs, which [P3] leaves to the stock conv).
 * Aliasing: y, cache_out and workspace may not overlap any other buffer of the
 * call (WVC_ERR_ALIAS); read-only buffers may overlap each other (residual ==
 * x is legal).  cache_in and cache_out must therefore be distinct buffers.
 * Upsampled input (d->upsample_in == 2): the decoder's nearest 2x spatial
 * upsample feeding this conv, read inside the conv's halo staging, so the
 * upsampled frames never reach memory.  The conv computes exactly the call
 * above on X'[.., 2i+a, 2j+b] = x[.., i, j] (a, b in {0, 1}), per frame, with
 * the cache carrying the past input frames before the upsample: x is
 * [N, C_in, t, h/2, w/2], cache_in / cache_out are [N, C_in, F, h/2, w/2], y
 * and residual are [N, C_out, t, h, w].  The result is bitwise that of
 * wvc_upsample_nearest2x followed by the conv on the upsampled frames and
 * caches.  h and w must be even; the call must take the MFMA 3x3x3 route
 * (bf16 here, or E4M3 codes through wvc_causal_conv3d_e4m3_fwd), else
 * WVC_ERR_UNSUPPORTED (no other route reads through the upsample).
 * 0 = no upsample; other values are WVC_ERR_ARG.
 */
int wvc_causal_conv3d_fwd(const wvc_conv3d_desc *d, const void *x, const void *cache_in,
                          void *cache_out, const void *weight, const void *bias,
                          const void *residual, void *y, void *workspace,
                          size_t workspace_bytes, void *stream);

/*
 * wvc_causal_conv3d_fwd for callers that cannot allocate device memory: code
 * under HIP graph capture, serving loops and harnesses that forbid hipMalloc.
 * The same kernels run; their scratch (split-K partial sums, and the packed
 * weights when standard-layout weights come in) lives in a fixed device array
 * inside the library, WVC_NOALLOC_SCRATCH_MIB MiB per GPU, held until the
 * process ends, instead of a caller workspace.  The call allocates nothing;
 * the caller still passes every input and output.
 *   Arguments, routes, results and errors as for wvc_causal_conv3d_fwd; a
 *   call whose wvc_causal_conv3d_workspace_bytes(d) exceeds the array fails
 *   with WVC_ERR_WORKSPACE before anything is enqueued.  The stream must
 *   belong to the current device.  The array's contents on entry do not
 *   matter (nothing in it needs clearing).
 *   Every call on one GPU shares that GPU's array, which keeps the last call's
 *   contents: calls that overlap in time on one GPU (different streams or
 *   threads) race on it and give wrong results.  Serialise them, e.g. on one
 *   stream.
 */
#define WVC_NOALLOC_SCRATCH_MIB 48
int wvc_causal_conv3d_fwd_noalloc(const wvc_conv3d_desc *d, const void *x, const void *cache_in,
                                  void *cache_out, const void *weight, const void *bias,
                                  const void *residual, void *y, void *stream);

/* Bytes of workspace wvc_causal_conv3d_fwd needs for this descriptor
 * (0 when none; (size_t)-1 for an invalid descriptor).  A call with
 * standard-layout weights on a fast route needs room to pack them. */
size_t wvc_causal_conv3d_workspace_bytes(const wvc_conv3d_desc *d);

/*
 * A causal conv followed by the RMS norm + SiLU of the layer it feeds
 * ([P1] 10.3 for the conv and the residual block, 10.2 and 10.4 for the norm
 * and SiLU: a block's conv1 feeds norm2, its conv2 plus the shortcut feeds
 * the next block's norm1):
 *   y = round_bf16(conv_d(x | cache_in) + bias + residual)   (C_out channels)
 *   h = round_bf16(silu(rmsnorm(y; gamma, beta, eps)))
 * y is bit for bit what wvc_causal_conv3d_fwd stores and h what
 * wvc_rmsnorm_silu stores for that y.  Arguments as for wvc_causal_conv3d_fwd
 * (d->upsample_in included: the decoder's conv after its upsample feeds the
 * next block's norm this way), plus gamma [C_out], beta [C_out] or NULL,
 * eps > 0 and the output
 * h [N, C_out, t_out, h_out, w_out]; y may be NULL when only h is wanted.
 * When the conv's plan splits K, its split sums go straight into the norm
 * kernel, which adds them in split order, then the bias and the residual,
 * rounds y once (storing it when y is given) and normalises it: the split-K
 * reduce and the norm are one kernel.  bf16 only, C_out % 8 == 0 and
 * C_out <= 2048 (WVC_ERR_UNSUPPORTED otherwise).  The workspace must hold
 * wvc_causal_conv3d_norm_workspace_bytes(d) bytes (the conv's workspace plus
 * room for y); its contents on entry do not matter.  Written buffers (y, h,
 * cache_out, workspace) may not overlap the others (WVC_ERR_ALIAS).
 */
int wvc_causal_conv3d_norm_fwd(const wvc_conv3d_desc *d, const void *x, const void *cache_in,
                               void *cache_out, const void *weight, const void *bias,
                               const void *residual, void *y, const void *gamma, const void *beta,
                               float eps, void *h, void *workspace, size_t workspace_bytes,
                               void *stream);
size_t wvc_causal_conv3d_norm_workspace_bytes(const wvc_conv3d_desc *d);

/*
 * Weights in MFMA fragment order.  The fast routes read each wave's weight
 * fragment (M output channels x one MFMA K-step, M = 32 or 16 by C_out) as
 * one contiguous 1 KiB block; wvc_conv3d_pack_weights writes that order once,
 * so repeated calls with the same weights (a streamed layer) skip the packing
 * pass.  The packed tensor depends only on C_out, C_in and the kernel size of
 * the descriptor (not on t, h or w).
 *   wvc_conv3d_packed_weight_bytes: size of the packed tensor, (size_t)-1 if
 *     the descriptor does not take a fast route (bf16, 3x3x3 or 1x1x1 as above).
 *   wvc_conv3d_pack_weights: weight (standard layout, read) -> packed
 *     (written, wvc_conv3d_packed_weight_bytes(d) bytes, must not overlap
 *     weight), enqueued on stream.  Channels past C_in are zero-filled.
 * Use the result with d->weight_layout = WVC_WEIGHT_PACKED.
 */
size_t wvc_conv3d_packed_weight_bytes(const wvc_conv3d_desc *d);
int wvc_conv3d_pack_weights(const wvc_conv3d_desc *d, const void *weight, void *packed,
                            void *stream);

/* Name of the kernel a wvc_causal_conv3d_fwd call with this descriptor
 * launches on the current device (with its template arguments, as profilers
 * print it; a split-K plan names its reduce kernel too), for profiling and
 * tests ([P3]: the counters show which route a call took; this names the
 * variant inside the route).  The aligned-tensor case is assumed.  "" for an
 * invalid descriptor.  The text lives in a thread-local buffer, valid until
 * the thread's next call of this function. */
const char *wvc_conv3d_kernel_name(const wvc_conv3d_desc *d);

/* Past frames F a causal conv keeps: dil_t * (kT - 1) ([P1] 10.3, the causal
 * pad tuple puts all temporal padding before frame 0).  -1 if d is invalid. */
int wvc_conv3d_cache_frames(const wvc_conv3d_desc *d);

/*
 * Channel RMS norm, optionally followed by SiLU, [P1] 10.2 and 10.4:
 * for each (n, t, h, w), with v the C channel values,
 *   u_c = v_c / max(||v||_2, eps) * sqrt(C) * gamma_c + beta_c
 *   y_c = apply_silu ? u_c * sigmoid(u_c) : u_c
 * computed in fp32 and rounded once to the storage type.
 *   x, y   [N, C, T, H, W] channels-last; y may not overlap x (WVC_ERR_ALIAS)
 *   gamma  [C]; beta [C] or NULL (zero)
 * eps must be > 0 (the pages print none; 1e-12 matches the L2-normalise call
 * the page names).
 */
int wvc_rmsnorm_silu(const void *x, const void *gamma, const void *beta, void *y, int n, int c,
                     int t, int h, int w, int dtype, float eps, int apply_silu, void *stream);

/* Descriptor of one residual-block call over a chunk of t frames. */
typedef struct wvc_resblock_desc {
    int n, c_in, c_out, t, h, w;
    int dtype;
    float eps;          /* RMS-norm clamp, > 0 */
    int weights_packed; /* 1: w1, w2, w_short were packed by wvc_conv3d_pack_weights */
    int cu_limit;       /* 0, or the number of CUs the block's convs plan their
                           grids for (wvc_conv3d_desc.cu_limit); < 0 is WVC_ERR_ARG */
} wvc_resblock_desc;

/* Parameters of one residual block ([P1] 10.4).  All device pointers. */
typedef struct wvc_resblock_params {
    const void *gamma1, *beta1; /* norm1 over C_in; beta1 may be NULL   */
    const void *w1, *b1;        /* conv1 3x3x3 C_in -> C_out; b1 may be NULL */
    const void *gamma2, *beta2; /* norm2 over C_out; beta2 may be NULL  */
    const void *w2, *b2;        /* conv2 3x3x3 C_out -> C_out           */
    const void *w_short, *b_short; /* 1x1x1 shortcut C_in -> C_out; must be
                                      given when C_in != C_out, NULL otherwise
                                      (identity shortcut) */
} wvc_resblock_params;

/*
 * Wan residual block on one chunk, [P1] 10.4:
 *   h1 = SiLU(norm1(x)); a1 = conv1(h1 | cache1); h2 = SiLU(norm2(a1));
 *   y  = conv2(h2 | cache2) + shortcut(x)
 * (Dropout is the identity at inference.)  The caches hold the conv inputs
 * h1 and h2 (post norm + SiLU): cache1 is [N, C_in, 2, H, W], cache2
 * [N, C_out, 2, H, W]; the *_in ones may be NULL (sequence start), the *_out
 * ones receive the last 2 frames of concat(cache_in, h) and may be NULL.
 * The residual is added in conv2's epilogue, before the single rounding.
 *   x [N, C_in, t, H, W] read; y [N, C_out, t, H, W] written.
 * Workspace: wvc_resblock_workspace_bytes(d) bytes (intermediates h1, a1, h2,
 * the shortcut output and the convs' scratch); it may not overlap any other
 * buffer, and its contents on entry do not matter.
 */
int wvc_resblock_fwd(const wvc_resblock_desc *d, const void *x, void *y,
                     const wvc_resblock_params *p, const void *cache1_in, void *cache1_out,
                     const void *cache2_in, void *cache2_out, void *workspace,
                     size_t workspace_bytes, void *stream);

size_t wvc_resblock_workspace_bytes(const wvc_resblock_desc *d);

/*
 * The same block in two halves ([P1] 10.4 read as front = the path up to
 * conv2's input, back = conv2 and the residual):
 *   wvc_resblock_front:  h2 = SiLU(norm2(conv1(SiLU(norm1(x)) | cache1)))
 *   wvc_resblock_back:   y  = conv2(h2 | cache2) + shortcut(x)
 * wvc_resblock_fwd is front then back.  The back half of chunk i and the
 * front half of chunk i+1 touch disjoint state (cache2 vs cache1), so a
 * caller may run them concurrently on two streams; each half then needs its
 * own workspace (wvc_resblock_workspace_bytes(d) bytes each, contents on
 * entry do not matter) and each chunk its own h2 until its back half is done.
 * h2 is [N, C_out, t, H, W] in the call's dtype, caller-owned, and may not
 * overlap any other buffer of the call.  Arguments and errors otherwise as
 * for wvc_resblock_fwd; the front half needs gamma1, w1, gamma2, the back
 * half w2 (and w_short when C_in != C_out).
 */
int wvc_resblock_front(const wvc_resblock_desc *d, const void *x, void *h2,
                       const wvc_resblock_params *p, const void *cache1_in, void *cache1_out,
                       void *workspace, size_t workspace_bytes, void *stream);
int wvc_resblock_back(const wvc_resblock_desc *d, const void *h2, const void *x, void *y,
                      const wvc_resblock_params *p, const void *cache2_in, void *cache2_out,
                      void *workspace, size_t workspace_bytes, void *stream);

/*
 * Zero-fills `bytes` bytes of a cache (a fill kernel, never a memset node, so
 * it can be recorded in a graph).  [P1] 10.3 pads the temporal axis with zeros
 * before frame 0 only (the causal pad tuple), and 8.5 concatenates the cached
 * past frames in front of each chunk; a zeroed cache therefore reproduces
 * that zero padding exactly, so this restarts a stream.  bytes % 4 == 0;
 * WVC_ERR_ARG for a NULL cache with bytes > 0 or a misaligned pointer/size.
 */
int wvc_cache_reset(void *cache, size_t bytes, void *stream);

/*
 * Nearest-neighbour 2x spatial upsample, per frame, no temporal change:
 * y[n, c, t, 2h+i, 2w+j] = x[n, c, t, h, w], i, j in {0, 1}.  The decoder
 * upsamples back towards pixels; the pages give no operator detail, so this is
 * the plainest reading.  x [N,C,T,H,W], y [N,C,T,2H,2W]; y may not overlap x.
 */
int wvc_upsample_nearest2x(const void *x, void *y, int n, int c, int t, int h, int w, int dtype,
                           void *stream);

/*
 * Spatial tiling with overlap blending ([P5] "VSR Hover Comparison", the
 * decoder-tiling paragraph: the latent is decoded in overlapping spatial
 * tiles, (60, 104) at stride (30, 52) there, and the decoded tiles are fused
 * with complementary linear-ramp weights).  A caller extracts each latent tile,
 * decodes it through the stack (its own caches, all frames), blends the
 * decoded tile into an fp32 accumulator, and finishes once all tiles are in.
 *
 * wvc_tile_extract: tile[n, c, t, i, j] = x[n, c, t, y0 + i, x0 + j] for
 *   i < th, j < tw.  x [N, C, T, H, W], tile [N, C, T, th, tw]; the window must
 *   lie inside the frame.
 * wvc_tile_blend: for i < th, j < tw, with w = wy(i) * wx(j):
 *   acc[n, c, t, y0 + i, x0 + j] += w * tile[n, c, t, i, j] and
 *   wsum[y0 + i, x0 + j] += w.  Along an axis of length L the weight is
 *   (i + 1/2)/lo over the lo = ramp_top (ramp_left) pixels shared with the
 *   previous tile, times (L - i - 1/2)/hi over the hi = ramp_bottom
 *   (ramp_right) pixels shared with the next tile, else 1 (a tile's two ramps
 *   may meet).  tile [N, C, T, th, tw] in the call's dtype; acc fp32
 *   [N, C, T, H, W] channels-last; wsum fp32 [H, W]; both zeroed by the
 *   caller (wvc_cache_reset) before the first tile.  C % 4 == 0; ramps in
 *   [0, th] / [0, tw]; the tile must lie inside [H, W].
 * wvc_tile_blend_finish: y = acc / wsum per position, rounded once to the
 *   dtype; every position must have been covered (wsum > 0).
 * All three only enqueue work; tiles blended into one accumulator must be
 * enqueued in order on one stream.  Written buffers may not overlap the
 * others (WVC_ERR_ALIAS).
 */
int wvc_tile_extract(const void *x, void *tile, int n, int c, int t, int h, int w, int y0, int x0,
                     int th, int tw, int dtype, void *stream);
int wvc_tile_blend(const void *tile, float *acc, float *wsum, int n, int c, int t, int th, int tw,
                   int h, int w, int y0, int x0, int ramp_top, int ramp_bottom, int ramp_left,
                   int ramp_right, int dtype, void *stream);
int wvc_tile_blend_finish(const float *acc, const float *wsum, void *y, int n, int c, int t, int h,
                          int w, int dtype, void *stream);

/*
 * Fused RMS norm + SiLU and the encoder's stride-2 spatial conv ([P1] 10.5:
 * the norm + SiLU before the per-frame zero pad and 3x3 stride-2 conv; 10.2
 * and 10.4 for the norm and SiLU):
 *   y = conv_d( round_bf16( silu( rmsnorm(x; gamma, beta, eps) ) ) ) + residual
 * with the norm of wvc_rmsnorm_silu over C_in and the conv of
 * wvc_causal_conv3d_fwd for descriptor d; the zero padding of the conv pads
 * the normalised tensor.  The normalised tensor is computed inside the conv's
 * staging and never stored: one pass over x instead of three.  d must take
 * the MFMA 1x3x3 stride (1,2,2) route (bf16, C_in % 32 == 0, C_out % 16 == 0,
 * C_out <= 256; WVC_ERR_UNSUPPORTED otherwise); all tensors 16-byte aligned.
 * gamma [C_in], beta [C_in] or NULL, bf16; eps > 0.  The norm's fp32 sum of
 * squares may be ordered differently from wvc_rmsnorm_silu's, so results can
 * differ from the unfused pair in the last bit of a few normalised values.
 */
int wvc_rmsnorm_silu_conv3d_fwd(const wvc_conv3d_desc *d, const void *x, const void *gamma,
                                const void *beta, float eps, const void *weight, const void *bias,
                                const void *residual, void *y, void *workspace,
                                size_t workspace_bytes, void *stream);

/*
 * 8-bit (E4M3) path.  [P1] sections 7 and 9 name 8-bit weights and
 * activations for the Conv3D as the way to cut the bytes of the 16-bit
 * engine; on MI355X the 8-bit float the matrix cores read is OCP E4M3
 * (OFP8: exponent bias 7, no infinities, largest finite 448, codes 0x7F and
 * 0xFF are NaN), which also runs the MFMA at twice the bf16 rate.  Codes are
 * carried as bytes.  Every quantiser rounds to the nearest code, ties to the
 * even code, and saturates at +-448; the code of a NaN input is unspecified.
 * Quantisation multiplies by the reciprocal of the scale, both rounded to
 * fp32: q = E4M3(fl32(x * fl32(1 / scale))); the real value of code q is
 * decode(q) * scale.
 *
 * wvc_quantize_e4m3: count elements of x (WVC_BF16 or WVC_F32, any layout)
 *   with one per-tensor scale (finite, > 0, host value) -> q (count bytes,
 *   written, may not overlap x).
 * wvc_quantize_rows_e4m3: x viewed as [rows][cols] (row-major) -> q, with one
 *   scale per row written to scale[rows] (fp32, device): scale_r =
 *   fl32(amax_r / 448), 1 for an all-zero row.  For conv weights in the
 *   standard layout a row is one output channel: the per-channel weight scales
 *   of the 8-bit conv.
 * wvc_rmsnorm_silu_e4m3: wvc_rmsnorm_silu of a bf16 x whose result is stored
 *   as codes (q [N, C, T, H, W] channels-last bytes, may not overlap x) with
 *   the per-tensor activation scale `scale` (finite, > 0): the norm writes the
 *   8-bit conv's input directly, 1 byte per element instead of 2.
 *
 * wvc_causal_conv3d_e4m3_fwd: the causal 3x3x3 conv of wvc_causal_conv3d_fwd
 *   on codes.  d->dtype must be WVC_E4M3; only 3x3x3, stride 1, pad 1,
 *   dilation 1 with C_in % 16 == 0 and C_out % 32 == 0 and 16-byte aligned
 *   tensors is supported (WVC_ERR_UNSUPPORTED / WVC_ERR_ARG otherwise; there
 *   is no generic 8-bit route).
 *     x, cache_in, cache_out  E4M3 codes, shapes and layouts as for the bf16
 *                             conv; the cache holds codes of the same scale
 *     weight                  E4M3 codes [C_out][3][3][3][C_in], or packed
 *                             by wvc_conv3d_pack_weights with an E4M3
 *                             descriptor (d->weight_layout)
 *     x_scale                 per-tensor activation scale (host, finite > 0)
 *     w_scale                 [C_out] fp32 per-output-channel weight scales
 *                             (device, 16-byte aligned)
 *     bias, residual, y       bf16, as for the bf16 conv
 *   y = round_bf16(x_scale * w_scale[co] * S + b[co] + residual), S the sum of
 *   decode(x code) * decode(w code) over the same taps as the bf16 conv
 *   (products exact, accumulated in fp32).  Workspace: as for the bf16 conv,
 *   wvc_causal_conv3d_workspace_bytes(d) with the E4M3 descriptor.
 *   wvc_causal_conv3d_fwd refuses E4M3 descriptors (WVC_ERR_UNSUPPORTED).
 */
int wvc_quantize_e4m3(const void *x, int dtype, int64_t count, float scale, void *q, void *stream);
int wvc_quantize_rows_e4m3(const void *x, int dtype, int64_t rows, int64_t cols, void *q,
                           float *scale, void *stream);
int wvc_rmsnorm_silu_e4m3(const void *x, const void *gamma, const void *beta, void *q, int n, int c,
                          int t, int h, int w, float eps, int apply_silu, float scale, void *stream);
int wvc_causal_conv3d_e4m3_fwd(const wvc_conv3d_desc *d, const void *x, float x_scale,
                               const void *cache_in, void *cache_out, const void *weight,
                               const float *w_scale, const void *bias, const void *residual,
                               void *y, void *workspace, size_t workspace_bytes, void *stream);

/*
 * wvc_causal_conv3d_e4m3_norm_fwd: the 8-bit conv followed by the RMS norm +
 * SiLU of the layer it feeds, that result stored as codes ([P1] 10.2-10.4
 * for the conv, the norm and the block; the 8-bit counterpart of
 * wvc_causal_conv3d_norm_fwd):
 *   y = round_bf16(x_scale * w_scale[co] * S + b[co] + residual)
 *   q = E4M3(silu(rmsnorm(y; gamma, beta, eps)) / q_scale)
 * y is bit for bit what wvc_causal_conv3d_e4m3_fwd stores, q what
 * wvc_rmsnorm_silu_e4m3 stores for that y at scale q_scale.  Arguments as for
 * wvc_causal_conv3d_e4m3_fwd (d->upsample_in included), plus gamma [C_out]
 * bf16, beta [C_out] bf16 or NULL, eps > 0, q_scale (finite, > 0) and q
 * [N, C_out, t_out, h_out, w_out] channels-last bytes; y may be NULL when
 * only q is wanted.  On a split-K plan the split sums go straight into the
 * norm kernel (split order, the scales, the bias, the residual, one bf16
 * rounding, stored as y when given), so the reduce and the norm are one
 * kernel.  C_out % 8 == 0 and C_out <= 2048 (WVC_ERR_UNSUPPORTED otherwise).
 * Workspace: wvc_causal_conv3d_e4m3_norm_workspace_bytes(d) bytes (the conv's
 * workspace plus room for y), contents on entry irrelevant.  Written buffers
 * (y, q, cache_out, workspace) may not overlap the others (WVC_ERR_ALIAS).
 */
int wvc_causal_conv3d_e4m3_norm_fwd(const wvc_conv3d_desc *d, const void *x, float x_scale,
                                    const void *cache_in, void *cache_out, const void *weight,
                                    const float *w_scale, const void *bias, const void *residual,
                                    void *y, const void *gamma, const void *beta, float eps,
                                    float q_scale, void *q, void *workspace,
                                    size_t workspace_bytes, void *stream);
size_t wvc_causal_conv3d_e4m3_norm_workspace_bytes(const wvc_conv3d_desc *d);

/*
 * The residual block of wvc_resblock_fwd on the 8-bit path (identity
 * shortcut, C_in == C_out): norm1 + SiLU stored as codes at activation scale
 * s1, the 8-bit conv1 (bf16 result), norm2 + SiLU as codes at s2, the 8-bit
 * conv2 plus x:
 *   q1 = E4M3(silu(norm1(x)) / s1)          (quantiser rule above)
 *   h  = round_bf16(s1 * w1_scale[co] * conv(q1 | cache1) + b1)
 *   q2 = E4M3(silu(norm2(h)) / s2)
 *   y  = round_bf16(s2 * w2_scale[co] * conv(q2 | cache2) + b2 + x)
 * d->dtype must be WVC_BF16 (x, y, gamma, beta, biases); w1 and w2 are E4M3
 * codes in the standard layout or packed by wvc_conv3d_pack_weights with an
 * E4M3 descriptor (d->weights_packed); w1_scale/w2_scale [C] fp32, 16-byte
 * aligned.  The caches hold codes: cache1 of q1, cache2 of q2, each
 * [N, C, 2, H, W] bytes (in NULL = zero causal padding; out NULL = skip).
 * The C_in/C_out, alignment and channel rules of the 8-bit conv apply.  On a
 * split-K plan conv1's partial sums are added, scaled and rounded inside the
 * norm2 kernel, bit for bit the h above, so h is never stored.  Workspace:
 * wvc_resblock_e4m3_workspace_bytes(d) bytes, contents on entry irrelevant.
 * Aliasing, errors and streams as for wvc_resblock_fwd.
 */
typedef struct wvc_resblock_e4m3_params {
    const void *gamma1, *beta1;  /* norm1 over C (bf16); beta1 may be NULL */
    const void *w1;              /* conv1 codes                            */
    const float *w1_scale;       /* [C] fp32                               */
    const void *b1;              /* [C] bf16 or NULL                       */
    const void *gamma2, *beta2;  /* norm2; beta2 may be NULL               */
    const void *w2;
    const float *w2_scale;
    const void *b2;
    float s1, s2;                /* activation scales of q1, q2 (> 0)      */
} wvc_resblock_e4m3_params;
int wvc_resblock_e4m3_fwd(const wvc_resblock_desc *d, const void *x, void *y,
                          const wvc_resblock_e4m3_params *p, const void *cache1_in,
                          void *cache1_out, const void *cache2_in, void *cache2_out,
                          void *workspace, size_t workspace_bytes, void *stream);
size_t wvc_resblock_e4m3_workspace_bytes(const wvc_resblock_desc *d);

/* Strict mode ([P3]: a strict mode stops on an unexpected fallback): when on,
 * a call that would take the generic route fails with WVC_ERR_STRICT.
 * Initialised from the environment variable WVC_STRICT (=1 turns it on). */
void wvc_set_strict(int on);
int wvc_get_strict(void);

/* Route counters, process-wide, atomically updated. */
void wvc_get_counters(wvc_counters *out);
void wvc_reset_counters(void);

/* Text of the calling thread's last failure ("" if none).  Valid until the
 * thread's next failing call. */
const char *wvc_last_error(void);

/* Library version string. */
const char *wvc_version(void);

/*
 * Graphs.  A streamed decode enqueues a few dozen short launches per latent
 * frame; [P1] section 8.5 counts the launches of its exported decoder per
 * iteration and section 8.7 lists graph capture as the remedy for their
 * overhead.  These calls record what the other entry points enqueue on one
 * stream into a HIP graph and replay it with one call.
 *
 * wvc_graph_capture_begin(stream): starts a capture (thread-local mode) on
 *   `stream`, which must be a created stream: the null stream cannot be
 *   captured (WVC_ERR_ARG).  Until the matching end, library calls that
 *   enqueue on `stream` from this thread are recorded instead of run.  They
 *   must not need a workspace allocation or a host synchronisation in
 *   between; the library's own calls never make either.
 * wvc_graph_capture_end(stream, graph): ends the capture and instantiates
 *   it.  *graph receives an opaque handle owned by the caller; it is NULL
 *   after a failure (WVC_ERR_HIP, e.g. when a recorded launch was invalid).
 * wvc_graph_launch(graph, stream): enqueues one replay on any stream (NULL
 *   included).  A replay reads and writes exactly the buffers the recorded
 *   calls named, at the sizes and values of their scalar arguments at capture
 *   time: the caller keeps those buffers allocated, at the same addresses,
 *   for the life of the graph.  Replays on one stream run in order, like the
 *   calls they record; the route counters count the recorded calls once.
 * wvc_graph_destroy(graph): releases the handle (NULL is a no-op).  Call it
 *   once every replay has completed (synchronise the replay streams first).
 *
 * The graph handle and the HIP runtime's instantiated graph are the only
 * things the library allocates; none of it is tensor memory.
 */
typedef struct wvc_graph wvc_graph;
int wvc_graph_capture_begin(void *stream);
int wvc_graph_capture_end(void *stream, wvc_graph **graph);
int wvc_graph_launch(const wvc_graph *graph, void *stream);
int wvc_graph_destroy(wvc_graph *graph);

#ifdef __cplusplus
}
#endif
#endif /* WVC_H */
