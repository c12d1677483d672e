// conv_strided.hip -- MFMA routes of the encoder's downsampling convs
// ("Cosmos3 Wan VAE -- engine size vs runtime context memory", section 10.5:
// per frame a zero pad and a stride-2 Conv2d halve H and W, then a causal
// conv with temporal stride 2 halves T).
//
// Both are one GEMM per output frame, y[p, co] = b[co] + sum_k W[co, k] X[k, p]
// with K = kT*kH*kW*C_in in the standard weight order (kt, kh, kw, ci), so
// K-step ks of 32 channels is tap ks / (C_in/32), channel block ks % (C_in/32).
//
//   * temporal (MODE 0): 3x1x1, temporal stride s, no spatial padding.  Output
//     frame j is anchored at chunk frame a = t0 + j*s and tap kt reads frame
//     a - 2 + kt (the cache's frames before the chunk, zeros at a sequence
//     start).  A position's K vector is its 3 tapped frames' channel vectors.
//   * spatial (MODE 1): 1x3x3, spatial stride 2, zero pad ph/pw before and
//     ph+eh/pw+ew after the frame.  Output (ho, wo) reads input rows
//     2ho - ph + kh and columns 2wo - pw + kw.
//
// A workgroup owns PT consecutive output positions (a run of a frame in MODE
// 0, a run of one output row in MODE 1) and every output channel, so the
// activation bytes cross HBM once.  It stages what those positions read in
// LDS with coalesced 16-byte loads:
//   MODE 0: [position][K/8 chunks + 1 pad];
//   MODE 1: [kh][column slot][C_in/8 chunks + 1 pad] for the 2*PT+1 input
//     columns of the 3 input rows, even columns in slots 0..PT and odd ones in
//     PT+1..2PT, so that the 16 lanes of a B-fragment read (16 consecutive
//     output columns, input columns 2 apart) hit consecutive slots.
// The rows are padded to an odd number of 16-byte entries, so those reads
// land in distinct LDS banks.  The weights stream from L2 as 16x16x32 MFMA A
// fragments, several K-steps ahead: a K-step is only FCO x FPOS MFMAs, far
// shorter than an L2 round trip.  Waves split output channels x positions:
// WCO groups of FCO 16-channel blocks times 4/WCO groups of FPOS 16-position
// blocks.
//
// Fused norm (NORM, spatial route): the conv's input is the RMS norm + SiLU
// of x (section 10.2 and 10.4 of the same page; the downsample path puts it
// right before the stride-2 conv).  Each staged input position holds all
// C_in channels, so after staging one thread per position computes its
// channel norm in LDS, applies gamma, beta and SiLU, rounds to bf16 (the value
// the norm kernel would have stored) and writes it back; positions in the
// zero padding stay zero.  The normalised tensor never goes through HBM.
#include <type_traits>

#include "wvc_internal.h"
#include "wvc.h"

namespace wvc {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr int BATCH = 20;              // staging loads in flight per thread (one batch at C_in = 96)
constexpr size_t LDS_MAX = 80 * 1024;  // two workgroups per CU

template <int I>
using Int = std::integral_constant<int, I>;

template <int N, int I = 0, typename F>
__device__ __forceinline__ void static_for(F &&f) {
    if constexpr (I < N) {
        f(Int<I>{});
        static_for<N, I + 1>(f);
    }
}

// q / d for 0 <= q < 2^15 and d >= 1, exactly: q + 0.5 is exact in fp32 and
// the rounded product is within (q + 0.5)/d * 2^-23 < 2^-8/d of (q + 0.5)/d,
// which lies at least 0.5/d away from every integer.
__device__ __forceinline__ int div_small(int q, float inv_d) {
    return (int)(((float)q + 0.5f) * inv_d);
}

struct SParams {
    const uint16_t *x, *cache, *wp, *bias, *res;
    uint16_t *y;
    const uint16_t *gamma, *beta;  // fused norm (NORM): gamma [C_in], beta [C_in] or null
    float eps, norm_scale;         // norm clamp and sqrt(C_in)
    int n, t, h, w, ho, wo, cin, cout;
    int F, st, t0, to;  // cache frames, temporal stride, first anchor, output frames
    int ph, pw;
    int tiles;          // position tiles per output frame (MODE 0) or row (MODE 1)
    int nb;             // K-steps of 32
    int pitch;          // LDS row pitch in 16-byte entries
    uint32_t w_bytes;
};

__device__ __forceinline__ bf16x8 as_bf16x8(uint4 v) { return __builtin_bit_cast(bf16x8, v); }

__device__ __forceinline__ uint4 wload(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0);
    return make_uint4(v.x, v.y, v.z, v.w);
}

// Workgroup ids are dispatched round-robin over the 8 XCDs, each with its own
// L2.  Hand XCD k the k-th contiguous slice of the logical order instead, so
// that neighbouring runs (which share input rows: an input row feeds two
// output rows at stride 2) are staged through the same L2.  A bijection on
// [0, total).
__device__ __forceinline__ long xcd_slice(long bid, long total) {
    const long xcd = bid & 7, local = bid >> 3;
    const long per = total >> 3, rem = total & 7;
    const long start = xcd < rem ? xcd * (per + 1) : rem * (per + 1) + (xcd - rem) * per;
    return start + local;
}

// C8T: C_in / 8 when known at compile time (0: read from p).  With it every
// division of the staging and K-step index arithmetic is by a constant, and
// the K loop's trip counts are constants; the 96-channel path uses it.
template <int MODE, int PT, int FCO, int FPOS, int WCO, int C8T = 0, bool NORM = false>
__global__ void __launch_bounds__(256) strided_kernel(SParams p) {
    static_assert(FPOS * 16 * (4 / WCO) == PT, "position groups must tile the run");
    static_assert(!NORM || MODE == 1, "the fused norm is on the spatial route");
    // A-fragment register sets = K-steps in flight.  The K-step count is
    // taps x C_in/32, a multiple of the tap count, so NS = taps divides it:
    // the K loop body then has no bounds checks, and the compiler's wait
    // counts stay exact across iterations instead of draining every load at
    // the loop head.
    constexpr int NS = MODE == 0 ? 3 : 9;
    extern __shared__ uint4 xs[];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wc = wave % WCO, wq = wave / WCO;  // channel group, position group
    const int lr = lane & 15, lg = lane >> 4;
    const int nblk = p.cout / 16;
    const int c8 = C8T ? C8T : p.cin / 8, cbs = c8 / 4;
    const int nb = C8T ? (MODE == 0 ? 3 : 9) * (C8T / 4) : p.nb;  // K-steps

    // Workgroup -> (n, output frame j, row / tile); MODE 1 adds the output row.
    long L = xcd_slice(blockIdx.x, gridDim.x);
    const int tile = (int)(L % p.tiles);
    L /= p.tiles;
    int oh = 0;
    if (MODE == 1) {
        oh = (int)(L % p.ho);
        L /= p.ho;
    }
    const int j = (int)(L % p.to);
    const int n = (int)(L / p.to);
    const int q0 = tile * PT;  // first output position (MODE 0) / column (MODE 1)
    const int npos = MODE == 0 ? p.ho * p.wo : p.wo;
    const int np = npos - q0 < PT ? npos - q0 : PT;
    const size_t frame = (size_t)p.h * p.w * p.cin;

    // ---- staging
    if constexpr (MODE == 0) {
        // Three tapped frames of the anchor: chunk frames a-2..a, or cache.
        const int a = p.t0 + j * p.st;
        const uint16_t *src[3];
#pragma unroll
        for (int kt = 0; kt < 3; ++kt) {
            const int f = a - 2 + kt;
            src[kt] = f >= 0 ? p.x + ((size_t)n * p.t + f) * frame
                             : (p.cache ? p.cache + ((size_t)n * p.F + p.F + f) * frame : nullptr);
        }
        const int ke = nb * 4;  // 16-byte chunks per position
        const int total = PT * ke;
        const float inv_ke = 1.0f / (float)ke, inv_c8 = 1.0f / (float)c8;
        for (int base = 0; base < total; base += 256 * BATCH) {
            uint4 v[BATCH];
            int dst[BATCH];
#pragma unroll
            for (int k = 0; k < BATCH; ++k) {
                const int q = base + tid + 256 * k;
                const int r = C8T ? q / ke : div_small(q, inv_ke), e = q - r * ke;
                const int kt = C8T ? e / c8 : div_small(e, inv_c8), ch = e - kt * c8;
                const uint16_t *sp = kt == 0 ? src[0] : (kt == 1 ? src[1] : src[2]);
                v[k] = make_uint4(0u, 0u, 0u, 0u);
                dst[k] = q < total ? r * p.pitch + e : -1;
                if (q < total && r < np && sp)
                    v[k] = *reinterpret_cast<const uint4 *>(sp + (size_t)(q0 + r) * p.cin + ch * 8);
            }
#pragma unroll
            for (int k = 0; k < BATCH; ++k)
                if (dst[k] >= 0) xs[dst[k]] = v[k];
        }
    } else if constexpr (C8T != 0) {
        // Constant channel count: one buffer resource per input row (bounded
        // to the row, so columns outside the frame -- negative offsets wrap
        // to huge ones -- and rows outside it read zero in hardware) and all
        // 3 rows' loads in flight before the first LDS store.
        const uint16_t *fp = p.x + ((size_t)n * p.t + j) * frame;
        constexpr int NC = 2 * PT + 1, PER_ROW = NC * C8T, KPR = (PER_ROW + 255) / 256;
        const int row_bytes = p.w * p.cin * 2;
        const int col0 = 2 * q0 - p.pw;
        uint4 v[3][KPR];
#pragma unroll
        for (int kh = 0; kh < 3; ++kh) {
            const int hs = 2 * oh - p.ph + kh;
            const bool ok = hs >= 0 && hs < p.h;
            const __amdgpu_buffer_rsrc_t rr = __builtin_amdgcn_make_buffer_rsrc(
                const_cast<uint16_t *>(fp + (size_t)(ok ? hs : 0) * p.w * p.cin), (short)0,
                ok ? row_bytes : 0, 0x00020000);
#pragma unroll
            for (int k = 0; k < KPR; ++k) {
                const int q = tid + 256 * k;
                const int cc = q / C8T, ch = q - cc * C8T;
                const int off = q < PER_ROW ? (col0 + cc) * p.cin * 2 + ch * 16 : -1;
                const u32x4 t4 = __builtin_amdgcn_raw_buffer_load_b128(rr, off, 0, 0);
                v[kh][k] = make_uint4(t4.x, t4.y, t4.z, t4.w);
            }
        }
#pragma unroll
        for (int kh = 0; kh < 3; ++kh)
#pragma unroll
            for (int k = 0; k < KPR; ++k) {
                const int q = tid + 256 * k;
                const int cc = q / C8T, ch = q - cc * C8T;
                const int slot = (cc & 1) ? PT + 1 + (cc >> 1) : (cc >> 1);
                if (q < PER_ROW) xs[(kh * NC + slot) * (C8T + 1) + ch] = v[kh][k];
            }
    } else {
        const uint16_t *fp = p.x + ((size_t)n * p.t + j) * frame;  // spatial: t_out == t
        constexpr int NC = 2 * PT + 1;                              // input columns
        const int total = 3 * NC * c8;
        const int col0 = 2 * q0 - p.pw;
        const float inv_c8 = 1.0f / (float)c8, inv_nc = 1.0f / (float)NC;
        for (int base = 0; base < total; base += 256 * BATCH) {
            uint4 v[BATCH];
            int dst[BATCH];
#pragma unroll
            for (int k = 0; k < BATCH; ++k) {
                const int q = base + tid + 256 * k;
                const int rest = C8T ? q / c8 : div_small(q, inv_c8), ch = q - rest * c8;
                const int kh = C8T ? rest / NC : div_small(rest, inv_nc), cc = rest - kh * NC;
                const int hs = 2 * oh - p.ph + kh, ws = col0 + cc;
                const int slot = (cc & 1) ? PT + 1 + (cc >> 1) : (cc >> 1);
                v[k] = make_uint4(0u, 0u, 0u, 0u);
                dst[k] = q < total ? (kh * NC + slot) * p.pitch + ch : -1;
                if (q < total && hs >= 0 && hs < p.h && ws >= 0 && ws < p.w)
                    v[k] = *reinterpret_cast<const uint4 *>(fp + ((size_t)hs * p.w + ws) * p.cin + ch * 8);
            }
#pragma unroll
            for (int k = 0; k < BATCH; ++k)
                if (dst[k] >= 0) xs[dst[k]] = v[k];
        }
    }

    // ---- fused norm + SiLU of the staged positions (spatial route)
    if constexpr (NORM) {
        __syncthreads();  // every staged chunk is in LDS
        constexpr int NC = 2 * PT + 1;
        const int col0 = 2 * q0 - p.pw;
        const uint4 *gq = reinterpret_cast<const uint4 *>(p.gamma);
        const uint4 *bq = reinterpret_cast<const uint4 *>(p.beta);
        auto unpack = [](uint4 u, float *o) {
            const uint32_t wd[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                o[2 * k] = bf16_to_f32(wd[k] & 0xffffu);
                o[2 * k + 1] = bf16_to_f32(wd[k] >> 16);
            }
        };
        for (int pos = tid; pos < 3 * NC; pos += 256) {
            const int kh = pos / NC, slot = pos - kh * NC;
            const int cc = slot <= PT ? 2 * slot : 2 * (slot - PT - 1) + 1;
            const int hs = 2 * oh - p.ph + kh, ws = col0 + cc;
            const bool in = hs >= 0 && hs < p.h && ws >= 0 && ws < p.w;
            uint4 *e = xs + (size_t)pos * (C8T ? C8T + 1 : p.pitch);
            float ss = 0.f;
            for (int k = 0; k < c8; ++k) {
                float v[8];
                unpack(e[k], v);
#pragma unroll
                for (int i = 0; i < 8; ++i) ss = fmaf(v[i], v[i], ss);
            }
            const float r = p.norm_scale / fmaxf(sqrtf(ss), p.eps);
            for (int k = 0; k < c8; ++k) {
                float v[8], g[8], b[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
                unpack(e[k], v);
                unpack(gq[k], g);
                if (bq) unpack(bq[k], b);
                uint32_t o[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const float u0 = fmaf(v[2 * i] * r, g[2 * i], b[2 * i]);
                    const float u1 = fmaf(v[2 * i + 1] * r, g[2 * i + 1], b[2 * i + 1]);
                    o[i] = pack2_bf16(u0 * __builtin_amdgcn_rcpf(1.f + __expf(-u0)),
                                      u1 * __builtin_amdgcn_rcpf(1.f + __expf(-u1)));
                }
                e[k] = in ? make_uint4(o[0], o[1], o[2], o[3]) : make_uint4(0u, 0u, 0u, 0u);
            }
        }
    }

    // ---- weights: packed [K-step][16-row block][lane] 1 KiB fragments
    const __amdgpu_buffer_rsrc_t wr =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t *>(p.wp), (short)0, (int)p.w_bytes, 0x00020000);
    bf16x8 A[NS][FCO];
    auto load_a = [&](auto set_tag, int ks) {
        constexpr int SET = decltype(set_tag)::value;
#pragma unroll
        for (int f = 0; f < FCO; ++f) {
            const int blk = wc * FCO + f;
            const int bc = blk < nblk ? blk : 0;  // surplus blocks read block 0, never stored
            A[SET][f] = as_bf16x8(wload(wr, (uint32_t)((ks * nblk + bc) * 1024 + lane * 16)));
        }
    };
    // K-steps 0 .. NS-2 in flight before the first MFMA.
    static_for<NS - 1>([&](auto i) {
        constexpr int I = decltype(i)::value;
        load_a(i, I < nb ? I : nb - 1);
    });

    f32x4 acc[FCO][FPOS];
#pragma unroll
    for (int f = 0; f < FCO; ++f)
#pragma unroll
        for (int b = 0; b < FPOS; ++b) acc[f][b] = f32x4{0.f, 0.f, 0.f, 0.f};
    __syncthreads();

    // LDS entry of the B fragment of position block b at K-step ks: the 16
    // lanes lr are 16 consecutive output positions, lg the 8-channel group.
    const int pos0 = wq * FPOS * 16 + lr;
    auto b_entry = [&](int ks, int b) -> int {
        if (MODE == 0) return (pos0 + b * 16) * p.pitch + ks * 4 + lg;
        const int tap = ks / cbs, cb = ks - tap * cbs;
        const int kh = tap / 3, kw = tap - kh * 3;
        const int pp = pos0 + b * 16;
        const int slot = kw == 1 ? PT + 1 + pp : pp + (kw >> 1);
        return (kh * (2 * PT + 1) + slot) * p.pitch + cb * 4 + lg;
    };
    // K-step ks uses set ks % NS and first refills the set of K-step ks-1
    // (whose MFMAs are issued) with K-step ks + NS - 1 (clamped at the end:
    // the surplus loads are never used).
    // The B fragments of K-step ks+1 are read from LDS (into one of three
    // sets) before the MFMAs of ks, so the LDS latency hides behind them.
    bf16x8 B[3][FPOS];
#pragma unroll
    for (int b = 0; b < FPOS; ++b) B[0][b] = as_bf16x8(xs[b_entry(0, b)]);
    for (int ks0 = 0; ks0 < nb; ks0 += NS) {
        static_for<NS>([&](auto i) {
            constexpr int SET = decltype(i)::value;
            constexpr int BS = SET % 3, BN = (SET + 1) % 3;
            const int ks = ks0 + SET;
            const int nxt = ks + NS - 1 < nb ? ks + NS - 1 : nb - 1;
            load_a(Int<(SET + NS - 1) % NS>{}, nxt);
            const int kb = ks + 1 < nb ? ks + 1 : ks;
#pragma unroll
            for (int b = 0; b < FPOS; ++b) B[BN][b] = as_bf16x8(xs[b_entry(kb, b)]);
#pragma unroll
            for (int b = 0; b < FPOS; ++b)
#pragma unroll
                for (int f = 0; f < FCO; ++f)
                    acc[f][b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A[SET][f], B[BS][b], acc[f][b], 0, 0, 0);
            __builtin_amdgcn_sched_barrier(0);
        });
    }

    // ---- epilogue: element e of tile (f, b) is channel blk*16 + lg*4 + e at
    // position pos0 + b*16; + bias, + residual, one rounding.
    const size_t obase = MODE == 0 ? ((size_t)n * p.to + j) * (size_t)npos + q0
                                   : (((size_t)n * p.to + j) * p.ho + oh) * (size_t)p.wo + q0;
#pragma unroll
    for (int f = 0; f < FCO; ++f) {
        const int blk = wc * FCO + f;
        if (blk >= nblk) continue;
        const int co = blk * 16 + lg * 4;
        float bv[4] = {0.f, 0.f, 0.f, 0.f};
        if (p.bias) {
            const uint2 bb = *reinterpret_cast<const uint2 *>(p.bias + co);
            bv[0] = bf16_to_f32(bb.x & 0xffffu);
            bv[1] = bf16_to_f32(bb.x >> 16);
            bv[2] = bf16_to_f32(bb.y & 0xffffu);
            bv[3] = bf16_to_f32(bb.y >> 16);
        }
#pragma unroll
        for (int b = 0; b < FPOS; ++b) {
            const int r = pos0 + b * 16;
            if (r >= np) continue;
            const size_t o = (obase + r) * p.cout + co;
            float v[4] = {acc[f][b][0] + bv[0], acc[f][b][1] + bv[1], acc[f][b][2] + bv[2],
                          acc[f][b][3] + bv[3]};
            if (p.res) {
                const uint2 rr = *reinterpret_cast<const uint2 *>(p.res + o);
                v[0] += bf16_to_f32(rr.x & 0xffffu);
                v[1] += bf16_to_f32(rr.x >> 16);
                v[2] += bf16_to_f32(rr.y & 0xffffu);
                v[3] += bf16_to_f32(rr.y >> 16);
            }
            *reinterpret_cast<uint2 *>(p.y + o) = make_uint2(pack2_bf16(v[0], v[1]), pack2_bf16(v[2], v[3]));
        }
    }
}

// ---------------------------------------------------------------------------
// Row-walking variant of the spatial route for C_in = C_out = 96 (the encoder
// level the downsample path runs at): persistent workgroups, one per CU, each
// walking down a run of output rows of one 63-column strip.
//
// An item is one output row of a strip: 64 output columns through the MFMAs,
// 63 of them stored (127 input columns per input row).  Output row oh reads
// input rows 2oh-ph .. 2oh-ph+2 and the next output row shares the last of
// them, so a ring of 3 input rows lives in LDS and each item stages 2 new
// rows: each input row is staged once instead of 1.5 times on average, and
// with the fused norm each input position is normalised once.
//
// Waves: 8 (two per SIMD), wave (wc, wq) = output channels 48 wc .. 48 wc + 47
// for the K quarter wq (K-steps 7 wq .. 7 wq + 6; the last quarter has 6 of
// the 27).  Its A fragments (84 VGPRs) stay in registers for the whole run
// instead of streaming 166 KB of weights from L2 per output row.  The K
// quarters of a channel group meet in LDS: each wave stores its partial sums
// of the three 16-column blocks other waves finish and finishes block wq
// itself, adding the four quarters' sums in quarter order (a fixed order,
// whichever wave adds them).
//
// Each wave finishes its block of an item one item late, between the next
// item's K-steps, so that those stores and partial-sum reads overlap MFMAs.
//
// Staging: before an item's MFMAs, the loads of the next item's two input
// rows are issued; after the K loop they go to the ring rows the current item
// was the last to read.  Two threads share a position, 48 channels each: lane
// l of wave w takes position 32 w + (l & 31) (128 per row, the 128th idle)
// and half l >> 5.  With the fused norm the staged values are normalised in
// registers right after the K loop, before the barrier (sum of squares with
// v_dot2_f32_bf16 over the two halves, gamma/beta, SiLU, one rounding to
// bf16), so a wave done with its MFMAs runs this VALU work while the others
// are still in theirs, and the ring receives normalised values only.  A
// strip's first item stages all three rows before its K loop.
//
// LDS row layout.  Column slots of 14 entries (12 chunks of 8 channels + 2
// idle): the even input columns at entries 14 s (s = column / 2), the odd
// ones at 897 + 14 s.  On gfx950 a 16-byte LDS read is served in four lane
// groups of 16 (lanes 0-3, 12-15, 20-23, 24-27 of a half-wave, and the other
// 16 of it), each conflict-free when its lanes hit distinct entries mod 16;
// a 16-byte write in eight groups of 8 consecutive lanes, each conflict-free
// when its lanes hit distinct entries mod 8 (fitted to the SQ bank-conflict
// counter over single-wave access patterns).  So:
//  - a B-fragment read (lane 16 g + r: output column r of a block, chunk g of
//    a 32-channel group) reads 16 consecutive slots of one parity: 14 r is
//    even and takes each even residue mod 16 once over r and r + 8, and each
//    read group holds, for every residue, one lane with g even and one with
//    g odd, so chunk g's own offset g makes the 16 entries distinct;
//  - a staging store (8 consecutive columns, one chunk) lands at 14 a + 14 j
//    for the even columns (4 distinct even residues mod 8) and 897 + 14 a +
//    14 j for the odd ones (the 4 odd residues).
constexpr int RW_C8 = 12;            // 16-byte chunks per position (96 channels)
constexpr int RW_COLS = 127;         // input columns staged per row
constexpr int RW_SROW = 128;         // staging positions per row (the last idle)
constexpr int RW_PT = 63;            // output columns stored per item
constexpr int RW_PITCH = 14;         // entries per column slot
constexpr int RW_ODD = 897;          // first entry of the odd columns
constexpr int RW_ROW = 1792;         // entries per ring row
constexpr int RW_KS = 27;            // K-steps: 9 taps x 3 blocks of 32 channels
constexpr int RW_KQ = 7;             // K-steps per quarter (the last has 6)
constexpr int RW_THREADS = 512;
constexpr int RW_HALF = RW_C8 / 2;   // chunks per staging thread (6)

__device__ __forceinline__ int rw_entry(int col) {
    return (col & 1) ? RW_ODD + (col >> 1) * RW_PITCH : (col >> 1) * RW_PITCH;
}
// Data: even slots 0..63, odd slots 0..62.  Reads of the discarded 64th
// output column also touch odd slot 63 and even slot 64.
static_assert(63 * RW_PITCH + RW_C8 <= RW_ODD && RW_ODD + 63 * RW_PITCH + RW_C8 <= RW_ROW &&
              64 * RW_PITCH + RW_C8 <= RW_ROW,
              "even and odd column regions of a ring row do not overlap; every read stays in the row");

template <bool NORM>
__global__ void __launch_bounds__(RW_THREADS) strided_rows_kernel(SParams p, int items) {
    __shared__ uint4 ring[3 * RW_ROW];
    // partial sums exchanged between the K quarters: red[block b][source
    // quarter, skipping b][wc][f][lane]
    __shared__ f32x4 red[4][3][2][3][64];
    __shared__ float4 gam_s[RW_C8 * 2], bet_s[RW_C8 * 2];
    __shared__ float4 bias_s[24];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wc = wave & 1, wq = wave >> 1;
    const int lr = lane & 15, lg = lane >> 4;
    const int i_begin = (int)((long)blockIdx.x * items / gridDim.x);
    const int i_end = (int)((long)(blockIdx.x + 1) * items / gridDim.x);
    if (i_begin >= i_end) return;  // uniform per workgroup, before any barrier

    if (tid < 24) {
        uint2 bb = make_uint2(0u, 0u);
        if (p.bias) bb = reinterpret_cast<const uint2 *>(p.bias)[tid];
        bias_s[tid] = make_float4(bf16_to_f32(bb.x & 0xffffu), bf16_to_f32(bb.x >> 16),
                                  bf16_to_f32(bb.y & 0xffffu), bf16_to_f32(bb.y >> 16));
    }
    if (NORM && tid < RW_C8 * 2) {
        const uint4 gq = reinterpret_cast<const uint4 *>(p.gamma)[tid >> 1];
        const uint4 bq = p.beta ? reinterpret_cast<const uint4 *>(p.beta)[tid >> 1] : make_uint4(0, 0, 0, 0);
        const uint32_t g0 = (tid & 1) ? gq.z : gq.x, g1 = (tid & 1) ? gq.w : gq.y;
        const uint32_t b0 = (tid & 1) ? bq.z : bq.x, b1 = (tid & 1) ? bq.w : bq.y;
        // gamma and beta times -log2(e): the norm works on t = -log2(e) u
        // (see norm_chunk)
        constexpr float NL2E = -1.4426950408889634f;
        gam_s[tid] = make_float4(NL2E * bf16_to_f32(g0 & 0xffffu), NL2E * bf16_to_f32(g0 >> 16),
                                 NL2E * bf16_to_f32(g1 & 0xffffu), NL2E * bf16_to_f32(g1 >> 16));
        bet_s[tid] = make_float4(NL2E * bf16_to_f32(b0 & 0xffffu), NL2E * bf16_to_f32(b0 >> 16),
                                 NL2E * bf16_to_f32(b1 & 0xffffu), NL2E * bf16_to_f32(b1 >> 16));
    }

    // ---- weights: this wave's A fragments, loaded once
    const __amdgpu_buffer_rsrc_t wr =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t *>(p.wp), (short)0, (int)p.w_bytes, 0x00020000);
    const int ks0 = wq * RW_KQ;
    bf16x8 A[RW_KQ][3];
#pragma unroll
    for (int m = 0; m < RW_KQ; ++m) {
        const int ks = ks0 + m < RW_KS ? ks0 + m : RW_KS - 1;
#pragma unroll
        for (int f = 0; f < 3; ++f)
            A[m][f] = as_bf16x8(wload(wr, (uint32_t)((ks * 6 + wc * 3 + f) * 1024 + lane * 16)));
    }

    const size_t frame = (size_t)p.h * p.w * 96;
    const int frame_bytes = (int)(frame * 2);
    const int tiles = p.tiles;

    // Staging of input rows hs0, hs0 + 1, ... of frame (n, j), columns col0 ..
    // col0 + 126.  Lane l of wave w takes position pbase + 32 w + (l & 31)
    // (row pos / 128, column pos % 128, the 128th idle) and half h = l >> 5
    // of it: chunks 6h .. 6h + 5, channels 48h .. 48h + 47.  A wave's load k
    // reads 16 of every 96 bytes of 32 neighbouring positions, its six loads
    // together read them whole.  The fused norm's sum of squares needs lanes
    // l and l ^ 32 only, and the staged values are normalised in registers
    // before their one store to the ring.
    constexpr int H8 = RW_HALF;
    const int half = lane >> 5;
    uint4 raw[H8];
    int ndst = -1;       // ring entry of this thread's first chunk, -1 when idle
    bool nin = false;    // the position lies inside the frame
    float nr = 0.f;      // its scale sqrt(C) / max(||v||, eps)
    auto issue_pos = [&](int n_, int j_, int hs0, int col0, int pbase, int pend) __attribute__((always_inline)) {
        const __amdgpu_buffer_rsrc_t fr = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<uint16_t *>(p.x + ((size_t)n_ * p.t + j_) * frame), (short)0, frame_bytes, 0x00020000);
        int pos = pbase + 32 * wave + (lane & 31);
        // recomputed per call: hoisted copies would stay live across the item loop
        asm volatile("" : "+v"(pos));
        const int row = pos / RW_SROW, col = pos % RW_SROW;
        const int hs = hs0 + row, ws = col0 + col;
        const bool act = pos < pend && col < RW_COLS;
        // out-of-frame positions (the zero padding) read zero in hardware;
        // a frame is below 2^31 bytes, so 32-bit offsets do
        nin = act && (unsigned)hs < (unsigned)p.h && (unsigned)ws < (unsigned)p.w;
        const uint32_t base = nin ? (uint32_t)(hs * p.w + ws) * 192u + (uint32_t)half * 96u : 0x80000000u;
#pragma unroll
        for (int k = 0; k < H8; ++k) {
            const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(fr, (int)(base + 16u * k), 0, 0);
            raw[k] = make_uint4(v.x, v.y, v.z, v.w);
        }
        ndst = act ? ((hs + 3) % 3) * RW_ROW + rw_entry(col) + H8 * half : -1;
    };
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
    auto norm_sum = [&]() __attribute__((always_inline)) {
        float ss = 0.f;
#pragma unroll
        for (int k = 0; k < H8; ++k) {
            ss = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, raw[k].x),
                                                 __builtin_bit_cast(bf16x2, raw[k].x), ss, false);
            ss = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, raw[k].y),
                                                 __builtin_bit_cast(bf16x2, raw[k].y), ss, false);
            ss = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, raw[k].z),
                                                 __builtin_bit_cast(bf16x2, raw[k].z), ss, false);
            ss = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, raw[k].w),
                                                 __builtin_bit_cast(bf16x2, raw[k].w), ss, false);
        }
        // both lanes of the pair add half 0 + half 1, so both get the same bits
        const float other = __shfl_xor(ss, 32);
        const float tot = half ? other + ss : ss + other;
        nr = p.norm_scale / fmaxf(sqrtf(tot), p.eps);
    };
    // Chunk k of this thread: gamma, beta, SiLU, one rounding.  With
    // u = x r gamma + beta and t = -log2(e) u (gamma and beta are stored
    // pre-scaled), SiLU(u) = u / (1 + e^-u) = t / (-log2(e) (1 + 2^t)): one
    // fma, one exp2, one fma, one reciprocal and one multiply per element.
    // Positions outside the frame are zeroed at the store (the conv's zero
    // padding applies to the norm's output).
    auto norm_chunk = [&](auto k_tag) __attribute__((always_inline)) {
        constexpr int k = decltype(k_tag)::value;
        const int c = half * H8 + k;
        const float4 g0 = gam_s[2 * c], g1 = gam_s[2 * c + 1];
        const float4 b0 = bet_s[2 * c], b1 = bet_s[2 * c + 1];
        const float gg[8] = {g0.x, g0.y, g0.z, g0.w, g1.x, g1.y, g1.z, g1.w};
        const float bb[8] = {b0.x, b0.y, b0.z, b0.w, b1.x, b1.y, b1.z, b1.w};
        const uint32_t wd[4] = {raw[k].x, raw[k].y, raw[k].z, raw[k].w};
        uint32_t o[4];
        constexpr float NL2E = -1.4426950408889634f;
#pragma unroll
        for (int d = 0; d < 4; ++d) {
            const float t0 = fmaf(bf16_to_f32(wd[d] & 0xffffu) * nr, gg[2 * d], bb[2 * d]);
            const float t1 = fmaf(__uint_as_float(wd[d] & 0xffff0000u) * nr, gg[2 * d + 1], bb[2 * d + 1]);
            const float d0 = fmaf(__builtin_amdgcn_exp2f(t0), NL2E, NL2E);
            const float d1 = fmaf(__builtin_amdgcn_exp2f(t1), NL2E, NL2E);
            o[d] = pack2_bf16(t0 * __builtin_amdgcn_rcpf(d0), t1 * __builtin_amdgcn_rcpf(d1));
        }
        raw[k] = make_uint4(o[0], o[1], o[2], o[3]);
    };
    // Without the norm, positions outside the frame already hold the zeros
    // their loads returned.
    auto store_pos = [&]() __attribute__((always_inline)) {
        if (ndst >= 0) {
            if (!NORM || nin) {
#pragma unroll
                for (int k = 0; k < H8; ++k) ring[ndst + k] = raw[k];
            } else {
#pragma unroll
                for (int k = 0; k < H8; ++k) ring[ndst + k] = make_uint4(0u, 0u, 0u, 0u);
            }
        }
    };
    // Epilogue of an item, finished one item late, during the next item's
    // MFMAs: block wq of the finished item, the four quarters' partial sums
    // in quarter order (its own from registers), + bias, + residual (loaded
    // at the top of the iteration, ahead of the staging loads that share the
    // load counter), one rounding.  Piece f covers 16 output channels.
    bool have_prev = false;
    size_t prev_obase = 0;
    bool prev_st = false;
    f32x4 prev_mine[3];
    uint2 prev_res[3];
    const int pp_mine = wq * 16 + lr;
    auto epi_piece = [&](int f) __attribute__((always_inline)) {
        const int co = wc * 48 + f * 16 + lg * 4;
        float v[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const f32x4 part = q == wq ? prev_mine[f] : red[wq][q < wq ? q : q - 1][wc][f][lane];
#pragma unroll
            for (int e = 0; e < 4; ++e) v[e] += part[e];
        }
        const float4 bv4 = bias_s[co / 4];
        v[0] += bv4.x;
        v[1] += bv4.y;
        v[2] += bv4.z;
        v[3] += bv4.w;
        if (p.res) {
            v[0] += bf16_to_f32(prev_res[f].x & 0xffffu);
            v[1] += bf16_to_f32(prev_res[f].x >> 16);
            v[2] += bf16_to_f32(prev_res[f].y & 0xffffu);
            v[3] += bf16_to_f32(prev_res[f].y >> 16);
        }
        if (prev_st)
            *reinterpret_cast<uint2 *>(p.y + prev_obase + co) =
                make_uint2(pack2_bf16(v[0], v[1]), pack2_bf16(v[2], v[3]));
    };

    bool fresh = true;
    for (int i = i_begin; i < i_end; ++i) {
        // item -> (n, j, ct, oh), oh fastest
        const int oh = i % p.ho;
        int r_ = i / p.ho;
        const int ct = r_ % tiles;
        r_ /= tiles;
        const int j = r_ % p.to, n = r_ / p.to;
        const int r0 = 2 * oh - p.ph;  // first input row of this item
        const int col0 = 2 * (ct * RW_PT) - p.pw;
        if (have_prev && p.res && prev_st) {
#pragma unroll
            for (int f = 0; f < 3; ++f)
                prev_res[f] = *reinterpret_cast<const uint2 *>(p.res + prev_obase + wc * 48 + f * 16 + lg * 4);
        }
        if (fresh) {  // all three rows, in two batches of loads
            for (int pb = 0; pb < 3 * RW_SROW; pb += RW_THREADS / 2) {
                issue_pos(n, j, r0, col0, pb, 3 * RW_SROW);
                if constexpr (NORM) {
                    norm_sum();
                    static_for<H8>([&](auto k) { norm_chunk(k); });
                }
                store_pos();
            }
            __syncthreads();
        }
        // next item continues this strip: its two new rows r0+3, r0+4
        const bool next = i + 1 < i_end && oh + 1 < p.ho;
        if (next) issue_pos(n, j, r0 + 3, col0, 0, 2 * RW_SROW);

        // ---- K loop over this wave's quarter.  Each quarter is its own
        // compile-time instance, so every B-fragment address is one of three
        // per-row bases plus an immediate offset.  The previous item's
        // epilogue pieces go between its K-steps.
        const uint4 *rowb[3];
#pragma unroll
        for (int kh = 0; kh < 3; ++kh) rowb[kh] = ring + ((r0 + kh + 3) % 3) * RW_ROW + lr * RW_PITCH + lg;
        f32x4 acc[3][4];
#pragma unroll
        for (int f = 0; f < 3; ++f)
#pragma unroll
            for (int b = 0; b < 4; ++b) acc[f][b] = f32x4{0.f, 0.f, 0.f, 0.f};
        const bool epi = have_prev;
        auto kloop = [&](auto wq_tag) __attribute__((always_inline)) {
            constexpr int WQ = decltype(wq_tag)::value;
            constexpr int K0 = WQ * RW_KQ;
            constexpr int NK = WQ == 3 ? RW_KS - 3 * RW_KQ : RW_KQ;
            // entry offset of K-step ks, column block b, relative to this lane's row base
            auto off = [](int ks, int b) constexpr {
                const int tap = ks / 3, cb = ks % 3, kw = tap % 3;
                return (kw == 1 ? RW_ODD + b * 16 * RW_PITCH : (b * 16 + (kw >> 1)) * RW_PITCH) + cb * 4;
            };
            bf16x8 B[2][4];
#pragma unroll
            for (int b = 0; b < 4; ++b) B[0][b] = as_bf16x8(rowb[K0 / 9][off(K0, b)]);
            static_for<NK>([&](auto mt) {
                constexpr int m = decltype(mt)::value;
                constexpr int cur = m & 1;
                if constexpr (m + 1 < NK) {
                    constexpr int ks = K0 + m + 1;
#pragma unroll
                    for (int b = 0; b < 4; ++b) B[cur ^ 1][b] = as_bf16x8(rowb[ks / 9][off(ks, b)]);
                }
#pragma unroll
                for (int b = 0; b < 4; ++b)
#pragma unroll
                    for (int f = 0; f < 3; ++f)
                        acc[f][b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A[m][f], B[cur][b], acc[f][b], 0, 0, 0);
                if constexpr (m <= 2) {
                    if (epi) epi_piece(m);
                }
                __builtin_amdgcn_sched_barrier(0);
            });
        };
        switch (wq) {
            case 0: kloop(Int<0>{}); break;
            case 1: kloop(Int<1>{}); break;
            case 2: kloop(Int<2>{}); break;
            default: kloop(Int<3>{}); break;
        }
        // NORM: the next item's positions, normalised in registers before the
        // barrier, so that a wave done with its K-steps runs this VALU work
        // while the waves still in theirs keep the matrix pipe busy
        if constexpr (NORM) {
            if (next) {
                norm_sum();
                static_for<H8>([&](auto k) { norm_chunk(k); });
            }
        }
        __syncthreads();  // K loops and the previous epilogue done: red free, ring rows r0, r0+1 free
        // partial sums of the blocks other waves finish
#pragma unroll
        for (int b = 0; b < 4; ++b)
            if (b != wq) {
#pragma unroll
                for (int f = 0; f < 3; ++f) red[b][wq < b ? wq : wq - 1][wc][f][lane] = acc[f][b];
            }
#pragma unroll
        for (int f = 0; f < 3; ++f)  // (selects keep acc in registers)
            prev_mine[f] = wq == 0 ? acc[f][0] : wq == 1 ? acc[f][1] : wq == 2 ? acc[f][2] : acc[f][3];
        prev_obase = ((((size_t)n * p.to + j) * p.ho + oh) * (size_t)p.wo + ct * RW_PT + pp_mine) * 96;
        prev_st = pp_mine < RW_PT && ct * RW_PT + pp_mine < p.wo;
        have_prev = true;
        if (next) store_pos();
        __syncthreads();  // new rows and partial sums in
        fresh = !next;
    }
    // the last item's epilogue
    if (p.res && prev_st) {
#pragma unroll
        for (int f = 0; f < 3; ++f)
            prev_res[f] = *reinterpret_cast<const uint2 *>(p.res + prev_obase + wc * 48 + f * 16 + lg * 4);
    }
#pragma unroll
    for (int f = 0; f < 3; ++f) epi_piece(f);
}

// Standard [C_out][K] bf16 weights -> [K-step][16-row block][lane] fragments:
// lane (lr, lg) of block b at K-step ks holds row b*16 + lr, columns
// ks*32 + lg*8 .. +7.
__global__ void __launch_bounds__(256) strided_pack_kernel(const uint16_t *__restrict__ w,
                                                           uint4 *__restrict__ out, int cout, int K) {
    const int nblk = cout / 16, nb = K / 32;
    const long total = (long)nb * nblk * 64;
    for (long i = (long)blockIdx.x * 256 + threadIdx.x; i < total; i += (long)gridDim.x * 256) {
        const int lane = (int)(i % 64);
        const long rest = i / 64;
        const int b = (int)(rest % nblk), ks = (int)(rest / nblk);
        const int row = b * 16 + (lane & 15), col = ks * 32 + (lane >> 4) * 8;
        out[i] = *reinterpret_cast<const uint4 *>(w + (size_t)row * K + col);
    }
}

int k_total(const ConvCall &c) { return c.kt * c.kh * c.kw * c.cin; }

bool is_temporal(const ConvCall &c) {
    return c.kt == 3 && c.kh == 1 && c.kw == 1 && c.dt == 1 && c.st >= 2 && c.sh == 1 &&
           c.sw == 1 && c.ph == 0 && c.pw == 0 && c.eh == 0 && c.ew == 0;
}

bool is_spatial2(const ConvCall &c) {
    return c.kt == 1 && c.kh == 3 && c.kw == 3 && c.dh == 1 && c.dw == 1 && c.st == 1 &&
           c.sh == 2 && c.sw == 2 && c.ph <= 1 && c.pw <= 1 && c.eh <= 1 && c.ew <= 1;
}

// Positions per workgroup and its LDS bytes.
int run_length(const ConvCall &c) {
    if (is_temporal(c)) return 64;
    return (size_t)3 * 129 * (c.cin / 8 + 1) * 16 <= LDS_MAX ? 64 : 32;
}

size_t lds_bytes(const ConvCall &c) {
    const int pt = run_length(c);
    if (is_temporal(c)) return (size_t)pt * (k_total(c) / 8 + 1) * 16;
    return (size_t)3 * (2 * pt + 1) * (c.cin / 8 + 1) * 16;
}

// Wave layout: channel groups x 16-channel blocks per group.
struct Layout {
    int wco, fco;
};
Layout layout_for(int cout) {
    const int nblk = cout / 16;
    if (nblk % 4 == 0) return {4, nblk / 4};
    if (nblk % 2 == 0) return {2, nblk / 2};
    return {1, nblk};
}

template <int MODE, int PT, int FCO, int WCO, bool NORM>
hipError_t launch_norm(const SParams &p, long blocks, size_t lds, hipStream_t s) {
    constexpr int FPOS = PT / 16 / (4 / WCO);
    if constexpr (FPOS >= 1 && FPOS * 16 * (4 / WCO) == PT && (!NORM || MODE == 1)) {
        if constexpr (FCO == 3 && WCO == 2 && PT == 64) {
            if (p.cin == 96) {  // the 96-channel encoder level: constant index arithmetic
                hipLaunchKernelGGL((strided_kernel<MODE, PT, FCO, FPOS, WCO, 12, NORM>),
                                   dim3((unsigned)blocks), dim3(256), lds, s, p);
                return hipGetLastError();
            }
        }
        hipLaunchKernelGGL((strided_kernel<MODE, PT, FCO, FPOS, WCO, 0, NORM>), dim3((unsigned)blocks),
                           dim3(256), lds, s, p);
        return hipGetLastError();
    } else {
        return hipErrorInvalidValue;
    }
}

template <int MODE, int PT, int FCO, int WCO>
hipError_t launch_one(const SParams &p, long blocks, size_t lds, hipStream_t s) {
    if (p.gamma) return launch_norm<MODE, PT, FCO, WCO, true>(p, blocks, lds, s);
    return launch_norm<MODE, PT, FCO, WCO, false>(p, blocks, lds, s);
}

template <int MODE, int PT>
hipError_t launch_mode(const SParams &p, Layout l, long blocks, size_t lds, hipStream_t s) {
    switch (l.wco * 10 + l.fco) {
        case 41: return launch_one<MODE, PT, 1, 4>(p, blocks, lds, s);
        case 42: return launch_one<MODE, PT, 2, 4>(p, blocks, lds, s);
        case 43: return launch_one<MODE, PT, 3, 4>(p, blocks, lds, s);
        case 44: return launch_one<MODE, PT, 4, 4>(p, blocks, lds, s);
        case 21: return launch_one<MODE, PT, 1, 2>(p, blocks, lds, s);
        case 23: return launch_one<MODE, PT, 3, 2>(p, blocks, lds, s);
        case 11: return launch_one<MODE, PT, 1, 1>(p, blocks, lds, s);
        case 13: return launch_one<MODE, PT, 3, 1>(p, blocks, lds, s);
        default: return hipErrorInvalidValue;
    }
}

// The row-walking kernel: the spatial stride-2 conv at 96 -> 96 channels
// (its weights are held in registers, which fixes both channel counts).
bool rows_route(const ConvCall &c) {
    return is_spatial2(c) && c.cin == 96 && c.cout == 96 &&
           (size_t)c.h * c.w * c.cin * 2 < ((size_t)1 << 31);
}

int num_cus_strided() {
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

bool layout_instantiated(Layout l) {
    switch (l.wco * 10 + l.fco) {
        case 41: case 42: case 43: case 44: case 21: case 23: case 11: case 13: return true;
        default: return false;
    }
}

}  // namespace

bool strided_supports(const ConvCall &c) {
    if (!(is_temporal(c) || is_spatial2(c))) return false;
    if (c.cin % 32 != 0 || c.cout % 16 != 0 || c.cout > 256) return false;
    if (!layout_instantiated(layout_for(c.cout))) return false;
    if (k_total(c) / 32 > 255) return false;
    if (is_spatial2(c) && (size_t)3 * 65 * (c.cin / 8 + 1) * 16 > LDS_MAX) return false;
    // 32-position runs need at least two channel groups (16 positions per group)
    if (is_spatial2(c) && run_length(c) == 32 && layout_for(c.cout).wco == 1) return false;
    if (is_temporal(c) && lds_bytes(c) > LDS_MAX) return false;
    // 32-bit fragment offsets
    return (size_t)c.cout * k_total(c) * 2 < ((size_t)1 << 31);
}

const char *strided_kernel_name(const ConvCall &c, bool norm) {
    if (rows_route(c)) return norm ? "strided_rows_kernel<true>" : "strided_rows_kernel<false>";
    if (is_temporal(c)) return "strided_kernel<0, 64, ...> (temporal stride)";
    return norm ? "strided_kernel<1, ..., true>" : "strided_kernel<1, ..., false>";
}

size_t strided_packed_weight_bytes(const ConvCall &c) { return (size_t)c.cout * k_total(c) * 2; }

size_t strided_workspace_bytes(const ConvCall &c, bool packed_given) {
    return packed_given ? 0 : (strided_packed_weight_bytes(c) + 255) & ~(size_t)255;
}

hipError_t launch_strided_pack(const ConvCall &c, const void *w, void *packed, hipStream_t s) {
    const long chunks = (long)strided_packed_weight_bytes(c) / 16;
    long blocks = (chunks + 255) / 256;
    if (blocks > 4096) blocks = 4096;
    if (blocks < 1) return hipSuccess;
    hipLaunchKernelGGL(strided_pack_kernel, dim3((unsigned)blocks), dim3(256), 0, s,
                       static_cast<const uint16_t *>(w), static_cast<uint4 *>(packed), c.cout, k_total(c));
    return hipGetLastError();
}

hipError_t launch_conv_strided(const ConvCall &c, ConvRoute r, bool packed_given, void *ws,
                               size_t ws_bytes, hipStream_t s) {
    if (!strided_supports(c)) return hipErrorInvalidValue;
    const void *wp = c.weight;
    if (!packed_given) {
        if (ws_bytes < strided_workspace_bytes(c, false) || !ws) return hipErrorInvalidValue;
        const hipError_t e = launch_strided_pack(c, c.weight, ws, s);
        if (e != hipSuccess) return e;
        wp = ws;
    }
    const bool temporal = r == ConvRoute::FastTemporal;
    if (temporal != is_temporal(c)) return hipErrorInvalidValue;
    SParams p{};
    p.x = static_cast<const uint16_t *>(c.x);
    p.cache = static_cast<const uint16_t *>(c.cache_in);
    p.wp = static_cast<const uint16_t *>(wp);
    p.bias = static_cast<const uint16_t *>(c.bias);
    p.res = static_cast<const uint16_t *>(c.residual);
    p.y = static_cast<uint16_t *>(c.y);
    if (c.norm_gamma) {
        if (temporal) return hipErrorInvalidValue;  // the fused norm is on the spatial route
        p.gamma = static_cast<const uint16_t *>(c.norm_gamma);
        p.beta = static_cast<const uint16_t *>(c.norm_beta);
        p.eps = c.norm_eps;
        p.norm_scale = sqrtf((float)c.cin);
    }
    p.n = c.n; p.t = c.t; p.h = c.h; p.w = c.w; p.ho = c.ho; p.wo = c.wo;
    p.cin = c.cin; p.cout = c.cout;
    p.F = c.frames; p.st = c.st; p.t0 = c.t0; p.to = c.to;
    p.ph = c.ph; p.pw = c.pw;
    p.nb = k_total(c) / 32;
    p.w_bytes = (uint32_t)strided_packed_weight_bytes(c);
    const int pt = run_length(c);
    p.pitch = temporal ? k_total(c) / 8 + 1 : c.cin / 8 + 1;
    p.tiles = temporal ? (c.ho * c.wo + pt - 1) / pt : (c.wo + pt - 1) / pt;
    const long blocks = temporal ? (long)c.n * c.to * p.tiles : (long)c.n * c.to * c.ho * p.tiles;
    if (blocks <= 0) return hipSuccess;
    if (blocks > 0x7fffffffL) return hipErrorInvalidValue;
    if (rows_route(c)) {
        // one persistent workgroup per CU over the output rows of 63-column strips
        p.tiles = (c.wo + RW_PT - 1) / RW_PT;
        const long items = (long)c.n * c.to * p.tiles * c.ho;
        if (items > 0x7fffffffL) return hipErrorInvalidValue;
        const unsigned grid = (unsigned)(items < num_cus_strided() ? items : num_cus_strided());
        if (p.gamma)
            hipLaunchKernelGGL(strided_rows_kernel<true>, dim3(grid), dim3(RW_THREADS), 0, s, p, (int)items);
        else
            hipLaunchKernelGGL(strided_rows_kernel<false>, dim3(grid), dim3(RW_THREADS), 0, s, p, (int)items);
        return hipGetLastError();
    }
    const size_t lds = lds_bytes(c);
    const Layout l = layout_for(c.cout);
    if (temporal) return launch_mode<0, 64>(p, l, blocks, lds, s);
    return pt == 64 ? launch_mode<1, 64>(p, l, blocks, lds, s) : launch_mode<1, 32>(p, l, blocks, lds, s);
}

}  // namespace wvc
