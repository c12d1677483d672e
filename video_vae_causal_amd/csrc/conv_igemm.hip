// conv_igemm.hip -- causal 3x3x3 (and 1x1x1) convolution as an implicit GEMM
// on CDNA4 bf16 MFMA with fp32 accumulation.
//
// What it computes ("Cosmos3 Wan VAE -- engine size vs runtime context
// memory", section 10.3): y[n,t,h,w,co] = b[co] + sum over ci, kt, kh, kw of
// W[co,kt,kh,kw,ci] * X'[n, t-2+kt, h-1+kh, w-1+kw, ci], where X' is the chunk
// with the two cached past frames in front (frames t-2+kt < 0 come from the
// cache, or are zero when there is none) and zero spatial padding.  The bias
// is added once, after the whole sum ("cache-aware video decoder lowering").
//
// GEMM view (same page, Conv3D as GEMM): rows = output channels (MFMA A
// operand = weights, K contiguous in the channels-last weight layout),
// columns = output positions (MFMA B operand = input patches), K = 27 taps x
// C_in.  Nothing is materialised: the patch matrix is read straight out of a
// spatial halo tile held in LDS.
//
// Work decomposition
//   workgroup : 256 threads (4 waves), CO_T output channels x POS_T output
//               positions of one output frame; positions form a TH x TW
//               spatial tile chosen by the host (TH*TW == POS_T).
//   K loop    : over 32-channel blocks of C_in.  Per block the halo of the
//               three input frames t-2, t-1, t (cache or chunk) is staged in
//               LDS as [frame][k-group(4)][(TH+2)(TW+2)][8 channels], 16 B per
//               entry, so the 16 lanes of one k-group read 16 neighbouring
//               positions as one contiguous run.  The 27 taps then read their
//               B fragments from the same tile at a shifted offset: the
//               temporal taps are accumulated in registers, never as
//               per-slice batches.
//   waves     : 2 (channels) x 2 (positions); a wave owns CO_T/2 x POS_T/2
//               outputs as 16x16 MFMA tiles (v_mfma_f32_16x16x32_bf16).
//   epilogue  : + bias, + residual (fused block shortcut), one rounding to
//               bf16, 8-byte stores of 4 consecutive channels.
//   mapping   : workgroup ids are remapped so each XCD (own L2) receives a
//               contiguous run of tiles: the channel tiles of one spatial tile
//               and its neighbours share the halo in that XCD's L2.
#include "wvc_internal.h"
#include "wvc.h"

namespace wvc {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

struct IgParams {
    const uint16_t *x;
    const uint16_t *cache;
    const uint16_t *w;
    const uint16_t *bias;
    const uint16_t *res;
    uint16_t *y;
    int T, H, W, Cin, Cout, F;
    int TH, TW, HC, HP;
    int tiles_w, tiles_h, co_tiles;
    int total;
};

__device__ __forceinline__ int xcd_remap(int bid, int total) {
    // Consecutive workgroup ids are dispatched round-robin over the 8 XCDs;
    // hand XCD k the k-th contiguous slice of the logical tile order instead.
    const int xcd = bid & 7;
    const int local = bid >> 3;
    const int per = total >> 3, rem = total & 7;
    const int start = xcd < rem ? xcd * (per + 1) : rem * (per + 1) + (xcd - rem) * per;
    return start + local;
}

__device__ __forceinline__ bf16x8 as_bf16x8(uint4 v) { return __builtin_bit_cast(bf16x8, v); }

template <int KS, int CO_T, int POS_T, int HP_MAX>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2))) igemm_kernel(IgParams p) {
    constexpr int KT = KS;
    constexpr int TAPS = KS * KS * KS;
    constexpr int PAD = KS / 2;
    constexpr int WCO = CO_T / 2, WPOS = POS_T / 2;
    constexpr int FCO = WCO / 16, FPOS = WPOS / 16;
    static_assert(WCO % 16 == 0 && WPOS % 16 == 0, "wave tile must be whole 16x16 MFMA tiles");

    __shared__ uint4 halo[KT * 4 * HP_MAX];

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int wco = wave & 1, wpos = wave >> 1;
    const int kg = lane >> 4, l16 = lane & 15;

    int L = xcd_remap(blockIdx.x, p.total);
    const int co_tile = L % p.co_tiles;
    L /= p.co_tiles;
    const int tw = L % p.tiles_w;
    L /= p.tiles_w;
    const int th = L % p.tiles_h;
    L /= p.tiles_h;
    const int t = L % p.T;
    const int n = L / p.T;
    const int h0 = th * p.TH, w0 = tw * p.TW;
    const int co0 = co_tile * CO_T + wco * WCO;

    // LDS entry (in 16-byte units) of this lane's B-fragment positions at tap (0,0,0).
    int boff[FPOS];
#pragma unroll
    for (int f = 0; f < FPOS; ++f) {
        const int q = wpos * WPOS + f * 16 + l16;
        const int r = q / p.TW, c = q - r * p.TW;
        boff[f] = kg * p.HP + r * p.HC + c;
    }
    // This lane's weight rows (A fragments): channel co, k-group kg.
    const uint16_t *wrow[FCO];
    bool wok[FCO];
#pragma unroll
    for (int f = 0; f < FCO; ++f) {
        const int co = co0 + f * 16 + l16;
        wok[f] = co < p.Cout;
        wrow[f] = p.w + (size_t)(wok[f] ? co : 0) * TAPS * p.Cin + kg * 8;
    }

    f32x4 acc[FCO][FPOS];
#pragma unroll
    for (int i = 0; i < FCO; ++i)
#pragma unroll
        for (int j = 0; j < FPOS; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    const size_t row_elems = (size_t)p.W * p.Cin;
    const size_t frame_elems = (size_t)p.H * row_elems;
    const int items = KT * p.HP * 4;

    for (int cb = 0; cb < p.Cin; cb += 32) {
        __syncthreads();  // every wave is done reading the previous block
        for (int it = tid; it < items; it += 256) {
            const int g = it & 3;
            const int pi = it >> 2;
            const int fr = pi / p.HP;
            const int hp = pi - fr * p.HP;
            const int r = hp / p.HC;
            const int c = hp - r * p.HC;
            const int hs = h0 + r - PAD, ws = w0 + c - PAD;
            const int ts = t - (KT - 1) + fr;
            const int ci = cb + g * 8;
            uint4 v = make_uint4(0u, 0u, 0u, 0u);
            if (hs >= 0 && hs < p.H && ws >= 0 && ws < p.W && ci < p.Cin) {
                const uint16_t *src = nullptr;
                const size_t off = (size_t)hs * row_elems + (size_t)ws * p.Cin + ci;
                if (ts >= 0)
                    src = p.x + (size_t)(n * p.T + ts) * frame_elems + off;
                else if (p.cache)
                    src = p.cache + (size_t)(n * p.F + p.F + ts) * frame_elems + off;
                if (src) v = *reinterpret_cast<const uint4 *>(src);
            }
            halo[(fr * 4 + g) * p.HP + hp] = v;
        }
        __syncthreads();

        const bool kok = (cb + kg * 8) < p.Cin;
        // Weights (A fragments) come from global memory and are prefetched one
        // tap ahead; input patches (B fragments) are read from the LDS tile.
        bf16x8 a_cur[FCO], a_nxt[FCO];
#pragma unroll
        for (int f = 0; f < FCO; ++f) {
            uint4 v = make_uint4(0u, 0u, 0u, 0u);
            if (wok[f] && kok) v = *reinterpret_cast<const uint4 *>(wrow[f] + cb);
            a_cur[f] = as_bf16x8(v);
        }
#pragma unroll 1
        for (int tap = 0; tap < TAPS; ++tap) {
            const int tn = tap + 1 < TAPS ? tap + 1 : tap;
#pragma unroll
            for (int f = 0; f < FCO; ++f) {
                uint4 v = make_uint4(0u, 0u, 0u, 0u);
                if (wok[f] && kok)
                    v = *reinterpret_cast<const uint4 *>(wrow[f] + (size_t)tn * p.Cin + cb);
                a_nxt[f] = as_bf16x8(v);
            }
            const int kt = tap / (KS * KS), kh = (tap / KS) % KS, kw = tap % KS;
            const int toff = kt * 4 * p.HP + kh * p.HC + kw;
            bf16x8 b[FPOS];
#pragma unroll
            for (int f = 0; f < FPOS; ++f) b[f] = as_bf16x8(halo[boff[f] + toff]);
#pragma unroll
            for (int i = 0; i < FCO; ++i)
#pragma unroll
                for (int j = 0; j < FPOS; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a_cur[i], b[j], acc[i][j], 0, 0, 0);
#pragma unroll
            for (int f = 0; f < FCO; ++f) a_cur[f] = a_nxt[f];
        }
    }

    // Epilogue.  Lane holds D[co = 4*kg + e][pos = l16] of each 16x16 tile.
#pragma unroll
    for (int j = 0; j < FPOS; ++j) {
        const int q = wpos * WPOS + j * 16 + l16;
        const int r = q / p.TW, c = q - r * p.TW;
        const int h = h0 + r, w = w0 + c;
        if (h >= p.H || w >= p.W) continue;
        const size_t obase = (((size_t)(n * p.T + t) * p.H + h) * p.W + w) * p.Cout;
#pragma unroll
        for (int i = 0; i < FCO; ++i) {
            const int co = co0 + i * 16 + kg * 4;
            if (co >= p.Cout) continue;
            float v[4] = {acc[i][j][0], acc[i][j][1], acc[i][j][2], acc[i][j][3]};
            if (p.bias) {
                const uint2 bb = *reinterpret_cast<const uint2 *>(p.bias + co);
                v[0] += bf16_to_f32(bb.x & 0xffffu);
                v[1] += bf16_to_f32(bb.x >> 16);
                v[2] += bf16_to_f32(bb.y & 0xffffu);
                v[3] += bf16_to_f32(bb.y >> 16);
            }
            if (p.res) {
                const uint2 rr = *reinterpret_cast<const uint2 *>(p.res + obase + co);
                v[0] += bf16_to_f32(rr.x & 0xffffu);
                v[1] += bf16_to_f32(rr.x >> 16);
                v[2] += bf16_to_f32(rr.y & 0xffffu);
                v[3] += bf16_to_f32(rr.y >> 16);
            }
            uint2 o;
            o.x = (uint32_t)f32_to_bf16(v[0]) | ((uint32_t)f32_to_bf16(v[1]) << 16);
            o.y = (uint32_t)f32_to_bf16(v[2]) | ((uint32_t)f32_to_bf16(v[3]) << 16);
            *reinterpret_cast<uint2 *>(p.y + obase + co) = o;
        }
    }
}

struct TileChoice {
    int th, tw;
};

// Pick a TH x TW tile (TH*TW == pos_t) that wastes the fewest positions on
// ragged edges; ties go to the wider tile (longer contiguous runs).
TileChoice choose_tile(int h, int w, int pos_t, int ks, int hp_max) {
    TileChoice best{0, 0};
    long best_cost = -1;
    for (int tw = 1; tw <= pos_t; tw *= 2) {
        const int th = pos_t / tw;
        if ((th + ks - 1) * (tw + ks - 1) > hp_max) continue;
        const long tiles = (long)((h + th - 1) / th) * ((w + tw - 1) / tw);
        const long cost = tiles * pos_t;
        if (best_cost < 0 || cost < best_cost || (cost == best_cost && tw > best.tw)) {
            best_cost = cost;
            best = {th, tw};
        }
    }
    return best;
}

template <int KS, int CO_T, int POS_T, int HP_MAX>
hipError_t launch_variant(const ConvCall &c, hipStream_t s) {
    IgParams p;
    p.x = static_cast<const uint16_t *>(c.x);
    p.cache = static_cast<const uint16_t *>(c.cache_in);
    p.w = static_cast<const uint16_t *>(c.weight);
    p.bias = static_cast<const uint16_t *>(c.bias);
    p.res = static_cast<const uint16_t *>(c.residual);
    p.y = static_cast<uint16_t *>(c.y);
    p.T = c.t;
    p.H = c.h;
    p.W = c.w;
    p.Cin = c.cin;
    p.Cout = c.cout;
    p.F = c.frames;
    const TileChoice tc = choose_tile(c.h, c.w, POS_T, KS, HP_MAX);
    if (tc.th == 0) return hipErrorInvalidValue;
    p.TH = tc.th;
    p.TW = tc.tw;
    p.HC = tc.tw + KS - 1;
    p.HP = (tc.th + KS - 1) * p.HC;
    p.tiles_w = (c.w + tc.tw - 1) / tc.tw;
    p.tiles_h = (c.h + tc.th - 1) / tc.th;
    p.co_tiles = (c.cout + CO_T - 1) / CO_T;
    const long total = (long)c.n * c.t * p.tiles_h * p.tiles_w * p.co_tiles;
    if (total <= 0) return hipSuccess;
    if (total > 0x7fffffffL) return hipErrorInvalidValue;
    p.total = (int)total;
    hipLaunchKernelGGL((igemm_kernel<KS, CO_T, POS_T, HP_MAX>), dim3(p.total), dim3(256), 0, s, p);
    return hipGetLastError();
}

}  // namespace

size_t igemm_workspace_bytes(const ConvCall &, ConvRoute) { return 0; }

hipError_t launch_conv_igemm(const ConvCall &c, ConvRoute r, void *, size_t, hipStream_t s) {
    if (r == ConvRoute::Fast3x3x3) {
        if (c.cout % 128 == 0) return launch_variant<3, 128, 256, 340>(c, s);
        if (c.cout % 96 == 0) return launch_variant<3, 96, 256, 340>(c, s);
        return launch_variant<3, 64, 256, 340>(c, s);
    }
    if (c.cout % 128 == 0) return launch_variant<1, 128, 256, 256>(c, s);
    if (c.cout % 96 == 0) return launch_variant<1, 96, 256, 256>(c, s);
    return launch_variant<1, 64, 256, 256>(c, s);
}

}  // namespace wvc
