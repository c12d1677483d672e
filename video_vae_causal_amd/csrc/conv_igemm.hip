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
// C_in.  Nothing is materialised: the patch matrix is read out of a spatial
// halo tile held in LDS.
//
// Work decomposition
//   workgroup : 256 threads (4 waves), one per CU (up to 512 registers per
//               lane), CO_T output channels x 256 output positions of one
//               output frame; the positions form a TH x TW spatial tile chosen
//               by the host (TH*TW == 256).  Whole-K grids of 16x16 bf16
//               tiles (96 and 64 channels) run two workgroups per CU instead
//               (igemm_occ2_kernel, 256 registers per lane): the weights are
//               prefetched one row ahead instead of two and the B fragments
//               pass through a 3-slot ring, and each workgroup's barrier and
//               epilogue stalls are covered by the other's MFMAs.
//   K loop    : over work units (kt, 32-channel block).  A unit stages the
//               halo of ONE input frame (t-2+kt: cache or chunk) for 32 input
//               channels in LDS as [k-group(4)][(TH+2)(TW+2)][8 channels]
//               (16 B entries, so the lanes of one k-group read neighbouring
//               positions as one contiguous run), then runs its 9 spatial
//               taps, each reading its B fragments from the same tile at a
//               shifted offset.  The three temporal taps accumulate into the
//               same registers: no per-slice batches exist.
//   waves     : 2 (channels) x 2 (positions); a wave owns CO_T/2 x 128 outputs
//               as M x M MFMA tiles (32x32x16 for 128 channels, 16x16x32 for
//               96 and 64).  The pipeline is described at the kernel.
//   loads     : buffer loads with the frame as the buffer range: positions
//               outside the frame and channels past C_in read as zero in
//               hardware, so staging has no branches.
//   split-K   : small grids (one 60x104 or 30x52 frame) split the units of a
//               tile over S workgroups.  Each writes its fp32 partial sums in
//               the output layout to the workspace (plain stores, no
//               inter-workgroup synchronisation), and a second kernel adds the
//               S partials in split order (deterministic), then bias and
//               residual, and rounds once.
//   epilogue  : + bias, + residual (fused block shortcut), one rounding to
//               bf16, 8-byte stores of 4 consecutive channels.  Bias and
//               residual are loaded before the first store.
//   cache     : the workgroups of the chunk's last output frame also write
//               the interior of the halos they stage for frames T-2 and T-1 to
//               cache_out (the channel tiles share out the channel blocks):
//               the rolling cache update costs no extra pass over the frames.
//   mapping   : workgroup ids are remapped so each XCD (own L2) receives a
//               contiguous run of tiles: splits and channel tiles of one
//               spatial tile, then (large grids) its other output frames,
//               then its neighbours, share that XCD's L2.
//
// 8-bit variant (FP8): activations, cache and weights are OCP E4M3 codes (the
// quantised Conv3D of "Cosmos3 Wan VAE", sections 7 and 9, in the format
// gfx950's matrix cores read).  A work unit is then 64 input channels: its
// halo slice is the same 64 bytes per position as a 32-channel bf16 unit, so
// staging, LDS layout and weight fragments are unchanged byte for byte, and
// the two 16-byte fragments a lane holds for the two bf16 K-steps form the
// 32-byte operand of one v_mfma_f32_32x32x64_f8f6f4 (64 channels per MFMA,
// twice the bf16 rate).  The sum is exact products accumulated in fp32; the
// epilogue (or the split-K reduce) multiplies it by x_scale * w_scale[co]
// before the bias.
#include <cstdio>
#include <type_traits>

#include "wvc_internal.h"
#include "wvc.h"

namespace wvc {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));

constexpr int POS_T = 256;
constexpr uint32_t OOB = 0x80000000u;  // an offset past every buffer range used here
constexpr int RSRC_WORD3 = 0x00020000;  // raw buffer, range-checked (CDNA data format)

struct IgParams {
    const void *x;      // bf16 or E4M3 codes
    const void *cache;  // same type as x
    const uint16_t *w;
    const uint16_t *bias;
    const uint16_t *res;
    uint16_t *y;
    void *cache_out;    // same type as x
    const float *wscale;  // E4M3: per-output-channel weight scale [Cout]
    float xscale;         // E4M3: activation scale
    float *part;  // split-K partial sums: [S][N][T][H][W][Cout] fp32
    size_t part_stride;  // N*T*H*W*Cout: elements of one split's partials
    int T, H, W, Cin, Cout, F;
    int tiles_w, tiles_h, co_tiles;
    int S, U;
    int total;
    int co_major;  // channel tile slowest in the workgroup order (small grids)
    int up;        // 1, or 2: x and the caches hold H/2 x W/2 frames read through a
                   // nearest 2x upsample (frame_bytes is then theirs)
    uint32_t frame_bytes, w_bytes;
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

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void *base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes,
                                             RSRC_WORD3);
}

__device__ __forceinline__ uint4 bload(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0);
    return make_uint4(v.x, v.y, v.z, v.w);
}

__device__ __forceinline__ uint4 bload_s(__amdgpu_buffer_rsrc_t r, uint32_t off, uint32_t soff) {
    const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, (int)soff, 0);
    return make_uint4(v.x, v.y, v.z, v.w);
}

__device__ __forceinline__ bf16x8 as_bf16x8(uint4 v) { return __builtin_bit_cast(bf16x8, v); }

typedef float f32x16 __attribute__((ext_vector_type(16)));

// MFMA shapes used here: M x M output tiles, 512/M deep in K.
template <int M>
struct Mfma;
template <>
struct Mfma<16> {
    typedef f32x4 acc_t;
    static constexpr int ACC = 4;
    __device__ static acc_t run(bf16x8 a, bf16x8 b, acc_t c) {
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
    }
};
template <>
struct Mfma<32> {
    typedef f32x16 acc_t;
    static constexpr int ACC = 16;
    __device__ static acc_t run(bf16x8 a, bf16x8 b, acc_t c) {
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
    }
};

// 32x32x64 MFMA of E4M3 operands (format 0 for A and B, no block scales):
// lane l holds 32 codes of A row / B column l % 32.
__device__ __forceinline__ f32x16 mfma_e4m3(i32x8 a, i32x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

template <int N>
using Int = std::integral_constant<int, N>;

// Compile-time loop: f(Int<0>{}), ..., f(Int<N-1>{}).
template <int N, int I = 0, typename F>
__device__ __forceinline__ void static_for(F &&f) {
    if constexpr (I < N) {
        f(Int<I>{});
        static_for<N, I + 1>(f);
    }
}

// Compile-time geometry of a TH x TW position tile (TH * TW == 256) and its
// halo: HC columns, HP entries per 8-channel group; each group gets NIT*64
// slots (every staging thread writes all of its slots unconditionally), plus
// GAP entries.
//
// LDS banks: gfx950's LDS has 64 four-byte banks, so a 16-byte entry e sits on
// the bank quad e % 16, and a ds_read_b128 / ds_write_b128 is served in cycles
// of 16 lanes whose lane numbers are distinct mod 16.  An access is therefore
// conflict-free whenever every lane's entry is congruent to its lane number
// mod 16, up to one offset shared by the wave (measured: a layout breaking
// this runs at about half the rate).
//   * 32x32 tiles: a B fragment's 64 lanes are two 32-lane halves, one per
//     k-group, which never share a cycle, so the group gap only matters to the
//     staging stores.  These keep the 4 groups of one position on 4
//     neighbouring lanes (one contiguous 64-byte global load per lane quad),
//     and with the groups 2 entries past a multiple of 16 apart (GAP = 2)
//     their stores are conflict-free as well (measured: gaps of 4 mod 16 and
//     of 0 mod 8 conflict).
//   * 16x16 tiles: the 4 k-groups sit on lanes 16 apart, so the groups must
//     start a multiple of 16 entries apart (GAP = 0), and the staging threads
//     are laid out so that their stores keep the congruence too.
template <int KS, int TW, bool CONG>
struct Geo {
    static constexpr int TH = POS_T / TW;
    static constexpr int HC = TW + KS - 1;
    static constexpr int HP = (TH + KS - 1) * HC;
    static constexpr int NIT = (HP + 63) / 64;  // staging slots per thread
    static constexpr int HPAD = NIT * 64 + (CONG ? 0 : 2);
};

// Row offset (dr) and column (c), inside its MFMA column tile, of the output
// position held by B column n.  Row-major order except for 32-column tiles of
// a 16-wide tile: their second tile row starts HC entries after the first, so
// its columns are rotated by HC mod 16 to put column n on entry == n (mod 16).
// Tiles 8 wide keep row-major order: no rotation can reach the congruence
// there, and the host charges them for it.
template <int M, int TW, int HC>
__device__ __forceinline__ void bcol(int n, int &dr, int &c) {
    if constexpr (M == 32 && TW == 16) {
        dr = n >> 4;
        c = dr ? ((n - 16 - HC) & 15) : n;
    } else {
        dr = n / TW;
        c = n % TW;
    }
}

// One workgroup = 256 threads = 4 waves laid out WAVES_CO (channels) x
// 4/WAVES_CO (positions).  M is the MFMA tile edge (16: 16x16x32, 32: 32x32x16);
// TW the tile width, a template parameter so that every LDS and weight
// address inside the K loop is a per-lane base plus an immediate offset.
//
// Pipeline (one workgroup per CU, up to 512 registers per lane):
//   * a stage is one work unit (kt, 32-channel block); its halo tile lives in
//     one half of a double-buffered LDS array.  The next stage's halo is loaded
//     into registers while the current stage computes and is written to the
//     other half at the end of the stage, followed by one barrier.
//   * a row is one kernel row kh of a stage: KS taps.  The weights (A
//     fragments) of a row are fetched two rows ahead into one of three
//     register sets (row r uses set r % 3), one load per MFMA group.
//   * the input patches (B fragments) of tap k+1 are read from LDS right after
//     the last MFMA of tap k that used the same registers.
//   Global loads complete in issue order: the weights a row uses were issued
//   during the row two rows back, and the halo written at the end of a stage
//   during that stage's first row, so every wait covers loads at least a row
//   old.
template <int KS, int CO_T, int M, int WAVES_CO, bool SPLIT, int TW, bool FP8, bool OCC2 = false>
__device__ __forceinline__ void igemm_body(const IgParams &p) {
    static_assert(!OCC2 || (KS == 3 && M == 16 && !FP8), "two waves per SIMD: 16x16 bf16 tiles");
    // Weight row sets: rows are prefetched NSETS - 1 rows ahead.  Two waves
    // per SIMD (OCC2) keep two sets; the other wave covers the shorter lead.
    constexpr int NSETS = OCC2 ? 2 : 3;
    static_assert(!FP8 || M == 32, "the 8-bit path uses 32x32x64 MFMAs");
    using MF = Mfma<M>;
    // 16x16 tiles take the bank-congruent group pitch and staging map
    constexpr bool CONG = M == 16;
    using G = Geo<KS, TW, CONG>;
    using acc_t = typename MF::acc_t;
    constexpr int ACC = MF::ACC;
    constexpr int PAD = KS / 2;
    constexpr int NIT = G::NIT, HPAD = G::HPAD, HC = G::HC, HP = G::HP;
    constexpr int WAVES_POS = 4 / WAVES_CO;
    constexpr int WCO = CO_T / WAVES_CO, WPOS = POS_T / WAVES_POS;
    constexpr int FCO = WCO / M, FPOS = WPOS / M;
    constexpr int NBLK = CO_T / M;  // M-row weight blocks per channel tile
    constexpr int KSTEPS = M / 16;  // MFMA K-steps per 32-channel block
    constexpr int GPL = 64 / M;     // 8-channel groups spanned by one K-step
    constexpr int FRAG = 1024;      // bytes of one packed A fragment
    constexpr int ESZ = FP8 ? 1 : 2;       // bytes per activation element
    constexpr int CPE = 16 / ESZ;          // channels per 16-byte LDS entry
    constexpr int CB = 4 * CPE;            // channels per work unit
    constexpr int KA = FP8 ? 1 : KSTEPS;   // MFMAs per (tap, block, column tile)
    using frag_t = std::conditional_t<FP8, i32x8, bf16x8>;
    static_assert(WCO % M == 0 && WPOS % M == 0, "wave tile must be whole MFMA tiles");
    static_assert(TW % M == 0 || M % TW == 0, "MFMA columns must tile the tile rows");
    static_assert(WPOS % TW == 0, "a wave's positions must start on a tile row");
    static_assert(NIT <= 32, "staging mask");
    static_assert((FCO * KSTEPS - 1) * FRAG < 4096, "weight offsets must fit the immediate");

    __shared__ uint4 halo[2][4 * HPAD];
    __shared__ uint2 bias_s[CO_T / 4];  // this channel tile's bias, read by the epilogue
    __shared__ float4 scale_s[FP8 ? CO_T / 4 : 1];  // x_scale * w_scale[co] (8-bit path)

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int wco = wave % WAVES_CO, wpos = wave / WAVES_CO;
    const int lr = lane % M;  // A row / B column of this lane inside an MFMA tile
    const int lg = lane / M;  // 8-channel group of this lane inside a K-step
    // staging: 8-channel group g and halo position (mod 64) sp of this
    // thread.  Either map has each wave cover 16 positions x all 4 groups (64
    // contiguous bytes per position).  The congruent map puts lane l on entry
    // g*HPAD + sp == l (mod 16); the other keeps a position's 4 groups on 4
    // neighbouring lanes, which halves the 384-channel conv's L2 misses.
    const int g = CONG ? (tid >> 4) & 3 : tid & 3;
    const int sp = CONG ? (tid & 15) + 16 * (tid >> 6) : tid >> 2;

    int L = xcd_remap(blockIdx.x, p.total);
    const int s = SPLIT ? L % p.S : 0;
    if (SPLIT) L /= p.S;
    // Order of the logical tiles.  Small grids: channel tile slowest (each XCD
    // then works on one channel tile, so its weight slice stays in L2), then
    // column, row, frame.  Large grids: channel tile fastest, then frame, then
    // column and row: the tiles an XCD runs at one time are the channel tiles
    // of one spatial block over consecutive output frames, which read the
    // same input-frame halos (each input frame feeds three output frames), so
    // those halos are fetched once into that XCD's L2.
    auto decode = [&](int l, int &ct_, int &t_, int &n_, int &h0_, int &w0_) {
        int tw_, th_;
        if (p.co_major) {
            const int per_ct = (int)(p.total / p.S) / p.co_tiles;
            ct_ = l / per_ct;
            l -= ct_ * per_ct;
            tw_ = l % p.tiles_w;
            l /= p.tiles_w;
            th_ = l % p.tiles_h;
            l /= p.tiles_h;
            t_ = l % p.T;
            n_ = l / p.T;
        } else {
            ct_ = l % p.co_tiles;
            l /= p.co_tiles;
            t_ = l % p.T;
            l /= p.T;
            tw_ = l % p.tiles_w;
            l /= p.tiles_w;
            th_ = l % p.tiles_h;
            n_ = l / p.tiles_h;
        }
        h0_ = th_ * G::TH;
        w0_ = tw_ * TW;
    };
    int ct, t, n, h0, w0;
    decode(L, ct, t, n, h0, w0);
    int co0 = ct * CO_T + wco * WCO;
    const int u0 = SPLIT ? (s * p.U) / p.S : 0;
    const int u1 = SPLIT ? ((s + 1) * p.U) / p.S : p.U;
    auto load_bias = [&](int ct_) {
        if (!SPLIT && tid < CO_T / 4) {
            bias_s[tid] = p.bias ? *reinterpret_cast<const uint2 *>(p.bias + ct_ * CO_T + tid * 4)
                                 : make_uint2(0u, 0u);
            if constexpr (FP8) {
                const float4 ws = *reinterpret_cast<const float4 *>(p.wscale + ct_ * CO_T + tid * 4);
                scale_s[tid] = make_float4(p.xscale * ws.x, p.xscale * ws.y, p.xscale * ws.z,
                                           p.xscale * ws.w);
            }
        }
    };
    load_bias(ct);

    // Staging: slot k of this thread is halo position sp + 64k of group g,
    // LDS entry lbase + 64k (slots past HP are padding).
    uint32_t soff[NIT];  // byte offset of the 16-byte chunk inside a frame, or OOB
    uint32_t interior = 0;
    const int lbase = g * HPAD + sp;
    auto stage_offsets = [&](int h0_, int w0_, uint32_t (&so)[NIT], uint32_t &inner) {
        inner = 0;
#pragma unroll
        for (int k = 0; k < NIT; ++k) {
            const int hp = sp + 64 * k;
            const int r = hp / HC, c = hp - r * HC;
            const int hs = h0_ + r - PAD, ws = w0_ + c - PAD;
            const bool inframe = hp < HP && hs >= 0 && hs < p.H && ws >= 0 && ws < p.W;
            // upsampled input: position (hs, ws) of the conv's frame is pixel
            // (hs/2, ws/2) of the stored one (hs, ws >= 0 when in frame)
            const int ush = p.up >> 1;
            const int sh = hs >> ush, sw = ws >> ush, srow = p.W >> ush;
            so[k] = inframe ? (uint32_t)((sh * srow + sw) * p.Cin * ESZ + g * 16) : OOB;
            if (inframe && r >= PAD && r < PAD + G::TH && c >= PAD && c < PAD + TW) inner |= 1u << k;
        }
    };
    stage_offsets(h0, w0, soff, interior);
    // B fragments: LDS entry of this lane's position (first MFMA column tile,
    // spatial tap (0,0), K-step 0).  Column tile j, K-step ks and tap (kh, kw)
    // add compile-time offsets.
    int bdr, bc;  // this lane's B column: row offset and column in its tile
    bcol<M, TW, HC>(lr, bdr, bc);
    const int bbase = lg * HPAD + ((wpos * WPOS) / TW + bdr) * HC + bc;
    // Weights: packed as [co tile][unit][kh][kw][M-row block][K-step][lane],
    // one 1 KiB fragment per (block, K-step); this wave's blocks start at
    // wco * FCO.  A row (unit, kh) is one contiguous run of KS fragment groups.
    const uint32_t wlane = (uint32_t)((wco * FCO * KSTEPS) * FRAG + lane * 16);
    const __amdgpu_buffer_rsrc_t wr = rsrc(p.w, p.w_bytes);
    const char *xb = static_cast<const char *>(p.x);
    const char *cb_base = static_cast<const char *>(p.cache);
    // Cache update: the workgroups of the chunk's last output frame write the
    // halo interiors they stage for frames T-2 and T-1, each channel tile the
    // 32-channel blocks cb with cb % co_tiles == its tile (balanced work).
    bool write_cache = KS == 3 && p.cache_out != nullptr && t == p.T - 1;

    acc_t acc[FCO][FPOS];
#pragma unroll
    for (int i = 0; i < FCO; ++i)
#pragma unroll
        for (int j = 0; j < FPOS; ++j)
#pragma unroll
            for (int e = 0; e < ACC; ++e) acc[i][j][e] = 0.f;

    // bf16: one fragment per K-step.  8-bit: one 32-byte operand whose halves
    // are the 16-byte fragments of K-steps 0 and 1.
    frag_t A[NSETS][KS][FCO][KA];  // row sets: [set][kw][co tile][K-step]
    frag_t B[OCC2 ? 1 : 2][FPOS][KA];  // two tap sets: tap k reads B[k & 1]
    // OCC2: the B fragment of column step q = tap * FPOS + j lives in ring
    // slot q % 3 and is read two column steps ahead (12 registers instead of
    // 2 * FPOS * 4), which fits a wave in the 256 registers of two waves per SIMD.
    frag_t Bq[3];
    uint4 hv[NIT];
    auto put = [](frag_t &dst, int ks, uint4 v) {
        if constexpr (FP8) {
            if (ks == 0)
                dst.lo = __builtin_bit_cast(i32x4, v);
            else
                dst.hi = __builtin_bit_cast(i32x4, v);
        } else {
            dst = as_bf16x8(v);
        }
    };

    auto load_row = [&](auto set_tag, int rho, int ct_) {
        constexpr int SET = decltype(set_tag)::value;
        const int u = u0 + rho / KS, kh = rho % KS;
        const uint32_t row = (uint32_t)((((ct_ * p.U + u) * KS + kh) * KS) * NBLK * KSTEPS) * FRAG;
#pragma unroll
        for (int kw = 0; kw < KS; ++kw)
#pragma unroll
            for (int f = 0; f < FCO; ++f)
#pragma unroll
                for (int ks = 0; ks < KSTEPS; ++ks)
                    put(A[SET][kw][f][FP8 ? 0 : ks], ks,
                        bload_s(wr, wlane + (f * KSTEPS + ks) * FRAG, row + kw * NBLK * KSTEPS * FRAG));
    };
    // One A fragment of row rho (IDX = (kw*FCO + f)*KSTEPS + ks) into set SET.
    auto load_a_one = [&](auto set_tag, auto idx_tag, int rho, int ct_) {
        constexpr int SET = decltype(set_tag)::value;
        constexpr int IDX = decltype(idx_tag)::value;
        constexpr int kw = IDX / (FCO * KSTEPS), f = (IDX / KSTEPS) % FCO, ks = IDX % KSTEPS;
        const int u = u0 + rho / KS, kh = rho % KS;
        const uint32_t row = (uint32_t)((((ct_ * p.U + u) * KS + kh) * KS) * NBLK * KSTEPS) * FRAG;
        put(A[SET][kw][f][FP8 ? 0 : ks], ks,
            bload_s(wr, wlane + (f * KSTEPS + ks) * FRAG, row + kw * NBLK * KSTEPS * FRAG));
    };
    // The next stage's halo, one staging slot at a time (halo_setup first).
    __amdgpu_buffer_rsrc_t hfr = rsrc(p.x, 0u);
    uint32_t hcb2 = 0;
    bool hgok = false;
    auto halo_setup = [&](int u) {
        const int kt = u % KS, cb = (u / KS) * CB;
        const int ts = t - (KS - 1) + kt;
        if (ts >= 0)
            hfr = rsrc(xb + (size_t)(n * p.T + ts) * p.frame_bytes, p.frame_bytes);
        else if (p.cache)
            hfr = rsrc(cb_base + (size_t)(n * p.F + p.F + ts) * p.frame_bytes, p.frame_bytes);
        else
            hfr = rsrc(p.x, 0u);  // zero causal padding: every load reads zero
        hcb2 = (uint32_t)cb * ESZ;
        hgok = cb + g * CPE < p.Cin;
    };
    auto halo_one = [&](auto k_tag) {
        constexpr int k = decltype(k_tag)::value;
        const uint32_t so = soff[k];
        hv[k] = bload(hfr, (hgok && so != OOB) ? so + hcb2 : OOB);
    };
    auto load_halo = [&](int u) {
        const int kt = u % KS, cb = (u / KS) * CB;
        const int ts = t - (KS - 1) + kt;
        __amdgpu_buffer_rsrc_t fr;
        if (ts >= 0)
            fr = rsrc(xb + (size_t)(n * p.T + ts) * p.frame_bytes, p.frame_bytes);
        else if (p.cache)
            fr = rsrc(cb_base + (size_t)(n * p.F + p.F + ts) * p.frame_bytes, p.frame_bytes);
        else
            fr = rsrc(p.x, 0u);  // zero causal padding: every load reads zero
        const bool gok = cb + g * CPE < p.Cin;
#pragma unroll
        for (int k = 0; k < NIT; ++k)
            hv[k] = bload(fr, (gok && soff[k] != OOB) ? soff[k] + (uint32_t)cb * ESZ : OOB);
    };
    auto store_halo = [&](int u, int buf) {
#pragma unroll
        for (int k = 0; k < NIT; ++k) halo[buf][lbase + 64 * k] = hv[k];
        const int kt = u % KS, cb = (u / KS) * CB;
        if (write_cache && kt >= 1 && (u / KS) % p.co_tiles == ct && cb + g * CPE < p.Cin) {
            char *dst = static_cast<char *>(p.cache_out) + (size_t)(n * 2 + kt - 1) * p.frame_bytes +
                        (size_t)cb * ESZ;
#pragma unroll
            for (int k = 0; k < NIT; ++k)
                if (interior & (1u << k)) *reinterpret_cast<uint4 *>(dst + soff[k]) = hv[k];
        }
    };
    // LDS entry offset of MFMA column tile j relative to column tile 0.
    auto offj = [](int j) { return ((j * M) / TW) * HC + (j * M) % TW; };
    auto load_bq = [&](auto slot_tag, const uint4 *hb, int j, int kh, int kw) {
        constexpr int SL = decltype(slot_tag)::value;
        put(Bq[SL], 0, hb[offj(j) + kh * HC + kw]);
    };
    auto load_b = [&](auto set_tag, const uint4 *hb, int j, int kh, int kw) {
        constexpr int BS = decltype(set_tag)::value;
#pragma unroll
        for (int ks = 0; ks < KSTEPS; ++ks)
            put(B[BS][j][FP8 ? 0 : ks], ks, hb[offj(j) + ks * GPL * HPAD + kh * HC + kw]);
    };

    const int R = (u1 - u0) * KS;  // rows this workgroup runs
    // One row: KS taps of stage u = u0 + rho/KS, kernel row kh = rho % KS.
    // The prefetches are unconditional (indices clamped to the last row or
    // stage; the surplus loads at the very end are never used) so the loads
    // stay where they are issued instead of moving next to their first use.
    auto row = [&](auto set_tag, auto kh_tag, int rho) {
        constexpr int SET = decltype(set_tag)::value;
        constexpr int kh = decltype(kh_tag)::value;
        const int u = u0 + rho / KS;
        const int buf = (u - u0) & 1;
        const uint4 *hb = &halo[buf][bbase];
        const bool last_stage = u + 1 >= u1;
        const int rnext = rho + NSETS - 1 < R ? rho + NSETS - 1 : R - 1;
        if (kh == 0) halo_setup(last_stage ? u : u + 1);
        // Tap tp = kh*KS + kw of the stage reads B[tp & 1]; the next tap's set is
        // filled while this tap's MFMAs run, so no LDS read ever overwrites
        // registers an in-flight MFMA is still reading.  The global loads (the
        // weights of row rho+2, and in a stage's first row the next halo) are
        // spread one at a time over the row's MFMA groups: the wave issues in
        // order, and a block of loads between two MFMAs would leave the matrix
        // pipe idle while it is issued.
        auto tap = [&](auto kw_tag) {
            constexpr int kw = decltype(kw_tag)::value;
            constexpr int tp = kh * KS + kw;
            constexpr int cur = tp & 1;
            constexpr bool next_in_stage = tp + 1 < KS * KS;
            constexpr int nkh = (tp + 1) / KS, nkw = (tp + 1) % KS;
            static_for<KA>([&](auto ks_tag) {
                constexpr int ks = decltype(ks_tag)::value;
                static_for<FPOS>([&](auto j_tag) {
                    constexpr int j = decltype(j_tag)::value;
                    if constexpr (OCC2) {
                        constexpr int q = tp * FPOS + j, q2 = q + 2;
#pragma unroll
                        for (int i = 0; i < FCO; ++i)
                            acc[i][j] = MF::run(A[SET][kw][i][0], Bq[q % 3], acc[i][j]);
                        if constexpr (q2 < KS * KS * FPOS)
                            load_bq(Int<q2 % 3>{}, hb, q2 % FPOS, (q2 / FPOS) / KS, (q2 / FPOS) % KS);
                    } else {
#pragma unroll
                        for (int i = 0; i < FCO; ++i) {
                            if constexpr (FP8)
                                acc[i][j] = mfma_e4m3(A[SET][kw][i][0], B[cur][j][0], acc[i][j]);
                            else
                                acc[i][j] = MF::run(A[SET][kw][i][ks], B[cur][j][ks], acc[i][j]);
                        }
                        if (ks == 0 && next_in_stage) load_b(Int<cur ^ 1>{}, hb, j, nkh, nkw);
                    }
                    // group index within the row, and the loads that fall on it
                    constexpr int NG = KS * KA * FPOS, NL = KS * FCO * KSTEPS;
                    constexpr int grp = (kw * KA + ks) * FPOS + j;
                    static_for<NL>([&](auto li) {
                        constexpr int L_ = decltype(li)::value;
                        if constexpr ((L_ * NG) / NL == grp)
                            load_a_one(Int<(SET + NSETS - 1) % NSETS>{}, Int<L_>{}, rnext, ct);
                    });
                    if constexpr (kh == 0) {
                        static_for<NIT>([&](auto hk) {
                            constexpr int K_ = decltype(hk)::value;
                            if constexpr ((K_ * NG + NG / 2) / NIT == grp) halo_one(Int<K_>{});
                        });
                    }
                    __builtin_amdgcn_sched_barrier(0);
                });
            });
        };
        tap(Int<0>{});
        if constexpr (KS > 1) {
            tap(Int<1>{});
            tap(Int<2>{});
        }
        if (kh == KS - 1 && !last_stage) {
            store_halo(u + 1, buf ^ 1);
            __syncthreads();
            const uint4 *hn = &halo[buf ^ 1][bbase];
            if constexpr (OCC2) {
                load_bq(Int<0>{}, hn, 0, 0, 0);
                load_bq(Int<1>{}, hn, 1 % FPOS, 1 / FPOS, 0);
            } else {
#pragma unroll
                for (int j = 0; j < FPOS; ++j) load_b(Int<0>{}, hn, j, 0, 0);
            }
        }
    };

    if (R <= 0) __syncthreads();  // (the prologue's barrier publishes bias_s otherwise)
    if (R > 0) {
        load_halo(u0);
        load_row(Int<0>{}, 0, ct);
        if constexpr (NSETS == 3) load_row(Int<1>{}, R > 1 ? 1 : 0, ct);
        store_halo(u0, 0);
        __syncthreads();
        const uint4 *h0p = &halo[0][bbase];
        if constexpr (OCC2) {
            load_bq(Int<0>{}, h0p, 0, 0, 0);
            load_bq(Int<1>{}, h0p, 1 % FPOS, 1 / FPOS, 0);
        } else {
#pragma unroll
            for (int j = 0; j < FPOS; ++j) load_b(Int<0>{}, h0p, j, 0, 0);
        }
    }
    if (R > 0) {
        if constexpr (OCC2) {
            // Two row sets alternate while the kernel rows cycle through 3:
            // two stages per iteration, then a last odd stage (R is a
            // multiple of 3).
            int rho = 0;
            for (; rho + 6 <= R; rho += 6) {
                row(Int<0>{}, Int<0>{}, rho);
                row(Int<1>{}, Int<1>{}, rho + 1);
                row(Int<0>{}, Int<2>{}, rho + 2);
                row(Int<1>{}, Int<0>{}, rho + 3);
                row(Int<0>{}, Int<1>{}, rho + 4);
                row(Int<1>{}, Int<2>{}, rho + 5);
            }
            if (rho < R) {
                row(Int<0>{}, Int<0>{}, rho);
                row(Int<1>{}, Int<1>{}, rho + 1);
                row(Int<0>{}, Int<2>{}, rho + 2);
            }
        } else if constexpr (KS == 3) {
            // R is a multiple of 3: one stage per iteration, no row guards.
            for (int rho = 0; rho < R; rho += 3) {
                row(Int<0>{}, Int<0>{}, rho);
                row(Int<1>{}, Int<1>{}, rho + 1);
                row(Int<2>{}, Int<2>{}, rho + 2);
            }
        } else {
            for (int rho = 0; rho < R; rho += 3) {
                row(Int<0>{}, Int<0>{}, rho);
                if (rho + 1 < R) row(Int<1>{}, Int<0>{}, rho + 1);
                if (rho + 2 < R) row(Int<2>{}, Int<0>{}, rho + 2);
            }
        }
    }

    // Epilogue.  Accumulator element e of tile (i, j) is output channel
    // co0 + i*M + (e/4)*8 + lg*4 + e%4 at the position of B column lr in
    // column tile j: tile row (wpos*WPOS + j*M)/TW + bdr, column
    // (wpos*WPOS + j*M)%TW + bc.
    if (SPLIT) {
        // fp32 partial sums of this split, in the output layout; the reduce
        // kernel adds bias and residual.
        float *mine = p.part + (size_t)s * p.part_stride;
#pragma unroll
        for (int j = 0; j < FPOS; ++j) {
            const int q0 = wpos * WPOS + j * M;
            const int r = q0 / TW + bdr, c = q0 % TW + bc;
            const int h = h0 + r, w = w0 + c;
            if (h >= p.H || w >= p.W) continue;
            const size_t obase = (((size_t)(n * p.T + t) * p.H + h) * p.W + w) * p.Cout;
#pragma unroll
            for (int i = 0; i < FCO; ++i)
#pragma unroll
                for (int e4 = 0; e4 < ACC / 4; ++e4) {
                    const int co = co0 + i * M + e4 * 8 + lg * 4;
                    *reinterpret_cast<f32x4 *>(mine + obase + co) =
                        f32x4{acc[i][j][e4 * 4], acc[i][j][e4 * 4 + 1], acc[i][j][e4 * 4 + 2],
                              acc[i][j][e4 * 4 + 3]};
                }
        }
        return;
    }
    // Global loads and stores share one completion counter, so every
    // residual load is issued before the first store: a load issued after a
    // store would wait for that store too.  The bias comes from LDS.
    uint2 bb[FCO][ACC / 4];
    uint2 rr[FPOS][FCO][ACC / 4];
#pragma unroll
    for (int i = 0; i < FCO; ++i)
#pragma unroll
        for (int e4 = 0; e4 < ACC / 4; ++e4)
            bb[i][e4] = bias_s[(wco * WCO + i * M + e4 * 8 + lg * 4) / 4];
#pragma unroll
    for (int j = 0; j < FPOS; ++j) {
        const int q0 = wpos * WPOS + j * M;
        const int r = q0 / TW + bdr, c = q0 % TW + bc;
        const int h = h0 + r, w = w0 + c;
        const bool inside = h < p.H && w < p.W;
        const size_t obase = (((size_t)(n * p.T + t) * p.H + h) * p.W + w) * p.Cout;
#pragma unroll
        for (int i = 0; i < FCO; ++i)
#pragma unroll
            for (int e4 = 0; e4 < ACC / 4; ++e4) {
                const int co = co0 + i * M + e4 * 8 + lg * 4;
                rr[j][i][e4] = (p.res && inside) ? *reinterpret_cast<const uint2 *>(p.res + obase + co)
                                                 : make_uint2(0u, 0u);
            }
    }
#pragma unroll
    for (int j = 0; j < FPOS; ++j) {
        const int q0 = wpos * WPOS + j * M;
        const int r = q0 / TW + bdr, c = q0 % TW + bc;
        const int h = h0 + r, w = w0 + c;
        if (h >= p.H || w >= p.W) continue;
        const size_t obase = (((size_t)(n * p.T + t) * p.H + h) * p.W + w) * p.Cout;
#pragma unroll
        for (int i = 0; i < FCO; ++i)
#pragma unroll
            for (int e4 = 0; e4 < ACC / 4; ++e4) {
                const int co = co0 + i * M + e4 * 8 + lg * 4;
                float v[4] = {acc[i][j][e4 * 4], acc[i][j][e4 * 4 + 1], acc[i][j][e4 * 4 + 2],
                              acc[i][j][e4 * 4 + 3]};
                // the sum (times the scales on the 8-bit path), then the bias,
                // then the residual: the order the split-K reduce kernel uses too
                if constexpr (FP8) {
                    const float4 sc = scale_s[(wco * WCO + i * M + e4 * 8 + lg * 4) / 4];
                    v[0] *= sc.x;
                    v[1] *= sc.y;
                    v[2] *= sc.z;
                    v[3] *= sc.w;
                }
                if (p.bias) {
                    v[0] += bf16_to_f32(bb[i][e4].x & 0xffffu);
                    v[1] += bf16_to_f32(bb[i][e4].x >> 16);
                    v[2] += bf16_to_f32(bb[i][e4].y & 0xffffu);
                    v[3] += bf16_to_f32(bb[i][e4].y >> 16);
                }
                if (p.res) {
                    v[0] += bf16_to_f32(rr[j][i][e4].x & 0xffffu);
                    v[1] += bf16_to_f32(rr[j][i][e4].x >> 16);
                    v[2] += bf16_to_f32(rr[j][i][e4].y & 0xffffu);
                    v[3] += bf16_to_f32(rr[j][i][e4].y >> 16);
                }
                uint2 o;
                o.x = pack2_bf16(v[0], v[1]);
                o.y = pack2_bf16(v[2], v[3]);
                *reinterpret_cast<uint2 *>(p.y + obase + co) = o;
            }
    }
}

// One tile per workgroup (split-K partial sums when SPLIT).
template <int KS, int CO_T, int M, int WAVES_CO, bool SPLIT, int TW, bool FP8 = false>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
igemm_kernel(IgParams p) {
    igemm_body<KS, CO_T, M, WAVES_CO, SPLIT, TW, FP8>(p);
}

// Two workgroups per CU, two waves per SIMD (whole-K 16x16 bf16 tiles): a
// wave's stall at a stage barrier or in its epilogue is covered by the other
// workgroup's MFMAs.
template <int CO_T, int WAVES_CO, int TW>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2)))
igemm_occ2_kernel(IgParams p) {
    igemm_body<3, CO_T, 16, WAVES_CO, false, TW, false, true>(p);
}

// Split-K reduction: y = round(sum_s part[s] (in split order) + bias + residual),
// 8 consecutive channels (one 16-byte output store) per thread.  On the 8-bit
// path (wscale given) the sum is multiplied by xscale * wscale[co] first.
__global__ void __launch_bounds__(256) splitk_reduce_kernel(const float *__restrict__ part,
                                                            size_t stride, int S,
                                                            const uint16_t *__restrict__ bias,
                                                            const uint16_t *__restrict__ res,
                                                            uint16_t *__restrict__ y, long groups,
                                                            int cout,
                                                            const float *__restrict__ wscale = nullptr,
                                                            float xscale = 1.f) {
    const long gi = (long)blockIdx.x * 256 + threadIdx.x;
    if (gi >= groups) return;
    const size_t e0 = (size_t)gi * 8;
    const int co = (int)(e0 % (size_t)cout);
    const uint4 bv = bias ? *reinterpret_cast<const uint4 *>(bias + co) : make_uint4(0u, 0u, 0u, 0u);
    const uint4 rv = res ? *reinterpret_cast<const uint4 *>(res + e0) : make_uint4(0u, 0u, 0u, 0u);
    float v[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) v[k] = 0.f;
    // Splits in order, four splits' loads in flight before their adds.
    for (int sp0 = 0; sp0 < S; sp0 += 4) {
        f32x4 a[4], b[4];
#pragma unroll
        for (int u = 0; u < 4; ++u)
            if (sp0 + u < S) {
                a[u] = *reinterpret_cast<const f32x4 *>(part + (sp0 + u) * stride + e0);
                b[u] = *reinterpret_cast<const f32x4 *>(part + (sp0 + u) * stride + e0 + 4);
            }
#pragma unroll
        for (int u = 0; u < 4; ++u)
            if (sp0 + u < S) {
                v[0] += a[u][0]; v[1] += a[u][1]; v[2] += a[u][2]; v[3] += a[u][3];
                v[4] += b[u][0]; v[5] += b[u][1]; v[6] += b[u][2]; v[7] += b[u][3];
            }
    }
    if (wscale) {
        const float4 s0 = *reinterpret_cast<const float4 *>(wscale + co);
        const float4 s1 = *reinterpret_cast<const float4 *>(wscale + co + 4);
        const float sc[8] = {s0.x, s0.y, s0.z, s0.w, s1.x, s1.y, s1.z, s1.w};
#pragma unroll
        for (int k = 0; k < 8; ++k) v[k] *= xscale * sc[k];
    }
    const uint32_t bw[4] = {bv.x, bv.y, bv.z, bv.w}, rw[4] = {rv.x, rv.y, rv.z, rv.w};
    uint32_t o[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        float lo = v[2 * k], hi = v[2 * k + 1];
        if (bias) {
            lo += bf16_to_f32(bw[k] & 0xffffu);
            hi += bf16_to_f32(bw[k] >> 16);
        }
        if (res) {
            lo += bf16_to_f32(rw[k] & 0xffffu);
            hi += bf16_to_f32(rw[k] >> 16);
        }
        o[k] = pack2_bf16(lo, hi);
    }
    *reinterpret_cast<uint4 *>(y + e0) = make_uint4(o[0], o[1], o[2], o[3]);
}

// Packs W[co][tap][ci] into the order the kernel reads, for channel tile CO_T
// and MFMA tile edge M:
//   packed[co tile][unit][kh][kw][block][ks][lane][16 bytes]
// with unit = (channel block cb) * KS + kt, block < CO_T/M, ks < M/16,
// lane < 64; row co = tile*CO_T + block*M + lane % M.  A 16-byte entry holds
// E = 8 bf16 or 16 E4M3 channels: channel 4E*cb + ks*(64/M)*E + (lane / M)*E
// onwards; zero past C_in.  One fragment (one wave load) is 1 KiB contiguous,
// and one kernel row (unit, kh) of a channel tile is one contiguous run.
template <int M, bool FP8 = false>
__global__ void __launch_bounds__(256) pack_weights_kernel(const void *__restrict__ wv,
                                                           uint4 *__restrict__ out, int cout,
                                                           int cin, int ks_, int co_t) {
    constexpr int KSTEPS = M / 16, GPL = 64 / M;
    constexpr int E = FP8 ? 16 : 8;
    const int nb = (cin + 4 * E - 1) / (4 * E);
    const int nblk = co_t / M, units = ks_ * nb, taps = ks_ * ks_ * ks_;
    const long chunks = (long)(cout / co_t) * units * ks_ * ks_ * nblk * KSTEPS * 64;
    for (long i = (long)blockIdx.x * 256 + threadIdx.x; i < chunks; i += (long)gridDim.x * 256) {
        long r = i;
        const int lane = (int)(r % 64);
        r /= 64;
        const int ks = (int)(r % KSTEPS);
        r /= KSTEPS;
        const int blk = (int)(r % nblk);
        r /= nblk;
        const int kw = (int)(r % ks_);
        r /= ks_;
        const int kh = (int)(r % ks_);
        r /= ks_;
        const int u = (int)(r % units);
        const int ct = (int)(r / units);
        const int kt = u % ks_, cb = u / ks_;
        const int tap = (kt * ks_ + kh) * ks_ + kw;
        const int co = ct * co_t + blk * M + lane % M;
        const int ch = cb * 4 * E + ks * GPL * E + (lane / M) * E;
        uint32_t wd[4] = {0u, 0u, 0u, 0u};
        if constexpr (FP8) {
            const uint8_t *w = static_cast<const uint8_t *>(wv);
#pragma unroll
            for (int k = 0; k < 16; ++k)
                if (ch + k < cin) wd[k / 4] |= (uint32_t)w[((size_t)co * taps + tap) * cin + ch + k] << (8 * (k % 4));
        } else {
            const uint16_t *w = static_cast<const uint16_t *>(wv);
#pragma unroll
            for (int k = 0; k < 8; ++k)
                if (ch + k < cin) wd[k / 2] |= (uint32_t)w[((size_t)co * taps + tap) * cin + ch + k] << (16 * (k % 2));
        }
        out[i] = make_uint4(wd[0], wd[1], wd[2], wd[3]);
    }
}

struct Plan {
    int th, tw, tiles_h, tiles_w, co_t, co_tiles, S, U, co_major;
    long tiles;  // n * t * tiles_h * tiles_w * co_tiles
};

int num_cus() {
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

// Pick a TH x TW tile (TH*TW == 256, TW one of the compiled widths 8, 16, 32)
// that wastes the fewest positions on ragged edges; ties go to the wider tile
// (longer contiguous runs).
void choose_tile(int h, int w, int *th_out, int *tw_out) {
    int bth = 0, btw = 0;
    long best = -1;
    for (int tw = 8; tw <= 32; tw *= 2) {
        const int th = POS_T / tw;
        // tiles narrower than 16 columns split a 16-lane LDS read over rows
        // 2*(tw+2) bytes * 8 apart, which collide in the LDS banks: count them
        // as 25% more expensive
        const long tiles = (long)((h + th - 1) / th) * ((w + tw - 1) / tw);
        const long cost = tw < 16 ? tiles * 5 : tiles * 4;
        if (best < 0 || cost < best || (cost == best && tw > btw)) {
            best = cost;
            bth = th;
            btw = tw;
        }
    }
    *th_out = bth;
    *tw_out = btw;
}

bool is_e4m3(const ConvCall &c) { return c.dtype == WVC_E4M3; }
// Input channels per work unit: one 64-byte slice of a position's channels.
int unit_channels(const ConvCall &c) { return is_e4m3(c) ? 64 : 32; }
int act_bytes(const ConvCall &c) { return is_e4m3(c) ? 1 : 2; }

int co_tile_for(int cout, bool e4m3 = false) {
    if (cout % 128 == 0) return 128;
    if (e4m3) return 32;  // the 8-bit path has 32x32 MFMA tiles only
    if (cout % 96 == 0) return 96;
    if (cout % 64 == 0) return 64;
    return 32;  // the route requires cout % 32 == 0
}

Plan make_plan(const ConvCall &c, ConvRoute r) {
    Plan pl{};
    const int ks = r == ConvRoute::Fast3x3x3 ? 3 : 1;
    choose_tile(c.h, c.w, &pl.th, &pl.tw);
    pl.tiles_h = (c.h + pl.th - 1) / pl.th;
    pl.tiles_w = (c.w + pl.tw - 1) / pl.tw;
    pl.co_t = co_tile_for(c.cout, is_e4m3(c));
    pl.U = ks * ((c.cin + unit_channels(c) - 1) / unit_channels(c));
    const long spatial = (long)c.n * c.t * pl.tiles_h * pl.tiles_w;
    const long cus = num_cus();
    // one workgroup per CU, on the CUs the call may plan for
    const long slots = c.cu_limit > 0 && c.cu_limit < cus ? c.cu_limit : cus;
    // Small grid (fewer tiles than resident slots): order channel tiles
    // slowest, so each XCD works on (about) one channel tile and keeps that
    // slice of the weights in its L2.
    pl.co_major = spatial * (c.cout / pl.co_t) < cus;
    pl.co_tiles = c.cout / pl.co_t;
    pl.tiles = spatial * pl.co_tiles;
    // Split K when the tiles alone leave CUs idle: minimise
    // (rounds of resident workgroups) * (units per split + fixed cost).
    int best_s = 1;
    double best_cost = -1.0;
    const int s_max = pl.U;
    for (int s = 1; s <= s_max && s <= 64; ++s) {
        const long wgs = pl.tiles * s;
        const double rounds = (double)((wgs + slots - 1) / slots);
        const double cost = rounds * ((double)((pl.U + s - 1) / s) + 1.0 + (s > 1 ? 0.5 : 0.0));
        if (best_cost < 0 || cost < best_cost - 1e-9) {
            best_cost = cost;
            best_s = s;
        }
    }
    pl.S = proj_supports(c) ? 1 : best_s;  // the projection kernel never splits K
    return pl;
}

size_t out_elems(const ConvCall &c) { return (size_t)c.n * c.t * c.h * c.w * c.cout; }

size_t part_bytes(const Plan &pl, const ConvCall &c) {
    if (pl.S <= 1) return 0;
    return (size_t)pl.S * out_elems(c) * sizeof(float);
}

int tile_m(int co_t) { return (co_t == 96 || co_t == 64) ? 16 : 32; }

// Channel tile and MFMA edge the packed weights are ordered for: one tile of
// all C_out channels in 16-row blocks for the 1x1x1 projection kernel,
// otherwise the implicit-GEMM kernel's tile.
struct PackGeom {
    int co_t, m;
};
PackGeom pack_geom(const ConvCall &c) {
    if (proj_supports(c)) return PackGeom{c.cout, 16};
    const int ct = co_tile_for(c.cout, is_e4m3(c));
    return PackGeom{ct, is_e4m3(c) ? 32 : tile_m(ct)};
}

size_t packed_bytes(const ConvCall &c) {
    // one 64-byte slice per (output channel, tap, unit)
    const size_t nb = (size_t)(c.cin + unit_channels(c) - 1) / unit_channels(c);
    return (size_t)c.cout * c.kt * c.kh * c.kw * nb * 64;
}

size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }

// Workspace: [split-K partial sums][packed weights when the call brings
// standard-layout weights].  Its contents on entry do not matter.
size_t ws_bytes_for(const Plan &pl, const ConvCall &c, bool need_pack) {
    return align256(part_bytes(pl, c)) + (need_pack ? align256(packed_bytes(c)) : 0);
}

// Whole-K 3x3x3 grids of 16x16 bf16 tiles run two workgroups per CU.
bool runs_occ2(int ks, int m, int S, bool fp8) { return ks == 3 && m == 16 && S == 1 && !fp8; }

template <int KS, int CO_T, int M, int WAVES_CO, int TW, bool FP8>
hipError_t launch_tw(const IgParams &p, hipStream_t s) {
    if (p.S > 1) {
        hipLaunchKernelGGL((igemm_kernel<KS, CO_T, M, WAVES_CO, true, TW, FP8>), dim3(p.total),
                           dim3(256), 0, s, p);
        return hipGetLastError();
    }
    if constexpr (KS == 3 && M == 16 && !FP8) {
        hipLaunchKernelGGL((igemm_occ2_kernel<CO_T, WAVES_CO, TW>), dim3(p.total), dim3(256), 0, s, p);
        return hipGetLastError();
    }
    hipLaunchKernelGGL((igemm_kernel<KS, CO_T, M, WAVES_CO, false, TW, FP8>), dim3(p.total),
                       dim3(256), 0, s, p);
    return hipGetLastError();
}

template <int KS, int CO_T, int M, int WAVES_CO, bool FP8 = false>
hipError_t launch_variant(const IgParams &p, int tw, hipStream_t s) {
    switch (tw) {
        case 8: return launch_tw<KS, CO_T, M, WAVES_CO, 8, FP8>(p, s);
        case 16: return launch_tw<KS, CO_T, M, WAVES_CO, 16, FP8>(p, s);
        case 32: return launch_tw<KS, CO_T, M, WAVES_CO, 32, FP8>(p, s);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

size_t igemm_workspace_bytes(const ConvCall &c, ConvRoute r, bool packed_given) {
    if (c.t <= 0) return 0;
    return ws_bytes_for(make_plan(c, r), c, !packed_given);
}

size_t igemm_packed_weight_bytes(const ConvCall &c) { return packed_bytes(c); }

hipError_t launch_pack_weights(const ConvCall &c, const void *w, void *packed, hipStream_t s) {
    const PackGeom pg = pack_geom(c);
    const int co_t = pg.co_t, m = pg.m;
    const long chunks = (long)packed_bytes(c) / 16;
    long blocks = (chunks + 255) / 256;
    if (blocks > 8192) blocks = 8192;
    if (blocks < 1) return hipSuccess;
    if (is_e4m3(c))
        hipLaunchKernelGGL((pack_weights_kernel<32, true>), dim3((unsigned)blocks), dim3(256), 0, s,
                           w, static_cast<uint4 *>(packed), c.cout, c.cin, c.kt, co_t);
    else if (m == 32)
        hipLaunchKernelGGL(pack_weights_kernel<32>, dim3((unsigned)blocks), dim3(256), 0, s, w,
                           static_cast<uint4 *>(packed), c.cout, c.cin, c.kt, co_t);
    else
        hipLaunchKernelGGL(pack_weights_kernel<16>, dim3((unsigned)blocks), dim3(256), 0, s, w,
                           static_cast<uint4 *>(packed), c.cout, c.cin, c.kt, co_t);
    return hipGetLastError();
}

bool igemm_supports(const ConvCall &c) {
    // 32-bit buffer offsets: one frame and the packed weights must stay below 2 GiB.
    const size_t frame = (size_t)c.h * c.w * c.cin * act_bytes(c);
    const size_t wbytes = packed_bytes(c);
    if (is_e4m3(c) && (c.cin % 16 != 0 || c.kt != 3)) return false;
    return frame < ((size_t)1 << 31) && wbytes < ((size_t)1 << 31) && c.cout % 32 == 0;
}

int igemm_kernel_name(const ConvCall &c, ConvRoute r, char *buf, size_t n) {
    if (r == ConvRoute::Fast1x1x1 && proj_supports(c))
        return snprintf(buf, n, "%s", proj_kernel_name(c));
    const Plan pl = make_plan(c, r);
    const int ks = r == ConvRoute::Fast3x3x3 ? 3 : 1;
    const bool fp8 = is_e4m3(c);
    const int co_t = pl.co_t;
    const int m = fp8 ? 32 : tile_m(co_t);
    const int waves_co = co_t == 32 ? 1 : 2;
    const char *f8 = fp8 ? "true" : "false";
    if (pl.S > 1)
        return snprintf(buf, n, "igemm_kernel<%d, %d, %d, %d, true, %d, %s> + splitk_reduce_kernel",
                        ks, co_t, m, waves_co, pl.tw, f8);
    if (runs_occ2(ks, m, pl.S, fp8))
        return snprintf(buf, n, "igemm_occ2_kernel<%d, %d, %d>", co_t, waves_co, pl.tw);
    return snprintf(buf, n, "igemm_kernel<%d, %d, %d, %d, false, %d, %s>", ks, co_t, m, waves_co,
                    pl.tw, f8);
}

hipError_t launch_conv_igemm(const ConvCall &c, ConvRoute r, bool packed_given, void *ws,
                             size_t ws_bytes, void *cache_out, hipStream_t s, ConvPartials *defer) {
    if (defer) *defer = ConvPartials{};
    // (8-bit conv: deferred partials are raw sums; the consumer applies the scales)
    if (is_e4m3(c) && r != ConvRoute::Fast3x3x3) return hipErrorInvalidValue;
    const Plan pl = make_plan(c, r);
    if (pl.th == 0) return hipErrorInvalidValue;
    if (ws_bytes < ws_bytes_for(pl, c, !packed_given) || (!ws && ws_bytes_for(pl, c, !packed_given)))
        return hipErrorInvalidValue;
    const void *wp = c.weight;
    if (!packed_given) {
        void *dst = static_cast<char *>(ws) + align256(part_bytes(pl, c));
        const hipError_t e = launch_pack_weights(c, c.weight, dst, s);
        if (e != hipSuccess) return e;
        wp = dst;
    }
    if (r == ConvRoute::Fast1x1x1 && proj_supports(c))
        return launch_conv_proj(c, wp, packed_bytes(c), s);
    IgParams p{};
    p.x = c.x;
    p.cache = c.cache_in;
    p.w = static_cast<const uint16_t *>(wp);
    p.bias = static_cast<const uint16_t *>(c.bias);
    p.res = static_cast<const uint16_t *>(c.residual);
    p.y = static_cast<uint16_t *>(c.y);
    p.cache_out = r == ConvRoute::Fast3x3x3 ? cache_out : nullptr;
    p.wscale = c.wscale;
    p.xscale = c.xscale;
    p.T = c.t;
    p.H = c.h;
    p.W = c.w;
    p.Cin = c.cin;
    p.Cout = c.cout;
    p.F = c.frames;
    p.tiles_w = pl.tiles_w;
    p.tiles_h = pl.tiles_h;
    p.co_tiles = pl.co_tiles;
    p.S = pl.S;
    p.U = pl.U;
    p.co_major = pl.co_major;
    p.up = c.up == 2 ? 2 : 1;
    p.frame_bytes = (uint32_t)((size_t)(c.h / p.up) * (c.w / p.up) * c.cin * act_bytes(c));
    p.w_bytes = (uint32_t)packed_bytes(c);
    if (pl.S > 1) {
        p.part = static_cast<float *>(ws);
        p.part_stride = out_elems(c);
    }
    const long total = pl.tiles * pl.S;
    if (total <= 0) return hipSuccess;
    if (total > 0x7fffffffL) return hipErrorInvalidValue;
    p.total = (int)total;
    const bool k3 = r == ConvRoute::Fast3x3x3;
    // 128 channels: 32x32x16 MFMAs on 2 x 2 waves of 64 x 128.  96 and 64:
    // 16x16x32 MFMAs on 2 x 2 waves (48 or 32 channels x 128 positions).
    // 32: 32x32x16 on 1 x 4 waves of 32 x 64.
    hipError_t e;
    if (is_e4m3(c))
        e = pl.co_t == 128 ? launch_variant<3, 128, 32, 2, true>(p, pl.tw, s)
                           : launch_variant<3, 32, 32, 1, true>(p, pl.tw, s);
    else switch (pl.co_t) {
        case 128: e = k3 ? launch_variant<3, 128, 32, 2>(p, pl.tw, s) : launch_variant<1, 128, 32, 2>(p, pl.tw, s); break;
        case 96: e = k3 ? launch_variant<3, 96, 16, 2>(p, pl.tw, s) : launch_variant<1, 96, 16, 2>(p, pl.tw, s); break;
        case 64: e = k3 ? launch_variant<3, 64, 16, 2>(p, pl.tw, s) : launch_variant<1, 64, 16, 2>(p, pl.tw, s); break;
        default: e = k3 ? launch_variant<3, 32, 32, 1>(p, pl.tw, s) : launch_variant<1, 32, 32, 1>(p, pl.tw, s); break;
    }
    if (e != hipSuccess || pl.S <= 1) return e;
    if (defer) {
        defer->part = p.part;
        defer->stride = p.part_stride;
        defer->S = pl.S;
        return hipSuccess;
    }
    const long groups = (long)(out_elems(c) / 8);  // Cout % 32 == 0 on this route
    const long blocks = (groups + 255) / 256;
    if (blocks > 0x7fffffffL) return hipErrorInvalidValue;
    hipLaunchKernelGGL(splitk_reduce_kernel, dim3((unsigned)blocks), dim3(256), 0, s, p.part,
                       p.part_stride, pl.S, p.bias, p.res, p.y, groups, c.cout,
                       is_e4m3(c) ? c.wscale : nullptr, c.xscale);
    return hipGetLastError();
}

}  // namespace wvc
