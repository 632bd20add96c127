// igemm_halo.hip -- implicit-GEMM convolution for stride 1 with the input
// staged once per channel chunk as a halo tile in LDS.
//
// Same GEMM as the gather kernel (lincklin.cn lesson 9, sections 7, 11, 19):
// per group, D[co][p] = sum_k W[co][k] * X_col[k][p] with k = (ci, kh, kw).
// What changes is where X_col comes from.  A tile is BM output channels x a
// TH x TW block of output pixels of one image.  For stride 1 every tap of
// that block reads inside one (TH + (Kh-1)D) x (TW + (Kw-1)D) input window --
// the block plus its halo (lincklin.cn section 12: a 16x16 output tile of a
// 3x3 filter needs an 18x18 input tile).  The window is loaded from HBM/L2
// once per 32-channel chunk into LDS (section 13: load the tile
// cooperatively, synchronise, let every thread read its windows), and each
// of the Kh*Kw taps then reads its B operand from that tile at a fixed
// offset (kh*D rows, kw*D columns): input reuse across taps happens in LDS
// instead of through the vector-memory path.  Dilation is only a larger
// offset, so exactly the Kh*Kw real taps are gathered (lpnh.cn section 4.2).
// Zero padding: window pixels outside the image are loaded as 0
// (lincklin.cn section 26).
//
// Schedule.  The kernel is persistent: workgroup b walks tiles b, b+G, ...
// as one continuous stream of K-steps (one step = one tap of one 32-channel
// chunk), so the loads of the next tile's first steps overlap the current
// tile's last ones and there is no per-tile prologue.  Per step:
//  * the BM x 32 weight slice is staged in a 3-slot LDS ring; its global
//    loads are issued two steps ahead of their LDS store (two register sets),
//  * one 16-byte piece per thread of the NEXT chunk's halo tile is loaded at
//    each of the chunk's first taps (a load that returns zero at the others,
//    so every step issues the same number of loads) and stored one step
//    later into the other halo buffer,
//  * v_mfma_f32_32x32x16_bf16 runs on two 16-wide K slices; the operands of
//    the second slice are read from LDS while the first slice's matrix ops
//    run, and the operands of the NEXT step's first slice while the second
//    slice's run -- the 3-slot ring makes that step's weights visible one
//    barrier earlier, so a wave leaves each barrier with its operands
//    already in registers,
//  * one barrier.
// fp32 accumulators stay in registers for the whole K loop of a tile
// (output stationary).  At a tile's last step the epilogue adds the bias,
// applies ReLU, rounds to bf16 and stores straight from registers
// (lincklin.cn section 31): a lane-half swap (v_permlane32_swap) turns the
// 32x32 result layout into 8 consecutive channels of one pixel per lane, one
// 16-byte store each.
#include "halo.hpp"
#include "../../include/conv2d.h"

namespace conv2d {

namespace {

// Tile configurations per range of output channels per group: threads,
// workgroups per CU the kernel is compiled for, BM output channels, WGM x WGN
// waves, two equal-size pixel-block shapes (rows x columns).  Two
// independent workgroups per CU (one wave per SIMD each) let one workgroup's
// epilogue, barrier and load waits overlap the other's matrix work.
// Overridable at build time for tuning sweeps.
#ifndef HALO_CFG_M128
#define HALO_CFG_M128 256, 2, 128, 1, 4, 16, 16, 8, 32
#endif
#ifndef HALO_CFG_M64
#define HALO_CFG_M64 256, 2, 64, 1, 4, 16, 16, 8, 32
#endif

constexpr int kKEmax = 5;    // largest effective filter extent (Kh-1)*D+1 the halo buffer holds

// LDS bytes of one workgroup: weight ring, two halo buffers, two bias buffers.
constexpr int halo_lds_bytes(int bm, int th, int tw, int ke, bool bias) {
    return kRing * bm * kBK * 2 + 2 * (th + ke - 1) * (tw + ke - 1) * kHP * 16 + (bias ? 2 * bm * 4 : 0);
}

// KE: largest effective filter extent the halo buffers hold (3 or 5).
template <int NT, int MINB, int BM, int TH, int TW, int WGM, int WGN, int KE, bool CFULL, bool BIAS, bool RELU>
__global__ __launch_bounds__(NT, waves_per_simd(NT, MINB, halo_lds_bytes(BM, TH, TW, KE, BIAS))) void halo_kernel(
    const bf16_t* __restrict__ x, const bf16_t* __restrict__ wp, const float* __restrict__ bias,
    bf16_t* __restrict__ y, Shape s, HaloGrid hg) {
    constexpr int BN = TH * TW;
    static_assert(WGM * WGN * 64 == NT, "one wave per sub-tile");
    constexpr int WTM = BM / WGM, WTN = BN / WGN;
    constexpr int TM = WTM / 32, TN = WTN / 32;
    static_assert(TM * 32 == WTM && TN * 32 == WTN, "32x32 MFMA tiles");
    constexpr int HCAP = (TH + KE - 1) * (TW + KE - 1);          // halo pixels per buffer
    constexpr int A_BYTES = BM * kBK * 2;                        // one weight slot
    constexpr int H_BYTES = HCAP * kHP * 16;                     // one halo buffer
    constexpr int AV = BM * 4 / NT;                              // weight loads per thread per step
    static_assert(AV * NT == BM * 4 && AV >= 1, "weight slice splits evenly");
    constexpr int NPMAX = (HCAP * 4 + NT - 1) / NT;              // halo parts per chunk, at most
    constexpr int B_BYTES = BIAS ? BM * 4 : 0;                   // one tile's bias
    // LDS: weight ring | two halo buffers | two bias buffers (current tile,
    // next tile)
    __shared__ uint4 lds[(kRing * A_BYTES + 2 * H_BYTES + 2 * B_BYTES) / 16];
    char* const ring = reinterpret_cast<char*>(lds);
    char* const halo = ring + kRing * A_BYTES;
    char* const sbias = halo + 2 * H_BYTES;

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave / WGN, wn = wave % WGN;

    // This workgroup's tiles: first, first + G, ... (the first index is
    // XCD-aware, so each XCD's L2 sees one run of neighbouring tiles).
    const int G = gridDim.x;
    const int first = xcd_tile_index();
    if (first >= hg.ntiles) return;
    const int nmine = (hg.ntiles - 1 - first) / G + 1;
    const int KK = s.Kh * s.Kw;
    const int nchunk = (s.cin_g + kBK - 1) / kBK;
    const int total = nmine * nchunk * KK;  // K-steps of this workgroup
    const int HWd = TW + (s.Kw - 1) * s.dil;  // halo window width
    const int hunits = (TH + (s.Kh - 1) * s.dil) * HWd * 4;
    const int tap_row = s.dil * HWd * (kHP * 16);  // LDS bytes between taps kh and kh+1
    const int tap_col = s.dil * (kHP * 16);
    const int wrow = KK * s.cin_g * 2;               // bytes of one packed weight row

    const __amdgpu_buffer_rsrc_t xr = make_rsrc(x, (uint32_t)s.N * s.H * s.W * s.Cin * 2u);
    const __amdgpu_buffer_rsrc_t wr = make_rsrc(wp, (uint32_t)s.Cout * (uint32_t)wrow);
    const __amdgpu_buffer_rsrc_t yr = make_rsrc(y, (uint32_t)s.N * s.Ho * s.Wo * s.Cout * 2u);
    const __amdgpu_buffer_rsrc_t br = make_rsrc(bias, BIAS ? (uint32_t)s.Cout * 4u : 0u);

    // ---- weight slots: row = output channel within the tile, 4 chunks of 8
    int a_row[AV], a_c[AV], a_lds[AV];
#pragma unroll
    for (int i = 0; i < AV; ++i) {
        const int q = tid + i * NT;
        a_row[i] = q >> 2;
        a_c[i] = (q & 3) * 8;
        a_lds[i] = swz<kBK>(q >> 2, q & 3) * 16;
    }
    // ---- MFMA operand reads: lane supplies row (lane % 32), K values
    // 8*(lane/32).. of each 16-wide K slice (chunks 2*ks, 2*ks+1 of a row)
    const int frow = lane & 31, fch = lane >> 5;
    int a_rd[2][TM];
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
        for (int i = 0; i < TM; ++i) a_rd[ks][i] = swz<kBK>(wm * WTM + i * 32 + frow, 2 * ks + fch) * 16;
    int b_rd[TN];  // byte offset in a halo buffer of this lane's operand at tap (0, 0)
#pragma unroll
    for (int j = 0; j < TN; ++j) {
        const int p = wn * WTN + j * 32 + frow;
        b_rd[j] = (((p / TW) * HWd + p % TW) * kHP + fch) * 16;
    }

    // Weight loads of K-step (tile coordinates T, chunk C, tap TP): the
    // per-lane offset holds the row (or lies past the end for a row beyond
    // this group's channels); tap and chunk ride in the scalar offset.
#define A_LOAD(RA, RB, CT0, C, TP)                                                           \
    do {                                                                                     \
        _Pragma("unroll") for (int i = 0; i < AV; ++i) {                                     \
            const bool ok_ = (CT0) + a_row[i] < s.cout_g &&                                  \
                             (CFULL || (C) * kBK + a_c[i] < s.cin_g);                        \
            (RA)[i] = load16(wr, ok_ ? (RB) + a_row[i] * wrow + a_c[i] * 2 : kOOB,           \
                             __builtin_amdgcn_readfirstlane(((TP) * s.cin_g + (C) * kBK) * 2)); \
        }                                                                                    \
    } while (0)
#define A_STORE(RA, SLOT)                                                                    \
    do {                                                                                     \
        _Pragma("unroll") for (int i = 0; i < AV; ++i)                                       \
            *reinterpret_cast<uint4*>(ring + (SLOT) * A_BYTES + a_lds[i]) = (RA)[i];         \
    } while (0)
    // Halo part U of chunk C of the tile at image N, origin (HO0, WO0), group
    // GG (VALID false: a load that returns 0): window unit v = tid + U*NT is
    // (pixel v/4, channel block v%4).  HL: LDS byte offset of the destination
    // in halo buffer HB (-1: nothing to store).
#define H_LOAD(RH, HL, N, GG, HO0, WO0, C, U, VALID, HB)                                     \
    do {                                                                                     \
        const int v_ = tid + (U) * NT;                                                       \
        const int hp_ = v_ >> 2, hch_ = v_ & 3;                                              \
        const int hr_ = (hp_ * hg.hwd_magic) >> 16;                                          \
        const int hi_ = (HO0) - s.pad + hr_, wi_ = (WO0) - s.pad + hp_ - hr_ * HWd;          \
        const bool in_ = (VALID) && v_ < hunits;                                             \
        const bool ok_ = in_ && (unsigned)hi_ < (unsigned)s.H && (unsigned)wi_ < (unsigned)s.W && \
                         (CFULL || (C) * kBK + hch_ * 8 < s.cin_g);                          \
        (RH) = load16(xr, ok_ ? (((N) * s.H + hi_) * s.W + wi_) * s.Cin * 2 +                \
                                    ((GG) * s.cin_g + hch_ * 8) * 2 : kOOB,                  \
                      __builtin_amdgcn_readfirstlane((C) * kBK * 2));                        \
        (HL) = in_ ? kRing * A_BYTES + (HB) * H_BYTES + (hp_ * kHP + hch_) * 16 : -1;        \
    } while (0)
    // The bias of the tile at (group GG, channel tile CT) into bias buffer BB:
    // four channels per thread.
#define B_LOAD(RH, HL, GG, CT, VALID, BB)                                                    \
    do {                                                                                     \
        const bool in_ = (VALID) && tid * 4 < BM;                                            \
        (RH) = load16(br, in_ ? ((GG) * s.cout_g + (CT) * BM + tid * 4) * 4 : kOOB);         \
        (HL) = in_ ? kRing * A_BYTES + 2 * H_BYTES + (BB) * B_BYTES + tid * 16 : -1;         \
    } while (0)
    // The piece loaded at tap t of a chunk: halo part t of the next chunk for
    // t < nparts; at t == nparts of a tile's last chunk, the next tile's bias;
    // else a load that returns 0 and is not stored.  Every step issues the
    // same number of loads.
#define PIECE_LOAD(RH, HL)                                                                   \
    do {                                                                                     \
        if (BIAS && t == hg.nparts && c + 1 == nchunk)                                       \
            B_LOAD(RH, HL, tn.g, tn.ct, k + 1 < nmine, (k + 1) & 1);                         \
        else                                                                                 \
            H_LOAD(RH, HL, h_n, h_g, h_ho0, h_wo0, h_c, t, h_ok && t < hg.nparts, hsel ^ 1); \
    } while (0)

    // ---- cursors (all wave-uniform; updated with scalar selects only, so
    // the load section of a step has no branch)
    int k = 0;                                       // tile iteration of the current step
    TileXY tc = tile_xy<TH, TW>(first, hg, s.groups);  // current tile
    TileXY tn = tile_xy<TH, TW>(nmine > 1 ? first + G : first, hg, s.groups);  // next tile
    int c = 0, t = 0, kh = 0, kw = 0;                // chunk and tap of the current step
    int hsel = 0;                                    // halo buffer of the current chunk
    int r0 = 0;                                      // ring slot of the current step
    // weight-load cursor: step + 3 (chunk, tap, row base and first channel of its tile)
    int ac = 0, at = 0;
    int a_rb = (tc.g * s.cout_g + tc.ct * BM) * wrow, a_ct = tc.ct * BM;
    for (int adv = 0; adv < 3; ++adv) {
        if (++at == KK) {
            at = 0;
            if (++ac == nchunk) {
                ac = 0;
                a_rb = (tn.g * s.cout_g + tn.ct * BM) * wrow;
                a_ct = tn.ct * BM;
            }
        }
    }
    // halo-load cursor: the chunk after the current one (its tile's image,
    // group, origin; false past the last tile)
    int h_n, h_g, h_ho0, h_wo0, h_c;
    bool h_ok;
#define HALO_NEXT_CHUNK()                                                                    \
    do {                                                                                     \
        const bool same_ = c + 1 < nchunk;                                                   \
        h_n = same_ ? tc.n : tn.n;                                                           \
        h_g = same_ ? tc.g : tn.g;                                                           \
        h_ho0 = same_ ? tc.ho0 : tn.ho0;                                                     \
        h_wo0 = same_ ? tc.wo0 : tn.wo0;                                                     \
        h_c = same_ ? c + 1 : 0;                                                             \
        h_ok = same_ || k + 1 < nmine;                                                       \
    } while (0)
    HALO_NEXT_CHUNK();

    f32x16 acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) acc[i][j] = f32x16{};

    uint4 ra0[AV], ra1[AV], rh0, rh1;
    int hl0 = -1, hl1 = -1;
    bf16x8 af0[TM], bf0[TN], af1[TM], bf1[TN];

    // ---- prologue: weight steps 0 and 1 and the first chunk's halo in LDS,
    // step 2's weights in flight (ra0), the first slice's operands read.
    // Steps 0..2 lie in the first tile: the host admits only Kh*Kw >= 3.
    {
        const int c1 = 1 / KK, t1 = 1 - c1 * KK;
        const int c2 = 2 / KK, t2 = 2 - c2 * KK;
        uint4 p0[AV], p1[AV], ph[NPMAX];
        int pl[NPMAX];
        const int rb0 = (tc.g * s.cout_g + tc.ct * BM) * wrow;
        A_LOAD(p0, rb0, tc.ct * BM, 0, 0);
        A_LOAD(p1, rb0, tc.ct * BM, c1, t1);
#pragma unroll
        for (int u = 0; u < NPMAX; ++u)
            H_LOAD(ph[u], pl[u], tc.n, tc.g, tc.ho0, tc.wo0, 0, u, u < hg.nparts, 0);
        uint4 pb;
        int pbl = -1;
        if (BIAS) B_LOAD(pb, pbl, tc.g, tc.ct, true, 0);
        A_LOAD(ra0, rb0, tc.ct * BM, c2, t2);
        A_STORE(p0, 0);
        A_STORE(p1, 1);
#pragma unroll
        for (int u = 0; u < NPMAX; ++u)
            if (pl[u] >= 0) *reinterpret_cast<uint4*>(ring + pl[u]) = ph[u];
        if (BIAS && pbl >= 0) *reinterpret_cast<uint4*>(ring + pbl) = pb;
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < TM; ++i) af0[i] = *reinterpret_cast<const bf16x8*>(ring + a_rd[0][i]);
#pragma unroll
    for (int j = 0; j < TN; ++j) bf0[j] = *reinterpret_cast<const bf16x8*>(halo + b_rd[j]);

    // Epilogue of the current tile (tc): bias (this tile's bias buffer),
    // ReLU, bf16, whole-line stores (the shared tile epilogue).
#define HALO_EPILOGUE()                                                                      \
    tile_epilogue<TM, TN, WTM, WTN, TH, TW, BIAS, RELU>(acc, sbias + (k & 1) * B_BYTES, yr, s, tc, tc.ct * BM, \
                                                        wm, wn, lane)

    // One K-step.  RA_LD/RA_ST: weight registers loaded now (for step + 3) /
    // stored now (step + 2, loaded one step ago); RH_LD/HL_LD, RH_ST/HL_ST:
    // the same for the halo piece.
#define HALO_STEP(RA_LD, RA_ST, RH_LD, HL_LD, RH_ST, HL_ST)                                  \
    do {                                                                                     \
        /* (1) loads: weights of step + 3, halo part t of the next chunk */                  \
        A_LOAD(RA_LD, a_rb, a_ct, ac, at);                                                   \
        PIECE_LOAD(RH_LD, HL_LD);                                                            \
        __builtin_amdgcn_sched_barrier(0);                                                   \
        /* (2) second slice's operands; first slice's matrix ops */                          \
        const char* acur_ = ring + r0 * A_BYTES;                                             \
        const char* hcur_ = halo + hsel * H_BYTES + kh * tap_row + kw * tap_col;             \
        _Pragma("unroll") for (int i = 0; i < TM; ++i)                                       \
            af1[i] = *reinterpret_cast<const bf16x8*>(acur_ + a_rd[1][i]);                   \
        _Pragma("unroll") for (int j = 0; j < TN; ++j)                                       \
            bf1[j] = *reinterpret_cast<const bf16x8*>(hcur_ + b_rd[j] + 32);                 \
        __builtin_amdgcn_sched_barrier(0);                                                   \
        _Pragma("unroll") for (int i = 0; i < TM; ++i)                                       \
            _Pragma("unroll") for (int j = 0; j < TN; ++j)                                   \
                acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af0[i], bf0[j], acc[i][j], 0, 0, 0); \
        /* (3) next step's first-slice operands; second slice's matrix ops */                \
        const int r1_ = r0 == kRing - 1 ? 0 : r0 + 1;                                        \
        const char* anext_ = ring + r1_ * A_BYTES;                                           \
        const char* hnext_;                                                                  \
        if (t + 1 < KK) {                                                                    \
            const int nkw_ = kw + 1 == s.Kw ? 0 : kw + 1;                                    \
            const int nkh_ = kw + 1 == s.Kw ? kh + 1 : kh;                                   \
            hnext_ = halo + hsel * H_BYTES + nkh_ * tap_row + nkw_ * tap_col;                \
        } else {                                                                             \
            hnext_ = halo + (hsel ^ 1) * H_BYTES;                                            \
        }                                                                                    \
        _Pragma("unroll") for (int i = 0; i < TM; ++i)                                       \
            af0[i] = *reinterpret_cast<const bf16x8*>(anext_ + a_rd[0][i]);                  \
        _Pragma("unroll") for (int j = 0; j < TN; ++j)                                       \
            bf0[j] = *reinterpret_cast<const bf16x8*>(hnext_ + b_rd[j]);                     \
        _Pragma("unroll") for (int i = 0; i < TM; ++i)                                       \
            _Pragma("unroll") for (int j = 0; j < TN; ++j)                                   \
                acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af1[i], bf1[j], acc[i][j], 0, 0, 0); \
        __builtin_amdgcn_sched_barrier(0);                                                   \
        /* (4) LDS stores: weights of step + 2; the piece loaded last step (none  \
           at a chunk's first tap: the last tap loads nothing) */                            \
        A_STORE(RA_ST, r1_ == kRing - 1 ? 0 : r1_ + 1);                                      \
        if ((HL_ST) >= 0) *reinterpret_cast<uint4*>(ring + (HL_ST)) = (RH_ST);               \
        /* (5) a tile's last step: epilogue, then the next tile */                           \
        if (t + 1 == KK && c + 1 == nchunk) {                                                \
            HALO_EPILOGUE();                                                                 \
            _Pragma("unroll") for (int i = 0; i < TM; ++i)                                   \
                _Pragma("unroll") for (int j = 0; j < TN; ++j) acc[i][j] = f32x16{};         \
            ++k;                                                                             \
            tc = tn;                                                                         \
            tn = tile_xy<TH, TW>(k + 1 < nmine ? first + (k + 1) * G : first, hg, s.groups); \
        }                                                                                    \
        __syncthreads();                                                                     \
        /* (6) advance the cursors */                                                        \
        r0 = r1_;                                                                            \
        if (++kw == s.Kw) { kw = 0; ++kh; }                                                  \
        if (++t == KK) {                                                                     \
            t = 0; kh = 0; kw = 0; hsel ^= 1;                                                \
            if (++c == nchunk) c = 0;                                                        \
            HALO_NEXT_CHUNK();                                                               \
        }                                                                                    \
        if (++at == KK) {                                                                    \
            at = 0;                                                                          \
            if (++ac == nchunk) {                                                            \
                /* the weight cursor enters the tile after the current one */                \
                ac = 0;                                                                      \
                a_rb = (tn.g * s.cout_g + tn.ct * BM) * wrow;                                \
                a_ct = tn.ct * BM;                                                           \
            }                                                                                \
        }                                                                                    \
    } while (0)

    // Two steps per iteration so the two register sets alternate statically.
    // An odd step count runs one extra step past the end: its loads read
    // zeros or in-range weights, its results are never stored.
    for (int st = 0; st < total; st += 2) {
        HALO_STEP(ra1, ra0, rh0, hl0, rh1, hl1);
        HALO_STEP(ra0, ra1, rh1, hl1, rh0, hl0);
    }
#undef HALO_STEP
#undef HALO_EPILOGUE
#undef A_LOAD
#undef A_STORE
#undef H_LOAD
#undef B_LOAD
#undef PIECE_LOAD
#undef HALO_NEXT_CHUNK
}

// 3x3 filters with dilation DIL (1 or 2): the same schedule as halo_kernel,
// with the nine taps of a chunk unrolled at compile time.  Ring slots, tap
// offsets and every LDS operand address are immediates; load offsets are
// computed once per chunk; a K-step issues little besides its global loads,
// LDS reads, matrix ops and LDS stores.  Per step (tap t of a chunk):
//  * weights of step + 3 are loaded into register set t % 3 and stored one
//    step later into ring slot (t + 2) % 3 (the slot read three steps later),
//  * at taps 0 .. NPS-1 two 64-unit copies per wave of the next chunk's halo
//    window go straight from memory into the other halo buffer (buffer loads
//    to LDS: no registers, no LDS store instruction); they have until the
//    barrier that closes tap 7 to land, four to seven steps later.  At tap
//    NPS of a tile's last chunk, the next tile's bias is loaded (stored one
//    step later),
//  * the second slice's operands are read, the first slice's matrix ops
//    issue, the next step's first-slice operands are read, the second
//    slice's matrix ops issue,
//  * one barrier.
// The nine steps of a chunk run in a function whose LDS buffers (ring, the
// current and the next halo buffer, bias) are distinct restrict arguments:
// the compiler can then tell the copies in flight into the next buffer from
// this chunk's operand reads and does not wait for them before each read.
// Each wave waits for its own copies before the barrier that closes tap 7
// (loads complete in order, so waiting until only tap 7's weight loads are
// outstanding covers them); the next chunk's first operands are read after
// that barrier.
template <int NT, int MINB, int BM, int TH, int TW, int WGM, int WGN, int DIL, bool CFULL, bool BIAS, bool RELU>
__global__ __launch_bounds__(NT, waves_per_simd(NT, MINB, halo_lds_bytes(BM, TH, TW, 2 * DIL + 1, BIAS)))
void halo3_kernel(const bf16_t* __restrict__ x, const bf16_t* __restrict__ wp, const float* __restrict__ bias,
                  bf16_t* __restrict__ y, Shape s, HaloGrid hg) {
    constexpr int BN = TH * TW;
    static_assert(WGM * WGN * 64 == NT, "one wave per sub-tile");
    constexpr int WTM = BM / WGM, WTN = BN / WGN;
    constexpr int TM = WTM / 32, TN = WTN / 32;
    static_assert(TM * 32 == WTM && TN * 32 == WTN, "32x32 MFMA tiles");
    static_assert(32 % TW == 0 || TW % 32 == 0, "32-pixel MFMA tiles cover whole block rows");
    constexpr int HWd = TW + 2 * DIL, HH = TH + 2 * DIL;  // halo window
    constexpr int A_BYTES = BM * kBK * 2;
    constexpr int HU5 = HH * HWd * kHP;                    // 16-byte units of a halo buffer (padding included)
    constexpr int H_BYTES = HU5 * 16;
    constexpr int B_BYTES = BIAS ? BM * 4 : 0;
    constexpr int AV = BM * 4 / NT;
    static_assert(AV * NT == BM * 4 && AV >= 1 && AV < 16, "weight slice splits evenly");
    constexpr int NW = NT / 64;                            // waves
    constexpr int NCOPY = (HU5 + 63) / 64;                 // 64-unit copies per halo window
    constexpr int DPW = (NCOPY + NW - 1) / NW;             // copies per wave per chunk
    constexpr int DPS = 2;                                 // copies per step
    constexpr int NPS = (DPW + DPS - 1) / DPS;             // steps that issue copies (taps 0 .. NPS-1)
    static_assert(NPS + 1 <= 6, "copies and the next tile's bias issue before tap 7");
    static_assert(HWd < 256 && HH < 256, "window coordinates pack into bytes");
    // LDS distance between MFMA column blocks j and j + 1 (32 pixels)
    constexpr int JSTRIDE = TW <= 32 ? (32 / TW) * HWd * kHP * 16 : 32 * kHP * 16;
    __shared__ uint4 lds[(kRing * A_BYTES + 2 * H_BYTES + 2 * B_BYTES) / 16];
    char* const ring = reinterpret_cast<char*>(lds);
    char* const halo = ring + kRing * A_BYTES;
    char* const sbias = halo + 2 * H_BYTES;

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave / WGN, wn = wave % WGN;
    const int G = gridDim.x;
    // This workgroup's tiles: first + k*G for the full rounds (first is
    // XCD-aware, so each XCD's L2 sees one run of neighbouring tiles), then at
    // most one of the last round's tiles, spread so that no two of them share
    // a CU.
    const int first = xcd_tile_index();
    if (first >= hg.ntiles) return;
    const int nfull = hg.ntiles / G, nextra = hg.ntiles - nfull * G;
    int e_extra;
    if (G % 8 == 0) {
        const int m = blockIdx.x >> 3;
        e_extra = m % hg.spread == 0 ? (blockIdx.x & 7) + 8 * (m / hg.spread) : nextra;
    } else {
        e_extra = blockIdx.x;
    }
    const int nmine = nfull + (e_extra < nextra ? 1 : 0);
    const int nchunk = (s.cin_g + kBK - 1) / kBK;
    const int wrow = 9 * s.cin_g * 2;  // bytes of one packed weight row

    const __amdgpu_buffer_rsrc_t xr = make_rsrc(x, (uint32_t)s.N * s.H * s.W * s.Cin * 2u);
    const __amdgpu_buffer_rsrc_t wr = make_rsrc(wp, (uint32_t)s.Cout * (uint32_t)wrow);
    const __amdgpu_buffer_rsrc_t yr = make_rsrc(y, (uint32_t)s.N * s.Ho * s.Wo * s.Cout * 2u);
    const __amdgpu_buffer_rsrc_t br = make_rsrc(bias, BIAS ? (uint32_t)s.Cout * 4u : 0u);

    // ---- per-lane constants
    int a_row[AV], a_c[AV], a_lds[AV];
#pragma unroll
    for (int i = 0; i < AV; ++i) {
        const int q = tid + i * NT;
        a_row[i] = q >> 2;
        a_c[i] = (q & 3) * 8;
        a_lds[i] = swz<kBK>(q >> 2, q & 3) * 16;
    }
    const int frow = lane & 31, fch = lane >> 5;
    // first-slice and second-slice weight operand offsets of MFMA row block 0
    // (row blocks i are i * 32 rows = i * 2048 bytes further)
    const int a_rd0 = swz<kBK>(wm * WTM + frow, fch) * 16;
    const int a_rd1 = swz<kBK>(wm * WTM + frow, 2 + fch) * 16;
    // pixel operand offset at tap (0, 0) of MFMA column block 0 (block j is
    // j * JSTRIDE bytes further)
    const int p0 = wn * WTN + frow;
    const int b_lane = ((p0 / TW) * HWd + p0 % TW) * (kHP * 16) + fch * 16;
    // halo copies: copy m of this wave writes units base .. base+63 of a halo
    // buffer, base = min(64 k, HU5 - 64) for k = wave + NW*m (the last copies
    // overlap, rewriting the same values, instead of running past the
    // buffer); this lane's unit is window pixel (row, column) and 16-byte
    // piece ch (ch 4 is the padding unit: it reads 0)
    int dm_rc[DPW], dm_base[DPW];
#pragma unroll
    for (int m = 0; m < DPW; ++m) {
        const int kk = wave + NW * m;
        const int base = 64 * kk < HU5 - 64 ? 64 * kk : HU5 - 64;
        const int u = base + lane;
        const int hp = u / kHP, ch = u - hp * kHP;
        const int hr = hp / HWd, hc = hp - hr * HWd;
        dm_rc[m] = hr | (hc << 8) | (ch << 16);
        dm_base[m] = base * 16;
    }

    // weight-load offsets of a tile (row within this group's channels, else past the end)
    auto a_offsets = [&](const TileXY& T, int* vo) {
#pragma unroll
        for (int i = 0; i < AV; ++i) {
            const int co = T.ct * BM + a_row[i];
            vo[i] = co < s.cout_g ? ((T.g * s.cout_g + co) * wrow + a_c[i] * 2) : kOOB;
        }
    };

    // copy m of channel chunk C of tile T into the halo buffer at DST (VALID
    // false: the copy is still issued, with every lane reading 0, so that
    // each step issues the same loads on every path and the compiler's load
    // counting stays exact)
    // (DST is deliberately not a restrict parameter: the copies then carry
    // only the alias scope of the chunk function's buffer argument, which
    // the compiler's load-wait tracking can follow for a few scopes at a
    // time; a scope per inlined copy would exhaust it and make every LDS
    // access wait for all copies in flight)
    auto h3_copy = [&](char* dst, const TileXY& T, int C, int m, bool valid) {
        const int rc = dm_rc[m];
        const int hr = rc & 255, hc = (rc >> 8) & 255, ch = rc >> 16;
        const int hi = T.ho0 - s.pad + hr, wi = T.wo0 - s.pad + hc;
        const bool ok = valid && ch < 4 && (unsigned)hi < (unsigned)s.H && (unsigned)wi < (unsigned)s.W &&
                        (CFULL || C * kBK + ch * 8 < s.cin_g);
        const int off = ok ? (((T.n * s.H + hi) * s.W + wi) * s.Cin + T.g * s.cin_g + ch * 8) * 2 : kOOB;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(xr, (halo_lds_t)(dst + dm_base[m]), 16, off,
                                                 __builtin_amdgcn_readfirstlane(C * kBK * 2), 0, 0);
    };

#define TILE_OF(KK) ((KK) < nfull ? first + (KK) * G : nfull * G + e_extra)
    TileXY tc = tile_xy<TH, TW>(TILE_OF(0), hg, s.groups);
    TileXY tn = tile_xy<TH, TW>(TILE_OF(nmine > 1 ? 1 : 0), hg, s.groups);
    int hsel = 0;

    f32x16 acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) acc[i][j] = f32x16{};

    uint4 ra[3][AV];           // weight register sets (step % 3)
    uint4 bv = make_uint4(0, 0, 0, 0);  // the next tile's bias piece
    bf16x8 af0[TM], bf0[TN], af1[TM], bf1[TN];

#define A3_LOAD(RA, VO, C, TAP)                                                              \
    do {                                                                                     \
        const int so_ = __builtin_amdgcn_readfirstlane(((TAP) * s.cin_g + (C) * kBK) * 2);  \
        _Pragma("unroll") for (int i = 0; i < AV; ++i) {                                     \
            const bool ok_ = CFULL || (C) * kBK + a_c[i] < s.cin_g;                          \
            (RA)[i] = load16(wr, ok_ ? (VO)[i] : kOOB, so_);                                 \
        }                                                                                    \
    } while (0)
#define A3_STORE(RG, RA, SLOT)                                                               \
    do {                                                                                     \
        _Pragma("unroll") for (int i = 0; i < AV; ++i)                                       \
            *reinterpret_cast<uint4*>((RG) + (SLOT) * A_BYTES + a_lds[i]) = (RA)[i];         \
    } while (0)

    // ---- prologue: weight steps 0, 1 in ring slots 0, 1; step 2's weights in
    // flight (set 2); the first chunk's halo window and the first tile's bias
    // in LDS; the first slice's operands of step 0 read
    int a_vo_c[AV], a_vo_n[AV];  // weight offsets of the current and the next chunk's tile
    a_offsets(tc, a_vo_c);
    {
        uint4 p0r[AV], p1r[AV];
        A3_LOAD(p0r, a_vo_c, 0, 0);
        A3_LOAD(p1r, a_vo_c, 0, 1);
        uint4 pb = make_uint4(0, 0, 0, 0);
        const bool bin = BIAS && tid * 4 < BM;
        if (BIAS) pb = load16(br, bin ? ((tc.g * s.cout_g + tc.ct * BM + tid * 4) * 4) : kOOB);
        A3_LOAD(ra[2], a_vo_c, 0, 2);
        A3_STORE(ring, p0r, 0);
        A3_STORE(ring, p1r, 1);
        if (bin) *reinterpret_cast<uint4*>(sbias + tid * 16) = pb;
#pragma unroll
        for (int m = 0; m < DPW; ++m) h3_copy(halo, tc, 0, m, true);
    }
    // every load of the prologue has landed (this wave's copies included),
    // then the barrier for everyone's.  Nothing of the prologue stays in
    // flight into the tile loop: the compiler merges the loop's entry and
    // back-edge states, and a prologue load still pending at the entry made
    // it wait at every tile start for all but the last few epilogue stores of
    // the previous tile.
    __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0)
    __syncthreads();
    {
        const char* ab = ring + a_rd0;
        const char* bb = halo + b_lane;
#pragma unroll
        for (int i = 0; i < TM; ++i) af0[i] = *reinterpret_cast<const bf16x8*>(ab + i * 2048);
#pragma unroll
        for (int j = 0; j < TN; ++j) bf0[j] = *reinterpret_cast<const bf16x8*>(bb + j * JSTRIDE);
    }

    // One tap T (a literal 0..8) of the current chunk; RG ring, HC / HX the
    // current / next halo buffer, SB the bias buffers.
#define TAPOFF(T) ((((T) / 3) * DIL * HWd + ((T) % 3) * DIL) * (kHP * 16))
#define HALO3_STEP(T)                                                                        \
    do {                                                                                     \
        /* (1) loads: weights of step + 3; halo copies / the next tile's bias */             \
        if ((T) + 3 < 9) A3_LOAD(ra[(T) % 3], a_vo_c, c, (T) + 3);                           \
        else A3_LOAD(ra[(T) % 3], a_vo_n, cn, (T) + 3 - 9);                                  \
        if ((T) < NPS) {                                                                     \
            _Pragma("unroll") for (int p = 0; p < DPS; ++p)                                  \
                if ((T) * DPS + p < DPW) h3_copy(HX, hn, cn, (T) * DPS + p, h_ok);           \
        } else if ((T) == NPS) {                                                             \
            const bool bin_ = BIAS && last_chunk && k + 1 < nmine && tid * 4 < BM;           \
            bv = load16(br, bin_ ? ((tn.g * s.cout_g + tn.ct * BM + tid * 4) * 4) : kOOB);   \
        }                                                                                    \
        __builtin_amdgcn_sched_barrier(0);                                                   \
        /* (2) second slice's operands of this step */                                       \
        {                                                                                    \
            const char* ab_ = (RG) + ((T) % 3) * A_BYTES + a_rd1;                            \
            const char* bb_ = (HC) + b_lane + TAPOFF(T) + 32;                                \
            _Pragma("unroll") for (int i = 0; i < TM; ++i)                                   \
                af1[i] = *reinterpret_cast<const bf16x8*>(ab_ + i * 2048);                   \
            _Pragma("unroll") for (int j = 0; j < TN; ++j)                                   \
                bf1[j] = *reinterpret_cast<const bf16x8*>(bb_ + j * JSTRIDE);                \
        }                                                                                    \
        __builtin_amdgcn_sched_barrier(0);                                                   \
        /* (3) first slice's matrix ops */                                                   \
        _Pragma("unroll") for (int i = 0; i < TM; ++i)                                       \
            _Pragma("unroll") for (int j = 0; j < TN; ++j)                                   \
                acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af0[i], bf0[j], acc[i][j], 0, 0, 0); \
        /* (4) next step's first-slice operands; second slice's matrix ops */                \
        {                                                                                    \
            const char* ab_ = (RG) + (((T) + 1) % 3) * A_BYTES + a_rd0;                      \
            const char* bb_ = (T) + 1 < 9 ? (HC) + b_lane + TAPOFF((T) + 1 < 9 ? (T) + 1 : 0) \
                                          : (HX) + b_lane;                                   \
            _Pragma("unroll") for (int i = 0; i < TM; ++i)                                   \
                af0[i] = *reinterpret_cast<const bf16x8*>(ab_ + i * 2048);                   \
            _Pragma("unroll") for (int j = 0; j < TN; ++j)                                   \
                bf0[j] = *reinterpret_cast<const bf16x8*>(bb_ + j * JSTRIDE);                \
        }                                                                                    \
        _Pragma("unroll") for (int i = 0; i < TM; ++i)                                       \
            _Pragma("unroll") for (int j = 0; j < TN; ++j)                                   \
                acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af1[i], bf1[j], acc[i][j], 0, 0, 0); \
        __builtin_amdgcn_sched_barrier(0);                                                   \
        /* (5) LDS stores: weights of step + 2; the bias loaded last step */                 \
        A3_STORE(RG, ra[((T) + 2) % 3], ((T) + 2) % 3);                                      \
        if ((T) == NPS + 1 && BIAS && last_chunk && k + 1 < nmine && tid * 4 < BM)           \
            *reinterpret_cast<uint4*>((SB) + ((k + 1) & 1) * B_BYTES + tid * 16) = bv;       \
        /* the next chunk's halo copies have landed before the barrier closing tap 7 */      \
        if ((T) == 7) __builtin_amdgcn_s_waitcnt(0x0f70 | AV);                               \
        halo_barrier();                                                                      \
    } while (0)

    const int half = lane >> 5;
    for (int k = 0; k < nmine; ++k) {
        // accumulators start at the tile's bias (its rows of the current bias
        // buffer), so the epilogue only applies ReLU and rounds
#pragma unroll
        for (int i = 0; i < TM; ++i) {
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                float4 b4 = make_float4(0.f, 0.f, 0.f, 0.f);
                if (BIAS)
                    b4 = *reinterpret_cast<const float4*>(sbias + (k & 1) * B_BYTES +
                                                          (wm * WTM + i * 32 + 8 * q + 4 * half) * 4);
#pragma unroll
                for (int j = 0; j < TN; ++j) {
                    acc[i][j][4 * q + 0] = b4.x;
                    acc[i][j][4 * q + 1] = b4.y;
                    acc[i][j][4 * q + 2] = b4.z;
                    acc[i][j][4 * q + 3] = b4.w;
                }
            }
        }
        for (int c = 0; c < nchunk; ++c) {
            // chunk state: the next chunk (its tile, channel chunk, validity)
            const bool last_chunk = c + 1 == nchunk;
            const int cn = last_chunk ? 0 : c + 1;
            const TileXY hn = last_chunk ? tn : tc;
            const bool h_ok = !last_chunk || k + 1 < nmine;
            if (last_chunk) a_offsets(tn, a_vo_n);
            else {
                _Pragma("unroll") for (int i = 0; i < AV; ++i) a_vo_n[i] = a_vo_c[i];
            }
            // the chunk's nine steps, with each LDS buffer a restrict argument
            auto chunk = [&](char* __restrict__ RG, const char* __restrict__ HC, char* __restrict__ HX,
                             char* __restrict__ SB) __attribute__((always_inline)) {
                HALO3_STEP(0);
                HALO3_STEP(1);
                HALO3_STEP(2);
                HALO3_STEP(3);
                HALO3_STEP(4);
                HALO3_STEP(5);
                HALO3_STEP(6);
                HALO3_STEP(7);
                HALO3_STEP(8);
            };
            chunk(ring, halo + hsel * H_BYTES, halo + (hsel ^ 1) * H_BYTES, sbias);
            hsel ^= 1;
        }
        // the tile is done: ReLU, bf16, store; then the next tile
        tile_epilogue<TM, TN, WTM, WTN, TH, TW, false, RELU>(acc, sbias, yr, s, tc, tc.ct * BM, wm, wn, lane);
        tc = tn;
        tn = tile_xy<TH, TW>(TILE_OF(k + 2 < nmine ? k + 2 : 0), hg, s.groups);
#pragma unroll
        for (int i = 0; i < AV; ++i) a_vo_c[i] = a_vo_n[i];
    }
#undef TILE_OF
#undef A3_LOAD
#undef A3_STORE
#undef TAPOFF
#undef HALO3_STEP
}

// Tile choice and launch parameters of one call; `ok` false when this
// kernel does not take the shape.
struct HaloPlan {
    bool ok;
    int cfg;        // 0: M128, 1: M64
    bool shape_b;   // second pixel-block shape of the configuration
    bool ke5;       // effective filter extent above 3: the larger halo buffers
    HaloGrid hg;
};

template <int NT, int MINB, int BM, int WGM, int WGN, int THA, int TWA, int THB, int TWB>
HaloPlan plan_cfg(const Shape& s, int cfg) {
    static_assert(THA * TWA == THB * TWB, "equal pixel blocks");
    HaloPlan p{};
    p.cfg = cfg;
    const long long pa = (long long)((s.Ho + THA - 1) / THA * THA) * ((s.Wo + TWA - 1) / TWA * TWA);
    const long long pb = (long long)((s.Ho + THB - 1) / THB * THB) * ((s.Wo + TWB - 1) / TWB * TWB);
    p.shape_b = pb < pa;
    p.ke5 = (s.Kh - 1) * s.dil + 1 > 3 || (s.Kw - 1) * s.dil + 1 > 3;
    const int TH = p.shape_b ? THB : THA, TW = p.shape_b ? TWB : TWA;
    const int HWd = TW + (s.Kw - 1) * s.dil, HH = TH + (s.Kh - 1) * s.dil;
    const int hunits = HH * HWd * 4;
    p.hg.nparts = (hunits + NT - 1) / NT;
    p.hg.hwd_magic = (65536 + HWd - 1) / HWd;
    p.hg.tiles_h = (s.Ho + TH - 1) / TH;
    p.hg.tiles_w = (s.Wo + TW - 1) / TW;
    p.hg.n_ctiles = (s.cout_g + BM - 1) / BM;
    const long long tiles = (long long)s.N * p.hg.tiles_h * p.hg.tiles_w * s.groups * p.hg.n_ctiles;
    p.hg.ntiles = (int)(tiles > 0x7fffffffLL ? 0 : tiles);
    p.hg.spread = 1;
    // row = (pixel * magic) >> 16 must be exact over the window
    bool magic_ok = true;
    for (int hp = 0; hp < HH * HWd && magic_ok; ++hp) magic_ok = ((hp * p.hg.hwd_magic) >> 16) == hp / HWd;
    // halo pieces are loaded at taps 0..nparts-1 (the bias at tap nparts),
    // stored one tap later, and read by the operand prefetch of the chunk's
    // last tap
    p.ok = tiles > 0 && tiles <= 0x7fffffffLL && magic_ok && s.Kh * s.Kw >= p.hg.nparts + 2;
    return p;
}

HaloPlan make_plan(const Shape& s) {
    HaloPlan p{};
    const long long xbytes = (long long)s.N * s.H * s.W * s.Cin * 2;
    const long long ybytes = (long long)s.N * s.Ho * s.Wo * s.Cout * 2;
    if (!(s.stride == 1 && (s.Kh - 1) * s.dil + 1 <= kKEmax && (s.Kw - 1) * s.dil + 1 <= kKEmax &&
          s.cin_g % 8 == 0 && s.cout_g % 4 == 0 && s.cout_g > 32 &&
          xbytes < 0x7fff0000LL && ybytes < 0x7fff0000LL))
        return p;
    if (s.cout_g > 64) return plan_cfg<HALO_CFG_M128>(s, 0);
    return plan_cfg<HALO_CFG_M64>(s, 1);
}

template <int NT, int MINB, int BM, int TH, int TW, int WGM, int WGN, int KE, bool CFULL, bool BIAS, bool RELU>
hipError_t launch_k(const Shape& s, const HaloGrid& hg, const bf16_t* x, const bf16_t* w,
                    const float* b, bf16_t* y, hipStream_t st) {
    auto kern = halo_kernel<NT, MINB, BM, TH, TW, WGM, WGN, KE, CFULL, BIAS, RELU>;
    int dev = 0;
    (void)hipGetDevice(&dev);
    const long long resident = persistent_slots(
        (long long)cu_count(dev) * blocks_per_cu<halo_kernel<NT, MINB, BM, TH, TW, WGM, WGN, KE, CFULL, BIAS, RELU>>(NT, dev));
    const int grid = (int)(hg.ntiles < resident ? hg.ntiles : resident);
    hipLaunchKernelGGL(kern, dim3(grid), dim3(NT), 0, st, x, w, b, y, s, hg);
    return hipGetLastError();
}

template <int NT, int MINB, int BM, int TH, int TW, int WGM, int WGN, int KE, bool CFULL>
hipError_t launch_epi(const Shape& s, const HaloGrid& hg, const bf16_t* x, const bf16_t* w,
                      const float* b, bf16_t* y, hipStream_t st) {
    const bool bias = s.epilogue & CONV2D_EPI_BIAS, relu = s.epilogue & CONV2D_EPI_RELU;
    if (bias && relu) return launch_k<NT, MINB, BM, TH, TW, WGM, WGN, KE, CFULL, true, true>(s, hg, x, w, b, y, st);
    if (bias) return launch_k<NT, MINB, BM, TH, TW, WGM, WGN, KE, CFULL, true, false>(s, hg, x, w, b, y, st);
    if (relu) return launch_k<NT, MINB, BM, TH, TW, WGM, WGN, KE, CFULL, false, true>(s, hg, x, w, b, y, st);
    return launch_k<NT, MINB, BM, TH, TW, WGM, WGN, KE, CFULL, false, false>(s, hg, x, w, b, y, st);
}

template <int NT, int MINB, int BM, int WGM, int WGN, int TH, int TW>
hipError_t launch_shape(const Shape& s, const HaloPlan& p, const bf16_t* x, const bf16_t* w,
                        const float* b, bf16_t* y, hipStream_t st) {
    const bool full = s.cin_g % kBK == 0;
    if (p.ke5) {
        if (full) return launch_epi<NT, MINB, BM, TH, TW, WGM, WGN, 5, true>(s, p.hg, x, w, b, y, st);
        return launch_epi<NT, MINB, BM, TH, TW, WGM, WGN, 5, false>(s, p.hg, x, w, b, y, st);
    }
    if (full) return launch_epi<NT, MINB, BM, TH, TW, WGM, WGN, 3, true>(s, p.hg, x, w, b, y, st);
    return launch_epi<NT, MINB, BM, TH, TW, WGM, WGN, 3, false>(s, p.hg, x, w, b, y, st);
}

template <int NT, int MINB, int BM, int TH, int TW, int WGM, int WGN, int DIL, bool CFULL, bool BIAS, bool RELU>
hipError_t launch3_k(const Shape& s, const HaloGrid& hg, const bf16_t* x, const bf16_t* w,
                     const float* b, bf16_t* y, hipStream_t st) {
    auto kern = halo3_kernel<NT, MINB, BM, TH, TW, WGM, WGN, DIL, CFULL, BIAS, RELU>;
    int dev = 0;
    (void)hipGetDevice(&dev);
    const int bpc = blocks_per_cu<halo3_kernel<NT, MINB, BM, TH, TW, WGM, WGN, DIL, CFULL, BIAS, RELU>>(NT, dev);
    const long long resident = persistent_slots((long long)cu_count(dev) * bpc);
    const int grid = (int)(hg.ntiles < resident ? hg.ntiles : resident);
    // Workgroups go round-robin over the 8 XCDs and, within one, fill every
    // CU once before any CU takes a second: the last round's tiles go to
    // every spread-th first-round workgroup of each XCD.
    HaloGrid h = hg;
    const int per_xcd = grid / 8, extra = hg.ntiles % grid;
    const int slots = per_xcd / (bpc > 0 ? bpc : 1), want = (extra + 7) / 8;
    h.spread = (grid % 8 == 0 && want > 0 && slots / want > 1) ? slots / want : 1;
    hipLaunchKernelGGL(kern, dim3(grid), dim3(NT), 0, st, x, w, b, y, s, h);
    return hipGetLastError();
}

template <int NT, int MINB, int BM, int TH, int TW, int WGM, int WGN, int DIL, bool CFULL>
hipError_t launch3_epi(const Shape& s, const HaloGrid& hg, const bf16_t* x, const bf16_t* w,
                       const float* b, bf16_t* y, hipStream_t st) {
    const bool bias = s.epilogue & CONV2D_EPI_BIAS, relu = s.epilogue & CONV2D_EPI_RELU;
    if (bias && relu) return launch3_k<NT, MINB, BM, TH, TW, WGM, WGN, DIL, CFULL, true, true>(s, hg, x, w, b, y, st);
    if (bias) return launch3_k<NT, MINB, BM, TH, TW, WGM, WGN, DIL, CFULL, true, false>(s, hg, x, w, b, y, st);
    if (relu) return launch3_k<NT, MINB, BM, TH, TW, WGM, WGN, DIL, CFULL, false, true>(s, hg, x, w, b, y, st);
    return launch3_k<NT, MINB, BM, TH, TW, WGM, WGN, DIL, CFULL, false, false>(s, hg, x, w, b, y, st);
}

template <int NT, int MINB, int BM, int WGM, int WGN, int TH, int TW>
hipError_t launch3_shape(const Shape& s, const HaloPlan& p, const bf16_t* x, const bf16_t* w,
                         const float* b, bf16_t* y, hipStream_t st) {
    const bool full = s.cin_g % kBK == 0;
    if (s.dil == 2) {
        if (full) return launch3_epi<NT, MINB, BM, TH, TW, WGM, WGN, 2, true>(s, p.hg, x, w, b, y, st);
        return launch3_epi<NT, MINB, BM, TH, TW, WGM, WGN, 2, false>(s, p.hg, x, w, b, y, st);
    }
    if (full) return launch3_epi<NT, MINB, BM, TH, TW, WGM, WGN, 1, true>(s, p.hg, x, w, b, y, st);
    return launch3_epi<NT, MINB, BM, TH, TW, WGM, WGN, 1, false>(s, p.hg, x, w, b, y, st);
}

// 3x3 with dilation 1 or 2: the kernel with the taps unrolled.
bool is_3x3(const Shape& s) { return s.Kh == 3 && s.Kw == 3 && (s.dil == 1 || s.dil == 2); }

template <int NT, int MINB, int BM, int WGM, int WGN, int THA, int TWA, int THB, int TWB>
hipError_t launch_cfg(const Shape& s, const HaloPlan& p, const bf16_t* x, const bf16_t* w,
                      const float* b, bf16_t* y, hipStream_t st) {
    if (is_3x3(s)) {
        if (p.shape_b) return launch3_shape<NT, MINB, BM, WGM, WGN, THB, TWB>(s, p, x, w, b, y, st);
        return launch3_shape<NT, MINB, BM, WGM, WGN, THA, TWA>(s, p, x, w, b, y, st);
    }
    if (p.shape_b) return launch_shape<NT, MINB, BM, WGM, WGN, THB, TWB>(s, p, x, w, b, y, st);
    return launch_shape<NT, MINB, BM, WGM, WGN, THA, TWA>(s, p, x, w, b, y, st);
}

}  // namespace

bool igemm_halo_supports(const Shape& s) { return make_plan(s).ok || halo_s2_supports(s); }
bool igemm_halo_auto(const Shape& s) { return make_plan(s).ok; }

hipError_t launch_igemm_halo(const Shape& s, const void* x, const void* w_packed, const float* bias,
                             void* y, hipStream_t st) {
    if (s.stride == 2) return launch_halo_s2(s, x, w_packed, bias, y, st);
    (void)hipGetLastError();  // report only this launch's error
    const HaloPlan p = make_plan(s);
    if (!p.ok) return hipErrorInvalidValue;
    const bf16_t* xt = static_cast<const bf16_t*>(x);
    const bf16_t* wt = static_cast<const bf16_t*>(w_packed);
    bf16_t* yt = static_cast<bf16_t*>(y);
    if (p.cfg == 0) return launch_cfg<HALO_CFG_M128>(s, p, xt, wt, bias, yt, st);
    return launch_cfg<HALO_CFG_M64>(s, p, xt, wt, bias, yt, st);
}

}  // namespace conv2d
