// igemm.hip -- implicit-GEMM convolution on gfx950 bf16 MFMA, and the 1x1
// convolution as a plain GEMM.
//
// GEMM view (lincklin.cn lesson 9, sections 7 and 19): per group g,
//   D[co][p] = sum_k  A[co][k] * B[k][p]
//   M = Cout/G (output channels), N = N*Ho*Wo (output pixels),
//   K = Kh*Kw*Cin/G ordered (kh, kw, ci) with ci fastest,
//   A = packed weight [Cout][Kh][Kw][Cin/G] (K-contiguous rows),
//   B[k][p] = X[n, hi, wi, g*Cin/G + ci] with hi = ho*S + kh*D - P,
//             wi = wo*S + kw*D - P, and 0 outside the image.
// B is never stored: its addresses are generated while the tile is loaded
// (implicit GEMM, lincklin.cn section 11; lpnh.cn section 3.3).  With
// channels-last input the Cin/G values of one tap are contiguous, so each
// K-step of 32 channels of one tap is a 64-byte contiguous read per pixel.
// Dilation only changes the tap offsets (kh*D, kw*D): exactly Kh*Kw taps are
// gathered, never a zero-filled dilated window (lpnh.cn section 4.2).  Zero
// padding is the address predicate (lincklin.cn section 26).
//
// Tiling.  A workgroup of 4 waves owns a BM x BN output tile (BM output
// channels x BN pixels) of one group.  Per K-step (one tap, 32 channels) it
// stages the BM x 32 weight slice and the BN x 32 im2col slice in LDS
// (double-buffered: the next step's global loads are in flight while the
// current step runs on the matrix cores), and each wave runs
// v_mfma_f32_32x32x16_bf16 on its (BM/WGM) x (BN/WGN) sub-tile.  fp32
// accumulators stay in registers for the whole K loop (output stationary,
// lincklin.cn section 15) and the epilogue adds the bias, applies ReLU,
// rounds to bf16 and stores once (lincklin.cn section 31).
//
// 1x1 / stride 1 / pad 0 / groups 1 (lincklin.cn sections 21-22; lpnh.cn
// section 4.3): B[k][p] = X[p][k], the NHWC activation read as a row-major
// [N*H*W][Cin] matrix -- a plain GEMM with no window arithmetic.
//
// Transposed convolution (lpnh.cn sections 2.3 and 4.2: the stride-1
// convolution of the input with S-1 zeros inserted between neighbouring
// pixels).  Most taps of that convolution meet an inserted zero.  Which taps
// do not depends only on the output pixel's phase (oh mod S, ow mod S): for
// the outputs oh = ph + S*u, tap kh reaches input row (oh + P - kh*D)/S when
// kh*D = (ph + P) mod S, i.e. for kh = k0, k0 + S/gcd(S,D), ...; the input
// row is then u + base - j*D/gcd(S,D) for the j-th such tap.  Each workgroup
// therefore owns one phase and runs the same implicit GEMM over only that
// phase's taps (per axis about K/S of them), on the packed weight
// [Cout][Kh][Kw][Cin/G] of the transposed weight; its output pixels sit S
// apart in the output.
#include "mfma.hpp"
#include "../../include/conv2d.h"

namespace conv2d {

namespace {

// Tile shapes (BM output channels, BN pixels, WGM x WGN waves, BK channels
// per K-step) per range of
// output channels per group; overridable at build time for tuning sweeps.
#ifndef IGEMM_TILE_M256
#define IGEMM_TILE_M256 128, 128, 2, 2, 64
#endif
#ifndef IGEMM_TILE_M128
#define IGEMM_TILE_M128 128, 128, 2, 2, 64
#endif
#ifndef IGEMM_TILE_M64
#define IGEMM_TILE_M64 64, 256, 1, 4, 64
#endif
#ifndef IGEMM_TILE_M32
#define IGEMM_TILE_M32 32, 256, 1, 4, 32
#endif

constexpr int kThreads = 256;

// What the implicit GEMM computes: a convolution, the 1x1 plain GEMM, or one
// output phase of a transposed convolution.
enum Mode { kConv = 0, kGemm1x1 = 1, kTransposed = 2 };

// The taps of one output phase along one axis (transposed convolution):
// taps k0 + j*kstep for j < n; tap j reads input u + base + j*d for the
// phase's output u.
struct TapAxis {
    int n, k0, kstep, base, d;
};

__device__ __forceinline__ TapAxis tap_axis(int ph, int K, int S, int P, int D) {
    TapAxis a;
    const int r = (ph + P) % S;
    int k0 = -1;
    for (int k = 0; k < S && k < K; ++k)
        if ((k * D) % S == r) { k0 = k; break; }
    int gcd = S, b = D;  // gcd(S, D)
    while (b) { const int t = gcd % b; gcd = b; b = t; }
    a.kstep = S / gcd;
    a.n = k0 < 0 ? 0 : (K - 1 - k0) / a.kstep + 1;
    a.k0 = k0 < 0 ? 0 : k0;
    a.base = (ph + P) / S - (a.k0 * D) / S;
    a.d = -(D / gcd);
    return a;
}

template <int BM, int BN, int WGM, int WGN, int BK, int MODE, bool BIAS, bool RELU>
__global__ __launch_bounds__(kThreads) void igemm_kernel(const bf16_t* __restrict__ x,
                                                         const bf16_t* __restrict__ wp,
                                                         const float* __restrict__ bias,
                                                         bf16_t* __restrict__ y, Shape s,
                                                         int n_ptiles, int n_ctiles) {
    static_assert(BK == 32 || BK == 64, "K step of 32 or 64 channels");
    constexpr bool IS1X1 = MODE == kGemm1x1, TR = MODE == kTransposed;
    constexpr int kChunks = BK / 8;                // 16-byte chunks per LDS row
    constexpr int KS = BK / 16;                    // MFMA K slices per step
    constexpr int WTM = BM / WGM, WTN = BN / WGN;  // wave tile
    constexpr int TM = WTM / 32, TN = WTN / 32;    // 32x32 MFMA tiles per wave
    constexpr int AQ = BM * kChunks, BQ = BN * kChunks;  // 16-byte vectors per step
    constexpr int AV = (AQ + kThreads - 1) / kThreads, BV = BQ / kThreads;
    static_assert(BQ % kThreads == 0, "B tile must split evenly");
    constexpr int STAGE = (BM + BN) * kChunks;            // 16-byte units per stage
    constexpr int ERS = BM * 2 + 16;                       // epilogue LDS row stride (bytes)
    constexpr int LDS_UNITS = (2 * STAGE > BN * ERS / 16) ? 2 * STAGE : BN * ERS / 16;
    __shared__ uint4 lds_raw[LDS_UNITS];
    __shared__ __align__(16) float sbias[BM];  // this tile's bias, read by the epilogue

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave / WGN, wn = wave % WGN;

    int tile = xcd_tile_index();
    const int ct = tile % n_ctiles;          // output-channel tile (fastest)
    tile /= n_ctiles;
    const int g = tile % s.groups;           // group
    int pt = tile / s.groups;                // pixel tile (slowest)

    // Transposed: the phase (ph_h, ph_w) sits between the group and the pixel
    // tile, so neighbouring workgroups share input rows.  Its pixel grid is
    // N x uh_n x uw_n with output (ph_h + S*uh, ph_w + S*uw).
    int ph_h = 0, ph_w = 0, uh_n = 1, uw_n = 1;
    TapAxis ah = {}, aw = {};
    if constexpr (TR) {
        const int nph = s.stride * s.stride;
        const int ph = pt % nph;
        pt /= nph;
        ph_h = ph / s.stride;
        ph_w = ph % s.stride;
        uh_n = (s.Ho - ph_h + s.stride - 1) / s.stride;
        uw_n = (s.Wo - ph_w + s.stride - 1) / s.stride;
        ah = tap_axis(ph_h, s.Kh, s.stride, s.pad, s.dil);
        aw = tap_axis(ph_w, s.Kw, s.stride, s.pad, s.dil);
    }
    const int npix = TR ? s.N * uh_n * uw_n : s.N * s.Ho * s.Wo;
    if (TR && pt * BN >= npix) return;  // a phase with fewer pixels than the largest (uniform)
    const int KK = s.Kh * s.Kw;                   // taps of the packed weight
    const int ntaps = TR ? ah.n * aw.n : KK;      // taps this workgroup walks
    const int tap_dh = TR ? ah.d : s.dil, tap_dw = TR ? aw.d : s.dil;
    const int ntw = TR ? aw.n : s.Kw;
    const int nchunk = (s.cin_g + BK - 1) / BK;
    const int nsteps = ntaps * nchunk;
    const int co_tile = ct * BM;

    const __amdgpu_buffer_rsrc_t xr = make_rsrc(x, (uint32_t)s.N * s.H * s.W * s.Cin * 2u);
    const __amdgpu_buffer_rsrc_t wr = make_rsrc(wp, (uint32_t)s.Cout * KK * s.cin_g * 2u);

    // ---- per-thread A (weight) slots: byte offset of the row's K start
    int a_off[AV], a_c[AV], a_lds[AV];
#pragma unroll
    for (int i = 0; i < AV; ++i) {
        const int q = tid + i * kThreads;
        const int row = q / kChunks, ch = q % kChunks;
        const int co = co_tile + row;
        const bool ok = (q < AQ) && (co < s.cout_g);
        a_off[i] = ok ? ((g * s.cout_g + co) * KK * s.cin_g + ch * 8) * 2 : kOOB;
        a_c[i] = ok ? ch * 8 : (1 << 29);   // channel of the chunk (huge: never valid)
        a_lds[i] = (q < AQ) ? swz<BK>(row, ch) : 0;
    }
    // ---- per-thread B (im2col) slots
    int b_base[BV], b_hb[BV], b_wb[BV], b_c[BV], b_lds[BV];
#pragma unroll
    for (int i = 0; i < BV; ++i) {
        const int q = tid + i * kThreads;
        const int prow = q / kChunks, ch = q % kChunks;
        const int p = pt * BN + prow;
        const bool ok = p < npix;
        const int pp = ok ? p : 0;
        const int ow_n = TR ? uw_n : s.Wo, oh_n = TR ? uh_n : s.Ho;
        const int wo = pp % ow_n;
        const int t = pp / ow_n;
        const int ho = t % oh_n;
        const int n = t / oh_n;
        if (TR) {
            b_base[i] = n * s.H * s.W * s.Cin + g * s.cin_g + ch * 8;
            b_hb[i] = ok ? ho + ah.base : -(1 << 29);  // never inside the image
            b_wb[i] = wo + aw.base;
        } else if (IS1X1) {
            b_base[i] = pp * s.Cin + ch * 8;
            b_hb[i] = 0;
            b_wb[i] = 0;
        } else {
            b_base[i] = n * s.H * s.W * s.Cin + g * s.cin_g + ch * 8;
            b_hb[i] = ok ? ho * s.stride - s.pad : -(1 << 29);  // never inside the image
            b_wb[i] = wo * s.stride - s.pad;
        }
        b_c[i] = ok ? ch * 8 : (1 << 29);
        b_lds[i] = swz<BK>(BM + prow, ch);
    }

    f32x16 acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) acc[i][j] = f32x16{};

    // Load cursor: the next K-step to fetch, tap (kh, kw) outer, channel chunk
    // inner (for a transposed phase, lkh and lkw count that phase's taps).
    int ltap = 0, lkh = 0, lkw = 0, lc0 = 0;

    // global -> registers for the cursor's K-step, then advance the cursor;
    // out-of-range reads give 0
#define IGEMM_LOAD_STEP(RA, RB)                                                             \
    do {                                                                                    \
        _Pragma("unroll") for (int i = 0; i < AV; ++i) {                                    \
            const bool ok = lc0 + a_c[i] < s.cin_g && ltap < ntaps;                         \
            const int wtap_ = TR ? (ah.k0 + lkh * ah.kstep) * s.Kw + aw.k0 + lkw * aw.kstep  \
                                 : ltap;                                                    \
            RA[i] = load16(wr, ok ? a_off[i] + (wtap_ * s.cin_g + lc0) * 2 : kOOB);         \
        }                                                                                   \
        _Pragma("unroll") for (int i = 0; i < BV; ++i) {                                    \
            int off;                                                                        \
            bool ok = lc0 + b_c[i] < s.cin_g && ltap < ntaps;                               \
            if (IS1X1) {                                                                    \
                off = b_base[i] + lc0;                                                      \
            } else {                                                                        \
                const int hi = b_hb[i] + lkh * tap_dh;                                      \
                const int wi = b_wb[i] + lkw * tap_dw;                                      \
                ok = ok && (unsigned)hi < (unsigned)s.H && (unsigned)wi < (unsigned)s.W;    \
                off = b_base[i] + (hi * s.W + wi) * s.Cin + lc0;                            \
            }                                                                               \
            RB[i] = load16(xr, ok ? off * 2 : kOOB);                                        \
        }                                                                                   \
        lc0 += BK;                                                                          \
        if (lc0 >= s.cin_g) {                                                               \
            lc0 = 0;                                                                        \
            ++ltap;                                                                         \
            if (++lkw == ntw) { lkw = 0; ++lkh; }                                           \
        }                                                                                   \
    } while (0)

#define IGEMM_STORE_STEP(RA, RB, BUF)                                                       \
    do {                                                                                    \
        uint4* st_ = lds_raw + (BUF) * STAGE;                                               \
        _Pragma("unroll") for (int i = 0; i < AV; ++i)                                      \
            if (AQ % kThreads == 0 || tid + i * kThreads < AQ) st_[a_lds[i]] = RA[i];       \
        _Pragma("unroll") for (int i = 0; i < BV; ++i) st_[b_lds[i]] = RB[i];               \
    } while (0)

    // v_mfma_f32_32x32x16_bf16 operands: lane l supplies row (l % 32) and the
    // 8 K values 8*(l / 32) .. +7 of the 16-wide K slice; a BK-wide K step is
    // BK/16 such slices (16-byte chunks 2*ks and 2*ks+1 of the LDS row).
    const int frow = lane & 31, fch = lane >> 5;
    int a_rd[KS][TM], b_rd[KS][TN];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
        for (int i = 0; i < TM; ++i) a_rd[ks][i] = swz<BK>(wm * WTM + i * 32 + frow, 2 * ks + fch);
#pragma unroll
        for (int j = 0; j < TN; ++j) b_rd[ks][j] = swz<BK>(BM + wn * WTN + j * 32 + frow, 2 * ks + fch);
    }

#define IGEMM_COMPUTE(BUF)                                                                  \
    do {                                                                                    \
        const uint4* cur = lds_raw + (BUF) * STAGE;                                         \
        _Pragma("unroll") for (int ks = 0; ks < KS; ++ks) {                                 \
            bf16x8 af[TM], bfr[TN];                                                         \
            _Pragma("unroll") for (int i = 0; i < TM; ++i)                                  \
                af[i] = __builtin_bit_cast(bf16x8, cur[a_rd[ks][i]]);                       \
            _Pragma("unroll") for (int j = 0; j < TN; ++j)                                  \
                bfr[j] = __builtin_bit_cast(bf16x8, cur[b_rd[ks][j]]);                      \
            _Pragma("unroll") for (int i = 0; i < TM; ++i)                                  \
                _Pragma("unroll") for (int j = 0; j < TN; ++j)                              \
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j],      \
                                                                        acc[i][j], 0, 0, 0); \
        }                                                                                   \
    } while (0)

    // Software pipeline, two K-steps of global loads in flight: while LDS
    // stage b holds step st for the matrix cores, the registers of one set
    // hold step st+1 (arriving) and the other set receives step st+2.  The
    // step count is rounded up to even so the loop body has no early exit; the
    // padding step (cursor past the last tap) loads zeros.
    const int nsteps2 = (nsteps + 1) & ~1;
    uint4 ra0[AV], rb0[BV], ra1[AV], rb1[BV];
    IGEMM_LOAD_STEP(ra0, rb0);
    IGEMM_LOAD_STEP(ra1, rb1);
    if (BIAS) {
        // stage the tile's bias once (visible after the barrier below)
        for (int i = tid; i < BM; i += kThreads)
            sbias[i] = co_tile + i < s.cout_g ? bias[g * s.cout_g + co_tile + i] : 0.0f;
    }
    IGEMM_STORE_STEP(ra0, rb0, 0);
    __syncthreads();
    // Loads and stores are unconditional (past the last step they read zeros)
    // so the loop body has no branch and the wait before each LDS store
    // counts exactly the older step's loads.
    // The scheduling fences keep each step's loads ahead of the matrix work
    // (the scheduler would otherwise sink them towards their LDS stores).
    for (int st = 0; st < nsteps2; st += 2) {
        IGEMM_LOAD_STEP(ra0, rb0);
        __builtin_amdgcn_sched_barrier(0);
        IGEMM_COMPUTE(0);
        IGEMM_STORE_STEP(ra1, rb1, 1);
        __syncthreads();
        IGEMM_LOAD_STEP(ra1, rb1);
        __builtin_amdgcn_sched_barrier(0);
        IGEMM_COMPUTE(1);
        IGEMM_STORE_STEP(ra0, rb0, 0);
        __syncthreads();
    }
#undef IGEMM_LOAD_STEP
#undef IGEMM_STORE_STEP
#undef IGEMM_COMPUTE

    // ---- epilogue: bias, ReLU, bf16 rounding in registers; the tile is
    // staged through LDS as [pixel][channel] rows so that every pixel's BM
    // output channels leave as contiguous 16-byte stores.
    // 32x32 MFMA result layout: lane l holds D[8*q + 4*(l/32) + r][l % 32]
    // in acc[16*0 + 4*q + r] for q, r = 0..3, i.e. four runs of four
    // consecutive output channels of one pixel.
    char* ep = reinterpret_cast<char*>(lds_raw);
    const Affine4 aff(s.scale, s.shift, s.Cout);
#pragma unroll
    for (int i = 0; i < TM; ++i) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int col = wm * WTM + i * 32 + 8 * q + 4 * (lane >> 5);  // channel within the tile
            const int co = co_tile + col;
            float4 b4 = make_float4(0.f, 0.f, 0.f, 0.f);
            if (BIAS) b4 = *reinterpret_cast<const float4*>(&sbias[col]);
#pragma unroll
            for (int j = 0; j < TN; ++j) {
                const int row = wn * WTN + j * 32 + (lane & 31);      // pixel within the tile
                float v[4];
#pragma unroll
                for (int r = 0; r < 4; ++r) v[r] = acc[i][j][4 * q + r] + (&b4.x)[r];
                if (s.scale) aff.apply(v, g * s.cout_g + co);
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    if (RELU) v[r] = fmaxf(v[r], 0.0f);
                *reinterpret_cast<uint2*>(ep + row * ERS + col * 2) =
                    make_uint2(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]));
            }
        }
    }
    __syncthreads();
    const bool vec16 = (s.Cout % 8 == 0) && (s.cout_g % 8 == 0);
    constexpr int RCH = BM / 8;   // 16-byte chunks per pixel row of the tile
    for (int q = tid; q < BN * RCH; q += kThreads) {
        const int row = q / RCH, c = q % RCH;
        const int p = pt * BN + row;
        const int co = co_tile + c * 8;
        if (p >= npix || co >= s.cout_g) continue;
        const uint4 v = *reinterpret_cast<const uint4*>(ep + row * ERS + c * 16);
        int opix = p;  // output pixel (n, ho, wo) as one index
        if (TR) {
            const int uw = p % uw_n, t = p / uw_n;
            const int uh = t % uh_n, n = t / uh_n;
            opix = (n * s.Ho + ph_h + s.stride * uh) * s.Wo + ph_w + s.stride * uw;
        }
        bf16_t* dst = y + (size_t)opix * s.Cout + g * s.cout_g + co;
        if (vec16 && co + 8 <= s.cout_g) {
            // streaming (nt) store: written once, never read here; keeps the
            // L2 for the input rows neighbouring tiles re-read (measured
            // 34.5 -> 33.3 us on the 3x3 stride-2 128->128 layer)
            typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));
            __builtin_nontemporal_store(__builtin_bit_cast(u32x4_t, v), reinterpret_cast<u32x4_t*>(dst));
        } else {
            *reinterpret_cast<uint2*>(dst) = make_uint2(v.x, v.y);
            if (co + 8 <= s.cout_g) *reinterpret_cast<uint2*>(dst + 4) = make_uint2(v.z, v.w);
        }
    }
}

template <int BM, int BN, int WGM, int WGN, int BK, int MODE>
hipError_t launch_cfg(const Shape& s, const bf16_t* x, const bf16_t* w, const float* b, bf16_t* y,
                      hipStream_t st) {
    // a transposed convolution: pixel tiles of the largest phase (phase 0), per phase
    const int S = s.stride;
    const long long npix = MODE == kTransposed
                               ? (long long)s.N * ((s.Ho + S - 1) / S) * ((s.Wo + S - 1) / S)
                               : (long long)s.N * s.Ho * s.Wo;
    const long long n_ptiles = (npix + BN - 1) / BN;
    const int n_ctiles = (s.cout_g + BM - 1) / BM;
    const long long blocks = n_ptiles * n_ctiles * s.groups * (MODE == kTransposed ? S * S : 1);
    if (blocks > 0x7fffffffLL) return hipErrorInvalidConfiguration;
    dim3 grid((unsigned)blocks);
    const int npt = (int)n_ptiles;
    const bool bias = s.epilogue & CONV2D_EPI_BIAS, relu = s.epilogue & CONV2D_EPI_RELU;
    if (bias && relu)
        hipLaunchKernelGGL((igemm_kernel<BM, BN, WGM, WGN, BK, MODE, true, true>), grid, dim3(kThreads), 0, st, x, w, b, y, s, npt, n_ctiles);
    else if (bias)
        hipLaunchKernelGGL((igemm_kernel<BM, BN, WGM, WGN, BK, MODE, true, false>), grid, dim3(kThreads), 0, st, x, w, b, y, s, npt, n_ctiles);
    else if (relu)
        hipLaunchKernelGGL((igemm_kernel<BM, BN, WGM, WGN, BK, MODE, false, true>), grid, dim3(kThreads), 0, st, x, w, b, y, s, npt, n_ctiles);
    else
        hipLaunchKernelGGL((igemm_kernel<BM, BN, WGM, WGN, BK, MODE, false, false>), grid, dim3(kThreads), 0, st, x, w, b, y, s, npt, n_ctiles);
    return hipGetLastError();
}

template <int MODE>
hipError_t launch_any(const Shape& s, const void* x, const void* w, const float* b, void* y, hipStream_t st) {
    const bf16_t* xt = static_cast<const bf16_t*>(x);
    const bf16_t* wt = static_cast<const bf16_t*>(w);
    bf16_t* yt = static_cast<bf16_t*>(y);
    // Tile shape by output channels per group: cover them in as few tiles as
    // possible so each input pixel is fetched once per tap for all of them.
    if (s.cout_g > 128) return launch_cfg<IGEMM_TILE_M256, MODE>(s, xt, wt, b, yt, st);
    if (s.cout_g > 64) return launch_cfg<IGEMM_TILE_M128, MODE>(s, xt, wt, b, yt, st);
    if (s.cout_g > 32) return launch_cfg<IGEMM_TILE_M64, MODE>(s, xt, wt, b, yt, st);
    return launch_cfg<IGEMM_TILE_M32, MODE>(s, xt, wt, b, yt, st);
}

bool mfma_channels_ok(const Shape& s) {
    // 16-byte K vectors and 4-channel output stores; zero taps and dropped
    // stores through the out-of-range buffer offset
    return s.cin_g % 8 == 0 && s.cout_g % 4 == 0 && buffer_addressable(s);
}

}  // namespace

bool igemm_supports(const Shape& s) { return mfma_channels_ok(s); }

bool gemm1x1_supports(const Shape& s) {
    return s.Kh == 1 && s.Kw == 1 && s.stride == 1 && s.pad == 0 && s.groups == 1 && mfma_channels_ok(s);
}

hipError_t launch_igemm(const Shape& s, const void* x, const void* w_packed, const float* bias,
                        void* y, hipStream_t st) {
    (void)hipGetLastError();  // report only this launch's error
    return launch_any<kConv>(s, x, w_packed, bias, y, st);
}

hipError_t launch_gemm1x1(const Shape& s, const void* x, const void* w_packed, const float* bias,
                          void* y, hipStream_t st) {
    (void)hipGetLastError();  // report only this launch's error
    return launch_any<kGemm1x1>(s, x, w_packed, bias, y, st);
}

bool igemm_transposed_supports(const Shape& s) { return mfma_channels_ok(s); }

hipError_t launch_igemm_transposed(const Shape& s, const void* x, const void* w_packed, const float* bias,
                                   void* y, hipStream_t st) {
    (void)hipGetLastError();  // report only this launch's error
    return launch_any<kTransposed>(s, x, w_packed, bias, y, st);
}

}  // namespace conv2d
