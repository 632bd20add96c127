// igemm_halo.hip -- implicit-GEMM convolution for stride 1 with the input
// staged once per channel chunk as a halo tile in LDS.
//
// Same GEMM as the gather kernel (lincklin.cn lesson 9, sections 7, 11, 19):
// per group, D[co][p] = sum_k W[co][k] * X_col[k][p] with k = (ci, kh, kw).
// What changes is where X_col comes from.  A workgroup owns BM output
// channels x a TH x TW block of output pixels of one image.  For stride 1
// every tap of that block reads inside one (TH + (Kh-1)D) x (TW + (Kw-1)D)
// input window -- the block plus its halo (lincklin.cn section 12: a 16x16
// output tile of a 3x3 filter needs an 18x18 input tile).  The window is
// loaded from HBM/L2 once per 32-channel chunk into LDS (section 13: load
// the tile cooperatively, synchronise, let every thread read its windows),
// and each of the Kh*Kw taps then reads its B operand from that tile at a
// fixed offset (kh*D rows, kw*D columns): input reuse across taps happens in
// LDS instead of through the vector-memory path.  Dilation is only a larger
// offset, so exactly the Kh*Kw real taps are gathered (lpnh.cn section 4.2).
// Zero padding: window pixels outside the image are loaded as 0
// (lincklin.cn section 26).
//
// K loop: chunk (32 input channels) outer, tap inner.  Per step the BM x 32
// weight slice of (tap, chunk) is staged in LDS (double-buffered, loaded one
// step ahead); the next chunk's halo tile is requested at the chunk's first
// tap and written to the other halo buffer a few taps later.  Matrix cores:
// v_mfma_f32_32x32x16_bf16, fp32 accumulators in registers for the whole K
// loop (output stationary), fused bias + ReLU + bf16 rounding, results
// staged through LDS so each pixel's channels are stored contiguously.
#include "mfma.hpp"
#include "../../include/conv2d.h"

namespace conv2d {

namespace {

// Tile configurations per range of output channels per group: threads,
// BM output channels, WGM x WGN waves, two equal-size pixel-block shapes
// (rows x columns).  Overridable at build time for tuning sweeps.
#ifndef HALO_CFG_M256
#define HALO_CFG_M256 512, 256, 2, 4, 16, 16, 8, 32
#endif
#ifndef HALO_CFG_M128
#define HALO_CFG_M128 256, 128, 2, 2, 16, 16, 8, 32
#endif
#ifndef HALO_CFG_M64
#define HALO_CFG_M64 256, 64, 1, 4, 16, 16, 8, 32
#endif

constexpr int kBK = 32;    // input channels per chunk: one 64-byte LDS row per pixel
constexpr int kKEmax = 5;  // largest effective filter extent (Kh-1)*D+1 the halo buffer holds

// Halo tile layout in LDS: one window pixel = 5 16-byte units (80 bytes:
// its 4 chunks of 8 channels plus one unit of padding).  Because 5 is odd,
// any 16 consecutive window pixels read at the same chunk fall in 16 distinct
// 16-byte bank slots (conflict-free ds_read_b128), and moving to another tap
// is a plain additive offset of (kh*D*width + kw*D) * 80 bytes.
constexpr int kHP = 5;

// Largest divisor of n that is <= cap (0 if none).
constexpr int largest_divisor_upto(int n, int cap) {
    for (int d = cap < n ? cap : n; d >= 1; --d)
        if (n % d == 0) return d;
    return 0;
}

template <int NT, int BM, int TH, int TW, int WGM, int WGN, bool CFULL, bool BIAS, bool RELU>
__global__ __launch_bounds__(NT) void halo_kernel(const bf16_t* __restrict__ x,
                                                  const bf16_t* __restrict__ wp,
                                                  const float* __restrict__ bias,
                                                  bf16_t* __restrict__ y, Shape s,
                                                  int tiles_h, int tiles_w, int n_ctiles) {
    constexpr int BN = TH * TW;
    static_assert(WGM * WGN * 64 == NT, "one wave per sub-tile");
    constexpr int WTM = BM / WGM, WTN = BN / WGN;
    constexpr int TM = WTM / 32, TN = WTN / 32;
    static_assert(TM * 32 == WTM && TN * 32 == WTN, "32x32 MFMA tiles");
    constexpr int HCAP = (TH + kKEmax - 1) * (TW + kKEmax - 1);  // halo pixels per buffer
    constexpr int A_UNITS = BM * 4;                              // 16-byte units per weight stage
    constexpr int H_UNITS = HCAP * kHP;                          // 16-byte units per halo buffer
    constexpr int AV = A_UNITS / NT;
    static_assert(AV * NT == A_UNITS, "weight stage splits evenly");
    constexpr int HV = (HCAP * 4 + NT - 1) / NT;
    constexpr int PIPE_UNITS = 2 * A_UNITS + 2 * H_UNITS;
    constexpr int ERS = BM * 2 + 16;  // epilogue LDS row stride in bytes (one pixel)
    constexpr int EPW0 = (PIPE_UNITS * 16 / ERS) / WTN;  // wave columns that fit one pass
    constexpr int EPW = largest_divisor_upto(WGN, EPW0);
    static_assert(EPW >= 1 && WGN % EPW == 0, "epilogue pass fits LDS");
    constexpr int NPASS = WGN / EPW;
    __shared__ uint4 lds[PIPE_UNITS];
    __shared__ __align__(16) float sbias[BM];  // this tile's bias, read by the epilogue
    uint4* const abuf = lds;                // [2][A_UNITS]
    uint4* const hbuf = lds + 2 * A_UNITS;  // [2][H_UNITS]

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave / WGN, wn = wave % WGN;

    int tile = xcd_tile_index();
    const int ct = tile % n_ctiles;  // output-channel tile (fastest)
    tile /= n_ctiles;
    const int g = tile % s.groups;
    tile /= s.groups;
    const int tw = tile % tiles_w;   // pixel blocks in row-major order over each image
    tile /= tiles_w;
    const int th = tile % tiles_h;
    const int n = tile / tiles_h;
    const int ho0 = th * TH, wo0 = tw * TW;
    const int HH = TH + (s.Kh - 1) * s.dil;   // halo window extent (stride 1)
    const int HWd = TW + (s.Kw - 1) * s.dil;
    const int KK = s.Kh * s.Kw;
    const int nchunk = (s.cin_g + kBK - 1) / kBK;
    const int co_tile = ct * BM;

    const __amdgpu_buffer_rsrc_t xr = make_rsrc(x, (uint32_t)s.N * s.H * s.W * s.Cin * 2u);
    const __amdgpu_buffer_rsrc_t wr = make_rsrc(wp, (uint32_t)s.Cout * KK * s.cin_g * 2u);

    // ---- weight (A) slots: row = output channel, 4 chunks of 8 channels;
    // byte offset of (tap 0, chunk 0), or past the end for a missing channel
    int a_off[AV], a_c[AV], a_lds[AV];
#pragma unroll
    for (int i = 0; i < AV; ++i) {
        const int q = tid + i * NT;
        const int row = q >> 2, ch = q & 3;
        const int co = co_tile + row;
        const bool ok = co < s.cout_g;
        a_off[i] = ok ? ((g * s.cout_g + co) * KK * s.cin_g + ch * 8) * 2 : kOOB;
        a_c[i] = ch * 8;
        a_lds[i] = swz<kBK>(row, ch);
    }
    // ---- halo (B) slots: window pixel hp, chunk ch; byte offset of the
    // pixel's channel block of chunk 0, or past the end outside the image
    int h_off[HV], h_c[HV], h_lds[HV];
    const int hunits = HH * HWd * 4;
#pragma unroll
    for (int k = 0; k < HV; ++k) {
        const int v = tid + k * NT;
        const int hp = v >> 2, ch = v & 3;
        const int hr = hp / HWd, hc = hp - hr * HWd;
        const int hi = ho0 - s.pad + hr, wi = wo0 - s.pad + hc;
        const bool in = v < hunits && (unsigned)hi < (unsigned)s.H && (unsigned)wi < (unsigned)s.W;
        h_off[k] = in ? (((n * s.H + hi) * s.W + wi) * s.Cin + g * s.cin_g + ch * 8) * 2 : kOOB;
        h_c[k] = ch * 8;
        h_lds[k] = v < hunits ? hp * kHP + ch : -1;
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
        const int r = p / TW, cc = p - r * TW;
        b_rd[j] = ((r * HWd + cc) * kHP + fch) * 16;
    }

    f32x16 acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) acc[i][j] = f32x16{};

    uint4 ra[AV], rh[HV];
    // With Cin/G a multiple of 32 every chunk is full: the offsets need no
    // per-lane check and the step's offset rides in the scalar field.
#define HALO_LOAD(CH)                                                                        \
    do {                                                                                     \
        _Pragma("unroll") for (int k = 0; k < HV; ++k) {                                     \
            if (CFULL) {                                                                     \
                rh[k] = load16(xr, h_off[k], (CH) * kBK * 2);                                \
            } else {                                                                         \
                const bool ok = (CH) * kBK + h_c[k] < s.cin_g;                               \
                rh[k] = load16(xr, ok ? h_off[k] : kOOB, (CH) * kBK * 2);                    \
            }                                                                                \
        }                                                                                    \
    } while (0)
#define HALO_STORE(BUF)                                                                      \
    do {                                                                                     \
        _Pragma("unroll") for (int k = 0; k < HV; ++k)                                       \
            if (h_lds[k] >= 0) hbuf[(BUF) * H_UNITS + h_lds[k]] = rh[k];                     \
    } while (0)
#define A_LOAD(CH, TAP)                                                                      \
    do {                                                                                     \
        _Pragma("unroll") for (int i = 0; i < AV; ++i) {                                     \
            if (CFULL) {                                                                     \
                ra[i] = load16(wr, a_off[i], ((TAP) * s.cin_g + (CH) * kBK) * 2);            \
            } else {                                                                         \
                const bool ok = (CH) * kBK + a_c[i] < s.cin_g;                               \
                ra[i] = load16(wr, ok ? a_off[i] : kOOB, ((TAP) * s.cin_g + (CH) * kBK) * 2); \
            }                                                                                \
        }                                                                                    \
    } while (0)
#define A_STORE(BUF)                                                                         \
    do {                                                                                     \
        _Pragma("unroll") for (int i = 0; i < AV; ++i) abuf[(BUF) * A_UNITS + a_lds[i]] = ra[i]; \
    } while (0)

    HALO_LOAD(0);
    A_LOAD(0, 0);
    if (BIAS) {
        // stage the tile's bias once (visible after the barrier below)
        for (int i = tid; i < BM; i += NT)
            sbias[i] = co_tile + i < s.cout_g ? bias[g * s.cout_g + co_tile + i] : 0.0f;
    }
    HALO_STORE(0);
    A_STORE(0);
    __syncthreads();

    // K loop: chunk outer, tap (kh, kw) inner.  Past the last step the weight
    // prefetch reads harmless in-range or zero data that is never used.
    int st = 0;
    for (int c = 0; c < nchunk; ++c) {
        const char* hcur = reinterpret_cast<const char*>(hbuf + (c & 1) * H_UNITS);
        int t = 0;
        for (int kh = 0; kh < s.Kh; ++kh) {
            for (int kw = 0; kw < s.Kw; ++kw, ++t, ++st) {
                const bool last_tap = t + 1 == KK;
                // Halo loads go out before the weight loads of the same step:
                // loads complete in order, so the wait for the weights also
                // covers them.  The next chunk's halo has the whole chunk to
                // arrive and is stored at its last tap.
                if (t == 0 && c + 1 < nchunk) HALO_LOAD(c + 1);
                if (last_tap) A_LOAD(c + 1, 0);
                else A_LOAD(c, t + 1);
                // keep the loads a full step ahead of their LDS stores
                __builtin_amdgcn_sched_barrier(0);
                const char* acur = reinterpret_cast<const char*>(abuf + (st & 1) * A_UNITS);
                const char* hb = hcur + (kh * s.dil * HWd + kw * s.dil) * (kHP * 16);
                // Both K slices' operands are requested before any matrix
                // op, so the second slice's LDS reads overlap the first
                // slice's MFMAs.
                bf16x8 af[2][TM], bfr[2][TN];
#pragma unroll
                for (int ks = 0; ks < 2; ++ks) {
#pragma unroll
                    for (int i = 0; i < TM; ++i)
                        af[ks][i] = *reinterpret_cast<const bf16x8*>(acur + a_rd[ks][i]);
#pragma unroll
                    for (int j = 0; j < TN; ++j)
                        bfr[ks][j] = *reinterpret_cast<const bf16x8*>(hb + b_rd[j] + ks * 32);
                }
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int ks = 0; ks < 2; ++ks)
#pragma unroll
                    for (int i = 0; i < TM; ++i)
#pragma unroll
                        for (int j = 0; j < TN; ++j)
                            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[ks][i], bfr[ks][j], acc[i][j], 0, 0, 0);
                A_STORE((st + 1) & 1);
                if (last_tap && c + 1 < nchunk) HALO_STORE((c + 1) & 1);
                __syncthreads();
            }
        }
    }
#undef HALO_LOAD
#undef HALO_STORE
#undef A_LOAD
#undef A_STORE

    // ---- epilogue: bias, ReLU, bf16 in registers; staged through LDS as
    // [pixel][channel] rows in NPASS passes over the wave columns, then each
    // pixel's channels leave as contiguous 16-byte stores.
    // 32x32 result layout: lane l holds D[8*q + 4*(l/32) + r][l % 32] in
    // acc[4*q + r]: four runs of four consecutive channels of one pixel.
    char* ep = reinterpret_cast<char*>(lds);
    const bool vec16 = (s.Cout % 8 == 0) && (s.cout_g % 8 == 0);
    constexpr int RCH = BM / 8;
    constexpr int PPX = EPW * WTN;  // pixels per pass
#pragma unroll 1
    for (int pass = 0; pass < NPASS; ++pass) {
        if (wn / EPW == pass) {
#pragma unroll
            for (int i = 0; i < TM; ++i) {
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int col = wm * WTM + i * 32 + 8 * q + 4 * (lane >> 5);
                    const int co = co_tile + col;
                    float4 b4 = make_float4(0.f, 0.f, 0.f, 0.f);
                    if (BIAS) b4 = *reinterpret_cast<const float4*>(&sbias[col]);
                    (void)co;
#pragma unroll
                    for (int j = 0; j < TN; ++j) {
                        const int row = (wn % EPW) * WTN + j * 32 + (lane & 31);
                        float v[4];
#pragma unroll
                        for (int r = 0; r < 4; ++r) {
                            v[r] = acc[i][j][4 * q + r] + (&b4.x)[r];
                            if (RELU) v[r] = fmaxf(v[r], 0.0f);
                        }
                        *reinterpret_cast<uint2*>(ep + row * ERS + col * 2) =
                            make_uint2(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]));
                    }
                }
            }
        }
        __syncthreads();
        for (int q = tid; q < PPX * RCH; q += NT) {
            const int row = q / RCH, cch = q - row * RCH;
            const int p = pass * PPX + row;
            const int r = p / TW, cc = p - r * TW;
            const int ho = ho0 + r, wo = wo0 + cc;
            const int co = co_tile + cch * 8;
            if (ho >= s.Ho || wo >= s.Wo || co >= s.cout_g) continue;
            const uint4 v = *reinterpret_cast<const uint4*>(ep + row * ERS + cch * 16);
            bf16_t* dst = y + ((size_t)(n * s.Ho + ho) * s.Wo + wo) * s.Cout + g * s.cout_g + co;
            if (vec16 && co + 8 <= s.cout_g) {
                *reinterpret_cast<uint4*>(dst) = v;
            } else {
                *reinterpret_cast<uint2*>(dst) = make_uint2(v.x, v.y);
                if (co + 8 <= s.cout_g) *reinterpret_cast<uint2*>(dst + 4) = make_uint2(v.z, v.w);
            }
        }
        __syncthreads();
    }
}

template <int NT, int BM, int TH, int TW, int WGM, int WGN, bool CFULL>
hipError_t launch_tile(const Shape& s, const bf16_t* x, const bf16_t* w, const float* b, bf16_t* y,
                       hipStream_t st) {
    const int tiles_h = (s.Ho + TH - 1) / TH, tiles_w = (s.Wo + TW - 1) / TW;
    const int n_ctiles = (s.cout_g + BM - 1) / BM;
    const long long blocks = (long long)s.N * tiles_h * tiles_w * s.groups * n_ctiles;
    if (blocks > 0x7fffffffLL) return hipErrorInvalidConfiguration;
    dim3 grid((unsigned)blocks);
    const bool bias = s.epilogue & CONV2D_EPI_BIAS, relu = s.epilogue & CONV2D_EPI_RELU;
    if (bias && relu)
        hipLaunchKernelGGL((halo_kernel<NT, BM, TH, TW, WGM, WGN, CFULL, true, true>), grid, dim3(NT), 0, st, x, w, b, y, s, tiles_h, tiles_w, n_ctiles);
    else if (bias)
        hipLaunchKernelGGL((halo_kernel<NT, BM, TH, TW, WGM, WGN, CFULL, true, false>), grid, dim3(NT), 0, st, x, w, b, y, s, tiles_h, tiles_w, n_ctiles);
    else if (relu)
        hipLaunchKernelGGL((halo_kernel<NT, BM, TH, TW, WGM, WGN, CFULL, false, true>), grid, dim3(NT), 0, st, x, w, b, y, s, tiles_h, tiles_w, n_ctiles);
    else
        hipLaunchKernelGGL((halo_kernel<NT, BM, TH, TW, WGM, WGN, CFULL, false, false>), grid, dim3(NT), 0, st, x, w, b, y, s, tiles_h, tiles_w, n_ctiles);
    return hipGetLastError();
}

template <int NT, int BM, int WGM, int WGN, int THA, int TWA, int THB, int TWB>
hipError_t launch_shape(const Shape& s, const bf16_t* x, const bf16_t* w, const float* b, bf16_t* y,
                        hipStream_t st) {
    static_assert(THA * TWA == THB * TWB, "equal pixel blocks");
    const bool full = s.cin_g % kBK == 0;
    const long long pa = (long long)((s.Ho + THA - 1) / THA * THA) * ((s.Wo + TWA - 1) / TWA * TWA);
    const long long pb = (long long)((s.Ho + THB - 1) / THB * THB) * ((s.Wo + TWB - 1) / TWB * TWB);
    if (pb < pa) {
        if (full) return launch_tile<NT, BM, THB, TWB, WGM, WGN, true>(s, x, w, b, y, st);
        return launch_tile<NT, BM, THB, TWB, WGM, WGN, false>(s, x, w, b, y, st);
    }
    if (full) return launch_tile<NT, BM, THA, TWA, WGM, WGN, true>(s, x, w, b, y, st);
    return launch_tile<NT, BM, THA, TWA, WGM, WGN, false>(s, x, w, b, y, st);
}

}  // namespace

bool igemm_halo_supports(const Shape& s) {
    const long long xbytes = (long long)s.N * s.H * s.W * s.Cin * 2;
    return s.stride == 1 && (s.Kh - 1) * s.dil + 1 <= kKEmax && (s.Kw - 1) * s.dil + 1 <= kKEmax &&
           s.cin_g % 8 == 0 && s.cout_g % 4 == 0 && s.cout_g > 32 && xbytes < 0x7fff0000LL;
}

hipError_t launch_igemm_halo(const Shape& s, const void* x, const void* w_packed, const float* bias,
                             void* y, hipStream_t st) {
    (void)hipGetLastError();  // report only this launch's error
    const bf16_t* xt = static_cast<const bf16_t*>(x);
    const bf16_t* wt = static_cast<const bf16_t*>(w_packed);
    bf16_t* yt = static_cast<bf16_t*>(y);
    if (s.cout_g > 128) return launch_shape<HALO_CFG_M256>(s, xt, wt, bias, yt, st);
    if (s.cout_g > 64) return launch_shape<HALO_CFG_M128>(s, xt, wt, bias, yt, st);
    return launch_shape<HALO_CFG_M64>(s, xt, wt, bias, yt, st);
}

}  // namespace conv2d
