// separable.hip -- the depthwise-separable block in one kernel: a 3x3
// depthwise convolution with its bias and ReLU, then a 1x1 convolution, bf16
// NHWC.
//
// lincklin.cn lesson 9, section 25 factors a standard convolution into a
// per-channel 3x3 filter followed by a 1x1 channel mix (also lpnh.cn section
// 4.1; lnrq.cn section 3.1).  Run as two layers, the depthwise output
// (N*Ho*Wo*C values) is written to HBM and read back by the 1x1 layer.  Here
// a workgroup computes the depthwise output of a band of RB output rows x CW
// columns, for all C channels, into LDS, applies the 1x1 convolution to it on
// the matrix cores and writes only the Cout final channels: the intermediate
// never leaves the CU, and the whole block reads x once and writes y once.
//
// Depthwise phase.  Thread t owns 4 channels, group t % (C/4) (their 3x3
// taps stay in its registers for the whole kernel; 4 rather than 8 channels
// keep a thread within the register budget of four waves per SIMD), and the
// band's output columns t / (C/4) + j * (NT / (C/4)).  For each column it
// loads the band's input rows (consecutive threads load consecutive 8-byte
// pieces of one row, so every wave's loads are coalesced; the neighbouring
// columns a tap needs come through L1), runs the row arithmetic of dwrow.hpp
// and writes the RB output pieces into the LDS tile [pixel][channel] (odd
// pitch of 16-byte units).  The value is rounded to bf16 after the depthwise bias and ReLU:
// the value a separate depthwise layer would store, so the fused result is
// the two-layer chain's.
//
// Pointwise phase.  Each wave takes 32-pixel tiles of the band.  The weights
// [Cout][C] sit in LDS for the whole kernel; v_mfma_f32_32x32x16_bf16 per 32
// output channels and 16 input channels, fp32 accumulators initialised with
// the bias; the register epilogue (ReLU, bf16, two lane swaps) stores 16
// bytes per lane, every pixel's channels contiguous.
#include "dwrow.hpp"
#include "../../include/conv2d.h"

namespace conv2d {

namespace {

using namespace dwrow;

constexpr int kSepThreads = 512;
constexpr int kSepWaves = kSepThreads / 64;
constexpr int kSepMaxC = 256;
constexpr int kSepMaxCout = 128;
constexpr int kSepKS = kSepMaxC / 16;  // 16-channel slices of the widest input

// LDS row pitch in 16-byte units: odd (conflict-free operand reads), and at
// least two units per 16-channel slice so that the second half of the last
// slice is a zero unit inside the row when C % 16 == 8.
__host__ __device__ constexpr int sep_pitch(int c) { return (2 * ((c + 15) / 16)) | 1; }

struct SepGrid {
    int N, C, H, W, Ho, Wo, Cout, pad;
    int CW;       // output columns per band
    int nrb, ncb;  // row bands and column chunks per image
    int nitems;   // N * nrb * ncb
    int ptiles;   // 32-pixel tiles of one band
    int dw_bias, dw_relu, pw_bias, pw_relu;
};

// S: depthwise stride; RB: output rows per band; MB: 32-row blocks of
// pointwise output channels (Cout <= 32 * MB).
template <int S, int RB, int MB>
__global__ __launch_bounds__(kSepThreads, 4) void sep_kernel(const bf16_t* __restrict__ x,
                                                         const bf16_t* __restrict__ wdw,  // [3][3][C]
                                                         const float* __restrict__ bdw,
                                                         const bf16_t* __restrict__ wpw,  // [Cout][C]
                                                         const float* __restrict__ bpw,
                                                         bf16_t* __restrict__ y, SepGrid g) {
    constexpr int NR = (RB - 1) * S + 3;  // input rows of a band
    constexpr int ROWS = MB * 32;
    // dynamic LDS: pointwise weights [ROWS][P], then the band's depthwise
    // output [ptiles * 32 pixels][P]
    extern __shared__ uint4 sep_lds[];
    __shared__ __align__(16) float sbp[kSepMaxCout];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int C = g.C, C8 = C >> 3, P = sep_pitch(C);
    uint4* const wl = sep_lds;
    uint4* const dl = sep_lds + ROWS * P;

    // pointwise weights (rows past Cout and units past C are zero): all loads
    // first, then the LDS stores
    {
        constexpr int kU = (ROWS * sep_pitch(kSepMaxC) + kSepThreads - 1) / kSepThreads;
        const __amdgpu_buffer_rsrc_t wr = make_rsrc(wpw, (uint32_t)g.Cout * (uint32_t)C * 2u);
        uint4 v[kU];
#pragma unroll
        for (int k = 0; k < kU; ++k) {
            const int u = tid + k * kSepThreads;
            const int r = u / P, c = u - r * P;
            v[k] = load16(wr, (u < ROWS * P && r < g.Cout && c < C8) ? (r * C + c * 8) * 2 : kOOB);
        }
#pragma unroll
        for (int k = 0; k < kU; ++k) {
            const int u = tid + k * kSepThreads;
            if (u < ROWS * P) wl[u] = v[k];
        }
    }
    for (int i = tid; i < ROWS; i += kSepThreads) sbp[i] = (g.pw_bias && i < g.Cout) ? bpw[i] : 0.0f;
    // the pad units of every pixel of the depthwise tile are never written
    // by the depthwise phase: zero them once
    for (int p = tid; p < g.ptiles * 32; p += kSepThreads)
        for (int u = C8; u < P; ++u) dl[p * P + u] = make_uint4(0, 0, 0, 0);

    // depthwise taps and bias of this thread's 4 channels
    const int C4 = C >> 2;
    const int cpp = kSepThreads / C4;  // columns per pass
    const int cg = tid % C4, cpos = tid / C4;
    uint32_t wp[3][4];
    float w2[3][4], b0[4];
    load_taps<2>(wdw, C, cg * 4, wp, w2);
#pragma unroll
    for (int i = 0; i < 4; ++i) b0[i] = g.dw_bias ? bdw[cg * 4 + i] : 0.0f;

    const __amdgpu_buffer_rsrc_t xr = make_rsrc(x, (uint32_t)g.N * g.H * g.W * C * 2u);
    const __amdgpu_buffer_rsrc_t yr = make_rsrc(y, (uint32_t)g.N * g.Ho * g.Wo * g.Cout * 2u);
    const int rstride = g.W * C * 2;

    // pointwise operands: weight row frow of block mb, unit 2s + h; pixel
    // frow of tile T, unit 2s + h
    const int frow = lane & 31, h = lane >> 5;
    const char* const a_base = reinterpret_cast<const char*>(wl) + (frow * P + h) * 16;
    const char* const b_base = reinterpret_cast<const char*>(dl) + (frow * P + h) * 16;
    // epilogue: this lane's 16-byte piece holds channels cl .. cl+7 of a
    // 32-channel block, of pixel 16 e + lane % 16 (e = 0, 1) of the tile
    const int cl = ((lane >> 4) & 1) * 16 + h * 8;
    const bool vec16 = g.Cout % 8 == 0;

    // consecutive logical blocks (those of one XCD) take consecutive bands,
    // which share their halo rows in that XCD's L2
    for (int item = xcd_tile_index(); item < g.nitems; item += gridDim.x) {
        const int cb = item % g.ncb, t = item / g.ncb;
        const int rb = t % g.nrb, n = t / g.nrb;
        const int ho0 = rb * RB, wo0 = cb * g.CW;
        __syncthreads();  // the previous band's pointwise reads (and the set-up stores) are done

        if (cpos < cpp) {
            const int img = n * g.H * g.W * C + cg * 4;
            const int hb = ho0 * S - g.pad;  // input row of filter row 0 for output row ho0
            for (int c = cpos; c < g.CW; c += cpp) {
                const int wi0 = (wo0 + c) * S - g.pad;
                int coff[3];
#pragma unroll
                for (int k = 0; k < 3; ++k)
                    coff[k] = ((unsigned)(wi0 + k) < (unsigned)g.W) ? (img + (wi0 + k) * C) * 2 : kOOB;
                V4 raw[NR][3];
#pragma unroll
                for (int i = 0; i < NR; ++i) {
                    const bool rin = (unsigned)(hb + i) < (unsigned)g.H;
#pragma unroll
                    for (int k = 0; k < 3; ++k)
                        raw[i][k] = load_v4(xr, (rin && coff[k] != kOOB) ? coff[k] + (hb + i) * rstride : kOOB);
                }
                RowXN<2> rx[NR];
#pragma unroll
                for (int i = 0; i < NR; ++i) prep_row(raw[i][0], raw[i][1], raw[i][2], rx[i]);
#pragma unroll
                for (int r = 0; r < RB; ++r) {
                    float acc[4];
#pragma unroll
                    for (int i = 0; i < 4; ++i) acc[i] = b0[i];
                    row_fma(acc, rx[r * S + 0], wp[0], w2[0]);
                    row_fma(acc, rx[r * S + 1], wp[1], w2[1]);
                    row_fma(acc, rx[r * S + 2], wp[2], w2[2]);
                    uint2 o;
                    float a[4];
#pragma unroll
                    for (int i = 0; i < 4; ++i) a[i] = g.dw_relu ? fmaxf(acc[i], 0.0f) : acc[i];
                    o.x = pack_bf16x2(a[0], a[1]);
                    o.y = pack_bf16x2(a[2], a[3]);
                    // 8-byte half cg & 1 of 16-byte unit cg / 2 of the pixel's row
                    reinterpret_cast<uint2*>(dl)[(r * g.CW + c) * P * 2 + cg] = o;
                }
            }
        }
        __syncthreads();

        // output-channel blocks two at a time (64 accumulators at most, next
        // to the depthwise taps that stay live)
        constexpr int MBG = MB < 2 ? MB : 2;
        for (int T = wave; T < g.ptiles; T += kSepWaves) {
            // output pixel of each half of the tile, or -1 past the band or the image
            int pix[2];
#pragma unroll
            for (int e = 0; e < 2; ++e) {
                const int p = T * 32 + 16 * e + (lane & 15);
                const int r = p / g.CW, c = p - r * g.CW;
                const bool ok = r < RB && ho0 + r < g.Ho && wo0 + c < g.Wo;
                pix[e] = ok ? ((n * g.Ho + ho0 + r) * g.Wo + wo0 + c) * g.Cout : -1;
            }
#pragma unroll 1
            for (int m0 = 0; m0 < MB; m0 += MBG) {
                f32x16 acc[MBG];
#pragma unroll
                for (int mb = 0; mb < MBG; ++mb)
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        const float4 b4 = *reinterpret_cast<const float4*>(&sbp[(m0 + mb) * 32 + 8 * q + 4 * h]);
                        acc[mb][4 * q + 0] = b4.x;
                        acc[mb][4 * q + 1] = b4.y;
                        acc[mb][4 * q + 2] = b4.z;
                        acc[mb][4 * q + 3] = b4.w;
                    }
                // slices past C are skipped (their weight reads would run past a row)
#pragma unroll
                for (int s = 0; s < kSepKS; ++s) {
                    if (s * 16 < C) {
                        const bf16x8 b = *reinterpret_cast<const bf16x8*>(b_base + (T * 32 * P + 2 * s) * 16);
#pragma unroll
                        for (int mb = 0; mb < MBG; ++mb) {
                            const bf16x8 a =
                                *reinterpret_cast<const bf16x8*>(a_base + ((m0 + mb) * 32 * P + 2 * s) * 16);
                            acc[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[mb], 0, 0, 0);
                        }
                    }
                }
#pragma unroll
                for (int mb = 0; mb < MBG; ++mb) {
                    uint32_t pk[4][2];
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        float v[4];
#pragma unroll
                        for (int r = 0; r < 4; ++r) {
                            v[r] = acc[mb][4 * q + r];
                            if (g.pw_relu) v[r] = fmaxf(v[r], 0.0f);
                        }
                        pk[q][0] = pack_bf16x2(v[0], v[1]);
                        pk[q][1] = pack_bf16x2(v[2], v[3]);
                    }
                    // D rows 8q + 4(lane/32) + r -> per lane 8 consecutive
                    // channels of one pixel: swap the upper half of the wave
                    // with the lower (32), then the 16-lane rows
                    uint32_t r8[2][4];
#pragma unroll
                    for (int pr = 0; pr < 2; ++pr)
#pragma unroll
                        for (int w = 0; w < 2; ++w) {
                            const auto sw =
                                __builtin_amdgcn_permlane32_swap(pk[2 * pr][w], pk[2 * pr + 1][w], false, false);
                            r8[pr][w] = sw[0];
                            r8[pr][2 + w] = sw[1];
                        }
                    uint32_t o[2][4];
#pragma unroll
                    for (int d = 0; d < 4; ++d) {
                        const auto sw = __builtin_amdgcn_permlane16_swap(r8[0][d], r8[1][d], false, false);
                        o[0][d] = sw[0];
                        o[1][d] = sw[1];
                    }
                    const int co = (m0 + mb) * 32 + cl;
#pragma unroll
                    for (int e = 0; e < 2; ++e) {
                        const int off = (pix[e] + co) * 2;
                        if (vec16) {
                            store16(yr, pix[e] >= 0 && co < g.Cout ? off : kOOB,
                                    make_uint4(o[e][0], o[e][1], o[e][2], o[e][3]));
                        } else {
                            store8(yr, pix[e] >= 0 && co < g.Cout ? off : kOOB, make_uint2(o[e][0], o[e][1]));
                            store8(yr, pix[e] >= 0 && co + 4 < g.Cout ? off + 8 : kOOB,
                                   make_uint2(o[e][2], o[e][3]));
                        }
                    }
                }
            }
        }
    }
}

// Rows per band: four at stride 1 (6 input rows for 4 output rows), two at
// stride 2 (5 for 2).
constexpr int sep_rows(int stride) { return stride == 1 ? 4 : 2; }

struct SepPlan {
    bool ok;
    int mb;
    long long lds;  // dynamic LDS bytes
    SepGrid g;
};

SepPlan sep_plan(const SepShape& s) {
    SepPlan pl{};
    pl.ok = false;
    if (s.C % 8 || s.C > kSepMaxC || s.Cout % 4 || s.Cout > kSepMaxCout) return pl;
    if (s.stride != 1 && s.stride != 2) return pl;
    if ((long long)s.N * s.H * s.W * s.C * 2 >= 0x7fff0000LL) return pl;
    if ((long long)s.N * s.Ho * s.Wo * s.Cout * 2 >= 0x7fff0000LL) return pl;
    const int RB = sep_rows(s.stride);
    const int mb = s.Cout <= 32 ? 1 : s.Cout <= 64 ? 2 : 4;
    const long long unit = (long long)sep_pitch(s.C) * 16;  // bytes per pixel row of LDS
    const long long wbytes = (long long)mb * 32 * unit;
    // two workgroups per CU if a band of at least one column fits, else one
    int cw = 0;
    for (int per_cu = 2; per_cu >= 1 && cw < 1; --per_cu) {
        const long long budget = 163840 / per_cu - kSepMaxCout * 4;
        const long long px = (budget - wbytes) / unit / 32 * 32;
        cw = (int)(px / RB < s.Wo ? px / RB : s.Wo);
    }
    if (cw < 1) return pl;
    const int ncb = (s.Wo + cw - 1) / cw;
    cw = (s.Wo + ncb - 1) / ncb;  // even the column chunks out
    SepGrid& g = pl.g;
    g.N = s.N; g.C = s.C; g.H = s.H; g.W = s.W; g.Ho = s.Ho; g.Wo = s.Wo; g.Cout = s.Cout; g.pad = s.pad;
    g.CW = cw;
    g.ncb = ncb;
    g.nrb = (s.Ho + RB - 1) / RB;
    const long long items = (long long)s.N * g.nrb * g.ncb;
    if (items >= 0x7fffffffLL) return pl;
    g.nitems = (int)items;
    g.ptiles = (RB * cw + 31) / 32;
    g.dw_bias = (s.dw_epilogue & CONV2D_EPI_BIAS) ? 1 : 0;
    g.dw_relu = (s.dw_epilogue & CONV2D_EPI_RELU) ? 1 : 0;
    g.pw_bias = (s.pw_epilogue & CONV2D_EPI_BIAS) ? 1 : 0;
    g.pw_relu = (s.pw_epilogue & CONV2D_EPI_RELU) ? 1 : 0;
    pl.mb = mb;
    pl.lds = wbytes + (long long)g.ptiles * 32 * unit;
    pl.ok = pl.lds + kSepMaxCout * 4 <= 163840;
    return pl;
}

template <int S, int MB>
hipError_t launch_sep(const SepPlan& pl, const bf16_t* x, const bf16_t* wdw, const float* bdw, const bf16_t* wpw,
                      const float* bpw, bf16_t* y, hipStream_t st) {
    auto kern = sep_kernel<S, sep_rows(S), MB>;
    int dev = 0;
    (void)hipGetDevice(&dev);
    static bool attr_set[64] = {};
    if (dev >= 0 && dev < 64 && !attr_set[dev]) {
        const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                                 hipFuncAttributeMaxDynamicSharedMemorySize,
                                                 163840 - kSepMaxCout * 4);
        if (e != hipSuccess) return e;
        attr_set[dev] = true;
    }
    const int by_regs = blocks_per_cu<sep_kernel<S, sep_rows(S), MB>>(kSepThreads, dev);
    const int by_lds = (int)(163840 / (pl.lds + kSepMaxCout * 4));
    const int bpc = by_lds < by_regs ? (by_lds < 1 ? 1 : by_lds) : by_regs;
    const long long resident = (long long)cu_count(dev) * bpc;
    const int grid = (int)(pl.g.nitems < resident ? pl.g.nitems : resident);
    hipLaunchKernelGGL(kern, dim3(grid), dim3(kSepThreads), (unsigned)pl.lds, st, x, wdw, bdw, wpw, bpw, y, pl.g);
    return hipGetLastError();
}

template <int S>
hipError_t launch_sep_mb(const SepPlan& pl, const bf16_t* x, const bf16_t* wdw, const float* bdw,
                         const bf16_t* wpw, const float* bpw, bf16_t* y, hipStream_t st) {
    if (pl.mb == 1) return launch_sep<S, 1>(pl, x, wdw, bdw, wpw, bpw, y, st);
    if (pl.mb == 2) return launch_sep<S, 2>(pl, x, wdw, bdw, wpw, bpw, y, st);
    return launch_sep<S, 4>(pl, x, wdw, bdw, wpw, bpw, y, st);
}

}  // namespace

bool separable_supports(const SepShape& s) { return sep_plan(s).ok; }

hipError_t launch_separable(const SepShape& s, const void* x, const void* w_dw, const float* b_dw,
                            const void* w_pw, const float* b_pw, void* y, hipStream_t st) {
    (void)hipGetLastError();  // report only this launch's error
    const SepPlan pl = sep_plan(s);
    if (!pl.ok) return hipErrorInvalidValue;
    const bf16_t* xt = static_cast<const bf16_t*>(x);
    const bf16_t* wd = static_cast<const bf16_t*>(w_dw);
    const bf16_t* wq = static_cast<const bf16_t*>(w_pw);
    bf16_t* yt = static_cast<bf16_t*>(y);
    if (s.stride == 1) return launch_sep_mb<1>(pl, xt, wd, b_dw, wq, b_pw, yt, st);
    return launch_sep_mb<2>(pl, xt, wd, b_dw, wq, b_pw, yt, st);
}

}  // namespace conv2d
