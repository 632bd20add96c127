// depthwise.hip -- depthwise convolution (groups == Cin == Cout), bf16 NHWC.
//
// Each channel is filtered by its own Kh x Kw kernel with no sum across
// channels (lincklin.cn lesson 9, section 23; lpnh.cn section 4.1), so the
// arithmetic intensity is a few FLOPs per byte and the kernel is bound by HBM
// bandwidth (lincklin.cn section 24).  No MFMA: the work is a handful of FMAs
// per loaded value, kept on the vector ALUs.
//
// Mapping.  A channels-last output row is W*C contiguous bf16 = W*C/8 16-byte
// vectors.  Thread v of the row owns vector v: output column wo = v / (C/8)
// and 8 channels.  Consecutive threads therefore touch consecutive 16-byte
// chunks of memory, so every load and store of a wave is fully coalesced, and
// the horizontal neighbours a tap needs (wo +- 1) are the vectors C/8 lanes
// away, already on their way into L1 for the neighbouring threads.  Each
// thread walks a strip of TH output rows (vertical input reuse).
//
// 3x3 stride-1 dilation-1 (the MobileNet case): the thread keeps the three
// input rows of its window in registers and loads only the one new row per
// output row (3 vector loads per output vector instead of 9; adjacent outputs
// share overlapping windows, lincklin.cn section 18).  Its 9 x 8 filter taps
// stay in registers for the whole strip (lincklin.cn section 14).
//
// Other kernel sizes, strides and dilations: the same mapping, all taps
// loaded per output (dilated taps at kh*D, kw*D only, never a zero-filled
// window; lpnh.cn section 4.2).
#include "dwrow.hpp"
#include "../../include/conv2d.h"

namespace conv2d {

namespace {

using namespace dwrow;

constexpr int kThreads = 256;

__device__ __forceinline__ void fma_v8(float acc[8], const V8& x, const float w[8]) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        acc[2 * i] = fmaf(lo(x.u[i]), w[2 * i], acc[2 * i]);
        acc[2 * i + 1] = fmaf(hi(x.u[i]), w[2 * i + 1], acc[2 * i + 1]);
    }
}

template <bool BIAS, bool RELU>
__device__ __forceinline__ V8 finish(const float acc[8], const float b[8], const float* scale, const float* shift,
                                     int c0) {
    V8 o;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        float a0 = acc[2 * i], a1 = acc[2 * i + 1];
        if (BIAS) { a0 += b[2 * i]; a1 += b[2 * i + 1]; }
        if (scale) {  // folded batch normalisation
            a0 = fmaf(a0, scale[c0 + 2 * i], shift[c0 + 2 * i]);
            a1 = fmaf(a1, scale[c0 + 2 * i + 1], shift[c0 + 2 * i + 1]);
        }
        if (RELU) { a0 = fmaxf(a0, 0.0f); a1 = fmaxf(a1, 0.0f); }
        o.u[i] = pack_bf16x2(a0, a1);
    }
    return o;
}

// 3x3, stride 1, dilation 1, any padding: the row arithmetic of dwrow.hpp.
// The thread's TH + 2 input rows are loaded PF rows ahead of their use (the
// row loop is unrolled at compile time, so every row has registers of its
// own and no register with a pending load is ever moved).  Work items are
// (image, strip of TH rows, 256-vector slice of a row), numbered so that each
// XCD takes one contiguous run of them: the strips of an image that share
// halo rows then read them through one L2.
template <int TH, int PF, bool BIAS, bool RELU>
__global__ __launch_bounds__(kThreads) void dw3x3s1_kernel(const bf16_t* __restrict__ x,
                                                           const bf16_t* __restrict__ w,   // [3][3][C]
                                                           const float* __restrict__ bias,
                                                           bf16_t* __restrict__ y, Shape s) {
    static_assert(PF >= 1 && PF <= TH + 2, "rows in flight");
    const int CV = s.Cin >> 3;                       // 16-byte vectors per pixel
    const int gx = (s.Wo * CV + kThreads - 1) / kThreads, gy = (s.Ho + TH - 1) / TH;
    const int item = xcd_tile_index();
    const int bx = item % gx, t = item / gx;
    const int by = t % gy, n = t / gy;
    const int v = bx * kThreads + threadIdx.x;
    if (n >= s.N || v >= s.Wo * CV) return;
    const int wo = v / CV;
    const int c0 = (v - wo * CV) << 3;
    const int ho0 = by * TH;
    const int ho1 = min(ho0 + TH, s.Ho);

    // weights: per filter row, the (kw0, kw1) pair of each channel and kw2 in fp32
    uint32_t wp[3][8];
    float w2[3][8];
    load_taps<4>(w, s.Cin, c0, wp, w2);
    float b0[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) b0[i] = BIAS ? bias[c0 + i] : 0.0f;

    const __amdgpu_buffer_rsrc_t xr = make_rsrc(x, (uint32_t)s.N * s.H * s.W * s.Cin * 2u);
    // byte offsets of the window's three input columns in row 0 of image n;
    // a column outside the image gets an offset past the end (reads 0)
    const int wi0 = wo - s.pad;
    const int img = n * s.H * s.W * s.Cin + c0;
    int coff[3];
#pragma unroll
    for (int k = 0; k < 3; ++k)
        coff[k] = ((unsigned)(wi0 + k) < (unsigned)s.W) ? (img + (wi0 + k) * s.Cin) * 2 : kOOB;
    const int rstride = s.W * s.Cin * 2;
    const int hb = ho0 - s.pad;  // input row of filter row 0 for output row ho0
    V8 raw[TH + 2][3];
    auto load_row = [&](int r) {
        const int hi_ = hb + r;
#pragma unroll
        for (int k = 0; k < 3; ++k)
            raw[r][k] = load_v8(xr, ((unsigned)hi_ < (unsigned)s.H && coff[k] != kOOB) ? coff[k] + hi_ * rstride
                                                                                        : kOOB);
    };

    bf16_t* yrow = y + ((size_t)n * s.Ho * s.Wo + wo) * s.Cout + c0;
    auto emit = [&](int ho, const RowX& r0, const RowX& r1, const RowX& r2) {
        float acc[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[i] = b0[i];
        row_fma(acc, r0, wp[0], w2[0]);
        row_fma(acc, r1, wp[1], w2[1]);
        row_fma(acc, r2, wp[2], w2[2]);
        if (s.scale) {  // folded batch normalisation
#pragma unroll
            for (int i = 0; i < 8; ++i) acc[i] = fmaf(acc[i], s.scale[c0 + i], s.shift[c0 + i]);
        }
        V8 o;
#pragma unroll
        for (int i = 0; i < 4; ++i) o.u[i] = pack_relu<RELU>(acc[2 * i], acc[2 * i + 1]);
        if (ho < ho1) {
            // streaming (nt) store: the output is written once and not read
            // here (measured 17.3 -> 16.1 us on the 144-channel layer)
            typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));
            __builtin_nontemporal_store(__builtin_bit_cast(u32x4_t, o),
                                        reinterpret_cast<u32x4_t*>(yrow + (size_t)ho * s.Wo * s.Cout));
        }
    };

#pragma unroll
    for (int r = 0; r < PF; ++r) load_row(r);
    RowX R[TH + 2];
#pragma unroll
    for (int r = 0; r < TH + 2; ++r) {
        if (r + PF < TH + 2) load_row(r + PF);
        prep_row(raw[r][0], raw[r][1], raw[r][2], R[r]);
        if (r >= 2) emit(ho0 + r - 2, R[r - 2], R[r - 1], R[r]);
    }
}

// Any Kh, Kw, stride, padding, dilation.
template <int TH, bool BIAS, bool RELU>
__global__ __launch_bounds__(kThreads) void dw_generic_kernel(const bf16_t* __restrict__ x,
                                                              const bf16_t* __restrict__ w,  // [Kh][Kw][C]
                                                              const float* __restrict__ bias,
                                                              bf16_t* __restrict__ y, Shape s) {
    const int CV = s.Cin >> 3;
    const int v = blockIdx.x * kThreads + threadIdx.x;
    if (v >= s.Wo * CV) return;
    const int wo = v / CV;
    const int c0 = (v - wo * CV) << 3;
    const int n = blockIdx.z;
    const int ho0 = blockIdx.y * TH;
    const int ho1 = min(ho0 + TH, s.Ho);
    float br[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) br[i] = BIAS ? bias[c0 + i] : 0.0f;
    const bf16_t* xn = x + (size_t)n * s.H * s.W * s.Cin + c0;
    for (int ho = ho0; ho < ho1; ++ho) {
        float acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
        for (int kh = 0; kh < s.Kh; ++kh) {
            const int hi_ = ho * s.stride + kh * s.dil - s.pad;
            if (hi_ < 0 || hi_ >= s.H) continue;
            for (int kw = 0; kw < s.Kw; ++kw) {
                const int wi = wo * s.stride + kw * s.dil - s.pad;
                if (wi < 0 || wi >= s.W) continue;
                const V8 xv = load_v8(xn + (hi_ * s.W + wi) * s.Cin);
                const V8 wv = load_v8(w + (kh * s.Kw + kw) * s.Cin + c0);
                float wf[8];
#pragma unroll
                for (int i = 0; i < 4; ++i) { wf[2 * i] = lo(wv.u[i]); wf[2 * i + 1] = hi(wv.u[i]); }
                fma_v8(acc, xv, wf);
            }
        }
        *reinterpret_cast<V8*>(y + (((size_t)n * s.Ho + ho) * s.Wo + wo) * s.Cout + c0) =
            finish<BIAS, RELU>(acc, br, s.scale, s.shift, c0);
    }
}

#ifndef DW_ROWS_PER_THREAD
#define DW_ROWS_PER_THREAD 14
#endif
#ifndef DW_ROWS_IN_FLIGHT
#define DW_ROWS_IN_FLIGHT 2
#endif
static_assert(DW_ROWS_PER_THREAD % 2 == 0, "rows per thread come in pairs");
constexpr int kTH = DW_ROWS_PER_THREAD;  // output rows per thread

template <bool BIAS, bool RELU>
hipError_t launch_epi(const Shape& s, const bf16_t* x, const bf16_t* w, const float* b, bf16_t* y,
                      hipStream_t st) {
    const int CV = s.Cin / 8;
    dim3 grid((s.Wo * CV + kThreads - 1) / kThreads, (s.Ho + kTH - 1) / kTH, s.N);
    if (s.Kh == 3 && s.Kw == 3 && s.stride == 1 && s.dil == 1)
        hipLaunchKernelGGL((dw3x3s1_kernel<kTH, DW_ROWS_IN_FLIGHT, BIAS, RELU>), dim3(grid.x * grid.y * grid.z),
                           dim3(kThreads), 0, st, x, w, b, y, s);
    else
        hipLaunchKernelGGL((dw_generic_kernel<kTH, BIAS, RELU>), grid, dim3(kThreads), 0, st, x, w, b, y, s);
    return hipGetLastError();
}

}  // namespace

bool depthwise_supports(const Shape& s) {
    // 16-byte channel vectors; the grid's y/z extents (and, for 3x3 stride 1,
    // their product with x) within launch limits
    const long long items = (long long)((s.Wo * (s.Cin / 8) + kThreads - 1) / kThreads) * ((s.Ho + kTH - 1) / kTH) * s.N;
    return s.Cin % 8 == 0 && s.N <= 65535 && (s.Ho + kTH - 1) / kTH <= 65535 && items < 0x7fffffffLL &&
           buffer_addressable(s);
}

hipError_t launch_depthwise(const Shape& s, const void* x, const void* w_dw, const float* bias,
                            void* y, hipStream_t st) {
    (void)hipGetLastError();  // report only this launch's error
    const bf16_t* xt = static_cast<const bf16_t*>(x);
    const bf16_t* wt = static_cast<const bf16_t*>(w_dw);
    bf16_t* yt = static_cast<bf16_t*>(y);
    const bool b = s.epilogue & CONV2D_EPI_BIAS, r = s.epilogue & CONV2D_EPI_RELU;
    if (b && r) return launch_epi<true, true>(s, xt, wt, bias, yt, st);
    if (b) return launch_epi<true, false>(s, xt, wt, bias, yt, st);
    if (r) return launch_epi<false, true>(s, xt, wt, bias, yt, st);
    return launch_epi<false, false>(s, xt, wt, bias, yt, st);
}

}  // namespace conv2d
