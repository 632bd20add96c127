// transposed.hip -- transposed convolution by the direct loop, and the weight
// repack of the transposed layout.
//
// A transposed convolution ("lpnh.cn/news/2674933" sections 2.3 and 4.2) adds
// each input pixel's products with the whole filter into the output window it
// spans: Y[oh, ow] += X[ih, iw] W[kh, kw] at oh = ih*S - P + kh*D.  Here each
// thread owns one output pixel and gathers instead: tap kh reaches output
// row oh from input row ih = (oh + P - kh*D) / S exactly when that division
// is exact and 0 <= ih < H (the zero rows the page inserts between input rows
// are the taps whose division is not exact; they are skipped, never read).
// The same per-thread structure as the direct convolution: one output pixel,
// COB output channels per thread, fp32 accumulation, any layout and dtype.
#include "common.hpp"
#include "../../include/conv2d.h"

namespace conv2d {

namespace {

constexpr int kThreads = 256;

template <typename T, int XL, int WL, int YL, int COB, bool BIAS, bool RELU>
__global__ __launch_bounds__(kThreads) void tconv_direct_kernel(const T* __restrict__ x,
                                                                const T* __restrict__ w,
                                                                const float* __restrict__ bias,
                                                                T* __restrict__ y, Shape s) {
    const int ncob = (s.cout_g + COB - 1) / COB;
    const int g = blockIdx.y / ncob;
    const int cb = blockIdx.y - g * ncob;
    const int npix = s.N * s.Ho * s.Wo;
    const int p = blockIdx.x * kThreads + threadIdx.x;
    if (p >= npix) return;
    const int ow = p % s.Wo;
    const int t = p / s.Wo;
    const int oh = t % s.Ho;
    const int n = t / s.Ho;
    const int col0 = cb * COB;                        // first output channel within the group
    const int nco = min(COB, s.cout_g - col0);        // valid channels in this block

    float acc[COB];
#pragma unroll
    for (int j = 0; j < COB; ++j) acc[j] = 0.0f;

    for (int kh = 0; kh < s.Kh; ++kh) {
        const int th = oh + s.pad - kh * s.dil;
        if (th < 0 || th % s.stride) continue;
        const int ih = th / s.stride;
        if (ih >= s.H) continue;
        for (int kw = 0; kw < s.Kw; ++kw) {
            const int tw = ow + s.pad - kw * s.dil;
            if (tw < 0 || tw % s.stride) continue;
            const int iw = tw / s.stride;
            if (iw >= s.W) continue;
            for (int ci = 0; ci < s.cin_g; ++ci) {
                const int c = g * s.cin_g + ci;
                const int xi = (XL == NCHW) ? ((n * s.Cin + c) * s.H + ih) * s.W + iw
                                            : ((n * s.H + ih) * s.W + iw) * s.Cin + c;
                const float xv = load_f32<T>(x, xi);
#pragma unroll
                for (int j = 0; j < COB; ++j) {
                    if (j < nco) {
                        const int col = col0 + j;
                        const int wi = (WL == W_IOHW)
                                           ? ((c * s.cout_g + col) * s.Kh + kh) * s.Kw + kw
                                           : (((g * s.cout_g + col) * s.Kh + kh) * s.Kw + kw) * s.cin_g + ci;
                        acc[j] = fmaf(xv, load_f32<T>(w, wi), acc[j]);
                    }
                }
            }
        }
    }
#pragma unroll
    for (int j = 0; j < COB; ++j) {
        if (j < nco) {
            const int co = g * s.cout_g + col0 + j;
            const float v = epilogue<BIAS, RELU>(acc[j], bias, s.scale, s.shift, co);
            const int yi = (YL == NCHW) ? ((n * s.Cout + co) * s.Ho + oh) * s.Wo + ow
                                        : ((n * s.Ho + oh) * s.Wo + ow) * s.Cout + co;
            store_f32<T>(y, yi, v);
        }
    }
}

template <typename T, int XL, int WL, int YL, int COB>
hipError_t launch_t(const Shape& s, const T* x, const T* w, const float* b, T* y, hipStream_t st) {
    const int npix = s.N * s.Ho * s.Wo;
    const int ncob = (s.cout_g + COB - 1) / COB;
    if ((long long)s.groups * ncob > 65535) return hipErrorInvalidConfiguration;
    dim3 grid((npix + kThreads - 1) / kThreads, s.groups * ncob);
    const bool bias = s.epilogue & CONV2D_EPI_BIAS, relu = s.epilogue & CONV2D_EPI_RELU;
    if (bias && relu)
        hipLaunchKernelGGL((tconv_direct_kernel<T, XL, WL, YL, COB, true, true>), grid, dim3(kThreads), 0, st, x, w, b, y, s);
    else if (bias)
        hipLaunchKernelGGL((tconv_direct_kernel<T, XL, WL, YL, COB, true, false>), grid, dim3(kThreads), 0, st, x, w, b, y, s);
    else if (relu)
        hipLaunchKernelGGL((tconv_direct_kernel<T, XL, WL, YL, COB, false, true>), grid, dim3(kThreads), 0, st, x, w, b, y, s);
    else
        hipLaunchKernelGGL((tconv_direct_kernel<T, XL, WL, YL, COB, false, false>), grid, dim3(kThreads), 0, st, x, w, b, y, s);
    return hipGetLastError();
}

template <typename T, int XL, int WL, int YL>
hipError_t launch_cob(const Shape& s, const void* x, const void* w, const float* b, void* y, hipStream_t st) {
    const T* xt = static_cast<const T*>(x);
    const T* wt = static_cast<const T*>(w);
    T* yt = static_cast<T*>(y);
    if (s.cout_g == 1) return launch_t<T, XL, WL, YL, 1>(s, xt, wt, b, yt, st);
    if (s.cout_g <= 4) return launch_t<T, XL, WL, YL, 4>(s, xt, wt, b, yt, st);
    if (s.cout_g <= 8) return launch_t<T, XL, WL, YL, 8>(s, xt, wt, b, yt, st);
    return launch_t<T, XL, WL, YL, 16>(s, xt, wt, b, yt, st);
}

template <typename T>
hipError_t launch_layouts(const Shape& s, const void* x, int xl, const void* w, int wl, const float* b,
                          void* y, int yl, hipStream_t st) {
    if (xl == NCHW && wl == W_IOHW && yl == NCHW) return launch_cob<T, NCHW, W_IOHW, NCHW>(s, x, w, b, y, st);
    if (xl == NHWC && wl == W_PACKED && yl == NHWC) return launch_cob<T, NHWC, W_PACKED, NHWC>(s, x, w, b, y, st);
    return hipErrorInvalidValue;
}

// [Cin][Cout/G][Kh][Kw] -> [Cout][Kh][Kw][Cin/G]: one thread per packed
// element (consecutive threads write consecutive input channels).
template <typename E>
__global__ __launch_bounds__(kThreads) void tpack_kernel(const E* __restrict__ w, E* __restrict__ wp, int Cin,
                                                         int cout_g, int groups, int Kh, int Kw) {
    const int cin_g = Cin / groups;
    const int total = cout_g * groups * Kh * Kw * cin_g;
    const int d = blockIdx.x * kThreads + threadIdx.x;
    if (d >= total) return;
    const int ci = d % cin_g;
    int t = d / cin_g;
    const int kw = t % Kw;
    t /= Kw;
    const int kh = t % Kh;
    const int co = t / Kh;
    const int g = co / cout_g, col = co % cout_g;
    wp[d] = w[(((g * cin_g + ci) * cout_g + col) * Kh + kh) * Kw + kw];
}

}  // namespace

hipError_t launch_tconv_direct(const Shape& s, const void* x, int xl, const void* w, int wl,
                               const float* bias, void* y, int yl, hipStream_t st) {
    (void)hipGetLastError();  // report only this launch's error
    if (s.dtype == CONV2D_F32) return launch_layouts<float>(s, x, xl, w, wl, bias, y, yl, st);
    return launch_layouts<bf16_t>(s, x, xl, w, wl, bias, y, yl, st);
}

hipError_t launch_tpack_weights(const void* w, void* wp, int Cin, int cout_g, int groups, int Kh, int Kw,
                                int elem_bytes, hipStream_t st) {
    (void)hipGetLastError();
    const long long total = (long long)cout_g * groups * Kh * Kw * (Cin / groups);
    if (total >= 0x7fffffffLL) return hipErrorInvalidValue;
    const dim3 grid((unsigned)((total + kThreads - 1) / kThreads));
    if (elem_bytes == 4)
        hipLaunchKernelGGL(tpack_kernel<uint32_t>, grid, dim3(kThreads), 0, st, static_cast<const uint32_t*>(w),
                           static_cast<uint32_t*>(wp), Cin, cout_g, groups, Kh, Kw);
    else
        hipLaunchKernelGGL(tpack_kernel<uint16_t>, grid, dim3(kThreads), 0, st, static_cast<const uint16_t*>(w),
                           static_cast<uint16_t*>(wp), Cin, cout_g, groups, Kh, Kw);
    return hipGetLastError();
}

}  // namespace conv2d
