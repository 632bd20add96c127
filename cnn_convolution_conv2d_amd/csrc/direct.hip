// direct.hip -- direct-loop convolution: the definition computed as written,
// one output pixel per thread, COB output channels per thread so that each
// input value loaded is reused COB times (lincklin.cn lesson 9, section 5 for
// the per-thread loop, section 17 for computing several output channels per
// thread, section 26 for zero padding by address predicate).
//
// Serves every shape and dtype: the fp32 path, shapes whose channels do not
// fit the MFMA paths, and the reference layouts (NCHW activations, OIHW
// weights) without any repack.  Accumulates in fp32.
//
// Grid: x = blocks of 256 output pixels (n, ho, wo); y = group * channel
// blocks.  All threads of a block share (group, channel block), so the weight
// reads are wave-uniform and go through the scalar cache.
#include "mfma.hpp"
#include "../../include/conv2d.h"

namespace conv2d {

namespace {

constexpr int kThreads = 256;

template <typename T, int XL, int WL, int YL, int COB, bool BIAS, bool RELU>
__global__ __launch_bounds__(kThreads) void direct_kernel(const T* __restrict__ x,
                                                          const T* __restrict__ w,
                                                          const float* __restrict__ bias,
                                                          T* __restrict__ y, Shape s) {
    const int ncob = (s.cout_g + COB - 1) / COB;
    const int g = blockIdx.y / ncob;
    const int cb = blockIdx.y - g * ncob;
    const int npix = s.N * s.Ho * s.Wo;
    const int p = blockIdx.x * kThreads + threadIdx.x;
    if (p >= npix) return;
    const int wo = p % s.Wo;
    const int t = p / s.Wo;
    const int ho = t % s.Ho;
    const int n = t / s.Ho;
    const int co_base = g * s.cout_g + cb * COB;   // first output channel of this block
    const int nco = min(COB, s.cout_g - cb * COB);  // valid channels in this block

    float acc[COB];
#pragma unroll
    for (int j = 0; j < COB; ++j) acc[j] = 0.0f;

    for (int ci = 0; ci < s.cin_g; ++ci) {
        const int c = g * s.cin_g + ci;
        for (int kh = 0; kh < s.Kh; ++kh) {
            const int hi = ho * s.stride + kh * s.dil - s.pad;
            if (hi < 0 || hi >= s.H) continue;
            for (int kw = 0; kw < s.Kw; ++kw) {
                const int wi = wo * s.stride + kw * s.dil - s.pad;
                if (wi < 0 || wi >= s.W) continue;
                const int xi = (XL == NCHW) ? ((n * s.Cin + c) * s.H + hi) * s.W + wi
                                            : ((n * s.H + hi) * s.W + wi) * s.Cin + c;
                const float xv = load_f32<T>(x, xi);
#pragma unroll
                for (int j = 0; j < COB; ++j) {
                    if (j < nco) {
                        const int co = co_base + j;
                        int wi_;
                        if (WL == W_OIHW) wi_ = ((co * s.cin_g + ci) * s.Kh + kh) * s.Kw + kw;
                        else if (WL == W_PACKED) wi_ = ((co * s.Kh + kh) * s.Kw + kw) * s.cin_g + ci;
                        else wi_ = (kh * s.Kw + kw) * s.Cout + co;  // depthwise [Kh][Kw][C]
                        acc[j] = fmaf(xv, load_f32<T>(w, wi_), acc[j]);
                    }
                }
            }
        }
    }
#pragma unroll
    for (int j = 0; j < COB; ++j) {
        if (j < nco) {
            const int co = co_base + j;
            const float v = epilogue<BIAS, RELU>(acc[j], bias, s.scale, s.shift, co);
            const int yi = (YL == NCHW) ? ((n * s.Cout + co) * s.Ho + ho) * s.Wo + wo
                                        : ((n * s.Ho + ho) * s.Wo + wo) * s.Cout + co;
            store_f32<T>(y, yi, v);
        }
    }
}

// 3x3 filters over few input channels per group (CI <= 4: a stem layer on an
// RGB image is the common case).  The K dimension is only CI*9, so the
// generic loop above is one dependent global load per tap; here the taps are
// unrolled, every input value of the window is requested at once (one memory
// latency instead of CI*9), and the block's weights sit in LDS as
// [tap][COB], read as broadcasts.  Work items are (pixel block, group and
// channel block) with the channel blocks of one pixel block consecutive, and
// each XCD takes one contiguous run of items, so the channel blocks that
// share an input window read it through one L2.
template <typename T, int XL, int WL, int YL, int CI, int COB, bool BIAS, bool RELU>
__global__ __launch_bounds__(kThreads) void direct3x3_small_kernel(const T* __restrict__ x,
                                                                   const T* __restrict__ w,
                                                                   const float* __restrict__ bias,
                                                                   T* __restrict__ y, Shape s) {
    constexpr int NT = CI * 9;  // taps per output
    __shared__ __align__(16) float ws[NT][COB];
    const int ncob = (s.cout_g + COB - 1) / COB;
    const int item = xcd_tile_index();
    const int pb = item / (s.groups * ncob), gc = item - pb * (s.groups * ncob);
    const int g = gc / ncob;
    const int cb = gc - g * ncob;
    const int co_base = g * s.cout_g + cb * COB;
    const int nco = min(COB, s.cout_g - cb * COB);
    for (int i = threadIdx.x; i < NT * COB; i += kThreads) {
        const int tap = i / COB, j = i - tap * COB;
        const int ci = tap / 9, kh = (tap / 3) % 3, kw = tap % 3;
        const int co = co_base + j;
        const int wi_ = (WL == W_OIHW) ? ((co * CI + ci) * 3 + kh) * 3 + kw : ((co * 3 + kh) * 3 + kw) * CI + ci;
        ws[tap][j] = j < nco ? load_f32<T>(w, wi_) : 0.0f;
    }
    __syncthreads();
    const int npix = s.N * s.Ho * s.Wo;
    const int p = pb * kThreads + threadIdx.x;
    if (p >= npix) return;
    const int wo = p % s.Wo;
    const int t = p / s.Wo;
    const int ho = t % s.Ho;
    const int n = t / s.Ho;

    float xv[NT];
#pragma unroll
    for (int ci = 0; ci < CI; ++ci) {
        const int c = g * CI + ci;
#pragma unroll
        for (int kh = 0; kh < 3; ++kh) {
            const int hi = ho * s.stride + kh * s.dil - s.pad;
#pragma unroll
            for (int kw = 0; kw < 3; ++kw) {
                const int wi = wo * s.stride + kw * s.dil - s.pad;
                const bool ok = (unsigned)hi < (unsigned)s.H && (unsigned)wi < (unsigned)s.W;
                const int xi = (XL == NCHW) ? ((n * s.Cin + c) * s.H + hi) * s.W + wi
                                            : ((n * s.H + hi) * s.W + wi) * s.Cin + c;
                xv[(ci * 3 + kh) * 3 + kw] = ok ? load_f32<T>(x, xi) : 0.0f;
            }
        }
    }
    float acc[COB];
#pragma unroll
    for (int j = 0; j < COB; ++j) acc[j] = 0.0f;
#pragma unroll
    for (int tap = 0; tap < NT; ++tap)
#pragma unroll
        for (int j = 0; j < COB; ++j) acc[j] = fmaf(xv[tap], ws[tap][j], acc[j]);
#pragma unroll
    for (int j = 0; j < COB; ++j) {
        if (j < nco) {
            const int co = co_base + j;
            const float v = epilogue<BIAS, RELU>(acc[j], bias, s.scale, s.shift, co);
            const int yi = (YL == NCHW) ? ((n * s.Cout + co) * s.Ho + ho) * s.Wo + wo
                                        : ((n * s.Ho + ho) * s.Wo + wo) * s.Cout + co;
            store_f32<T>(y, yi, v);
        }
    }
}

#ifndef DIRECT_SMALL_COB
#define DIRECT_SMALL_COB 4
#endif

template <typename T, int XL, int WL, int YL, int CI>
hipError_t launch_small(const Shape& s, const T* x, const T* w, const float* b, T* y, hipStream_t st) {
    constexpr int COB = DIRECT_SMALL_COB;  // output channels per thread
    const int npix = s.N * s.Ho * s.Wo;
    const int ncob = (s.cout_g + COB - 1) / COB;
    const long long items = (long long)((npix + kThreads - 1) / kThreads) * s.groups * ncob;
    if (items > 0x7fffffffLL) return hipErrorInvalidConfiguration;
    const dim3 grid((unsigned)items);
    const bool bias = s.epilogue & CONV2D_EPI_BIAS, relu = s.epilogue & CONV2D_EPI_RELU;
#define SMALL_LAUNCH(B_, R_)                                                                 \
    hipLaunchKernelGGL((direct3x3_small_kernel<T, XL, WL, YL, CI, COB, B_, R_>), grid, dim3(kThreads), 0, st, x, w, \
                       b, y, s)
    if (bias && relu) SMALL_LAUNCH(true, true);
    else if (bias) SMALL_LAUNCH(true, false);
    else if (relu) SMALL_LAUNCH(false, true);
    else SMALL_LAUNCH(false, false);
#undef SMALL_LAUNCH
    return hipGetLastError();
}

template <typename T, int XL, int WL, int YL, int COB>
hipError_t launch_t(const Shape& s, const T* x, const T* w, const float* b, T* y, hipStream_t st) {
    const int npix = s.N * s.Ho * s.Wo;
    const int ncob = (s.cout_g + COB - 1) / COB;
    if ((long long)s.groups * ncob > 65535) return hipErrorInvalidConfiguration;
    dim3 grid((npix + kThreads - 1) / kThreads, s.groups * ncob);
    const bool bias = s.epilogue & CONV2D_EPI_BIAS, relu = s.epilogue & CONV2D_EPI_RELU;
    if (bias && relu)
        hipLaunchKernelGGL((direct_kernel<T, XL, WL, YL, COB, true, true>), grid, dim3(kThreads), 0, st, x, w, b, y, s);
    else if (bias)
        hipLaunchKernelGGL((direct_kernel<T, XL, WL, YL, COB, true, false>), grid, dim3(kThreads), 0, st, x, w, b, y, s);
    else if (relu)
        hipLaunchKernelGGL((direct_kernel<T, XL, WL, YL, COB, false, true>), grid, dim3(kThreads), 0, st, x, w, b, y, s);
    else
        hipLaunchKernelGGL((direct_kernel<T, XL, WL, YL, COB, false, false>), grid, dim3(kThreads), 0, st, x, w, b, y, s);
    return hipGetLastError();
}

template <typename T, int XL, int WL, int YL>
hipError_t launch_cob(const Shape& s, const void* x, const void* w, const float* b, void* y, hipStream_t st) {
    const T* xt = static_cast<const T*>(x);
    const T* wt = static_cast<const T*>(w);
    T* yt = static_cast<T*>(y);
    // 3x3 over at most 4 input channels per group, at least 8 outputs per
    // group: the unrolled small-K kernel.
    if (WL != W_DW && s.Kh == 3 && s.Kw == 3 && s.cout_g >= 8 && s.cin_g <= 4) {
        if (s.cin_g == 1) return launch_small<T, XL, WL, YL, 1>(s, xt, wt, b, yt, st);
        if (s.cin_g == 2) return launch_small<T, XL, WL, YL, 2>(s, xt, wt, b, yt, st);
        if (s.cin_g == 3) return launch_small<T, XL, WL, YL, 3>(s, xt, wt, b, yt, st);
        return launch_small<T, XL, WL, YL, 4>(s, xt, wt, b, yt, st);
    }
    // Few output channels per group (depthwise, small layers): 1 or 4 per
    // thread; otherwise 8, or 16 when the pixel grid alone would not fill the
    // chip.
    if (s.cout_g == 1) return launch_t<T, XL, WL, YL, 1>(s, xt, wt, b, yt, st);
    if (s.cout_g <= 4) return launch_t<T, XL, WL, YL, 4>(s, xt, wt, b, yt, st);
    if (s.cout_g <= 8) return launch_t<T, XL, WL, YL, 8>(s, xt, wt, b, yt, st);
    return launch_t<T, XL, WL, YL, 16>(s, xt, wt, b, yt, st);
}

template <typename T>
hipError_t launch_layouts(const Shape& s, const void* x, int xl, const void* w, int wl,
                          const float* b, void* y, int yl, hipStream_t st) {
    if (xl == NCHW && wl == W_OIHW && yl == NCHW) return launch_cob<T, NCHW, W_OIHW, NCHW>(s, x, w, b, y, st);
    if (xl == NHWC && wl == W_PACKED && yl == NHWC) return launch_cob<T, NHWC, W_PACKED, NHWC>(s, x, w, b, y, st);
    if (xl == NHWC && wl == W_DW && yl == NHWC) return launch_cob<T, NHWC, W_DW, NHWC>(s, x, w, b, y, st);
    return hipErrorInvalidValue;
}

// ---------------------------------------------------------------- repacks

// Batched 2-D transpose through a 64x64 LDS tile: src [batch][rows][cols] ->
// dst [batch][cols][rows].  NCHW->NHWC is rows=C, cols=H*W; NHWC->NCHW is
// rows=H*W, cols=C.  Reads and writes are both coalesced along the
// contiguous dimension; the +1 column pad keeps LDS columns conflict-free.
constexpr int kTile = 64;

template <typename T>
__global__ __launch_bounds__(256) void transpose_kernel(const T* __restrict__ src, T* __restrict__ dst,
                                                        int batch, int rows, int cols) {
    __shared__ T tile[kTile][kTile + 1];
    const size_t plane = (size_t)rows * cols;
    const int tx = threadIdx.x & 63, ty = threadIdx.x >> 6;  // 64 x 4
    const int c0 = blockIdx.x * kTile;
    // y and z grid extents are capped by the launch limits: stride over them
    for (int b = blockIdx.z; b < batch; b += gridDim.z) {
        const T* s = src + b * plane;
        T* d = dst + b * plane;
        for (int r0 = blockIdx.y * kTile; r0 < rows; r0 += gridDim.y * kTile) {
            for (int i = ty; i < kTile; i += 4) {
                const int r = r0 + i, c = c0 + tx;
                if (r < rows && c < cols) tile[i][tx] = s[(size_t)r * cols + c];
            }
            __syncthreads();
            for (int i = ty; i < kTile; i += 4) {
                const int c = c0 + i, r = r0 + tx;
                if (r < rows && c < cols) d[(size_t)c * rows + r] = tile[tx][i];
            }
            __syncthreads();
        }
    }
}

// The same transpose for 2-byte elements when rows and cols are multiples of
// 8 (and both tensors 16-byte aligned): each thread moves one 8x8 block with
// eight 16-byte loads (eight consecutive source rows, the same eight
// columns), a transpose in registers, and eight 16-byte stores (eight
// consecutive destination rows, the same eight source rows).  Lane l of a
// wave takes column block l % 8 and row block l / 8 of a 64x64 tile, so each
// load or store instruction of a wave covers eight whole 128-byte runs; no
// LDS and no barrier.  A workgroup's four waves take four tiles side by side.
__global__ __launch_bounds__(256) void transpose8x8_kernel(const uint16_t* __restrict__ src,
                                                           uint16_t* __restrict__ dst, int batch, int rows,
                                                           int cols) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int c = (blockIdx.x * 4 + wave) * 64 + (lane & 7) * 8;
    const size_t plane = (size_t)rows * cols;
    if (c >= cols) return;
    for (int b = blockIdx.z; b < batch; b += gridDim.z) {
        for (int r0 = blockIdx.y * 64; r0 < rows; r0 += gridDim.y * 64) {
            const int r = r0 + (lane >> 3) * 8;
            if (r >= rows) continue;  // rows % 8 == 0: the block is whole or absent
            const uint16_t* sp = src + b * plane + (size_t)r * cols + c;
            uint4 v[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) v[i] = *reinterpret_cast<const uint4*>(sp + (size_t)i * cols);
            uint16_t* dp = dst + b * plane + (size_t)c * rows + r;
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                // column j: word k holds rows 2k (low half) and 2k + 1 (high half);
                // v_perm_b32 takes the low (j even) or high (j odd) half of each
                const uint32_t sel = (j & 1) ? 0x07060302u : 0x05040100u;
                uint32_t o[4];
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    const uint32_t* lo = reinterpret_cast<const uint32_t*>(&v[2 * k]);
                    const uint32_t* hi = reinterpret_cast<const uint32_t*>(&v[2 * k + 1]);
                    o[k] = __builtin_amdgcn_perm(hi[j >> 1], lo[j >> 1], sel);
                }
                *reinterpret_cast<uint4*>(dp + (size_t)j * rows) = make_uint4(o[0], o[1], o[2], o[3]);
            }
        }
    }
}

// Weight repack: [Cout][Cin/G][Kh][Kw] -> [Cout][Kh][Kw][Cin/G], or for a
// depthwise filter bank [C][1][Kh][Kw] -> [Kh][Kw][C].  One thread per element.
template <typename T>
__global__ void pack_weights_kernel(const T* __restrict__ w, T* __restrict__ wp, int Cout, int cin_g,
                                    int Kh, int Kw, int depthwise) {
    const int total = Cout * cin_g * Kh * Kw;
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= total) return;
    const int kw = i % Kw;
    int t = i / Kw;
    const int kh = t % Kh;
    t /= Kh;
    const int ci = t % cin_g;
    const int co = t / cin_g;
    const int o = depthwise ? (kh * Kw + kw) * Cout + co : ((co * Kh + kh) * Kw + kw) * cin_g + ci;
    wp[o] = w[i];
}

}  // namespace

hipError_t launch_direct(const Shape& s, const void* x, int xl, const void* w, int wl,
                         const float* bias, void* y, int yl, hipStream_t st) {
    (void)hipGetLastError();  // report only this launch's error
    if (s.dtype == CONV2D_F32) return launch_layouts<float>(s, x, xl, w, wl, bias, y, yl, st);
    return launch_layouts<bf16_t>(s, x, xl, w, wl, bias, y, yl, st);
}

hipError_t launch_transpose(const void* src, void* dst, int batch, int rows, int cols,
                            int elem_bytes, hipStream_t st) {
    (void)hipGetLastError();  // report only this launch's error
    const int ty = (rows + kTile - 1) / kTile;
    if (elem_bytes == 2 && rows % 8 == 0 && cols % 8 == 0 &&
        ((reinterpret_cast<uintptr_t>(src) | reinterpret_cast<uintptr_t>(dst)) & 15) == 0) {
        dim3 grid((cols + 4 * kTile - 1) / (4 * kTile), ty < 65535 ? ty : 65535, batch < 65535 ? batch : 65535);
        hipLaunchKernelGGL(transpose8x8_kernel, grid, dim3(256), 0, st, static_cast<const uint16_t*>(src),
                           static_cast<uint16_t*>(dst), batch, rows, cols);
        return hipGetLastError();
    }
    dim3 grid((cols + kTile - 1) / kTile, ty < 65535 ? ty : 65535, batch < 65535 ? batch : 65535);
    if (elem_bytes == 4)
        hipLaunchKernelGGL(transpose_kernel<float>, grid, dim3(256), 0, st,
                           static_cast<const float*>(src), static_cast<float*>(dst), batch, rows, cols);
    else
        hipLaunchKernelGGL(transpose_kernel<bf16_t>, grid, dim3(256), 0, st,
                           static_cast<const bf16_t*>(src), static_cast<bf16_t*>(dst), batch, rows, cols);
    return hipGetLastError();
}

hipError_t launch_pack_weights(const void* w, void* wp, int Cout, int cin_g, int Kh, int Kw,
                               int depthwise, int elem_bytes, hipStream_t st) {
    (void)hipGetLastError();  // report only this launch's error
    const int total = Cout * cin_g * Kh * Kw;
    dim3 grid((total + 255) / 256);
    if (elem_bytes == 4)
        hipLaunchKernelGGL(pack_weights_kernel<float>, grid, dim3(256), 0, st,
                           static_cast<const float*>(w), static_cast<float*>(wp), Cout, cin_g, Kh, Kw, depthwise);
    else
        hipLaunchKernelGGL(pack_weights_kernel<bf16_t>, grid, dim3(256), 0, st,
                           static_cast<const bf16_t*>(w), static_cast<bf16_t*>(wp), Cout, cin_g, Kh, Kw, depthwise);
    return hipGetLastError();
}

}  // namespace conv2d
