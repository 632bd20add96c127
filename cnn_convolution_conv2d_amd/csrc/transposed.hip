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
#include "mfma.hpp"
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

namespace {

// ---------------------------------------------------------------------------
// Stride-2, 4x4 transposed convolution on an LDS window shared by all taps and
// phases.  Output phase (ph_h, ph_w) at phase-grid position (u, v) is output
// pixel (2u + ph_h, 2v + ph_w); its taps are kh = k0 + 2j (k0 = (ph_h + P) mod
// 2, j = 0, 1) reading input row u + (ph_h + P)/2 - j, likewise along the
// width (lpnh.cn section 4.2: the stride-1 convolution of the zero-inserted
// input, of which only these taps meet real pixels).  All four phases of a
// block of positions read rows u - 1 .. u + 2 at most, so a workgroup stages
// that input window once per channel block and every tap of every phase reads
// its MFMA operands from it at a shifted offset -- instead of gathering each
// tap's slice again from L2 as the phase-split gather kernel does.
//
// Workgroup: 8 x 32 phase-grid positions of one image x 64 output channels;
// 8 waves, wave w computes phase p = w % 4 = (ph_h, ph_w) for position rows
// 4*(w / 4) .. +3 and all 64 channels: eight 32x32 MFMA tiles (two channel
// blocks x four rows of 32 positions), so per 16-channel step two A and four
// B operand reads feed eight MFMAs.  Waves w and w + 4 share a SIMD and hide
// each other's LDS latency.
//
// The channel loop runs over blocks of 64 input channels, so that each
// pixel's and each weight row's slice of a block is one whole 128-byte line
// (the copies' cost is set by the number of lines they touch, not by their
// bytes).  Per block, the 10 x 34 input window (48 KB) is copied once and
// double-buffered; the block is then worked in four steps (jh, jw), in each
// of which every phase applies its tap (k0h + 2jh, k0w + 2jw), whose weights
// for the four phases (32 KB) are copied one step ahead into a double
// buffer.  All copies are buffer-to-LDS loads.  LDS layout, in 16-byte units:
//   weights [2][4 phases][64 co][8 pieces of 8 channels]  (a row's pieces
//           XOR-swizzled with (row / 2) mod 8)
//   window  [2][10 rows][34 columns][9 units]  (8 pieces and one unit of
//           padding: an odd pitch)
// With either layout 16 consecutive rows read at one logical piece fall in
// 16 distinct 16-byte bank groups, and lanes 16..31 read 16 rows further,
// a multiple of 16 units away.
constexpr int kThBK = 64;                               // input channels per block
constexpr int kThWin = 10, kTwWin = 34;                 // window rows, columns
constexpr int kThPos = 8, kTwPos = 32;                  // positions per tile
constexpr int kThCo = 64;                               // output channels per workgroup
constexpr int kThThreads = 512, kThWaves = kThThreads / 64;
constexpr int kThRows = kThPos / 2;                     // position rows per wave
constexpr int kThPitch = 9;                             // window units per pixel
constexpr int kThWUnits = 4 * kThCo * 8;                // 2048 per step
constexpr int kThXUnits = kThWin * kTwWin * kThPitch;   // 3060 per block
constexpr int kThWCopies = kThWUnits / 64;              // 32: 4 per wave per step
constexpr int kThXCopies = 48;                          // 6 per wave per block, the last ones overlapping
constexpr int kThLds = (2 * kThWUnits + 2 * kThXUnits) * 16;   // 163456 bytes
static_assert(kThWCopies == 4 * kThWaves && kThXCopies == 6 * kThWaves, "copy split below");
static_assert(64 * (kThXCopies - 1) >= kThXUnits - 64, "window copies cover the window");
static_assert(kThLds <= 163840, "LDS");

struct TconvHaloGrid {
    int N, Cin, H, W, Cout, pad, Ho, Wo;
    int lo;            // window origin relative to the tile: floor(P/2) - 1
    int nbu, nbv, ncb; // tiles along u, along v, output-channel groups
    int nblk;          // 64-channel blocks
};

typedef __attribute__((address_space(3))) void* th_lds_t;

// This wave's LDS operations complete, then the workgroup barrier; copies in
// flight into other buffers are not waited for (a plain __syncthreads would
// wait for every outstanding load).
__device__ __forceinline__ void th_barrier() {
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0); vmcnt and expcnt at their maxima (no wait)
    __builtin_amdgcn_s_barrier();
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// Weights of step t (jh = t / 2, jw = t % 2) of block b: instruction i
// writes units 64i .. 64i+63, i.e. rows 8i .. 8i+7 of [phase][co], each row
// the 8 pieces of one 128-byte line.
__device__ __forceinline__ void th_stage_w(uint4* __restrict__ wdst, const TconvHaloGrid& g,
                                           __amdgpu_buffer_rsrc_t wr, int b, int t, int co0, int wave,
                                           int lane) {
    const int c0 = b * kThBK, jh = t >> 1, jw = t & 1;
#pragma unroll
    for (int m = 0; m < kThWCopies / kThWaves; ++m) {
        const int i = wave + kThWaves * m;
        const int row = 8 * i + (lane >> 3);
        const int p = row >> 6, col = row & 63;
        const int piece = (lane & 7) ^ ((col >> 1) & 7);
        const int kh = (((p >> 1) + g.pad) & 1) + 2 * jh, kw = (((p & 1) + g.pad) & 1) + 2 * jw;
        const int co = co0 + col, ci = c0 + 8 * piece;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            wr, (th_lds_t)(wdst + i * 64), 16,
            co < g.Cout && ci < g.Cin ? ((co * 16 + kh * 4 + kw) * g.Cin + ci) * 2 : kOOB, 0, 0, 0);
    }
}

// Window of block b, copy instructions k = wave + 8j for j in [j0, j1):
// instruction k writes units base .. base+63, base = min(64k, 3060-64) (the
// last ones overlap, rewriting the same values, instead of running past the
// window); unit s is slot s % 9 of window pixel s / 9 = row*34 + column,
// slot 8 the padding (written with zeros).
__device__ __forceinline__ void th_stage_x(uint4* __restrict__ xdst, const TconvHaloGrid& g,
                                           __amdgpu_buffer_rsrc_t xr, int b, int j0, int j1, int n, int ih0,
                                           int iw0, int wave, int lane) {
    const int c0 = b * kThBK;
#pragma unroll
    for (int j = j0; j < j1; ++j) {
        const int k = wave + kThWaves * j;
        const int base = min(64 * k, kThXUnits - 64);
        const int s = base + lane;
        const int wp = s / kThPitch, slot = s - wp * kThPitch;
        const int wrow = wp / kTwWin, wcol = wp - wrow * kTwWin;
        const int ih = ih0 + wrow, iw = iw0 + wcol, ci = c0 + 8 * slot;
        const bool ok = slot < 8 && ci < g.Cin && (unsigned)ih < (unsigned)g.H && (unsigned)iw < (unsigned)g.W;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(xr, (th_lds_t)(xdst + base), 16,
                                                 ok ? (((n * g.H + ih) * g.W + iw) * g.Cin + ci) * 2 : kOOB,
                                                 0, 0, 0);
    }
}

// One step: four 16-channel K-steps of eight MFMAs from this wave's phase
// row of the weight buffer and its tap's shifted view of the window (tapo:
// the window pixel of position (r0, 0) for this step's tap).
__device__ __forceinline__ void th_step(const uint4* __restrict__ wc, const uint4* __restrict__ xc,
                                        f32x16 (&acc)[2][kThRows], int p, int tapo, int lane) {
    const int frow = lane & 31, half = lane >> 5;
    const int wsw = (frow >> 1) & 7;                         // swizzle of weight row 32i + frow
    const uint4* const wrow = wc + (p * kThCo + frow) * 8;
    const uint4* const xrow = xc + (tapo + frow) * kThPitch;
    // Two register sets: K-step ks+1 is read while ks's MFMAs issue; the
    // scheduling fence keeps the compiler from collapsing the pipeline into
    // one read per MFMA.
    bf16x8 a[2][2], bb[2][kThRows];
    auto load_group = [&](int ks, int set) {
        const int q = 2 * ks + half;                         // this lane's 8-channel piece
#pragma unroll
        for (int i = 0; i < 2; ++i) a[set][i] = __builtin_bit_cast(bf16x8, wrow[32 * 8 * i + (q ^ wsw)]);
#pragma unroll
        for (int r = 0; r < kThRows; ++r)
            bb[set][r] = __builtin_bit_cast(bf16x8, xrow[r * kTwWin * kThPitch + q]);
    };
    load_group(0, 0);
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
        if (ks + 1 < 4) load_group(ks + 1, (ks + 1) & 1);
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int r = 0; r < kThRows; ++r)
                acc[i][r] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[ks & 1][i], bb[ks & 1][r], acc[i][r], 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
    }
}

// Pack one 32x32 result block into bf16 with ReLU: out[h] holds channels
// cl .. cl+7 (cl = 16*((lane/16) % 2) + 8*(lane/32)) of position
// 16h + lane % 16.  In the 32x32 result layout lane l < 32 holds channels
// 8q + r (q, r = 0..3) of position l and lane l + 32 channels 8q + 4 + r; a
// lane-half swap gives each lane 8 consecutive channels, a row swap then
// 16 positions per register.
template <bool RELU>
__device__ __forceinline__ void th_pack(const f32x16& acc, uint32_t (&out)[2][4]) {
    uint32_t pk[4][2];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        float v[4] = {acc[4 * q], acc[4 * q + 1], acc[4 * q + 2], acc[4 * q + 3]};
        if (RELU)
#pragma unroll
            for (int i = 0; i < 4; ++i) v[i] = fmaxf(v[i], 0.0f);
        pk[q][0] = pack_bf16x2(v[0], v[1]);
        pk[q][1] = pack_bf16x2(v[2], v[3]);
    }
    uint32_t r8[2][4];
#pragma unroll
    for (int pr = 0; pr < 2; ++pr)
#pragma unroll
        for (int w = 0; w < 2; ++w) {
            const auto sw = __builtin_amdgcn_permlane32_swap(pk[2 * pr][w], pk[2 * pr + 1][w], false, false);
            r8[pr][w] = sw[0];
            r8[pr][2 + w] = sw[1];
        }
#pragma unroll
    for (int d = 0; d < 4; ++d) {
        const auto sw = __builtin_amdgcn_permlane16_swap(r8[0][d], r8[1][d], false, false);
        out[0][d] = sw[0];
        out[1][d] = sw[1];
    }
}

// Window copies a wave issues during step t of a block for the next block:
// j in [th_xj(t), th_xj(t+1)), two in each of the first two steps, one in
// each of the last two.
constexpr int th_xj(int t) { return t < 2 ? 2 * t : t + 2; }

template <bool BIAS, bool RELU>
__global__ __launch_bounds__(kThThreads, 1) void tconv_halo_kernel(const bf16_t* __restrict__ x,
                                                            const bf16_t* __restrict__ wp,  // [Cout][4][4][Cin]
                                                            const float* __restrict__ bias,
                                                            bf16_t* __restrict__ y, TconvHaloGrid g) {
    extern __shared__ uint4 thlds[];
    uint4* const wbuf = thlds;                       // [2][kThWUnits]
    uint4* const xbuf = thlds + 2 * kThWUnits;       // [2][kThXUnits]
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    int item = xcd_tile_index();
    const int cb = item % g.ncb;   // output-channel group fastest: neighbours share the window
    item /= g.ncb;
    const int bv = item % g.nbv;
    item /= g.nbv;
    const int bu = item % g.nbu;
    const int n = item / g.nbu;
    const int co0 = cb * kThCo;
    const int u0 = bu * kThPos, v0 = bv * kTwPos;
    const int ih0 = u0 + g.lo, iw0 = v0 + g.lo;

    const __amdgpu_buffer_rsrc_t xr = make_rsrc(x, (uint32_t)g.N * g.H * g.W * g.Cin * 2u);
    const __amdgpu_buffer_rsrc_t wr = make_rsrc(wp, (uint32_t)g.Cout * 16u * g.Cin * 2u);
    const __amdgpu_buffer_rsrc_t yr = make_rsrc(y, (uint32_t)g.N * g.Ho * g.Wo * g.Cout * 2u);

    // this wave's phase, its first position row, and for each step t = (jh,
    // jw) the window pixel of position (r0, 0) under that step's tap
    const int p = wave & 3, ph_h = p >> 1, ph_w = p & 1, r0 = kThRows * (wave >> 2);
    const int bh = (ph_h + g.pad) >> 1, bw = (ph_w + g.pad) >> 1;
    int tapo[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) tapo[t] = (r0 + bh - (t >> 1) - g.lo) * kTwWin + (bw - (t & 1) - g.lo);
    // rows of this phase inside the output: 2u + ph_h < Ho; a wave whose
    // four rows all lie below takes part in the copies and barriers only
    const bool act = 2 * (u0 + r0) + ph_h < g.Ho;

    // accumulators start at the bias: lane holds channels co0 + 32i + 8q +
    // 4*(lane/32) + (0..3) in acc[i][r][4q + 0..3]
    const __amdgpu_buffer_rsrc_t br = make_rsrc(bias, BIAS ? (uint32_t)g.Cout * 4u : 0u);
    f32x16 acc[2][kThRows];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        f32x16 b0 = f32x16{};
        if (BIAS)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int co = co0 + 32 * i + 8 * q + 4 * (lane >> 5);
                const float4 b4 = __builtin_bit_cast(float4, load16(br, co < g.Cout ? co * 4 : kOOB));
                b0[4 * q] = b4.x;
                b0[4 * q + 1] = b4.y;
                b0[4 * q + 2] = b4.z;
                b0[4 * q + 3] = b4.w;
            }
#pragma unroll
        for (int r = 0; r < kThRows; ++r) acc[i][r] = b0;
    }

    th_stage_x(xbuf, g, xr, 0, 0, 6, n, ih0, iw0, wave, lane);
    th_stage_w(wbuf, g, wr, 0, 0, co0, wave, lane);
    for (int b = 0; b < g.nblk; ++b) {
        const bool more = b + 1 < g.nblk;   // the next block's window is copied during this one
        uint4* const xc = xbuf + (b & 1) * kThXUnits;
        uint4* const xn = xbuf + ((b + 1) & 1) * kThXUnits;
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            // This wave's copies of this step's weights have landed: issued at
            // the start of the previous step, they are followed only by that
            // step's window copies for this block (if it issued any); the
            // first step also needs all of this block's window.  Loads
            // complete in order.  Then the barrier for everyone's copies; it
            // also frees the buffers the copies below overwrite (the previous
            // step's weights, the previous block's window).
            if (t == 0 || !more) __builtin_amdgcn_s_waitcnt(0x0f70);   // vmcnt(0)
            else if (t == 3) __builtin_amdgcn_s_waitcnt(0x0f71);       // vmcnt(1)
            else __builtin_amdgcn_s_waitcnt(0x0f72);                   // vmcnt(2)
            th_barrier();
            if (t < 3) th_stage_w(wbuf + ((t + 1) & 1) * kThWUnits, g, wr, b, t + 1, co0, wave, lane);
            else if (more) th_stage_w(wbuf, g, wr, b + 1, 0, co0, wave, lane);
            if (more) th_stage_x(xn, g, xr, b + 1, th_xj(t), th_xj(t + 1), n, ih0, iw0, wave, lane);
            if (act) th_step(wbuf + (t & 1) * kThWUnits, xc, acc, p, tapo[t], lane);
        }
    }
    if (!act) return;

    if (g.Cout % 8 == 0) {
        // Per position row: both channel blocks packed (th_pack), then
        // regrouped with 8-lane row shifts (DPP) so that lane l holds
        // channels cl2 = cl + 32*((l/8) % 2) of position (l % 8) (+8 in the
        // second register): one store instruction writes the 64 channels
        // (128 contiguous bytes) of each of 8 pixels, whole lines, with the
        // streaming (nt) policy.
        const int cl = ((lane >> 4) & 1) * 16 + (lane >> 5) * 8;
        const int co = co0 + cl + ((lane & 8) ? 32 : 0);
#pragma unroll
        for (int r = 0; r < kThRows; ++r) {
            const int oh = 2 * (u0 + r0 + r) + ph_h;
            uint32_t o0[2][4], o1[2][4];
            th_pack<RELU>(acc[0][r], o0);
            th_pack<RELU>(acc[1][r], o1);
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                uint32_t ra_[4], rb_[4];
#pragma unroll
                for (int d = 0; d < 4; ++d) {
                    // lanes 8..15 of each row: block 1's piece from 8 lanes lower
                    ra_[d] = __builtin_amdgcn_update_dpp(o0[h][d], o1[h][d], 0x118 /* row_shr:8 */, 0xf, 0xc, false);
                    // lanes 0..7 of each row: block 0's piece from 8 lanes higher
                    rb_[d] = __builtin_amdgcn_update_dpp(o1[h][d], o0[h][d], 0x108 /* row_shl:8 */, 0xf, 0x3, false);
                }
                const int owa = 2 * (v0 + 16 * h + (lane & 7)) + ph_w, owb = owa + 16;
                const bool oka = oh < g.Ho && owa < g.Wo && co < g.Cout;
                const bool okb = oh < g.Ho && owb < g.Wo && co < g.Cout;
                store16<kStoreStream>(yr, oka ? (((n * g.Ho + oh) * g.Wo + owa) * g.Cout + co) * 2 : kOOB,
                                      make_uint4(ra_[0], ra_[1], ra_[2], ra_[3]));
                store16<kStoreStream>(yr, okb ? (((n * g.Ho + oh) * g.Wo + owb) * g.Cout + co) * 2 : kOOB,
                                      make_uint4(rb_[0], rb_[1], rb_[2], rb_[3]));
            }
        }
        return;
    }
    const int ow = 2 * (v0 + (lane & 31)) + ph_w;
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int co = co0 + 32 * i + 8 * q + 4 * (lane >> 5);
#pragma unroll
            for (int r = 0; r < kThRows; ++r) {
                const int oh = 2 * (u0 + r0 + r) + ph_h;
                float v[4] = {acc[i][r][4 * q], acc[i][r][4 * q + 1], acc[i][r][4 * q + 2], acc[i][r][4 * q + 3]};
                if (RELU)
#pragma unroll
                    for (int e = 0; e < 4; ++e) v[e] = fmaxf(v[e], 0.0f);
                const bool ok = oh < g.Ho && ow < g.Wo && co < g.Cout;
                store8(yr, ok ? (((n * g.Ho + oh) * g.Wo + ow) * g.Cout + co) * 2 : kOOB,
                       make_uint2(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])));
            }
        }
}

template <bool BIAS, bool RELU>
hipError_t launch_th(const TconvHaloGrid& g, const bf16_t* x, const bf16_t* w, const float* b, bf16_t* y,
                     hipStream_t st) {
    int dev = 0;
    (void)hipGetDevice(&dev);
    const hipError_t ea = ensure_dynamic_lds<tconv_halo_kernel<BIAS, RELU>>(kThLds, dev);
    if (ea != hipSuccess) return ea;
    const long long blocks = (long long)g.N * g.nbu * g.nbv * g.ncb;
    hipLaunchKernelGGL((tconv_halo_kernel<BIAS, RELU>), dim3((unsigned)blocks), dim3(kThThreads), kThLds, st, x, w, b,
                       y, g);
    return hipGetLastError();
}

}  // namespace

bool tconv_halo_supports(const Shape& s) {
    const long long blocks = (long long)s.N * ((s.Ho + 1) / 2 + kThPos - 1) / kThPos *
                             (((s.Wo + 1) / 2 + kTwPos - 1) / kTwPos) * ((s.Cout + kThCo - 1) / kThCo);
    return s.dtype == CONV2D_BF16 && s.groups == 1 && s.stride == 2 && s.Kh == 4 && s.Kw == 4 && s.dil == 1 &&
           s.pad <= 3 && s.Cin % 32 == 0 && s.Cout % 4 == 0 && blocks < 0x7fffffffLL &&
           (long long)s.N * s.H * s.W * s.Cin * 2 < 0x7fff0000LL &&
           (long long)s.N * s.Ho * s.Wo * s.Cout * 2 < 0x7fff0000LL && (long long)s.Cout * 16 * s.Cin * 2 < 0x7fff0000LL;
}

hipError_t launch_tconv_halo(const Shape& s, const void* x, const void* w_packed, const float* bias, void* y,
                             hipStream_t st) {
    (void)hipGetLastError();  // report only this launch's error
    if (!tconv_halo_supports(s)) return hipErrorInvalidValue;
    TconvHaloGrid g;
    g.N = s.N; g.Cin = s.Cin; g.H = s.H; g.W = s.W; g.Cout = s.Cout; g.pad = s.pad; g.Ho = s.Ho; g.Wo = s.Wo;
    g.lo = s.pad / 2 - 1;
    g.nbu = ((s.Ho + 1) / 2 + kThPos - 1) / kThPos;
    g.nbv = ((s.Wo + 1) / 2 + kTwPos - 1) / kTwPos;
    g.ncb = (s.Cout + kThCo - 1) / kThCo;
    g.nblk = (s.Cin + kThBK - 1) / kThBK;
    const bf16_t* xt = static_cast<const bf16_t*>(x);
    const bf16_t* wt = static_cast<const bf16_t*>(w_packed);
    bf16_t* yt = static_cast<bf16_t*>(y);
    const bool bb = s.epilogue & CONV2D_EPI_BIAS, rr = s.epilogue & CONV2D_EPI_RELU;
    if (bb && rr) return launch_th<true, true>(g, xt, wt, bias, yt, st);
    if (bb) return launch_th<true, false>(g, xt, wt, bias, yt, st);
    if (rr) return launch_th<false, true>(g, xt, wt, bias, yt, st);
    return launch_th<false, false>(g, xt, wt, bias, yt, st);
}

}  // namespace conv2d
