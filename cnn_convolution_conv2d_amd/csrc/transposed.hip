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
// that input window once per channel chunk and every tap of every phase reads
// its MFMA operands from it at a shifted offset -- instead of gathering each
// tap's slice again from L2 as the phase-split gather kernel does.
//
// Workgroup: 8 x 32 phase-grid positions of one image x 32 output channels;
// 8 waves, wave w computes phase ((w % 4) / 2, w % 2) for position rows
// 4*(w / 4) .. +3: four 32x32 MFMA tiles (32 channels x one row of 32
// positions); two waves per SIMD hide each other's LDS latency.  Per chunk
// of 32 input channels, copied into LDS by buffer-to-LDS loads,
// triple-buffered (a chunk's copies are issued two chunks ahead, so their
// latency is covered by two chunks of work):
//   weights [16 taps][32 co][4 pieces of 8 channels]  (32 KB)
//   window  [10 rows][34 columns][4 pieces]             (21 KB)
// A 64-byte row (one co and tap, or one pixel) holds its four 16-byte pieces
// XOR-swizzled with (row / 4) mod 4, so any 16 consecutive rows read at the
// same logical piece land in 16 distinct 16-byte bank groups; the copies apply
// the swizzle on the global side (lane order in LDS is fixed).
constexpr int kThWin = 10, kTwWin = 34;                // window rows, columns
constexpr int kThPos = 8, kTwPos = 32;                  // positions per tile
constexpr int kThCo = 32;                               // output channels per workgroup
constexpr int kThThreads = 512, kThWaves = kThThreads / 64;
constexpr int kThRows = kThPos / 2;                     // position rows per wave
constexpr int kThWUnits = 16 * kThCo * 4;               // 2048
constexpr int kThXUnits = kThWin * kTwWin * 4;          // 1360
constexpr int kThXCopies = 24;                          // window copy instructions: 3 per wave
constexpr int kThBuf = kThWUnits + kThXUnits;           // 3408 units
constexpr int kThLds = 3 * kThBuf * 16;                 // 163584 bytes
// copy instructions each wave issues per chunk (4 weight + 3 window): the
// wait for a chunk leaves exactly the next chunk's copies outstanding
constexpr int kThCopiesPerWave = 32 / kThWaves + kThXCopies / kThWaves;
static_assert(kThCopiesPerWave == 7, "vmcnt immediate below");

struct TconvHaloGrid {
    int N, Cin, H, W, Cout, pad, Ho, Wo;
    int lo;            // window origin relative to the tile: floor(P/2) - 1
    int nbu, nbv, ncb; // tiles along u, along v, output-channel groups
    int nchunk;        // 32-channel chunks
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

__device__ __forceinline__ void th_stage(uint4* __restrict__ wdst, uint4* __restrict__ xdst,
                                         const TconvHaloGrid& g, __amdgpu_buffer_rsrc_t wr,
                                         __amdgpu_buffer_rsrc_t xr, int kc, int co0, int n, int ih0, int iw0,
                                         int wave, int lane) {
    const int c0 = kc * 32;
    // weights: instruction i covers tap i/2, output channels 16*(i%2) + lane/4
#pragma unroll
    for (int m = 0; m < 32 / kThWaves; ++m) {
        const int i = wave + kThWaves * m;
        const int tap = i >> 1, col = 16 * (i & 1) + (lane >> 2);
        const int piece = (lane & 3) ^ ((col >> 2) & 3);
        const int co = co0 + col;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(wr, (th_lds_t)(wdst + i * 64), 16,
                                                 co < g.Cout ? ((co * 16 + tap) * g.Cin + c0 + 8 * piece) * 2 : kOOB,
                                                 0, 0, 0);
    }
    // window: unit s = pixel*4 + slot, pixel = row*34 + column; instruction k
    // writes units base .. base+63 with base = min(64k, 1360-64), so the last
    // instructions overlap (rewriting the same values) instead of running past
    // the window
#pragma unroll
    for (int m = 0; m < kThXCopies / kThWaves; ++m) {
        const int k = wave + kThWaves * m;
        const int base = min(64 * k, kThXUnits - 64);
        const int s = base + lane;
        const int wp = s >> 2, piece = (s & 3) ^ ((wp >> 2) & 3);
        const int wrow = wp / kTwWin, wcol = wp - wrow * kTwWin;
        const int ih = ih0 + wrow, iw = iw0 + wcol;
        const bool ok = (unsigned)ih < (unsigned)g.H && (unsigned)iw < (unsigned)g.W;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(xr, (th_lds_t)(xdst + base), 16,
                                                 ok ? (((n * g.H + ih) * g.W + iw) * g.Cin + c0 + 8 * piece) * 2 : kOOB,
                                                 0, 0, 0);
    }
}

// One chunk: start the copies of chunk `next` (two ahead), then the phase's four taps x two
// 16-channel steps x four position rows of MFMAs from the current buffers
// (tapo already includes this wave's first row).
__device__ __forceinline__ void th_chunk(const uint4* __restrict__ wc, const uint4* __restrict__ xc,
                                         uint4* __restrict__ wn, uint4* __restrict__ xn, f32x16 acc[kThRows],
                                         const TconvHaloGrid& g, __amdgpu_buffer_rsrc_t wr,
                                         __amdgpu_buffer_rsrc_t xr, int next, int co0, int n, int ih0, int iw0,
                                         int wave, int lane, const int tapk[4], const int tapo[4]) {
    if (next >= 0) th_stage(wn, xn, g, wr, xr, next, co0, n, ih0, iw0, wave, lane);
    const int frow = lane & 31, half = lane >> 5;
    // Eight operand groups per chunk: (tap t, 16-channel step ks) = (gi / 2,
    // gi % 2), each one A operand and four B operands (the wave's position
    // rows).  Two register sets: group gi+1 is read while group gi's MFMAs
    // issue; the scheduling fence keeps the compiler from collapsing the
    // pipeline into one read per MFMA.
    bf16x8 a[2], b[2][kThRows];
    auto load_group = [&](int gi, int set) {
        const int t = gi >> 1, q = 2 * (gi & 1) + half;   // this lane's 8-channel piece
        a[set] = __builtin_bit_cast(bf16x8, wc[(tapk[t] * kThCo + frow) * 4 + (q ^ ((frow >> 2) & 3))]);
#pragma unroll
        for (int r = 0; r < kThRows; ++r) {
            const int wp = tapo[t] + r * kTwWin + frow;   // window pixel of position (r, frow)
            b[set][r] = __builtin_bit_cast(bf16x8, xc[wp * 4 + (q ^ ((wp >> 2) & 3))]);
        }
    };
    load_group(0, 0);
#pragma unroll
    for (int gi = 0; gi < 8; ++gi) {
        if (gi + 1 < 8) load_group(gi + 1, (gi + 1) & 1);
#pragma unroll
        for (int r = 0; r < kThRows; ++r)
            acc[r] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[gi & 1], b[gi & 1][r], acc[r], 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
    }
}

template <bool BIAS, bool RELU>
__global__ __launch_bounds__(kThThreads, 1) void tconv_halo_kernel(const bf16_t* __restrict__ x,
                                                            const bf16_t* __restrict__ wp,  // [Cout][4][4][Cin]
                                                            const float* __restrict__ bias,
                                                            bf16_t* __restrict__ y, TconvHaloGrid g) {
    extern __shared__ uint4 thlds[];
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

    // this wave's phase, its first position row, and its four taps: weight tap
    // index kh*4 + kw and the window pixel of position (r0, 0) for that tap
    const int ph_h = (wave >> 1) & 1, ph_w = wave & 1, r0 = kThRows * (wave >> 2);
    const int k0h = (ph_h + g.pad) & 1, bh = (ph_h + g.pad) >> 1;
    const int k0w = (ph_w + g.pad) & 1, bw = (ph_w + g.pad) >> 1;
    int tapk[4], tapo[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
        const int jh = t >> 1, jw = t & 1;
        tapk[t] = (k0h + 2 * jh) * 4 + k0w + 2 * jw;
        tapo[t] = (r0 + bh - jh - g.lo) * kTwWin + (bw - jw - g.lo);
    }

    f32x16 acc[kThRows];
#pragma unroll
    for (int r = 0; r < kThRows; ++r) acc[r] = f32x16{};
    th_stage(thlds, thlds + kThWUnits, g, wr, xr, 0, co0, n, ih0, iw0, wave, lane);
    if (g.nchunk > 1) th_stage(thlds + kThBuf, thlds + kThBuf + kThWUnits, g, wr, xr, 1, co0, n, ih0, iw0, wave, lane);
    int bc = 0;   // buffer of chunk kc
    for (int kc = 0; kc < g.nchunk; ++kc) {
        // this wave's copies of chunk kc have landed (those of kc+1 may still
        // be in flight: loads complete in order), then the barrier for
        // everyone's; it also frees the buffer of chunk kc-1 for chunk kc+2
        if (kc + 1 < g.nchunk) __builtin_amdgcn_s_waitcnt(0x0f77);  // vmcnt(7)
        else __builtin_amdgcn_s_waitcnt(0x0f70);                    // vmcnt(0)
        th_barrier();
        const int bn = bc == 0 ? 2 : bc - 1;   // buffer of chunk kc+2 (= that of kc-1)
        uint4* const cur = thlds + bc * kThBuf;
        uint4* const nxt = thlds + bn * kThBuf;
        th_chunk(cur, cur + kThWUnits, nxt, nxt + kThWUnits, acc, g, wr, xr, kc + 2 < g.nchunk ? kc + 2 : -1,
                 co0, n, ih0, iw0, wave, lane, tapk, tapo);
        bc = bc == 2 ? 0 : bc + 1;
    }

    // epilogue: lane holds position (r, lane % 32), output channels
    // 8q + 4*(lane/32) + (0..3) in acc[r][4q + 0..3]
    const __amdgpu_buffer_rsrc_t br = make_rsrc(bias, BIAS ? (uint32_t)g.Cout * 4u : 0u);
    float4 b4[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const int co = co0 + 8 * q + 4 * (lane >> 5);
        b4[q] = make_float4(0.f, 0.f, 0.f, 0.f);
        if (BIAS) b4[q] = __builtin_bit_cast(float4, load16(br, co < g.Cout ? co * 4 : kOOB));
    }
    if (g.Cout % 8 == 0) {
        // Two lane swaps regroup a row's 32 x 32 block so that each lane holds
        // 8 consecutive channels (16 bytes) of one position: channels
        // co0 + cl .. +7 of position 16*h + lane % 16 (h = 0, 1), and one
        // store instruction writes 64 contiguous bytes of each of 16 pixels,
        // with the streaming (nt) policy (measured 46.1 -> 39.7 us on the
        // 4x4 stride-2 256->128 layer against 8-byte stores).
        const int cl = ((lane >> 4) & 1) * 16 + (lane >> 5) * 8;
#pragma unroll
        for (int r = 0; r < kThRows; ++r) {
            const int oh = 2 * (u0 + r0 + r) + ph_h;
            uint32_t pk[4][2];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                float v[4] = {acc[r][4 * q] + b4[q].x, acc[r][4 * q + 1] + b4[q].y, acc[r][4 * q + 2] + b4[q].z,
                              acc[r][4 * q + 3] + b4[q].w};
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
            uint32_t out[2][4];
#pragma unroll
            for (int d = 0; d < 4; ++d) {
                const auto sw = __builtin_amdgcn_permlane16_swap(r8[0][d], r8[1][d], false, false);
                out[0][d] = sw[0];
                out[1][d] = sw[1];
            }
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const int ow = 2 * (v0 + 16 * h + (lane & 15)) + ph_w;
                const int co = co0 + cl;
                const bool ok = oh < g.Ho && ow < g.Wo && co < g.Cout;
                store16<kStoreStream>(yr, ok ? (((n * g.Ho + oh) * g.Wo + ow) * g.Cout + co) * 2 : kOOB,
                                      make_uint4(out[h][0], out[h][1], out[h][2], out[h][3]));
            }
        }
        return;
    }
    const int ow = 2 * (v0 + (lane & 31)) + ph_w;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const int co = co0 + 8 * q + 4 * (lane >> 5);
#pragma unroll
        for (int r = 0; r < kThRows; ++r) {
            const int oh = 2 * (u0 + r0 + r) + ph_h;
            float v[4] = {acc[r][4 * q] + b4[q].x, acc[r][4 * q + 1] + b4[q].y, acc[r][4 * q + 2] + b4[q].z,
                          acc[r][4 * q + 3] + b4[q].w};
            if (RELU)
#pragma unroll
                for (int i = 0; i < 4; ++i) v[i] = fmaxf(v[i], 0.0f);
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
    g.nchunk = s.Cin / 32;
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
