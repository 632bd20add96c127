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
// never leaves the CU, and the block reads x once and writes y once.
//
// Input staging.  A band needs its input rows x CWI columns x C channels;
// each input row of it is one contiguous run of the NHWC tensor, copied as
// 16-byte units straight from memory into LDS (buffer loads to LDS, 64 units
// per wave instruction, one row per wave, no registers); units outside the
// image read zero, which is the zero padding.  Two staging buffers
// alternate: the next band's rows are in flight while this band is computed.
//
// Depthwise phase.  The threads form two halves, one per half of the band's
// rows.  Thread t of a half owns 4 channels, group t % (C/4) (their 3x3 taps
// stay in its registers), and column t / (C/4) of the band.  It reads its
// window rows from the staging buffer, runs the row arithmetic of dwrow.hpp
// (each input row prepared once and applied to the output rows that use it)
// and writes its results into the LDS tile [pixel][channel] (odd pitch of
// 16-byte units).  The value is rounded to bf16 after the depthwise bias and
// ReLU: the value a separate depthwise layer would store, so the fused result
// is the two-layer chain's.
//
// Pointwise phase.  The band's output is cut into blocks of 16 pixels x 16
// output channels, spread over all waves; each is a chain of
// v_mfma_f32_16x16x32_bf16 over the input channels, 32 at a time, with the
// weights [Cout][C] in LDS for the whole kernel and an fp32 accumulator
// initialised with the bias.  A lane ends with 4 consecutive output channels
// of one pixel: ReLU, bf16, one 8-byte store.
#include "dwrow.hpp"
#include "../../include/conv2d.h"

namespace conv2d {

namespace {

using namespace dwrow;

constexpr int kSepThreads = 1024;
constexpr int kSepWaves = kSepThreads / 64;
constexpr int kSepHalf = kSepThreads / 2;          // threads of one half of a band's rows
constexpr int kSepMaxC = 256;
constexpr int kSepMaxCout = 128;
constexpr int kSepLds = 163840 - kSepMaxCout * 4;  // dynamic LDS next to the static bias table

// Row pitch of the depthwise tile and of the pointwise weights in 16-byte
// units: odd (conflict-free operand reads) and covering whole 32-channel
// steps of the matrix op, so the units of the last step past C are zero
// units inside the row.
__host__ __device__ constexpr int sep_pitch(int c) { return (4 * ((c + 31) / 32)) | 1; }

// Output rows per band: seven at stride 1 (split 4 + 3 between the halves),
// three at stride 2 (2 + 1).
constexpr int sep_rows(int stride) { return stride == 1 ? 7 : 3; }

// Input rows staged per band: those of the RB output rows, plus, when RB is
// odd, those the second half reads for its unstored last row.
__host__ __device__ constexpr int sep_staged_rows(int S, int RB) { return (2 * ((RB + 1) / 2) - 1) * S + 3; }

struct SepGrid {
    int N, C, H, W, Ho, Wo, Cout, pad;
    int CW;             // output columns per band
    int nrb, ncb;       // row bands and column chunks per image
    int nitems;         // N * nrb * ncb
    int pblocks;        // 16-pixel blocks of one band
    int rowp;           // 16-byte units per staged input row (a multiple of 64)
    uint32_t cw_magic;  // ceil(2^32 / CW): p / CW == umulhi(p, cw_magic) for a band's pixels
    int dw_bias, pw_bias, pw_relu;  // (the depthwise ReLU is a template flag)
};

// This wave's LDS operations complete, then the workgroup barrier.  Buffer
// loads still in flight (the next band's staging) are not waited for.
__device__ __forceinline__ void lds_barrier() {
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0); vmcnt and expcnt at their maxima (no wait)
    __builtin_amdgcn_s_barrier();
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

typedef __attribute__((address_space(3))) void* lds_ptr_t;

// Copy the input rows of band `item` into staging buffer xs, one row per
// wave: row i of the band is the run of units [wi0 * C/8, wi0 * C/8 + rowp)
// of image row hb + i (units outside the row, or a row outside the image,
// read 0).
template <int S, int RB>
__device__ __forceinline__ void sep_stage(uint4* __restrict__ xs, const SepGrid& g, __amdgpu_buffer_rsrc_t xr,
                                          int item, int wave, int lane) {
    constexpr int NR = sep_staged_rows(S, RB);
    static_assert(NR <= kSepWaves, "one staged row per wave");
    if (wave >= NR) return;
    const int C8 = g.C >> 3;
    const int cb = item % g.ncb, t = item / g.ncb;
    const int rb = t % g.nrb, n = t / g.nrb;
    const int hi = rb * RB * S - g.pad + wave;
    const bool rin = (unsigned)hi < (unsigned)g.H;
    const int q0 = (cb * g.CW * S - g.pad) * C8 + lane;  // this lane's unit of the image row
    const int rowbase = (n * g.H + hi) * g.W * C8;
    uint4* const dst = xs + wave * g.rowp;
    for (int ch = 0; ch < g.rowp; ch += 64) {
        const int q = q0 + ch;
        const bool ok = rin && (unsigned)q < (unsigned)(g.W * C8);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(xr, (lds_ptr_t)(dst + ch), 16, ok ? (rowbase + q) * 16 : kOOB, 0, 0,
                                                 0);
    }
}

// One band: start the next band's staging (next >= 0), the depthwise phase
// from the staged rows xc into the tile dl, then the pointwise phase from dl
// with the weights wl and bias sb.  Every LDS buffer is a separate restrict
// argument, so the compiler can tell the staging copies in flight apart from
// the LDS accesses of this band and does not wait for them; the caller waits
// for a band's staging before passing it in.
template <int S, int RB, bool DWR>
__device__ __forceinline__ void sep_band(const uint4* __restrict__ xc, uint4* __restrict__ xn,
                                         uint4* __restrict__ dl, const uint4* __restrict__ wl,
                                         const float* __restrict__ sb, const SepGrid& g,
                                         __amdgpu_buffer_rsrc_t xr, __amdgpu_buffer_rsrc_t yr, int item, int next,
                                         const uint32_t (&wp)[3][4], const float (&w2)[3][4], const float (&b0)[4]) {
    constexpr int RA = (RB + 1) / 2;      // output rows of the first half (the second has RB - RA)
    constexpr int NA = (RA - 1) * S + 3;  // input rows one half reads
    const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int C = g.C, P = sep_pitch(C);
    const int cb = item % g.ncb, t = item / g.ncb;
    const int rb = t % g.nrb, n = t / g.nrb;
    const int ho0 = rb * RB, wo0 = cb * g.CW;
    if (next >= 0) sep_stage<S, RB>(xn, g, xr, next, wave, lane);

    // Depthwise: the two halves of the threads take output rows [0, RA) and
    // [RA, RB) of the band (when RB is odd, the second half's last row is
    // computed from staged rows past the band and not stored).
    const int C4 = C >> 2;
    const int cpp = kSepHalf / C4;  // columns per pass
    // (a half is whole waves: r0 is uniform, which the compiler is told)
    const int th = tid & (kSepHalf - 1), r0 = __builtin_amdgcn_readfirstlane(tid >= kSepHalf ? RA : 0);
    const int cg = th % C4, cpos = th / C4;
    if (cpos < cpp) {
        // LDS byte addresses: the window origin of the thread's column and the
        // tile pixel of its first output row, each advanced per pass; the
        // offsets of the window rows and taps, and of the tile rows, are
        // uniform
        const int rowb = g.rowp * 16, tapb = C * 2, colb = S * C * 2, trow = g.CW * P * 16;
        const char* xp = reinterpret_cast<const char*>(xc) + r0 * S * rowb + cpos * colb + cg * 8;
        char* dp = reinterpret_cast<char*>(dl) + (r0 * g.CW + cpos) * P * 16 + cg * 8;
        for (int c = cpos; c < g.CW; c += cpp, xp += cpp * colb, dp += cpp * P * 16) {
            V4 raw[NA][3];
#pragma unroll
            for (int i = 0; i < NA; ++i)
#pragma unroll
                for (int kk = 0; kk < 3; ++kk) raw[i][kk] = *reinterpret_cast<const V4*>(xp + i * rowb + kk * tapb);
            // every read of the window is issued before the first wait (left
            // to itself the compiler waits for each read before the next)
            __builtin_amdgcn_sched_barrier(0);
            // input rows in order: each is prepared once, applied to the (up
            // to three) output rows whose window covers it, and dropped; an
            // output row is finished and written to the tile with its last
            // filter row
            float acc[RA][4];
#pragma unroll
            for (int i = 0; i < NA; ++i) {
                RowXN<2> rx;
                prep_row(raw[i][0], raw[i][1], raw[i][2], rx);
#pragma unroll
                for (int r = 0; r < RA; ++r) {
                    const int kh = i - r * S;  // filter row of input row i for output row r0 + r
                    if (kh < 0 || kh > 2) continue;
                    if (kh == 0)
#pragma unroll
                        for (int q = 0; q < 4; ++q) acc[r][q] = b0[q];
                    row_fma(acc[r], rx, wp[kh], w2[kh]);
                    if (kh == 2 && (RB % 2 == 0 || r0 + r < RB))
                        *reinterpret_cast<uint2*>(dp + r * trow) =
                            make_uint2(pack_relu<DWR>(acc[r][0], acc[r][1]), pack_relu<DWR>(acc[r][2], acc[r][3]));
                }
            }
        }
    }
    lds_barrier();

    // Pointwise: block u is pixels 16 pb .. +15 and output channels
    // 16 cb .. +15 of the band.  Operands of step k (input channels 32 k ..
    // +31): weight row 16 cb + l % 16 and tile pixel 16 pb + l % 16, both at
    // unit 4 k + l / 16; the result in lane l is output channels 16 cb +
    // 4 (l / 16) .. +3 of pixel l % 16.
    const int lr = lane & 15, kq = lane >> 4;
    const int nk = (C + 31) / 32;          // 32-channel steps
    const int nblk = (g.Cout + 15) / 16;   // 16-channel output blocks
    for (int u = wave; u < g.pblocks * nblk; u += kSepWaves) {
        const int pb = u / nblk, cbk = u - pb * nblk;
        const char* ap = reinterpret_cast<const char*>(wl) + ((cbk * 16 + lr) * P + kq) * 16;
        const char* bp = reinterpret_cast<const char*>(dl) + ((pb * 16 + lr) * P + kq) * 16;
        const int co = cbk * 16 + 4 * kq;
        f32x4 acc = *reinterpret_cast<const f32x4*>(&sb[co]);
        for (int k = 0; k < nk; ++k, ap += 64, bp += 64)
            acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(*reinterpret_cast<const bf16x8*>(ap),
                                                         *reinterpret_cast<const bf16x8*>(bp), acc, 0, 0, 0);
        const int p = pb * 16 + lr;
        const int r = __umulhi(p, g.cw_magic), c = p - r * g.CW;
        const bool ok = r < RB && ho0 + r < g.Ho && wo0 + c < g.Wo && co < g.Cout;
        float v[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) v[q] = g.pw_relu ? fmaxf(acc[q], 0.0f) : acc[q];
        store8(yr, ok ? (((n * g.Ho + ho0 + r) * g.Wo + wo0 + c) * g.Cout + co) * 2 : kOOB,
               make_uint2(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])));
    }
}

// S: depthwise stride; RB: output rows per band; DWR: ReLU after the
// depthwise.
template <int S, int RB, bool DWR>
__global__ __launch_bounds__(kSepThreads, 4) void sep_kernel(const bf16_t* __restrict__ x,
                                                         const bf16_t* __restrict__ wdw,  // [3][3][C]
                                                         const float* __restrict__ bdw,
                                                         const bf16_t* __restrict__ wpw,  // [Cout][C]
                                                         const float* __restrict__ bpw,
                                                         bf16_t* __restrict__ y, SepGrid g) {
    constexpr int NR = sep_staged_rows(S, RB);
    // dynamic LDS: pointwise weights [rows][P] (rows = Cout rounded up to
    // 16); the band's depthwise output [pblocks * 16 pixels][P]; two staging
    // buffers [NR][rowp] of input rows
    extern __shared__ uint4 sep_lds[];
    __shared__ __align__(16) float sbp[kSepMaxCout];
    const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int C = g.C, C8 = C >> 3, P = sep_pitch(C);
    const int ROWS = (g.Cout + 15) / 16 * 16;
    uint4* const wl = sep_lds;
    uint4* const dl = wl + ROWS * P;
    uint4* const xin = dl + g.pblocks * 16 * P;
    const int xbuf = NR * g.rowp;  // units of one staging buffer
    const __amdgpu_buffer_rsrc_t xr = make_rsrc(x, (uint32_t)g.N * g.H * g.W * C * 2u);
    const __amdgpu_buffer_rsrc_t yr = make_rsrc(y, (uint32_t)g.N * g.Ho * g.Wo * g.Cout * 2u);

    const int first = xcd_tile_index();
    if (first < g.nitems) sep_stage<S, RB>(xin, g, xr, first, wave, lane);

    // Set-up in one memory round trip: every load (pointwise weights with
    // zero rows past Cout and zero units past C, the depthwise taps and bias
    // of this thread's 4 channels, the pointwise bias) goes out before the
    // first LDS store.
    constexpr int kU = (kSepMaxCout * sep_pitch(kSepMaxC) + kSepThreads - 1) / kSepThreads;
    const __amdgpu_buffer_rsrc_t wr = make_rsrc(wpw, (uint32_t)g.Cout * (uint32_t)C * 2u);
    uint4 v[kU];
#pragma unroll
    for (int k = 0; k < kU; ++k) {
        const int u = tid + k * kSepThreads;
        const int r = u / P, c = u - r * P;
        v[k] = load16(wr, (u < ROWS * P && r < g.Cout && c < C8) ? (r * C + c * 8) * 2 : kOOB);
    }
    const int cg = (tid & (kSepHalf - 1)) % (C >> 2);
    uint32_t wp[3][4];
    float w2[3][4], b0[4];
    load_taps<2>(wdw, C, cg * 4, wp, w2);
#pragma unroll
    for (int i = 0; i < 4; ++i) b0[i] = g.dw_bias ? bdw[cg * 4 + i] : 0.0f;
    const float bp = (g.pw_bias && tid < g.Cout) ? bpw[tid] : 0.0f;
#pragma unroll
    for (int k = 0; k < kU; ++k) {
        const int u = tid + k * kSepThreads;
        if (u < ROWS * P) wl[u] = v[k];
    }
    if (tid < kSepMaxCout) sbp[tid] = bp;
    // the pad units of every pixel of the depthwise tile are never written
    // by the depthwise phase: zero them once
    for (int p = tid; p < g.pblocks * 16; p += kSepThreads)
        for (int u = C8; u < P; ++u) dl[p * P + u] = make_uint4(0, 0, 0, 0);

    // consecutive logical blocks (those of one XCD) take consecutive bands,
    // which share their halo rows in that XCD's L2
    int k = 0;
    for (int item = first; item < g.nitems; item += gridDim.x, ++k) {
        const int b = k & 1;
        // this band's staging has landed: each wave waits for its own
        // copies, then the barrier (which also orders the previous band's
        // pointwise reads of the tile, and the first time the set-up stores)
        __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0)
        __syncthreads();
        const int next = item + (int)gridDim.x;
        sep_band<S, RB, DWR>(xin + b * xbuf, xin + (b ^ 1) * xbuf, dl, wl, sbp, g, xr, yr, item,
                                 next < g.nitems ? next : -1, wp, w2, b0);
    }
}

struct SepPlan {
    bool ok;
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
    const int S = s.stride, RB = sep_rows(S), NR = sep_staged_rows(S, RB), C8 = s.C / 8;
    const long long unit = (long long)sep_pitch(s.C) * 16;  // bytes per pixel of the tile
    const long long wbytes = (long long)(s.Cout + 15) / 16 * 16 * unit;
    // band width: at most one column per thread of a channel group and half,
    // and what LDS holds (weights, tile, two staging buffers)
    auto rowp_of = [&](int cw) { return ((((cw - 1) * S + 3) * C8 + 63) / 64) * 64; };
    auto lds_of = [&](int cw) {
        const long long pblocks = (RB * cw + 15) / 16;
        return wbytes + pblocks * 16 * unit + 2LL * NR * rowp_of(cw) * 16;
    };
    int cw = kSepHalf / (s.C / 4);
    if (cw > s.Wo) cw = s.Wo;
    while (cw > 0 && lds_of(cw) > kSepLds) --cw;
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
    g.pblocks = (RB * cw + 15) / 16;
    g.rowp = rowp_of(cw);
    g.cw_magic = (uint32_t)((0x100000000ULL + cw - 1) / cw);
    g.dw_bias = (s.dw_epilogue & CONV2D_EPI_BIAS) ? 1 : 0;
    g.pw_bias = (s.pw_epilogue & CONV2D_EPI_BIAS) ? 1 : 0;
    g.pw_relu = (s.pw_epilogue & CONV2D_EPI_RELU) ? 1 : 0;
    pl.lds = lds_of(cw);
    pl.ok = pl.lds <= kSepLds;
    return pl;
}

template <int S, bool DWR>
hipError_t launch_sep(const SepPlan& pl, const bf16_t* x, const bf16_t* wdw, const float* bdw, const bf16_t* wpw,
                      const float* bpw, bf16_t* y, hipStream_t st) {
    auto kern = sep_kernel<S, sep_rows(S), DWR>;
    int dev = 0;
    (void)hipGetDevice(&dev);
    const hipError_t ea = ensure_dynamic_lds<sep_kernel<S, sep_rows(S), DWR>>(kSepLds, dev);
    if (ea != hipSuccess) return ea;
    const int by_regs = blocks_per_cu<sep_kernel<S, sep_rows(S), DWR>>(kSepThreads, dev);
    const int by_lds = (int)(163840 / (pl.lds + kSepMaxCout * 4));
    const int bpc = by_lds < by_regs ? (by_lds < 1 ? 1 : by_lds) : by_regs;
    const long long resident = persistent_slots((long long)cu_count(dev) * bpc);
    const int grid = (int)(pl.g.nitems < resident ? pl.g.nitems : resident);
    hipLaunchKernelGGL(kern, dim3(grid), dim3(kSepThreads), (unsigned)pl.lds, st, x, wdw, bdw, wpw, bpw, y, pl.g);
    return hipGetLastError();
}

template <int S>
hipError_t launch_sep_relu(const SepShape& s, const SepPlan& pl, const bf16_t* x, const bf16_t* wdw,
                           const float* bdw, const bf16_t* wpw, const float* bpw, bf16_t* y, hipStream_t st) {
    if (s.dw_epilogue & CONV2D_EPI_RELU) return launch_sep<S, true>(pl, x, wdw, bdw, wpw, bpw, y, st);
    return launch_sep<S, false>(pl, x, wdw, bdw, wpw, bpw, y, st);
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
    if (s.stride == 1) return launch_sep_relu<1>(s, pl, xt, wd, b_dw, wq, b_pw, yt, st);
    return launch_sep_relu<2>(s, pl, xt, wd, b_dw, wq, b_pw, yt, st);
}

}  // namespace conv2d
