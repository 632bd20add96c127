// winograd.hip -- 3x3 stride-1 convolution by Winograd's minimal filtering
// F(2x2, 3x3) on gfx950 bf16 MFMA ("lpnh.cn/news/2674933" section 3.3 and
// "lnrq.cn/news/4475" section 2.2: transform input and filter, multiply
// element-wise, transform back; 16 multiplications per 2x2 output block
// instead of 36).
//
// For a 2x2 output block with 4x4 input patch d and 3x3 filter g:
//   Y = A^T [ (G g G^T) (.) (B^T d B) ] A
//   B^T = [1 0 -1 0; 0 1 1 0; 0 -1 1 0; 0 1 0 -1]
//   G   = [1 0 0; 1/2 1/2 1/2; 1/2 -1/2 1/2; 0 0 1]
//   A^T = [1 1 1 0; 0 1 -1 -1]
// and summed over input channels: for each of the 16 positions xi of the
// 4x4 transformed block, M_xi[co][t] = sum_c V_xi[co][c] U_xi[c][t] is a GEMM
// (V = G g G^T per (co, c), U = B^T d B per (c, block t)).  The 16 GEMMs run
// on v_mfma_f32_32x32x16_bf16 with fp32 accumulation; U and V are rounded to
// bf16 (the only roundings besides the final one).
//
// Workgroup: 8x8 output blocks (16x16 outputs) of one image x 64 output
// channels; 4 waves, wave w owns block rows 2w, 2w+1 (16 blocks) and all 64
// output channels: for each of the 16 xi, four 16x16 MFMA tiles (16 output
// channels x 16 blocks; 256 fp32 accumulators per lane).  Input channels are
// walked in chunks of 32:
//   - V of the chunk ([16 xi][4 quarters][64 co][8 c] bf16, 64 KB) is copied
//     into LDS with buffer-to-LDS loads, double-buffered (the next chunk's
//     copy is in flight during this chunk); the 18x18 input patch of the
//     chunk ([18][18][4 quarters + 1 pad][8 c], 26 KB) is single-buffered:
//     its next copy starts once every wave has transformed this one;
//   - each lane transforms the 4x4 patch of its own block for its 8 channels
//     in registers (B^T d B, fp32 adds, one bf16 rounding) -- exactly that
//     lane's MFMA B operand for each xi, so U never goes through memory, and
//     every block is transformed once per workgroup;
//   - 64 MFMAs v_mfma_f32_16x16x32_bf16 (16 xi x 4 channel tiles).
// After the last chunk every lane holds all 16 M_xi of its (channel, block)
// pairs, so the output transform A^T M A, bias, ReLU and the bf16 rounding
// happen in registers before one store per output.
#include "mfma.hpp"
#include "../../include/conv2d.h"

namespace conv2d {

namespace {

constexpr int kWThreads = 256;
constexpr int kWBlk = 8;                            // output blocks per workgroup side
constexpr int kWCo = 64;                            // output channels per workgroup
constexpr int kWPatch = 2 * kWBlk + 2;              // input patch side: 18
constexpr int kWPix = 5;                            // 16-byte units per patch pixel: 4 quarters + 1 pad
constexpr int kWXUnits = kWPatch * kWPatch * kWPix; // 1620
constexpr int kWXPad = (kWXUnits + 63) / 64 * 64;   // whole waves of units: 1664
constexpr int kWVUnits = 16 * 4 * kWCo;             // 16-byte units of one V chunk: 4096
constexpr int kWLds = (2 * kWVUnits + kWXPad) * 16; // bytes of dynamic LDS: 157696

struct WinoGrid {
    int N, Cin, H, W, Cout, pad, Ho, Wo;
    int C8;            // Cin / 8
    int nbr, nbc;      // 8x8-block groups per image (rows, columns)
    int ncb;           // 64-channel output groups
    int nchunk;        // 32-channel input chunks
    int bias, relu;
};

typedef __attribute__((address_space(3))) void* lds_ptr_t;

// This wave's LDS operations complete, then the workgroup barrier; buffer
// loads in flight (copies into the other buffers) are not waited for.
__device__ __forceinline__ void lds_barrier() {
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0); vmcnt and expcnt at their maxima (no wait)
    __builtin_amdgcn_s_barrier();
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// Copy V of chunk kc (input channels 32*kc ..) into vdst: unit (xi, quarter,
// co), one wave instruction per (xi, quarter) with lane = output channel.
// Output channels >= Cout and channels >= Cin read 0.
__device__ __forceinline__ void wino_stage_v(uint4* __restrict__ vdst, const WinoGrid& g, __amdgpu_buffer_rsrc_t vr,
                                             int kc, int co0, int wave, int lane) {
    const int co = co0 + lane;
#pragma unroll
    for (int m = 0; m < 16; ++m) {
        const int i = wave + 4 * m;   // (xi, quarter)
        const int xi = i >> 2, qt = i & 3;
        const int cg = 4 * kc + qt;   // 8-channel group of the whole input
        const bool ok = co < g.Cout && cg < g.C8;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(vr, (lds_ptr_t)(vdst + i * 64), 16,
                                                 ok ? ((xi * g.C8 + cg) * g.Cout + co) * 16 : kOOB, 0, 0, 0);
    }
}

// Copy the input patch of chunk kc into xdst: unit pixel*5 + quarter (the
// fifth unit of a pixel is padding, so that neighbouring blocks' reads fall
// in different banks).  Pixels outside the image, channels >= Cin and the
// padding units read 0.
__device__ __forceinline__ void wino_stage_x(uint4* __restrict__ xdst, const WinoGrid& g, __amdgpu_buffer_rsrc_t xr,
                                             int kc, int n, int ih0, int iw0, int wave, int lane) {
#pragma unroll
    for (int m = 0; m < (kWXPad / 64 + 3) / 4; ++m) {
        const int k = wave + 4 * m;
        if (k * 64 >= kWXPad) break;
        const int s = k * 64 + lane;
        const int p = s / kWPix, qt = s - p * kWPix;
        const int row = p / kWPatch, col = p - row * kWPatch;
        const int ih = ih0 + row, iw = iw0 + col;
        const int cg = 4 * kc + qt;
        const bool ok = qt < 4 && p < kWPatch * kWPatch && (unsigned)ih < (unsigned)g.H &&
                        (unsigned)iw < (unsigned)g.W && cg < g.C8;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(xr, (lds_ptr_t)(xdst + k * 64), 16,
                                                 ok ? (((n * g.H + ih) * g.W + iw) * g.C8 + cg) * 16 : kOOB, 0, 0, 0);
    }
}

__device__ __forceinline__ float blo(uint32_t u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float bhi(uint32_t u) { return __uint_as_float(u & 0xffff0000u); }

// U = B^T d B for 2 channels (the two bf16 of 32-bit word w of each unit of
// the 4x4 patch d); out[xi] = the bf16 pair of U[xi] for those channels.
__device__ __forceinline__ void wino_transform2(const uint4 d[4][4], int w, uint32_t out[16]) {
    float lo_[4][4], hi_[4][4];
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            const uint32_t u = w == 0 ? d[a][b].x : w == 1 ? d[a][b].y : w == 2 ? d[a][b].z : d[a][b].w;
            lo_[a][b] = blo(u);
            hi_[a][b] = bhi(u);
        }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        float rl[4], rh[4];   // row i of B^T d
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            if (i == 0) { rl[b] = lo_[0][b] - lo_[2][b]; rh[b] = hi_[0][b] - hi_[2][b]; }
            else if (i == 1) { rl[b] = lo_[1][b] + lo_[2][b]; rh[b] = hi_[1][b] + hi_[2][b]; }
            else if (i == 2) { rl[b] = lo_[2][b] - lo_[1][b]; rh[b] = hi_[2][b] - hi_[1][b]; }
            else { rl[b] = lo_[1][b] - lo_[3][b]; rh[b] = hi_[1][b] - hi_[3][b]; }
        }
        out[4 * i + 0] = pack_bf16x2(rl[0] - rl[2], rh[0] - rh[2]);
        out[4 * i + 1] = pack_bf16x2(rl[1] + rl[2], rh[1] + rh[2]);
        out[4 * i + 2] = pack_bf16x2(rl[2] - rl[1], rh[2] - rh[1]);
        out[4 * i + 3] = pack_bf16x2(rl[1] - rl[3], rh[1] - rh[3]);
    }
}

// Read this lane's 4x4 patch (block (tr, tc), channel quarter kq) from the
// patch buffer and transform it: bo[xi] = the MFMA B operand of xi.
__device__ __forceinline__ void wino_transform(const uint4* __restrict__ xc, int xoff, bf16x8 bo[16]) {
    uint4 d[4][4];
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int b = 0; b < 4; ++b) d[a][b] = xc[xoff + (a * kWPatch + b) * kWPix];
    uint32_t u0[16], u1[16], u2[16], u3[16];
    wino_transform2(d, 0, u0);
    wino_transform2(d, 1, u1);
    wino_transform2(d, 2, u2);
    wino_transform2(d, 3, u3);
#pragma unroll
    for (int xi = 0; xi < 16; ++xi) bo[xi] = __builtin_bit_cast(bf16x8, make_uint4(u0[xi], u1[xi], u2[xi], u3[xi]));
}

// acc[xi][cb] += V_xi (output channels 16cb.., this chunk) x U_xi (16 blocks).
__device__ __forceinline__ void wino_mfma(const uint4* __restrict__ vc, int voff, const bf16x8 bo[16],
                                          f32x4 acc[16][4]) {
    // two-stage pipeline: the A operands of xi+1 are read while the MFMAs of
    // xi issue; the scheduling fence keeps the compiler from hoisting every
    // read to the front (64 operands would not fit in registers)
    bf16x8 av[2][4];
#pragma unroll
    for (int cb = 0; cb < 4; ++cb) av[0][cb] = __builtin_bit_cast(bf16x8, vc[voff + 16 * cb]);
#pragma unroll
    for (int xi = 0; xi < 16; ++xi) {
        if (xi + 1 < 16)
#pragma unroll
            for (int cb = 0; cb < 4; ++cb)
                av[(xi + 1) & 1][cb] = __builtin_bit_cast(bf16x8, vc[voff + (xi + 1) * 4 * kWCo + 16 * cb]);
#pragma unroll
        for (int cb = 0; cb < 4; ++cb)
            acc[xi][cb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av[xi & 1][cb], bo[xi], acc[xi][cb], 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
    }
}

// One chunk after its copies have landed: start the next chunk's V copy,
// transform the patch, release the patch buffer to the next chunk's copy,
// then the matrix products.  Every LDS buffer is its own restrict argument
// so the compiler does not wait for copies in flight into the others.
__device__ __forceinline__ void wino_chunk(const uint4* __restrict__ vc, uint4* __restrict__ vn,
                                           uint4* __restrict__ xb, f32x4 acc[16][4], const WinoGrid& g,
                                           __amdgpu_buffer_rsrc_t vr, __amdgpu_buffer_rsrc_t xr, int kc, int co0,
                                           int n, int ih0, int iw0, int wave, int lane, int xoff, int voff) {
    const bool more = kc + 1 < g.nchunk;
    if (more) wino_stage_v(vn, g, vr, kc + 1, co0, wave, lane);
    bf16x8 bo[16];
    wino_transform(xb, xoff, bo);
    lds_barrier();   // every wave has read the patch
    if (more) wino_stage_x(xb, g, xr, kc + 1, n, ih0, iw0, wave, lane);
    wino_mfma(vc, voff, bo, acc);
}

template <bool BIAS, bool RELU>
__global__ __launch_bounds__(kWThreads, 1) void wino_kernel(const bf16_t* __restrict__ x,
                                                            const bf16_t* __restrict__ v,  // [16][Cin/8][Cout][8]
                                                            const float* __restrict__ bias,
                                                            bf16_t* __restrict__ y, WinoGrid g) {
    extern __shared__ uint4 wlds[];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);

    int item = xcd_tile_index();
    const int cblk = item % g.ncb;   // output-channel group fastest: neighbours share the input patch
    item /= g.ncb;
    const int bc = item % g.nbc;
    item /= g.nbc;
    const int br = item % g.nbr;
    const int n = item / g.nbr;
    const int co0 = cblk * kWCo;
    const int oh0 = br * 2 * kWBlk, ow0 = bc * 2 * kWBlk;   // first output row/column of the group
    const int ih0 = oh0 - g.pad, iw0 = ow0 - g.pad;         // first input row/column of the patch

    const __amdgpu_buffer_rsrc_t xr = make_rsrc(x, (uint32_t)g.N * g.H * g.W * g.Cin * 2u);
    const __amdgpu_buffer_rsrc_t vr = make_rsrc(v, (uint32_t)16 * g.Cin * g.Cout * 2u);
    const __amdgpu_buffer_rsrc_t yr = make_rsrc(y, (uint32_t)g.N * g.Ho * g.Wo * g.Cout * 2u);

    // this lane: MFMA column t = lane % 16 is its block (tr, tc) of the
    // wave's 2x8 blocks; kq = lane / 16 its 8 channels of the chunk (the K
    // rows 8kq .. 8kq+7 of its A and B operands)
    const int t = lane & 15, kq = lane >> 4;
    const int tr = 2 * wave + (t >> 3), tc = t & 7;
    const int xoff = ((2 * tr) * kWPatch + 2 * tc) * kWPix + kq;
    const int voff = kq * kWCo + t;   // + xi*4*64 + 16*cb: V row of output channel 16*cb + t

    f32x4 acc[16][4];
#pragma unroll
    for (int i = 0; i < 16; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{};

    uint4* const v0 = wlds;
    uint4* const v1 = wlds + kWVUnits;
    uint4* const xb = wlds + 2 * kWVUnits;
    wino_stage_v(v0, g, vr, 0, co0, wave, lane);
    wino_stage_x(xb, g, xr, 0, n, ih0, iw0, wave, lane);
    for (int kc = 0; kc < g.nchunk; ++kc) {
        // chunk kc has landed (each wave waits for its own copies, the barrier
        // for everyone's) and every wave is done with the other V buffer
        __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0)
        __syncthreads();
        wino_chunk((kc & 1) ? v1 : v0, (kc & 1) ? v0 : v1, xb, acc, g, vr, xr, kc, co0, n, ih0, iw0, wave, lane,
                   xoff, voff);
    }

    // Output transform.  MFMA result layout: lane l holds column l % 16 (its
    // block) and rows 4*(l/16) + r of each 16-channel tile cb in acc[xi][cb][r].
    const int oh = oh0 + 2 * tr, ow = ow0 + 2 * tc;
    const __amdgpu_buffer_rsrc_t br_ = make_rsrc(bias, (uint32_t)g.Cout * 4u);
#pragma unroll
    for (int cb = 0; cb < 4; ++cb) {
        const int co = co0 + 16 * cb + 4 * kq;   // 4 consecutive output channels
        float bq[4] = {0.f, 0.f, 0.f, 0.f};
        if (BIAS) {
            const float4 b4 = __builtin_bit_cast(float4, load16(br_, co < g.Cout ? co * 4 : kOOB));
            bq[0] = b4.x; bq[1] = b4.y; bq[2] = b4.z; bq[3] = b4.w;
        }
        float out[4][4];  // [output (i, j) = 2i + j][channel r]
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            float m[16];
#pragma unroll
            for (int xi = 0; xi < 16; ++xi) m[xi] = acc[xi][cb][r];
            float z0[4], z1[4];   // A^T M
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                z0[j] = m[j] + m[4 + j] + m[8 + j];
                z1[j] = m[4 + j] - m[8 + j] - m[12 + j];
            }
            out[0][r] = z0[0] + z0[1] + z0[2] + bq[r];
            out[1][r] = z0[1] - z0[2] - z0[3] + bq[r];
            out[2][r] = z1[0] + z1[1] + z1[2] + bq[r];
            out[3][r] = z1[1] - z1[2] - z1[3] + bq[r];
        }
#pragma unroll
        for (int o = 0; o < 4; ++o) {
            const int yh = oh + (o >> 1), yw = ow + (o & 1);
            float* vv = out[o];
            if (RELU)
#pragma unroll
                for (int r = 0; r < 4; ++r) vv[r] = fmaxf(vv[r], 0.0f);
            const bool ok = yh < g.Ho && yw < g.Wo && co < g.Cout;
            store8(yr, ok ? (((n * g.Ho + yh) * g.Wo + yw) * g.Cout + co) * 2 : kOOB,
                   make_uint2(pack_bf16x2(vv[0], vv[1]), pack_bf16x2(vv[2], vv[3])));
        }
    }
}

// V = G g G^T of one (output channel, input channel) pair, rounded to bf16,
// into [16][Cin/8][Cout][8]; w is [Cout][Cin][3][3] bf16.
__global__ __launch_bounds__(kWThreads) void wino_weight_kernel(const bf16_t* __restrict__ w, bf16_t* __restrict__ v,
                                                                int Cout, int Cin) {
    const int idx = blockIdx.x * kWThreads + threadIdx.x;
    if (idx >= Cout * Cin) return;
    const int ci = idx % Cin, co = idx / Cin;
    float f[3][3];
#pragma unroll
    for (int a = 0; a < 3; ++a)
#pragma unroll
        for (int b = 0; b < 3; ++b) f[a][b] = bf16_to_f32(w[(idx * 3 + a) * 3 + b]);
    float gg[4][3];  // G g
#pragma unroll
    for (int b = 0; b < 3; ++b) {
        gg[0][b] = f[0][b];
        gg[1][b] = 0.5f * (f[0][b] + f[1][b] + f[2][b]);
        gg[2][b] = 0.5f * (f[0][b] - f[1][b] + f[2][b]);
        gg[3][b] = f[2][b];
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const float vv[4] = {gg[i][0], 0.5f * (gg[i][0] + gg[i][1] + gg[i][2]),
                             0.5f * (gg[i][0] - gg[i][1] + gg[i][2]), gg[i][2]};   // (G g) G^T
#pragma unroll
        for (int j = 0; j < 4; ++j)
            v[(((size_t)(4 * i + j) * (Cin / 8) + ci / 8) * Cout + co) * 8 + (ci & 7)] = f32_to_bf16(vv[j]);
    }
}

WinoGrid wino_grid(const Shape& s) {
    WinoGrid g;
    g.N = s.N; g.Cin = s.Cin; g.H = s.H; g.W = s.W; g.Cout = s.Cout; g.pad = s.pad; g.Ho = s.Ho; g.Wo = s.Wo;
    g.C8 = s.Cin / 8;
    const int bh = (s.Ho + 1) / 2, bw = (s.Wo + 1) / 2;   // 2x2 output blocks
    g.nbr = (bh + kWBlk - 1) / kWBlk;
    g.nbc = (bw + kWBlk - 1) / kWBlk;
    g.ncb = (s.Cout + kWCo - 1) / kWCo;
    g.nchunk = (s.Cin + 31) / 32;
    g.bias = (s.epilogue & CONV2D_EPI_BIAS) != 0;
    g.relu = (s.epilogue & CONV2D_EPI_RELU) != 0;
    return g;
}

template <bool BIAS, bool RELU>
hipError_t launch_w(const WinoGrid& g, const bf16_t* x, const bf16_t* v, const float* b, bf16_t* y, hipStream_t st) {
    int dev = 0;
    (void)hipGetDevice(&dev);
    const hipError_t ea = ensure_dynamic_lds<wino_kernel<BIAS, RELU>>(kWLds, dev);
    if (ea != hipSuccess) return ea;
    const long long blocks = (long long)g.N * g.nbr * g.nbc * g.ncb;
    hipLaunchKernelGGL((wino_kernel<BIAS, RELU>), dim3((unsigned)blocks), dim3(kWThreads), kWLds, st, x, v, b, y, g);
    return hipGetLastError();
}

}  // namespace

bool winograd_supports(const Shape& s) {
    const long long blocks = (long long)s.N * ((s.Ho + 15) / 16) * ((s.Wo + 15) / 16) * ((s.Cout + kWCo - 1) / kWCo);
    return s.dtype == CONV2D_BF16 && s.Kh == 3 && s.Kw == 3 && s.stride == 1 && s.dil == 1 && s.groups == 1 &&
           s.Cin % 8 == 0 && s.Cout % 4 == 0 && blocks < 0x7fffffffLL &&
           (long long)s.N * s.H * s.W * s.Cin * 2 < 0x7fff0000LL &&
           (long long)s.N * s.Ho * s.Wo * s.Cout * 2 < 0x7fff0000LL &&
           16LL * s.Cin * s.Cout * 2 < 0x7fff0000LL;
}

hipError_t launch_winograd(const Shape& s, const void* x, const void* v, const float* bias, void* y,
                           hipStream_t st) {
    (void)hipGetLastError();  // report only this launch's error
    if (!winograd_supports(s)) return hipErrorInvalidValue;
    const WinoGrid g = wino_grid(s);
    const bf16_t* xt = static_cast<const bf16_t*>(x);
    const bf16_t* vt = static_cast<const bf16_t*>(v);
    bf16_t* yt = static_cast<bf16_t*>(y);
    if (g.bias && g.relu) return launch_w<true, true>(g, xt, vt, bias, yt, st);
    if (g.bias) return launch_w<true, false>(g, xt, vt, bias, yt, st);
    if (g.relu) return launch_w<false, true>(g, xt, vt, bias, yt, st);
    return launch_w<false, false>(g, xt, vt, bias, yt, st);
}

hipError_t launch_winograd_weights(const void* w, void* v, int Cout, int Cin, hipStream_t st) {
    (void)hipGetLastError();
    const long long total = (long long)Cout * Cin;
    if (total >= 0x7fffffffLL || Cin % 8) return hipErrorInvalidValue;
    hipLaunchKernelGGL(wino_weight_kernel, dim3((unsigned)((total + kWThreads - 1) / kWThreads)), dim3(kWThreads), 0,
                       st, static_cast<const bf16_t*>(w), static_cast<bf16_t*>(v), Cout, Cin);
    return hipGetLastError();
}

}  // namespace conv2d
