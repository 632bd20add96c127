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
// channels; 4 waves, wave w owns output channels 32*(w/2).. and block rows
// 4*(w%2).. of the 8x8, i.e. one 32x32 MFMA tile for each of the 16 xi (256
// fp32 accumulators per lane).  Input channels are walked in chunks of 16:
//   - V of the chunk ([16 xi][2 halves][64 co][8 c] bf16, 32 KB) and the
//     18x18 input patch ([18][18][2 halves][8 c], 10 KB) are copied into LDS
//     with buffer-to-LDS loads, double-buffered: the next chunk's copies are
//     in flight while this one computes;
//   - each lane transforms the 4x4 patch of its own block for its 8 channels
//     in registers (B^T d B, fp32 adds, one bf16 rounding) -- exactly the MFMA
//     B operand of that lane for each xi, so U never goes through memory;
//   - 16 MFMAs, one per xi.
// After the last chunk every lane holds all 16 M_xi of its (channel, block)
// pairs, so the output transform A^T M A, bias, ReLU and the bf16 rounding
// happen in registers before one store per output.
#include "mfma.hpp"
#include "../../include/conv2d.h"

namespace conv2d {

namespace {

constexpr int kWThreads = 256;
constexpr int kWBlk = 8;                          // output blocks per workgroup side
constexpr int kWCo = 64;                          // output channels per workgroup
constexpr int kWPatch = 2 * kWBlk + 2;            // input patch side: 18
constexpr int kWXSlots = kWPatch * kWPatch * 2;   // 16-byte units of one patch chunk: 648
constexpr int kWXPad = (kWXSlots + 63) / 64 * 64; // whole waves of units: 704
constexpr int kWVSlots = 16 * 2 * kWCo;           // 16-byte units of one V chunk: 2048
constexpr int kWBuf = kWVSlots + kWXPad;          // units per buffer
constexpr int kWLds = 2 * kWBuf * 16;             // bytes of dynamic LDS: 88064

struct WinoGrid {
    int N, Cin, H, W, Cout, pad, Ho, Wo;
    int C8;            // Cin / 8
    int nbr, nbc;      // 8x8-block groups per image (rows, columns)
    int ncb;           // 64-channel output groups
    int nchunk;        // 16-channel input chunks
    int bias, relu;
};

typedef __attribute__((address_space(3))) void* lds_ptr_t;

// Copy chunk kc (input channels 16*kc ..) of V and of the input patch into
// one LDS buffer.  V: unit (xi, half, co) -> one wave instruction per (xi,
// half), lane = output channel.  Patch: unit ((row*18 + col)*2 + half) ->
// eleven wave instructions of 64 consecutive units.  Units past the tensor
// (output channels >= Cout, channels >= Cin, pixels outside the image) read 0.
__device__ __forceinline__ void wino_stage(uint4* __restrict__ vdst, uint4* __restrict__ xdst, const WinoGrid& g,
                                           __amdgpu_buffer_rsrc_t vr, __amdgpu_buffer_rsrc_t xr, int kc, int co0,
                                           int n, int ih0, int iw0, int wave, int lane) {
    const int co = co0 + lane;
#pragma unroll
    for (int m = 0; m < 8; ++m) {
        const int i = wave + 4 * m;             // (xi, half) pair
        const int xi = i >> 1, half = i & 1;
        const int cg = 2 * kc + half;           // 8-channel group of the whole input
        const bool ok = co < g.Cout && cg < g.C8;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(vr, (lds_ptr_t)(vdst + i * 64),
                                                 16, ok ? ((xi * g.C8 + cg) * g.Cout + co) * 16 : kOOB, 0, 0, 0);
    }
#pragma unroll
    for (int m = 0; m < 3; ++m) {
        const int k = wave + 4 * m;
        if (k * 64 >= kWXPad) break;
        const int s = k * 64 + lane;
        const int p = s >> 1, half = s & 1;
        const int row = p / kWPatch, col = p - row * kWPatch;
        const int ih = ih0 + row, iw = iw0 + col;
        const int cg = 2 * kc + half;
        const bool ok = s < kWXSlots && (unsigned)ih < (unsigned)g.H && (unsigned)iw < (unsigned)g.W && cg < g.C8;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(xr, (lds_ptr_t)(xdst + k * 64), 16,
                                                 ok ? (((n * g.H + ih) * g.W + iw) * g.C8 + cg) * 16 : kOOB, 0, 0, 0);
    }
}

__device__ __forceinline__ float blo(uint32_t u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float bhi(uint32_t u) { return __uint_as_float(u & 0xffff0000u); }

// 8 bf16 (one 16-byte unit) -> 8 fp32
__device__ __forceinline__ void unpack8(const uint4& v, float f[8]) {
    f[0] = blo(v.x); f[1] = bhi(v.x); f[2] = blo(v.y); f[3] = bhi(v.y);
    f[4] = blo(v.z); f[5] = bhi(v.z); f[6] = blo(v.w); f[7] = bhi(v.w);
}

__device__ __forceinline__ bf16x8 pack8(const float f[8]) {
    const uint4 u = make_uint4(pack_bf16x2(f[0], f[1]), pack_bf16x2(f[2], f[3]), pack_bf16x2(f[4], f[5]),
                               pack_bf16x2(f[6], f[7]));
    return __builtin_bit_cast(bf16x8, u);
}

// One chunk: start copying the next chunk (next >= 0) into (vn, xn), then
// for this lane's block and 8 channels: U = B^T d B, and acc[xi] += V_xi U_xi.
// Each LDS buffer is its own restrict argument, so the compiler does not
// wait for the copies in flight before reading the current buffers.
__device__ __forceinline__ void wino_chunk(const uint4* __restrict__ vc, const uint4* __restrict__ xc,
                                           uint4* __restrict__ vn, uint4* __restrict__ xn, f32x16 acc[16],
                                           const WinoGrid& g, __amdgpu_buffer_rsrc_t vr, __amdgpu_buffer_rsrc_t xr,
                                           int next, int co0, int n, int ih0, int iw0, int wave, int lane,
                                           int xoff, int voff) {
    if (next >= 0) wino_stage(vn, xn, g, vr, xr, next, co0, n, ih0, iw0, wave, lane);
    // the 4x4 patch of this lane's block, rows a, columns b: units
    // ((2*tr + a)*18 + 2*tc + b)*2 + half
    uint4 d[4][4];
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int b = 0; b < 4; ++b) d[a][b] = xc[xoff + (a * kWPatch + b) * 2];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        bf16x8 av[4];   // V of xi = 4i .. 4i+3 for this lane's output channel and 8 channels
#pragma unroll
        for (int j = 0; j < 4; ++j) av[j] = __builtin_bit_cast(bf16x8, vc[voff + (4 * i + j) * 2 * kWCo]);
        // row i of B^T d, per column b and channel
        float r[4][8];
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            float d0[8], d1[8], d2[8], d3[8];
            unpack8(d[0][b], d0);
            unpack8(d[1][b], d1);
            unpack8(d[2][b], d2);
            unpack8(d[3][b], d3);
#pragma unroll
            for (int c = 0; c < 8; ++c) {
                if (i == 0) r[b][c] = d0[c] - d2[c];
                else if (i == 1) r[b][c] = d1[c] + d2[c];
                else if (i == 2) r[b][c] = d2[c] - d1[c];
                else r[b][c] = d1[c] - d3[c];
            }
        }
        // (B^T d B)[i][j] = the same combination of the row's columns
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            float u[8];
#pragma unroll
            for (int c = 0; c < 8; ++c) {
                if (j == 0) u[c] = r[0][c] - r[2][c];
                else if (j == 1) u[c] = r[1][c] + r[2][c];
                else if (j == 2) u[c] = r[2][c] - r[1][c];
                else u[c] = r[1][c] - r[3][c];
            }
            const int xi = 4 * i + j;
            acc[xi] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av[j], pack8(u), acc[xi], 0, 0, 0);
        }
    }
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

    // this lane: MFMA column t = lane % 32 is its block (tr, tc) of the
    // wave's 4x8 blocks; half = lane / 32 its 8 channels of the chunk
    const int cb = wave >> 1, tb = wave & 1;
    const int t = lane & 31, half = lane >> 5;
    const int tr = 4 * tb + (t >> 3), tc = t & 7;
    const int xoff = ((2 * tr) * kWPatch + 2 * tc) * 2 + half;
    const int voff = half * kWCo + 32 * cb + t;   // + xi * 2 * 64: V row of output channel 32*cb + t

    f32x16 acc[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[i] = f32x16{};

    uint4* const buf0 = wlds;
    uint4* const buf1 = wlds + kWBuf;
    wino_stage(buf0, buf0 + kWVSlots, g, vr, xr, 0, co0, n, ih0, iw0, wave, lane);
    for (int kc = 0; kc < g.nchunk; ++kc) {
        // chunk kc has landed (each wave waits for its own copies, the barrier
        // for everyone's) and every wave is done with the other buffer
        __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0)
        __syncthreads();
        uint4* const cur = (kc & 1) ? buf1 : buf0;
        uint4* const nxt = (kc & 1) ? buf0 : buf1;
        wino_chunk(cur, cur + kWVSlots, nxt, nxt + kWVSlots, acc, g, vr, xr, kc + 1 < g.nchunk ? kc + 1 : -1, co0,
                   n, ih0, iw0, wave, lane, xoff, voff);
    }

    // Output transform.  MFMA result layout: lane l holds column l % 32 (its
    // block) and rows 8q + 4*(l/32) + r (output channels) in acc[xi][4q + r].
    const int oh = oh0 + 2 * tr, ow = ow0 + 2 * tc;
    const __amdgpu_buffer_rsrc_t br_ = make_rsrc(bias, (uint32_t)g.Cout * 4u);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const int co = co0 + 32 * cb + 8 * q + 4 * half;   // 4 consecutive output channels
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
            for (int xi = 0; xi < 16; ++xi) m[xi] = acc[xi][4 * q + r];
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
    g.nchunk = (s.Cin + 15) / 16;
    g.bias = (s.epilogue & CONV2D_EPI_BIAS) != 0;
    g.relu = (s.epilogue & CONV2D_EPI_RELU) != 0;
    return g;
}

template <bool BIAS, bool RELU>
hipError_t launch_w(const WinoGrid& g, const bf16_t* x, const bf16_t* v, const float* b, bf16_t* y, hipStream_t st) {
    static bool attr = false;   // dynamic LDS above 64 KB needs the kernel attribute once per process
    if (!attr) {
        const hipError_t e = hipFuncSetAttribute((const void*)wino_kernel<BIAS, RELU>,
                                                 hipFuncAttributeMaxDynamicSharedMemorySize, kWLds);
        if (e != hipSuccess) return e;
        attr = true;
    }
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
