// igemm.hip -- implicit-GEMM convolution on gfx950 bf16 MFMA, and the 1x1
// convolution as a plain GEMM.
//
// GEMM view (lincklin.cn lesson 9, sections 7 and 19): per group g,
//   D[co][p] = sum_k  A[co][k] * B[k][p]
//   M = Cout/G (output channels), N = N*Ho*Wo (output pixels),
//   K = Kh*Kw*Cin/G ordered (kh, kw, ci) with ci fastest,
//   A = packed weight [Cout][Kh][Kw][Cin/G] (K-contiguous rows),
//   B[k][p] = X[n, hi, wi, g*Cin/G + ci] with hi = ho*S + kh*D - P,
//             wi = wo*S + kw*D - P, and 0 outside the image.
// B is never stored: its addresses are generated while the tile is loaded
// (implicit GEMM, lincklin.cn section 11; lpnh.cn section 3.3).  With
// channels-last input the Cin/G values of one tap are contiguous, so each
// K-step of 32 channels of one tap is a 64-byte contiguous read per pixel.
// Dilation only changes the tap offsets (kh*D, kw*D): exactly Kh*Kw taps are
// gathered, never a zero-filled dilated window (lpnh.cn section 4.2).  Zero
// padding is the address predicate (lincklin.cn section 26).
//
// Tiling.  A workgroup of 4 waves owns a BM x BN output tile (BM output
// channels x BN pixels) of one group.  Per K-step (one tap, 32 channels) it
// stages the BM x 32 weight slice and the BN x 32 im2col slice in LDS
// (double-buffered: the next step's global loads are in flight while the
// current step runs on the matrix cores), and each wave runs
// v_mfma_f32_16x16x32_bf16 on its (BM/WGM) x (BN/WGN) sub-tile.  fp32
// accumulators stay in registers for the whole K loop (output stationary,
// lincklin.cn section 15) and the epilogue adds the bias, applies ReLU,
// rounds to bf16 and stores once (lincklin.cn section 31).
//
// 1x1 / stride 1 / pad 0 / groups 1 (lincklin.cn sections 21-22; lpnh.cn
// section 4.3): B[k][p] = X[p][k], the NHWC activation read as a row-major
// [N*H*W][Cin] matrix -- a plain GEMM with no window arithmetic.
#include "common.hpp"
#include "../../include/conv2d.h"

namespace conv2d {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
constexpr int kBK = 32;           // K per step (one MFMA K)
constexpr int kChunks = kBK / 8;  // 16-byte chunks per LDS row

// LDS rows are 64 bytes (32 bf16).  The 16-byte chunk index is XOR-swizzled
// with the row so that the 16 rows one MFMA operand read touches spread over
// all banks.
__device__ __forceinline__ int swz(int row, int chunk) { return row * kChunks + (chunk ^ ((row >> 1) & 3)); }

template <int BM, int BN, int WGM, int WGN, bool IS1X1, bool BIAS, bool RELU>
__global__ __launch_bounds__(kThreads) void igemm_kernel(const bf16_t* __restrict__ x,
                                                         const bf16_t* __restrict__ wp,
                                                         const float* __restrict__ bias,
                                                         bf16_t* __restrict__ y, Shape s,
                                                         int n_ptiles, int n_ctiles) {
    constexpr int WTM = BM / WGM, WTN = BN / WGN;  // wave tile
    constexpr int TM = WTM / 16, TN = WTN / 16;    // MFMA tiles per wave
    constexpr int AQ = BM * kChunks, BQ = BN * kChunks;  // 16-byte vectors per step
    constexpr int AV = (AQ + kThreads - 1) / kThreads, BV = BQ / kThreads;
    static_assert(BQ % kThreads == 0, "B tile must split evenly");
    __shared__ uint4 lds[2][(BM + BN) * kChunks];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave / WGN, wn = wave % WGN;

    int bid = blockIdx.x;
    const int pt = bid % n_ptiles;
    bid /= n_ptiles;
    const int ct = bid % n_ctiles;
    const int g = bid / n_ctiles;

    const int npix = s.N * s.Ho * s.Wo;
    const int KK = s.Kh * s.Kw;
    const int nchunk = (s.cin_g + kBK - 1) / kBK;
    const int nsteps = KK * nchunk;
    const int co_tile = ct * BM;

    // ---- per-thread A (weight) load slots
    const bf16_t* a_src[AV];
    bool a_ok[AV];
    int a_lds[AV], a_c[AV];
#pragma unroll
    for (int i = 0; i < AV; ++i) {
        const int q = tid + i * kThreads;
        const int row = q / kChunks, ch = q % kChunks;
        const int co = co_tile + row;
        a_ok[i] = (q < AQ) && (co < s.cout_g);
        a_src[i] = wp + (size_t)(g * s.cout_g + (a_ok[i] ? co : 0)) * KK * s.cin_g + ch * 8;
        a_c[i] = ch * 8;
        a_lds[i] = swz(row, ch);
    }
    // ---- per-thread B (im2col) load slots
    int b_base[BV], b_hb[BV], b_wb[BV], b_lds[BV], b_c[BV];
    bool b_ok[BV];
#pragma unroll
    for (int i = 0; i < BV; ++i) {
        const int q = tid + i * kThreads;
        const int prow = q / kChunks, ch = q % kChunks;
        const int p = pt * BN + prow;
        b_ok[i] = p < npix;
        const int pp = b_ok[i] ? p : 0;
        const int wo = pp % s.Wo;
        const int t = pp / s.Wo;
        const int ho = t % s.Ho;
        const int n = t / s.Ho;
        if (IS1X1) {
            b_base[i] = pp * s.Cin + ch * 8;
            b_hb[i] = b_wb[i] = 0;
        } else {
            b_base[i] = n * s.H * s.W * s.Cin + g * s.cin_g + ch * 8;
            b_hb[i] = ho * s.stride - s.pad;
            b_wb[i] = wo * s.stride - s.pad;
        }
        b_c[i] = ch * 8;
        b_lds[i] = (BM + prow) * kChunks + (ch ^ ((prow >> 1) & 3));
    }

    uint4 ra[AV], rb[BV];
    const uint4 z4 = make_uint4(0, 0, 0, 0);

    // global -> registers for step (tap, c0)
    auto load_step = [&](int tap, int kh, int kw, int c0) {
#pragma unroll
        for (int i = 0; i < AV; ++i) {
            const bool ok = a_ok[i] && (c0 + a_c[i] < s.cin_g);
            ra[i] = ok ? *reinterpret_cast<const uint4*>(a_src[i] + tap * s.cin_g + c0) : z4;
        }
#pragma unroll
        for (int i = 0; i < BV; ++i) {
            bool ok = b_ok[i] && (c0 + b_c[i] < s.cin_g);
            int off;
            if (IS1X1) {
                off = b_base[i] + c0;
            } else {
                const int hi = b_hb[i] + kh * s.dil;
                const int wi = b_wb[i] + kw * s.dil;
                ok = ok && hi >= 0 && hi < s.H && wi >= 0 && wi < s.W;
                off = b_base[i] + (hi * s.W + wi) * s.Cin + c0;
            }
            rb[i] = ok ? *reinterpret_cast<const uint4*>(x + off) : z4;
        }
    };
    auto store_step = [&](int buf) {
#pragma unroll
        for (int i = 0; i < AV; ++i)
            if (tid + i * kThreads < AQ) lds[buf][a_lds[i]] = ra[i];
#pragma unroll
        for (int i = 0; i < BV; ++i) lds[buf][b_lds[i]] = rb[i];
    };

    f32x4 acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    // step counters: tap (kh, kw) outer, channel chunk inner
    int tap = 0, kh = 0, kw = 0, c0 = 0;
    load_step(tap, kh, kw, c0);
    store_step(0);
    __syncthreads();

    const int frow = lane & 15, fch = lane >> 4;
    for (int st = 0; st < nsteps; ++st) {
        const int buf = st & 1;
        const bool more = st + 1 < nsteps;
        if (more) {
            c0 += kBK;
            if (c0 >= s.cin_g) {
                c0 = 0;
                ++tap;
                if (++kw == s.Kw) { kw = 0; ++kh; }
            }
            load_step(tap, kh, kw, c0);
        }
        bf16x8 af[TM], bfr[TN];
#pragma unroll
        for (int i = 0; i < TM; ++i) {
            const int row = wm * WTM + i * 16 + frow;
            af[i] = __builtin_bit_cast(bf16x8, lds[buf][swz(row, fch)]);
        }
#pragma unroll
        for (int j = 0; j < TN; ++j) {
            const int prow = wn * WTN + j * 16 + frow;
            bfr[j] = __builtin_bit_cast(bf16x8, lds[buf][(BM + prow) * kChunks + (fch ^ ((prow >> 1) & 3))]);
        }
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
            for (int j = 0; j < TN; ++j)
                acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
        if (more) store_step(buf ^ 1);
        __syncthreads();
    }

    // ---- epilogue: lane holds D[co0 + r][p] for r = 0..3 (4 consecutive
    // output channels of one pixel) -> one 8-byte store per MFMA tile.
#pragma unroll
    for (int i = 0; i < TM; ++i) {
        const int co = co_tile + wm * WTM + i * 16 + 4 * (lane >> 4);
        if (co >= s.cout_g) continue;
        const int cg = g * s.cout_g + co;
        float b4[4] = {0.f, 0.f, 0.f, 0.f};
        if (BIAS) {
#pragma unroll
            for (int r = 0; r < 4; ++r) b4[r] = bias[cg + r];
        }
#pragma unroll
        for (int j = 0; j < TN; ++j) {
            const int p = pt * BN + wn * WTN + j * 16 + (lane & 15);
            if (p >= npix) continue;
            float v[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                v[r] = acc[i][j][r] + b4[r];
                if (RELU) v[r] = fmaxf(v[r], 0.0f);
            }
            uint2 o = make_uint2(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]));
            *reinterpret_cast<uint2*>(y + (size_t)p * s.Cout + cg) = o;
        }
    }
}

template <int BM, int BN, int WGM, int WGN, bool IS1X1>
hipError_t launch_cfg(const Shape& s, const bf16_t* x, const bf16_t* w, const float* b, bf16_t* y,
                      hipStream_t st) {
    const int npix = s.N * s.Ho * s.Wo;
    const int n_ptiles = (npix + BN - 1) / BN;
    const int n_ctiles = (s.cout_g + BM - 1) / BM;
    const long long blocks = (long long)n_ptiles * n_ctiles * s.groups;
    if (blocks > 0x7fffffffLL) return hipErrorInvalidConfiguration;
    dim3 grid((unsigned)blocks);
    const bool bias = s.epilogue & CONV2D_EPI_BIAS, relu = s.epilogue & CONV2D_EPI_RELU;
    if (bias && relu)
        hipLaunchKernelGGL((igemm_kernel<BM, BN, WGM, WGN, IS1X1, true, true>), grid, dim3(kThreads), 0, st, x, w, b, y, s, n_ptiles, n_ctiles);
    else if (bias)
        hipLaunchKernelGGL((igemm_kernel<BM, BN, WGM, WGN, IS1X1, true, false>), grid, dim3(kThreads), 0, st, x, w, b, y, s, n_ptiles, n_ctiles);
    else if (relu)
        hipLaunchKernelGGL((igemm_kernel<BM, BN, WGM, WGN, IS1X1, false, true>), grid, dim3(kThreads), 0, st, x, w, b, y, s, n_ptiles, n_ctiles);
    else
        hipLaunchKernelGGL((igemm_kernel<BM, BN, WGM, WGN, IS1X1, false, false>), grid, dim3(kThreads), 0, st, x, w, b, y, s, n_ptiles, n_ctiles);
    return hipGetLastError();
}

template <bool IS1X1>
hipError_t launch_any(const Shape& s, const void* x, const void* w, const float* b, void* y, hipStream_t st) {
    const bf16_t* xt = static_cast<const bf16_t*>(x);
    const bf16_t* wt = static_cast<const bf16_t*>(w);
    bf16_t* yt = static_cast<bf16_t*>(y);
    if (s.cout_g > 64) return launch_cfg<128, 128, 2, 2, IS1X1>(s, xt, wt, b, yt, st);
    if (s.cout_g > 32) return launch_cfg<64, 256, 1, 4, IS1X1>(s, xt, wt, b, yt, st);
    return launch_cfg<32, 256, 1, 4, IS1X1>(s, xt, wt, b, yt, st);
}

bool mfma_channels_ok(const Shape& s) {
    // 16-byte K vectors and 4-channel output stores
    return s.cin_g % 8 == 0 && s.cout_g % 4 == 0;
}

}  // namespace

bool igemm_supports(const Shape& s) { return mfma_channels_ok(s); }

bool gemm1x1_supports(const Shape& s) {
    return s.Kh == 1 && s.Kw == 1 && s.stride == 1 && s.pad == 0 && s.groups == 1 && mfma_channels_ok(s);
}

hipError_t launch_igemm(const Shape& s, const void* x, const void* w_packed, const float* bias,
                        void* y, hipStream_t st) {
    (void)hipGetLastError();  // report only this launch's error
    return launch_any<false>(s, x, w_packed, bias, y, st);
}

hipError_t launch_gemm1x1(const Shape& s, const void* x, const void* w_packed, const float* bias,
                          void* y, hipStream_t st) {
    (void)hipGetLastError();  // report only this launch's error
    return launch_any<true>(s, x, w_packed, bias, y, st);
}

}  // namespace conv2d
