// pointwise.hip -- 1x1 convolution (stride 1, no padding, one group) as a
// streaming GEMM for the bandwidth-bound shapes.
//
// A 1x1 convolution is exactly a GEMM (lincklin.cn lesson 9, sections 21-22;
// lpnh.cn section 4.3): with channels-last input the activation is a
// row-major [N*H*W][Cin] matrix, and y[p][co] = sum_ci x[p][ci] * w[co][ci].
// At the channel counts of the workloads the arithmetic intensity is 20-50
// FLOP per byte, far below the matrix cores' ridge point, so the kernel is
// built around the memory stream:
//  * the whole weight matrix is staged in LDS once per workgroup (rows at an
//    odd pitch of 16-byte units, so the 16 rows read together by a quarter
//    wave land in 16 distinct bank slots);
//  * every wave walks its own 32-pixel tiles with no barrier; a tile's
//    activations are loaded straight into MFMA operand registers (lane l
//    holds 8 channels of pixel l % 32), one tile ahead of the one being
//    computed;
//  * v_mfma_f32_32x32x16_bf16 per 32 output channels and 16 input channels,
//    fp32 accumulators initialised with the bias;
//  * the same register epilogue as the halo kernel: ReLU, bf16, two lane
//    swaps, and stores of 64 contiguous bytes per pixel per instruction.
#include "mfma.hpp"
#include "../../include/conv2d.h"

namespace conv2d {

namespace {

constexpr int kPwThreads = 256;
constexpr int kPwMaxLds = 64 * 1024;  // bytes of staged weights
constexpr int kPwMaxCout = 256;

// Row pitch of the staged weights in 16-byte units: odd.
__host__ __device__ constexpr int pw_pitch(int cin) { return ((cin + 7) / 8) | 1; }

// MB: 32-row blocks of output channels per work item; KS: 16-channel slices
// of the input (Cin <= 16*KS).  A work item is one 32-pixel tile and one
// group of MB*32 output channels (nmh groups cover Cout); the items of one
// tile are consecutive, so the later ones find its activations in cache.
template <int MB, int KS>
__global__ __launch_bounds__(kPwThreads, 2) void pw_kernel(const bf16_t* __restrict__ x,
                                                       const bf16_t* __restrict__ wp,
                                                       const float* __restrict__ bias,
                                                       bf16_t* __restrict__ y, int npix, int cin,
                                                       int cout, int ntiles, int nmh, int has_bias,
                                                       int relu) {
    __shared__ uint4 wl[kPwMaxLds / 16];
    __shared__ __align__(16) float sb[kPwMaxCout];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int P = pw_pitch(cin);

    // stage the weights (rows past Cout and channels past Cin are zero) and
    // the bias
    const int rows = nmh * MB * 32;
    {
        // all loads first (zero for padding units), then the LDS stores, so
        // the staging costs one memory latency
        constexpr int kUnits = kPwMaxLds / 16 / kPwThreads;
        const __amdgpu_buffer_rsrc_t wr = make_rsrc(wp, (uint32_t)cout * (uint32_t)cin * 2u);
        uint4 v[kUnits];
#pragma unroll
        for (int k = 0; k < kUnits; ++k) {
            const int u = tid + k * kPwThreads;
            const int r = u / P, c = u - r * P;
            v[k] = load16(wr, (u < rows * P && r < cout && c * 8 < cin) ? (r * cin + c * 8) * 2 : kOOB);
        }
#pragma unroll
        for (int k = 0; k < kUnits; ++k) {
            const int u = tid + k * kPwThreads;
            if (u < rows * P) wl[u] = v[k];
        }
    }
    for (int i = tid; i < rows; i += kPwThreads) sb[i] = (has_bias && i < cout) ? bias[i] : 0.0f;
    __syncthreads();

    const __amdgpu_buffer_rsrc_t xr = make_rsrc(x, (uint32_t)npix * (uint32_t)cin * 2u);
    const __amdgpu_buffer_rsrc_t yr = make_rsrc(y, (uint32_t)npix * (uint32_t)cout * 2u);
    const int frow = lane & 31, h = lane >> 5;
    // weight operand: row frow of block mb, 16-byte chunk 2s + h
    const char* const a_base = reinterpret_cast<const char*>(wl) + (frow * P + h) * 16;
    // epilogue: this lane's 16-byte piece holds channels cl .. cl+7 of a
    // 32-channel block, of pixel 16*e + lane % 16 (e = 0, 1) of the tile
    const int cl = ((lane >> 4) & 1) * 16 + h * 8;
    const bool vec16 = cout % 8 == 0;

    const int nw = gridDim.x * (kPwThreads / 64);
    const int w0 = blockIdx.x * (kPwThreads / 64) + wave;
    const int nitems = ntiles * nmh;

    uint4 b0[KS], b1[KS];
    f32x16 acc[MB];

    // activations of tile T: lane supplies pixel T*32 + lane % 32, channels
    // 16 s + 8 (lane / 32) .. +7 (zero past the image or past Cin)
#define PW_LOAD(B, I)                                                                        \
    do {                                                                                     \
        const int p_ = ((I) / nmh) * 32 + frow;                                              \
        const bool pin_ = (I) < nitems && p_ < npix;                                         \
        _Pragma("unroll") for (int s = 0; s < KS; ++s) {                                     \
            const bool ok_ = pin_ && s * 16 + 8 * h < cin;                                   \
            (B)[s] = load16(xr, ok_ ? (p_ * cin + s * 16 + 8 * h) * 2 : kOOB);               \
        }                                                                                    \
    } while (0)

    // one tile: bias-initialised accumulators, KS x MB matrix ops, epilogue
#define PW_TILE(B, I)                                                                        \
    do {                                                                                     \
        const int T = (I) / nmh, c0_ = ((I) - T * nmh) * (MB * 32);                          \
        _Pragma("unroll") for (int mb = 0; mb < MB; ++mb)                                    \
            _Pragma("unroll") for (int q = 0; q < 4; ++q) {                                  \
                const float4 b4_ = *reinterpret_cast<const float4*>(&sb[c0_ + mb * 32 + 8 * q + 4 * h]); \
                acc[mb][4 * q + 0] = b4_.x;                                                  \
                acc[mb][4 * q + 1] = b4_.y;                                                  \
                acc[mb][4 * q + 2] = b4_.z;                                                  \
                acc[mb][4 * q + 3] = b4_.w;                                                  \
            }                                                                                \
        _Pragma("unroll") for (int s = 0; s < KS; ++s)                                       \
            _Pragma("unroll") for (int mb = 0; mb < MB; ++mb) {                              \
                const bf16x8 a_ = *reinterpret_cast<const bf16x8*>(a_base + ((c0_ + mb * 32) * P + 2 * s) * 16); \
                acc[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a_, __builtin_bit_cast(bf16x8, (B)[s]), \
                                                                 acc[mb], 0, 0, 0);          \
            }                                                                                \
        int pix_[2];                                                                         \
        _Pragma("unroll") for (int e = 0; e < 2; ++e) {                                      \
            const int p_ = (T) * 32 + 16 * e + (lane & 15);                                  \
            pix_[e] = p_ < npix ? p_ * cout : -1;                                            \
        }                                                                                    \
        _Pragma("unroll") for (int mb = 0; mb < MB; ++mb) {                                  \
            uint32_t pk_[4][2];                                                              \
            _Pragma("unroll") for (int q = 0; q < 4; ++q) {                                  \
                float v_[4];                                                                 \
                _Pragma("unroll") for (int r = 0; r < 4; ++r) {                              \
                    v_[r] = acc[mb][4 * q + r];                                              \
                    if (relu) v_[r] = fmaxf(v_[r], 0.0f);                                    \
                }                                                                            \
                pk_[q][0] = pack_bf16x2(v_[0], v_[1]);                                       \
                pk_[q][1] = pack_bf16x2(v_[2], v_[3]);                                       \
            }                                                                                \
            uint32_t r8_[2][4];                                                              \
            _Pragma("unroll") for (int pr = 0; pr < 2; ++pr)                                 \
                _Pragma("unroll") for (int w = 0; w < 2; ++w) {                              \
                    const auto sw_ = __builtin_amdgcn_permlane32_swap(pk_[2 * pr][w], pk_[2 * pr + 1][w], false, false); \
                    r8_[pr][w] = sw_[0];                                                     \
                    r8_[pr][2 + w] = sw_[1];                                                 \
                }                                                                            \
            uint32_t o_[2][4];                                                               \
            _Pragma("unroll") for (int d = 0; d < 4; ++d) {                                  \
                const auto sw_ = __builtin_amdgcn_permlane16_swap(r8_[0][d], r8_[1][d], false, false); \
                o_[0][d] = sw_[0];                                                           \
                o_[1][d] = sw_[1];                                                           \
            }                                                                                \
            const int co_ = c0_ + mb * 32 + cl;                                              \
            _Pragma("unroll") for (int e = 0; e < 2; ++e) {                                  \
                const int off_ = (pix_[e] + co_) * 2;                                        \
                if (vec16) {                                                                 \
                    store16(yr, pix_[e] >= 0 && co_ < cout ? off_ : kOOB,                    \
                            make_uint4(o_[e][0], o_[e][1], o_[e][2], o_[e][3]));             \
                } else {                                                                     \
                    store8(yr, pix_[e] >= 0 && co_ < cout ? off_ : kOOB, make_uint2(o_[e][0], o_[e][1])); \
                    store8(yr, pix_[e] >= 0 && co_ + 4 < cout ? off_ + 8 : kOOB,             \
                           make_uint2(o_[e][2], o_[e][3]));                                  \
                }                                                                            \
            }                                                                                \
        }                                                                                    \
    } while (0)

    // Two tiles per iteration so the two register sets alternate statically;
    // the loads of the tile after next go out before a tile is computed.
    int it = w0;
    PW_LOAD(b0, it);
    for (; it < nitems; it += 2 * nw) {
        PW_LOAD(b1, it + nw);
        __builtin_amdgcn_sched_barrier(0);
        PW_TILE(b0, it);
        if (it + nw >= nitems) break;
        PW_LOAD(b0, it + 2 * nw);
        __builtin_amdgcn_sched_barrier(0);
        PW_TILE(b1, it + nw);
    }
#undef PW_LOAD
#undef PW_TILE
}

template <int MB, int KS>
hipError_t launch_pw(const Shape& s, const bf16_t* x, const bf16_t* w, const float* b, bf16_t* y,
                     hipStream_t st) {
    auto kern = pw_kernel<MB, KS>;
    const int npix = s.N * s.Ho * s.Wo;
    const int ntiles = (npix + 31) / 32;
    const int nmh = (s.Cout + MB * 32 - 1) / (MB * 32);
    int dev = 0;
    (void)hipGetDevice(&dev);
    const long long resident = (long long)cu_count(dev) * blocks_per_cu(kern, kPwThreads, dev);
    const long long want = ((long long)ntiles * nmh + 3) / 4;
    const int grid = (int)(want < resident ? want : resident);
    hipLaunchKernelGGL(kern, dim3(grid), dim3(kPwThreads), 0, st, x, w, b, y, npix, s.Cin, s.Cout, ntiles, nmh,
                       (s.epilogue & CONV2D_EPI_BIAS) ? 1 : 0, (s.epilogue & CONV2D_EPI_RELU) ? 1 : 0);
    return hipGetLastError();
}

template <int MB>
hipError_t launch_pw_ks(const Shape& s, const bf16_t* x, const bf16_t* w, const float* b, bf16_t* y,
                        hipStream_t st) {
    const int ks = (s.Cin + 15) / 16;
    if (ks <= 4) return launch_pw<MB, 4>(s, x, w, b, y, st);
    if (ks <= 8) return launch_pw<MB, 8>(s, x, w, b, y, st);
    if (ks <= 12) return launch_pw<MB, 12>(s, x, w, b, y, st);
    return launch_pw<MB, 16>(s, x, w, b, y, st);
}

}  // namespace

// 32-row output-channel blocks per work item (the launcher's choice).
int pw_blocks(int cout) {
    const int mb = (cout + 31) / 32;
    return mb <= 1 ? 1 : mb <= 2 ? 2 : 4;
}

bool pointwise_supports(const Shape& s) {
    const long long npix = (long long)s.N * s.Ho * s.Wo;
    const int mb = pw_blocks(s.Cout);
    const long long rows = (long long)(s.Cout + mb * 32 - 1) / (mb * 32) * (mb * 32);
    return s.Kh == 1 && s.Kw == 1 && s.stride == 1 && s.pad == 0 && s.groups == 1 && s.dtype == CONV2D_BF16 &&
           s.Cin % 8 == 0 && s.Cin <= 256 && s.Cout % 4 == 0 && s.Cout <= kPwMaxCout &&
           rows * pw_pitch(s.Cin) * 16 <= kPwMaxLds &&
           npix * s.Cin * 2 < 0x7fff0000LL && npix * s.Cout * 2 < 0x7fff0000LL;
}

hipError_t launch_pointwise(const Shape& s, const void* x, const void* w_packed, const float* bias,
                            void* y, hipStream_t st) {
    (void)hipGetLastError();  // report only this launch's error
    if (!pointwise_supports(s)) return hipErrorInvalidValue;
    const bf16_t* xt = static_cast<const bf16_t*>(x);
    const bf16_t* wt = static_cast<const bf16_t*>(w_packed);
    bf16_t* yt = static_cast<bf16_t*>(y);
    const int mb = pw_blocks(s.Cout);
    if (mb == 1) return launch_pw_ks<1>(s, xt, wt, bias, yt, st);
    if (mb == 2) return launch_pw_ks<2>(s, xt, wt, bias, yt, st);
    return launch_pw_ks<4>(s, xt, wt, bias, yt, st);
}

}  // namespace conv2d
