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
//  * every wave walks its own 32-pixel tiles with no barrier.  A tile's
//    activations are one contiguous run of 32*Cin channels, fetched one tile
//    ahead with fully coalesced 1 KB loads, written to the wave's own LDS
//    region at an odd pixel pitch, and read back in MFMA operand layout
//    (lane l: 8 channels of pixel l % 32);
//  * v_mfma_f32_32x32x16_bf16 per 32 output channels and 16 input channels,
//    fp32 accumulators initialised with the bias;
//  * the same register epilogue as the halo kernel: ReLU, bf16, two lane
//    swaps, and stores of 64 contiguous bytes per pixel per instruction.
//
// Pixel-shuffle mode (SHUF): a transposed convolution whose kernel equals its
// stride (K = S, no padding, lpnh.cn sections 2.3 and 4.2) has windows that
// do not overlap, so Y = W^T X needs no col2im: input pixel (n, ih, iw) times
// weight row (tap, co) lands in output pixel (ih*S + kh, iw*S + kw), channel
// co, and every output receives exactly one such row.  The kernel then runs
// the same GEMM with Cout*S*S rows, ordered (tap, co) when the packed
// transposed weight [Cout][Kh][Kw][Cin] is staged, and the epilogue sends
// each row to its output pixel.
#include "mfma.hpp"
#include "../../include/conv2d.h"

namespace conv2d {

namespace {

constexpr int kPwThreads = 256;
constexpr int kPwWaves = kPwThreads / 64;
constexpr int kPwMaxLds = 64 * 1024;  // bytes of staged weights
constexpr int kPwMaxCout = 256;
constexpr int kPwMaxLdsShuf = 72 * 1024;
// How a wave's activations reach the matrix ops: straight into operand
// registers, through a whole tile in LDS, or through half tiles in LDS.
constexpr int kPwDirect = 0, kPwStaged = 1, kPwHalf = 2;  // staged weights in pixel-shuffle mode (256 rows x 17 units)
// Pixel-shuffle mode: activations through LDS (one workgroup per CU: 72 KB
// of weights plus the tiles) or straight into operand registers; overridable
// at build time for tuning.
#ifndef PW_SHUF_STAGED
#define PW_SHUF_STAGED 0
#endif

// Pixel-shuffle mode: output channels, kernel width, stride, input and
// output extents.
struct PwShuf {
    int cout, kk, kw, stride, h, w, ho, wo;
};

// Row pitch of the staged weights and activations in 16-byte units: odd (no
// bank conflicts), and at least two units per 16-channel slice, so the last
// slice's second half is a zero pad unit inside the row when Cin % 16 == 8.
__host__ __device__ constexpr int pw_pitch(int cin) { return (2 * ((cin + 15) / 16)) | 1; }

// Work items in flight per wave: register sets of KS 16-byte units each, as
// many as fit beside the accumulators (overridable at build time for tuning).
#ifndef PW_DEPTH4
#define PW_DEPTH4 6
#endif
#ifndef PW_DEPTH8
#define PW_DEPTH8 2
#endif
#ifndef PW_DEPTH12
#define PW_DEPTH12 2
#endif
#ifndef PW_DEPTH16
#define PW_DEPTH16 2
#endif
constexpr int pw_depth(int ks) {
    return ks <= 4 ? PW_DEPTH4 : ks <= 8 ? PW_DEPTH8 : ks <= 12 ? PW_DEPTH12 : PW_DEPTH16;
}

// MB: 32-row blocks of output channels per work item; KS: 16-channel slices
// of the input (Cin <= 16*KS).  A work item is one 32-pixel tile and one
// group of MB*32 output channels (nmh groups cover Cout); the items of one
// tile are consecutive, so the later ones find its activations in cache.
template <int MB, int KS, int STG, bool SHUF>
__global__ __launch_bounds__(kPwThreads, 2) void pw_kernel(const bf16_t* __restrict__ x,
                                                       const bf16_t* __restrict__ wp,
                                                       const float* __restrict__ bias,
                                                       bf16_t* __restrict__ y, int npix, int cin,
                                                       int cout, int ntiles, int nmh, int has_bias,
                                                       int relu, int cin8_magic, const float* scale,
                                                       const float* shift, PwShuf sh) {
    // dynamic LDS: weights [rows][P units], then one activation tile
    // [32 pixels][P units] per wave
    extern __shared__ uint4 pw_lds[];
    __shared__ __align__(16) float sb[kPwMaxCout];
    constexpr bool STAGED = STG == kPwStaged, HALF = STG == kPwHalf;
    static_assert(!HALF || KS % 2 == 0, "half tiles of whole 16-channel slices");
    constexpr int PH = KS + 1;  // HALF: pitch of a half-tile pixel row (odd)
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int P = pw_pitch(cin);
    const int XP = HALF ? PH : P;  // pitch of the wave's activation tile
    uint4* const wl = pw_lds;
    const int rows = nmh * MB * 32;  // staged weight rows

    const __amdgpu_buffer_rsrc_t xr = make_rsrc(x, (uint32_t)npix * (uint32_t)cin * 2u);
    const __amdgpu_buffer_rsrc_t yr = make_rsrc(y, (uint32_t)npix * (uint32_t)cout * 2u);
    const int frow = lane & 31, h = lane >> 5;
    // weight operand: row frow of block mb, 16-byte chunk 2s + h
    const char* const a_base = reinterpret_cast<const char*>(wl) + (frow * P + h) * 16;
    // this wave's activation tile; operand of slice s: pixel frow, chunk 2s + h
    char* const xt = reinterpret_cast<char*>(wl + rows * P + wave * 32 * XP);
    const char* const b_base = xt + (frow * XP + h) * 16;
    const int cin8 = cin / 8, tunits = 32 * cin8;  // 16-byte units of one tile
    // epilogue: this lane's 16-byte piece holds channels cl .. cl+7 of a
    // 32-channel block, of pixel 16*e + lane % 16 (e = 0, 1) of the tile
    const int cl = ((lane >> 4) & 1) * 16 + h * 8;
    const bool vec16 = cout % 8 == 0;
    // Output blocks in pairs (MB even, 16-byte pieces, no pixel shuffle):
    // two 32-channel blocks are merged with 8-lane row shifts (DPP) so that
    // each store instruction writes the 64 channels of 8 pixels, i.e. whole
    // 128-byte lines.  Streaming (nt) stores then add no partial-line writes
    // and free L2 for the activations (measured: 256->64 32.6 -> 30.0 us,
    // 64->256 33.4 -> 29.0 us).  Without the merge, streaming stores were
    // measured faster only for the pixel-shuffle epilogue and for outputs
    // narrower than 64 channels (the merge itself measured no faster for the
    // pixel-shuffle layer).
    const bool merged = MB % 2 == 0 && vec16 && !SHUF;
    const bool stream = SHUF || cout < 64 || merged;
    const Affine4 aff(scale, shift, cout);  // folded batch normalisation, when scale is given

    const int nw = gridDim.x * (kPwThreads / 64);
    const int w0 = blockIdx.x * (kPwThreads / 64) + wave;
    const int nitems = ntiles * nmh;
    constexpr int PD = pw_depth(KS);
    static_assert(PD >= 2, "at least one item ahead");

    uint4 bs[PD][KS];  // register sets of the items in flight
    f32x16 acc[MB];

    // STAGED: activations of item I's tile as units u = 64 k + lane of the
    // tile's contiguous run (coalesced), later written to the wave's tile in
    // LDS.  HALF (Cin = 16 KS): loads k < KS/2 cover the first KS units
    // (Cin/2 channels) of every pixel of the tile, the others the second KS
    // units, 64 consecutive units of such half rows per load (whole 128-byte
    // lines).  Otherwise: straight into operand layout, k = slice, lane l
    // holding channels 16k + 8 (l / 32) .. +7 of pixel l % 32.  Zero past the
    // image or past Cin.
#define PW_LOAD(B, I)                                                                        \
    do {                                                                                     \
        const int p0_ = ((I) / nmh) * 32;                                                    \
        const bool tin_ = (I) < nitems;                                                      \
        _Pragma("unroll") for (int k = 0; k < KS; ++k) {                                     \
            if (STAGED) {                                                                    \
                const int u_ = k * 64 + lane;                                                \
                const int pl_ = (u_ * cin8_magic) >> 16;                                     \
                const bool ok_ = tin_ && u_ < tunits && p0_ + pl_ < npix;                    \
                (B)[k] = load16(xr, ok_ ? (p0_ * cin + u_ * 8) * 2 : kOOB);                  \
            } else if (HALF) {                                                               \
                const int hf_ = k / (KS / 2), uh_ = (k - hf_ * (KS / 2)) * 64 + lane;        \
                const int pl_ = uh_ / KS, c_ = uh_ - pl_ * KS + hf_ * KS;                    \
                const bool ok_ = tin_ && p0_ + pl_ < npix;                                   \
                (B)[k] = load16(xr, ok_ ? ((p0_ + pl_) * cin + c_ * 8) * 2 : kOOB);          \
            } else {                                                                         \
                const bool ok_ = tin_ && p0_ + frow < npix && k * 16 + 8 * h < cin;          \
                (B)[k] = load16(xr, ok_ ? ((p0_ + frow) * cin + k * 16 + 8 * h) * 2 : kOOB); \
            }                                                                                \
        }                                                                                    \
    } while (0)
    // STAGED: the loaded units into the wave's tile at the odd pixel pitch
#define PW_STAGE(B)                                                                          \
    do {                                                                                     \
        if (STAGED) {                                                                        \
            _Pragma("unroll") for (int k = 0; k < KS; ++k) {                                 \
                const int u_ = k * 64 + lane;                                                \
                const int pl_ = (u_ * cin8_magic) >> 16;                                     \
                if (u_ < tunits)                                                             \
                    *reinterpret_cast<uint4*>(xt + (pl_ * P + u_ - pl_ * cin8) * 16) = (B)[k]; \
            }                                                                                \
        }                                                                                    \
    } while (0)

    // HALF: half HF of the loaded units into the wave's tile (pixel rows of KS
    // units at the odd pitch PH); in-order LDS access within the wave lets it
    // overwrite the other half once that half's operands have been read
#define PW_STAGE_HALF(B, HF)                                                                 \
    do {                                                                                     \
        _Pragma("unroll") for (int k = 0; k < KS / 2; ++k) {                                 \
            const int uh_ = k * 64 + lane;                                                   \
            const int pl_ = uh_ / KS;                                                        \
            *reinterpret_cast<uint4*>(xt + (pl_ * PH + uh_ - pl_ * KS) * 16) = (B)[(HF) * (KS / 2) + k]; \
        }                                                                                    \
    } while (0)

    // the first PD-1 items' activations go out before the weight staging, so
    // the two memory latencies overlap
#pragma unroll
    for (int d = 0; d + 1 < PD; ++d) PW_LOAD(bs[d], w0 + d * nw);
    // stage the weights (rows past Cout and channels past Cin are zero) and
    // the bias
    {
        // all loads first (zero for padding units), then the LDS stores, so
        // the staging costs one memory latency
        constexpr int kUnits = ((SHUF ? kPwMaxLdsShuf : kPwMaxLds) / 16 + kPwThreads - 1) / kPwThreads;
        const __amdgpu_buffer_rsrc_t wr = make_rsrc(wp, (uint32_t)cout * (uint32_t)cin * 2u);
        uint4 v[kUnits];
#pragma unroll
        for (int k = 0; k < kUnits; ++k) {
            const int u = tid + k * kPwThreads;
            const int r = u / P, c = u - r * P;
            // pixel shuffle: LDS row (tap, co) is packed row co*kk + tap
            const int gr = SHUF ? (r % sh.cout) * sh.kk + r / sh.cout : r;
            v[k] = load16(wr, (u < rows * P && r < cout && c * 8 < cin) ? (gr * cin + c * 8) * 2 : kOOB);
        }
#pragma unroll
        for (int k = 0; k < kUnits; ++k) {
            const int u = tid + k * kPwThreads;
            if (u < rows * P) wl[u] = v[k];
        }
    }
    for (int i = tid; i < rows; i += kPwThreads)
        sb[i] = (has_bias && i < cout) ? bias[SHUF ? i % sh.cout : i] : 0.0f;
    // pad units of every pixel row of the activation tiles (never written
    // by the staging) are zero
    if (STAGED)
        for (int u = tid; u < kPwWaves * 32 * P; u += kPwThreads)
            if ((u % P) * 8 >= cin) wl[rows * P + u] = make_uint4(0, 0, 0, 0);
    __syncthreads();

    int cur_c0 = 0;  // first output channel of the tile being finished (for pw_pack)
    // output offset of tile pixel p (-1: past the end); pixel shuffle:
    // output pixel (n, ih*S, iw*S), to which a row's tap adds kh*Wo + kw
    auto pw_pix = [&](int p) {
        if (SHUF) {
            const int iw = p % sh.w, t = p / sh.w;
            const int ih = t % sh.h, n = t / sh.h;
            return p < npix ? (n * sh.ho + ih * sh.stride) * sh.wo + iw * sh.stride : -1;
        }
        return p < npix ? p * cout : -1;
    };
    // block mb of the accumulators -> two 16-byte pieces per lane: o[e] holds
    // rows (channels) cl .. cl+7 of the block, of tile pixel 16*e + lane % 16
    auto pw_pack = [&](int mb, uint32_t (&o)[2][4]) __attribute__((always_inline)) {
        uint32_t pk[4][2];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            float v[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) v[r] = acc[mb][4 * q + r];
            if (scale) aff.apply(v, cur_c0 + mb * 32 + 8 * q + 4 * h);
#pragma unroll
            for (int r = 0; r < 4; ++r)
                if (relu) v[r] = fmaxf(v[r], 0.0f);
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
            o[0][d] = sw[0];
            o[1][d] = sw[1];
        }
    };

    // one tile: bias-initialised accumulators, KS x MB matrix ops, epilogue
#define PW_TILE(B, I)                                                                        \
    do {                                                                                     \
        const int T = (I) / nmh, c0_ = ((I) - T * nmh) * (MB * 32);                          \
        cur_c0 = c0_;                                                                        \
        PW_STAGE(B);                                                                         \
        _Pragma("unroll") for (int mb = 0; mb < MB; ++mb)                                    \
            _Pragma("unroll") for (int q = 0; q < 4; ++q) {                                  \
                const float4 b4_ = *reinterpret_cast<const float4*>(&sb[c0_ + mb * 32 + 8 * q + 4 * h]); \
                acc[mb][4 * q + 0] = b4_.x;                                                  \
                acc[mb][4 * q + 1] = b4_.y;                                                  \
                acc[mb][4 * q + 2] = b4_.z;                                                  \
                acc[mb][4 * q + 3] = b4_.w;                                                  \
            }                                                                                \
        /* slices past Cin are skipped: their weight reads would run past a row */          \
        _Pragma("unroll") for (int s = 0; s < KS; ++s) {                                     \
            if (s * 16 < cin) {                                                              \
                if (HALF && s % (KS / 2) == 0) PW_STAGE_HALF(B, s / (KS / 2));               \
                const bf16x8 b_ = STAGED ? *reinterpret_cast<const bf16x8*>(b_base + 2 * s * 16) \
                                  : HALF ? *reinterpret_cast<const bf16x8*>(b_base + 2 * (s % (KS / 2)) * 16) \
                                         : __builtin_bit_cast(bf16x8, (B)[s]);               \
                _Pragma("unroll") for (int mb = 0; mb < MB; ++mb) {                          \
                    const bf16x8 a_ = *reinterpret_cast<const bf16x8*>(a_base + ((c0_ + mb * 32) * P + 2 * s) * 16); \
                    acc[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a_, b_, acc[mb], 0, 0, 0); \
                }                                                                            \
            }                                                                                \
        }                                                                                    \
        int pix_[2], pix8_[2][2];                                                            \
        _Pragma("unroll") for (int e = 0; e < 2; ++e) {                                      \
            pix_[e] = pw_pix((T) * 32 + 16 * e + (lane & 15));                              \
            pix8_[e][0] = pw_pix((T) * 32 + 16 * e + (lane & 7));                           \
            pix8_[e][1] = pw_pix((T) * 32 + 16 * e + 8 + (lane & 7));                       \
        }                                                                                    \
        if (merged) {                                                                        \
            /* blocks in pairs, merged so that each store writes whole 128-byte */          \
            /* lines: lane l holds pixel (l & 7) (+8 in the second register) */             \
            _Pragma("unroll") for (int mb = 0; mb < MB; mb += 2) {                           \
                uint32_t o0_[2][4], o1_[2][4];                                               \
                pw_pack(mb, o0_);                                                            \
                pw_pack(mb + 1, o1_);                                                        \
                const int co_ = c0_ + mb * 32 + cl + ((lane & 8) ? 32 : 0);                  \
                int tapoff_ = 0, cc_ = co_;                                                  \
                if (SHUF) {                                                                  \
                    const int tap_ = co_ / sh.cout;                                          \
                    cc_ = co_ - tap_ * sh.cout;                                              \
                    const int kh_ = tap_ / sh.kw;                                            \
                    tapoff_ = kh_ * sh.wo + tap_ - kh_ * sh.kw;                              \
                }                                                                            \
                _Pragma("unroll") for (int e = 0; e < 2; ++e) {                              \
                    uint32_t ra_[4], rb_[4];                                                 \
                    _Pragma("unroll") for (int d = 0; d < 4; ++d) {                          \
                        ra_[d] = __builtin_amdgcn_update_dpp(o0_[e][d], o1_[e][d], 0x118, 0xf, 0xc, false); \
                        rb_[d] = __builtin_amdgcn_update_dpp(o1_[e][d], o0_[e][d], 0x108, 0xf, 0x3, false); \
                    }                                                                        \
                    _Pragma("unroll") for (int g_ = 0; g_ < 2; ++g_) {                       \
                        const int pp_ = pix8_[e][g_];                                        \
                        const int off_ = SHUF ? ((pp_ + tapoff_) * sh.cout + cc_) * 2 : (pp_ + co_) * 2; \
                        const int so_ = pp_ >= 0 && co_ < cout ? off_ : kOOB;                \
                        const uint4 ov_ = g_ ? make_uint4(rb_[0], rb_[1], rb_[2], rb_[3])   \
                                             : make_uint4(ra_[0], ra_[1], ra_[2], ra_[3]);  \
                        if (stream) store16<kStoreStream>(yr, so_, ov_);                     \
                        else store16(yr, so_, ov_);                                          \
                    }                                                                        \
                }                                                                            \
            }                                                                                \
        } else {                                                                             \
        _Pragma("unroll") for (int mb = 0; mb < MB; ++mb) {                                  \
            uint32_t o_[2][4];                                                               \
            pw_pack(mb, o_);                                                                 \
            const int co_ = c0_ + mb * 32 + cl;                                              \
            int tapoff_ = 0, cc_ = co_;  /* pixel shuffle: row (tap, cc) */                  \
            if (SHUF) {                                                                      \
                const int tap_ = co_ / sh.cout;                                              \
                cc_ = co_ - tap_ * sh.cout;                                                  \
                const int kh_ = tap_ / sh.kw;                                                \
                tapoff_ = kh_ * sh.wo + tap_ - kh_ * sh.kw;                                  \
            }                                                                                \
            _Pragma("unroll") for (int e = 0; e < 2; ++e) {                                  \
                const int off_ = SHUF ? ((pix_[e] + tapoff_) * sh.cout + cc_) * 2 : (pix_[e] + co_) * 2; \
                if (vec16) {                                                                 \
                    const int so_ = pix_[e] >= 0 && co_ < cout ? off_ : kOOB;                \
                    const uint4 ov_ = make_uint4(o_[e][0], o_[e][1], o_[e][2], o_[e][3]);    \
                    if (stream) store16<kStoreStream>(yr, so_, ov_);                         \
                    else store16(yr, so_, ov_);                                              \
                } else {                                                                     \
                    store8(yr, pix_[e] >= 0 && co_ < cout ? off_ : kOOB, make_uint2(o_[e][0], o_[e][1])); \
                    store8(yr, pix_[e] >= 0 && co_ + 4 < cout ? off_ + 8 : kOOB,             \
                           make_uint2(o_[e][2], o_[e][3]));                                  \
                }                                                                            \
            }                                                                                \
        }                                                                                    \
        }                                                                                    \
    } while (0)

    // PD items per iteration so the register sets rotate statically: before
    // an item is computed, the loads of the item PD-1 steps later go out into
    // the set the previous item has just freed.
    for (int it = w0; it < nitems; it += PD * nw) {
#pragma unroll
        for (int d = 0; d < PD; ++d) {
            const int cur = it + d * nw;
            if (cur >= nitems) break;
            PW_LOAD(bs[(d + PD - 1) % PD], cur + (PD - 1) * nw);
            __builtin_amdgcn_sched_barrier(0);
            PW_TILE(bs[d], cur);
        }
    }
#undef PW_LOAD
#undef PW_STAGE
#undef PW_STAGE_HALF
#undef PW_TILE
}

// LDS bytes of one workgroup: weights plus one activation tile (or half
// tile) per wave.
long long pw_lds_bytes(int cin, int rows, int stg) {
    const long long w = (long long)rows * pw_pitch(cin) * 16;
    if (stg == kPwStaged) return w + (long long)kPwWaves * 32 * pw_pitch(cin) * 16;
    if (stg == kPwHalf) return w + (long long)kPwWaves * 32 * (cin / 16 + 1) * 16;
    return w;
}

// How the activations reach the matrix ops (each choice measured against
// the others on the workload layers):
//  * whole tiles through LDS (coalesced 1 KB loads) for narrow inputs with
//    wide outputs, and for 129..191 input channels with at most 64 outputs
//    (the 144 -> 24 layer: the weights are small, so two workgroups per CU
//    still fit);
//  * half tiles through LDS for 192 or 256 input channels (whole-line loads;
//    half a tile keeps two workgroups per CU beside the weights);
//  * straight into operand registers otherwise.
int pw_stage_mode(int cin, int cout) {
    if (cin <= 128 && cout >= 128) return kPwStaged;
    if (cin == 192 || cin == 256) return kPwHalf;
    if (cin > 128 && cin < 192 && cout <= 64) return kPwStaged;
    return kPwDirect;
}

// One launch: npix rows of the activation matrix, cin channels, cout GEMM
// rows (output channels, or (tap, channel) rows in pixel-shuffle mode).
struct PwArgs {
    int npix, cin, cout, epilogue;
    const float* scale;
    const float* shift;
    PwShuf sh;
};

template <int MB, int KS, int STG, bool SHUF>
hipError_t launch_pw(const PwArgs& a, const bf16_t* x, const bf16_t* w, const float* b, bf16_t* y,
                     hipStream_t st) {
    auto kern = pw_kernel<MB, KS, STG, SHUF>;
    const int npix = a.npix;
    const int ntiles = (npix + 31) / 32;
    const int nmh = (a.cout + MB * 32 - 1) / (MB * 32);
    const long long lds = pw_lds_bytes(a.cin, nmh * MB * 32, STG);
    // unit -> pixel of a tile: (u * magic) >> 16 == u / (Cin/8) for u < 32*Cin/8
    const int cin8 = a.cin / 8, magic = (65536 + cin8 - 1) / cin8;
    int dev = 0;
    (void)hipGetDevice(&dev);
    if (lds > 64 * 1024) {
        const hipError_t ea = ensure_dynamic_lds<pw_kernel<MB, KS, STG, SHUF>>((int)lds, dev);
        if (ea != hipSuccess) return ea;
    }
    const int by_regs = blocks_per_cu<pw_kernel<MB, KS, STG, SHUF>>(kPwThreads, dev);
    const int by_lds = (int)(163840 / (lds + kPwMaxCout * 4));
    const int bpc = by_lds < by_regs ? (by_lds < 1 ? 1 : by_lds) : by_regs;
    // at most two workgroups per CU: with more, the waves' activation streams
    // evict each other's lines from L1 between the slices that share them
    // (measured slower)
    const long long resident = persistent_slots((long long)cu_count(dev) * (bpc < 2 ? bpc : 2));
    const long long want = ((long long)ntiles * nmh + kPwWaves - 1) / kPwWaves;
    const int grid = (int)(want < resident ? want : resident);
    hipLaunchKernelGGL(kern, dim3(grid), dim3(kPwThreads), (unsigned)lds, st, x, w, b, y, npix, a.cin, a.cout,
                       ntiles, nmh, (a.epilogue & CONV2D_EPI_BIAS) ? 1 : 0, (a.epilogue & CONV2D_EPI_RELU) ? 1 : 0,
                       magic, a.scale, a.shift, a.sh);
    return hipGetLastError();
}

template <int MB, int STG, bool SHUF>
hipError_t launch_pw_ks(const PwArgs& a, const bf16_t* x, const bf16_t* w, const float* b, bf16_t* y,
                        hipStream_t st) {
    const int ks = (a.cin + 15) / 16;
    if constexpr (STG == kPwHalf) {
        // half tiles: Cin exactly 16 KS with KS even
        if (a.cin == 192) return launch_pw<MB, 12, STG, SHUF>(a, x, w, b, y, st);
        if constexpr (MB <= 2)
            if (a.cin == 256) return launch_pw<MB, 16, STG, SHUF>(a, x, w, b, y, st);
        return hipErrorInvalidValue;
    } else {
        if (ks <= 4) return launch_pw<MB, 4, STG, SHUF>(a, x, w, b, y, st);
        if (ks <= 8) return launch_pw<MB, 8, STG, SHUF>(a, x, w, b, y, st);
        if (ks <= 12) return launch_pw<MB, 12, STG, SHUF>(a, x, w, b, y, st);
        if constexpr (MB <= 2 && STG == kPwDirect) return launch_pw<MB, 16, STG, SHUF>(a, x, w, b, y, st);
        return hipErrorInvalidValue;  // more than 192 input channels: at most two blocks, not staged
    }
}

template <int MB>
hipError_t launch_pw_mb(const PwArgs& a, const bf16_t* x, const bf16_t* w, const float* b, bf16_t* y,
                        hipStream_t st) {
    const int stg = pw_stage_mode(a.cin, a.cout);
    if (stg == kPwStaged) return launch_pw_ks<MB, kPwStaged, false>(a, x, w, b, y, st);
    if (stg == kPwHalf) return launch_pw_ks<MB, kPwHalf, false>(a, x, w, b, y, st);
    return launch_pw_ks<MB, kPwDirect, false>(a, x, w, b, y, st);
}

}  // namespace

// 32-row output-channel blocks per work item (the launcher's choice): up to
// four, up to two with more than 192 input channels (register budget).
int pw_blocks(int cin, int cout) {
    const int mb = (cout + 31) / 32;
    const int cap = cin > 192 ? 2 : 4;
    const int b = mb <= 1 ? 1 : mb <= 2 ? 2 : 4;
    return b < cap ? b : cap;
}

bool pointwise_supports(const Shape& s) {
    const long long npix = (long long)s.N * s.Ho * s.Wo;
    const int mb = pw_blocks(s.Cin, s.Cout);
    const long long rows = (long long)(s.Cout + mb * 32 - 1) / (mb * 32) * (mb * 32);
    return s.Kh == 1 && s.Kw == 1 && s.stride == 1 && s.pad == 0 && s.groups == 1 && s.dtype == CONV2D_BF16 &&
           s.Cin % 8 == 0 && s.Cin <= 256 && s.Cout % 4 == 0 && s.Cout <= kPwMaxCout &&
           rows * pw_pitch(s.Cin) * 16 <= kPwMaxLds &&
           pw_lds_bytes(s.Cin, (int)rows, pw_stage_mode(s.Cin, s.Cout)) + kPwMaxCout * 4 <= 163840 &&
           npix * s.Cin * 2 < 0x7fff0000LL && npix * s.Cout * 2 < 0x7fff0000LL;
}

hipError_t launch_pointwise(const Shape& s, const void* x, const void* w_packed, const float* bias,
                            void* y, hipStream_t st) {
    (void)hipGetLastError();  // report only this launch's error
    if (!pointwise_supports(s)) return hipErrorInvalidValue;
    const bf16_t* xt = static_cast<const bf16_t*>(x);
    const bf16_t* wt = static_cast<const bf16_t*>(w_packed);
    bf16_t* yt = static_cast<bf16_t*>(y);
    const int mb = pw_blocks(s.Cin, s.Cout);
    PwArgs a{};
    a.npix = s.N * s.Ho * s.Wo;
    a.cin = s.Cin;
    a.cout = s.Cout;
    a.epilogue = s.epilogue;
    a.scale = s.scale;
    a.shift = s.shift;
    if (mb == 1) return launch_pw_mb<1>(a, xt, wt, bias, yt, st);
    if (mb == 2) return launch_pw_mb<2>(a, xt, wt, bias, yt, st);
    return launch_pw_mb<4>(a, xt, wt, bias, yt, st);
}

// Pixel-shuffle transposed convolution: kernel = stride, no padding, no
// output padding, dilation 1, one group; Cout % 32 == 0 so a 32-row block
// never straddles two taps; Cout*Kh*Kw GEMM rows within the staged-weight
// budget.  Activations straight into operand registers (the weights alone
// take up to 72 KB of LDS).
bool pw_shuffle_supports(const Shape& s) {
    const long long rows = (long long)s.Cout * s.Kh * s.Kw;
    const long long npix = (long long)s.N * s.H * s.W;
    return s.dtype == CONV2D_BF16 && s.groups == 1 && s.Kh == s.stride && s.Kw == s.stride && s.stride > 1 &&
           s.pad == 0 && s.out_pad == 0 && s.dil == 1 && s.Cin % 8 == 0 && s.Cin <= 256 && s.Cout % 32 == 0 &&
           rows <= kPwMaxCout && rows * pw_pitch(s.Cin) * 16 <= kPwMaxLdsShuf &&
           pw_lds_bytes(s.Cin, (int)rows, kPwDirect) + kPwMaxCout * 4 <= 163840 && npix * s.Cin * 2 < 0x7fff0000LL &&
           (long long)s.N * s.Ho * s.Wo * s.Cout * 2 < 0x7fff0000LL;
}

hipError_t launch_pw_shuffle(const Shape& s, const void* x, const void* w_packed, const float* bias, void* y,
                             hipStream_t st) {
    (void)hipGetLastError();  // report only this launch's error
    if (!pw_shuffle_supports(s)) return hipErrorInvalidValue;
    const bf16_t* xt = static_cast<const bf16_t*>(x);
    const bf16_t* wt = static_cast<const bf16_t*>(w_packed);
    bf16_t* yt = static_cast<bf16_t*>(y);
    PwArgs a{};
    a.npix = s.N * s.H * s.W;
    a.cin = s.Cin;
    a.cout = s.Cout * s.Kh * s.Kw;
    a.epilogue = s.epilogue;
    a.scale = nullptr;
    a.shift = nullptr;
    a.sh = PwShuf{s.Cout, s.Kh * s.Kw, s.Kw, s.stride, s.H, s.W, s.Ho, s.Wo};
    const int mb = pw_blocks(a.cin, a.cout);
    constexpr int kStaged = PW_SHUF_STAGED != 0 ? kPwStaged : kPwDirect;
    if (pw_lds_bytes(a.cin, (a.cout + 127) / 128 * 128, kStaged) + kPwMaxCout * 4 > 163840)
        return hipErrorInvalidValue;
    if (mb == 1) return launch_pw_ks<1, kStaged, true>(a, xt, wt, bias, yt, st);
    if (mb == 2) return launch_pw_ks<2, kStaged, true>(a, xt, wt, bias, yt, st);
    return launch_pw_ks<4, kStaged, true>(a, xt, wt, bias, yt, st);
}

}  // namespace conv2d
