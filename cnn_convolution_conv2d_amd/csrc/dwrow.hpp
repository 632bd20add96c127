// dwrow.hpp -- the 3x3 depthwise arithmetic on 2*NW channels (NW 32-bit
// words of bf16 pairs) of one output column, shared by the depthwise kernel
// and the fused depthwise-separable kernel.
//
// Each input row a thread touches (its 3 columns wo-1..wo+1 around the
// output column) is converted once into the form the arithmetic uses and then
// serves every output row whose window covers it (lincklin.cn lesson 9,
// section 18: adjacent outputs share inputs):
//   - taps kw=0 and kw=1 of channel c become one bf16 pair (x[wo-1][c],
//     x[wo][c]) built with v_perm_b32, multiplied by the matching weight pair
//     with v_dot2_f32_bf16 (two products and the running sum in one op);
//   - tap kw=2 is kept as fp32 for a plain FMA.
// The accumulator starts at the bias, so the bias is added with the taps.
#pragma once

#include "mfma.hpp"

namespace conv2d {
namespace dwrow {

template <int NW>
struct alignas(4 * NW) Vec { uint32_t u[NW]; };  // 2*NW bf16
typedef Vec<4> V8;
typedef Vec<2> V4;

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ V8 load_v8(const bf16_t* p) { return *reinterpret_cast<const V8*>(p); }

// Buffer loads: an offset past the tensor returns zero (padding taps, rows
// outside the image).
__device__ __forceinline__ V8 load_v8(__amdgpu_buffer_rsrc_t r, int byte_off) {
    return __builtin_bit_cast(V8, __builtin_amdgcn_raw_buffer_load_b128(r, byte_off, 0, 0));
}
__device__ __forceinline__ V4 load_v4(__amdgpu_buffer_rsrc_t r, int byte_off) {
    return __builtin_bit_cast(V4, __builtin_amdgcn_raw_buffer_load_b64(r, byte_off, 0, 0));
}
template <int NW>
__device__ __forceinline__ Vec<NW> load_vec(__amdgpu_buffer_rsrc_t r, int byte_off) {
    if constexpr (NW == 4) return load_v8(r, byte_off);
    else return load_v4(r, byte_off);
}

__device__ __forceinline__ float lo(uint32_t u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float hi(uint32_t u) { return __uint_as_float(u & 0xffff0000u); }

template <int NW>
struct RowXN {
    uint32_t p01[2 * NW];  // per channel: (x[wo-1][c], x[wo][c]) as a bf16 pair
    float x2[2 * NW];      // per channel: x[wo+1][c]
};
typedef RowXN<4> RowX;

// a, b, c: the channels at input columns wo-1, wo, wo+1 of one row.
template <int NW>
__device__ __forceinline__ void prep_row(const Vec<NW>& a, const Vec<NW>& b, const Vec<NW>& c, RowXN<NW>& r) {
#pragma unroll
    for (int i = 0; i < NW; ++i) {
        // v_perm_b32: bytes 0-3 select from the second operand, 4-7 from the first
        r.p01[2 * i] = __builtin_amdgcn_perm(b.u[i], a.u[i], 0x05040100u);      // low halves
        r.p01[2 * i + 1] = __builtin_amdgcn_perm(b.u[i], a.u[i], 0x07060302u);  // high halves
        r.x2[2 * i] = lo(c.u[i]);
        r.x2[2 * i + 1] = hi(c.u[i]);
    }
}

// acc += one filter row applied to one prepared input row: the kw=2 tap
// first (a three-operand FMA, so a bias held in acc's source register needs
// no copy), then the (kw0, kw1) pair.
template <int NW>
__device__ __forceinline__ void row_fma(float acc[2 * NW], const RowXN<NW>& r, const uint32_t wp[2 * NW],
                                        const float w2[2 * NW]) {
#pragma unroll
    for (int ch = 0; ch < 2 * NW; ++ch) {
        acc[ch] = fmaf(r.x2[ch], w2[ch], acc[ch]);
        acc[ch] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, r.p01[ch]),
                                                  __builtin_bit_cast(bf16x2_t, wp[ch]), acc[ch], false);
    }
}

// Two fp32 values -> a bf16 pair (nearest even), then ReLU on the pair: a
// bf16 is sign-magnitude, so as a 16-bit integer every negative value is
// below zero and max(v, 0) per half zeroes exactly the negatives.  Rounding
// keeps the sign, so this equals rounding max(v, 0) for every finite value.
template <bool RELU>
__device__ __forceinline__ uint32_t pack_relu(float a, float b) {
    uint32_t p = pack_bf16x2(a, b);
    if (!RELU) return p;
    // keep the pair opaque: seen through, the 16-bit max splits the pair
    // conversion into two single conversions and a permute
    asm("" : "+v"(p));
    typedef short s16x2 __attribute__((ext_vector_type(2)));
    const s16x2 z = {0, 0};
    return __builtin_bit_cast(uint32_t, __builtin_elementwise_max(__builtin_bit_cast(s16x2, p), z));
}

// The 3x3 filter of channels c0..c0+2*NW-1 from the packed depthwise weights
// [3][3][C]: per filter row, the (kw0, kw1) pair of each channel and kw2 in
// fp32.
template <int NW>
__device__ __forceinline__ void load_taps(const bf16_t* w, int C, int c0, uint32_t wp[3][2 * NW],
                                          float w2[3][2 * NW]) {
#pragma unroll
    for (int kh = 0; kh < 3; ++kh) {
        const Vec<NW> a = *reinterpret_cast<const Vec<NW>*>(w + (kh * 3 + 0) * C + c0);
        const Vec<NW> b = *reinterpret_cast<const Vec<NW>*>(w + (kh * 3 + 1) * C + c0);
        const Vec<NW> c = *reinterpret_cast<const Vec<NW>*>(w + (kh * 3 + 2) * C + c0);
#pragma unroll
        for (int i = 0; i < NW; ++i) {
            wp[kh][2 * i] = __builtin_amdgcn_perm(b.u[i], a.u[i], 0x05040100u);
            wp[kh][2 * i + 1] = __builtin_amdgcn_perm(b.u[i], a.u[i], 0x07060302u);
            w2[kh][2 * i] = lo(c.u[i]);
            w2[kh][2 * i + 1] = hi(c.u[i]);
        }
    }
}

}  // namespace dwrow
}  // namespace conv2d
