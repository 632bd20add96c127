// mfma.hpp -- device helpers shared by the MFMA implicit-GEMM kernels:
// operand vector types, raw buffer loads with hardware zero for
// out-of-range offsets, and the LDS chunk swizzle.
#pragma once

#include "common.hpp"

namespace conv2d {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// Raw buffer access: a load whose byte offset lies beyond the descriptor's
// size returns zero, which is how out-of-image taps (zero padding) and
// out-of-range rows read 0 without a branch.
constexpr int kOOB = 0x7ffffff0;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

__device__ __forceinline__ uint4 load16(__amdgpu_buffer_rsrc_t r, int byte_off) {
    return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, byte_off, 0, 0));
}

// Same, with a wave-uniform part of the offset in the instruction's scalar
// offset (added by the hardware, no vector arithmetic).
__device__ __forceinline__ uint4 load16(__amdgpu_buffer_rsrc_t r, int byte_off, int uniform_off) {
    return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, byte_off, uniform_off, 0));
}

// Buffer stores: an offset past the descriptor's size drops the store, so
// out-of-range pixels and channels need no branch.  POLICY is the
// instruction's cache-policy field: 0, or kStoreStream for output written
// once and not read again by the kernel (the nt bit: the lines do not
// displace the inputs the kernel re-reads from L2).  Streaming measured
// faster for epilogues that write 64 contiguous bytes per pixel per
// instruction and much slower for scattered 8-byte pieces.
constexpr int kStoreStream = 2;

template <int POLICY = 0>
__device__ __forceinline__ void store16(__amdgpu_buffer_rsrc_t r, int byte_off, uint4 v) {
    typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), r, byte_off, 0, POLICY);
}

template <int POLICY = 0>
__device__ __forceinline__ void store8(__amdgpu_buffer_rsrc_t r, int byte_off, uint2 v) {
    typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
    __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2, v), r, byte_off, 0, POLICY);
}

// The folded batch-normalisation step of an epilogue: v = v * scale[c] +
// shift[c] for four consecutive output channels c .. c+3 (c a multiple of 4).
// Both tables are read through descriptors sized to Cout, so the channels of
// a tile's padding rows past Cout read zero (they are never stored).
struct Affine4 {
    __amdgpu_buffer_rsrc_t sc, sh;
    __device__ __forceinline__ Affine4(const float* scale, const float* shift, int cout)
        : sc(make_rsrc(scale, (uint32_t)cout * 4u)), sh(make_rsrc(shift, (uint32_t)cout * 4u)) {}
    __device__ __forceinline__ void apply(float v[4], int c) const {
        const float4 a = __builtin_bit_cast(float4, load16(sc, c * 4));
        const float4 b = __builtin_bit_cast(float4, load16(sh, c * 4));
        v[0] = fmaf(v[0], a.x, b.x);
        v[1] = fmaf(v[1], a.y, b.y);
        v[2] = fmaf(v[2], a.z, b.z);
        v[3] = fmaf(v[3], a.w, b.w);
    }
};

// An LDS row holds the BK channels of one K-step for one output channel (A)
// or one pixel (B): BK*2 bytes = BK/8 16-byte chunks.  The chunk index is
// XOR-swizzled with the row so that any 16 consecutive rows read at the same
// logical chunk land in 16 distinct 16-byte slots of a 256-byte bank line
// (conflict-free ds_read_b128 / ds_write_b128): 64-byte rows swizzle with
// row/4, 128-byte rows with row/2.
template <int BK>
__device__ __forceinline__ int swz(int row, int chunk) {
    if (BK == 32) return row * 4 + (chunk ^ ((row >> 2) & 3));
    return row * 8 + (chunk ^ ((row >> 1) & 7));
}

// Workgroups are dispatched round-robin over the 8 XCDs (block b runs on XCD
// b % 8), each with its own L2.  Renumber blocks so that every XCD walks one
// contiguous run of tiles: neighbouring tiles, which share input rows, then
// meet in the same L2.
__device__ __forceinline__ int xcd_tile_index() {
    const int nblk = gridDim.x;
    const int xcd = blockIdx.x & 7, slot = blockIdx.x >> 3;
    const int per = nblk >> 3, rem = nblk & 7;
    return xcd * per + min(xcd, rem) + slot;
}

}  // namespace conv2d
