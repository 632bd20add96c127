// halo.hpp -- pieces shared by the halo-tile implicit-GEMM kernels (stride 1
// in igemm_halo.hip, stride 2 in igemm_halo_s2.hip): the LDS layout
// constants, the persistent tile grid, the tile-to-position map, the register
// epilogue and the barrier that leaves buffer-to-LDS copies in flight.
#pragma once

#include "mfma.hpp"

namespace conv2d {

namespace {

constexpr int kBK = 32;      // input channels per chunk: one 64-byte LDS row per pixel
constexpr int kRing = 3;     // weight slices staged in LDS

// Halo tile layout in LDS: one window pixel = 5 16-byte units (80 bytes:
// its 4 chunks of 8 channels plus one unit of padding).  Because 5 is odd,
// any 16 consecutive window pixels read at the same chunk fall in 16 distinct
// 16-byte bank slots (conflict-free ds_read_b128), and moving to another tap
// is a plain additive offset of (kh*D*width + kw*D) * 80 bytes.
constexpr int kHP = 5;

struct HaloGrid {
    int tiles_h, tiles_w, n_ctiles, ntiles;
    int hwd_magic;  // ceil(2^16 / window width): row = (pixel * magic) >> 16 inside the window
    int nparts;     // 16-byte halo loads per thread per chunk (one per tap)
    int spread;     // last-round tiles go to every spread-th first-round workgroup of an XCD
};

// Minimum waves per SIMD the registers are budgeted for: the requested
// workgroups per CU, or fewer where their LDS does not fit (160 KB per CU).
constexpr int waves_per_simd(int nt, int minb, int lds_bytes) {
    const int fit = 163840 / lds_bytes;
    const int b = minb < fit ? minb : fit;
    return b * nt / 256 < 1 ? 1 : b * nt / 256;
}

// Tile t -> (output-channel tile, group, image, pixel-block origin); the
// channel tile varies fastest, then the group, then pixel blocks in row-major
// order over each image.
struct TileXY {
    int ct, g, n, ho0, wo0;
};

template <int TH, int TW>
__device__ __forceinline__ TileXY tile_xy(int tile, const HaloGrid& hg, int groups) {
    TileXY t;
    t.ct = tile % hg.n_ctiles;
    tile /= hg.n_ctiles;
    t.g = tile % groups;
    tile /= groups;
    const int tw = tile % hg.tiles_w;
    tile /= hg.tiles_w;
    const int th = tile % hg.tiles_h;
    t.n = tile / hg.tiles_h;
    t.ho0 = th * TH;
    t.wo0 = tw * TW;
    return t;
}

// LDS address space for the destination of buffer-to-LDS copies.
typedef __attribute__((address_space(3))) void* halo_lds_t;

// This wave's LDS operations complete, then the workgroup barrier.  Unlike
// __syncthreads, it does not wait for buffer-to-LDS copies still in flight
// (those into the next chunk's halo buffer); the kernel waits for them
// explicitly before the barrier after which they are read.
__device__ __forceinline__ void halo_barrier() {
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0); vmcnt and expcnt at their maxima (no wait)
    __builtin_amdgcn_s_barrier();
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// Epilogue of one tile from registers: bias, ReLU, bf16.  In the 32x32
// result layout lane l < 32 of a block holds channels 8q+r (q = 0..3,
// r = 0..3) of pixel l and lane l + 32 channels 8q+4+r.  A lane-half swap
// (v_permlane32_swap) gives each lane 8 consecutive channels; a row swap
// (v_permlane16_swap) then puts 32 consecutive channels of 16 pixels in one
// register: lanes l, l+16, l+32, l+48 hold the four 16-byte pieces of one
// pixel's 64 contiguous bytes.  Two row blocks (64 channels) are then merged
// with 8-lane row shifts (DPP) so that one store instruction writes the 128
// contiguous bytes of each of 8 pixels: every 128-byte line of the output
// leaves in one instruction, and the streaming (nt) stores add no partial
// line writes.  Pixels and channels outside the output get an offset past
// the end: the buffer store drops them.
template <int TM, int TN, int WTM, int WTN, int TH, int TW, bool BIAS, bool RELU>
__device__ __forceinline__ void tile_epilogue(f32x16 (&acc)[TM][TN], const char* sb,
                                              __amdgpu_buffer_rsrc_t yr, const Shape& s,
                                              const TileXY& tc, int co0, int wm, int wn, int lane) {
    const int half = lane >> 5;
    const bool vec16 = (s.Cout % 8 == 0) && (s.cout_g % 8 == 0);
    // output offset of a pixel of the wave's tile (-1: outside the output)
    auto pix_of = [&](int p) {
        const int ho = tc.ho0 + p / TW, wo = tc.wo0 + p % TW;
        return (ho < s.Ho && wo < s.Wo) ? ((tc.n * s.Ho + ho) * s.Wo + wo) * s.Cout : -1;
    };
    int pix[TN][2], pix8[TN][2][2];
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int p = wn * WTN + j * 32 + 16 * h;
            pix[j][h] = pix_of(p + (lane & 15));
            pix8[j][h][0] = pix_of(p + (lane & 7));
            pix8[j][h][1] = pix_of(p + 8 + (lane & 7));
        }
    // channel of this lane's 16-byte piece within a 32-channel block
    const int cl = ((lane >> 4) & 1) * 16 + half * 8;
    const int cw = co0 + wm * WTM;  // first channel (within the group) of the wave's rows
    const Affine4 aff(s.scale, s.shift, s.Cout);
    const int cga = tc.g * s.cout_g + cw;  // absolute channel of cw
    // Pack block (i, j) into two 16-byte pieces per lane: out[h] holds
    // channels cl .. cl+7 (of the block's 32) of pixel 16*h + lane % 16.
    auto pack_block = [&](int i, int j, uint32_t (&out)[2][4]) __attribute__((always_inline)) {
        float4 b4[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            b4[q] = make_float4(0.f, 0.f, 0.f, 0.f);
            if (BIAS) b4[q] = *reinterpret_cast<const float4*>(sb + (wm * WTM + i * 32 + 8 * q + 4 * half) * 4);
        }
        uint32_t pk[4][2];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            float v[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) v[r] = BIAS ? acc[i][j][4 * q + r] + (&b4[q].x)[r] : acc[i][j][4 * q + r];
            if (s.scale) aff.apply(v, cga + i * 32 + 8 * q + 4 * half);
#pragma unroll
            for (int r = 0; r < 4; ++r)
                if (RELU) v[r] = fmaxf(v[r], 0.0f);
            pk[q][0] = pack_bf16x2(v[0], v[1]);
            pk[q][1] = pack_bf16x2(v[2], v[3]);
        }
        // r8[pr]: 8 channels 16*pr + 8*half .. +7 of pixel lane % 32
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
    };
    if (TM % 2 == 0 && vec16) {
        // Row blocks in pairs: the two blocks' pieces of the same pixels are
        // regrouped with row shifts of 8 lanes so that each store
        // instruction writes the 64 channels of 8 pixels, i.e. whole 128-byte
        // lines (one instruction per line: no line leaves L2 as two partial
        // writes).  Lane l then holds pixel (l & 7) (+8 in the second
        // register) and channels cl + (l & 8 ? 32 : 0) of the pair.
        const int cl2 = cl + ((lane & 8) ? 32 : 0);
#pragma unroll
        for (int i = 0; i < TM; i += 2) {
            const int co = cw + i * 32 + cl2;
#pragma unroll
            for (int j = 0; j < TN; ++j) {
                uint32_t o0[2][4], o1[2][4];
                pack_block(i, j, o0);
                pack_block(i + 1, j, o1);
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    uint32_t ra_[4], rb_[4];
#pragma unroll
                    for (int d = 0; d < 4; ++d) {
                        // lanes 8..15 of each row: block i+1's piece from 8 lanes lower
                        ra_[d] = __builtin_amdgcn_update_dpp(o0[h][d], o1[h][d], 0x118 /* row_shr:8 */, 0xf, 0xc,
                                                             false);
                        // lanes 0..7 of each row: block i's piece from 8 lanes higher
                        rb_[d] = __builtin_amdgcn_update_dpp(o1[h][d], o0[h][d], 0x108 /* row_shl:8 */, 0xf, 0x3,
                                                             false);
                    }
                    const int pa = pix8[j][h][0], pb = pix8[j][h][1];
                    store16<kStoreStream>(yr, pa >= 0 && co < s.cout_g ? (pa + tc.g * s.cout_g + co) * 2 : kOOB,
                                          make_uint4(ra_[0], ra_[1], ra_[2], ra_[3]));
                    store16<kStoreStream>(yr, pb >= 0 && co < s.cout_g ? (pb + tc.g * s.cout_g + co) * 2 : kOOB,
                                          make_uint4(rb_[0], rb_[1], rb_[2], rb_[3]));
                }
            }
        }
        return;
    }
#pragma unroll
    for (int i = 0; i < TM; ++i) {
        const int co = cw + i * 32 + cl;
#pragma unroll
        for (int j = 0; j < TN; ++j) {
            uint32_t out[2][4];
            pack_block(i, j, out);
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const int off = (pix[j][h] + tc.g * s.cout_g + co) * 2;
                if (vec16) {
                    store16<kStoreStream>(yr, pix[j][h] >= 0 && co < s.cout_g ? off : kOOB,
                                          make_uint4(out[h][0], out[h][1], out[h][2], out[h][3]));
                } else {
                    store8(yr, pix[j][h] >= 0 && co < s.cout_g ? off : kOOB, make_uint2(out[h][0], out[h][1]));
                    store8(yr, pix[j][h] >= 0 && co + 4 < s.cout_g ? off + 8 : kOOB, make_uint2(out[h][2], out[h][3]));
                }
            }
        }
    }
}

}  // namespace

}  // namespace conv2d
