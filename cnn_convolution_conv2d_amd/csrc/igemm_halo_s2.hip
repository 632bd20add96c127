// igemm_halo_s2.hip -- 3x3 stride-2 convolution as an implicit GEMM whose
// input window is staged once per channel chunk in LDS, split by phase.
//
// The GEMM is the one of the other implicit-GEMM kernels (lincklin.cn lesson
// 9, sections 7, 11, 19): per group, D[co][p] = sum_k W[co][k] X_col[k][p],
// k = (kh, kw, ci).  A tile is BM output channels x a 4 x 32 block of output
// pixels of one image.  With stride 2 the block's nine taps read inside one
// (2*4+1) x (2*32+1) input window (the block plus its halo, section 12, at
// stride 2; section 27: stride changes how far apart neighbouring outputs'
// windows start, so the input a tile shares between its taps is the window,
// read once per chunk instead of once per tap).
//
// Phase split.  Output (ho, wo) reads tap (kh, kw) at window position
// (2(ho-ho0) + kh, 2(wo-wo0) + kw).  Keyed by (kh mod 2, kw mod 2), the
// window splits into four sub-windows of stride-1 pixels: sub-window (a, b)
// holds window positions (2r + a, 2c + b), and tap (kh, kw) reads pixel
// (ho-ho0 + kh/2, wo-wo0 + kw/2) of sub-window (kh mod 2, kw mod 2).  Every
// tap is therefore a fixed additive LDS offset from the output pixel's lane
// base, and neighbouring lanes read neighbouring 80-byte pixels (an odd
// number of 16-byte units: conflict-free ds_read_b128), as in the stride-1
// kernel.  The four sub-windows hold 4x32, 4x33, 5x32 and 5x33 pixels (rows of
// 33 pixels each, so one row pitch serves all), each its own LDS object.
//
// One window buffer, refilled piecewise.  A chunk's nine taps run sub-window
// by sub-window: (1,1); (1,0), (1,2); (0,1), (2,1); then the four corner
// taps.  As soon as a sub-window's last tap of this chunk has passed a
// barrier, the next chunk's copy of that sub-window is started straight from
// memory into it (buffer loads to LDS: no registers): (1,1) at step 1, (1,0)
// at step 3, (0,1) at step 5, and the corner sub-window at step 0 of the
// chunk that uses it.  Each wave waits for its own copies (loads complete in
// order; the wait counts the later loads) before the barrier after which the
// copied sub-window is first read.  A double-buffered window would not fit
// two workgroups per CU; this gives each copy 3 (corner) to 6 steps of
// slack with one.
//
// Weights.  A step here has half the matrix work of the stride-1 kernel's,
// so the weight slices travel further ahead: nine register sets, one per tap,
// each loaded a whole chunk (nine steps) before its step and stored into the
// 3-slot LDS ring two steps before it (seven steps of slack for the load).
//
// Everything else follows the stride-1 kernel: persistent workgroups, two K
// slices of v_mfma_f32_32x32x16_bf16 per step with the next slice's operands
// read during the matrix ops, bias-initialised fp32 accumulators, and the
// register epilogue (lincklin.cn section 31).
#include "halo.hpp"
#include "../../include/conv2d.h"

namespace conv2d {

namespace {

constexpr int kS2TH = 4, kS2TW = 32;  // output rows x columns of a tile's pixel block
constexpr int kS2Pitch = kS2TW + 1;   // pixels per sub-window row (all four)
// sub-window x (0: (1,1), 1: (1,0), 2: (0,1), 3: (0,0)): rows
constexpr int s2_rows(int x) { return x < 2 ? kS2TH : kS2TH + 1; }
constexpr int kS2WinPix = (4 * kS2TH + 2) * kS2Pitch;
constexpr int s2_lds_bytes(int bm) { return kRing * bm * kBK * 2 + kS2WinPix * kHP * 16 + 2 * bm * 4 + 16; }

// K-step t of a chunk -> tap kh*3 + kw: sub-window by sub-window.
constexpr int s2_tap(int t) {
    return t == 0 ? 4 : t == 1 ? 3 : t == 2 ? 5 : t == 3 ? 1 : t == 4 ? 7 : t == 5 ? 0 : t == 6 ? 2 : t == 7 ? 6 : 8;
}
// sub-window of a tap, and the tap's pixel offset inside it
constexpr int s2_sub(int tap) {
    return (tap / 3) % 2 == 1 ? ((tap % 3) % 2 == 1 ? 0 : 1) : ((tap % 3) % 2 == 1 ? 2 : 3);
}
constexpr int s2_inoff(int tap) { return ((tap / 3) / 2) * kS2Pitch + (tap % 3) / 2; }

// s_waitcnt immediate for vmcnt(n) (n < 64), lgkmcnt and expcnt left at their maxima
constexpr int vmcnt_imm(int n) { return (n & 15) | ((n >> 4) << 14) | 0x0f70; }

template <int NT, int BM, int WGM, int WGN, int NSET, bool CFULL, bool BIAS, bool RELU>
__global__ __launch_bounds__(NT, waves_per_simd(NT, 2, s2_lds_bytes(BM)))
void halo_s2_kernel(const bf16_t* __restrict__ x, const bf16_t* __restrict__ wp, const float* __restrict__ bias,
                    bf16_t* __restrict__ y, Shape s, HaloGrid hg) {
    constexpr int TH = kS2TH, TW = kS2TW, BN = TH * TW;
    static_assert(WGM * WGN * 64 == NT, "one wave per sub-tile");
    constexpr int WTM = BM / WGM, WTN = BN / WGN;
    constexpr int TM = WTM / 32, TN = WTN / 32;
    static_assert(TM * 32 == WTM && TN * 32 == WTN, "32x32 MFMA tiles");
    constexpr int A_BYTES = BM * kBK * 2;
    constexpr int B_BYTES = BIAS ? BM * 4 : 0;
    constexpr int AV = BM * 4 / NT;
    static_assert(AV * NT == BM * 4 && AV >= 1, "weight slice splits evenly");
    constexpr int NW = NT / 64;
    // 64-unit copies per wave of each sub-window
    constexpr int CPW0 = ((s2_rows(0) * kS2Pitch * kHP + 63) / 64 + NW - 1) / NW;
    constexpr int CPW1 = ((s2_rows(1) * kS2Pitch * kHP + 63) / 64 + NW - 1) / NW;
    constexpr int CPW2 = ((s2_rows(2) * kS2Pitch * kHP + 63) / 64 + NW - 1) / NW;
    constexpr int CPW3 = ((s2_rows(3) * kS2Pitch * kHP + 63) / 64 + NW - 1) / NW;
    constexpr int CPWMAX = CPW2 > CPW0 ? CPW2 : CPW0;
    // VMEM loads per step, in issue order: at step 0 the next tile's bias
    // piece, then at every step AV weight loads, then the step's copies (step
    // 0: the corner sub-window of this chunk; steps 1, 3, 5: sub-windows 0,
    // 1, 2 of the next chunk).  The bias goes first: the compiler waits for
    // it (and so, loads completing in order, for everything before it) where
    // it is stored at step 7 or where its register is reused, and issued
    // after a copy it would pull that copy's wait forward.
    // Loads complete in order, so a copy has landed once no more loads are
    // outstanding than were issued in the steps after it.  The counts below
    // take only the weight loads and copies of those later steps: the bias
    // load is left out because the compiler may drop it (no bias) or move it,
    // and a load counted but not issued would let the wait pass early;
    // anything issued but not counted (the bias, a tile's output stores)
    // only makes the wait longer.  Each copy is waited for at the barrier
    // before the step whose next-step operand reads first touch it:
    //   end of step 1: step 5's copies of the previous chunk (sub-window 2,
    //                  read from step 3)  -> steps 6..8 and 0..1 issue
    //                  5 AV + CPW3 + CPW0
    //   end of step 3: step 0's copies (corner, read from step 5)
    //                  -> steps 1..3 issue 3 AV + CPW0 + CPW1
    //   end of step 7: step 1's copies (sub-window 0, read at step 0 of the
    //                  next chunk) -> steps 2..7 issue 6 AV + CPW1 + CPW2
    //   end of step 8: step 3's copies (sub-window 1, read from step 1 of
    //                  the next chunk) -> steps 4..8 issue 5 AV + CPW2
    constexpr int WAIT1 = 5 * AV + CPW3 + CPW0;
    constexpr int WAIT3 = 3 * AV + CPW0 + CPW1;
    constexpr int WAIT7 = 6 * AV + CPW1 + CPW2;
    constexpr int WAIT8 = 5 * AV + CPW2;
    static_assert(WAIT1 < 64 && WAIT7 < 64 && WAIT8 < 64, "vmcnt range");
    constexpr int JSTRIDE = (32 / TW) * kS2Pitch * kHP * 16;  // MFMA column block j -> j+1 (one pixel row)
    static_assert(32 % TW == 0 || TW == 32, "32-pixel MFMA tiles cover whole block rows");
    // Separate LDS objects for the ring, each sub-window and the bias: the
    // compiler then tells the copies into one sub-window from every access to
    // the others by their objects alone, and waits only where they meet.
    __shared__ uint4 lds_ring[kRing * A_BYTES / 16];
    __shared__ uint4 lds_w0[s2_rows(0) * kS2Pitch * kHP];
    __shared__ uint4 lds_w1[s2_rows(1) * kS2Pitch * kHP];
    __shared__ uint4 lds_w2[s2_rows(2) * kS2Pitch * kHP];
    __shared__ uint4 lds_w3[s2_rows(3) * kS2Pitch * kHP];
    __shared__ uint4 lds_bias[2 * B_BYTES / 16 + 1];
    char* const ring = reinterpret_cast<char*>(lds_ring);
    char* const sbias = reinterpret_cast<char*>(lds_bias);

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave / WGN, wn = wave % WGN;
    const int G = gridDim.x;
    // this workgroup's tiles: as in the stride-1 kernel (full rounds, then at
    // most one tile of the last round, spread over CUs)
    const int first = xcd_tile_index();
    if (first >= hg.ntiles) return;
    const int nfull = hg.ntiles / G, nextra = hg.ntiles - nfull * G;
    int e_extra;
    if (G % 8 == 0) {
        const int m = blockIdx.x >> 3;
        e_extra = m % hg.spread == 0 ? (blockIdx.x & 7) + 8 * (m / hg.spread) : nextra;
    } else {
        e_extra = blockIdx.x;
    }
    const int nmine = nfull + (e_extra < nextra ? 1 : 0);
    const int nchunk = (s.cin_g + kBK - 1) / kBK;
    const int wrow = 9 * s.cin_g * 2;  // bytes of one packed weight row

    const __amdgpu_buffer_rsrc_t xr = make_rsrc(x, (uint32_t)s.N * s.H * s.W * s.Cin * 2u);
    const __amdgpu_buffer_rsrc_t wr = make_rsrc(wp, (uint32_t)s.Cout * (uint32_t)wrow);
    const __amdgpu_buffer_rsrc_t yr = make_rsrc(y, (uint32_t)s.N * s.Ho * s.Wo * s.Cout * 2u);
    const __amdgpu_buffer_rsrc_t br = make_rsrc(bias, BIAS ? (uint32_t)s.Cout * 4u : 0u);

    // ---- per-lane constants
    int a_row[AV], a_c[AV], a_lds[AV];
#pragma unroll
    for (int i = 0; i < AV; ++i) {
        const int q = tid + i * NT;
        a_row[i] = q >> 2;
        a_c[i] = (q & 3) * 8;
        a_lds[i] = swz<kBK>(q >> 2, q & 3) * 16;
    }
    const int frow = lane & 31, fch = lane >> 5;
    const int a_rd0 = swz<kBK>(wm * WTM + frow, fch) * 16;
    const int a_rd1 = swz<kBK>(wm * WTM + frow, 2 + fch) * 16;
    // this lane's output pixel of MFMA column block 0, as a sub-window pixel
    const int p0 = wn * WTN + frow;
    const int b_lane = ((p0 / TW) * kS2Pitch + p0 % TW) * (kHP * 16) + fch * 16;
    // copies: copy m of sub-window X writes units base .. base+63 of it,
    // base = min(64 k, units - 64), k = wave + NW*m; this lane's unit is
    // sub-window pixel (r, c), 16-byte piece ch (ch 4: the padding unit)
    int dm[4][CPWMAX], dmb[4][CPWMAX];
#pragma unroll
    for (int xs = 0; xs < 4; ++xs) {
        const int units = s2_rows(xs) * kS2Pitch * kHP;
#pragma unroll
        for (int m = 0; m < CPWMAX; ++m) {
            const int kk = wave + NW * m;
            const int base = 64 * kk < units - 64 ? 64 * kk : units - 64;
            const int u = base + lane;
            const int q = u / kHP, ch = u - q * kHP;
            const int r = q / kS2Pitch, c = q - r * kS2Pitch;
            dm[xs][m] = r | (c << 8) | (ch << 16);
            dmb[xs][m] = base * 16;
        }
    }

    auto a_offsets = [&](const TileXY& T, int* vo) {
#pragma unroll
        for (int i = 0; i < AV; ++i) {
            const int co = T.ct * BM + a_row[i];
            vo[i] = co < s.cout_g ? ((T.g * s.cout_g + co) * wrow + a_c[i] * 2) : kOOB;
        }
    };

    // copy m of sub-window XS, channel chunk C of tile T, into DST (VALID
    // false: still issued, every lane reading 0, so every path issues the same
    // loads and the wait counts stay exact)
    // (DST is deliberately not a restrict parameter: the copies then carry
    // only the alias scope of the chunk function's buffer argument, which
    // the compiler's load-wait tracking can follow for a few scopes at a
    // time; a scope per inlined copy would exhaust it and make every LDS
    // access wait for all copies in flight)
    auto s2_copy = [&](char* dst, int xs, const TileXY& T, int C, int m, bool valid) {
        const int rc = dm[xs][m];
        const int r = rc & 255, c = (rc >> 8) & 255, ch = rc >> 16;
        const int a = xs < 2 ? 1 : 0, b = (xs == 0 || xs == 2) ? 1 : 0;
        const int hi = 2 * T.ho0 - s.pad + 2 * r + a, wi = 2 * T.wo0 - s.pad + 2 * c + b;
        const bool ok = valid && ch < 4 && (unsigned)hi < (unsigned)s.H && (unsigned)wi < (unsigned)s.W &&
                        (CFULL || C * kBK + ch * 8 < s.cin_g);
        const int off = ok ? (((T.n * s.H + hi) * s.W + wi) * s.Cin + T.g * s.cin_g + ch * 8) * 2 : kOOB;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(xr, (halo_lds_t)(dst + dmb[xs][m]), 16, off,
                                                 __builtin_amdgcn_readfirstlane(C * kBK * 2), 0, 0);
    };

#define TILE_OF(KK) ((KK) < nfull ? first + (KK) * G : nfull * G + e_extra)
    TileXY tc = tile_xy<TH, TW>(TILE_OF(0), hg, s.groups);
    TileXY tn = tile_xy<TH, TW>(TILE_OF(nmine > 1 ? 1 : 0), hg, s.groups);

    f32x16 acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) acc[i][j] = f32x16{};

    static_assert(NSET == 3 || NSET == 9, "weight register sets: one per ring slot, or one per tap");
    uint4 ra[NSET][AV];
    uint4 bv = make_uint4(0, 0, 0, 0);
    bf16x8 af0[TM], bf0[TN], af1[TM], bf1[TN];

#define S2_LOAD(RA, VO, C, TAP)                                                              \
    do {                                                                                     \
        const int so_ = __builtin_amdgcn_readfirstlane(((TAP) * s.cin_g + (C) * kBK) * 2);  \
        _Pragma("unroll") for (int i = 0; i < AV; ++i) {                                     \
            const bool ok_ = CFULL || (C) * kBK + a_c[i] < s.cin_g;                          \
            (RA)[i] = load16(wr, ok_ ? (VO)[i] : kOOB, so_);                                 \
        }                                                                                    \
    } while (0)
#define S2_STORE(RG, RA, SLOT)                                                               \
    do {                                                                                     \
        _Pragma("unroll") for (int i = 0; i < AV; ++i)                                       \
            *reinterpret_cast<uint4*>((RG) + (SLOT) * A_BYTES + a_lds[i]) = (RA)[i];         \
    } while (0)

    char* const w0 = reinterpret_cast<char*>(lds_w0);
    char* const w1 = reinterpret_cast<char*>(lds_w1);
    char* const w2 = reinterpret_cast<char*>(lds_w2);
    char* const w3 = reinterpret_cast<char*>(lds_w3);

    // ---- prologue: weights of steps 0, 1 in ring slots 0, 1, step 2's in
    // flight; sub-windows 0..2 of the first chunk (the corner sub-window comes
    // with step 0's copies); the first tile's bias; step 0's first-slice
    // operands
    int a_vo_c[AV], a_vo_n[AV];
    a_offsets(tc, a_vo_c);
    {
        uint4 p0r[AV], p1r[AV];
        S2_LOAD(p0r, a_vo_c, 0, s2_tap(0));
        S2_LOAD(p1r, a_vo_c, 0, s2_tap(1));
        uint4 pb = make_uint4(0, 0, 0, 0);
        const bool bin = BIAS && tid * 4 < BM;
        if (BIAS) pb = load16(br, bin ? ((tc.g * s.cout_g + tc.ct * BM + tid * 4) * 4) : kOOB);
        if (NSET == 9) {
            // steps 2..8 of the first chunk in flight, one register set each
#pragma unroll
            for (int t = 2; t < 9; ++t) S2_LOAD(ra[t % NSET], a_vo_c, 0, s2_tap(t));
        } else {
            S2_LOAD(ra[2], a_vo_c, 0, s2_tap(2));
        }
        S2_STORE(ring, p0r, 0);
        S2_STORE(ring, p1r, 1);
        if (bin) *reinterpret_cast<uint4*>(sbias + tid * 16) = pb;
#pragma unroll
        for (int m = 0; m < CPW0; ++m) s2_copy(w0, 0, tc, 0, m, true);
#pragma unroll
        for (int m = 0; m < CPW1; ++m) s2_copy(w1, 1, tc, 0, m, true);
#pragma unroll
        for (int m = 0; m < CPW2; ++m) s2_copy(w2, 2, tc, 0, m, true);
    }
    __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0): nothing of the prologue stays in flight
    __syncthreads();
    {
        const char* ab = ring + a_rd0;
        const char* bb = w0 + b_lane + s2_inoff(s2_tap(0)) * (kHP * 16);
#pragma unroll
        for (int i = 0; i < TM; ++i) af0[i] = *reinterpret_cast<const bf16x8*>(ab + i * 2048);
#pragma unroll
        for (int j = 0; j < TN; ++j) bf0[j] = *reinterpret_cast<const bf16x8*>(bb + j * JSTRIDE);
    }

    // sub-window pointer of a tap, and the tap's byte offset inside it
#define S2_WIN(TAP) (s2_sub(TAP) == 0 ? W0 : s2_sub(TAP) == 1 ? W1 : s2_sub(TAP) == 2 ? W2 : W3)
#define S2_OFF(TAP) (s2_inoff(TAP) * (kHP * 16))
#define S2_STEP(T)                                                                           \
    do {                                                                                     \
        /* (1) loads: the bias (step 0), weights, then the step's copies */                   \
        if ((T) == 0) {                                                                      \
            const bool bin_ = BIAS && last_chunk && k + 1 < nmine && tid * 4 < BM;           \
            bv = load16(br, bin_ ? ((tn.g * s.cout_g + tn.ct * BM + tid * 4) * 4) : kOOB);   \
        }                                                                                    \
        if (NSET == 9) S2_LOAD(ra[(T) % NSET], a_vo_n, cn, s2_tap(T));                       \
        else if ((T) + 3 < 9) S2_LOAD(ra[(T) % NSET], a_vo_c, c, s2_tap((T) + 3));           \
        else S2_LOAD(ra[(T) % NSET], a_vo_n, cn, s2_tap((T) + 3 - 9));                       \
        if ((T) == 0) {                                                                      \
            _Pragma("unroll") for (int m = 0; m < CPW3; ++m) s2_copy(W3, 3, tc, c, m, true); \
        } else if ((T) == 1) {                                                               \
            _Pragma("unroll") for (int m = 0; m < CPW0; ++m) s2_copy(W0, 0, hn, cn, m, h_ok); \
        } else if ((T) == 3) {                                                               \
            _Pragma("unroll") for (int m = 0; m < CPW1; ++m) s2_copy(W1, 1, hn, cn, m, h_ok); \
        } else if ((T) == 5) {                                                               \
            _Pragma("unroll") for (int m = 0; m < CPW2; ++m) s2_copy(W2, 2, hn, cn, m, h_ok); \
        }                                                                                    \
        __builtin_amdgcn_sched_barrier(0);                                                   \
        /* (2) second slice's operands of this step */                                       \
        {                                                                                    \
            const char* ab_ = (RG) + ((T) % 3) * A_BYTES + a_rd1;                            \
            const char* bb_ = S2_WIN(s2_tap(T)) + b_lane + S2_OFF(s2_tap(T)) + 32;           \
            _Pragma("unroll") for (int i = 0; i < TM; ++i)                                   \
                af1[i] = *reinterpret_cast<const bf16x8*>(ab_ + i * 2048);                   \
            _Pragma("unroll") for (int j = 0; j < TN; ++j)                                   \
                bf1[j] = *reinterpret_cast<const bf16x8*>(bb_ + j * JSTRIDE);                \
        }                                                                                    \
        __builtin_amdgcn_sched_barrier(0);                                                   \
        /* (3) first slice's matrix ops */                                                   \
        _Pragma("unroll") for (int i = 0; i < TM; ++i)                                       \
            _Pragma("unroll") for (int j = 0; j < TN; ++j)                                   \
                acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af0[i], bf0[j], acc[i][j], 0, 0, 0); \
        /* (4) next step's first-slice operands (step 8: the next chunk's step 0, */         \
        /* sub-window 0, refilled at step 1); second slice's matrix ops */                   \
        {                                                                                    \
            constexpr int TN_ = s2_tap((T) + 1 < 9 ? (T) + 1 : 0);                           \
            const char* ab_ = (RG) + (((T) + 1) % 3) * A_BYTES + a_rd0;                      \
            const char* bb_ = S2_WIN(TN_) + b_lane + S2_OFF(TN_);                            \
            _Pragma("unroll") for (int i = 0; i < TM; ++i)                                   \
                af0[i] = *reinterpret_cast<const bf16x8*>(ab_ + i * 2048);                   \
            _Pragma("unroll") for (int j = 0; j < TN; ++j)                                   \
                bf0[j] = *reinterpret_cast<const bf16x8*>(bb_ + j * JSTRIDE);                \
        }                                                                                    \
        _Pragma("unroll") for (int i = 0; i < TM; ++i)                                       \
            _Pragma("unroll") for (int j = 0; j < TN; ++j)                                   \
                acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af1[i], bf1[j], acc[i][j], 0, 0, 0); \
        __builtin_amdgcn_sched_barrier(0);                                                   \
        /* (5) LDS stores: weights of step + 2; at step 7 the bias loaded at step 0 */        \
        S2_STORE(RG, ra[((T) + 2) % NSET], ((T) + 2) % 3);                                   \
        if ((T) == 7 && BIAS && last_chunk && k + 1 < nmine && tid * 4 < BM)                 \
            *reinterpret_cast<uint4*>((SB) + ((k + 1) & 1) * B_BYTES + tid * 16) = bv;       \
        /* copies read after this barrier have landed (this wave's; the barrier */           \
        /* covers the others') */                                                            \
        if ((T) == 1) __builtin_amdgcn_s_waitcnt(vmcnt_imm(WAIT1));                          \
        if ((T) == 3) __builtin_amdgcn_s_waitcnt(vmcnt_imm(WAIT3));                          \
        if ((T) == 7) __builtin_amdgcn_s_waitcnt(vmcnt_imm(WAIT7));                          \
        if ((T) == 8) __builtin_amdgcn_s_waitcnt(vmcnt_imm(WAIT8));                          \
        halo_barrier();                                                                      \
    } while (0)

    const int half = lane >> 5;
    for (int k = 0; k < nmine; ++k) {
#pragma unroll
        for (int i = 0; i < TM; ++i) {
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                float4 b4 = make_float4(0.f, 0.f, 0.f, 0.f);
                if (BIAS)
                    b4 = *reinterpret_cast<const float4*>(sbias + (k & 1) * B_BYTES +
                                                          (wm * WTM + i * 32 + 8 * q + 4 * half) * 4);
#pragma unroll
                for (int j = 0; j < TN; ++j) {
                    acc[i][j][4 * q + 0] = b4.x;
                    acc[i][j][4 * q + 1] = b4.y;
                    acc[i][j][4 * q + 2] = b4.z;
                    acc[i][j][4 * q + 3] = b4.w;
                }
            }
        }
        for (int c = 0; c < nchunk; ++c) {
            const bool last_chunk = c + 1 == nchunk;
            const int cn = last_chunk ? 0 : c + 1;
            const TileXY hn = last_chunk ? tn : tc;
            const bool h_ok = !last_chunk || k + 1 < nmine;
            if (last_chunk) a_offsets(tn, a_vo_n);
            else {
                _Pragma("unroll") for (int i = 0; i < AV; ++i) a_vo_n[i] = a_vo_c[i];
            }
            // the chunk's nine steps; every LDS buffer a restrict argument
            auto chunk = [&](char* __restrict__ RG, char* __restrict__ W0, char* __restrict__ W1,
                             char* __restrict__ W2, char* __restrict__ W3, char* __restrict__ SB)
                             __attribute__((always_inline)) {
                S2_STEP(0);
                S2_STEP(1);
                S2_STEP(2);
                S2_STEP(3);
                S2_STEP(4);
                S2_STEP(5);
                S2_STEP(6);
                S2_STEP(7);
                S2_STEP(8);
            };
            chunk(ring, w0, w1, w2, w3, sbias);
        }
        tile_epilogue<TM, TN, WTM, WTN, TH, TW, false, RELU>(acc, sbias, yr, s, tc, tc.ct * BM, wm, wn, lane);
        tc = tn;
        tn = tile_xy<TH, TW>(TILE_OF(k + 2 < nmine ? k + 2 : 0), hg, s.groups);
#pragma unroll
        for (int i = 0; i < AV; ++i) a_vo_c[i] = a_vo_n[i];
    }
#undef TILE_OF
#undef S2_LOAD
#undef S2_STORE
#undef S2_WIN
#undef S2_OFF
#undef S2_STEP
}

// Grid of one call, or ok = false when the kernel does not take the shape.
struct S2Plan {
    bool ok;
    bool m128;  // 128 output channels per tile (else 64)
    HaloGrid hg;
};

S2Plan s2_plan(const Shape& s) {
    S2Plan p{};
    if (!(s.dtype == CONV2D_BF16 && s.stride == 2 && s.Kh == 3 && s.Kw == 3 && s.dil == 1 && s.cin_g % 8 == 0 &&
          s.cout_g % 4 == 0 && s.cout_g > 32 && buffer_addressable(s)))
        return p;
    p.m128 = s.cout_g > 64;
    const int bm = p.m128 ? 128 : 64;
    p.hg.tiles_h = (s.Ho + kS2TH - 1) / kS2TH;
    p.hg.tiles_w = (s.Wo + kS2TW - 1) / kS2TW;
    p.hg.n_ctiles = (s.cout_g + bm - 1) / bm;
    const long long tiles = (long long)s.N * p.hg.tiles_h * p.hg.tiles_w * s.groups * p.hg.n_ctiles;
    p.hg.ntiles = (int)(tiles > 0x7fffffffLL ? 0 : tiles);
    p.hg.spread = 1;
    p.ok = tiles > 0 && tiles <= 0x7fffffffLL;
    return p;
}

template <int BM, int WGM, int WGN, bool CFULL, bool BIAS, bool RELU>
hipError_t launch_s2_k(const Shape& s, const HaloGrid& hg, const bf16_t* x, const bf16_t* w, const float* b,
                       bf16_t* y, hipStream_t st) {
    constexpr int NT = 256;
    constexpr int NSET = 9;
    auto kern = halo_s2_kernel<NT, BM, WGM, WGN, NSET, CFULL, BIAS, RELU>;
    int dev = 0;
    (void)hipGetDevice(&dev);
    const int bpc = blocks_per_cu<halo_s2_kernel<NT, BM, WGM, WGN, NSET, CFULL, BIAS, RELU>>(NT, dev);
    const long long resident = persistent_slots((long long)cu_count(dev) * bpc);
    const int grid = (int)(hg.ntiles < resident ? hg.ntiles : resident);
    HaloGrid h = hg;
    const int per_xcd = grid / 8, extra = hg.ntiles % grid;
    const int slots = per_xcd / (bpc > 0 ? bpc : 1), want = (extra + 7) / 8;
    h.spread = (grid % 8 == 0 && want > 0 && slots / want > 1) ? slots / want : 1;
    hipLaunchKernelGGL(kern, dim3(grid), dim3(NT), 0, st, x, w, b, y, s, h);
    return hipGetLastError();
}

template <int BM, int WGM, int WGN, bool CFULL>
hipError_t launch_s2_epi(const Shape& s, const HaloGrid& hg, const bf16_t* x, const bf16_t* w, const float* b,
                         bf16_t* y, hipStream_t st) {
    const bool bias = s.epilogue & CONV2D_EPI_BIAS, relu = s.epilogue & CONV2D_EPI_RELU;
    if (bias && relu) return launch_s2_k<BM, WGM, WGN, CFULL, true, true>(s, hg, x, w, b, y, st);
    if (bias) return launch_s2_k<BM, WGM, WGN, CFULL, true, false>(s, hg, x, w, b, y, st);
    if (relu) return launch_s2_k<BM, WGM, WGN, CFULL, false, true>(s, hg, x, w, b, y, st);
    return launch_s2_k<BM, WGM, WGN, CFULL, false, false>(s, hg, x, w, b, y, st);
}

}  // namespace

bool halo_s2_supports(const Shape& s) { return s2_plan(s).ok; }

hipError_t launch_halo_s2(const Shape& s, const void* x, const void* w_packed, const float* bias, void* y,
                          hipStream_t st) {
    (void)hipGetLastError();  // report only this launch's error
    const S2Plan p = s2_plan(s);
    if (!p.ok) return hipErrorInvalidValue;
    const bf16_t* xt = static_cast<const bf16_t*>(x);
    const bf16_t* wt = static_cast<const bf16_t*>(w_packed);
    bf16_t* yt = static_cast<bf16_t*>(y);
    const bool full = s.cin_g % kBK == 0;
    if (p.m128) {
        if (full) return launch_s2_epi<128, 2, 2, true>(s, p.hg, xt, wt, bias, yt, st);
        return launch_s2_epi<128, 2, 2, false>(s, p.hg, xt, wt, bias, yt, st);
    }
    if (full) return launch_s2_epi<64, 1, 4, true>(s, p.hg, xt, wt, bias, yt, st);
    return launch_s2_epi<64, 1, 4, false>(s, p.hg, xt, wt, bias, yt, st);
}

}  // namespace conv2d
