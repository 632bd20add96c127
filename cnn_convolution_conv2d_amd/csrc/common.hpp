// common.hpp -- types and small device helpers shared by the conv2d kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace conv2d {

// One convolution call, validated on the host.  All sizes fit int32; element
// offsets of x and y fit int32 (checked by the dispatcher).
struct Shape {
    int N, Cin, H, W, Cout, Kh, Kw;
    int stride, pad, dil, groups;
    int Ho, Wo;
    int cin_g, cout_g;   // channels per group
    int dtype;           // CONV2D_F32 / CONV2D_BF16
    int epilogue;        // CONV2D_EPI_* bits
    // Folded batch normalisation of the epilogue (both null: none):
    // v = (sum [+ bias]) * scale[co] + shift[co], then the ReLU.
    const float* scale;
    const float* shift;
    // Transposed convolution only: extra output rows/columns at the far edge
    // (H, W are then the input extent and Ho, Wo the upsampled output).
    int out_pad;
};

// One fused depthwise-separable call (3x3 depthwise, then 1x1), validated on
// the host.
struct SepShape {
    int N, C, H, W, Cout;
    int stride, pad;
    int Ho, Wo;
    int dw_epilogue, pw_epilogue;  // CONV2D_EPI_* bits of each stage
};

enum Layout { NCHW = 0, NHWC = 1 };
// raw [Cout][Cin/G][Kh][Kw], packed [Cout][Kh][Kw][Cin/G], depthwise [Kh][Kw][C],
// transposed-convolution raw [Cin][Cout/G][Kh][Kw]
enum WLayout { W_OIHW = 0, W_PACKED = 1, W_DW = 2, W_IOHW = 3 };

typedef uint16_t bf16_t;   // raw bf16 bit pattern

__device__ __forceinline__ float bf16_to_f32(bf16_t b) {
    return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// fp32 -> bf16, round to nearest, ties to even (v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ bf16_t f32_to_bf16(float f) {
    return __builtin_bit_cast(bf16_t, static_cast<__bf16>(f));
}

// Two fp32 -> two packed bf16 in one 32-bit word (low half = a), one
// v_cvt_pk_bf16_f32.
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
    typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
    const bf16x2_t v = {static_cast<__bf16>(a), static_cast<__bf16>(b)};
    return __builtin_bit_cast(uint32_t, v);
}

template <typename T> __device__ __forceinline__ float load_f32(const T* p, int i);
template <> __device__ __forceinline__ float load_f32<float>(const float* p, int i) { return p[i]; }
template <> __device__ __forceinline__ float load_f32<bf16_t>(const bf16_t* p, int i) { return bf16_to_f32(p[i]); }

template <typename T> __device__ __forceinline__ void store_f32(T* p, int i, float v);
template <> __device__ __forceinline__ void store_f32<float>(float* p, int i, float v) { p[i] = v; }
template <> __device__ __forceinline__ void store_f32<bf16_t>(bf16_t* p, int i, float v) { p[i] = f32_to_bf16(v); }

// Epilogue of every kernel: bias after the full sum, then the folded batch
// normalisation scale and shift when given, then ReLU (the fused bias ->
// scale/shift -> activation -> single store of the "Epilogue Fusion"
// passage).
template <bool BIAS, bool RELU>
__device__ __forceinline__ float epilogue(float acc, const float* bias, const float* scale, const float* shift,
                                          int co) {
    float v = acc;
    if (BIAS) v += bias[co];
    if (scale) v = fmaf(v, scale[co], shift[co]);
    if (RELU) v = fmaxf(v, 0.0f);
    return v;
}

// Compute units of a device (cached per device id).
inline int cu_count(int dev) {
    static int cache[64] = {};
    if (dev < 0 || dev >= 64) return 256;
    int v = __atomic_load_n(&cache[dev], __ATOMIC_RELAXED);
    if (v > 0) return v;
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n < 1) n = 256;
    __atomic_store_n(&cache[dev], n, __ATOMIC_RELAXED);
    return n;
}

// Resident workgroups per CU of one kernel on a device (cached per kernel
// and device id; at least 1).  The kernel is a template argument so that
// every kernel, including those that share a signature, has its own cache.
template <auto Kernel>
int blocks_per_cu(int nt, int dev) {
    static int cache[64] = {};
    if (dev < 0 || dev >= 64) dev = 0;
    int v = __atomic_load_n(&cache[dev], __ATOMIC_RELAXED);
    if (v > 0) return v;
    int b = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&b, Kernel, nt, 0) != hipSuccess || b < 1) b = 1;
    __atomic_store_n(&cache[dev], b, __ATOMIC_RELAXED);
    return b;
}

// The MFMA and depthwise kernels read and write through buffer resources whose
// out-of-range offset (0x7ffffff0) stands for a zero tap or a dropped store;
// that only works while x, y and the packed weights stay below it.  Larger
// tensors go to the direct kernel.  (Transposed shapes: H, W are the input
// extent and Ho, Wo the output's, so the same byte counts apply.)
inline bool buffer_addressable(const Shape& s) {
    const long long eb = s.dtype == 0 /* CONV2D_F32 */ ? 4 : 2;
    const long long xb = (long long)s.N * s.H * s.W * s.Cin * eb;
    const long long yb = (long long)s.N * s.Ho * s.Wo * s.Cout * eb;
    const long long wb = (long long)s.Cout * s.cin_g * s.Kh * s.Kw * eb;
    return xb < 0x7fff0000LL && yb < 0x7fff0000LL && wb < 0x7fff0000LL;
}

// Process-wide cap on the workgroups of one persistent launch (0: none), set
// by conv2d_set_grid_limit.  The persistent kernels (halo tiles, streaming
// 1x1, fused separable) launch min(work items, resident slots, this cap)
// workgroups and walk their items in a grid-stride loop, so any cap >= 1 is
// valid; a small one makes every workgroup walk several items.
int grid_limit();
inline long long persistent_slots(long long resident) {
    const int lim = grid_limit();
    return (lim > 0 && lim < resident) ? lim : resident;
}

// Allow a kernel more than the default 64 KB of dynamic LDS (up to `bytes`),
// once per kernel and device.
template <auto Kernel>
hipError_t ensure_dynamic_lds(int bytes, int dev) {
    static int done[64] = {};   // largest size set per device
    if (dev < 0 || dev >= 64) dev = 0;
    if (__atomic_load_n(&done[dev], __ATOMIC_RELAXED) >= bytes) return hipSuccess;
    const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(Kernel),
                                             hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
    if (e == hipSuccess) __atomic_store_n(&done[dev], bytes, __ATOMIC_RELAXED);
    return e;
}

// Host-side launchers (each defined in its kernel's source file).  They
// return hipSuccess or the launch error.
hipError_t launch_direct(const Shape& s, const void* x, int xl, const void* w, int wl,
                         const float* bias, void* y, int yl, hipStream_t st);
hipError_t launch_depthwise(const Shape& s, const void* x, const void* w_dw, const float* bias,
                            void* y, hipStream_t st);
hipError_t launch_gemm1x1(const Shape& s, const void* x, const void* w_packed, const float* bias,
                          void* y, hipStream_t st);
hipError_t launch_igemm(const Shape& s, const void* x, const void* w_packed, const float* bias,
                        void* y, hipStream_t st);
hipError_t launch_igemm_halo(const Shape& s, const void* x, const void* w_packed, const float* bias,
                             void* y, hipStream_t st);
bool igemm_supports(const Shape& s);
// the halo kernels can run the shape (stride 1 plans, and 3x3 stride 2)
bool igemm_halo_supports(const Shape& s);
// the halo kernel the automatic path choice takes (stride 1 plans only)
bool igemm_halo_auto(const Shape& s);
// 3x3 stride 2: the phase-split staged window (served by launch_igemm_halo)
bool halo_s2_supports(const Shape& s);
hipError_t launch_halo_s2(const Shape& s, const void* x, const void* w_packed, const float* bias, void* y,
                          hipStream_t st);
bool gemm1x1_supports(const Shape& s);
bool depthwise_supports(const Shape& s);
hipError_t launch_pointwise(const Shape& s, const void* x, const void* w_packed, const float* bias,
                            void* y, hipStream_t st);
bool pointwise_supports(const Shape& s);
hipError_t launch_separable(const SepShape& s, const void* x, const void* w_dw, const float* b_dw,
                            const void* w_pw, const float* b_pw, void* y, hipStream_t st);
bool separable_supports(const SepShape& s);

// Transposed convolution (s.H, s.W input; s.Ho, s.Wo output).
hipError_t launch_tconv_direct(const Shape& s, const void* x, int xl, const void* w, int wl,
                               const float* bias, void* y, int yl, hipStream_t st);
hipError_t launch_igemm_transposed(const Shape& s, const void* x, const void* w_packed, const float* bias,
                                   void* y, hipStream_t st);
bool igemm_transposed_supports(const Shape& s);
// stride 2, 4x4: all phases on one staged input window
bool tconv_halo_supports(const Shape& s);
hipError_t launch_tconv_halo(const Shape& s, const void* x, const void* w_packed, const float* bias, void* y,
                             hipStream_t st);
// kernel == stride, no padding: the pointwise GEMM with pixel-shuffled output
bool pw_shuffle_supports(const Shape& s);
hipError_t launch_pw_shuffle(const Shape& s, const void* x, const void* w_packed, const float* bias, void* y,
                             hipStream_t st);
hipError_t launch_tpack_weights(const void* w, void* wp, int Cin, int cout_g, int groups, int Kh, int Kw,
                                int elem_bytes, hipStream_t st);

// Winograd F(2x2, 3x3) (bf16, 3x3, stride 1, dilation 1, groups 1).
bool winograd_supports(const Shape& s);
hipError_t launch_winograd(const Shape& s, const void* x, const void* w_wino, const float* bias, void* y,
                           hipStream_t st);
hipError_t launch_winograd_weights(const void* w, void* w_wino, int Cout, int Cin, hipStream_t st);

hipError_t launch_transpose(const void* src, void* dst, int batch, int rows, int cols,
                            int elem_bytes, hipStream_t st);
hipError_t launch_pack_weights(const void* w, void* wp, int Cout, int cin_g, int Kh, int Kw,
                               int depthwise, int elem_bytes, hipStream_t st);

}  // namespace conv2d
