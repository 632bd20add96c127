/*
 * conv2d.h -- C ABI of the gfx950 (MI355X) 2D convolution forward library,
 * libconv2d.so.
 *
 * The operation (page "How a GPU executes NN convolution", lincklin.cn,
 * sections 1-2, with dilation from its section 28 and groups from
 * "lpnh.cn/news/2674933" sections 2.2 and 4.3):
 *
 *   Y[n,co,ho,wo] = epi( sum_{ci<Cin/G, kh<Kh, kw<Kw}
 *                        X[n, g*Cin/G + ci, ho*S + kh*D - P, wo*S + kw*D - P]
 *                        * W[co, ci, kh, kw] )
 *   g = co / (Cout/G);  taps outside the input read 0 (zero padding,
 *   lincklin.cn section 26);  epi(v) = [max](v [+ bias[co]]), bias added after
 *   the full sum and ReLU last (lincklin.cn section 31);
 *   Ho = floor((H + 2P - D(Kh-1) - 1)/S) + 1, likewise Wo
 *   (lpnh.cn section 6.2).
 *
 * Stride S, padding P and dilation D apply equally to both spatial axes;
 * Kh and Kw are independent.
 *
 * Types.  dtype CONV2D_F32: x, w, y are fp32.  dtype CONV2D_BF16: x, w, y are
 * bf16 (raw 16-bit patterns), products are accumulated in fp32 and the result
 * is rounded to bf16 to nearest-even once, after the epilogue.  bias is always
 * fp32 [Cout].
 *
 * Memory.  Every tensor pointer is device memory owned by the caller; the
 * library never frees or keeps it.  Element counts of x and y must each stay
 * below 2^31 (32-bit element offsets in the kernels).  The MFMA paths need
 * x, w and y 16-byte aligned (any hipMalloc / torch allocation is).
 *
 * Streams.  Every call that takes a stream only enqueues work on it and
 * returns; nothing synchronises the host.  Errors of the asynchronous work
 * surface at the caller's next synchronisation.  Passing 0 means the null
 * stream.
 *
 * Errors.  Arguments are validated on the host before anything is enqueued;
 * an invalid call returns a negative CONV2D_ERR_* code and touches no memory.
 * A failed launch returns CONV2D_ERR_HIP.  conv2d_strerror() names a code and
 * conv2d_last_error() gives the calling thread's last detailed message.
 */
#ifndef CONV2D_H
#define CONV2D_H

#include <stddef.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* element types */
enum { CONV2D_F32 = 0, CONV2D_BF16 = 1 };

/* epilogue flags (bitwise or): bias is added after the sum, ReLU last */
enum { CONV2D_EPI_NONE = 0, CONV2D_EPI_BIAS = 1, CONV2D_EPI_RELU = 2 };

/* kernel paths (see conv2d_select_path) */
enum {
    CONV2D_PATH_AUTO = 0,
    CONV2D_PATH_DIRECT = 1,     /* direct loop, any shape and dtype             */
    CONV2D_PATH_DEPTHWISE = 2,  /* bf16, groups == Cin == Cout                  */
    CONV2D_PATH_GEMM1X1 = 3,    /* bf16, 1x1, stride 1, pad 0, groups 1         */
    CONV2D_PATH_IGEMM = 4,      /* bf16 implicit GEMM on MFMA (as an override:
                                   the library picks one of the two below)      */
    CONV2D_PATH_IGEMM_GATHER = 5, /* implicit GEMM gathering every tap from
                                     memory; any stride, Cin/G % 8 == 0,
                                     Cout/G % 4 == 0                             */
    CONV2D_PATH_IGEMM_HALO = 6  /* implicit GEMM on an LDS halo tile; stride 1,
                                   (K-1)*D+1 <= 5, Cin/G % 8 == 0,
                                   Cout/G % 4 == 0 and > 32; also 3x3 stride 2,
                                   dilation 1 on a phase-split window, run only
                                   when this path is forced (the automatic
                                   choice gives stride 2 to the gather)         */
};

/* return codes */
enum {
    CONV2D_OK = 0,
    CONV2D_ERR_ARG = -1,          /* a size, stride, pad or dilation out of range   */
    CONV2D_ERR_GROUPS = -2,       /* Cin or Cout not divisible by groups            */
    CONV2D_ERR_EMPTY_OUTPUT = -3, /* Ho or Wo < 1                                   */
    CONV2D_ERR_UNSUPPORTED = -4,  /* valid convolution this path/build cannot run   */
    CONV2D_ERR_HIP = -5,          /* a HIP runtime call or launch failed            */
    CONV2D_ERR_NULL = -6,         /* a required pointer is NULL                     */
    CONV2D_ERR_DTYPE = -7,        /* unknown dtype                                  */
    CONV2D_ERR_EPILOGUE = -8,     /* unknown epilogue bits                          */
    CONV2D_ERR_ALIGN = -9         /* pointer not aligned as the chosen path needs   */
};

/*
 * conv2d_fwd -- the forward pass in the pages' own layouts.
 *   x    [N][Cin][H][W]            (NCHW, lincklin.cn section 1)
 *   w    [Cout][Cin/G][Kh][Kw]     (lincklin.cn section 1; grouped weight of
 *                                   lpnh.cn section 4.1)
 *   bias fp32 [Cout], required iff epilogue has CONV2D_EPI_BIAS (else ignored)
 *   y    [N][Cout][Ho][Wo]         (NCHW), written completely
 * fp32 runs the direct kernel on these layouts.  bf16 repacks x to NHWC and
 * w to the packed layout, runs the chosen kernel and repacks y back to NCHW
 * (lincklin.cn sections 29-30), using a scratch block per device and stream
 * that the library grows on demand with hipMalloc (so this entry may
 * allocate, and waits for earlier work on its stream while it does) and
 * frees in conv2d_release_scratch().  Calls on different streams use
 * different blocks and may overlap; calls on one stream share its block and
 * run in order.  A block stays allocated, per stream used, until
 * conv2d_release_scratch().  A call that
 * would have to grow the scratch while its stream is being captured into a
 * graph returns CONV2D_ERR_UNSUPPORTED instead (nothing is enqueued).
 */
int conv2d_fwd(const void* x, const void* w, const float* bias, void* y,
               int N, int Cin, int H, int W, int Cout, int Kh, int Kw,
               int stride, int pad, int dilation, int groups,
               int dtype, int epilogue, hipStream_t stream);

/*
 * conv2d_fwd_noalloc -- conv2d_fwd for callers that cannot allocate device
 * memory: code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc.  Same arguments, layouts, paths, results and errors as
 * conv2d_fwd, but the bf16 staging (packed weights, NHWC x, NHWC y) goes to a
 * static device array of 64 MiB per GPU, reserved when the library's code
 * object is loaded on that GPU and held until the process ends; the call
 * never calls hipMalloc or hipFree and never synchronises.  A bf16 call whose
 * staging needs more than 64 MiB returns CONV2D_ERR_UNSUPPORTED before
 * enqueuing anything.  fp32 calls run the direct kernel in place and use no
 * staging.  Every call on one GPU shares that GPU's array and leaves its
 * contents behind; each call writes every staging byte it reads, so nothing
 * needs clearing, but calls that overlap in time on one GPU (different
 * streams, or host threads) race on the array: serialise them.
 */
int conv2d_fwd_noalloc(const void* x, const void* w, const float* bias, void* y,
                       int N, int Cin, int H, int W, int Cout, int Kh, int Kw,
                       int stride, int pad, int dilation, int groups,
                       int dtype, int epilogue, hipStream_t stream);

/*
 * conv2d_fwd_nhwc_packed -- the same operation on channels-last data
 * (lincklin.cn section 29; lnrq.cn section 5.3); allocates nothing.
 *   x        [N][H][W][Cin]        (NHWC)
 *   w_packed output of conv2d_pack_weights for the same Cout, Cin, Kh, Kw,
 *            groups and dtype
 *   y        [N][Ho][Wo][Cout]     (NHWC), written completely
 */
int conv2d_fwd_nhwc_packed(const void* x, const void* w_packed, const float* bias, void* y,
                           int N, int Cin, int H, int W, int Cout, int Kh, int Kw,
                           int stride, int pad, int dilation, int groups,
                           int dtype, int epilogue, hipStream_t stream);

/*
 * conv2d_fwd_bn, conv2d_fwd_nhwc_packed_bn -- the same two forward entries
 * with batch normalisation (inference form) folded into the epilogue
 * (lincklin.cn lesson 9, section 31: bias, then the normalisation's
 * per-channel scale and shift, then the activation, in registers before the
 * single store):
 *   Y[n,co,ho,wo] = [max]( (sum [+ bias[co]]) * scale[co] + shift[co] )
 * For a normalisation with mean mu, variance var, gain gamma, offset beta and
 * epsilon eps: scale = gamma / sqrt(var + eps), shift = beta - mu * scale.
 *   scale, shift  fp32 [Cout] device memory, both required (non-NULL)
 * Every other argument, layout, path and error as for conv2d_fwd /
 * conv2d_fwd_nhwc_packed (epilogue: CONV2D_EPI_BIAS and CONV2D_EPI_RELU as
 * there).  Every kernel path supports it.
 */
int conv2d_fwd_bn(const void* x, const void* w, const float* bias, const float* scale, const float* shift,
                  void* y, int N, int Cin, int H, int W, int Cout, int Kh, int Kw,
                  int stride, int pad, int dilation, int groups,
                  int dtype, int epilogue, hipStream_t stream);
int conv2d_fwd_nhwc_packed_bn(const void* x, const void* w_packed, const float* bias, const float* scale,
                              const float* shift, void* y, int N, int Cin, int H, int W, int Cout,
                              int Kh, int Kw, int stride, int pad, int dilation, int groups,
                              int dtype, int epilogue, hipStream_t stream);

/*
 * conv2d_fwd_separable_nhwc -- the depthwise-separable block as one fused
 * pass (lincklin.cn lesson 9, section 25; lpnh.cn section 4.1; lnrq.cn
 * section 3.1): a 3x3 depthwise convolution (groups == C, stride S, padding
 * P, dilation 1) with its epilogue, then a 1x1 convolution C -> Cout with
 * its own epilogue:
 *   t[n,c,ho,wo]  = bf16( epi_dw( sum_{kh,kw<3} X[n,c,ho*S+kh-P,wo*S+kw-P]
 *                                               . w_dw[c,kh,kw] ) )
 *   Y[n,co,ho,wo] = epi_pw( sum_{c<C} t[n,c,ho,wo] . w_pw[co,c] )
 * t is what a separate depthwise layer would store (bias, then ReLU, then
 * rounding to nearest even); it stays on chip and is never written to
 * memory.  Ho = floor((H + 2P - 3)/S) + 1, likewise Wo.
 *   x       [N][H][W][C]      bf16 (NHWC)
 *   w_dw    [3][3][C]         bf16: conv2d_pack_weights of the [C][1][3][3]
 *                             depthwise weight (Cout = Cin = groups = C)
 *   bias_dw fp32 [C], required iff dw_epilogue has CONV2D_EPI_BIAS
 *   w_pw    [Cout][C]         bf16 (the [Cout][C][1][1] weight as it is)
 *   bias_pw fp32 [Cout], required iff pw_epilogue has CONV2D_EPI_BIAS
 *   y       [N][Ho][Wo][Cout] bf16 (NHWC), written completely
 * Runs dtype CONV2D_BF16 with C % 8 == 0, C <= 256, Cout % 4 == 0,
 * Cout <= 128 and stride 1 or 2; other valid calls return
 * CONV2D_ERR_UNSUPPORTED (run the two layers through conv2d_fwd_nhwc_packed
 * instead).  x, w_dw, w_pw and y must be 16-byte aligned.  Allocates
 * nothing; errors as for the other entries.
 */
int conv2d_fwd_separable_nhwc(const void* x, const void* w_dw, const float* bias_dw,
                              const void* w_pw, const float* bias_pw, void* y,
                              int N, int C, int H, int W, int Cout, int stride, int pad,
                              int dtype, int dw_epilogue, int pw_epilogue, hipStream_t stream);

/*
 * Winograd minimal filtering F(2x2, 3x3) (lpnh.cn section 3.3; lnrq.cn
 * section 2.2): the same 3x3, stride-1 convolution as conv2d_fwd_nhwc_packed
 * (dilation 1, groups 1, padding P, epilogue bias/ReLU), computed per 2x2
 * output block as Y = A^T [ (G g G^T) (.) (B^T d B) ] A summed over input
 * channels: 16 multiplications per block and channel pair instead of 36.
 * Numerics: the transformed input B^T d B and the transformed filter
 * G g G^T are each rounded to bf16 before the fp32-accumulated products, so
 * the result is not the direct path's bit for bit; integer-valued data with
 * small magnitudes stays exact.
 *
 * conv2d_winograd_transform_weights -- w [Cout][Cin][3][3] bf16 (the pages'
 *   layout) -> w_wino [16][Cin/8][Cout][8] bf16 holding G g G^T (computed in
 *   fp32, rounded to nearest even); conv2d_winograd_weight_bytes(Cout, Cin,
 *   dtype) bytes (0 on bad arguments).  Needs bf16 and Cin % 8 == 0
 *   (else CONV2D_ERR_UNSUPPORTED).  Enqueued on the stream.
 * conv2d_fwd_winograd_nhwc -- x [N][H][W][Cin] bf16 (NHWC), w_wino from the
 *   transform, bias fp32 [Cout] (iff CONV2D_EPI_BIAS), y [N][Ho][Wo][Cout]
 *   bf16 with Ho = H + 2P - 2, Wo = W + 2P - 2.  Runs bf16 with Cin % 8 == 0
 *   and Cout % 4 == 0; other valid calls return CONV2D_ERR_UNSUPPORTED.
 *   x, w_wino and y 16-byte aligned.  Allocates nothing; errors as for
 *   conv2d_fwd_nhwc_packed.
 */
size_t conv2d_winograd_weight_bytes(int Cout, int Cin, int dtype);
int conv2d_winograd_transform_weights(const void* w, void* w_wino, int Cout, int Cin, int dtype,
                                      hipStream_t stream);
int conv2d_fwd_winograd_nhwc(const void* x, const void* w_wino, const float* bias, void* y,
                             int N, int Cin, int H, int W, int Cout, int pad,
                             int dtype, int epilogue, hipStream_t stream);

/*
 * Transposed convolution (lpnh.cn sections 2.3 and 4.2: upsampling; the
 * stride-1 convolution of the input with S-1 zeros inserted between
 * neighbouring pixels; in matrix form Y = W^T X, the transpose of the
 * standard convolution's matrix).  Every input pixel's products with the
 * whole filter are added into the output window it spans:
 *   Y[n, co, ih*S - P + kh*D, iw*S - P + kw*D] += X[n, ci, ih, iw] * W[ci, co', kh, kw]
 *   ci in group g = co / (Cout/G), co' = co - g*Cout/G; sums that land
 *   outside the output are dropped; then epi (bias, ReLU) as above.
 *   Ho = (H-1)*S - 2P + D*(Kh-1) + OP + 1, likewise Wo, with the output
 *   padding OP (extra rows/columns at the far edge) 0 <= OP < max(S, D).
 *
 * conv2d_transpose_fwd -- the pages' layouts:
 *   x    [N][Cin][H][W]         (NCHW)
 *   w    [Cin][Cout/G][Kh][Kw]  (the standard weight's shapes reversed)
 *   bias fp32 [Cout], required iff epilogue has CONV2D_EPI_BIAS
 *   y    [N][Cout][Ho][Wo]      (NCHW), written completely
 * fp32 runs the direct kernel on these layouts; bf16 repacks x and w, runs
 * the chosen kernel and repacks y, in the same per-(device, stream) scratch
 * as conv2d_fwd (so it may allocate, and wait for its stream while it does).
 *
 * conv2d_transpose_fwd_nhwc_packed -- channels-last, allocates nothing:
 *   x        [N][H][W][Cin]     (NHWC)
 *   w_packed conv2d_transpose_pack_weights of w: [Cout][Kh][Kw][Cin/G]
 *   y        [N][Ho][Wo][Cout]  (NHWC)
 *
 * Paths: CONV2D_PATH_GEMM1X1 when the kernel equals the stride (Kh == Kw ==
 * S > 1, no padding, no output padding, dilation 1, groups 1, bf16,
 * Cin % 8 == 0, Cin <= 256, Cout % 32 == 0, Cout*Kh*Kw <= 256): the windows do
 * not overlap, so Y = W^T X is one GEMM of Cout*Kh*Kw rows over the input
 * pixels whose rows land in distinct output pixels.  CONV2D_PATH_IGEMM_HALO
 * for stride 2 with a 4x4 kernel (dilation 1, groups 1, padding <= 3, bf16,
 * Cin % 32 == 0, Cout % 4 == 0): each workgroup stages one input window per
 * block of 64 input channels in LDS and computes all four output phases from
 * it.
 * CONV2D_PATH_IGEMM_GATHER
 * (bf16, Cin/G % 8 == 0, Cout/G % 4 == 0) splits the output into its S x S
 * phases (rows and columns of one residue mod S); each phase is an implicit
 * GEMM on MFMA over only the taps that reach it.  CONV2D_PATH_DIRECT serves
 * every other shape and dtype.  conv2d_set_path_override applies
 * (CONV2D_PATH_IGEMM means the phase GEMM; a forced path that cannot run the
 * shape, or any other forced path, returns CONV2D_ERR_UNSUPPORTED).  Alignment, stream
 * and error behaviour as for conv2d_fwd / conv2d_fwd_nhwc_packed; an output
 * padding out of range returns CONV2D_ERR_ARG.
 */
int conv2d_transpose_fwd(const void* x, const void* w, const float* bias, void* y,
                         int N, int Cin, int H, int W, int Cout, int Kh, int Kw,
                         int stride, int pad, int output_padding, int dilation, int groups,
                         int dtype, int epilogue, hipStream_t stream);
int conv2d_transpose_fwd_nhwc_packed(const void* x, const void* w_packed, const float* bias, void* y,
                                     int N, int Cin, int H, int W, int Cout, int Kh, int Kw,
                                     int stride, int pad, int output_padding, int dilation, int groups,
                                     int dtype, int epilogue, hipStream_t stream);

/* [Cin][Cout/G][Kh][Kw] -> [Cout][Kh][Kw][Cin/G] (the packed layout below;
 * conv2d_packed_weight_bytes(Cout, Cin, Kh, Kw, groups, dtype) bytes).
 * Enqueued on the stream; w and w_packed must not overlap. */
int conv2d_transpose_pack_weights(const void* w, void* w_packed, int Cin, int Cout, int Kh, int Kw,
                                  int groups, int dtype, hipStream_t stream);

/* (in-1)*stride - 2*pad + dilation*(k-1) + output_padding + 1, or a value
 * <= 0 when that is empty; CONV2D_ERR_ARG for a stride/dilation/k/pad out of
 * range or output_padding outside [0, max(stride, dilation)).  Host only. */
int conv2d_transpose_out_dim(int in, int k, int stride, int pad, int dilation, int output_padding);

/* Host-only: the code a transposed call with these arguments would return
 * (CONV2D_OK if valid), and the path it would run. */
int conv2d_transpose_check_args(const void* x, const void* w, const float* bias, const void* y,
                                int N, int Cin, int H, int W, int Cout, int Kh, int Kw,
                                int stride, int pad, int output_padding, int dilation, int groups,
                                int dtype, int epilogue);
int conv2d_transpose_select_path(int N, int Cin, int H, int W, int Cout, int Kh, int Kw,
                                 int stride, int pad, int output_padding, int dilation, int groups,
                                 int dtype);

/*
 * Packed weight layout (the reduction order the NHWC kernels walk: tap
 * (kh, kw) outer, input channel inner; the row/column order of W_matrix,
 * lincklin.cn section 7, with K ordered to match channels-last input):
 *   depthwise (groups == Cin == Cout):  [Kh][Kw][C]
 *   otherwise:                          [Cout][Kh][Kw][Cin/G]
 * conv2d_packed_weight_bytes returns its size in bytes (0 on bad arguments).
 */
size_t conv2d_packed_weight_bytes(int Cout, int Cin, int Kh, int Kw, int groups, int dtype);
int conv2d_pack_weights(const void* w, void* w_packed, int Cout, int Cin, int Kh, int Kw,
                        int groups, int dtype, hipStream_t stream);

/* Activation layout passes (a full read and write of the tensor,
 * lincklin.cn section 30).  src and dst must not overlap. */
int conv2d_nchw_to_nhwc(const void* src, void* dst, int N, int C, int H, int W, int dtype,
                        hipStream_t stream);
int conv2d_nhwc_to_nchw(const void* src, void* dst, int N, int C, int H, int W, int dtype,
                        hipStream_t stream);

/* floor((in + 2*pad - dilation*(k-1) - 1)/stride) + 1, or a value <= 0 when
 * the window does not fit (lpnh.cn section 6.2); CONV2D_ERR_ARG on a bad
 * stride/dilation/k/pad. Host only. */
int conv2d_out_dim(int in, int k, int stride, int pad, int dilation);

/* Host-only validation of a conv2d_fwd / conv2d_fwd_nhwc_packed call: returns
 * CONV2D_OK or the code the call would return.  Needs no GPU. */
int conv2d_check_args(const void* x, const void* w, const float* bias, const void* y,
                      int N, int Cin, int H, int W, int Cout, int Kh, int Kw,
                      int stride, int pad, int dilation, int groups, int dtype, int epilogue);

/* Kernel the NHWC entry would run for this shape (CONV2D_PATH_DIRECT,
 * _DEPTHWISE, _GEMM1X1, _IGEMM_GATHER or _IGEMM_HALO), or a negative error
 * code.  Honours conv2d_set_path_override.  Host only. */
int conv2d_select_path(int N, int Cin, int H, int W, int Cout, int Kh, int Kw,
                       int stride, int pad, int dilation, int groups, int dtype);

/* Force a path for both forward entries (CONV2D_PATH_AUTO restores automatic
 * choice); a forced path that cannot run a shape makes the call return
 * CONV2D_ERR_UNSUPPORTED.  Process-wide; returns the previous setting, or
 * CONV2D_ERR_ARG for an unknown path.  Meant for tests and A/B timing. */
int conv2d_set_path_override(int path);

/* Cap the workgroups of every persistent launch (the halo-tile implicit
 * GEMMs, the streaming 1x1 kernel and the fused separable kernel) at
 * max_workgroups; 0 (the default) launches as many as fit on the device.
 * These kernels walk their output tiles in a grid-stride loop, so results do
 * not depend on the cap: a small cap makes every workgroup walk several tiles
 * (tests reach the cross-tile hand-over on small problems that way), and a
 * caller sharing the GPU with concurrent work can bound the footprint of one
 * call.  Process-wide; returns the previous cap, or CONV2D_ERR_ARG if
 * max_workgroups < 0.  Host only. */
int conv2d_set_grid_limit(int max_workgroups);

/* Diagnostics: with the environment variable CONV2D_LOG set (and not "0")
 * when the library first checks it, every conv2d_fwd*, conv2d_transpose_fwd*
 * call prints one line to stderr naming its shape and the kernel path it
 * chose (lpnh.cn section 6.3: check that the intended kernel ran). */

/* Free the NCHW entries' scratch blocks of every device and stream (after
 * synchronising the devices). */
void conv2d_release_scratch(void);

/* Static text for a return code, and the calling thread's last detailed
 * error message ("" if none). */
const char* conv2d_strerror(int code);
const char* conv2d_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* CONV2D_H */
