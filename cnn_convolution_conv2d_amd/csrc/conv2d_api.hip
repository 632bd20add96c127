// conv2d_api.hip -- C ABI of libconv2d.so: argument validation, output size,
// path selection, NCHW-entry scratch, and launches on the caller's stream.
#include <hip/hip_runtime.h>

#include <climits>
#include <initializer_list>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <vector>

#include "../../include/conv2d.h"
#include "common.hpp"

using namespace conv2d;

namespace {

thread_local char g_last_error[512] = "";

int set_error(int code, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
    va_end(ap);
    return code;
}

int hip_fail(hipError_t e, const char* what) {
    return set_error(CONV2D_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

int g_path_override = CONV2D_PATH_AUTO;
int g_grid_limit = 0;

// CONV2D_LOG (environment, read once): when set and not "0", every forward
// entry prints the kernel path it chose to stderr, one line per call, so a
// caller can check which kernel served a layer.
bool log_enabled() {
    static const bool on = [] {
        const char* v = getenv("CONV2D_LOG");
        return v && *v && strcmp(v, "0") != 0;
    }();
    return on;
}

const char* path_name(int path) {
    switch (path) {
    case CONV2D_PATH_DIRECT: return "direct";
    case CONV2D_PATH_DEPTHWISE: return "depthwise";
    case CONV2D_PATH_GEMM1X1: return "gemm1x1";
    case CONV2D_PATH_IGEMM_GATHER: return "igemm_gather";
    case CONV2D_PATH_IGEMM_HALO: return "igemm_halo";
    default: return "?";
    }
}

void log_path(const char* entry, const Shape& s, int path) {
    if (!log_enabled()) return;
    fprintf(stderr,
            "conv2d: %s N=%d Cin=%d H=%d W=%d Cout=%d K=%dx%d S=%d P=%d D=%d G=%d dtype=%s epi=%d -> %s\n",
            entry, s.N, s.Cin, s.H, s.W, s.Cout, s.Kh, s.Kw, s.stride, s.pad, s.dil, s.groups,
            s.dtype == CONV2D_F32 ? "f32" : "bf16", s.epilogue, path_name(path));
}

// Product of non-negative sizes, saturated at LLONG_MAX instead of
// overflowing (the size checks compare it with 2^31).
long long sat_mul(std::initializer_list<long long> f) {
    long long r = 1;
    for (long long v : f)
        if (__builtin_mul_overflow(r, v, &r)) return LLONG_MAX;
    return r;
}

// Output extent: floor((in + 2p - d(k-1) - 1)/s) + 1 (floor division of a
// possibly negative numerator).
long long out_extent(long long in, long long k, long long s, long long p, long long d) {
    long long num = in + 2 * p - d * (k - 1) - 1;
    long long q = num / s;
    if (num % s != 0 && num < 0) q -= 1;
    return q + 1;
}

int validate(const void* x, const void* w, const float* bias, const void* y,
             int N, int Cin, int H, int W, int Cout, int Kh, int Kw,
             int stride, int pad, int dilation, int groups, int dtype, int epilogue,
             Shape* out) {
    if (dtype != CONV2D_F32 && dtype != CONV2D_BF16)
        return set_error(CONV2D_ERR_DTYPE, "unknown dtype %d", dtype);
    if (epilogue < 0 || (epilogue & ~(CONV2D_EPI_BIAS | CONV2D_EPI_RELU)))
        return set_error(CONV2D_ERR_EPILOGUE, "unknown epilogue bits 0x%x", epilogue);
    if (N < 1 || Cin < 1 || H < 1 || W < 1 || Cout < 1 || Kh < 1 || Kw < 1)
        return set_error(CONV2D_ERR_ARG, "sizes must be >= 1 (N=%d Cin=%d H=%d W=%d Cout=%d Kh=%d Kw=%d)",
                         N, Cin, H, W, Cout, Kh, Kw);
    if (stride < 1 || dilation < 1 || pad < 0 || groups < 1)
        return set_error(CONV2D_ERR_ARG, "need stride>=1, dilation>=1, pad>=0, groups>=1 (got %d %d %d %d)",
                         stride, dilation, pad, groups);
    if (Cin % groups || Cout % groups)
        return set_error(CONV2D_ERR_GROUPS, "Cin=%d and Cout=%d must be divisible by groups=%d", Cin, Cout, groups);
    if (!x || !w || !y) return set_error(CONV2D_ERR_NULL, "x, w and y must be non-NULL");
    if ((epilogue & CONV2D_EPI_BIAS) && !bias)
        return set_error(CONV2D_ERR_NULL, "bias is NULL but the epilogue asks for it");
    long long Ho = out_extent(H, Kh, stride, pad, dilation);
    long long Wo = out_extent(W, Kw, stride, pad, dilation);
    if (Ho < 1 || Wo < 1)
        return set_error(CONV2D_ERR_EMPTY_OUTPUT, "empty output (Ho=%lld Wo=%lld)", Ho, Wo);
    const long long xe = sat_mul({N, Cin, H, W});
    const long long ye = sat_mul({N, Cout, Ho, Wo});
    const long long we = sat_mul({Cout, Cin / groups, Kh, Kw});
    if (xe >= INT_MAX || ye >= INT_MAX || we >= INT_MAX || (long long)H + 2LL * pad >= INT_MAX / 2)
        return set_error(CONV2D_ERR_UNSUPPORTED, "tensor too large for 32-bit element offsets");
    if (out) {
        Shape s;
        s.N = N; s.Cin = Cin; s.H = H; s.W = W; s.Cout = Cout; s.Kh = Kh; s.Kw = Kw;
        s.stride = stride; s.pad = pad; s.dil = dilation; s.groups = groups;
        s.Ho = (int)Ho; s.Wo = (int)Wo;
        s.cin_g = Cin / groups; s.cout_g = Cout / groups;
        s.dtype = dtype; s.epilogue = epilogue;
        s.scale = nullptr; s.shift = nullptr;
        s.out_pad = 0;
        *out = s;
    }
    return CONV2D_OK;
}

bool is_depthwise(const Shape& s) { return s.groups == s.Cin && s.Cout == s.Cin; }

bool path_can_run(int path, const Shape& s) {
    switch (path) {
    case CONV2D_PATH_DIRECT: return true;
    case CONV2D_PATH_DEPTHWISE: return s.dtype == CONV2D_BF16 && is_depthwise(s) && depthwise_supports(s);
    case CONV2D_PATH_GEMM1X1: return s.dtype == CONV2D_BF16 && gemm1x1_supports(s);
    case CONV2D_PATH_IGEMM:
    case CONV2D_PATH_IGEMM_GATHER: return s.dtype == CONV2D_BF16 && !is_depthwise(s) && igemm_supports(s);
    case CONV2D_PATH_IGEMM_HALO: return s.dtype == CONV2D_BF16 && !is_depthwise(s) && igemm_halo_supports(s);
    default: return false;
    }
}

// Implicit-GEMM variant: the halo-tile kernel where it is the faster one
// (stride 1, small filter span, enough output channels), else the per-tap
// gather.  3x3 stride 2 also runs on a halo-tile kernel, but only when that
// path is forced: on the measured stride-2 layer the gather is a few
// percent faster, although the staged window reads less of memory.
int igemm_variant(const Shape& s) {
    return igemm_halo_auto(s) ? CONV2D_PATH_IGEMM_HALO : CONV2D_PATH_IGEMM_GATHER;
}

// Automatic choice (host only): 1x1 -> GEMM; depthwise -> depthwise direct;
// channel-aligned bf16 -> implicit GEMM; anything else -> direct loop.
int auto_path(const Shape& s) {
    if (s.dtype != CONV2D_BF16) return CONV2D_PATH_DIRECT;
    if (is_depthwise(s)) return depthwise_supports(s) ? CONV2D_PATH_DEPTHWISE : CONV2D_PATH_DIRECT;
    if (gemm1x1_supports(s)) return CONV2D_PATH_GEMM1X1;
    if (igemm_supports(s)) return igemm_variant(s);
    return CONV2D_PATH_DIRECT;
}

int choose_path(const Shape& s) {
    int forced = __atomic_load_n(&g_path_override, __ATOMIC_RELAXED);
    if (forced == CONV2D_PATH_AUTO) return auto_path(s);
    if (!path_can_run(forced, s))
        return set_error(CONV2D_ERR_UNSUPPORTED, "forced path %d cannot run this shape", forced);
    return forced == CONV2D_PATH_IGEMM ? igemm_variant(s) : forced;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int run_nhwc(int path, const Shape& s, const void* x, const void* wp, const float* bias, void* y,
             hipStream_t st) {
    hipError_t e = hipSuccess;
    if (path != CONV2D_PATH_DIRECT && !(aligned16(x) && aligned16(wp) && aligned16(y)))
        return set_error(CONV2D_ERR_ALIGN, "x, w_packed and y must be 16-byte aligned for path %d", path);
    switch (path) {
    case CONV2D_PATH_DIRECT:
        e = launch_direct(s, x, NHWC, wp, is_depthwise(s) ? W_DW : W_PACKED, bias, y, NHWC, st);
        break;
    case CONV2D_PATH_DEPTHWISE: e = launch_depthwise(s, x, wp, bias, y, st); break;
    case CONV2D_PATH_GEMM1X1:
        // the streaming kernel where the weights fit in LDS, else the tiled GEMM
        e = pointwise_supports(s) ? launch_pointwise(s, x, wp, bias, y, st)
                                  : launch_gemm1x1(s, x, wp, bias, y, st);
        break;
    case CONV2D_PATH_IGEMM_GATHER: e = launch_igemm(s, x, wp, bias, y, st); break;
    case CONV2D_PATH_IGEMM_HALO: e = launch_igemm_halo(s, x, wp, bias, y, st); break;
    default: return set_error(CONV2D_ERR_UNSUPPORTED, "unknown path %d", path);
    }
    if (e != hipSuccess) return hip_fail(e, "kernel launch");
    return CONV2D_OK;
}

size_t elem_bytes(int dtype) { return dtype == CONV2D_F32 ? 4 : 2; }

size_t round_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

// Scratch of the NCHW entries: one block per (device, stream), so calls on
// different streams never share staging memory.  A block only grows; the
// work that may still read the old block is the earlier work of the same
// stream, so growing waits for that stream.
constexpr int kMaxDevices = 64;
struct ScratchBlock {
    int dev;
    hipStream_t stream;
    void* ptr;
    size_t bytes;
};
std::mutex g_scratch_mu;
std::vector<ScratchBlock> g_scratch;

int get_scratch(size_t bytes, hipStream_t stream, void** out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
    if (dev < 0 || dev >= kMaxDevices) return set_error(CONV2D_ERR_UNSUPPORTED, "device id %d", dev);
    std::lock_guard<std::mutex> lk(g_scratch_mu);
    ScratchBlock* b = nullptr;
    for (auto& sb : g_scratch)
        if (sb.dev == dev && sb.stream == stream) b = &sb;
    if (!b) {
        g_scratch.push_back(ScratchBlock{dev, stream, nullptr, 0});
        b = &g_scratch.back();
    }
    if (b->bytes < bytes) {
        // Growing waits for the stream and allocates, neither of which a
        // stream capture allows.
        hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
        e = hipStreamIsCapturing(stream, &cs);
        if (e != hipSuccess) return hip_fail(e, "hipStreamIsCapturing");
        if (cs != hipStreamCaptureStatusNone)
            return set_error(CONV2D_ERR_UNSUPPORTED,
                             "the NCHW entry's scratch must grow to %zu bytes, which cannot happen during a stream "
                             "capture: call it once before capturing, or use conv2d_fwd_nhwc_packed", bytes);
        if (b->ptr) {
            // earlier work on this stream may still read the old block
            e = hipStreamSynchronize(stream);
            if (e != hipSuccess) return hip_fail(e, "hipStreamSynchronize");
            e = hipFree(b->ptr);
            b->ptr = nullptr;
            b->bytes = 0;
            if (e != hipSuccess) return hip_fail(e, "hipFree");
        }
        size_t want = round_up(bytes, size_t(1) << 21);
        e = hipMalloc(&b->ptr, want);
        if (e != hipSuccess) {
            b->ptr = nullptr;
            return hip_fail(e, "hipMalloc(scratch)");
        }
        b->bytes = want;
    }
    *out = b->ptr;
    return CONV2D_OK;
}

// Validation shared by the forward entries; with_bn: the folded batch
// normalisation tables are required (non-NULL) and stored in the shape.
int validate_fwd(const void* x, const void* w, const float* bias, const float* scale, const float* shift,
                 const void* y, int N, int Cin, int H, int W, int Cout, int Kh, int Kw, int stride, int pad,
                 int dilation, int groups, int dtype, int epilogue, bool with_bn, Shape* s) {
    int rc = validate(x, w, bias, y, N, Cin, H, W, Cout, Kh, Kw, stride, pad, dilation, groups, dtype, epilogue, s);
    if (rc) return rc;
    if (with_bn) {
        if (!scale || !shift) return set_error(CONV2D_ERR_NULL, "scale and shift must be non-NULL");
        s->scale = scale;
        s->shift = shift;
    }
    return CONV2D_OK;
}

int fwd_nhwc_packed(const void* x, const void* w_packed, const float* bias, const float* scale, const float* shift,
                    void* y, int N, int Cin, int H, int W, int Cout, int Kh, int Kw, int stride, int pad,
                    int dilation, int groups, int dtype, int epilogue, hipStream_t stream, bool with_bn) {
    Shape s;
    int rc = validate_fwd(x, w_packed, bias, scale, shift, y, N, Cin, H, W, Cout, Kh, Kw, stride, pad, dilation,
                          groups, dtype, epilogue, with_bn, &s);
    if (rc) return rc;
    int path = choose_path(s);
    if (path < 0) return path;
    log_path(with_bn ? "conv2d_fwd_nhwc_packed_bn" : "conv2d_fwd_nhwc_packed", s, path);
    return run_nhwc(path, s, x, w_packed, bias, y, stream);
}

// Staging of the NCHW entry's channels-last path: packed weights, the NHWC
// copy of x and the NHWC result, each 256-byte aligned, in one block.
struct Staging {
    size_t wb, xb, yb;
    size_t total() const { return wb + xb + yb; }
};

Staging staging_of(const Shape& s) {
    const size_t eb = elem_bytes(s.dtype);
    Staging g;
    g.wb = round_up(conv2d_packed_weight_bytes(s.Cout, s.Cin, s.Kh, s.Kw, s.groups, s.dtype), 256);
    g.xb = round_up((size_t)s.N * s.Cin * s.H * s.W * eb, 256);
    g.yb = round_up((size_t)s.N * s.Cout * s.Ho * s.Wo * eb, 256);
    return g;
}

// Repack w and x into the block at `base`, run the kernel of `path` on the
// channels-last copies and write y back as NCHW (lincklin.cn lesson 9,
// sections 29-30).  Every byte of the block that is read was written earlier
// in the same call, on the same stream.
int run_staged(int path, const Shape& s, const Staging& g, char* base, const void* x, const void* w,
               const float* bias, void* y, hipStream_t stream) {
    void* wp = base;
    void* xn = base + g.wb;
    void* yn = base + g.wb + g.xb;
    int rc = conv2d_pack_weights(w, wp, s.Cout, s.Cin, s.Kh, s.Kw, s.groups, s.dtype, stream);
    if (rc) return rc;
    rc = conv2d_nchw_to_nhwc(x, xn, s.N, s.Cin, s.H, s.W, s.dtype, stream);
    if (rc) return rc;
    rc = run_nhwc(path, s, xn, wp, bias, yn, stream);
    if (rc) return rc;
    return conv2d_nhwc_to_nchw(yn, y, s.N, s.Cout, s.Ho, s.Wo, s.dtype, stream);
}

int fwd_nchw(const void* x, const void* w, const float* bias, const float* scale, const float* shift, void* y,
             int N, int Cin, int H, int W, int Cout, int Kh, int Kw, int stride, int pad, int dilation, int groups,
             int dtype, int epilogue, hipStream_t stream, bool with_bn) {
    Shape s;
    int rc = validate_fwd(x, w, bias, scale, shift, y, N, Cin, H, W, Cout, Kh, Kw, stride, pad, dilation, groups,
                          dtype, epilogue, with_bn, &s);
    if (rc) return rc;
    int path = choose_path(s);
    if (path < 0) return path;
    log_path(with_bn ? "conv2d_fwd_bn" : "conv2d_fwd", s, path);
    if (path == CONV2D_PATH_DIRECT) {
        // The direct loop reads the pages' layouts as they are: no repack.
        hipError_t e = launch_direct(s, x, NCHW, w, W_OIHW, bias, y, NCHW, stream);
        return e == hipSuccess ? CONV2D_OK : hip_fail(e, "direct launch");
    }
    const Staging g = staging_of(s);
    void* scratch = nullptr;
    rc = get_scratch(g.total(), stream, &scratch);
    if (rc) return rc;
    return run_staged(path, s, g, static_cast<char*>(scratch), x, w, bias, y, stream);
}

// ---- the allocation-free NCHW entry
//
// Its staging lives in one statically sized device array per GPU, reserved
// when the code object is loaded and kept until the process ends.  In host
// code `scratch` names a host-side stand-in, not device memory: the array's
// address on each device comes from hipGetSymbolAddress, taken once per
// device with that device current, and only that address is handed to
// kernels.
constexpr size_t kNoAllocScratchBytes = size_t(64) << 20;
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

std::mutex g_noalloc_mu;
void* g_noalloc_ptr[kMaxDevices] = {};

int noalloc_scratch(void** out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
    if (dev < 0 || dev >= kMaxDevices) return set_error(CONV2D_ERR_UNSUPPORTED, "device id %d", dev);
    std::lock_guard<std::mutex> lk(g_noalloc_mu);
    if (!g_noalloc_ptr[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !p) return hip_fail(e != hipSuccess ? e : hipErrorInvalidSymbol,
                                                  "hipGetSymbolAddress(scratch)");
        g_noalloc_ptr[dev] = p;
    }
    *out = g_noalloc_ptr[dev];
    return CONV2D_OK;
}

// ---- transposed convolution

// Output extent of the transposed convolution: (in-1)S - 2P + D(k-1) + OP + 1.
long long tout_extent(long long in, long long k, long long s, long long p, long long d, long long op) {
    return (in - 1) * s - 2 * p + d * (k - 1) + op + 1;
}

int validate_transposed(const void* x, const void* w, const float* bias, const void* y, int N, int Cin, int H,
                        int W, int Cout, int Kh, int Kw, int stride, int pad, int out_pad, int dilation,
                        int groups, int dtype, int epilogue, Shape* out) {
    if (dtype != CONV2D_F32 && dtype != CONV2D_BF16)
        return set_error(CONV2D_ERR_DTYPE, "unknown dtype %d", dtype);
    if (epilogue < 0 || (epilogue & ~(CONV2D_EPI_BIAS | CONV2D_EPI_RELU)))
        return set_error(CONV2D_ERR_EPILOGUE, "unknown epilogue bits 0x%x", epilogue);
    if (N < 1 || Cin < 1 || H < 1 || W < 1 || Cout < 1 || Kh < 1 || Kw < 1)
        return set_error(CONV2D_ERR_ARG, "sizes must be >= 1 (N=%d Cin=%d H=%d W=%d Cout=%d Kh=%d Kw=%d)",
                         N, Cin, H, W, Cout, Kh, Kw);
    if (stride < 1 || dilation < 1 || pad < 0 || groups < 1)
        return set_error(CONV2D_ERR_ARG, "need stride>=1, dilation>=1, pad>=0, groups>=1 (got %d %d %d %d)",
                         stride, dilation, pad, groups);
    if (out_pad < 0 || (out_pad >= stride && out_pad >= dilation))
        return set_error(CONV2D_ERR_ARG, "output padding %d must be >= 0 and below stride %d or dilation %d",
                         out_pad, stride, dilation);
    if (Cin % groups || Cout % groups)
        return set_error(CONV2D_ERR_GROUPS, "Cin=%d and Cout=%d must be divisible by groups=%d", Cin, Cout, groups);
    if (!x || !w || !y) return set_error(CONV2D_ERR_NULL, "x, w and y must be non-NULL");
    if ((epilogue & CONV2D_EPI_BIAS) && !bias)
        return set_error(CONV2D_ERR_NULL, "bias is NULL but the epilogue asks for it");
    const long long Ho = tout_extent(H, Kh, stride, pad, dilation, out_pad);
    const long long Wo = tout_extent(W, Kw, stride, pad, dilation, out_pad);
    if (Ho < 1 || Wo < 1) return set_error(CONV2D_ERR_EMPTY_OUTPUT, "empty output (Ho=%lld Wo=%lld)", Ho, Wo);
    const long long xe = sat_mul({N, Cin, H, W}), ye = sat_mul({N, Cout, Ho, Wo});
    const long long we = sat_mul({Cout, Cin / groups, Kh, Kw});
    if (xe >= INT_MAX || ye >= INT_MAX || we >= INT_MAX || Ho >= INT_MAX / 2 || Wo >= INT_MAX / 2 ||
        (long long)pad + (long long)dilation * Kh >= INT_MAX / 2 || (long long)dilation * Kw >= INT_MAX / 2)
        return set_error(CONV2D_ERR_UNSUPPORTED, "tensor too large for 32-bit element offsets");
    if (out) {
        Shape s;
        s.N = N; s.Cin = Cin; s.H = H; s.W = W; s.Cout = Cout; s.Kh = Kh; s.Kw = Kw;
        s.stride = stride; s.pad = pad; s.dil = dilation; s.groups = groups;
        s.Ho = (int)Ho; s.Wo = (int)Wo;
        s.cin_g = Cin / groups; s.cout_g = Cout / groups;
        s.dtype = dtype; s.epilogue = epilogue;
        s.scale = nullptr; s.shift = nullptr;
        s.out_pad = out_pad;
        *out = s;
    }
    return CONV2D_OK;
}

// Transposed paths: kernel == stride without padding -> the pointwise GEMM
// with pixel-shuffled output (reported as the 1x1 path); stride 2 with a 4x4
// kernel -> all phases on one staged input window (reported as the halo
// path); other channel-aligned bf16 -> the phase-split implicit GEMM
// (reported as the gather path); the direct loop otherwise.
int choose_tpath(const Shape& s) {
    const bool mfma = s.dtype == CONV2D_BF16 && igemm_transposed_supports(s);
    const bool shuf = pw_shuffle_supports(s);
    const bool halo = tconv_halo_supports(s);
    const int forced = __atomic_load_n(&g_path_override, __ATOMIC_RELAXED);
    if (forced == CONV2D_PATH_AUTO)
        return shuf ? CONV2D_PATH_GEMM1X1 : halo ? CONV2D_PATH_IGEMM_HALO
                                                 : mfma ? CONV2D_PATH_IGEMM_GATHER : CONV2D_PATH_DIRECT;
    if (forced == CONV2D_PATH_DIRECT) return CONV2D_PATH_DIRECT;
    if ((forced == CONV2D_PATH_IGEMM || forced == CONV2D_PATH_IGEMM_GATHER) && mfma)
        return CONV2D_PATH_IGEMM_GATHER;
    if (forced == CONV2D_PATH_GEMM1X1 && shuf) return CONV2D_PATH_GEMM1X1;
    if (forced == CONV2D_PATH_IGEMM_HALO && halo) return CONV2D_PATH_IGEMM_HALO;
    return set_error(CONV2D_ERR_UNSUPPORTED, "forced path %d cannot run this transposed convolution", forced);
}

int run_tnhwc(int path, const Shape& s, const void* x, const void* wp, const float* bias, void* y,
              hipStream_t st) {
    hipError_t e;
    if (path == CONV2D_PATH_DIRECT) {
        e = launch_tconv_direct(s, x, NHWC, wp, W_PACKED, bias, y, NHWC, st);
    } else {
        if (!(aligned16(x) && aligned16(wp) && aligned16(y)))
            return set_error(CONV2D_ERR_ALIGN, "x, w_packed and y must be 16-byte aligned for path %d", path);
        e = path == CONV2D_PATH_GEMM1X1     ? launch_pw_shuffle(s, x, wp, bias, y, st)
            : path == CONV2D_PATH_IGEMM_HALO ? launch_tconv_halo(s, x, wp, bias, y, st)
                                             : launch_igemm_transposed(s, x, wp, bias, y, st);
    }
    return e == hipSuccess ? CONV2D_OK : hip_fail(e, "transposed kernel launch");
}

}  // namespace

int conv2d::grid_limit() { return __atomic_load_n(&g_grid_limit, __ATOMIC_RELAXED); }

extern "C" {

int conv2d_set_grid_limit(int max_workgroups) {
    if (max_workgroups < 0) return set_error(CONV2D_ERR_ARG, "grid limit %d must be >= 0", max_workgroups);
    return __atomic_exchange_n(&g_grid_limit, max_workgroups, __ATOMIC_RELAXED);
}

int conv2d_out_dim(int in, int k, int stride, int pad, int dilation) {
    if (stride < 1 || dilation < 1 || k < 1 || pad < 0 || in < 1) return CONV2D_ERR_ARG;
    long long r = out_extent(in, k, stride, pad, dilation);
    if (r > INT_MAX) return CONV2D_ERR_ARG;
    return r < 0 ? 0 : (int)r;
}

int conv2d_check_args(const void* x, const void* w, const float* bias, const void* y,
                      int N, int Cin, int H, int W, int Cout, int Kh, int Kw,
                      int stride, int pad, int dilation, int groups, int dtype, int epilogue) {
    return validate(x, w, bias, y, N, Cin, H, W, Cout, Kh, Kw, stride, pad, dilation, groups,
                    dtype, epilogue, nullptr);
}

int conv2d_select_path(int N, int Cin, int H, int W, int Cout, int Kh, int Kw,
                       int stride, int pad, int dilation, int groups, int dtype) {
    Shape s;
    static const char dummy[16] = {};
    int rc = validate(dummy, dummy, nullptr, dummy, N, Cin, H, W, Cout, Kh, Kw, stride, pad,
                      dilation, groups, dtype, 0, &s);
    if (rc) return rc;
    return choose_path(s);
}

int conv2d_set_path_override(int path) {
    if (path < CONV2D_PATH_AUTO || path > CONV2D_PATH_IGEMM_HALO) return CONV2D_ERR_ARG;
    return __atomic_exchange_n(&g_path_override, path, __ATOMIC_RELAXED);
}

size_t conv2d_packed_weight_bytes(int Cout, int Cin, int Kh, int Kw, int groups, int dtype) {
    if (Cout < 1 || Cin < 1 || Kh < 1 || Kw < 1 || groups < 1 || Cin % groups || Cout % groups)
        return 0;
    if (dtype != CONV2D_F32 && dtype != CONV2D_BF16) return 0;
    const long long bytes = sat_mul({Cout, Cin / groups, Kh, Kw, (long long)elem_bytes(dtype)});
    return bytes == LLONG_MAX ? 0 : (size_t)bytes;
}

int conv2d_pack_weights(const void* w, void* w_packed, int Cout, int Cin, int Kh, int Kw,
                        int groups, int dtype, hipStream_t stream) {
    if (dtype != CONV2D_F32 && dtype != CONV2D_BF16) return set_error(CONV2D_ERR_DTYPE, "unknown dtype %d", dtype);
    if (Cout < 1 || Cin < 1 || Kh < 1 || Kw < 1 || groups < 1)
        return set_error(CONV2D_ERR_ARG, "sizes must be >= 1");
    if (Cin % groups || Cout % groups) return set_error(CONV2D_ERR_GROUPS, "channels not divisible by groups");
    if (!w || !w_packed) return set_error(CONV2D_ERR_NULL, "w and w_packed must be non-NULL");
    if (sat_mul({Cout, Cin / groups, Kh, Kw}) >= INT_MAX)
        return set_error(CONV2D_ERR_UNSUPPORTED, "weight too large");
    int dw = (groups == Cin && Cout == Cin) ? 1 : 0;
    hipError_t e = launch_pack_weights(w, w_packed, Cout, Cin / groups, Kh, Kw, dw,
                                       (int)elem_bytes(dtype), stream);
    return e == hipSuccess ? CONV2D_OK : hip_fail(e, "pack_weights launch");
}

static int transpose_args(const void* src, void* dst, int N, int C, int H, int W, int dtype) {
    if (dtype != CONV2D_F32 && dtype != CONV2D_BF16) return set_error(CONV2D_ERR_DTYPE, "unknown dtype %d", dtype);
    if (N < 1 || C < 1 || H < 1 || W < 1) return set_error(CONV2D_ERR_ARG, "sizes must be >= 1");
    if (!src || !dst) return set_error(CONV2D_ERR_NULL, "src and dst must be non-NULL");
    if (sat_mul({N, C, H, W}) >= INT_MAX) return set_error(CONV2D_ERR_UNSUPPORTED, "tensor too large");
    return CONV2D_OK;
}

int conv2d_nchw_to_nhwc(const void* src, void* dst, int N, int C, int H, int W, int dtype,
                        hipStream_t stream) {
    int rc = transpose_args(src, dst, N, C, H, W, dtype);
    if (rc) return rc;
    hipError_t e = launch_transpose(src, dst, N, C, H * W, (int)elem_bytes(dtype), stream);
    return e == hipSuccess ? CONV2D_OK : hip_fail(e, "nchw_to_nhwc launch");
}

int conv2d_nhwc_to_nchw(const void* src, void* dst, int N, int C, int H, int W, int dtype,
                        hipStream_t stream) {
    int rc = transpose_args(src, dst, N, C, H, W, dtype);
    if (rc) return rc;
    hipError_t e = launch_transpose(src, dst, N, H * W, C, (int)elem_bytes(dtype), stream);
    return e == hipSuccess ? CONV2D_OK : hip_fail(e, "nhwc_to_nchw launch");
}

int conv2d_fwd_nhwc_packed(const void* x, const void* w_packed, const float* bias, void* y,
                           int N, int Cin, int H, int W, int Cout, int Kh, int Kw,
                           int stride, int pad, int dilation, int groups,
                           int dtype, int epilogue, hipStream_t stream) {
    return fwd_nhwc_packed(x, w_packed, bias, nullptr, nullptr, y, N, Cin, H, W, Cout, Kh, Kw, stride, pad,
                           dilation, groups, dtype, epilogue, stream, false);
}

int conv2d_fwd_nhwc_packed_bn(const void* x, const void* w_packed, const float* bias, const float* scale,
                              const float* shift, void* y, int N, int Cin, int H, int W, int Cout, int Kh,
                              int Kw, int stride, int pad, int dilation, int groups, int dtype, int epilogue,
                              hipStream_t stream) {
    return fwd_nhwc_packed(x, w_packed, bias, scale, shift, y, N, Cin, H, W, Cout, Kh, Kw, stride, pad,
                           dilation, groups, dtype, epilogue, stream, true);
}

int conv2d_fwd(const void* x, const void* w, const float* bias, void* y,
               int N, int Cin, int H, int W, int Cout, int Kh, int Kw,
               int stride, int pad, int dilation, int groups,
               int dtype, int epilogue, hipStream_t stream) {
    return fwd_nchw(x, w, bias, nullptr, nullptr, y, N, Cin, H, W, Cout, Kh, Kw, stride, pad, dilation, groups,
                    dtype, epilogue, stream, false);
}

int conv2d_fwd_noalloc(const void* x, const void* w, const float* bias, void* y,
                       int N, int Cin, int H, int W, int Cout, int Kh, int Kw,
                       int stride, int pad, int dilation, int groups,
                       int dtype, int epilogue, hipStream_t stream) {
    Shape s;
    int rc = validate(x, w, bias, y, N, Cin, H, W, Cout, Kh, Kw, stride, pad, dilation, groups, dtype, epilogue,
                      &s);
    if (rc) return rc;
    const int path = choose_path(s);
    if (path < 0) return path;
    log_path("conv2d_fwd_noalloc", s, path);
    if (path == CONV2D_PATH_DIRECT) {
        const hipError_t e = launch_direct(s, x, NCHW, w, W_OIHW, bias, y, NCHW, stream);
        return e == hipSuccess ? CONV2D_OK : hip_fail(e, "direct launch");
    }
    const Staging g = staging_of(s);
    if (g.total() > kNoAllocScratchBytes)
        return set_error(CONV2D_ERR_UNSUPPORTED,
                         "conv2d_fwd_noalloc needs %zu bytes of staging (packed weights, NHWC x and y) but its "
                         "static scratch holds %zu; use conv2d_fwd or conv2d_fwd_nhwc_packed",
                         g.total(), kNoAllocScratchBytes);
    void* base = nullptr;
    rc = noalloc_scratch(&base);
    if (rc) return rc;
    return run_staged(path, s, g, static_cast<char*>(base), x, w, bias, y, stream);
}

int conv2d_fwd_bn(const void* x, const void* w, const float* bias, const float* scale, const float* shift,
                  void* y, int N, int Cin, int H, int W, int Cout, int Kh, int Kw, int stride, int pad,
                  int dilation, int groups, int dtype, int epilogue, hipStream_t stream) {
    return fwd_nchw(x, w, bias, scale, shift, y, N, Cin, H, W, Cout, Kh, Kw, stride, pad, dilation, groups,
                    dtype, epilogue, stream, true);
}

int conv2d_fwd_separable_nhwc(const void* x, const void* w_dw, const float* bias_dw, const void* w_pw,
                              const float* bias_pw, void* y, int N, int C, int H, int W, int Cout,
                              int stride, int pad, int dtype, int dw_epilogue, int pw_epilogue,
                              hipStream_t stream) {
    if (dtype != CONV2D_F32 && dtype != CONV2D_BF16) return set_error(CONV2D_ERR_DTYPE, "unknown dtype %d", dtype);
    const int known = CONV2D_EPI_BIAS | CONV2D_EPI_RELU;
    if (dw_epilogue < 0 || (dw_epilogue & ~known) || pw_epilogue < 0 || (pw_epilogue & ~known))
        return set_error(CONV2D_ERR_EPILOGUE, "unknown epilogue bits (depthwise 0x%x, pointwise 0x%x)",
                         dw_epilogue, pw_epilogue);
    if (N < 1 || C < 1 || H < 1 || W < 1 || Cout < 1)
        return set_error(CONV2D_ERR_ARG, "sizes must be >= 1 (N=%d C=%d H=%d W=%d Cout=%d)", N, C, H, W, Cout);
    if (stride < 1 || pad < 0) return set_error(CONV2D_ERR_ARG, "need stride>=1, pad>=0 (got %d %d)", stride, pad);
    if (!x || !w_dw || !w_pw || !y) return set_error(CONV2D_ERR_NULL, "x, w_dw, w_pw and y must be non-NULL");
    if ((dw_epilogue & CONV2D_EPI_BIAS) && !bias_dw)
        return set_error(CONV2D_ERR_NULL, "bias_dw is NULL but the depthwise epilogue asks for it");
    if ((pw_epilogue & CONV2D_EPI_BIAS) && !bias_pw)
        return set_error(CONV2D_ERR_NULL, "bias_pw is NULL but the pointwise epilogue asks for it");
    if ((long long)H + 2LL * pad >= INT_MAX / 2) return set_error(CONV2D_ERR_UNSUPPORTED, "padding too large");
    const long long Ho = out_extent(H, 3, stride, pad, 1), Wo = out_extent(W, 3, stride, pad, 1);
    if (Ho < 1 || Wo < 1) return set_error(CONV2D_ERR_EMPTY_OUTPUT, "empty output (Ho=%lld Wo=%lld)", Ho, Wo);
    if (sat_mul({N, C, H, W}) >= INT_MAX || sat_mul({N, Cout, Ho, Wo}) >= INT_MAX)
        return set_error(CONV2D_ERR_UNSUPPORTED, "tensor too large for 32-bit element offsets");
    if (dtype != CONV2D_BF16)
        return set_error(CONV2D_ERR_UNSUPPORTED, "the fused depthwise-separable kernel runs bf16 only");
    SepShape ss;
    ss.N = N; ss.C = C; ss.H = H; ss.W = W; ss.Cout = Cout; ss.stride = stride; ss.pad = pad;
    ss.Ho = (int)Ho; ss.Wo = (int)Wo; ss.dw_epilogue = dw_epilogue; ss.pw_epilogue = pw_epilogue;
    if (!separable_supports(ss))
        return set_error(CONV2D_ERR_UNSUPPORTED,
                         "fused depthwise-separable needs C %% 8 == 0, C <= 256, Cout %% 4 == 0, Cout <= 128, "
                         "stride 1 or 2 and tensors below 2 GiB (got C=%d Cout=%d stride=%d)", C, Cout, stride);
    if (!(aligned16(x) && aligned16(w_dw) && aligned16(w_pw) && aligned16(y)))
        return set_error(CONV2D_ERR_ALIGN, "x, w_dw, w_pw and y must be 16-byte aligned");
    const hipError_t e = launch_separable(ss, x, w_dw, bias_dw, w_pw, bias_pw, y, stream);
    return e == hipSuccess ? CONV2D_OK : hip_fail(e, "separable launch");
}

size_t conv2d_winograd_weight_bytes(int Cout, int Cin, int dtype) {
    if (Cout < 1 || Cin < 1 || Cin % 8 || dtype != CONV2D_BF16) return 0;
    if (sat_mul({16, Cout, Cin, 2}) >= INT_MAX) return 0;
    return (size_t)16 * Cout * Cin * 2;
}

int conv2d_winograd_transform_weights(const void* w, void* w_wino, int Cout, int Cin, int dtype, hipStream_t stream) {
    if (dtype != CONV2D_F32 && dtype != CONV2D_BF16) return set_error(CONV2D_ERR_DTYPE, "unknown dtype %d", dtype);
    if (Cout < 1 || Cin < 1) return set_error(CONV2D_ERR_ARG, "sizes must be >= 1");
    if (!w || !w_wino) return set_error(CONV2D_ERR_NULL, "w and w_wino must be non-NULL");
    if (dtype != CONV2D_BF16 || Cin % 8 || sat_mul({16, Cout, Cin, 2}) >= INT_MAX)
        return set_error(CONV2D_ERR_UNSUPPORTED, "Winograd weights need bf16, Cin %% 8 == 0 (got Cin=%d)", Cin);
    const hipError_t e = launch_winograd_weights(w, w_wino, Cout, Cin, stream);
    return e == hipSuccess ? CONV2D_OK : hip_fail(e, "winograd weight transform launch");
}

int conv2d_fwd_winograd_nhwc(const void* x, const void* w_wino, const float* bias, void* y, int N, int Cin, int H,
                             int W, int Cout, int pad, int dtype, int epilogue, hipStream_t stream) {
    Shape s;
    int rc = validate(x, w_wino, bias, y, N, Cin, H, W, Cout, 3, 3, 1, pad, 1, 1, dtype, epilogue, &s);
    if (rc) return rc;
    if (!winograd_supports(s))
        return set_error(CONV2D_ERR_UNSUPPORTED,
                         "Winograd F(2x2,3x3) needs bf16, Cin %% 8 == 0, Cout %% 4 == 0 and tensors below 2 GiB "
                         "(got dtype %d Cin=%d Cout=%d)", dtype, Cin, Cout);
    if (!(aligned16(x) && aligned16(w_wino) && aligned16(y)))
        return set_error(CONV2D_ERR_ALIGN, "x, w_wino and y must be 16-byte aligned");
    const hipError_t e = launch_winograd(s, x, w_wino, bias, y, stream);
    return e == hipSuccess ? CONV2D_OK : hip_fail(e, "winograd launch");
}

int conv2d_transpose_out_dim(int in, int k, int stride, int pad, int dilation, int output_padding) {
    if (stride < 1 || dilation < 1 || k < 1 || pad < 0 || in < 1 || output_padding < 0 ||
        (output_padding >= stride && output_padding >= dilation))
        return CONV2D_ERR_ARG;
    const long long r = tout_extent(in, k, stride, pad, dilation, output_padding);
    if (r > INT_MAX) return CONV2D_ERR_ARG;
    return r < 0 ? 0 : (int)r;
}

int conv2d_transpose_check_args(const void* x, const void* w, const float* bias, const void* y, int N, int Cin,
                                int H, int W, int Cout, int Kh, int Kw, int stride, int pad, int output_padding,
                                int dilation, int groups, int dtype, int epilogue) {
    return validate_transposed(x, w, bias, y, N, Cin, H, W, Cout, Kh, Kw, stride, pad, output_padding, dilation,
                               groups, dtype, epilogue, nullptr);
}

int conv2d_transpose_select_path(int N, int Cin, int H, int W, int Cout, int Kh, int Kw, int stride, int pad,
                                 int output_padding, int dilation, int groups, int dtype) {
    Shape s;
    static const char dummy[16] = {};
    int rc = validate_transposed(dummy, dummy, nullptr, dummy, N, Cin, H, W, Cout, Kh, Kw, stride, pad,
                                 output_padding, dilation, groups, dtype, 0, &s);
    if (rc) return rc;
    return choose_tpath(s);
}

int conv2d_transpose_pack_weights(const void* w, void* w_packed, int Cin, int Cout, int Kh, int Kw, int groups,
                                  int dtype, hipStream_t stream) {
    if (dtype != CONV2D_F32 && dtype != CONV2D_BF16) return set_error(CONV2D_ERR_DTYPE, "unknown dtype %d", dtype);
    if (Cout < 1 || Cin < 1 || Kh < 1 || Kw < 1 || groups < 1)
        return set_error(CONV2D_ERR_ARG, "sizes must be >= 1");
    if (Cin % groups || Cout % groups) return set_error(CONV2D_ERR_GROUPS, "channels not divisible by groups");
    if (!w || !w_packed) return set_error(CONV2D_ERR_NULL, "w and w_packed must be non-NULL");
    if (sat_mul({Cout, Cin / groups, Kh, Kw}) >= INT_MAX)
        return set_error(CONV2D_ERR_UNSUPPORTED, "weight too large");
    hipError_t e = launch_tpack_weights(w, w_packed, Cin, Cout / groups, groups, Kh, Kw, (int)elem_bytes(dtype),
                                        stream);
    return e == hipSuccess ? CONV2D_OK : hip_fail(e, "transpose_pack_weights launch");
}

int conv2d_transpose_fwd_nhwc_packed(const void* x, const void* w_packed, const float* bias, void* y, int N,
                                     int Cin, int H, int W, int Cout, int Kh, int Kw, int stride, int pad,
                                     int output_padding, int dilation, int groups, int dtype, int epilogue,
                                     hipStream_t stream) {
    Shape s;
    int rc = validate_transposed(x, w_packed, bias, y, N, Cin, H, W, Cout, Kh, Kw, stride, pad, output_padding,
                                 dilation, groups, dtype, epilogue, &s);
    if (rc) return rc;
    const int path = choose_tpath(s);
    if (path < 0) return path;
    log_path("conv2d_transpose_fwd_nhwc_packed", s, path);
    return run_tnhwc(path, s, x, w_packed, bias, y, stream);
}

int conv2d_transpose_fwd(const void* x, const void* w, const float* bias, void* y, int N, int Cin, int H, int W,
                         int Cout, int Kh, int Kw, int stride, int pad, int output_padding, int dilation,
                         int groups, int dtype, int epilogue, hipStream_t stream) {
    Shape s;
    int rc = validate_transposed(x, w, bias, y, N, Cin, H, W, Cout, Kh, Kw, stride, pad, output_padding,
                                 dilation, groups, dtype, epilogue, &s);
    if (rc) return rc;
    const int path = choose_tpath(s);
    if (path < 0) return path;
    log_path("conv2d_transpose_fwd", s, path);
    if (path == CONV2D_PATH_DIRECT) {
        // the direct loop reads the pages' layouts as they are
        const hipError_t e = launch_tconv_direct(s, x, NCHW, w, W_IOHW, bias, y, NCHW, stream);
        return e == hipSuccess ? CONV2D_OK : hip_fail(e, "transposed direct launch");
    }
    const size_t eb = elem_bytes(dtype);
    const size_t wb = round_up(conv2d_packed_weight_bytes(Cout, Cin, Kh, Kw, groups, dtype), 256);
    const size_t xb = round_up((size_t)N * Cin * H * W * eb, 256);
    const size_t yb = round_up((size_t)N * Cout * s.Ho * s.Wo * eb, 256);
    void* scratch = nullptr;
    rc = get_scratch(wb + xb + yb, stream, &scratch);
    if (rc) return rc;
    char* base = static_cast<char*>(scratch);
    void* wp = base;
    void* xn = base + wb;
    void* yn = base + wb + xb;
    rc = conv2d_transpose_pack_weights(w, wp, Cin, Cout, Kh, Kw, groups, dtype, stream);
    if (rc) return rc;
    rc = conv2d_nchw_to_nhwc(x, xn, N, Cin, H, W, dtype, stream);
    if (rc) return rc;
    rc = run_tnhwc(path, s, xn, wp, bias, yn, stream);
    if (rc) return rc;
    return conv2d_nhwc_to_nchw(yn, y, N, Cout, s.Ho, s.Wo, dtype, stream);
}

void conv2d_release_scratch(void) {
    std::lock_guard<std::mutex> lk(g_scratch_mu);
    int cur = 0;
    if (hipGetDevice(&cur) != hipSuccess) return;
    for (auto& b : g_scratch) {
        if (b.ptr && hipSetDevice(b.dev) == hipSuccess) {
            (void)hipDeviceSynchronize();
            (void)hipFree(b.ptr);
        }
    }
    g_scratch.clear();
    (void)hipSetDevice(cur);
}

const char* conv2d_strerror(int code) {
    switch (code) {
    case CONV2D_OK: return "ok";
    case CONV2D_ERR_ARG: return "invalid size, stride, padding or dilation";
    case CONV2D_ERR_GROUPS: return "channels not divisible by groups";
    case CONV2D_ERR_EMPTY_OUTPUT: return "output would be empty";
    case CONV2D_ERR_UNSUPPORTED: return "unsupported by this path or build";
    case CONV2D_ERR_HIP: return "HIP runtime error";
    case CONV2D_ERR_NULL: return "required pointer is NULL";
    case CONV2D_ERR_DTYPE: return "unknown dtype";
    case CONV2D_ERR_EPILOGUE: return "unknown epilogue flags";
    case CONV2D_ERR_ALIGN: return "pointer not 16-byte aligned";
    default: return "unknown error code";
    }
}

const char* conv2d_last_error(void) { return g_last_error; }

}  // extern "C"
