// Memory and undefined-behaviour check of libconv2d.so's host-side logic:
// argument validation, output sizes and kernel-path choice (the tile plans of
// every kernel's support check), built with AddressSanitizer and UBSan on
// the host and run over a sweep of valid, invalid and extreme arguments
// (sizes up to INT_MAX, negative values, products that overflow 32 bits).
// Only host-only entry points are called: nothing touches a GPU.
#include <climits>
#include <cstdio>

#include "conv2d.h"

// a + b, clamped to INT_MAX (the driver's own arithmetic must not overflow)
static int sat(long long v) { return v > INT_MAX ? INT_MAX : (int)v; }

int main() {
    static const char d[16] = {};
    const float* b = reinterpret_cast<const float*>(d);
    long calls = 0, ok = 0;
    const int Ns[] = {-1, 0, 1, 2, INT_MAX};
    const int Cs[] = {-8, 0, 3, 8, 64, 144, 260, INT_MAX};
    const int Hs[] = {-1, 0, 1, 5, 56, 4100, INT_MAX / 2, INT_MAX};
    const int Ks[] = {-1, 0, 1, 2, 3, 5, 4097, INT_MAX};
    const int Ss[] = {0, 1, 2, INT_MAX};
    const int Ps[] = {-1, 0, 1, INT_MAX / 2};
    const int Ds[] = {0, 1, 2};
    for (int N : Ns) for (int C : Cs) for (int H : Hs) for (int K : Ks)
    for (int S : Ss) for (int P : Ps) for (int D : Ds) for (int G : {1, 2})
    for (int dt : {CONV2D_F32, CONV2D_BF16}) {
        const int r1 = conv2d_check_args(d, d, b, d, N, C, H, sat(H + 1LL), sat(2LL * C), K, K, S, P, D, G, dt, 3);
        const int r2 = conv2d_select_path(N, C, H, H, C, K, K, S, P, D, G, dt);
        const int r3 = conv2d_select_path(N, C, H, sat(2LL * H + 1), C, K, sat(K + 1LL), S, P, D, C > 0 ? C : 1, dt);
        const int r4 = conv2d_transpose_select_path(N, C, H, H, C, K, K, S, P, 0, D, G, dt);
        const int r5 = conv2d_transpose_check_args(d, d, b, d, N, C, H, H, C, K, K, S, P, S > 1 ? S - 1 : 0, D, G,
                                                   dt, 1);
        const int r6 = conv2d_out_dim(H, K, S, P, D);
        const int r7 = conv2d_transpose_out_dim(H, K, S, P, D, 0);
        const size_t r8 = conv2d_winograd_weight_bytes(C, sat(2LL * C), dt);
        const size_t r9 = conv2d_packed_weight_bytes(sat(2LL * C), C, K, K, G, dt);
        ok += (r8 > 0) + (r9 > 0);
        ok += (r1 == 0) + (r2 > 0) + (r3 > 0) + (r4 > 0) + (r5 == 0) + (r6 > 0) + (r7 > 0);
        ++calls;
    }
    // unknown dtype and epilogue bits
    ok += conv2d_check_args(d, d, b, d, 1, 8, 8, 8, 8, 3, 3, 1, 1, 1, 1, 7, 0) == CONV2D_ERR_DTYPE;
    ok += conv2d_check_args(d, d, b, d, 1, 8, 8, 8, 8, 3, 3, 1, 1, 1, 1, CONV2D_BF16, 8) == CONV2D_ERR_EPILOGUE;
    // every forced path, on one shape per family
    for (int path = 0; path <= CONV2D_PATH_IGEMM_HALO; ++path) {
        conv2d_set_path_override(path);
        ok += conv2d_select_path(2, 64, 56, 56, 128, 3, 3, 1, 1, 1, 1, CONV2D_BF16) > 0;
        ok += conv2d_select_path(2, 144, 56, 56, 144, 3, 3, 1, 1, 1, 144, CONV2D_BF16) > 0;
        ok += conv2d_select_path(2, 256, 56, 56, 64, 1, 1, 1, 0, 1, 1, CONV2D_BF16) > 0;
        ok += conv2d_transpose_select_path(2, 256, 28, 28, 128, 4, 4, 2, 1, 0, 1, 1, CONV2D_BF16) > 0;
    }
    conv2d_set_path_override(CONV2D_PATH_AUTO);
    std::printf("dispatch sanitize ok: %ld argument sets, %ld accepted results\n", calls, ok);
    return ok > 0 ? 0 : 1;
}
