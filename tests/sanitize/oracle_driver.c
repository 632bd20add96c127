/* Memory and undefined-behaviour check of the fp64 oracle (test
 * infrastructure): built with AddressSanitizer and UBSan on the host and run
 * over a sweep of small shapes, degenerate ones included (filters larger than
 * the input, strides beyond the filter, padding beyond the filter, one-pixel
 * images, empty outputs, out-of-range point indices).  Every buffer is
 * allocated at exactly the size the oracle's contract names, so a read or
 * write past it is reported.  Exits non-zero on any unexpected return code. */
#include <stdio.h>
#include <stdlib.h>

int oracle_conv2d_f64(const double*, const double*, const double*, int, double*, double*, long, long, long, long,
                      long, long, long, long, long, long, long);
int oracle_conv2d_points_f64(const double*, const double*, const double*, int, const long*, long, double*, double*,
                             long, long, long, long, long, long, long, long, long, long, long);
int oracle_im2col_f64(const double*, double*, long, long, long, long, long, long, long, long, long);
long oracle_out_dim(long, long, long, long, long);
long oracle_transpose_out_dim(long, long, long, long, long, long);
int oracle_conv_transpose2d_f64(const double*, const double*, const double*, int, double*, double*, long, long, long,
                                long, long, long, long, long, long, long, long, long);
int oracle_conv_transpose2d_points_f64(const double*, const double*, const double*, int, const long*, long, double*,
                                       double*, long, long, long, long, long, long, long, long, long, long, long, long);

static double* filled(long n, unsigned* seed) {
    double* p = (double*)malloc((size_t)(n > 0 ? n : 1) * sizeof(double));
    for (long i = 0; i < n; ++i) {
        *seed = *seed * 1103515245u + 12345u;
        p[i] = (double)((*seed >> 16) % 7) - 3.0;
    }
    return p;
}

int main(void) {
    unsigned seed = 1;
    long runs = 0, empty = 0;
    const long Ns[] = {1, 2}, Cs[] = {1, 4}, Hs[] = {1, 3, 6}, Ks[] = {1, 2, 3, 5}, Ss[] = {1, 2, 3},
               Ps[] = {0, 1, 3}, Ds[] = {1, 2}, Gs[] = {1, 2};
    for (int a = 0; a < 2; ++a) for (int b = 0; b < 2; ++b) for (int c = 0; c < 3; ++c) for (int d = 0; d < 4; ++d)
    for (int e = 0; e < 3; ++e) for (int f = 0; f < 3; ++f) for (int g = 0; g < 2; ++g) for (int h = 0; h < 2; ++h) {
        const long N = Ns[a], C = Cs[b], H = Hs[c], W = Hs[(c + 1) % 3], K = Ks[d], S = Ss[e], P = Ps[f], D = Ds[g],
                   G = Gs[h];
        if (C % G) continue;
        const long Cout = 2 * G;
        const long Ho = oracle_out_dim(H, K, S, P, D), Wo = oracle_out_dim(W, K, S, P, D);
        double* x = filled(N * C * H * W, &seed);
        double* w = filled(Cout * (C / G) * K * K, &seed);
        double* bias = filled(Cout, &seed);
        if (Ho < 1 || Wo < 1) {
            double dummy[1];
            if (oracle_conv2d_f64(x, w, bias, 1, dummy, dummy, N, C, H, W, Cout, K, K, S, P, D, G) != -3) {
                printf("empty output not rejected\n");
                return 1;
            }
            ++empty;
        } else {
            const long no = N * Cout * Ho * Wo;
            double* y = filled(no, &seed);
            double* s = filled(no, &seed);
            if (oracle_conv2d_f64(x, w, bias, (int)(runs & 1), y, s, N, C, H, W, Cout, K, K, S, P, D, G)) return 2;
            long idx[4] = {0, no - 1, no / 2, no};
            double yp[4], sp[4];
            if (oracle_conv2d_points_f64(x, w, bias, 1, idx, 3, yp, sp, N, C, H, W, Cout, K, K, S, P, D, G)) return 3;
            if (oracle_conv2d_points_f64(x, w, bias, 1, idx, 4, yp, sp, N, C, H, W, Cout, K, K, S, P, D, G) != -4)
                return 4;
            double* xcol = filled(C * K * K * N * Ho * Wo, &seed);
            if (oracle_im2col_f64(x, xcol, N, C, H, W, K, K, S, P, D)) return 5;
            free(xcol);
            free(y);
            free(s);
        }
        /* the transposed convolution: weight [C][Cout/G][K][K], output padding 0 and the largest allowed */
        for (long op = 0; op < (S > D ? S : D); op += (S > D ? S : D) - 1 > 0 ? (S > D ? S : D) - 1 : 1) {
            const long To = oracle_transpose_out_dim(H, K, S, P, D, op), Tw = oracle_transpose_out_dim(W, K, S, P, D, op);
            if (To < 1 || Tw < 1) continue;
            const long nt = N * Cout * To * Tw;
            double* yt = filled(nt, &seed);
            double* st = filled(nt, &seed);
            if (oracle_conv_transpose2d_f64(x, w, bias, 1, yt, st, N, C, H, W, Cout, K, K, S, P, op, D, G)) return 6;
            long ti[3] = {0, nt - 1, nt / 3};
            double ty[3], ts[3];
            if (oracle_conv_transpose2d_points_f64(x, w, bias, 0, ti, 3, ty, ts, N, C, H, W, Cout, K, K, S, P, op, D, G))
                return 7;
            free(yt);
            free(st);
        }
        free(x);
        free(w);
        free(bias);
        ++runs;
    }
    printf("oracle sanitize ok: %ld shapes, %ld empty outputs rejected\n", runs, empty);
    return 0;
}
