/*
 * conv2d_oracle.c -- plain, slow, fp64 CPU reference for the 2D convolution
 * forward pass.  TEST INFRASTRUCTURE ONLY: only the test suite, the smoke
 * check and the benchmark's CPU-baseline leg may load it.  It shares no code,
 * header or table with the GPU library.
 *
 * What it computes (page "How a GPU executes NN convolution", lincklin.cn,
 * sections 1-2): every output element is the dot product of one input window
 * with one filter,
 *
 *     Y[n,co,ho,wo] = sum_{ci,kh,kw} X[n,ci,hi,wi] * W[co,ci,kh,kw]
 *     hi = ho*S + kh*D - P,   wi = wo*S + kw*D - P
 *
 * extended with:
 *   - dilation D: the taps of the filter sit D pixels apart
 *     (same page, section 28; "lpnh.cn/news/2674933" section 4.2: skip D-1
 *     pixels between taps);
 *   - groups G: input and output channels split into G contiguous blocks and
 *     each block is an independent convolution ("lpnh.cn" sections 2.2, 4.3);
 *     the weight is [Cout][Cin/G][Kh][Kw];
 *   - zero padding by address predicate: a tap whose (hi, wi) falls outside
 *     the input contributes nothing (lincklin.cn section 26);
 *   - epilogue: add bias after the full sum, then ReLU = max(v, 0)
 *     (lincklin.cn section 31; lpnh.cn section 2.1: sum the products, then add
 *     the bias).
 *
 * Loop order is the seven-deep nest n, co, ho, wo, ci, kh, kw that the
 * lincklin.cn page gives in section 34.  Accumulation is in fp64; products of
 * two fp32 (or bf16) values are exact in fp64.  Besides the value, it returns
 * S = sum |x*w| over the valid taps, the scale of the rounding error of any
 * reordered fp32 sum of the same products (used for tolerances).
 *
 * Layouts: X is NCHW, W is [Cout][Cin/G][Kh][Kw], Y and S are NCHW, all
 * dense, fp64.  Output size Ho = floor((H + 2P - D(Kh-1) - 1)/S) + 1
 * (lpnh.cn section 6.2, whose printed formula lost its '+' and '/' signs; the
 * reading here is the one that gives its section 2.1 example 224 -> 112 at
 * stride 2, pad 1, 3x3).
 *
 * Also exported, for the oracle's own self-tests only: an explicit im2col
 * (every window flattened into one column, rows ordered (ci, kh, kw),
 * columns ordered (n, ho, wo); lincklin.cn sections 7-8, lpnh.cn section 3.1).
 *
 * Error behaviour: functions return 0 on success and a negative value for
 * inconsistent shapes; they never allocate.
 */
#include <stddef.h>
#include <math.h>
#include <omp.h>

/* Threads the OpenMP loops below will use (for reporting timings). */
int oracle_num_threads(void) { return omp_get_max_threads(); }

/* floor division for possibly negative numerators, positive divisor */
static long floordiv(long a, long b) {
    long q = a / b;
    if ((a % b != 0) && ((a < 0) != (b < 0))) q -= 1;
    return q;
}

long oracle_out_dim(long in, long k, long stride, long pad, long dil) {
    if (stride < 1 || dil < 1 || k < 1 || in < 1 || pad < 0) return -1;
    return floordiv(in + 2 * pad - dil * (k - 1) - 1, stride) + 1;
}

static int check_shape(long N, long Cin, long H, long W, long Cout, long Kh, long Kw,
                       long stride, long pad, long dil, long groups, long* Ho, long* Wo) {
    if (N < 1 || Cin < 1 || H < 1 || W < 1 || Cout < 1 || Kh < 1 || Kw < 1) return -1;
    if (stride < 1 || dil < 1 || pad < 0 || groups < 1) return -1;
    if (Cin % groups != 0 || Cout % groups != 0) return -2;
    *Ho = oracle_out_dim(H, Kh, stride, pad, dil);
    *Wo = oracle_out_dim(W, Kw, stride, pad, dil);
    if (*Ho < 1 || *Wo < 1) return -3;
    return 0;
}

/* One output element: the dot product of one window with one filter. */
static void one_output(const double* x, const double* w, const double* bias, int relu,
                       long n, long co, long ho, long wo,
                       long Cin, long H, long W, long Cout, long Kh, long Kw,
                       long stride, long pad, long dil, long groups,
                       double* out_y, double* out_s) {
    const long cin_g = Cin / groups;
    const long cout_g = Cout / groups;
    const long g = co / cout_g;               /* group that owns this output channel */
    double acc = 0.0, s = 0.0;
    for (long ci = 0; ci < cin_g; ++ci) {
        const long c = g * cin_g + ci;        /* input channel in the whole tensor */
        for (long kh = 0; kh < Kh; ++kh) {
            const long hi = ho * stride + kh * dil - pad;
            for (long kw = 0; kw < Kw; ++kw) {
                const long wi = wo * stride + kw * dil - pad;
                if (hi >= 0 && hi < H && wi >= 0 && wi < W) {
                    const double xv = x[((n * Cin + c) * H + hi) * W + wi];
                    const double wv = w[((co * cin_g + ci) * Kh + kh) * Kw + kw];
                    const double p = xv * wv;
                    acc += p;
                    s += fabs(p);
                }
            }
        }
    }
    double v = acc + (bias ? bias[co] : 0.0);
    if (relu && v < 0.0) v = 0.0;
    *out_y = v;
    if (out_s) *out_s = s;
}

/* Full convolution: y (and s, if non-NULL) receive N*Cout*Ho*Wo values. */
int oracle_conv2d_f64(const double* x, const double* w, const double* bias, int relu,
                      double* y, double* s,
                      long N, long Cin, long H, long W, long Cout, long Kh, long Kw,
                      long stride, long pad, long dil, long groups) {
    long Ho, Wo;
    int rc = check_shape(N, Cin, H, W, Cout, Kh, Kw, stride, pad, dil, groups, &Ho, &Wo);
    if (rc) return rc;
#pragma omp parallel for collapse(2) schedule(dynamic)
    for (long n = 0; n < N; ++n)
        for (long co = 0; co < Cout; ++co)
            for (long ho = 0; ho < Ho; ++ho)
                for (long wo = 0; wo < Wo; ++wo) {
                    const long o = ((n * Cout + co) * Ho + ho) * Wo + wo;
                    one_output(x, w, bias, relu, n, co, ho, wo, Cin, H, W, Cout, Kh, Kw,
                               stride, pad, dil, groups, &y[o], s ? &s[o] : NULL);
                }
    return 0;
}

/* Selected outputs only: idx[i] is a flat NCHW output index. */
int oracle_conv2d_points_f64(const double* x, const double* w, const double* bias, int relu,
                             const long* idx, long count, double* y, double* s,
                             long N, long Cin, long H, long W, long Cout, long Kh, long Kw,
                             long stride, long pad, long dil, long groups) {
    long Ho, Wo;
    int rc = check_shape(N, Cin, H, W, Cout, Kh, Kw, stride, pad, dil, groups, &Ho, &Wo);
    if (rc) return rc;
    const long total = N * Cout * Ho * Wo;
    for (long i = 0; i < count; ++i)
        if (idx[i] < 0 || idx[i] >= total) return -4;
#pragma omp parallel for schedule(dynamic, 16)
    for (long i = 0; i < count; ++i) {
        long o = idx[i];
        const long wo = o % Wo; o /= Wo;
        const long ho = o % Ho; o /= Ho;
        const long co = o % Cout; o /= Cout;
        const long n = o;
        one_output(x, w, bias, relu, n, co, ho, wo, Cin, H, W, Cout, Kh, Kw,
                   stride, pad, dil, groups, &y[i], s ? &s[i] : NULL);
    }
    return 0;
}

/* Explicit im2col of a whole NCHW tensor: xcol is [C*Kh*Kw][N*Ho*Wo],
 * rows (c, kh, kw), columns (n, ho, wo); out-of-range taps are 0. */
int oracle_im2col_f64(const double* x, double* xcol,
                      long N, long C, long H, long W, long Kh, long Kw,
                      long stride, long pad, long dil) {
    if (N < 1 || C < 1 || H < 1 || W < 1 || Kh < 1 || Kw < 1) return -1;
    const long Ho = oracle_out_dim(H, Kh, stride, pad, dil);
    const long Wo = oracle_out_dim(W, Kw, stride, pad, dil);
    if (Ho < 1 || Wo < 1) return -3;
    const long cols = N * Ho * Wo;
    for (long c = 0; c < C; ++c)
        for (long kh = 0; kh < Kh; ++kh)
            for (long kw = 0; kw < Kw; ++kw) {
                const long row = (c * Kh + kh) * Kw + kw;
                for (long n = 0; n < N; ++n)
                    for (long ho = 0; ho < Ho; ++ho)
                        for (long wo = 0; wo < Wo; ++wo) {
                            const long hi = ho * stride + kh * dil - pad;
                            const long wi = wo * stride + kw * dil - pad;
                            double v = 0.0;
                            if (hi >= 0 && hi < H && wi >= 0 && wi < W)
                                v = x[((n * C + c) * H + hi) * W + wi];
                            xcol[row * cols + (n * Ho + ho) * Wo + wo] = v;
                        }
            }
    return 0;
}

/*
 * Transposed convolution ("lpnh.cn/news/2674933" sections 2.3 and 4.2): the
 * matrix form is Y_col = W^T * X, i.e. every input pixel is multiplied by the
 * whole filter and the products are added into the output window it spans:
 *
 *     Y[n, co, ih*S - P + kh*D, iw*S - P + kw*D] += X[n, ci, ih, iw] * W[ci, co', kh, kw]
 *
 * for every input pixel (ih, iw), every tap (kh, kw) and, per group g, input
 * channel ci in g's block and output channel co = g*Cout/G + co'.  Sums that
 * land outside the output are dropped (the padding P trims the border).  The
 * weight is [Cin][Cout/G][Kh][Kw], the shapes of a standard convolution's
 * weight reversed (same section 4.2).  Output size: the smallest output that
 * a standard convolution with the same (K, S, P, D) maps back onto the input,
 * plus OP extra rows/columns at the far edge (0 <= OP < max(S, D)):
 *
 *     Ho = (H - 1)*S - 2P + D*(Kh - 1) + OP + 1
 *
 * Epilogue as above: bias after the full sum, then ReLU.  S = sum |x*w| of
 * the products each output received.
 */
long oracle_transpose_out_dim(long in, long k, long stride, long pad, long dil, long out_pad) {
    if (stride < 1 || dil < 1 || k < 1 || in < 1 || pad < 0 || out_pad < 0) return -1;
    if (out_pad >= stride && out_pad >= dil) return -1;
    return (in - 1) * stride - 2 * pad + dil * (k - 1) + out_pad + 1;
}

static int check_transpose(long N, long Cin, long H, long W, long Cout, long Kh, long Kw, long stride,
                           long pad, long out_pad, long dil, long groups, long* Ho, long* Wo) {
    if (N < 1 || Cin < 1 || H < 1 || W < 1 || Cout < 1 || Kh < 1 || Kw < 1) return -1;
    if (stride < 1 || dil < 1 || pad < 0 || out_pad < 0 || groups < 1) return -1;
    if (out_pad >= stride && out_pad >= dil) return -1;
    if (Cin % groups != 0 || Cout % groups != 0) return -2;
    *Ho = oracle_transpose_out_dim(H, Kh, stride, pad, dil, out_pad);
    *Wo = oracle_transpose_out_dim(W, Kw, stride, pad, dil, out_pad);
    if (*Ho < 1 || *Wo < 1) return -3;
    return 0;
}

/* The whole transposed convolution by scattering each product into its
 * output.  One (n, co) output plane per thread, so no two threads add into
 * the same element. */
int oracle_conv_transpose2d_f64(const double* x, const double* w, const double* bias, int relu,
                                double* y, double* s,
                                long N, long Cin, long H, long W, long Cout, long Kh, long Kw,
                                long stride, long pad, long out_pad, long dil, long groups) {
    long Ho, Wo;
    int rc = check_transpose(N, Cin, H, W, Cout, Kh, Kw, stride, pad, out_pad, dil, groups, &Ho, &Wo);
    if (rc) return rc;
    const long cin_g = Cin / groups, cout_g = Cout / groups;
#pragma omp parallel for collapse(2) schedule(dynamic)
    for (long n = 0; n < N; ++n)
        for (long co = 0; co < Cout; ++co) {
            double* yp = y + (n * Cout + co) * Ho * Wo;
            double* sp = s ? s + (n * Cout + co) * Ho * Wo : NULL;
            for (long o = 0; o < Ho * Wo; ++o) {
                yp[o] = 0.0;
                if (sp) sp[o] = 0.0;
            }
            const long g = co / cout_g, col = co % cout_g;
            for (long ci = 0; ci < cin_g; ++ci) {
                const long c = g * cin_g + ci;
                for (long ih = 0; ih < H; ++ih)
                    for (long iw = 0; iw < W; ++iw) {
                        const double xv = x[((n * Cin + c) * H + ih) * W + iw];
                        for (long kh = 0; kh < Kh; ++kh) {
                            const long oh = ih * stride - pad + kh * dil;
                            if (oh < 0 || oh >= Ho) continue;
                            for (long kw = 0; kw < Kw; ++kw) {
                                const long ow = iw * stride - pad + kw * dil;
                                if (ow < 0 || ow >= Wo) continue;
                                const double p = xv * w[((c * cout_g + col) * Kh + kh) * Kw + kw];
                                yp[oh * Wo + ow] += p;
                                if (sp) sp[oh * Wo + ow] += fabs(p);
                            }
                        }
                    }
            }
            for (long o = 0; o < Ho * Wo; ++o) {
                double v = yp[o] + (bias ? bias[co] : 0.0);
                if (relu && v < 0.0) v = 0.0;
                yp[o] = v;
            }
        }
    return 0;
}

/* Selected outputs of the transposed convolution, each gathered on its own:
 * output (oh, ow) receives tap (kh, kw) of input pixel (ih, iw) exactly when
 * oh + P - kh*D = ih*S with 0 <= ih < H (and the same along the width).
 * idx[i] is a flat NCHW output index. */
int oracle_conv_transpose2d_points_f64(const double* x, const double* w, const double* bias, int relu,
                                       const long* idx, long count, double* y, double* s,
                                       long N, long Cin, long H, long W, long Cout, long Kh, long Kw,
                                       long stride, long pad, long out_pad, long dil, long groups) {
    long Ho, Wo;
    int rc = check_transpose(N, Cin, H, W, Cout, Kh, Kw, stride, pad, out_pad, dil, groups, &Ho, &Wo);
    if (rc) return rc;
    const long total = N * Cout * Ho * Wo;
    for (long i = 0; i < count; ++i)
        if (idx[i] < 0 || idx[i] >= total) return -4;
    const long cin_g = Cin / groups, cout_g = Cout / groups;
#pragma omp parallel for schedule(dynamic, 16)
    for (long i = 0; i < count; ++i) {
        long o = idx[i];
        const long ow = o % Wo; o /= Wo;
        const long oh = o % Ho; o /= Ho;
        const long co = o % Cout; o /= Cout;
        const long n = o;
        const long g = co / cout_g, col = co % cout_g;
        double acc = 0.0, sa = 0.0;
        for (long ci = 0; ci < cin_g; ++ci) {
            const long c = g * cin_g + ci;
            for (long kh = 0; kh < Kh; ++kh) {
                const long th = oh + pad - kh * dil;
                if (th < 0 || th % stride != 0 || th / stride >= H) continue;
                for (long kw = 0; kw < Kw; ++kw) {
                    const long tw = ow + pad - kw * dil;
                    if (tw < 0 || tw % stride != 0 || tw / stride >= W) continue;
                    const double p = x[((n * Cin + c) * H + th / stride) * W + tw / stride] *
                                     w[((c * cout_g + col) * Kh + kh) * Kw + kw];
                    acc += p;
                    sa += fabs(p);
                }
            }
        }
        double v = acc + (bias ? bias[co] : 0.0);
        if (relu && v < 0.0) v = 0.0;
        y[i] = v;
        if (s) s[i] = sa;
    }
    return 0;
}
