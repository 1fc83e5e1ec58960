/*
 * CPU oracle for im2win convolution.
 *
 * TEST INFRASTRUCTURE ONLY. Nothing here is part of the product: only the
 * test suite, the smoke check and the CPU-baseline leg of the benchmark load
 * this library. It shares no code with the HIP library.
 *
 * Plain nested loops, written to be checked by eye against the pages:
 *
 *  - "Enabling Memory-efficient Im2win Convolution with Multi-precision
 *    Support on GPU CUDA and Tensor Cores" (Abstract; Fig. 1; Table I):
 *    NCHW input Ci x Hi x Wi, filters Co x Ci x Hf x Wf, row stride sh and
 *    column stride sw (the table writes s_h(s_w); every row it lists has the
 *    two equal), output Co x Ho x Wo; fp32 and fp16 inputs.
 *  - "Im2win: Memory Efficient Convolution On SIMD Architectures" (Abstract):
 *    the im2win transform takes one row of dot-product windows and flattens
 *    the distinct input elements those windows cover into one row of the
 *    transformed tensor.
 *
 * Readings taken where the pages leave a step open (each is stated again at
 * the function that uses it):
 *  - convolution is cross-correlation (no filter flip), no padding, no
 *    dilation, no bias;
 *  - Ho = floor((Hi - Hf) / sh) + 1 and Wo = floor((Wi - Wf) / sw) + 1
 *    (Table I, cv4: 224, 7, stride 2 gives 109);
 *  - an im2win row for (image n, channel ci, output row ho) holds the Hf
 *    input rows ho*sh .. ho*sh+Hf-1 over all Wi columns, column by column:
 *    element w*Hf + kh is x[n][ci][ho*sh+kh][w]. Then the window of output
 *    column wo is the single contiguous run starting at wo*sw*Hf of length
 *    Wf*Hf.
 *
 * Floating point: products of the rounded inputs are accumulated in double
 * (fp64) in one fixed order -- ci outermost, then kh, then kw -- with
 * -ffp-contract=off so no fused multiply-add changes that order. The *_f32acc
 * twins use a float accumulator in the same order.
 *
 * Pinned by tests/test_oracle.py: Table I output extents, the Fig. 1 sizes,
 * library special cases (scipy correlate2d, torch conv2d in fp64), closed
 * forms (delta filter, constant and ramp inputs) and the window-contiguity
 * property of the transform.
 */
#include <stddef.h>
#include <stdint.h>
#include <string.h>
#include <math.h>

/* Output extent along one axis; 0 when the filter does not fit. */
int oracle_out_extent(int in, int f, int s)
{
    if (in < 1 || f < 1 || s < 1 || f > in)
        return 0;
    return (in - f) / s + 1;
}

/* Elements of the im2win tensor: one row of Wi*Hf per (n, ci, ho). */
int64_t oracle_im2win_elems(int N, int Ci, int Hi, int Wi, int Hf, int Wf, int sh, int sw)
{
    int Ho = oracle_out_extent(Hi, Hf, sh);
    int Wo = oracle_out_extent(Wi, Wf, sw);
    if (N < 1 || Ci < 1 || Ho == 0 || Wo == 0)
        return 0;
    return (int64_t)N * Ci * Ho * ((int64_t)Wi * Hf);
}

/* Elements of the im2col matrix: one column of Ci*Hf*Wf per output pixel. */
int64_t oracle_im2col_elems(int N, int Ci, int Hi, int Wi, int Hf, int Wf, int sh, int sw)
{
    int Ho = oracle_out_extent(Hi, Hf, sh);
    int Wo = oracle_out_extent(Wi, Wf, sw);
    if (N < 1 || Ci < 1 || Ho == 0 || Wo == 0)
        return 0;
    return (int64_t)N * Ci * Hf * Wf * Ho * (int64_t)Wo;
}

/*
 * The im2win transform as a bit copy of elem_bytes-wide elements:
 *   ws[n][ci][ho][w*Hf + kh] = x[n][ci][ho*sh + kh][w]
 * for every w < Wi and kh < Hf. Every column is kept, even columns no window
 * reads; rows shared by overlapping windows (sh < Hf) appear in each im2win
 * row that needs them. The column stride sw does not enter the transform
 * (it only places the windows inside a row).
 */
void oracle_im2win_pack(const void *x, void *ws, int N, int Ci, int Hi, int Wi,
                        int Hf, int Wf, int sh, int sw, int elem_bytes)
{
    const unsigned char *src = (const unsigned char *)x;
    unsigned char *dst = (unsigned char *)ws;
    int Ho = oracle_out_extent(Hi, Hf, sh);
    if (Ho == 0 || oracle_out_extent(Wi, Wf, sw) == 0)
        return;
    for (int n = 0; n < N; ++n)
        for (int ci = 0; ci < Ci; ++ci)
            for (int ho = 0; ho < Ho; ++ho)
                for (int w = 0; w < Wi; ++w)
                    for (int kh = 0; kh < Hf; ++kh) {
                        int64_t plane = (int64_t)n * Ci + ci;
                        int64_t out = ((plane * Ho + ho) * Wi + w) * Hf + kh;
                        int64_t in = (plane * Hi + (int64_t)ho * sh + kh) * Wi + w;
                        memcpy(dst + out * elem_bytes, src + in * elem_bytes,
                               (size_t)elem_bytes);
                    }
}

/*
 * The im2win transform for NHWC tensors (x is N x Hi x Wi x Ci): the same
 * flattening of a row of windows, channels innermost:
 *   ws[n][ho][w][kh][c] = x[n][ho*sh + kh][w][c]
 * so the window of output (ho, wo) is the single contiguous run of
 * Wf*Hf*Ci elements starting at wo*sw*Hf*Ci in row (n, ho); its element
 * (kw*Hf + kh)*Ci + c is x[n][ho*sh + kh][wo*sw + kw][c]. A bit copy.
 */
void oracle_im2win_pack_nhwc(const void *x, void *ws, int N, int Ci, int Hi, int Wi, int Hf,
                             int Wf, int sh, int sw, int elem_bytes)
{
    const unsigned char *src = (const unsigned char *)x;
    unsigned char *dst = (unsigned char *)ws;
    int Ho = oracle_out_extent(Hi, Hf, sh);
    if (Ho == 0 || oracle_out_extent(Wi, Wf, sw) == 0)
        return;
    for (int n = 0; n < N; ++n)
        for (int ho = 0; ho < Ho; ++ho)
            for (int w = 0; w < Wi; ++w)
                for (int kh = 0; kh < Hf; ++kh)
                    for (int c = 0; c < Ci; ++c) {
                        int64_t out = ((((int64_t)n * Ho + ho) * Wi + w) * Hf + kh) * Ci + c;
                        int64_t in = (((int64_t)n * Hi + (int64_t)ho * sh + kh) * Wi + w) * Ci + c;
                        memcpy(dst + out * elem_bytes, src + in * elem_bytes, (size_t)elem_bytes);
                    }
}

/*
 * The im2col transform (the unfolding the GEMM-based baseline of the GPU page,
 * Fig. 1 right, multiplies): one row per output pixel q = (n*Ho + ho)*Wo + wo
 * holding its receptive field in (ci, kh, kw) order, K = Ci*Hf*Wf elements,
 * then zeros up to the row pitch KP >= K:
 *   col[q][(ci*Hf + kh)*Wf + kw] = x[n][ci][ho*sh + kh][wo*sw + kw]
 * A bit copy of elem_bytes-wide elements.
 */
void oracle_im2col_pack(const void *x, void *col, int N, int Ci, int Hi, int Wi, int Hf, int Wf,
                        int sh, int sw, int KP, int elem_bytes)
{
    const unsigned char *src = (const unsigned char *)x;
    unsigned char *dst = (unsigned char *)col;
    int Ho = oracle_out_extent(Hi, Hf, sh);
    int Wo = oracle_out_extent(Wi, Wf, sw);
    int64_t K = (int64_t)Ci * Hf * Wf;
    if (Ho == 0 || Wo == 0 || KP < K)
        return;
    for (int n = 0; n < N; ++n)
        for (int ho = 0; ho < Ho; ++ho)
            for (int wo = 0; wo < Wo; ++wo) {
                int64_t q = ((int64_t)n * Ho + ho) * Wo + wo;
                unsigned char *row = dst + q * KP * elem_bytes;
                memset(row, 0, (size_t)KP * elem_bytes);
                for (int ci = 0; ci < Ci; ++ci)
                    for (int kh = 0; kh < Hf; ++kh)
                        for (int kw = 0; kw < Wf; ++kw) {
                            int64_t k = ((int64_t)ci * Hf + kh) * Wf + kw;
                            int64_t in = (((int64_t)n * Ci + ci) * Hi + (int64_t)ho * sh + kh) * Wi +
                                         (int64_t)wo * sw + kw;
                            memcpy(row + k * elem_bytes, src + in * elem_bytes, (size_t)elem_bytes);
                        }
            }
}

/* Index helpers for the NCHW tensors. */
static inline int64_t xi(int n, int ci, int h, int w, int Ci, int Hi, int Wi)
{
    return (((int64_t)n * Ci + ci) * Hi + h) * Wi + w;
}
static inline int64_t wi(int co, int ci, int kh, int kw, int Ci, int Hf, int Wf)
{
    return (((int64_t)co * Ci + ci) * Hf + kh) * Wf + kw;
}

/*
 * One output of the direct convolution (cross-correlation), fp64:
 *   y[n][co][ho][wo] = sum_ci sum_kh sum_kw x[n][ci][ho*sh+kh][wo*sw+kw] * w[co][ci][kh][kw]
 * If absdot is non-NULL it also receives sum |x * w| over the same terms.
 */
static double direct_point_f64(const float *x, const float *w, int n, int co, int ho,
                               int wo, int Ci, int Hi, int Wi, int Hf, int Wf, int sh, int sw,
                               double *absdot)
{
    double acc = 0.0, aacc = 0.0;
    for (int ci = 0; ci < Ci; ++ci)
        for (int kh = 0; kh < Hf; ++kh)
            for (int kw = 0; kw < Wf; ++kw) {
                double p = (double)x[xi(n, ci, ho * sh + kh, wo * sw + kw, Ci, Hi, Wi)] *
                           (double)w[wi(co, ci, kh, kw, Ci, Hf, Wf)];
                acc += p;
                aacc += fabs(p);
            }
    if (absdot)
        *absdot = aacc;
    return acc;
}

/* Direct convolution over the whole output, fp64 accumulation. */
void oracle_conv_direct_f64(const float *x, const float *w, double *y, double *absdot,
                            int N, int Ci, int Hi, int Wi, int Co, int Hf, int Wf, int sh, int sw)
{
    int Ho = oracle_out_extent(Hi, Hf, sh);
    int Wo = oracle_out_extent(Wi, Wf, sw);
    if (Ho == 0 || Wo == 0)
        return;
#pragma omp parallel for collapse(2) schedule(dynamic)
    for (int n = 0; n < N; ++n)
        for (int co = 0; co < Co; ++co)
            for (int ho = 0; ho < Ho; ++ho)
                for (int wo = 0; wo < Wo; ++wo) {
                    int64_t o = (((int64_t)n * Co + co) * Ho + ho) * Wo + wo;
                    double a;
                    y[o] = direct_point_f64(x, w, n, co, ho, wo, Ci, Hi, Wi, Hf, Wf, sh, sw, &a);
                    if (absdot)
                        absdot[o] = a;
                }
}

/* Direct convolution with a float accumulator, same order (ci, kh, kw). */
void oracle_conv_direct_f32acc(const float *x, const float *w, float *y, int N, int Ci,
                               int Hi, int Wi, int Co, int Hf, int Wf, int sh, int sw)
{
    int Ho = oracle_out_extent(Hi, Hf, sh);
    int Wo = oracle_out_extent(Wi, Wf, sw);
    if (Ho == 0 || Wo == 0)
        return;
#pragma omp parallel for collapse(2) schedule(dynamic)
    for (int n = 0; n < N; ++n)
        for (int co = 0; co < Co; ++co)
            for (int ho = 0; ho < Ho; ++ho)
                for (int wo = 0; wo < Wo; ++wo) {
                    float acc = 0.0f;
                    for (int ci = 0; ci < Ci; ++ci)
                        for (int kh = 0; kh < Hf; ++kh)
                            for (int kw = 0; kw < Wf; ++kw)
                                acc += x[xi(n, ci, ho * sh + kh, wo * sw + kw, Ci, Hi, Wi)] *
                                       w[wi(co, ci, kh, kw, Ci, Hf, Wf)];
                    y[(((int64_t)n * Co + co) * Ho + ho) * Wo + wo] = acc;
                }
}

/*
 * im2win convolution on a packed im2win tensor, fp64 accumulation. The window
 * of (ho, wo) is the contiguous run ws[n][ci][ho][wo*sw*Hf ...] of Wf*Hf
 * elements; element kw*Hf + kh of that run multiplies w[co][ci][kh][kw].
 * Terms are taken ci, then kh, then kw -- the direct order -- so the result
 * is bit-identical to oracle_conv_direct_f64.
 */
void oracle_conv_im2win_f64(const float *ws, const float *w, double *y, int N, int Ci,
                            int Hi, int Wi, int Co, int Hf, int Wf, int sh, int sw)
{
    int Ho = oracle_out_extent(Hi, Hf, sh);
    int Wo = oracle_out_extent(Wi, Wf, sw);
    if (Ho == 0 || Wo == 0)
        return;
    int64_t row = (int64_t)Wi * Hf;
#pragma omp parallel for collapse(2) schedule(dynamic)
    for (int n = 0; n < N; ++n)
        for (int co = 0; co < Co; ++co)
            for (int ho = 0; ho < Ho; ++ho)
                for (int wo = 0; wo < Wo; ++wo) {
                    double acc = 0.0;
                    for (int ci = 0; ci < Ci; ++ci) {
                        const float *win = ws + (((int64_t)n * Ci + ci) * Ho + ho) * row +
                                           (int64_t)wo * sw * Hf;
                        for (int kh = 0; kh < Hf; ++kh)
                            for (int kw = 0; kw < Wf; ++kw)
                                acc += (double)win[kw * Hf + kh] *
                                       (double)w[wi(co, ci, kh, kw, Ci, Hf, Wf)];
                    }
                    y[(((int64_t)n * Co + co) * Ho + ho) * Wo + wo] = acc;
                }
}

/* im2win convolution with a float accumulator, same order as the f64 one. */
void oracle_conv_im2win_f32acc(const float *ws, const float *w, float *y, int N, int Ci,
                               int Hi, int Wi, int Co, int Hf, int Wf, int sh, int sw)
{
    int Ho = oracle_out_extent(Hi, Hf, sh);
    int Wo = oracle_out_extent(Wi, Wf, sw);
    if (Ho == 0 || Wo == 0)
        return;
    int64_t row = (int64_t)Wi * Hf;
#pragma omp parallel for collapse(2) schedule(dynamic)
    for (int n = 0; n < N; ++n)
        for (int co = 0; co < Co; ++co)
            for (int ho = 0; ho < Ho; ++ho)
                for (int wo = 0; wo < Wo; ++wo) {
                    float acc = 0.0f;
                    for (int ci = 0; ci < Ci; ++ci) {
                        const float *win = ws + (((int64_t)n * Ci + ci) * Ho + ho) * row +
                                           (int64_t)wo * sw * Hf;
                        for (int kh = 0; kh < Hf; ++kh)
                            for (int kw = 0; kw < Wf; ++kw)
                                acc += win[kw * Hf + kh] * w[wi(co, ci, kh, kw, Ci, Hf, Wf)];
                    }
                    y[(((int64_t)n * Co + co) * Ho + ho) * Wo + wo] = acc;
                }
}

/*
 * Direct convolution at selected outputs only (flat NCHW output indices), for
 * checking full-size results one element at a time. Same order and precision
 * as oracle_conv_direct_f64, so each value is bit-identical to the full run.
 */
void oracle_conv_points_f64(const float *x, const float *w, const int64_t *idx,
                            int64_t npts, double *y, double *absdot, int N, int Ci,
                            int Hi, int Wi, int Co, int Hf, int Wf, int sh, int sw)
{
    int Ho = oracle_out_extent(Hi, Hf, sh);
    int Wo = oracle_out_extent(Wi, Wf, sw);
    if (Ho == 0 || Wo == 0)
        return;
    (void)N;
#pragma omp parallel for schedule(dynamic, 64)
    for (int64_t i = 0; i < npts; ++i) {
        int64_t o = idx[i];
        int wo = (int)(o % Wo);
        int ho = (int)((o / Wo) % Ho);
        int co = (int)((o / ((int64_t)Wo * Ho)) % Co);
        int n = (int)(o / ((int64_t)Wo * Ho * Co));
        double a;
        y[i] = direct_point_f64(x, w, n, co, ho, wo, Ci, Hi, Wi, Hf, Wf, sh, sw, &a);
        if (absdot)
            absdot[i] = a;
    }
}

/* Number of OpenMP threads the parallel loops above use (1 without OpenMP). */
int oracle_num_threads(void)
{
#ifdef _OPENMP
    extern int omp_get_max_threads(void);
    return omp_get_max_threads();
#else
    return 1;
#endif
}
