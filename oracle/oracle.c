/*
 * Plain fp64 CPU convolution oracle (forward, backward-data and weight
 * gradient, NHWC / KRSC).
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may link, load or
 * call this file; only the test suite, the smoke check and the benchmark's
 * CPU-baseline leg use it.  It shares no code with the HIP library.
 *
 * What it computes is the definition of 2D convolution that the rocKE pull
 * requests describe, with nothing but nested loops and one fp64 accumulator:
 *
 *  - forward (cross-correlation, no filter flip): each output pixel is the sum
 *    over filter taps and the group's input channels of input times weight
 *    ("perf(rocke/conv): add the pointwise fast path dgrad was missing",
 *    Motivation; "feat(rocke): split-C and grouped LDS-halo direct conv fwd
 *    kernels", description);
 *  - backward-data (dgrad) is the adjoint of that forward map: an input pixel
 *    receives dY at every output pixel whose window covers it, times the
 *    unflipped weight of the covering tap ("feat(rocke): channel-packed and
 *    large-filter depthwise dgrad", Rotated-filter dgrad: the same quantity
 *    written as a correlation with the 180-degree-rotated filter);
 *  - the weight gradient (wgrad) is the derivative of the forward map with
 *    respect to the weight, the third pass the first page lists beside
 *    forward and dgrad (Motivation);
 *  - per-axis padding: pad_h pads top and bottom, pad_w left and right, and
 *    the output width follows pad_w (same page, Per-axis padding section and
 *    the review that counts 22 against 24 output columns);
 *  - groups own contiguous channel blocks of x and y, and the weight's last
 *    axis has C/groups entries (first page, follow-ups of the fast-path
 *    commit: "cpg as the W stride").
 *
 * Output size uses floor division:  Ho = (H + 2*pad_h - R) / stride + 1,
 * Wo = (W + 2*pad_w - S) / stride + 1.  Input pixels no output window covers
 * get dgrad value 0.  Dilation is 1.  Indices are 64-bit throughout (the
 * second page reports a reference that returned garbage past 2^31 bytes).
 *
 * Layouts: x, dx  [N][H][W][C];  y, dy  [N][Ho][Wo][K];  w  [K][R][S][C/groups].
 *
 * A deliberate-mistake build (-DORACLE_MUTATION=m, m > 0) exists only so the
 * test suite can show that its pins catch each planted mistake.
 */
#include <stdint.h>
#include <stddef.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#ifndef ORACLE_MUTATION
#define ORACLE_MUTATION 0
#endif

/* Shared argument checks; returns 0 when the descriptor is usable. */
static int oracle_dims(int64_t N, int64_t H, int64_t W, int64_t C, int64_t K,
                       int64_t R, int64_t S, int64_t stride, int64_t pad_h,
                       int64_t pad_w, int64_t groups, int64_t* Ho, int64_t* Wo)
{
    if (N < 1 || H < 1 || W < 1 || C < 1 || K < 1 || R < 1 || S < 1)
        return 1;
    if (stride < 1 || pad_h < 0 || pad_w < 0 || groups < 1)
        return 1;
    if (C % groups != 0 || K % groups != 0)
        return 1;
    int64_t hn = H + 2 * pad_h - R, wn = W + 2 * pad_w - S;
    if (hn < 0 || wn < 0)
        return 1;
    *Ho = hn / stride + 1;
    *Wo = wn / stride + 1;
    return 0;
}

int oracle_out_dims(int64_t N, int64_t H, int64_t W, int64_t C, int64_t K,
                    int64_t R, int64_t S, int64_t stride, int64_t pad_h,
                    int64_t pad_w, int64_t groups, int64_t* Ho, int64_t* Wo)
{
    return oracle_dims(N, H, W, C, K, R, S, stride, pad_h, pad_w, groups, Ho, Wo);
}

/* y[n,ho,wo,k] = sum_{r,t,j} x[n, ho*s - pad_h + r, wo*s - pad_w + t, g*Cg + j]
 *                            * w[k, r, t, j],   g = k / Kg,
 * with x taken as 0 outside the image. */
int oracle_conv_fwd_f64(int64_t N, int64_t H, int64_t W, int64_t C, int64_t K,
                        int64_t R, int64_t S, int64_t stride, int64_t pad_h,
                        int64_t pad_w, int64_t groups, const double* x,
                        const double* w, double* y)
{
    int64_t Ho, Wo;
    if (oracle_dims(N, H, W, C, K, R, S, stride, pad_h, pad_w, groups, &Ho, &Wo))
        return 1;
    const int64_t Cg = C / groups, Kg = K / groups;

#pragma omp parallel for collapse(2) schedule(static)
    for (int64_t n = 0; n < N; ++n) {
        for (int64_t ho = 0; ho < Ho; ++ho) {
            for (int64_t wo = 0; wo < Wo; ++wo) {
                for (int64_t k = 0; k < K; ++k) {
                    const int64_t g = k / Kg;
                    double acc = 0.0;
                    for (int64_t r = 0; r < R; ++r) {
#if ORACLE_MUTATION == 1 /* planted: filter rows flipped */
                        const int64_t h = ho * stride - pad_h + (R - 1 - r);
#elif ORACLE_MUTATION == 2 /* planted: padding applied with the wrong sign */
                        const int64_t h = ho * stride + pad_h + r;
#else
                        const int64_t h = ho * stride - pad_h + r;
#endif
                        if (h < 0 || h >= H)
                            continue;
                        for (int64_t t = 0; t < S; ++t) {
#if ORACLE_MUTATION == 3 /* planted: pad_h used for columns too */
                            const int64_t ww = wo * stride - pad_h + t;
#else
                            const int64_t ww = wo * stride - pad_w + t;
#endif
                            if (ww < 0 || ww >= W)
                                continue;
                            const double* xp = x + ((n * H + h) * W + ww) * C + g * Cg;
                            const double* wp = w + ((k * R + r) * S + t) * Cg;
                            for (int64_t j = 0; j < Cg; ++j) {
#if ORACLE_MUTATION == 4 /* planted: group block taken from the wrong end */
                                acc += x[((n * H + h) * W + ww) * C + (groups - 1 - g) * Cg + j] * wp[j];
#else
                                acc += xp[j] * wp[j];
#endif
                            }
                        }
                    }
                    y[((n * Ho + ho) * Wo + wo) * K + k] = acc;
                }
            }
        }
    }
    return 0;
}

/* dx[n,h,w,c] = sum_{r,t,k'} [u = h + pad_h - r >= 0, u % s == 0, u/s < Ho]
 *                           * [v = w + pad_w - t >= 0, v % s == 0, v/s < Wo]
 *                           * dy[n, u/s, v/s, g*Kg + k'] * w[g*Kg + k', r, t, j],
 * with g = c / Cg and j = c - g*Cg.  The sign test comes before '%' because C's
 * remainder of a negative number is not the mathematical residue. */
int oracle_conv_dgrad_f64(int64_t N, int64_t H, int64_t W, int64_t C, int64_t K,
                          int64_t R, int64_t S, int64_t stride, int64_t pad_h,
                          int64_t pad_w, int64_t groups, const double* dy,
                          const double* w, double* dx)
{
    int64_t Ho, Wo;
    if (oracle_dims(N, H, W, C, K, R, S, stride, pad_h, pad_w, groups, &Ho, &Wo))
        return 1;
    const int64_t Cg = C / groups, Kg = K / groups;

#pragma omp parallel for collapse(2) schedule(static)
    for (int64_t n = 0; n < N; ++n) {
        for (int64_t h = 0; h < H; ++h) {
            for (int64_t ww = 0; ww < W; ++ww) {
                for (int64_t c = 0; c < C; ++c) {
                    const int64_t g = c / Cg, j = c - g * Cg;
                    double acc = 0.0;
                    for (int64_t r = 0; r < R; ++r) {
                        const int64_t u = h + pad_h - r;
#if ORACLE_MUTATION == 5 /* planted: stride divisibility not checked */
                        if (u < 0 || u / stride >= Ho)
                            continue;
#else
                        if (u < 0 || u % stride != 0 || u / stride >= Ho)
                            continue;
#endif
                        for (int64_t t = 0; t < S; ++t) {
                            const int64_t v = ww + pad_w - t;
                            if (v < 0 || v % stride != 0 || v / stride >= Wo)
                                continue;
                            const double* dyp =
                                dy + ((n * Ho + u / stride) * Wo + v / stride) * K + g * Kg;
                            for (int64_t kk = 0; kk < Kg; ++kk) {
#if ORACLE_MUTATION == 6 /* planted: weight read with its channel index transposed */
                                const int64_t widx = ((((g * Kg + kk) * R + r) * S + t) * Cg + (Cg - 1 - j));
#else
                                const int64_t widx = (((g * Kg + kk) * R + r) * S + t) * Cg + j;
#endif
                                acc += dyp[kk] * w[widx];
                            }
                        }
                    }
                    dx[((n * H + h) * W + ww) * C + c] = acc;
                }
            }
        }
    }
    return 0;
}

/* dw[k,r,t,j] = sum_{n,ho,wo} dy[n,ho,wo,k] * x[n, ho*s - pad_h + r, wo*s - pad_w + t, g*Cg + j],
 * g = k / Kg, with x taken as 0 outside the image: the gradient of the
 * forward map with respect to the weight (its value at each weight entry is
 * the sum, over the output pixels, of dY times the input the forward
 * multiplies that entry with). */
int oracle_conv_wgrad_f64(int64_t N, int64_t H, int64_t W, int64_t C, int64_t K,
                          int64_t R, int64_t S, int64_t stride, int64_t pad_h,
                          int64_t pad_w, int64_t groups, const double* x,
                          const double* dy, double* dw)
{
    int64_t Ho, Wo;
    if (oracle_dims(N, H, W, C, K, R, S, stride, pad_h, pad_w, groups, &Ho, &Wo))
        return 1;
    const int64_t Cg = C / groups, Kg = K / groups;

#pragma omp parallel for collapse(2) schedule(static)
    for (int64_t k = 0; k < K; ++k) {
        for (int64_t r = 0; r < R; ++r) {
            const int64_t g = k / Kg;
            for (int64_t t = 0; t < S; ++t) {
                for (int64_t j = 0; j < Cg; ++j) {
                    double acc = 0.0;
                    for (int64_t n = 0; n < N; ++n) {
                        for (int64_t ho = 0; ho < Ho; ++ho) {
                            const int64_t h = ho * stride - pad_h + r;
                            if (h < 0 || h >= H)
                                continue;
                            for (int64_t wo = 0; wo < Wo; ++wo) {
#if ORACLE_MUTATION == 7 /* planted: filter columns mirrored in the weight gradient */
                                const int64_t ww = wo * stride - pad_w + (S - 1 - t);
#else
                                const int64_t ww = wo * stride - pad_w + t;
#endif
                                if (ww < 0 || ww >= W)
                                    continue;
                                acc += dy[((n * Ho + ho) * Wo + wo) * K + k] *
                                       x[((n * H + h) * W + ww) * C + g * Cg + j];
                            }
                        }
                    }
                    dw[((k * R + r) * S + t) * Cg + j] = acc;
                }
            }
        }
    }
    return 0;
}

/* Number of threads the parallel loops above use (1 without OpenMP). */
int oracle_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

void oracle_set_num_threads(int n)
{
#ifdef _OPENMP
    if (n > 0)
        omp_set_num_threads(n);
#else
    (void)n;
#endif
}
