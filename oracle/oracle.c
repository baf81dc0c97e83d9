/*
 * oracle.c -- plain, slow, obviously correct fp64 reference for the fp16 3D
 * convolution and the GroupNorm+SiLU of a video-VAE decoder block.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the checker the GPU path is compared
 * against.  Only the test suite, the package smoke check and the benchmark's
 * CPU-baseline leg may load it.  It shares no code, header, table or helper
 * with the HIP library: it is written from the definitions below and nothing
 * else.  Inputs arrive already widened (exactly) from fp16 to double.
 *
 * What is computed, and where it is defined:
 *
 *  conv3d  -- the direct definition of a stride-1, dilation-1, single-group 3D
 *    cross-correlation over an NDHWC tensor.  The implicit-GEMM shader of the
 *    Draw Things engineering feed (post on the Codex-written Metal conv3d
 *    shaders for the LTX-2.3 video VAE, implicit-GEMM paragraph) computes
 *    exactly this result, only reorganised as a GEMM; the oracle therefore is
 *    the definition, as seven nested loops over (t,h,w,co) x (tau,r,s) with the
 *    input channel innermost and the batch outermost.
 *    Padding: zero outside [0,H) and [0,W); in time either zero outside [0,T)
 *    or "replicate", where an out-of-range frame index is clamped to the
 *    nearest frame (the causal video-VAE convention: the first frame repeated
 *    in front).  The magnitude S = |b| + sum |w * xhat| is accumulated in the
 *    same loop; it scales the acceptance bound of the fp16 path.
 *
 *  groupnorm_silu -- the two-pass definition of GroupNorm (fused with SiLU
 *    in the A1111 Metal fork summary, news.bugfactory.tech item 4286,
 *    paragraph on MPS tweaks): per (sample, group) the mean, then the biased
 *    variance as the mean of squared deviations, then
 *    yhat = (x - mean) / sqrt(var + eps) * gamma_c + beta_c and
 *    out = yhat / (1 + exp(-yhat)).  Groups are contiguous channel ranges.
 *    groupnorm_silu_points evaluates the same definition at selected elements
 *    of tensors too large to widen to fp64 whole.
 *
 * Parity pins for every function here live in tests/test_oracle_*.py.
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>
#include <stdlib.h>

#ifdef _OPENMP
#include <omp.h>
#endif

#define ORACLE_TPAD_ZERO 0
#define ORACLE_TPAD_REPLICATE 1

int oracle_num_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/*
 * IEEE 754 binary16 bit pattern -> double, exactly: sign, 5-bit biased
 * exponent, 10-bit fraction; subnormals are fraction * 2^-24.
 */
double oracle_f16_to_f64(uint16_t h) {
    int e = (h >> 10) & 31, f = h & 1023;
    double v;
    if (e == 0)
        v = ldexp((double)f, -24);
    else if (e == 31)
        v = f ? NAN : INFINITY;
    else
        v = ldexp((double)(1024 + f), e - 25);
    return (h & 0x8000) ? -v : v;
}

/* Output extent of a stride-1 correlation along one axis. */
static int out_extent(int in, int pad_lo, int pad_hi, int k) { return in + pad_lo + pad_hi - k + 1; }

/* One output element, straight from the definition.  Returns y and writes S. */
static double conv_point(const void *xv, int x_f16, const double *w, const double *b,
                         int T, int H, int W, int Cin, int kt, int kh, int kw,
                         int ptf, int ph, int pw, int tmode,
                         int n, int to, int ho, int wo, int co, double *mag) {
    double acc = 0.0, s = 0.0;
    if (b) {
        acc = b[co];
        s = fabs(b[co]);
    }
    for (int tau = 0; tau < kt; ++tau) {
        int ts = to + tau - ptf;
        if (tmode == ORACLE_TPAD_REPLICATE) {
            if (ts < 0) ts = 0;
            if (ts > T - 1) ts = T - 1;
        } else if (ts < 0 || ts >= T) {
            continue; /* zero padding: the tap contributes 0 */
        }
        for (int r = 0; r < kh; ++r) {
            int hs = ho + r - ph;
            if (hs < 0 || hs >= H) continue;
            for (int q = 0; q < kw; ++q) {
                int ws = wo + q - pw;
                if (ws < 0 || ws >= W) continue;
                size_t xo = ((((size_t)n * T + ts) * H + hs) * W + ws) * (size_t)Cin;
                const double *wp = w + ((((size_t)co * kt + tau) * kh + r) * kw + q) * (size_t)Cin;
                if (x_f16) {
                    const uint16_t *xp = (const uint16_t *)xv + xo;
                    for (int ci = 0; ci < Cin; ++ci) {
                        double p = wp[ci] * oracle_f16_to_f64(xp[ci]);
                        acc += p;
                        s += fabs(p);
                    }
                } else {
                    const double *xp = (const double *)xv + xo;
                    for (int ci = 0; ci < Cin; ++ci) {
                        double p = wp[ci] * xp[ci];
                        acc += p;
                        s += fabs(p);
                    }
                }
            }
        }
    }
    *mag = s;
    return acc;
}

/*
 * Full conv3d.  x: [N][T][H][W][Cin], w: [Cout][kt][kh][kw][Cin], b: [Cout] or
 * NULL, res: [N][To][Ho][Wo][Cout] or NULL (added after the bias; not part of
 * S).  y and mag: [N][To][Ho][Wo][Cout].  mag may be NULL.
 * Returns 0, or -1 on an invalid shape.
 */
int oracle_conv3d(const double *x, const double *w, const double *b, const double *res,
                  int N, int T, int H, int W, int Cin, int Cout, int kt, int kh, int kw,
                  int ptf, int ptb, int ph, int pw, int tmode, double *y, double *mag) {
    int To = out_extent(T, ptf, ptb, kt);
    int Ho = out_extent(H, ph, ph, kh);
    int Wo = out_extent(W, pw, pw, kw);
    if (N < 1 || T < 1 || H < 1 || W < 1 || Cin < 1 || Cout < 1 || To < 1 || Ho < 1 || Wo < 1)
        return -1;
    long rows = (long)N * To * Ho;
#pragma omp parallel for schedule(dynamic, 1)
    for (long row = 0; row < rows; ++row) {
        int n = (int)(row / ((long)To * Ho));
        int to = (int)((row / Ho) % To);
        int ho = (int)(row % Ho);
        for (int wo = 0; wo < Wo; ++wo) {
            size_t base = ((((size_t)n * To + to) * Ho + ho) * Wo + wo) * (size_t)Cout;
            for (int co = 0; co < Cout; ++co) {
                double s;
                double v = conv_point(x, 0, w, b, T, H, W, Cin, kt, kh, kw, ptf, ph, pw, tmode,
                                      n, to, ho, wo, co, &s);
                if (res) v += res[base + co];
                y[base + co] = v;
                if (mag) mag[base + co] = s;
            }
        }
    }
    return 0;
}

/*
 * Selected outputs only, for full-size tensors.  m[i] is the flat output-voxel
 * index ((n*To + to)*Ho + ho)*Wo + wo and co[i] the output channel.  x and
 * res (the full residual tensor, or NULL) are fp16 bit patterns when
 * x_f16 / res_f16 is set, doubles otherwise; they are widened exactly.
 * Writes y[i], mag[i].
 */
int oracle_conv3d_points(const void *x, int x_f16, const double *w, const double *b,
                         const void *res, int res_f16,
                         int N, int T, int H, int W, int Cin, int Cout, int kt, int kh, int kw,
                         int ptf, int ptb, int ph, int pw, int tmode,
                         const int64_t *m, const int32_t *co, int64_t npts, double *y, double *mag) {
    int To = out_extent(T, ptf, ptb, kt);
    int Ho = out_extent(H, ph, ph, kh);
    int Wo = out_extent(W, pw, pw, kw);
    if (N < 1 || To < 1 || Ho < 1 || Wo < 1) return -1;
    int64_t M = (int64_t)N * To * Ho * Wo;
    for (int64_t i = 0; i < npts; ++i)
        if (m[i] < 0 || m[i] >= M || co[i] < 0 || co[i] >= Cout) return -1;
#pragma omp parallel for schedule(dynamic, 64)
    for (int64_t i = 0; i < npts; ++i) {
        int64_t mi = m[i];
        int wo = (int)(mi % Wo);
        int ho = (int)((mi / Wo) % Ho);
        int to = (int)((mi / ((int64_t)Wo * Ho)) % To);
        int n = (int)(mi / ((int64_t)Wo * Ho * To));
        double s;
        double v = conv_point(x, x_f16, w, b, T, H, W, Cin, kt, kh, kw, ptf, ph, pw, tmode,
                              n, to, ho, wo, co[i], &s);
        if (res) {
            size_t ri = (size_t)mi * Cout + co[i];
            v += res_f16 ? oracle_f16_to_f64(((const uint16_t *)res)[ri]) : ((const double *)res)[ri];
        }
        y[i] = v;
        if (mag) mag[i] = s;
    }
    return 0;
}

/*
 * GroupNorm (+ optional SiLU), two passes in fp64.  x, y: [N][THW][C];
 * gamma, beta: [C]; groups divide C into contiguous ranges of C/groups
 * channels.  mean_out, var_out: [N][groups] or NULL (biased variance).
 */
int oracle_groupnorm_silu(const double *x, int N, int64_t thw, int C, int groups,
                          const double *gamma, const double *beta, double eps, int apply_silu,
                          double *y, double *mean_out, double *var_out) {
    if (N < 1 || thw < 1 || C < 1 || groups < 1 || C % groups != 0) return -1;
    int cg = C / groups;
    long ng = (long)N * groups;
#pragma omp parallel for schedule(dynamic, 1)
    for (long i = 0; i < ng; ++i) {
        int n = (int)(i / groups), g = (int)(i % groups);
        const double *xs = x + (size_t)n * thw * C;
        double *ys = y + (size_t)n * thw * C;
        double cnt = (double)thw * cg;
        double sum = 0.0;
        for (int64_t v = 0; v < thw; ++v)
            for (int c = g * cg; c < (g + 1) * cg; ++c) sum += xs[(size_t)v * C + c];
        double mean = sum / cnt;
        double ss = 0.0;
        for (int64_t v = 0; v < thw; ++v)
            for (int c = g * cg; c < (g + 1) * cg; ++c) {
                double d = xs[(size_t)v * C + c] - mean;
                ss += d * d;
            }
        double var = ss / cnt;
        double inv = 1.0 / sqrt(var + eps);
        for (int64_t v = 0; v < thw; ++v)
            for (int c = g * cg; c < (g + 1) * cg; ++c) {
                double yh = (xs[(size_t)v * C + c] - mean) * inv * gamma[c] + beta[c];
                ys[(size_t)v * C + c] = apply_silu ? yh / (1.0 + exp(-yh)) : yh;
            }
        if (mean_out) mean_out[i] = mean;
        if (var_out) var_out[i] = var;
    }
    return 0;
}

/*
 * GroupNorm (+ optional SiLU) at selected elements of a large tensor, with
 * the same two-pass statistics as oracle_groupnorm_silu.  x: [N][THW][C],
 * fp16 bit patterns when x_f16 is set (widened exactly on the fly, so a
 * multi-GB activation needs no fp64 copy), doubles otherwise.  Element i is
 * voxel vox[i] (flat over N*THW) at channel ch[i].  Each pass sums a fixed
 * partition of the voxels into 64 ranges and adds the range sums in order,
 * so the result does not depend on the thread count.  Writes y[i] and, per
 * (sample, group), mean_out / var_out (biased variance).
 */
static double gn_elem(const void *x, int x_f16, size_t i) {
    return x_f16 ? oracle_f16_to_f64(((const uint16_t *)x)[i]) : ((const double *)x)[i];
}

int oracle_groupnorm_silu_points(const void *x, int x_f16, int N, int64_t thw, int C, int groups,
                                 const double *gamma, const double *beta, double eps, int apply_silu,
                                 const int64_t *vox, const int32_t *ch, int64_t npts, double *y,
                                 double *mean_out, double *var_out) {
    enum { NB = 64 };
    if (N < 1 || thw < 1 || C < 1 || groups < 1 || C % groups != 0) return -1;
    for (int64_t i = 0; i < npts; ++i)
        if (vox[i] < 0 || vox[i] >= (int64_t)N * thw || ch[i] < 0 || ch[i] >= C) return -1;
    int cg = C / groups;
    double cnt = (double)thw * cg;
    double *part = (double *)calloc((size_t)NB * groups, sizeof(double));
    if (!part) return -1;
    for (int n = 0; n < N; ++n) {
        size_t base = (size_t)n * thw * C;
        double *mean = mean_out + (size_t)n * groups, *var = var_out + (size_t)n * groups;
        for (int pass = 0; pass < 2; ++pass) {
#pragma omp parallel for schedule(dynamic, 1)
            for (int b = 0; b < NB; ++b) {
                int64_t v0 = thw * b / NB, v1 = thw * (b + 1) / NB;
                double *ps = part + (size_t)b * groups;
                for (int g = 0; g < groups; ++g) ps[g] = 0.0;
                for (int64_t v = v0; v < v1; ++v)
                    for (int c = 0; c < C; ++c) {
                        double e = gn_elem(x, x_f16, base + (size_t)v * C + c);
                        if (pass == 0) {
                            ps[c / cg] += e;
                        } else {
                            double d = e - mean[c / cg];
                            ps[c / cg] += d * d;
                        }
                    }
            }
            for (int g = 0; g < groups; ++g) {
                double s = 0.0;
                for (int b = 0; b < NB; ++b) s += part[(size_t)b * groups + g];
                if (pass == 0)
                    mean[g] = s / cnt;
                else
                    var[g] = s / cnt;
            }
        }
    }
    free(part);
    for (int64_t i = 0; i < npts; ++i) {
        int n = (int)(vox[i] / thw), c = ch[i], g = c / cg;
        double e = gn_elem(x, x_f16, (size_t)vox[i] * C + c);
        double yh = (e - mean_out[(size_t)n * groups + g]) / sqrt(var_out[(size_t)n * groups + g] + eps) * gamma[c] +
                    beta[c];
        y[i] = apply_silu ? yh / (1.0 + exp(-yh)) : yh;
    }
    return 0;
}
