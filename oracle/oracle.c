/*
 * oracle.c -- plain, slow, obviously correct CPU reference for the fused
 * Conv2d + BatchNorm + SiLU block, in FP32-input / FP64-arithmetic form and in
 * the INT8 (int8 weights per output channel, int8 activations per tensor,
 * int32 accumulation) form.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load this library.  It shares no code,
 * header, table or constant with the GPU library, and it never reads anything
 * the GPU library produced.
 *
 * What it follows:
 *  - "YOLO26N Inference Optimisation" (vision-rs docs), section "nsys
 *    kernel-level breakdown" and "Key observations" 2: the op is one fused
 *    convolution + batch norm + SiLU; section "Baseline benchmark": batch norm
 *    is folded into the conv weights at load time.
 *  - Same page, section "NHWC migration -- What NHWC is and why it matters":
 *    the convolution is the contraction over (C_in, kH, kW); here it is
 *    written directly as that sum over NCHW tensors (the plain definition),
 *    with no GEMM lowering, blocking or reordering.
 *  - "Edge optimisation of YOLO26" (edge-optimization README), sections
 *    "Highlights" and "Design notes": int8 weights with one scale per output
 *    channel, symmetric ranges, activations with a percentile-calibrated
 *    per-tensor scale.
 *
 * Readings where the pages are silent (each also listed with the design notes):
 *  - SiLU(z) = z / (1 + exp(-z)).
 *  - Batch norm in inference mode with running statistics:
 *      bn = (conv - mean) / sqrt(var + eps) * gamma + beta.
 *  - Folding: sc = gamma / sqrt(var + eps), W' = W * sc, b' = beta - mean * sc,
 *    all in double.
 *  - INT8 weights: s_w = max|W'[co,:]| / 127 (1.0 for an all-zero channel),
 *    q_w = clamp(rne(W' / s_w), -127, 127), in double.
 *  - INT8 activations: q_x = clamp(rne(fp32(x / s_x)), -127, 127) with an
 *    fp32, correctly rounded division; zero padding quantises to 0.
 *  - INT8 epilogue: y = SiLU(acc * f[co] + b'[co]) with f = fp32(s_x * s_w).
 *  - Percentile: the 'linear' definition (position q*(n-1) in the sorted
 *    sample, linear interpolation between the two neighbours).
 *  - Fused epilogue options ("YOLO26N Inference Optimisation", section
 *    "Improvements" #7: bias and residual adds in the conv epilogue; the
 *    plain conv2d_forward + nchw_bias_add of section "nsys kernel-level
 *    breakdown"): the activation is SiLU or the identity, and a residual r is
 *    added after the activation, y = act(z) + r (the shortcut of a YOLO
 *    bottleneck adds its input to the output of its second conv block).
 *  - Asymmetric activations (edge-optimization README, "Design notes": ONNX
 *    Runtime's default is asymmetric uint8 activations with symmetric
 *    weights, because activations after SiLU are mostly positive):
 *    q = clamp(rne(fp32(x / s_x)) + z_x, 0, 255) with an integer zero point
 *    z_x in [0, 255], so x ~ s_x (q - z_x).  The convolution sums
 *    q_w (q - z_x) over the taps inside the image: zero padding is a real
 *    zero, i.e. the code z_x, and contributes nothing.
 *  - INT8 output (edge-optimization README, "Highlights": the network runs in
 *    INT8 end to end): the output codes are the activation quantiser applied
 *    to the fp32 value of y, q_y = clamp(rne(fp32(fp32(y) / s_y)), -127, 127);
 *    an int8 residual contributes r = s_r * q_r.
 *
 * Build: gcc -O2 -fopenmp -ffp-contract=off -shared -fPIC (see build.py).
 * -ffp-contract=off keeps every multiply and add separately rounded, so the
 * double results follow the written expressions exactly.
 */
#include <math.h>
#include <omp.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* Output size of one spatial axis: floor((in + 2p - k) / s) + 1. */
int oracle_out_dim(int in, int k, int s, int p) {
    if (in + 2 * p < k || s <= 0) return 0;
    return (in + 2 * p - k) / s + 1;
}

/* Input value with zero padding: x~[n,c,iy,ix] = 0 outside the image. */
static double xin(const float *x, int c_in, int h, int w, int n, int c, int iy, int ix) {
    if (iy < 0 || iy >= h || ix < 0 || ix >= w) return 0.0;
    return (double)x[(((size_t)n * c_in + c) * h + iy) * w + ix];
}

/* Shapes of one convolution, in the definition's notation. */
typedef struct {
    int n, c_in, h, w, c_out, k, s, p, oh, ow;
} dims_t;

static dims_t make_dims(int n, int c_in, int h, int w, int c_out, int k, int s, int p) {
    dims_t d = {n, c_in, h, w, c_out, k, s, p, oracle_out_dim(h, k, s, p), oracle_out_dim(w, k, s, p)};
    return d;
}

/* One output of the convolution:
 *   sum_{ci,i,j} W[co,ci,i,j] * x~[b,ci, oh*s - p + i, ow*s - p + j]
 * summed in the order ci, i, j.  With absmode set it instead returns
 *   sum |W[co,ci,i,j] * scale * x~[...]|   (the tolerance magnitude). */
static double conv_at(const float *x, const float *wt, const dims_t *d, int b, int co, int oh, int ow,
                      int absmode, double scale) {
    double acc = 0.0;
    for (int ci = 0; ci < d->c_in; ci++)
        for (int i = 0; i < d->k; i++)
            for (int j = 0; j < d->k; j++) {
                double wv = (double)wt[(((size_t)co * d->c_in + ci) * d->k + i) * d->k + j];
                double xv = xin(x, d->c_in, d->h, d->w, b, ci, oh * d->s - d->p + i, ow * d->s - d->p + j);
                if (absmode)
                    acc += fabs(wv * scale * xv);
                else
                    acc += wv * xv;
            }
    return acc;
}

/* One output of the integer convolution; *absacc (if not NULL) gets sum |q_w q_x|. */
static int64_t conv_i8_at(const int8_t *qx, const int8_t *qw, const dims_t *d, int b, int co, int oh,
                          int ow, int64_t *absacc) {
    int64_t acc = 0, aacc = 0;
    for (int ci = 0; ci < d->c_in; ci++)
        for (int i = 0; i < d->k; i++)
            for (int j = 0; j < d->k; j++) {
                int iy = oh * d->s - d->p + i, ix = ow * d->s - d->p + j;
                if (iy < 0 || iy >= d->h || ix < 0 || ix >= d->w) continue;
                int64_t t = (int64_t)qw[(((size_t)co * d->c_in + ci) * d->k + i) * d->k + j] *
                            (int64_t)qx[(((size_t)b * d->c_in + ci) * d->h + iy) * d->w + ix];
                acc += t;
                aacc += t < 0 ? -t : t;
            }
    if (absacc) *absacc = aacc;
    return acc;
}

/*
 * Plain 2-D cross-correlation (the "convolution" of deep-learning frameworks):
 *   out[n,co,oh,ow] = sum_{ci,i,j} W[co,ci,i,j] * x~[n,ci, oh*s - p + i, ow*s - p + j]
 * x is NCHW fp32, W is OIHW fp32, out is NCHW double.  The sum runs in the
 * order ci, i, j for every output, whatever the stride.
 */
void oracle_conv2d(const float *x, const float *wt, int n, int c_in, int h, int w,
                   int c_out, int k, int s, int p, double *out) {
    dims_t d = make_dims(n, c_in, h, w, c_out, k, s, p);
#pragma omp parallel for collapse(2) schedule(static)
    for (int b = 0; b < n; b++)
        for (int co = 0; co < c_out; co++)
            for (int oh = 0; oh < d.oh; oh++)
                for (int ow = 0; ow < d.ow; ow++)
                    out[(((size_t)b * c_out + co) * d.oh + oh) * d.ow + ow] = conv_at(x, wt, &d, b, co, oh, ow, 0, 0.0);
}

/* SiLU(z) = z * sigmoid(z) = z / (1 + e^-z). */
double oracle_silu1(double z) { return z / (1.0 + exp(-z)); }

/* The activation of the epilogue: act 0 = SiLU, act 1 = identity. */
static double act1(int act, double z) { return act == 1 ? z : oracle_silu1(z); }

void oracle_silu(const double *z, double *y, long count) {
    for (long i = 0; i < count; i++) y[i] = oracle_silu1(z[i]);
}

/* Inference batch norm with running statistics, applied per output channel
 * to an NCHW double tensor, in place. */
void oracle_batchnorm(double *t, int n, int c, int hw, const float *gamma, const float *beta,
                      const float *mean, const float *var, double eps) {
    for (int b = 0; b < n; b++)
        for (int ch = 0; ch < c; ch++) {
            double g = gamma[ch], be = beta[ch], mu = mean[ch], v = var[ch];
            double *row = t + ((size_t)b * c + ch) * hw;
            for (int i = 0; i < hw; i++) row[i] = (row[i] - mu) / sqrt(v + eps) * g + be;
        }
}

/*
 * Batch-norm folding (done once, at load): sc = gamma / sqrt(var + eps),
 * W'[co,...] = W[co,...] * sc[co], b'[co] = beta[co] - mean[co] * sc[co].
 * per_co = C_in * kH * kW weights per output channel.
 */
void oracle_bn_fold(const float *wt, int c_out, int per_co, const float *gamma, const float *beta,
                    const float *mean, const float *var, double eps, double *w_folded,
                    double *b_folded) {
    for (int co = 0; co < c_out; co++) {
        double sc = (double)gamma[co] / sqrt((double)var[co] + eps);
        for (int i = 0; i < per_co; i++)
            w_folded[(size_t)co * per_co + i] = (double)wt[(size_t)co * per_co + i] * sc;
        b_folded[co] = (double)beta[co] - (double)mean[co] * sc;
    }
}

/*
 * The fused FP32 block, unfolded: y = act(BN(conv(x, W))) (+ residual),
 * computed as conv -> batch norm -> activation -> residual add in double
 * (act 0 = SiLU, 1 = identity; residual is an NCHW double tensor shaped like
 * y, or NULL).  Also returns, per output,
 *   sabs[n,co,oh,ow] = sum |W'[co,ci,i,j] * x~[...]|   with W' the folded weights,
 * the magnitude that scales the parity tolerance.
 */
void oracle_conv_bn_act_f32(const float *x, const float *wt, const float *gamma,
                            const float *beta, const float *mean, const float *var, double eps,
                            int n, int c_in, int h, int w, int c_out, int k, int s, int p, int act,
                            const double *residual, double *y, double *sabs) {
    int oh_n = oracle_out_dim(h, k, s, p), ow_n = oracle_out_dim(w, k, s, p);
    size_t count = (size_t)n * c_out * oh_n * ow_n;
    oracle_conv2d(x, wt, n, c_in, h, w, c_out, k, s, p, y);
    oracle_batchnorm(y, n, c_out, oh_n * ow_n, gamma, beta, mean, var, eps);
    for (size_t i = 0; i < count; i++) {
        y[i] = act1(act, y[i]);
        if (residual) y[i] += residual[i];
    }
    if (sabs) {
        dims_t d = make_dims(n, c_in, h, w, c_out, k, s, p);
#pragma omp parallel for collapse(2) schedule(static)
        for (int b = 0; b < n; b++)
            for (int co = 0; co < c_out; co++) {
                double sc = (double)gamma[co] / sqrt((double)var[co] + eps);
                for (int oh = 0; oh < oh_n; oh++)
                    for (int ow = 0; ow < ow_n; ow++)
                        sabs[(((size_t)b * c_out + co) * oh_n + oh) * ow_n + ow] =
                            conv_at(x, wt, &d, b, co, oh, ow, 1, sc);
            }
    }
}

/* The plain block, y = SiLU(BN(conv(x, W))). */
void oracle_conv_bn_silu_f32(const float *x, const float *wt, const float *gamma,
                             const float *beta, const float *mean, const float *var, double eps,
                             int n, int c_in, int h, int w, int c_out, int k, int s, int p,
                             double *y, double *sabs) {
    oracle_conv_bn_act_f32(x, wt, gamma, beta, mean, var, eps, n, c_in, h, w, c_out, k, s, p, 0, NULL, y,
                           sabs);
}

/*
 * The same fused FP32 block evaluated only at the given outputs: pts holds
 * npts quadruples (b, co, oh, ow); y[i] and sabs[i] (may be NULL) receive the
 * value and the tolerance magnitude of output i.  Used to check full-size
 * layers on a sample of outputs.
 */
void oracle_conv_bn_act_f32_points(const float *x, const float *wt, const float *gamma,
                                   const float *beta, const float *mean, const float *var,
                                   double eps, int n, int c_in, int h, int w, int c_out, int k,
                                   int s, int p, int act, const double *res_pts,
                                   const int32_t *pts, long npts, double *y, double *sabs) {
    dims_t d = make_dims(n, c_in, h, w, c_out, k, s, p);
#pragma omp parallel for schedule(dynamic, 16)
    for (long t = 0; t < npts; t++) {
        int b = pts[4 * t], co = pts[4 * t + 1], oh = pts[4 * t + 2], ow = pts[4 * t + 3];
        double conv = conv_at(x, wt, &d, b, co, oh, ow, 0, 0.0);
        double bn = (conv - (double)mean[co]) / sqrt((double)var[co] + eps) * (double)gamma[co] + (double)beta[co];
        y[t] = act1(act, bn);
        if (res_pts) y[t] += res_pts[t];
        if (sabs) sabs[t] = conv_at(x, wt, &d, b, co, oh, ow, 1, (double)gamma[co] / sqrt((double)var[co] + eps));
    }
}

void oracle_conv_bn_silu_f32_points(const float *x, const float *wt, const float *gamma,
                                    const float *beta, const float *mean, const float *var,
                                    double eps, int n, int c_in, int h, int w, int c_out, int k,
                                    int s, int p, const int32_t *pts, long npts, double *y,
                                    double *sabs) {
    oracle_conv_bn_act_f32_points(x, wt, gamma, beta, mean, var, eps, n, c_in, h, w, c_out, k, s, p, 0, NULL,
                                  pts, npts, y, sabs);
}

/* ---------------------------------------------------------------- INT8 -- */

/* Round half to even at integer resolution, then clamp to [-127, 127]. */
static int clamp127(double r) {
    if (r > 127.0) return 127;
    if (r < -127.0) return -127;
    return (int)r;
}

/*
 * Per-output-channel symmetric weight quantisation of the folded weights:
 *   s_w[co] = max_i |W'[co,i]| / 127   (1.0 when the channel is all zero)
 *   q_w[co,i] = clamp(rne(W'[co,i] / s_w[co]), -127, 127)
 */
void oracle_quantize_weights(const double *w_folded, int c_out, int per_co, int8_t *q,
                             double *s_w) {
    for (int co = 0; co < c_out; co++) {
        const double *row = w_folded + (size_t)co * per_co;
        double m = 0.0;
        for (int i = 0; i < per_co; i++)
            if (fabs(row[i]) > m) m = fabs(row[i]);
        double s = (m > 0.0) ? m / 127.0 : 1.0;
        s_w[co] = s;
        for (int i = 0; i < per_co; i++) q[(size_t)co * per_co + i] = (int8_t)clamp127(nearbyint(row[i] / s));
    }
}

/*
 * Per-tensor symmetric activation quantisation:
 *   q_x = clamp(rne(fp32(x / s_x)), -127, 127), with the division done in fp32.
 */
void oracle_quantize_activations(const float *x, long count, float s_x, int8_t *q) {
    for (long i = 0; i < count; i++) {
        volatile float r = x[i] / s_x; /* one correctly rounded fp32 division */
        q[i] = (int8_t)clamp127(nearbyint((double)r));
    }
}

/*
 * Per-tensor asymmetric uint8 activation quantisation:
 *   q = clamp(rne(fp32(x / s_x)) + z, 0, 255), the division in fp32.
 */
void oracle_quantize_activations_u8(const float *x, long count, float s_x, int z, uint8_t *q) {
    for (long i = 0; i < count; i++) {
        volatile float r = x[i] / s_x; /* one correctly rounded fp32 division */
        double v = nearbyint((double)r) + (double)z;
        if (v < 0.0) v = 0.0;
        if (v > 255.0) v = 255.0;
        q[i] = (uint8_t)v;
    }
}

/* One output of the asymmetric integer convolution: sum over the taps inside
 * the image of q_w * (q - z); *absacc (if not NULL) gets sum |q_w (q - z)|. */
static int64_t conv_u8_at(const uint8_t *qx, int z, const int8_t *qw, const dims_t *d, int b, int co, int oh,
                          int ow, int64_t *absacc) {
    int64_t acc = 0, aacc = 0;
    for (int ci = 0; ci < d->c_in; ci++)
        for (int i = 0; i < d->k; i++)
            for (int j = 0; j < d->k; j++) {
                int iy = oh * d->s - d->p + i, ix = ow * d->s - d->p + j;
                if (iy < 0 || iy >= d->h || ix < 0 || ix >= d->w) continue;
                int64_t t = (int64_t)qw[(((size_t)co * d->c_in + ci) * d->k + i) * d->k + j] *
                            ((int64_t)qx[(((size_t)b * d->c_in + ci) * d->h + iy) * d->w + ix] - (int64_t)z);
                acc += t;
                aacc += t < 0 ? -t : t;
            }
    if (absacc) *absacc = aacc;
    return acc;
}

/*
 * Asymmetric integer convolution: acc = sum q_w (q - z) over the taps inside
 * the image (padding is the real value 0), exact in int64, stored as int32.
 * Returns the number of sums outside the int32 range (0 expected).
 */
long oracle_conv_u8_acc(const uint8_t *qx, int z, const int8_t *qw, int n, int c_in, int h, int w, int c_out,
                        int k, int s, int p, int32_t *acc_out, int64_t *absacc_out) {
    dims_t d = make_dims(n, c_in, h, w, c_out, k, s, p);
    long overflow = 0;
#pragma omp parallel for collapse(2) schedule(static) reduction(+ : overflow)
    for (int b = 0; b < n; b++)
        for (int co = 0; co < c_out; co++)
            for (int oh = 0; oh < d.oh; oh++)
                for (int ow = 0; ow < d.ow; ow++) {
                    int64_t a;
                    int64_t acc = conv_u8_at(qx, z, qw, &d, b, co, oh, ow, &a);
                    if (acc > INT32_MAX || acc < INT32_MIN) overflow++;
                    size_t o = (((size_t)b * c_out + co) * d.oh + oh) * d.ow + ow;
                    acc_out[o] = (int32_t)acc;
                    if (absacc_out) absacc_out[o] = a;
                }
    return overflow;
}

/*
 * Integer convolution with zero padding, accumulated exactly (int64) and
 * stored as int32: acc[n,co,oh,ow] = sum_{ci,i,j} q_w[co,ci,i,j] * q_x~[...].
 * Returns the number of accumulators outside the int32 range (0 expected:
 * |acc| <= 127^2 * C_in * k^2).
 */
long oracle_conv_i8_acc(const int8_t *qx, const int8_t *qw, int n, int c_in, int h, int w,
                        int c_out, int k, int s, int p, int32_t *acc_out) {
    dims_t d = make_dims(n, c_in, h, w, c_out, k, s, p);
    long overflow = 0;
#pragma omp parallel for collapse(2) schedule(static) reduction(+ : overflow)
    for (int b = 0; b < n; b++)
        for (int co = 0; co < c_out; co++)
            for (int oh = 0; oh < d.oh; oh++)
                for (int ow = 0; ow < d.ow; ow++) {
                    int64_t acc = conv_i8_at(qx, qw, &d, b, co, oh, ow, NULL);
                    if (acc > INT32_MAX || acc < INT32_MIN) overflow++;
                    acc_out[(((size_t)b * c_out + co) * d.oh + oh) * d.ow + ow] = (int32_t)acc;
                }
    return overflow;
}

/*
 * INT8 epilogue: dequantise, add the folded bias, activation, residual, all
 * in double:
 *   f[co] = fp32(s_x * s_w[co]),  y = act(acc * f[co] + b'[co]) (+ residual).
 * act 0 = SiLU, 1 = identity; residual (NCHW double like y) may be NULL.
 * f_out (may be NULL) receives the fp32 dequantisation factors.
 */
void oracle_epilogue_i8_act(const int32_t *acc, int n, int c_out, int hw, float s_x, const double *s_w,
                            const double *b_folded, int act, const double *residual, double *y,
                            float *f_out) {
    for (int co = 0; co < c_out; co++) {
        float f = (float)((double)s_x * s_w[co]);
        if (f_out) f_out[co] = f;
        for (int b = 0; b < n; b++) {
            size_t base = ((size_t)b * c_out + co) * hw;
            for (int i = 0; i < hw; i++) {
                y[base + i] = act1(act, (double)acc[base + i] * (double)f + b_folded[co]);
                if (residual) y[base + i] += residual[base + i];
            }
        }
    }
}

void oracle_epilogue_i8(const int32_t *acc, int n, int c_out, int hw, float s_x, const double *s_w,
                        const double *b_folded, double *y, float *f_out) {
    oracle_epilogue_i8_act(acc, n, c_out, hw, s_x, s_w, b_folded, 0, NULL, y, f_out);
}

/*
 * sum |q_w * q_x~| per output, the integer magnitude that (times f[co])
 * scales the INT8 parity tolerance.
 */
void oracle_conv_i8_absacc(const int8_t *qx, const int8_t *qw, int n, int c_in, int h, int w,
                           int c_out, int k, int s, int p, int64_t *out) {
    dims_t d = make_dims(n, c_in, h, w, c_out, k, s, p);
#pragma omp parallel for collapse(2) schedule(static)
    for (int b = 0; b < n; b++)
        for (int co = 0; co < c_out; co++)
            for (int oh = 0; oh < d.oh; oh++)
                for (int ow = 0; ow < d.ow; ow++) {
                    int64_t a;
                    (void)conv_i8_at(qx, qw, &d, b, co, oh, ow, &a);
                    out[(((size_t)b * c_out + co) * d.oh + oh) * d.ow + ow] = a;
                }
}

/* ------------------------------------------------------- calibration -- */

static int cmp_double(const void *a, const void *b) {
    double x = *(const double *)a, y = *(const double *)b;
    return (x > y) - (x < y);
}

/*
 * q-th percentile (0 <= q <= 100) of |x| by the 'linear' definition: sort,
 * take position t = q/100 * (count-1), interpolate between the neighbours
 * floor(t) and floor(t)+1.
 */
double oracle_percentile_abs(const float *x, long count, double q) {
    if (count <= 0) return 0.0;
    double *a = (double *)malloc(sizeof(double) * (size_t)count);
    if (!a) return -1.0;
    for (long i = 0; i < count; i++) a[i] = fabs((double)x[i]);
    qsort(a, (size_t)count, sizeof(double), cmp_double);
    double t = q / 100.0 * (double)(count - 1);
    long lo = (long)floor(t);
    if (lo >= count - 1) {
        double r = a[count - 1];
        free(a);
        return r;
    }
    double frac = t - (double)lo;
    double r = a[lo] + frac * (a[lo + 1] - a[lo]);
    free(a);
    return r;
}

/*
 * The whole INT8 block from float inputs: fold BN, quantise weights per
 * channel, quantise activations with the given per-tensor scale, integer
 * convolution, dequant + bias + SiLU.  Any output pointer may be NULL except y.
 * Returns the int32 overflow count of the accumulators (0 expected).
 */
long oracle_conv_bn_act_i8(const float *x, float s_x, const float *wt, const float *gamma,
                           const float *beta, const float *mean, const float *var, double eps,
                           int n, int c_in, int h, int w, int c_out, int k, int s, int p, int act,
                           const double *residual, double *y, int32_t *acc_out, int8_t *qw_out,
                           double *sw_out, float *f_out, int64_t *absacc_out) {
    int per_co = c_in * k * k;
    int oh_n = oracle_out_dim(h, k, s, p), ow_n = oracle_out_dim(w, k, s, p);
    size_t nx = (size_t)n * c_in * h * w, ny = (size_t)n * c_out * oh_n * ow_n;
    double *wf = (double *)malloc(sizeof(double) * (size_t)c_out * per_co);
    double *bf = (double *)malloc(sizeof(double) * (size_t)c_out);
    double *sw = (double *)malloc(sizeof(double) * (size_t)c_out);
    int8_t *qw = (int8_t *)malloc((size_t)c_out * per_co);
    int8_t *qx = (int8_t *)malloc(nx ? nx : 1);
    int32_t *acc = (int32_t *)malloc(sizeof(int32_t) * (ny ? ny : 1));
    long ovf = -1;
    if (!wf || !bf || !sw || !qw || !qx || !acc) goto done;
    oracle_bn_fold(wt, c_out, per_co, gamma, beta, mean, var, eps, wf, bf);
    oracle_quantize_weights(wf, c_out, per_co, qw, sw);
    oracle_quantize_activations(x, (long)nx, s_x, qx);
    ovf = oracle_conv_i8_acc(qx, qw, n, c_in, h, w, c_out, k, s, p, acc);
    oracle_epilogue_i8_act(acc, n, c_out, oh_n * ow_n, s_x, sw, bf, act, residual, y, f_out);
    if (acc_out) memcpy(acc_out, acc, sizeof(int32_t) * ny);
    if (qw_out) memcpy(qw_out, qw, (size_t)c_out * per_co);
    if (sw_out) memcpy(sw_out, sw, sizeof(double) * (size_t)c_out);
    if (absacc_out) oracle_conv_i8_absacc(qx, qw, n, c_in, h, w, c_out, k, s, p, absacc_out);
done:
    free(wf); free(bf); free(sw); free(qw); free(qx); free(acc);
    return ovf;
}

long oracle_conv_bn_silu_i8(const float *x, float s_x, const float *wt, const float *gamma,
                            const float *beta, const float *mean, const float *var, double eps,
                            int n, int c_in, int h, int w, int c_out, int k, int s, int p,
                            double *y, int32_t *acc_out, int8_t *qw_out, double *sw_out,
                            float *f_out, int64_t *absacc_out) {
    return oracle_conv_bn_act_i8(x, s_x, wt, gamma, beta, mean, var, eps, n, c_in, h, w, c_out, k, s, p, 0,
                                 NULL, y, acc_out, qw_out, sw_out, f_out, absacc_out);
}

/*
 * The INT8 block evaluated only at the given outputs (pts: npts quadruples
 * b, co, oh, ow): fold, quantise weights, quantise the whole input, then the
 * integer sums and the epilogue at each point.  acc_out / absacc_out may be
 * NULL.  Returns the int32 overflow count (0 expected), -1 on allocation failure.
 */
long oracle_conv_bn_act_i8_points(const float *x, float s_x, const float *wt, const float *gamma,
                                  const float *beta, const float *mean, const float *var,
                                  double eps, int n, int c_in, int h, int w, int c_out, int k,
                                  int s, int p, int act, const double *res_pts, const int32_t *pts,
                                  long npts, double *y, int32_t *acc_out, int64_t *absacc_out) {
    dims_t d = make_dims(n, c_in, h, w, c_out, k, s, p);
    int per_co = c_in * k * k;
    size_t nx = (size_t)n * c_in * h * w;
    double *wf = (double *)malloc(sizeof(double) * (size_t)c_out * per_co);
    double *bf = (double *)malloc(sizeof(double) * (size_t)c_out);
    double *sw = (double *)malloc(sizeof(double) * (size_t)c_out);
    int8_t *qw = (int8_t *)malloc((size_t)c_out * per_co);
    int8_t *qx = (int8_t *)malloc(nx ? nx : 1);
    long ovf = -1;
    if (!wf || !bf || !sw || !qw || !qx) goto done;
    oracle_bn_fold(wt, c_out, per_co, gamma, beta, mean, var, eps, wf, bf);
    oracle_quantize_weights(wf, c_out, per_co, qw, sw);
    oracle_quantize_activations(x, (long)nx, s_x, qx);
    ovf = 0;
    for (long t = 0; t < npts; t++) {
        int b = pts[4 * t], co = pts[4 * t + 1], oh = pts[4 * t + 2], ow = pts[4 * t + 3];
        int64_t a;
        int64_t acc = conv_i8_at(qx, qw, &d, b, co, oh, ow, &a);
        if (acc > INT32_MAX || acc < INT32_MIN) ovf++;
        float f = (float)((double)s_x * sw[co]);
        y[t] = act1(act, (double)(int32_t)acc * (double)f + bf[co]);
        if (res_pts) y[t] += res_pts[t];
        if (acc_out) acc_out[t] = (int32_t)acc;
        if (absacc_out) absacc_out[t] = a;
    }
done:
    free(wf); free(bf); free(sw); free(qw); free(qx);
    return ovf;
}

long oracle_conv_bn_silu_i8_points(const float *x, float s_x, const float *wt, const float *gamma,
                                   const float *beta, const float *mean, const float *var,
                                   double eps, int n, int c_in, int h, int w, int c_out, int k,
                                   int s, int p, const int32_t *pts, long npts, double *y,
                                   int32_t *acc_out, int64_t *absacc_out) {
    return oracle_conv_bn_act_i8_points(x, s_x, wt, gamma, beta, mean, var, eps, n, c_in, h, w, c_out, k, s, p,
                                        0, NULL, pts, npts, y, acc_out, absacc_out);
}

/*
 * The whole block with asymmetric uint8 activations: fold BN, quantise the
 * weights per channel (symmetric), quantise the activations with (s_x, z_x),
 * asymmetric integer convolution, then the same epilogue as the symmetric
 * block: y = act(acc * f[co] + b'[co]) (+ residual), f = fp32(s_x * s_w[co]).
 * Any output pointer may be NULL except y.  Returns the int32 overflow count.
 */
long oracle_conv_bn_act_u8(const float *x, float s_x, int z_x, const float *wt, const float *gamma,
                           const float *beta, const float *mean, const float *var, double eps, int n,
                           int c_in, int h, int w, int c_out, int k, int s, int p, int act,
                           const double *residual, double *y, int32_t *acc_out, int8_t *qw_out,
                           double *sw_out, float *f_out, int64_t *absacc_out) {
    int per_co = c_in * k * k;
    int oh_n = oracle_out_dim(h, k, s, p), ow_n = oracle_out_dim(w, k, s, p);
    size_t nx = (size_t)n * c_in * h * w, ny = (size_t)n * c_out * oh_n * ow_n;
    double *wf = (double *)malloc(sizeof(double) * (size_t)c_out * per_co);
    double *bf = (double *)malloc(sizeof(double) * (size_t)c_out);
    double *sw = (double *)malloc(sizeof(double) * (size_t)c_out);
    int8_t *qw = (int8_t *)malloc((size_t)c_out * per_co);
    uint8_t *qx = (uint8_t *)malloc(nx ? nx : 1);
    int32_t *acc = (int32_t *)malloc(sizeof(int32_t) * (ny ? ny : 1));
    long ovf = -1;
    if (!wf || !bf || !sw || !qw || !qx || !acc) goto done;
    oracle_bn_fold(wt, c_out, per_co, gamma, beta, mean, var, eps, wf, bf);
    oracle_quantize_weights(wf, c_out, per_co, qw, sw);
    oracle_quantize_activations_u8(x, (long)nx, s_x, z_x, qx);
    ovf = oracle_conv_u8_acc(qx, z_x, qw, n, c_in, h, w, c_out, k, s, p, acc, absacc_out);
    oracle_epilogue_i8_act(acc, n, c_out, oh_n * ow_n, s_x, sw, bf, act, residual, y, f_out);
    if (acc_out) memcpy(acc_out, acc, sizeof(int32_t) * ny);
    if (qw_out) memcpy(qw_out, qw, (size_t)c_out * per_co);
    if (sw_out) memcpy(sw_out, sw, sizeof(double) * (size_t)c_out);
done:
    free(wf); free(bf); free(sw); free(qw); free(qx); free(acc);
    return ovf;
}

/* Threads used by the parallel loops (for the harness that times the oracle
 * with all cores and with one); n <= 0 leaves the setting unchanged. */
void oracle_set_threads(int n) {
    if (n > 0) omp_set_num_threads(n);
}

int oracle_get_threads(void) { return omp_get_max_threads(); }
