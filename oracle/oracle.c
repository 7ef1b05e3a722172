/*
 * Plain fp64 CPU oracle for the CosmoFlow-style 3D-CNN training step.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the slow, obviously-correct
 * reference against which the HIP path is checked.  Only the tests, the
 * smoke check and the CPU-baseline leg of the benchmark may load it; the
 * product library never links or calls it, and the two share no code.
 *
 * Every function is the written-out definition of one step of the method:
 *   - 3D convolution as cross-correlation, kernel 3^3, stride 1, zero padding 1
 *     ("same" padding, stride-1 convolutions, no bias: Oyama et al., "The Case
 *     for Strong Scaling in Deep Learning", Sec. IV and Table I);
 *   - its backward-data and backward-weight operators (Mathuriya et al.,
 *     "CosmoFlow", Sec. III-C: forward, backward-data and backward-weight are
 *     separate convolution operators);
 *   - leaky ReLU followed by 2^3 max pooling with stride 2, and its backward;
 *   - fully connected layers with bias, leaky ReLU on all but the last
 *     (Oyama et al., Sec. IV), mean squared error loss (Oyama et al., Sec. IV);
 *   - the SGD update W <- W - eta * grad (Oyama et al., Sec. II-A, the
 *     mini-batch SGD equation).
 *
 * Layouts: activations NDHWC (channels innermost), conv weights DHWIO
 * ([kd][kh][kw][cin][cout]), dense weights [in][out], all packed row-major.
 * Loops follow the definitions directly; OpenMP only splits independent output
 * elements across threads, so every output is a plain sequential fp64 sum.
 */
#include <stdint.h>
#include <math.h>
#include <string.h>

typedef int64_t i64;

/* ---------------------------------------------------------------- helpers */

static inline i64 vox_index(i64 n, i64 d, i64 h, i64 w, i64 D, i64 H, i64 W)
{
    return ((n * D + d) * H + h) * W + w;
}

static inline int in_range(i64 v, i64 hi) { return v >= 0 && v < hi; }

/* Number of omp threads actually used (for reporting the CPU baseline). */
#ifdef _OPENMP
#include <omp.h>
int or_num_threads(void) { return omp_get_max_threads(); }
void or_set_num_threads(int n) { if (n > 0) omp_set_num_threads(n); }
#else
int or_num_threads(void) { return 1; }
void or_set_num_threads(int n) { (void)n; }
#endif

/* ------------------------------------------------------ bf16 rounding model
 * bfloat16 keeps the fp32 exponent range (8 exponent bits) and 7 explicit
 * fraction bits, i.e. 8 significant bits for normal numbers.  Values are
 * rounded to the nearest representable one, ties to even.  The smallest
 * normal is 2^-126; below it the spacing is fixed at 2^-133 (subnormals).
 * The oracle uses this only to model the storage points of the bf16 path
 * (activations and activation gradients are stored in bf16).  */
double or_round_bf16(double x)
{
    if (x == 0.0 || isnan(x) || isinf(x)) return x;
    int e;
    frexp(x, &e);                 /* |x| = m * 2^e, 0.5 <= m < 1 */
    int q = e - 8;                /* spacing of 8-significant-bit numbers */
    if (q < -133) q = -133;       /* subnormal spacing */
    double scaled = ldexp(x, -q); /* exact: power-of-two scaling */
    double r = nearbyint(scaled); /* default rounding mode: ties to even */
    double y = ldexp(r, q);
    /* largest finite bf16 is (2 - 2^-7) * 2^127 */
    const double maxbf = ldexp(255.0, 120);
    if (fabs(y) > maxbf) return x > 0 ? INFINITY : -INFINITY;
    return y;
}

void or_round_bf16_array(i64 n, double* x)
{
    #pragma omp parallel for schedule(static)
    for (i64 i = 0; i < n; ++i) x[i] = or_round_bf16(x[i]);
}

void or_round_f32_array(i64 n, double* x)
{
    #pragma omp parallel for schedule(static)
    for (i64 i = 0; i < n; ++i) x[i] = (double)(float)x[i];
}

/* ------------------------------------------------------------- conv3d fwd
 * Y[n,d,h,w,co] = sum_{kd,kh,kw in 0..2} sum_ci X[n,d+kd-1,h+kh-1,w+kw-1,ci]
 *                                                * Wt[kd,kh,kw,ci,co]
 * with X read as zero outside the volume. */
void or_conv3d_fwd(i64 N, i64 D, i64 H, i64 W, i64 Ci, i64 Co,
                   const double* X, const double* Wt, double* Y)
{
    #pragma omp parallel for collapse(3) schedule(static)
    for (i64 n = 0; n < N; ++n)
    for (i64 d = 0; d < D; ++d)
    for (i64 h = 0; h < H; ++h)
    for (i64 w = 0; w < W; ++w)
    for (i64 co = 0; co < Co; ++co) {
        double s = 0.0;
        for (i64 kd = 0; kd < 3; ++kd)
        for (i64 kh = 0; kh < 3; ++kh)
        for (i64 kw = 0; kw < 3; ++kw) {
            i64 id = d + kd - 1, ih = h + kh - 1, iw = w + kw - 1;
            if (!in_range(id, D) || !in_range(ih, H) || !in_range(iw, W)) continue;
            const double* xp = X + vox_index(n, id, ih, iw, D, H, W) * Ci;
            const double* wp = Wt + ((kd * 3 + kh) * 3 + kw) * Ci * Co + co;
            for (i64 ci = 0; ci < Ci; ++ci) s += xp[ci] * wp[ci * Co];
        }
        Y[vox_index(n, d, h, w, D, H, W) * Co + co] = s;
    }
}

/* ------------------------------------------------------- conv3d bwd-data
 * Adjoint of the forward operator with respect to X:
 * dX[n,d,h,w,ci] = sum_{kd,kh,kw} sum_co dY[n,d-kd+1,h-kh+1,w-kw+1,co]
 *                                        * Wt[kd,kh,kw,ci,co]
 * (the output voxel that read input voxel (d,h,w) through tap (kd,kh,kw) is
 * (d-kd+1, h-kh+1, w-kw+1)). */
void or_conv3d_bwd_data(i64 N, i64 D, i64 H, i64 W, i64 Ci, i64 Co,
                        const double* dY, const double* Wt, double* dX)
{
    #pragma omp parallel for collapse(3) schedule(static)
    for (i64 n = 0; n < N; ++n)
    for (i64 d = 0; d < D; ++d)
    for (i64 h = 0; h < H; ++h)
    for (i64 w = 0; w < W; ++w)
    for (i64 ci = 0; ci < Ci; ++ci) {
        double s = 0.0;
        for (i64 kd = 0; kd < 3; ++kd)
        for (i64 kh = 0; kh < 3; ++kh)
        for (i64 kw = 0; kw < 3; ++kw) {
            i64 od = d - kd + 1, oh = h - kh + 1, ow = w - kw + 1;
            if (!in_range(od, D) || !in_range(oh, H) || !in_range(ow, W)) continue;
            const double* gp = dY + vox_index(n, od, oh, ow, D, H, W) * Co;
            const double* wp = Wt + (((kd * 3 + kh) * 3 + kw) * Ci + ci) * Co;
            for (i64 co = 0; co < Co; ++co) s += gp[co] * wp[co];
        }
        dX[vox_index(n, d, h, w, D, H, W) * Ci + ci] = s;
    }
}

/* ----------------------------------------------------- conv3d bwd-weight
 * Adjoint of the forward operator with respect to Wt:
 * dW[kd,kh,kw,ci,co] = sum_{n,d,h,w} X[n,d+kd-1,h+kh-1,w+kw-1,ci] * dY[n,d,h,w,co]
 */
void or_conv3d_bwd_weight(i64 N, i64 D, i64 H, i64 W, i64 Ci, i64 Co,
                          const double* X, const double* dY, double* dW)
{
    #pragma omp parallel for collapse(2) schedule(dynamic)
    for (i64 t = 0; t < 27; ++t)
    for (i64 ci = 0; ci < Ci; ++ci) {
        i64 kd = t / 9, kh = (t / 3) % 3, kw = t % 3;
        for (i64 co = 0; co < Co; ++co) {
            double s = 0.0;
            for (i64 n = 0; n < N; ++n)
            for (i64 d = 0; d < D; ++d)
            for (i64 h = 0; h < H; ++h)
            for (i64 w = 0; w < W; ++w) {
                i64 id = d + kd - 1, ih = h + kh - 1, iw = w + kw - 1;
                if (!in_range(id, D) || !in_range(ih, H) || !in_range(iw, W)) continue;
                s += X[vox_index(n, id, ih, iw, D, H, W) * Ci + ci]
                   * dY[vox_index(n, d, h, w, D, H, W) * Co + co];
            }
            dW[(t * Ci + ci) * Co + co] = s;
        }
    }
}

/* --------------------------------------------- sampled-output conv variants
 * The same three definitions evaluated only at a list of flat output indices,
 * for checking very large tensors one element at a time.  Inputs are fp32
 * arrays holding exactly representable values (bf16 or fp32 data); every
 * product and sum is formed in fp64. */
void or_conv3d_fwd_points(i64 N, i64 D, i64 H, i64 W, i64 Ci, i64 Co,
                          const float* X, const float* Wt,
                          i64 npts, const i64* pts, double* out)
{
    (void)N;
    #pragma omp parallel for schedule(dynamic, 16)
    for (i64 p = 0; p < npts; ++p) {
        i64 flat = pts[p];
        i64 co = flat % Co, v = flat / Co;
        i64 w = v % W, h = (v / W) % H, d = (v / (W * H)) % D, n = v / (W * H * D);
        double s = 0.0;
        for (i64 kd = 0; kd < 3; ++kd)
        for (i64 kh = 0; kh < 3; ++kh)
        for (i64 kw = 0; kw < 3; ++kw) {
            i64 id = d + kd - 1, ih = h + kh - 1, iw = w + kw - 1;
            if (!in_range(id, D) || !in_range(ih, H) || !in_range(iw, W)) continue;
            const float* xp = X + vox_index(n, id, ih, iw, D, H, W) * Ci;
            const float* wp = Wt + ((kd * 3 + kh) * 3 + kw) * Ci * Co + co;
            for (i64 ci = 0; ci < Ci; ++ci) s += (double)xp[ci] * (double)wp[ci * Co];
        }
        out[p] = s;
    }
}

void or_conv3d_bwd_data_points(i64 N, i64 D, i64 H, i64 W, i64 Ci, i64 Co,
                               const float* dY, const float* Wt,
                               i64 npts, const i64* pts, double* out)
{
    (void)N;
    #pragma omp parallel for schedule(dynamic, 16)
    for (i64 p = 0; p < npts; ++p) {
        i64 flat = pts[p];
        i64 ci = flat % Ci, v = flat / Ci;
        i64 w = v % W, h = (v / W) % H, d = (v / (W * H)) % D, n = v / (W * H * D);
        double s = 0.0;
        for (i64 kd = 0; kd < 3; ++kd)
        for (i64 kh = 0; kh < 3; ++kh)
        for (i64 kw = 0; kw < 3; ++kw) {
            i64 od = d - kd + 1, oh = h - kh + 1, ow = w - kw + 1;
            if (!in_range(od, D) || !in_range(oh, H) || !in_range(ow, W)) continue;
            const float* gp = dY + vox_index(n, od, oh, ow, D, H, W) * Co;
            const float* wp = Wt + (((kd * 3 + kh) * 3 + kw) * Ci + ci) * Co;
            for (i64 co = 0; co < Co; ++co) s += (double)gp[co] * (double)wp[co];
        }
        out[p] = s;
    }
}

void or_conv3d_bwd_weight_points(i64 N, i64 D, i64 H, i64 W, i64 Ci, i64 Co,
                                 const float* X, const float* dY,
                                 i64 npts, const i64* pts, double* out)
{
    for (i64 p = 0; p < npts; ++p) {
        i64 flat = pts[p];
        i64 co = flat % Co, ci = (flat / Co) % Ci, t = flat / (Co * Ci);
        i64 kd = t / 9, kh = (t / 3) % 3, kw = t % 3;
        double s = 0.0;
        #pragma omp parallel for collapse(2) reduction(+:s) schedule(static)
        for (i64 n = 0; n < N; ++n)
        for (i64 d = 0; d < D; ++d)
        for (i64 h = 0; h < H; ++h)
        for (i64 w = 0; w < W; ++w) {
            i64 id = d + kd - 1, ih = h + kh - 1, iw = w + kw - 1;
            if (!in_range(id, D) || !in_range(ih, H) || !in_range(iw, W)) continue;
            s += (double)X[vox_index(n, id, ih, iw, D, H, W) * Ci + ci]
               * (double)dY[vox_index(n, d, h, w, D, H, W) * Co + co];
        }
        out[p] = s;
    }
}

/* ------------------------------------------------------------ leaky ReLU
 * lrelu(z) = z if z > 0, slope * z otherwise; its derivative is taken as 1
 * for z > 0 and slope otherwise (the kink at z = 0 gets the slope). */
static inline double lrelu(double z, double slope) { return z > 0.0 ? z : slope * z; }

void or_lrelu_fwd(i64 n, double slope, const double* x, double* y)
{
    #pragma omp parallel for schedule(static)
    for (i64 i = 0; i < n; ++i) y[i] = lrelu(x[i], slope);
}

void or_lrelu_bwd(i64 n, double slope, const double* x, const double* dy, double* dx)
{
    #pragma omp parallel for schedule(static)
    for (i64 i = 0; i < n; ++i) dx[i] = x[i] > 0.0 ? dy[i] : slope * dy[i];
}

/* ------------------------------------ leaky ReLU then 2^3 max pool, stride 2
 * P[n,i,j,k,c] = max over (a,b,e) in {0,1}^3 of lrelu(Z[n,2i+a,2j+b,2k+e,c]).
 * idx records the window position of the maximum as a*4 + b*2 + e, scanning
 * (a,b,e) in lexicographic order and keeping the first strict maximum. */
void or_lrelu_maxpool_fwd(i64 N, i64 D, i64 H, i64 W, i64 C, double slope,
                          const double* Z, double* P, uint8_t* idx)
{
    i64 Dp = D / 2, Hp = H / 2, Wp = W / 2;
    #pragma omp parallel for collapse(3) schedule(static)
    for (i64 n = 0; n < N; ++n)
    for (i64 i = 0; i < Dp; ++i)
    for (i64 j = 0; j < Hp; ++j)
    for (i64 k = 0; k < Wp; ++k)
    for (i64 c = 0; c < C; ++c) {
        double best = -INFINITY;
        int bi = 0;
        for (int a = 0; a < 2; ++a)
        for (int b = 0; b < 2; ++b)
        for (int e = 0; e < 2; ++e) {
            double v = lrelu(Z[vox_index(n, 2 * i + a, 2 * j + b, 2 * k + e, D, H, W) * C + c], slope);
            if (v > best) { best = v; bi = a * 4 + b * 2 + e; }
        }
        i64 o = vox_index(n, i, j, k, Dp, Hp, Wp) * C + c;
        P[o] = best;
        idx[o] = (uint8_t)bi;
    }
}

/* Backward of the block above: the pooled gradient flows only to the window
 * position that produced the maximum, scaled by the leaky-ReLU derivative
 * there (1 if the pooled value is positive, slope otherwise); the other seven
 * positions of the window receive zero. */
void or_maxpool_lrelu_bwd(i64 N, i64 D, i64 H, i64 W, i64 C, double slope,
                          const double* dP, const double* P, const uint8_t* idx,
                          double* dZ)
{
    i64 Dp = D / 2, Hp = H / 2, Wp = W / 2;
    memset(dZ, 0, sizeof(double) * (size_t)(N * D * H * W * C));
    #pragma omp parallel for collapse(3) schedule(static)
    for (i64 n = 0; n < N; ++n)
    for (i64 i = 0; i < Dp; ++i)
    for (i64 j = 0; j < Hp; ++j)
    for (i64 k = 0; k < Wp; ++k)
    for (i64 c = 0; c < C; ++c) {
        i64 o = vox_index(n, i, j, k, Dp, Hp, Wp) * C + c;
        int bi = idx[o];
        int a = (bi >> 2) & 1, b = (bi >> 1) & 1, e = bi & 1;
        double g = P[o] > 0.0 ? dP[o] : slope * dP[o];
        dZ[vox_index(n, 2 * i + a, 2 * j + b, 2 * k + e, D, H, W) * C + c] = g;
    }
}

/* ----------------------------------------------------------- dense layers
 * pre[b,o] = sum_i X[b,i] * Wt[i,o] + bias[o];
 * Y = lrelu(pre) if slope >= 0, else Y = pre (linear last layer). */
void or_dense_fwd(i64 B, i64 In, i64 Out, const double* X, const double* Wt,
                  const double* bias, double slope, double* pre, double* Y)
{
    #pragma omp parallel for collapse(2) schedule(static)
    for (i64 b = 0; b < B; ++b)
    for (i64 o = 0; o < Out; ++o) {
        double s = bias ? bias[o] : 0.0;
        for (i64 i = 0; i < In; ++i) s += X[b * In + i] * Wt[i * Out + o];
        pre[b * Out + o] = s;
        Y[b * Out + o] = slope >= 0.0 ? lrelu(s, slope) : s;
    }
}

/* Chain rule through one dense layer:
 * dpre = dY * lrelu'(pre) (or dY for the linear layer);
 * dW[i,o] = sum_b X[b,i] dpre[b,o];  db[o] = sum_b dpre[b,o];
 * dX[b,i] = sum_o dpre[b,o] Wt[i,o]  (skipped when dX is NULL). */
void or_dense_bwd(i64 B, i64 In, i64 Out, const double* X, const double* Wt,
                  const double* pre, const double* dY, double slope,
                  double* dX, double* dW, double* db)
{
    #pragma omp parallel for schedule(static)
    for (i64 o = 0; o < Out; ++o) {
        double sb = 0.0;
        for (i64 b = 0; b < B; ++b) {
            double g = dY[b * Out + o];
            if (slope >= 0.0 && !(pre[b * Out + o] > 0.0)) g *= slope;
            sb += g;
        }
        db[o] = sb;
    }
    #pragma omp parallel for collapse(2) schedule(static)
    for (i64 i = 0; i < In; ++i)
    for (i64 o = 0; o < Out; ++o) {
        double s = 0.0;
        for (i64 b = 0; b < B; ++b) {
            double g = dY[b * Out + o];
            if (slope >= 0.0 && !(pre[b * Out + o] > 0.0)) g *= slope;
            s += X[b * In + i] * g;
        }
        dW[i * Out + o] = s;
    }
    if (dX) {
        #pragma omp parallel for collapse(2) schedule(static)
        for (i64 b = 0; b < B; ++b)
        for (i64 i = 0; i < In; ++i) {
            double s = 0.0;
            for (i64 o = 0; o < Out; ++o) {
                double g = dY[b * Out + o];
                if (slope >= 0.0 && !(pre[b * Out + o] > 0.0)) g *= slope;
                s += g * Wt[i * Out + o];
            }
            dX[b * In + i] = s;
        }
    }
}

/* ------------------------------------------------------------------- MSE
 * L = (1 / (B*K)) * sum (yhat - t)^2 ;  dyhat = 2 (yhat - t) / (B*K). */
double or_mse(i64 B, i64 K, const double* yhat, const double* t, double* dyhat)
{
    double s = 0.0;
    i64 n = B * K;
    for (i64 i = 0; i < n; ++i) {
        double r = yhat[i] - t[i];
        s += r * r;
        if (dyhat) dyhat[i] = 2.0 * r / (double)n;
    }
    return s / (double)n;
}

/* ------------------------------------------------------------------- SGD
 * W <- W - lr * dW. */
void or_sgd(i64 n, double lr, double* w, const double* dw)
{
    #pragma omp parallel for schedule(static)
    for (i64 i = 0; i < n; ++i) w[i] -= lr * dw[i];
}

/* ------------------------------------------------ strided conv3d, any pad
 * The convolution with stride s and low-side zero padding p (the extended
 * network of Oyama et al., Table I, has one stride-2 convolution, c4, with
 * "same" padding):
 * Y[n,od,oh,ow,co] = sum_{kd,kh,kw in 0..2} sum_ci
 *                      X[n, s*od+kd-p, s*oh+kh-p, s*ow+kw-p, ci] * Wt[kd,kh,kw,ci,co]
 * X [N,D,H,W,Ci] read as zero outside the volume; Y [N,Do,Ho,Wo,Co].
 * With s = 1, p = 1, Do = D (etc.) this is or_conv3d_fwd. */
void or_conv3d_fwd_s(i64 N, i64 D, i64 H, i64 W, i64 Ci, i64 Co, i64 s, i64 p,
                     i64 Do, i64 Ho, i64 Wo, const double* X, const double* Wt, double* Y)
{
    #pragma omp parallel for collapse(3) schedule(static)
    for (i64 n = 0; n < N; ++n)
    for (i64 od = 0; od < Do; ++od)
    for (i64 oh = 0; oh < Ho; ++oh)
    for (i64 ow = 0; ow < Wo; ++ow)
    for (i64 co = 0; co < Co; ++co) {
        double acc = 0.0;
        for (i64 kd = 0; kd < 3; ++kd)
        for (i64 kh = 0; kh < 3; ++kh)
        for (i64 kw = 0; kw < 3; ++kw) {
            i64 id = s * od + kd - p, ih = s * oh + kh - p, iw = s * ow + kw - p;
            if (!in_range(id, D) || !in_range(ih, H) || !in_range(iw, W)) continue;
            const double* xp = X + vox_index(n, id, ih, iw, D, H, W) * Ci;
            const double* wp = Wt + ((kd * 3 + kh) * 3 + kw) * Ci * Co + co;
            for (i64 ci = 0; ci < Ci; ++ci) acc += xp[ci] * wp[ci * Co];
        }
        Y[vox_index(n, od, oh, ow, Do, Ho, Wo) * Co + co] = acc;
    }
}

/* Adjoint in X: input voxel i received tap k from output voxel o exactly
 * when s*o + k - p = i, i.e. o = (i + p - k) / s with no remainder. */
void or_conv3d_bwd_data_s(i64 N, i64 D, i64 H, i64 W, i64 Ci, i64 Co, i64 s, i64 p,
                          i64 Do, i64 Ho, i64 Wo, const double* dY, const double* Wt, double* dX)
{
    #pragma omp parallel for collapse(3) schedule(static)
    for (i64 n = 0; n < N; ++n)
    for (i64 d = 0; d < D; ++d)
    for (i64 h = 0; h < H; ++h)
    for (i64 w = 0; w < W; ++w)
    for (i64 ci = 0; ci < Ci; ++ci) {
        double acc = 0.0;
        for (i64 kd = 0; kd < 3; ++kd)
        for (i64 kh = 0; kh < 3; ++kh)
        for (i64 kw = 0; kw < 3; ++kw) {
            i64 td = d + p - kd, th = h + p - kh, tw = w + p - kw;
            if (td < 0 || th < 0 || tw < 0 || td % s || th % s || tw % s) continue;
            i64 od = td / s, oh = th / s, ow = tw / s;
            if (od >= Do || oh >= Ho || ow >= Wo) continue;
            const double* gp = dY + vox_index(n, od, oh, ow, Do, Ho, Wo) * Co;
            const double* wp = Wt + (((kd * 3 + kh) * 3 + kw) * Ci + ci) * Co;
            for (i64 co = 0; co < Co; ++co) acc += gp[co] * wp[co];
        }
        dX[vox_index(n, d, h, w, D, H, W) * Ci + ci] = acc;
    }
}

/* Adjoint in Wt: dW[kd,kh,kw,ci,co] = sum_{n,o} X[n, s*o+k-p, ci] * dY[n, o, co]. */
void or_conv3d_bwd_weight_s(i64 N, i64 D, i64 H, i64 W, i64 Ci, i64 Co, i64 s, i64 p,
                            i64 Do, i64 Ho, i64 Wo, const double* X, const double* dY, double* dW)
{
    #pragma omp parallel for collapse(2) schedule(dynamic)
    for (i64 t = 0; t < 27; ++t)
    for (i64 ci = 0; ci < Ci; ++ci) {
        i64 kd = t / 9, kh = (t / 3) % 3, kw = t % 3;
        for (i64 co = 0; co < Co; ++co) {
            double acc = 0.0;
            for (i64 n = 0; n < N; ++n)
            for (i64 od = 0; od < Do; ++od)
            for (i64 oh = 0; oh < Ho; ++oh)
            for (i64 ow = 0; ow < Wo; ++ow) {
                i64 id = s * od + kd - p, ih = s * oh + kh - p, iw = s * ow + kw - p;
                if (!in_range(id, D) || !in_range(ih, H) || !in_range(iw, W)) continue;
                acc += X[vox_index(n, id, ih, iw, D, H, W) * Ci + ci]
                     * dY[vox_index(n, od, oh, ow, Do, Ho, Wo) * Co + co];
            }
            dW[(t * Ci + ci) * Co + co] = acc;
        }
    }
}

/* ---------------------------------------------------- 2^3 average pooling
 * CosmoFlow, Sec. III-A and III-C: stride-2 average pooling, each channel
 * separately, constant weights 1/(KS)^3 = 1/8 for KS = 2:
 * P[n,i,j,k,c] = (1/8) sum_{a,b,e in {0,1}} Z[n,2i+a,2j+b,2k+e,c]. */
void or_avgpool_fwd(i64 N, i64 D, i64 H, i64 W, i64 C, const double* Z, double* P)
{
    i64 Dp = D / 2, Hp = H / 2, Wp = W / 2;
    #pragma omp parallel for collapse(3) schedule(static)
    for (i64 n = 0; n < N; ++n)
    for (i64 i = 0; i < Dp; ++i)
    for (i64 j = 0; j < Hp; ++j)
    for (i64 k = 0; k < Wp; ++k)
    for (i64 c = 0; c < C; ++c) {
        double acc = 0.0;
        for (i64 a = 0; a < 2; ++a)
        for (i64 b = 0; b < 2; ++b)
        for (i64 e = 0; e < 2; ++e)
            acc += Z[vox_index(n, 2 * i + a, 2 * j + b, 2 * k + e, D, H, W) * C + c];
        P[vox_index(n, i, j, k, Dp, Hp, Wp) * C + c] = acc / 8.0;
    }
}

/* Backward: every window position receives dP / 8. */
void or_avgpool_bwd(i64 N, i64 D, i64 H, i64 W, i64 C, const double* dP, double* dZ)
{
    i64 Dp = D / 2, Hp = H / 2, Wp = W / 2;
    #pragma omp parallel for collapse(3) schedule(static)
    for (i64 n = 0; n < N; ++n)
    for (i64 d = 0; d < D; ++d)
    for (i64 h = 0; h < H; ++h)
    for (i64 w = 0; w < W; ++w)
    for (i64 c = 0; c < C; ++c)
        dZ[vox_index(n, d, h, w, D, H, W) * C + c] = dP[vox_index(n, d / 2, h / 2, w / 2, Dp, Hp, Wp) * C + c] / 8.0;
}
