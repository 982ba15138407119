/*
 * oracle.c -- plain float64 CPU reference for the Hyena operator's long
 * convolution chain (1D causal, 2D and 3D non-causal).
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the GPU library links, includes or
 * calls this file, and this file uses nothing from the GPU library.  Only the
 * test suite, the package smoke check and the benchmark's CPU-baseline leg may
 * load it.  It is deliberately slow and literal: every function is the
 * definition written out, with no blocking, fusion or reordering beyond what
 * the definition states.
 *
 * Sources (the pages this follows):
 *   [P1] "Week 11: Hyena, Long Convolution, and Linear Attention", sections
 *        "The Hyena operator" (order-N chain of long convolutions and gates)
 *        and "FFTConv" (causal sum plus the feedthrough b_d u_{b,t,d};
 *        zero-pad to twice the length, multiply spectra, invert, truncate).
 *   [P2] "Hyena -- Long Convolutions Math", sections "The primitive" (causal
 *        sum, depthwise over channels), "The Toeplitz picture" (order-2 form
 *        x2 . (h2 * (x1 . (h1 * v)))), "The convolution theorem" and
 *        "Linear vs circular" (padding to 2N rounded up to a power of two,
 *        keep the first N outputs), "Counting the cost" (radix-2 FFT).
 *   [P3] "How HyenaND works", section "The convolution theorem (FFT)" (the
 *        ND FFT convolution on the native grid) and the worked trace's
 *        zero padding with is_causal=False (non-causal linear 2D conv).
 *
 * Layouts (row-major, channels last):
 *   1D: z, u, gates[n], y : [B][N][d];  h : [order][d][N];  D : [order][d]
 *   2D: z, u, gates[n], y : [B][X][Y][d];
 *       K : [order][d][2X-1][2Y-1], tap at signed offset (i, j) stored at
 *       index (i + X - 1, j + Y - 1);  D : [order][d]
 *   3D: z, u, gates[n], y : [B][X][Y][Z][d];
 *       K : [order][d][2X-1][2Y-1][2Z-1], offset (i, j, l) at
 *       (i + X - 1, j + Y - 1, l + Z - 1)
 *
 * Parity pins (all in tests/): the printed worked example of [P2] "Linear vs
 * circular"; numpy.convolve / numpy.fft / the O(M^2) DFT definition; closed
 * forms (impulse, step response of a damped sinusoid, extreme tap, 2D delta
 * shifts, separable kernels); invariants (causality, linearity, shift
 * equivariance, channel independence); direct vs FFT routes.
 */
#include <math.h>
#include <omp.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#ifndef M_PI
#define M_PI 3.14159265358979323846
#endif

/* Threads the OpenMP loops below will use (reported beside oracle timings). */
int oracle_num_threads(void) { return omp_get_max_threads(); }

static int64_t next_pow2(int64_t n)
{
    int64_t m = 1;
    while (m < n) m <<= 1;
    return m;
}

static int is_pow2(int64_t n) { return n > 0 && (n & (n - 1)) == 0; }

/* ------------------------------------------------------------------------ */
/* Radix-2 FFT ([P2] "Counting the cost")                                    */
/* ------------------------------------------------------------------------ */

/*
 * In-place iterative radix-2 decimation-in-time DFT of length n (a power of
 * two).  sign = -1 computes X[k] = sum_t x[t] exp(-2 pi i k t / n);
 * sign = +1 computes the same sum with exp(+2 pi i k t / n) (no 1/n scale).
 * Bit-reversal permutation first, then log2(n) butterfly stages.  Every
 * twiddle is computed from its own angle with cos/sin in double; there is no
 * recurrence.  Returns 0, or -1 if n is not a power of two.
 */
int oracle_fft(int64_t n, double* re, double* im, int sign)
{
    if (!is_pow2(n)) return -1;
    /* bit reversal */
    for (int64_t i = 1, j = 0; i < n; ++i) {
        int64_t bit = n >> 1;
        for (; j & bit; bit >>= 1) j ^= bit;
        j ^= bit;
        if (i < j) {
            double t = re[i]; re[i] = re[j]; re[j] = t;
            t = im[i]; im[i] = im[j]; im[j] = t;
        }
    }
    for (int64_t len = 2; len <= n; len <<= 1) {
        int64_t half = len >> 1;
        for (int64_t start = 0; start < n; start += len) {
            for (int64_t k = 0; k < half; ++k) {
                double ang = sign * 2.0 * M_PI * (double)k / (double)len;
                double wr = cos(ang), wi = sin(ang);
                int64_t a = start + k, b = start + k + half;
                double tr = re[b] * wr - im[b] * wi;
                double ti = re[b] * wi + im[b] * wr;
                re[b] = re[a] - tr;
                im[b] = im[a] - ti;
                re[a] += tr;
                im[a] += ti;
            }
        }
    }
    return 0;
}

/* ------------------------------------------------------------------------ */
/* 1D causal depthwise convolution with skip                                 */
/* ------------------------------------------------------------------------ */

/*
 * Direct sum ([P2] "The primitive"; [P1] "FFTConv" equation):
 *   w[b,t,c] = sum_{s=0}^{t} h[c,s] * z[b,t-s,c]  +  D[c] * z[b,t,c]
 * summed in ascending s.  h holds N taps per channel; tap s multiplies the
 * input s steps in the past (s = 0 is the current token).
 */
void oracle_causal_conv_direct(int64_t B, int64_t N, int64_t d, const double* z,
                               const double* h, const double* D, double* w)
{
#pragma omp parallel for collapse(2) schedule(dynamic)
    for (int64_t b = 0; b < B; ++b)
        for (int64_t c = 0; c < d; ++c)
            for (int64_t t = 0; t < N; ++t) {
                double acc = 0.0;
                for (int64_t s = 0; s <= t; ++s)
                    acc += h[c * N + s] * z[(b * N + (t - s)) * d + c];
                w[(b * N + t) * d + c] = acc + D[c] * z[(b * N + t) * d + c];
            }
}

/*
 * The same result through the convolution theorem ([P2] "The convolution
 * theorem", "Linear vs circular"; [P1] "FFTConv"): pad z[b,:,c] and h[c,:]
 * with zeros to M = the power of two >= 2N, transform both, multiply bin by
 * bin, invert with the 1/M scale, keep the first N outputs, add D[c] z.
 * Real data is carried as complex with zero imaginary part.
 */
int oracle_causal_conv_fft(int64_t B, int64_t N, int64_t d, const double* z,
                           const double* h, const double* D, double* w)
{
    const int64_t M = next_pow2(2 * N);
    int fail = 0;
#pragma omp parallel
    {
        double* xr = (double*)malloc(sizeof(double) * M);
        double* xi = (double*)malloc(sizeof(double) * M);
        double* hr = (double*)malloc(sizeof(double) * M);
        double* hi = (double*)malloc(sizeof(double) * M);
        if (!xr || !xi || !hr || !hi) {
#pragma omp atomic write
            fail = 1;
        } else {
#pragma omp for collapse(2) schedule(dynamic)
            for (int64_t b = 0; b < B; ++b)
                for (int64_t c = 0; c < d; ++c) {
                    for (int64_t t = 0; t < M; ++t) {
                        xr[t] = t < N ? z[(b * N + t) * d + c] : 0.0;
                        hr[t] = t < N ? h[c * N + t] : 0.0;
                        xi[t] = 0.0;
                        hi[t] = 0.0;
                    }
                    oracle_fft(M, xr, xi, -1);
                    oracle_fft(M, hr, hi, -1);
                    for (int64_t k = 0; k < M; ++k) {
                        double pr = xr[k] * hr[k] - xi[k] * hi[k];
                        double pi = xr[k] * hi[k] + xi[k] * hr[k];
                        xr[k] = pr;
                        xi[k] = pi;
                    }
                    oracle_fft(M, xr, xi, +1);
                    for (int64_t t = 0; t < N; ++t)
                        w[(b * N + t) * d + c] =
                            xr[t] / (double)M + D[c] * z[(b * N + t) * d + c];
                }
        }
        free(xr); free(xi); free(hr); free(hi);
    }
    return fail ? -1 : 0;
}

/*
 * Length-N circular convolution with no padding, kept only to show what the
 * padding prevents ([P2] "Linear vs circular": the wrapped term at t = 0).
 *   w[b,t,c] = sum_{s=0}^{N-1} h[c,(t-s) mod N] * z[b,s,c]   (N a power of 2)
 */
int oracle_circular_conv_fft(int64_t B, int64_t N, int64_t d, const double* z,
                             const double* h, double* w)
{
    if (!is_pow2(N)) return -1;
    double* xr = (double*)malloc(sizeof(double) * N);
    double* xi = (double*)malloc(sizeof(double) * N);
    double* hr = (double*)malloc(sizeof(double) * N);
    double* hi = (double*)malloc(sizeof(double) * N);
    if (!xr || !xi || !hr || !hi) { free(xr); free(xi); free(hr); free(hi); return -1; }
    for (int64_t b = 0; b < B; ++b)
        for (int64_t c = 0; c < d; ++c) {
            for (int64_t t = 0; t < N; ++t) {
                xr[t] = z[(b * N + t) * d + c]; xi[t] = 0.0;
                hr[t] = h[c * N + t];          hi[t] = 0.0;
            }
            oracle_fft(N, xr, xi, -1);
            oracle_fft(N, hr, hi, -1);
            for (int64_t k = 0; k < N; ++k) {
                double pr = xr[k] * hr[k] - xi[k] * hi[k];
                double pi = xr[k] * hi[k] + xi[k] * hr[k];
                xr[k] = pr; xi[k] = pi;
            }
            oracle_fft(N, xr, xi, +1);
            for (int64_t t = 0; t < N; ++t) w[(b * N + t) * d + c] = xr[t] / (double)N;
        }
    free(xr); free(xi); free(hr); free(hi);
    return 0;
}

/*
 * Order-N Hyena chain ([P1] "The Hyena operator"; [P2] "The Toeplitz
 * picture", order-2 form):
 *   z_0 = u;  z_n = gates[n-1] . (h_n * z_{n-1} + D_n z_{n-1});  y = z_order
 * The gate multiplies the output of each convolution (gate n after conv n).
 * method 0 = direct sum, 1 = FFT route.  Returns 0 on success.
 */
int oracle_hyena1d(int64_t B, int64_t N, int64_t d, int32_t order, const double* u,
                   const double* gates, const double* h, const double* D, double* y,
                   int32_t method)
{
    const int64_t E = B * N * d;
    double* z = (double*)malloc(sizeof(double) * E);
    double* w = (double*)malloc(sizeof(double) * E);
    if (!z || !w) { free(z); free(w); return -1; }
    memcpy(z, u, sizeof(double) * E);
    int rc = 0;
    for (int32_t n = 0; n < order && rc == 0; ++n) {
        const double* hn = h + (int64_t)n * d * N;
        const double* Dn = D + (int64_t)n * d;
        if (method == 0)
            oracle_causal_conv_direct(B, N, d, z, hn, Dn, w);
        else
            rc = oracle_causal_conv_fft(B, N, d, z, hn, Dn, w);
        const double* g = gates + (int64_t)n * E;
        for (int64_t i = 0; i < E; ++i) z[i] = g[i] * w[i];
    }
    if (rc == 0) memcpy(y, z, sizeof(double) * E);
    free(z); free(w);
    return rc;
}

/* ------------------------------------------------------------------------ */
/* 2D non-causal convolution with skip ([P3])                                */
/* ------------------------------------------------------------------------ */

/*
 * Direct sum over the whole grid (linear, zero outside the grid, "same"
 * output positions):
 *   w[b,p,q,c] = sum_{p'<X} sum_{q'<Y} K[c][p-p'][q-q'] z[b,p',q',c] + D[c] z[b,p,q,c]
 * where K[c][i][j] is the tap at signed offset (i, j).
 */
void oracle_conv2d_direct(int64_t B, int64_t X, int64_t Y, int64_t d, const double* z,
                          const double* K, const double* D, double* w)
{
    const int64_t KX = 2 * X - 1, KY = 2 * Y - 1;
#pragma omp parallel for collapse(3) schedule(dynamic)
    for (int64_t b = 0; b < B; ++b)
        for (int64_t c = 0; c < d; ++c)
            for (int64_t p = 0; p < X; ++p)
                for (int64_t q = 0; q < Y; ++q) {
                    double acc = 0.0;
                    for (int64_t pp = 0; pp < X; ++pp)
                        for (int64_t qq = 0; qq < Y; ++qq)
                            acc += K[(c * KX + (p - pp + X - 1)) * KY + (q - qq + Y - 1)] *
                                   z[((b * X + pp) * Y + qq) * d + c];
                    const int64_t o = ((b * X + p) * Y + q) * d + c;
                    w[o] = acc + D[c] * z[o];
                }
}

/*
 * The same through the 2D convolution theorem: grid and taps placed in a
 * P1 x P2 periodic array, P1 = power of two >= 2X, P2 = power of two >= 2Y;
 * the tap at offset (i, j) goes to (i mod P1, j mod P2).  2D DFT = 1D DFTs
 * along rows, then along columns.  Bin-by-bin product, inverse with 1/(P1 P2),
 * keep [0,X) x [0,Y), add D z.  Because P1 >= 2X - 1 and P2 >= 2Y - 1 no
 * offset that reaches the kept window aliases onto another.
 */
static void fft2d(int64_t P1, int64_t P2, double* re, double* im, int sign,
                  double* colr, double* coli)
{
    for (int64_t r = 0; r < P1; ++r) oracle_fft(P2, re + r * P2, im + r * P2, sign);
    for (int64_t col = 0; col < P2; ++col) {
        for (int64_t r = 0; r < P1; ++r) { colr[r] = re[r * P2 + col]; coli[r] = im[r * P2 + col]; }
        oracle_fft(P1, colr, coli, sign);
        for (int64_t r = 0; r < P1; ++r) { re[r * P2 + col] = colr[r]; im[r * P2 + col] = coli[r]; }
    }
}

int oracle_conv2d_fft(int64_t B, int64_t X, int64_t Y, int64_t d, const double* z,
                      const double* K, const double* D, double* w)
{
    const int64_t P1 = next_pow2(2 * X), P2 = next_pow2(2 * Y);
    const int64_t KX = 2 * X - 1, KY = 2 * Y - 1;
    const int64_t S = P1 * P2;
    int fail = 0;
#pragma omp parallel
    {
        double* xr = (double*)malloc(sizeof(double) * S);
        double* xi = (double*)malloc(sizeof(double) * S);
        double* kr = (double*)malloc(sizeof(double) * S);
        double* ki = (double*)malloc(sizeof(double) * S);
        double* cr = (double*)malloc(sizeof(double) * P1);
        double* ci = (double*)malloc(sizeof(double) * P1);
        if (!xr || !xi || !kr || !ki || !cr || !ci) {
#pragma omp atomic write
            fail = 1;
        } else {
#pragma omp for collapse(2) schedule(dynamic)
            for (int64_t b = 0; b < B; ++b)
                for (int64_t c = 0; c < d; ++c) {
                    memset(xr, 0, sizeof(double) * S); memset(xi, 0, sizeof(double) * S);
                    memset(kr, 0, sizeof(double) * S); memset(ki, 0, sizeof(double) * S);
                    for (int64_t p = 0; p < X; ++p)
                        for (int64_t q = 0; q < Y; ++q)
                            xr[p * P2 + q] = z[((b * X + p) * Y + q) * d + c];
                    for (int64_t i = -(X - 1); i <= X - 1; ++i)
                        for (int64_t j = -(Y - 1); j <= Y - 1; ++j) {
                            int64_t ri = (i + P1) % P1, rj = (j + P2) % P2;
                            kr[ri * P2 + rj] = K[(c * KX + (i + X - 1)) * KY + (j + Y - 1)];
                        }
                    fft2d(P1, P2, xr, xi, -1, cr, ci);
                    fft2d(P1, P2, kr, ki, -1, cr, ci);
                    for (int64_t k = 0; k < S; ++k) {
                        double pr = xr[k] * kr[k] - xi[k] * ki[k];
                        double pi = xr[k] * ki[k] + xi[k] * kr[k];
                        xr[k] = pr; xi[k] = pi;
                    }
                    fft2d(P1, P2, xr, xi, +1, cr, ci);
                    for (int64_t p = 0; p < X; ++p)
                        for (int64_t q = 0; q < Y; ++q) {
                            const int64_t o = ((b * X + p) * Y + q) * d + c;
                            w[o] = xr[p * P2 + q] / (double)S + D[c] * z[o];
                        }
                }
        }
        free(xr); free(xi); free(kr); free(ki); free(cr); free(ci);
    }
    return fail ? -1 : 0;
}

/*
 * Order-N chain on a 2D grid: the same gating structure as the 1D chain,
 * with the non-causal 2D convolution in place of the causal 1D one.
 */
int oracle_hyena2d(int64_t B, int64_t X, int64_t Y, int64_t d, int32_t order, const double* u,
                   const double* gates, const double* K, const double* D, double* y,
                   int32_t method)
{
    const int64_t E = B * X * Y * d;
    const int64_t KS = (2 * X - 1) * (2 * Y - 1);
    double* z = (double*)malloc(sizeof(double) * E);
    double* w = (double*)malloc(sizeof(double) * E);
    if (!z || !w) { free(z); free(w); return -1; }
    memcpy(z, u, sizeof(double) * E);
    int rc = 0;
    for (int32_t n = 0; n < order && rc == 0; ++n) {
        const double* Kn = K + (int64_t)n * d * KS;
        const double* Dn = D + (int64_t)n * d;
        if (method == 0)
            oracle_conv2d_direct(B, X, Y, d, z, Kn, Dn, w);
        else
            rc = oracle_conv2d_fft(B, X, Y, d, z, Kn, Dn, w);
        const double* g = gates + (int64_t)n * E;
        for (int64_t i = 0; i < E; ++i) z[i] = g[i] * w[i];
    }
    if (rc == 0) memcpy(y, z, sizeof(double) * E);
    free(z); free(w);
    return rc;
}

/* ------------------------------------------------------------------------ */
/* 3D non-causal convolution with skip ([P3]: the same operator on a native  */
/* 3D grid; the convolution theorem holds along each axis)                   */
/* ------------------------------------------------------------------------ */

/*
 * Direct sum over the whole X x Y x Z grid (zero outside it, "same" output
 * positions):
 *   w[b,p,q,r,c] = sum_{p',q',r'} K[c][p-p'][q-q'][r-r'] z[b,p',q',r',c] + D[c] z[b,p,q,r,c]
 * K[c] holds the tap at signed offset (i, j, l) at index
 * (i + X - 1, j + Y - 1, l + Z - 1) of a (2X-1) x (2Y-1) x (2Z-1) array.
 */
void oracle_conv3d_direct(int64_t B, int64_t X, int64_t Y, int64_t Z, int64_t d,
                          const double* z, const double* K, const double* D, double* w)
{
    const int64_t KX = 2 * X - 1, KY = 2 * Y - 1, KZ = 2 * Z - 1;
#pragma omp parallel for collapse(3) schedule(dynamic)
    for (int64_t b = 0; b < B; ++b)
        for (int64_t c = 0; c < d; ++c)
            for (int64_t p = 0; p < X; ++p)
                for (int64_t q = 0; q < Y; ++q)
                    for (int64_t r = 0; r < Z; ++r) {
                        double acc = 0.0;
                        for (int64_t pp = 0; pp < X; ++pp)
                            for (int64_t qq = 0; qq < Y; ++qq)
                                for (int64_t rr = 0; rr < Z; ++rr)
                                    acc += K[((c * KX + (p - pp + X - 1)) * KY + (q - qq + Y - 1)) * KZ +
                                             (r - rr + Z - 1)] *
                                           z[(((b * X + pp) * Y + qq) * Z + rr) * d + c];
                        const int64_t o = (((b * X + p) * Y + q) * Z + r) * d + c;
                        w[o] = acc + D[c] * z[o];
                    }
}

/* 3D DFT of a P1 x P2 x P3 array (r fastest): 1D DFTs along r, then q, then p. */
static void fft3d(int64_t P1, int64_t P2, int64_t P3, double* re, double* im, int sign,
                  double* lr, double* li)
{
    for (int64_t row = 0; row < P1 * P2; ++row) oracle_fft(P3, re + row * P3, im + row * P3, sign);
    for (int64_t p = 0; p < P1; ++p)
        for (int64_t r = 0; r < P3; ++r) {
            const int64_t base = p * P2 * P3 + r;
            for (int64_t q = 0; q < P2; ++q) { lr[q] = re[base + q * P3]; li[q] = im[base + q * P3]; }
            oracle_fft(P2, lr, li, sign);
            for (int64_t q = 0; q < P2; ++q) { re[base + q * P3] = lr[q]; im[base + q * P3] = li[q]; }
        }
    for (int64_t qr = 0; qr < P2 * P3; ++qr) {
        for (int64_t p = 0; p < P1; ++p) { lr[p] = re[p * P2 * P3 + qr]; li[p] = im[p * P2 * P3 + qr]; }
        oracle_fft(P1, lr, li, sign);
        for (int64_t p = 0; p < P1; ++p) { re[p * P2 * P3 + qr] = lr[p]; im[p * P2 * P3 + qr] = li[p]; }
    }
}

/*
 * The same through the 3D convolution theorem: grid and taps in a
 * P1 x P2 x P3 periodic array (each a power of two >= twice the side), the
 * tap at offset (i, j, l) at (i mod P1, j mod P2, l mod P3); bin-by-bin
 * product; inverse with 1/(P1 P2 P3); keep the input grid; add D z.
 */
int oracle_conv3d_fft(int64_t B, int64_t X, int64_t Y, int64_t Z, int64_t d, const double* z,
                      const double* K, const double* D, double* w)
{
    const int64_t P1 = next_pow2(2 * X), P2 = next_pow2(2 * Y), P3 = next_pow2(2 * Z);
    const int64_t KX = 2 * X - 1, KY = 2 * Y - 1, KZ = 2 * Z - 1;
    const int64_t S = P1 * P2 * P3;
    const int64_t Lmax = P1 > P2 ? (P1 > P3 ? P1 : P3) : (P2 > P3 ? P2 : P3);
    int fail = 0;
#pragma omp parallel
    {
        double* xr = (double*)malloc(sizeof(double) * S);
        double* xi = (double*)malloc(sizeof(double) * S);
        double* kr = (double*)malloc(sizeof(double) * S);
        double* ki = (double*)malloc(sizeof(double) * S);
        double* lr = (double*)malloc(sizeof(double) * Lmax);
        double* li = (double*)malloc(sizeof(double) * Lmax);
        if (!xr || !xi || !kr || !ki || !lr || !li) {
#pragma omp atomic write
            fail = 1;
        } else {
#pragma omp for collapse(2) schedule(dynamic)
            for (int64_t b = 0; b < B; ++b)
                for (int64_t c = 0; c < d; ++c) {
                    memset(xr, 0, sizeof(double) * S); memset(xi, 0, sizeof(double) * S);
                    memset(kr, 0, sizeof(double) * S); memset(ki, 0, sizeof(double) * S);
                    for (int64_t p = 0; p < X; ++p)
                        for (int64_t q = 0; q < Y; ++q)
                            for (int64_t r = 0; r < Z; ++r)
                                xr[(p * P2 + q) * P3 + r] = z[(((b * X + p) * Y + q) * Z + r) * d + c];
                    for (int64_t i = -(X - 1); i <= X - 1; ++i)
                        for (int64_t j = -(Y - 1); j <= Y - 1; ++j)
                            for (int64_t l = -(Z - 1); l <= Z - 1; ++l) {
                                const int64_t ri = (i + P1) % P1, rj = (j + P2) % P2, rl = (l + P3) % P3;
                                kr[(ri * P2 + rj) * P3 + rl] =
                                    K[((c * KX + (i + X - 1)) * KY + (j + Y - 1)) * KZ + (l + Z - 1)];
                            }
                    fft3d(P1, P2, P3, xr, xi, -1, lr, li);
                    fft3d(P1, P2, P3, kr, ki, -1, lr, li);
                    for (int64_t k = 0; k < S; ++k) {
                        const double pr = xr[k] * kr[k] - xi[k] * ki[k];
                        const double pi = xr[k] * ki[k] + xi[k] * kr[k];
                        xr[k] = pr; xi[k] = pi;
                    }
                    fft3d(P1, P2, P3, xr, xi, +1, lr, li);
                    for (int64_t p = 0; p < X; ++p)
                        for (int64_t q = 0; q < Y; ++q)
                            for (int64_t r = 0; r < Z; ++r) {
                                const int64_t o = (((b * X + p) * Y + q) * Z + r) * d + c;
                                w[o] = xr[(p * P2 + q) * P3 + r] / (double)S + D[c] * z[o];
                            }
                }
        }
        free(xr); free(xi); free(kr); free(ki); free(lr); free(li);
    }
    return fail ? -1 : 0;
}

/* Order-N chain on a 3D grid, gated as in 1D and 2D. */
int oracle_hyena3d(int64_t B, int64_t X, int64_t Y, int64_t Z, int64_t d, int32_t order,
                   const double* u, const double* gates, const double* K, const double* D,
                   double* y, int32_t method)
{
    const int64_t E = B * X * Y * Z * d;
    const int64_t KS = (2 * X - 1) * (2 * Y - 1) * (2 * Z - 1);
    double* z = (double*)malloc(sizeof(double) * E);
    double* w = (double*)malloc(sizeof(double) * E);
    if (!z || !w) { free(z); free(w); return -1; }
    memcpy(z, u, sizeof(double) * E);
    int rc = 0;
    for (int32_t n = 0; n < order && rc == 0; ++n) {
        const double* Kn = K + (int64_t)n * d * KS;
        const double* Dn = D + (int64_t)n * d;
        if (method == 0)
            oracle_conv3d_direct(B, X, Y, Z, d, z, Kn, Dn, w);
        else
            rc = oracle_conv3d_fft(B, X, Y, Z, d, z, Kn, Dn, w);
        const double* g = gates + (int64_t)n * E;
        for (int64_t i = 0; i < E; ++i) z[i] = g[i] * w[i];
    }
    if (rc == 0) memcpy(y, z, sizeof(double) * E);
    free(z); free(w);
    return rc;
}

/* ------------------------------------------------------------------------ */
/* Implicit filter ([P2] "Implicit filters: an MLP over positions" and "The  */
/* decay window")                                                            */
/* ------------------------------------------------------------------------ */

/*
 * Filter taps generated by a small MLP over positions instead of stored:
 *   h_n[c, t] = exp(-alpha[n][c] t) * FFN(gamma(t))[n d + c],  t = 0..N-1
 * gamma(t) is the positional encoding [t/N, cos(2 pi j t/N), sin(2 pi j t/N)]
 * for j = 1..K (m = 2K + 1 features, in that order: t/N first, then for each
 * j its cosine and its sine).  FFN : R^m -> R^(order d) is shared over all t:
 *   z1 = sin(omega (W1 gamma + b1))      W1 [H][m],  b1 [H]
 *   z2 = sin(omega (W2 z1 + b2))         W2 [H][H],  b2 [H]
 *   out = W3 z2 + b3                     W3 [order d][H], b3 [order d]
 * (the sine activations of [P3] "1. An implicit filter", whose filter network
 * is a sine MLP; the pages leave depth and width open: two hidden layers).
 * Output h [order][d][N].
 */
void oracle_implicit_filter(int64_t N, int64_t d, int32_t order, int32_t K, int32_t H,
                            double omega, const double* W1, const double* b1,
                            const double* W2, const double* b2, const double* W3,
                            const double* b3, const double* alpha, double* h)
{
    const int64_t m = 2 * (int64_t)K + 1;
    const int64_t nout = (int64_t)order * d;
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < N; ++t) {
        double g[2 * 64 + 1], z1[256], z2[256];
        const double tn = (double)t / (double)N;
        g[0] = tn;
        for (int64_t j = 1; j <= K; ++j) {
            g[2 * j - 1] = cos(2.0 * M_PI * (double)j * tn);
            g[2 * j] = sin(2.0 * M_PI * (double)j * tn);
        }
        for (int64_t i = 0; i < H; ++i) {
            double acc = b1[i];
            for (int64_t k = 0; k < m; ++k) acc += W1[i * m + k] * g[k];
            z1[i] = sin(omega * acc);
        }
        for (int64_t i = 0; i < H; ++i) {
            double acc = b2[i];
            for (int64_t k = 0; k < H; ++k) acc += W2[i * H + k] * z1[k];
            z2[i] = sin(omega * acc);
        }
        for (int64_t o = 0; o < nout; ++o) {
            double acc = b3[o];
            for (int64_t k = 0; k < H; ++k) acc += W3[o * H + k] * z2[k];
            h[o * N + t] = exp(-alpha[o] * (double)t) * acc;
        }
    }
}

/* ------------------------------------------------------------------------ */
/* Periodic (circular) boundary: the unpadded convolution as an operator     */
/* ([P2] "Linear vs circular" contrasts it with the padded, causal one; the  */
/* ops layer of [P3] lists periodic boundaries as a variant)                  */
/* ------------------------------------------------------------------------ */

/*
 * w[b,t,c] = sum_{s=0}^{N-1} h[c,s] z[b,(t-s) mod N,c] + D[c] z[b,t,c]
 * (the sum written out; any N).
 */
void oracle_circular_conv_direct(int64_t B, int64_t N, int64_t d, const double* z,
                                 const double* h, const double* D, double* w)
{
#pragma omp parallel for collapse(2) schedule(static)
    for (int64_t b = 0; b < B; ++b)
        for (int64_t c = 0; c < d; ++c)
            for (int64_t t = 0; t < N; ++t) {
                double acc = 0.0;
                for (int64_t s = 0; s < N; ++s) {
                    int64_t r = (t - s) % N;
                    if (r < 0) r += N;
                    acc += h[c * N + s] * z[(b * N + r) * d + c];
                }
                w[(b * N + t) * d + c] = acc + D[c] * z[(b * N + t) * d + c];
            }
}

/*
 * The order-N chain with periodic convolutions:
 *   z_n = gates[n-1] . (h_n (*)_N z_{n-1} + D_n z_{n-1})
 * method 0 = direct sum, 1 = FFT route (oracle_circular_conv_fft + D z;
 * N a power of two).
 */
int oracle_hyena1d_circular(int64_t B, int64_t N, int64_t d, int32_t order, const double* u,
                            const double* gates, const double* h, const double* D, double* y,
                            int32_t method)
{
    const int64_t E = B * N * d;
    double* z = (double*)malloc(sizeof(double) * E);
    double* w = (double*)malloc(sizeof(double) * E);
    if (!z || !w) { free(z); free(w); return -1; }
    memcpy(z, u, sizeof(double) * E);
    int rc = 0;
    for (int32_t n = 0; n < order && rc == 0; ++n) {
        const double* hn = h + (int64_t)n * d * N;
        const double* Dn = D + (int64_t)n * d;
        if (method == 0) {
            oracle_circular_conv_direct(B, N, d, z, hn, Dn, w);
        } else {
            rc = oracle_circular_conv_fft(B, N, d, z, hn, w);
            if (rc == 0)
                for (int64_t i = 0; i < E; ++i) w[i] += Dn[i % d] * z[i];
        }
        const double* g = gates + (int64_t)n * E;
        for (int64_t i = 0; i < E; ++i) z[i] = g[i] * w[i];
    }
    if (rc == 0) memcpy(y, z, sizeof(double) * E);
    free(z); free(w);
    return rc;
}

/* ------------------------------------------------------------------------ */
/* HyenaND block ([P3] "Putting it together: the HyenaND operator" and "A   */
/* worked trace"): depthwise 3x3 short convolution on q, k, v; inner gate   */
/* Z = q . SiLU(k); the 2D long convolution; outer gate SiLU(v)              */
/* ------------------------------------------------------------------------ */

static double silu(double x) { return x / (1.0 + exp(-x)); }

/*
 * Depthwise 3x3 cross-correlation with zero padding of one (a grouped
 * Conv2d with kernel 3, padding 1, groups = channels):
 *   o[b,p,q,c] = bias[c] + sum_{a,e in -1..1} w[c][a+1][e+1] x[b,p+a,q+e,c]
 * x and o [B][X][Y][d]; w [d][3][3]; bias [d] or NULL.
 */
void oracle_dwconv3x3(int64_t B, int64_t X, int64_t Y, int64_t d, const double* x,
                      const double* w, const double* bias, double* o)
{
#pragma omp parallel for collapse(2) schedule(static)
    for (int64_t b = 0; b < B; ++b)
        for (int64_t p = 0; p < X; ++p)
            for (int64_t q = 0; q < Y; ++q)
                for (int64_t c = 0; c < d; ++c) {
                    double acc = bias ? bias[c] : 0.0;
                    for (int a = -1; a <= 1; ++a)
                        for (int e = -1; e <= 1; ++e) {
                            const int64_t pp = p + a, qq = q + e;
                            if (pp < 0 || pp >= X || qq < 0 || qq >= Y) continue;
                            acc += w[(c * 3 + (a + 1)) * 3 + (e + 1)] *
                                   x[((b * X + pp) * Y + qq) * d + c];
                        }
                    o[((b * X + p) * Y + q) * d + c] = acc;
                }
}

/*
 * One HyenaND mixer with a single long convolution:
 *   qs, ks, vs = dwconv3x3(q | k | v)     (sw [3][d][3][3], sb [3][d] or NULL)
 *   z = qs . SiLU(ks)
 *   y = SiLU(vs) . (K * z + D z)          (K as in oracle_conv2d_direct)
 * method 0 = direct 2D sum, 1 = FFT route.
 */
int oracle_hyena2d_block(int64_t B, int64_t X, int64_t Y, int64_t d, const double* q,
                         const double* k, const double* v, const double* sw, const double* sb,
                         const double* K, const double* D, double* y, int32_t method)
{
    const int64_t E = B * X * Y * d;
    double* qs = (double*)malloc(sizeof(double) * E);
    double* ks = (double*)malloc(sizeof(double) * E);
    double* vs = (double*)malloc(sizeof(double) * E);
    double* w = (double*)malloc(sizeof(double) * E);
    if (!qs || !ks || !vs || !w) { free(qs); free(ks); free(vs); free(w); return -1; }
    oracle_dwconv3x3(B, X, Y, d, q, sw, sb ? sb : NULL, qs);
    oracle_dwconv3x3(B, X, Y, d, k, sw + 9 * d, sb ? sb + d : NULL, ks);
    oracle_dwconv3x3(B, X, Y, d, v, sw + 18 * d, sb ? sb + 2 * d : NULL, vs);
    for (int64_t i = 0; i < E; ++i) qs[i] *= silu(ks[i]);
    int rc = 0;
    if (method == 0) oracle_conv2d_direct(B, X, Y, d, qs, K, D, w);
    else rc = oracle_conv2d_fft(B, X, Y, d, qs, K, D, w);
    if (rc == 0)
        for (int64_t i = 0; i < E; ++i) y[i] = silu(vs[i]) * w[i];
    free(qs); free(ks); free(vs); free(w);
    return rc;
}

/* ------------------------------------------------------------------------ */
/* HyenaND mixer on a 3D grid: the same block with 3x3x3 short convolutions */
/* ------------------------------------------------------------------------ */

/*
 * Depthwise 3x3x3 cross-correlation with zero padding of one:
 *   o[b,p,q,r,c] = bias[c] + sum_{a,e,f in -1..1} w[c][a+1][e+1][f+1] x[b,p+a,q+e,r+f,c]
 * x and o [B][X][Y][Z][d]; w [d][3][3][3]; bias [d] or NULL.
 */
void oracle_dwconv3x3x3(int64_t B, int64_t X, int64_t Y, int64_t Z, int64_t d, const double* x,
                        const double* w, const double* bias, double* o)
{
#pragma omp parallel for collapse(2) schedule(static)
    for (int64_t b = 0; b < B; ++b)
        for (int64_t p = 0; p < X; ++p)
            for (int64_t q = 0; q < Y; ++q)
                for (int64_t r = 0; r < Z; ++r)
                    for (int64_t c = 0; c < d; ++c) {
                        double acc = bias ? bias[c] : 0.0;
                        for (int a = -1; a <= 1; ++a)
                            for (int e = -1; e <= 1; ++e)
                                for (int f = -1; f <= 1; ++f) {
                                    const int64_t pp = p + a, qq = q + e, rr = r + f;
                                    if (pp < 0 || pp >= X || qq < 0 || qq >= Y || rr < 0 || rr >= Z)
                                        continue;
                                    acc += w[((c * 3 + (a + 1)) * 3 + (e + 1)) * 3 + (f + 1)] *
                                           x[(((b * X + pp) * Y + qq) * Z + rr) * d + c];
                                }
                        o[(((b * X + p) * Y + q) * Z + r) * d + c] = acc;
                    }
}

/*
 * The mixer on a 3D grid:
 *   qs, ks, vs = dwconv3x3x3(q | k | v)   (sw [3][d][3][3][3], sb [3][d] or NULL)
 *   z = qs . SiLU(ks)
 *   y = SiLU(vs) . (K * z + D z)          (K as in oracle_conv3d_direct)
 */
int oracle_hyena3d_block(int64_t B, int64_t X, int64_t Y, int64_t Z, int64_t d, const double* q,
                         const double* k, const double* v, const double* sw, const double* sb,
                         const double* K, const double* D, double* y, int32_t method)
{
    const int64_t E = B * X * Y * Z * d;
    double* qs = (double*)malloc(sizeof(double) * E);
    double* ks = (double*)malloc(sizeof(double) * E);
    double* vs = (double*)malloc(sizeof(double) * E);
    double* w = (double*)malloc(sizeof(double) * E);
    if (!qs || !ks || !vs || !w) { free(qs); free(ks); free(vs); free(w); return -1; }
    oracle_dwconv3x3x3(B, X, Y, Z, d, q, sw, sb ? sb : NULL, qs);
    oracle_dwconv3x3x3(B, X, Y, Z, d, k, sw + 27 * d, sb ? sb + d : NULL, ks);
    oracle_dwconv3x3x3(B, X, Y, Z, d, v, sw + 54 * d, sb ? sb + 2 * d : NULL, vs);
    for (int64_t i = 0; i < E; ++i) qs[i] *= silu(ks[i]);
    int rc = 0;
    if (method == 0) oracle_conv3d_direct(B, X, Y, Z, d, qs, K, D, w);
    else rc = oracle_conv3d_fft(B, X, Y, Z, d, qs, K, D, w);
    if (rc == 0)
        for (int64_t i = 0; i < E; ++i) y[i] = silu(vs[i]) * w[i];
    free(qs); free(ks); free(vs); free(w);
    return rc;
}
