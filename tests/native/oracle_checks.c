/*
 * oracle_checks.c -- runs every function of the float64 oracle on small,
 * ragged shapes under AddressSanitizer and UndefinedBehaviorSanitizer (built
 * by tests/test_host_sanitizers.py together with oracle/oracle.c).  Beyond
 * the sanitizers' own reports it checks that the direct and FFT routes agree
 * (both are pinned to the pages elsewhere; here the point is memory safety
 * on shapes with odd channel counts and non-power-of-two lengths).
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

int oracle_fft(int64_t n, double* re, double* im, int sign);
int oracle_hyena1d(int64_t B, int64_t N, int64_t d, int32_t order, const double* u,
                   const double* gates, const double* h, const double* D, double* y,
                   int32_t method);
int oracle_hyena2d(int64_t B, int64_t X, int64_t Y, int64_t d, int32_t order, const double* u,
                   const double* gates, const double* K, const double* D, double* y,
                   int32_t method);
int oracle_hyena3d(int64_t B, int64_t X, int64_t Y, int64_t Z, int64_t d, int32_t order,
                   const double* u, const double* gates, const double* K, const double* D,
                   double* y, int32_t method);
int oracle_hyena1d_circular(int64_t B, int64_t N, int64_t d, int32_t order, const double* u,
                            const double* gates, const double* h, const double* D, double* y,
                            int32_t method);
void oracle_implicit_filter(int64_t N, int64_t d, int32_t order, int32_t K, int32_t H,
                            double omega, const double* W1, const double* b1,
                            const double* W2, const double* b2, const double* W3,
                            const double* b3, const double* alpha, double* h);
int oracle_hyena2d_block(int64_t B, int64_t X, int64_t Y, int64_t d, const double* q,
                         const double* k, const double* v, const double* sw, const double* sb,
                         const double* K, const double* D, double* y, int32_t method);
int oracle_hyena3d_block(int64_t B, int64_t X, int64_t Y, int64_t Z, int64_t d, const double* q,
                         const double* k, const double* v, const double* sw, const double* sb,
                         const double* K, const double* D, double* y, int32_t method);

static int g_fail = 0;
static uint64_t g_state = 0x9E3779B97F4A7C15ull;

/* xorshift64* draws in [-1, 1): test inputs only */
static double draw(void)
{
    g_state ^= g_state >> 12;
    g_state ^= g_state << 25;
    g_state ^= g_state >> 27;
    return (double)((g_state * 0x2545F4914F6CDD1Dull) >> 11) * (2.0 / 9007199254740992.0) - 1.0;
}

static double* fresh(int64_t n)
{
    double* a = (double*)malloc(sizeof(double) * (size_t)(n > 0 ? n : 1));
    for (int64_t i = 0; i < n; ++i) a[i] = draw();
    return a;
}

static void agree(const char* what, const double* a, const double* b, int64_t n, double tol)
{
    double e = 0.0, m = 1e-300;
    for (int64_t i = 0; i < n; ++i) {
        e = fmax(e, fabs(a[i] - b[i]));
        m = fmax(m, fabs(b[i]));
    }
    if (!(e / m <= tol)) {
        fprintf(stderr, "%s: direct and FFT routes differ by %.3e\n", what, e / m);
        ++g_fail;
    }
}

static void chain1d(int64_t B, int64_t N, int64_t d, int32_t order)
{
    const int64_t E = B * N * d;
    double *u = fresh(E), *g = fresh(order * E), *h = fresh(order * d * N), *D = fresh(order * d);
    double *y0 = fresh(E), *y1 = fresh(E);
    if (oracle_hyena1d(B, N, d, order, u, g, h, D, y0, 0) != 0) ++g_fail;
    if (oracle_hyena1d(B, N, d, order, u, g, h, D, y1, 1) != 0) ++g_fail;
    agree("1d", y0, y1, E, 1e-12);
    if ((N & (N - 1)) == 0) {
        if (oracle_hyena1d_circular(B, N, d, order, u, g, h, D, y0, 0) != 0) ++g_fail;
        if (oracle_hyena1d_circular(B, N, d, order, u, g, h, D, y1, 1) != 0) ++g_fail;
        agree("1d circular", y0, y1, E, 1e-12);
    }
    free(u); free(g); free(h); free(D); free(y0); free(y1);
}

static void chain2d(int64_t B, int64_t X, int64_t Y, int64_t d, int32_t order)
{
    const int64_t E = B * X * Y * d, T = (2 * X - 1) * (2 * Y - 1);
    double *u = fresh(E), *g = fresh(order * E), *K = fresh(order * d * T), *D = fresh(order * d);
    double *y0 = fresh(E), *y1 = fresh(E);
    if (oracle_hyena2d(B, X, Y, d, order, u, g, K, D, y0, 0) != 0) ++g_fail;
    if (oracle_hyena2d(B, X, Y, d, order, u, g, K, D, y1, 1) != 0) ++g_fail;
    agree("2d", y0, y1, E, 1e-12);
    if (order == 1) {
        double *k = fresh(E), *v = fresh(E), *sw = fresh(3 * d * 9), *sb = fresh(3 * d);
        if (oracle_hyena2d_block(B, X, Y, d, u, k, v, sw, sb, K, D, y0, 0) != 0) ++g_fail;
        if (oracle_hyena2d_block(B, X, Y, d, u, k, v, sw, sb, K, D, y1, 1) != 0) ++g_fail;
        agree("2d block", y0, y1, E, 1e-12);
        free(k); free(v); free(sw); free(sb);
    }
    free(u); free(g); free(K); free(D); free(y0); free(y1);
}

static void chain3d(int64_t B, int64_t X, int64_t Y, int64_t Z, int64_t d, int32_t order)
{
    const int64_t E = B * X * Y * Z * d, T = (2 * X - 1) * (2 * Y - 1) * (2 * Z - 1);
    double *u = fresh(E), *g = fresh(order * E), *K = fresh(order * d * T), *D = fresh(order * d);
    double *y0 = fresh(E), *y1 = fresh(E);
    if (oracle_hyena3d(B, X, Y, Z, d, order, u, g, K, D, y0, 0) != 0) ++g_fail;
    if (oracle_hyena3d(B, X, Y, Z, d, order, u, g, K, D, y1, 1) != 0) ++g_fail;
    agree("3d", y0, y1, E, 1e-12);
    if (order == 1) {
        double *k = fresh(E), *v = fresh(E), *sw = fresh(3 * d * 27), *sb = fresh(3 * d);
        if (oracle_hyena3d_block(B, X, Y, Z, d, u, k, v, sw, sb, K, D, y0, 0) != 0) ++g_fail;
        if (oracle_hyena3d_block(B, X, Y, Z, d, u, k, v, sw, sb, K, D, y1, 1) != 0) ++g_fail;
        agree("3d block", y0, y1, E, 1e-12);
        free(k); free(v); free(sw); free(sb);
    }
    free(u); free(g); free(K); free(D); free(y0); free(y1);
}

int main(void)
{
    for (int64_t n = 1; n <= 64; n *= 2) {
        double *re = fresh(n), *im = fresh(n);
        if (oracle_fft(n, re, im, -1) != 0 || oracle_fft(n, re, im, +1) != 0) ++g_fail;
        free(re); free(im);
    }
    {
        double re[3] = {0, 0, 0}, im[3] = {0, 0, 0};
        if (oracle_fft(3, re, im, -1) == 0) ++g_fail; /* not a power of two: refused */
    }
    const int64_t Ns[] = {1, 2, 3, 5, 8, 13, 16, 31, 64};
    for (int i = 0; i < 9; ++i)
        for (int64_t d = 1; d <= 3; ++d) chain1d(1 + (d & 1), Ns[i], d, (int32_t)(1 + i % 3));
    chain2d(1, 4, 4, 3, 2);
    chain2d(2, 8, 4, 1, 1);
    chain2d(1, 4, 16, 2, 1);
    chain3d(1, 4, 4, 4, 3, 2);
    chain3d(1, 4, 8, 4, 1, 1);
    {
        const int64_t N = 37, d = 3, K = 4, H = 5;
        const int32_t order = 2;
        const int64_t m = 2 * K + 1;
        double *W1 = fresh(H * m), *b1 = fresh(H), *W2 = fresh(H * H), *b2 = fresh(H);
        double *W3 = fresh(order * d * H), *b3 = fresh(order * d), *al = fresh(order * d);
        for (int64_t i = 0; i < order * d; ++i) al[i] = fabs(al[i]) * 1e-2;
        double* h = fresh(order * d * N);
        oracle_implicit_filter(N, d, order, (int32_t)K, (int32_t)H, 8.0, W1, b1, W2, b2, W3, b3,
                               al, h);
        for (int64_t i = 0; i < order * d * N; ++i)
            if (!isfinite(h[i])) ++g_fail;
        free(W1); free(b1); free(W2); free(b2); free(W3); free(b3); free(al); free(h);
    }
    if (g_fail) {
        fprintf(stderr, "%d oracle checks failed\n", g_fail);
        return 1;
    }
    printf("oracle checks passed\n");
    return 0;
}
