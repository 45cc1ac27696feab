/*
 * Calls every entry point of the fp64 oracle (oracle/ssm_oracle.c) on small
 * shapes, edge cases included, with every array allocated at exactly the size
 * the layout needs, so that a build with AddressSanitizer and
 * UndefinedBehaviorSanitizer reports any access outside them or any undefined
 * arithmetic on indices. tests/test_oracle_sanitized.py compiles and runs it;
 * it prints "ok" and returns 0 when every call returns its expected status
 * and every output is finite.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

int oracle_max_dstate(void);
int oracle_scan_fwd(int64_t batch, int64_t seqlen, int64_t dim, int64_t dstate,
                    const double* x, const double* delta, const double* A,
                    const double* Bm, const double* Cm, const double* Dskip,
                    const double* z, const double* h0, double* y, double* hL,
                    int zoh, const double* delta_bias, int delta_softplus);
int oracle_state_update(int64_t batch, int64_t dim, int64_t dstate, double* h,
                        const double* x, const double* delta, const double* A,
                        const double* Bm, const double* Cm, const double* Dskip,
                        const double* z, double* y, const double* delta_bias,
                        int delta_softplus);
int oracle_conv1d_fwd(int64_t batch, int64_t seqlen, int64_t dim, int64_t width,
                      const double* x, const double* weight, const double* bias,
                      const double* state_in, double* y, double* state_out, int silu);
int oracle_conv1d_update(int64_t batch, int64_t dim, int64_t width, double* state,
                         const double* x, const double* weight, const double* bias,
                         double* y, int silu);
int oracle_scan_bwd(int64_t batch, int64_t seqlen, int64_t dim, int64_t dstate,
                    const double* x, const double* delta, const double* A,
                    const double* Bm, const double* Cm, const double* Dskip,
                    const double* z, const double* h0, const double* delta_bias,
                    int delta_softplus, const double* dy, const double* dhL,
                    double* dx, double* ddelta, double* dA, double* dB, double* dC,
                    double* dD, double* dz, double* dh0, double* ddelta_bias);
int oracle_ssd_fwd(int64_t batch, int64_t seqlen, int64_t nheads, int64_t headdim,
                   int64_t dstate, const double* x, const double* dt, const double* A,
                   const double* Bm, const double* Cm, const double* Dskip, const double* z,
                   const double* h0, double* y, double* hL, const double* dt_bias,
                   int dt_softplus);

static uint64_t rng_state = 0x9e3779b97f4a7c15ull;

static double uniform(double lo, double hi)
{
    rng_state = rng_state * 6364136223846793005ull + 1442695040888963407ull;
    return lo + (hi - lo) * (double)(rng_state >> 11) * (1.0 / 9007199254740992.0);
}

/* exactly n doubles (at least one byte so malloc never returns NULL for 0) */
static double* arr(int64_t n, double lo, double hi)
{
    double* p = malloc(n > 0 ? (size_t)n * sizeof(double) : 1);
    if (!p) exit(3);
    for (int64_t i = 0; i < n; ++i) p[i] = uniform(lo, hi);
    return p;
}

static int failures = 0;

static void expect(int got, int want, const char* what)
{
    if (got != want) {
        printf("%s: status %d, expected %d\n", what, got, want);
        ++failures;
    }
}

static void finite(const double* p, int64_t n, const char* what)
{
    for (int64_t i = 0; i < n; ++i)
        if (!isfinite(p[i])) {
            printf("%s: non-finite value at %lld\n", what, (long long)i);
            ++failures;
            return;
        }
}

static void scan_case(int64_t b, int64_t L, int64_t d, int64_t n, int opt, int zoh, int sp)
{
    const int64_t e = b * L * d, bc = b * L * n, st = b * d * n;
    double *x = arr(e, -1, 1), *dl = arr(e, sp ? -2 : 0.01, sp ? 2 : 0.5), *A = arr(d * n, -3, -0.1);
    double *B = arr(bc, -1, 1), *C = arr(bc, -1, 1), *D = arr(d, -1, 1), *z = arr(e, -2, 2);
    double *h0 = arr(st, -1, 1), *y = arr(e, 0, 0), *hL = arr(st, 0, 0), *bias = arr(d, -1, 1);
    expect(oracle_scan_fwd(b, L, d, n, x, dl, A, B, C, opt ? D : NULL, opt ? z : NULL,
                           opt ? h0 : NULL, y, opt ? hL : NULL, zoh, sp ? bias : NULL, sp),
           0, "scan_fwd");
    finite(y, e, "scan_fwd y");
    if (opt) finite(hL, st, "scan_fwd hL");
    /* hL aliasing h0 */
    expect(oracle_scan_fwd(b, L, d, n, x, dl, A, B, C, D, z, h0, y, h0, zoh, NULL, 0), 0,
           "scan_fwd aliased");
    finite(h0, st, "scan_fwd aliased state");

    double *dy = arr(e, -1, 1), *dhL = arr(st, -1, 1);
    double *dx = arr(e, 0, 0), *ddl = arr(e, 0, 0), *dA = arr(d * n, 0, 0), *dB = arr(bc, 0, 0);
    double *dC = arr(bc, 0, 0), *dD = arr(d, 0, 0), *dz = arr(e, 0, 0), *dh0 = arr(st, 0, 0);
    double* dbias = arr(d, 0, 0);
    expect(oracle_scan_bwd(b, L, d, n, x, dl, A, B, C, opt ? D : NULL, opt ? z : NULL,
                           opt ? h0 : NULL, sp ? bias : NULL, sp, dy, opt ? dhL : NULL, dx, ddl, dA,
                           dB, dC, opt ? dD : NULL, opt ? dz : NULL, opt ? dh0 : NULL,
                           sp ? dbias : NULL),
           0, "scan_bwd");
    finite(dx, e, "scan_bwd dx");
    finite(dA, d * n, "scan_bwd dA");
    free(dy); free(dhL); free(dx); free(ddl); free(dA); free(dB); free(dC); free(dD); free(dz);
    free(dh0); free(dbias);

    /* decode on the first token's inputs (batch rows of one token) */
    if (L > 0) {
        double *hx = arr(b * d, -1, 1), *hd = arr(b * d, 0.01, 0.5), *hb = arr(b * n, -1, 1);
        double *hc = arr(b * n, -1, 1), *hz = arr(b * d, -1, 1), *hy = arr(b * d, 0, 0);
        expect(oracle_state_update(b, d, n, hL, hx, hd, A, hb, hc, opt ? D : NULL,
                                   opt ? hz : NULL, hy, NULL, 0),
               0, "state_update");
        finite(hy, b * d, "state_update y");
        free(hx); free(hd); free(hb); free(hc); free(hz); free(hy);
    }
    free(x); free(dl); free(A); free(B); free(C); free(D); free(z); free(h0); free(y); free(hL);
    free(bias);
}

static void conv_case(int64_t b, int64_t L, int64_t d, int64_t w, int with_state)
{
    const int64_t e = b * L * d, s = b * d * w;
    double *x = arr(e, -1, 1), *wt = arr(d * w, -0.5, 0.5), *bias = arr(d, -0.5, 0.5);
    double *sin = arr(s, -1, 1), *y = arr(e, 0, 0), *sout = arr(s, 0, 0);
    expect(oracle_conv1d_fwd(b, L, d, w, x, wt, bias, with_state ? sin : NULL, y,
                             with_state ? sout : NULL, 1),
           0, "conv1d_fwd");
    finite(y, e, "conv1d_fwd y");
    /* the decode step updates its state in place */
    double *x1 = arr(b * d, -1, 1), *y1 = arr(b * d, 0, 0);
    expect(oracle_conv1d_update(b, d, w, sin, x1, wt, NULL, y1, 0), 0, "conv1d_update");
    finite(y1, b * d, "conv1d_update y");
    free(x); free(wt); free(bias); free(sin); free(y); free(sout); free(x1); free(y1);
}

static void ssd_case(int64_t b, int64_t L, int64_t H, int64_t P, int64_t n, int opt, int sp)
{
    const int64_t dim = H * P, e = b * L * dim, bc = b * L * n, st = b * H * P * n;
    double *x = arr(e, -1, 1), *dt = arr(b * L * H, sp ? -2 : 0.01, sp ? 2 : 0.5);
    double *A = arr(H, -3, -0.1), *B = arr(bc, -1, 1), *C = arr(bc, -1, 1), *D = arr(dim, -1, 1);
    double *z = arr(e, -2, 2), *h0 = arr(st, -1, 1), *y = arr(e, 0, 0), *hL = arr(st, 0, 0);
    double* bias = arr(H, -1, 1);
    expect(oracle_ssd_fwd(b, L, H, P, n, x, dt, A, B, C, opt ? D : NULL, opt ? z : NULL,
                          opt ? h0 : NULL, y, opt ? hL : NULL, sp ? bias : NULL, sp),
           0, "ssd_fwd");
    finite(y, e, "ssd_fwd y");
    free(x); free(dt); free(A); free(B); free(C); free(D); free(z); free(h0); free(y); free(hL);
    free(bias);
}

int main(void)
{
    const int64_t nmax = oracle_max_dstate();
    /* shapes: ragged, one channel, one state, the largest state, no tokens */
    const int64_t shapes[][4] = {{2, 7, 3, 4}, {1, 1, 1, 1}, {3, 5, 2, 16}, {2, 0, 3, 2},
                                 {1, 9, 5, 7}};
    for (size_t k = 0; k < sizeof(shapes) / sizeof(shapes[0]); ++k)
        for (int opt = 0; opt < 2; ++opt)
            for (int sp = 0; sp < 2; ++sp)
                scan_case(shapes[k][0], shapes[k][1], shapes[k][2],
                          shapes[k][3] <= nmax ? shapes[k][3] : nmax, opt, 0, sp);
    scan_case(2, 6, 3, 4, 1, 1, 0); /* zero-order hold */
    /* rejected arguments leave everything untouched */
    expect(oracle_scan_fwd(1, 1, 1, nmax + 1, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL,
                           NULL, NULL, 0, NULL, 0),
           -1, "scan_fwd dstate too large");
    for (int64_t w = 1; w <= 4; ++w)
        for (int64_t L = 0; L <= 5; L += 1) {
            conv_case(2, L, 3, w, 1);
            conv_case(1, L, 2, w, 0);
        }
    for (int opt = 0; opt < 2; ++opt)
        for (int sp = 0; sp < 2; ++sp) {
            ssd_case(2, 9, 2, 3, 4, opt, sp);
            ssd_case(1, 1, 1, 1, 1, opt, sp);
            ssd_case(1, 0, 3, 2, 5, opt, sp);
        }
    if (failures) {
        printf("%d failures\n", failures);
        return 1;
    }
    printf("ok\n");
    return 0;
}
