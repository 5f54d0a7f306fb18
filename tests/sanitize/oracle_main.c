/* Drives the oracle (oracle/ssd_oracle.c) over its paths on small inputs, for
 * a build with AddressSanitizer and UndefinedBehaviorSanitizer: whole rows,
 * several rows with grouped heads, packed sequences (empty ones included),
 * incoming and outgoing states, the forward stream alone, and the backward.
 * Exits 0 when every call accepts its arguments and every output is finite;
 * the sanitizers abort on any bad access. Test infrastructure. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

int oracle_bissd_f64(int batch, int L, int H, int P, int N, int G, const double *xf,
                     const double *dtf, const double *Af, const double *Bf, const double *Cf,
                     const double *Df, const double *xb, const double *dtb, const double *Ab,
                     const double *Bb, const double *Cb, const double *Db,
                     const int32_t *cu_seqlens, int nseq, const double *init_state,
                     double *final_state, double *y);
int oracle_bissd_bwd_f64(int batch, int L, int H, int P, int N, int G, const double *xf,
                         const double *dtf, const double *Af, const double *Bf, const double *Cf,
                         const double *Df, const double *xb, const double *dtb, const double *Ab,
                         const double *Bb, const double *Cb, const double *Db,
                         const int32_t *cu_seqlens, int nseq, const double *dy,
                         double *const *gf, double *const *gb);

static unsigned long long rng = 88172645463325252ull;
static double uni(void) {   /* xorshift64, in (-1, 1) */
    rng ^= rng << 13; rng ^= rng >> 7; rng ^= rng << 17;
    return (double)(rng >> 11) / 4503599627370496.0 - 1.0;
}
static double *arr(size_t n, double lo, double hi) {
    double *a = malloc(n * sizeof(double));
    for (size_t i = 0; i < n; ++i) a[i] = lo + (hi - lo) * 0.5 * (uni() + 1.0);
    return a;
}
static int finite_all(const double *a, size_t n) {
    for (size_t i = 0; i < n; ++i) if (!isfinite(a[i])) return 0;
    return 1;
}

static int run(int batch, int L, int H, int P, int N, int G, const int32_t *cu, int nseq,
               int states, int bidir) {
    const size_t nx = (size_t)batch * L * H * P, nt = (size_t)batch * L * H,
                 nb = (size_t)batch * L * G * N;
    double *p[12];
    for (int d = 0; d < 2; ++d) {
        p[6 * d + 0] = arr(nx, -1, 1);
        p[6 * d + 1] = arr(nt, 0.01, 0.5);
        p[6 * d + 2] = arr(H, -4, -0.5);
        p[6 * d + 3] = arr(nb, -0.5, 0.5);
        p[6 * d + 4] = arr(nb, -0.5, 0.5);
        p[6 * d + 5] = arr(H, -1, 1);
    }
    const int units = cu ? nseq : batch;
    const size_t ns = (size_t)units * H * P * N;
    double *init = states ? arr(ns, -0.5, 0.5) : NULL;
    double *fin = states ? malloc(ns * sizeof(double)) : NULL;
    double *y = malloc(nx * sizeof(double));
    int ok = oracle_bissd_f64(batch, L, H, P, N, G, p[0], p[1], p[2], p[3], p[4], p[5],
                              bidir ? p[6] : NULL, bidir ? p[7] : NULL, bidir ? p[8] : NULL,
                              bidir ? p[9] : NULL, bidir ? p[10] : NULL, bidir ? p[11] : NULL,
                              cu, nseq, init, fin, y) == 0 && finite_all(y, nx) &&
             (!states || finite_all(fin, ns));
    if (!states) {
        /* the backward of the same problem */
        double *dy = arr(nx, -1, 1);
        double *gf[6], *gb[6];
        const size_t sz[6] = {nx, nt, (size_t)H, nb, nb, (size_t)H};
        for (int k = 0; k < 6; ++k) {
            gf[k] = malloc(sz[k] * sizeof(double));
            gb[k] = malloc(sz[k] * sizeof(double));
        }
        ok = ok && oracle_bissd_bwd_f64(batch, L, H, P, N, G, p[0], p[1], p[2], p[3], p[4], p[5],
                                        bidir ? p[6] : NULL, bidir ? p[7] : NULL,
                                        bidir ? p[8] : NULL, bidir ? p[9] : NULL,
                                        bidir ? p[10] : NULL, bidir ? p[11] : NULL, cu, nseq, dy,
                                        gf, bidir ? gb : NULL) == 0;
        for (int k = 0; k < 6; ++k) {
            ok = ok && finite_all(gf[k], sz[k]) && (!bidir || finite_all(gb[k], sz[k]));
            free(gf[k]);
            free(gb[k]);
        }
        free(dy);
    }
    for (int k = 0; k < 12; ++k) free(p[k]);
    free(init); free(fin); free(y);
    return ok;
}

int main(void) {
    const int32_t cu[] = {0, 5, 5, 17, 18, 40};
    int ok = 1;
    ok &= run(1, 33, 2, 4, 8, 1, NULL, 0, 0, 1);
    ok &= run(3, 20, 4, 3, 5, 2, NULL, 0, 1, 1);
    ok &= run(2, 1, 2, 4, 4, 1, NULL, 0, 1, 0);
    ok &= run(1, 40, 2, 4, 8, 1, cu, 5, 0, 1);
    ok &= run(1, 40, 2, 4, 8, 2, cu, 5, 0, 0);
    printf(ok ? "oracle sanitized runs: ok\n" : "oracle sanitized runs: FAILED\n");
    return ok ? 0 : 1;
}
