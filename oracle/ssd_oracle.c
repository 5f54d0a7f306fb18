/*
 * Oracle for the bidirectional Mamba-2 selective state-space (SSD) mixer.
 *
 * TEST INFRASTRUCTURE ONLY. Nothing on the product path may include, link or
 * call this file; only the test-suite, the smoke check and the CPU-baseline leg
 * of the benchmark use it. It shares no code, header, table or helper with the
 * HIP library.
 *
 * What it computes (plain fp64, one token at a time, no chunking, no fusion):
 *
 *   Mamba-2 selective recurrence per head h (the mixer named by
 *   "Fixed state, long reach: constant-size caches in large-scale block
 *   diffusion", Sec. 1, as a linear-time recurrence whose hidden state is a
 *   fixed-size summary of the history; DiffuMamba summaries, Methodology /
 *   proposed-method sections, name it "Mamba-2"):
 *
 *     forward : h_t = exp(dt_t * A_h) * h_{t-1} + dt_t * B_t x_t^T
 *               y_t = C_t^T h_t + D_h * x_t,            t = 0 .. L-1
 *     backward: the same recurrence over the time-reversed sequence with its
 *               own parameters. Written out without a flip:
 *               h_t = exp(dt_t * A_h) * h_{t+1} + dt_t * B_t x_t^T,
 *               t = L-1 .. 0 (DiffuMamba blog, "network architecture":
 *               flip, run the second Mamba, flip back).
 *     output  : y = y_fwd + y_bwd (the two streams are merged by addition,
 *               gist.science/ja DiffuMamba summary, Sec. 2 "proposed method").
 *
 *   h is a d_state x headdim matrix per (sequence, head), stored [p][n].
 *   A head uses group g = h / (nheads / ngroups) for B and C.
 *
 *   Packed sequences (cu_seqlens): every sequence starts from a zero state in
 *   both directions; nothing crosses a sequence boundary.
 *
 *   Block step ("Fixed state, long reach", Sec. 1: the forward SSM state of
 *   the finalized prefix is the block cache and the reverse scan is restricted
 *   to the active block): the forward part starts from the carried state, the
 *   backward part starts from zero at the block end. That is this same routine
 *   with init_state = the cache and L = block length.
 *
 * Layouts (row-major, per batch row or packed stream):
 *   x [batch][L][H][P], dt [batch][L][H], B,C [batch][L][G][N], A,D [H],
 *   y [batch][L][H][P], init_state/final_state [nseq][H][P][N].
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* Runs one direction of the recurrence for one head over tokens [t0, t1)
 * of one row, starting from `state` (P*N, [p][n]); adds its y into `y`. */
static void scan_one_head(int reverse, int t0, int t1, int h,
                          int H, int P, int N, int G,
                          const double *x, const double *dt, const double *A,
                          const double *B, const double *C, const double *D,
                          double *state, double *y)
{
    const int g = h / (H / G);
    const double Dh = D ? D[h] : 0.0;
    for (int step = 0; step < t1 - t0; ++step) {
        const int t = reverse ? (t1 - 1 - step) : (t0 + step);
        const double dtt = dt[(size_t)t * H + h];
        const double decay = exp(dtt * A[h]);
        const double *Bt = B + ((size_t)t * G + g) * N;
        const double *Ct = C + ((size_t)t * G + g) * N;
        const double *xt = x + ((size_t)t * H + h) * P;
        double *yt = y + ((size_t)t * H + h) * P;
        for (int p = 0; p < P; ++p) {
            double *hp = state + (size_t)p * N;
            double acc = 0.0;
            for (int n = 0; n < N; ++n) {
                hp[n] = decay * hp[n] + dtt * Bt[n] * xt[p];
                acc += Ct[n] * hp[n];
            }
            yt[p] += acc + Dh * xt[p];
        }
    }
}

/*
 * Bidirectional SSD over `batch` rows of length L, or, when cu_seqlens is
 * given (then batch must be 1), over nseq packed sequences
 * [cu_seqlens[i], cu_seqlens[i+1]) of the single row.
 *
 * xb == NULL runs the forward direction only.
 * init_state (NULL = zeros) seeds the forward state of every sequence;
 * final_state (NULL = not wanted) receives the forward state after each
 * sequence's last token. Both are [nseq or batch][H][P][N].
 * y is fully overwritten. Returns 0, or -1 on inconsistent arguments.
 */
int oracle_bissd_f64(int batch, int L, int H, int P, int N, int G,
                     const double *xf, const double *dtf, const double *Af,
                     const double *Bf, const double *Cf, const double *Df,
                     const double *xb, const double *dtb, const double *Ab,
                     const double *Bb, const double *Cb, const double *Db,
                     const int32_t *cu_seqlens, int nseq,
                     const double *init_state, double *final_state, double *y)
{
    if (batch < 0 || L < 0 || H <= 0 || P <= 0 || N <= 0 || G <= 0 || H % G)
        return -1;
    if ((long)P * N > 128 * 128)
        return -1;
    if (cu_seqlens && (batch != 1 || nseq < 0 || cu_seqlens[0] != 0 ||
                       cu_seqlens[nseq] != L))
        return -1;
    if (cu_seqlens)
        for (int i = 0; i < nseq; ++i)
            if (cu_seqlens[i + 1] < cu_seqlens[i])
                return -1;

    const int nunits = cu_seqlens ? nseq : batch;
    const size_t row_tokens = (size_t)L;
    memset(y, 0, sizeof(double) * (size_t)batch * L * H * P);

    #pragma omp parallel for schedule(dynamic) collapse(2)
    for (int u = 0; u < nunits; ++u) {
        for (int h = 0; h < H; ++h) {
            /* which row and which token range this unit covers */
            const int row = cu_seqlens ? 0 : u;
            const int t0 = cu_seqlens ? cu_seqlens[u] : 0;
            const int t1 = cu_seqlens ? cu_seqlens[u + 1] : L;
            const size_t xo = row * row_tokens * H * P;
            const size_t to = row * row_tokens * H;
            const size_t bo = row * row_tokens * G * N;
            double state[128 * 128];            /* P*N <= 16384 */
            const size_t sz = (size_t)P * N;
            const size_t so = ((size_t)u * H + h) * sz;

            if (init_state)
                memcpy(state, init_state + so, sizeof(double) * sz);
            else
                memset(state, 0, sizeof(double) * sz);
            scan_one_head(0, t0, t1, h, H, P, N, G, xf + xo, dtf + to, Af,
                          Bf + bo, Cf + bo, Df, state, y + xo);
            if (final_state)
                memcpy(final_state + so, state, sizeof(double) * sz);

            if (xb) {
                memset(state, 0, sizeof(double) * sz);
                scan_one_head(1, t0, t1, h, H, P, N, G, xb + xo, dtb + to, Ab,
                              Bb + bo, Cb + bo, Db, state, y + xo);
            }
        }
    }
    return 0;
}

/*
 * Gradients of the bidirectional SSD (the training backward), by the adjoint
 * of the recurrence above: the chain rule applied token by token, nothing
 * chunked. For one direction and head, with a_t = exp(dt_t A) and the
 * incoming output gradient dy_t (shared by both directions, y being their
 * sum), walking the tokens in the opposite order of the scan:
 *
 *   g_t   = a_{t+1} g_{t+1} + C_t dy_t^T      (gradient of h_t; g = 0 after
 *                                             the last token of the sequence)
 *   dC_t  = h_t dy_t                          (summed over the heads of C's group)
 *   dx_t  = D dy_t + dt_t g_t^T B_t
 *   dB_t  = dt_t g_t x_t                      (summed over the heads of B's group)
 *   ddt_t = <g_t, B_t x_t^T> + A a_t <g_t, h_{t-1}>
 *   dA    = sum_t dt_t a_t <g_t, h_{t-1}>
 *   dD    = sum_t <x_t, dy_t>
 *
 * where t+1 and t-1 are the next and previous tokens in the scan's own
 * order (reversed for the reverse stream) and h_{-1} = 0. h_t is kept for
 * every token of the sequence (obviously correct, memory-hungry). Packed
 * sequences are independent; init_state is zero.
 */
static int adjoint_one_head(int reverse, int t0, int t1, int h,
                            int H, int P, int N, int G,
                            const double *x, const double *dt, const double *A,
                            const double *B, const double *C, const double *D,
                            const double *dy, double *dx, double *ddt,
                            double *dB, double *dC, double *dA, double *dD)
{
    const int T = t1 - t0;
    const int g = h / (H / G);
    const size_t sz = (size_t)P * N;
    double *hs = (double *)malloc(sizeof(double) * sz * (T > 0 ? T : 1));
    double *gs = (double *)calloc(sz, sizeof(double));
    if (!hs || !gs) {
        free(hs);
        free(gs);
        return -1;
    }
    const double Dh = D ? D[h] : 0.0;
    /* forward sweep: h_t for every step of the scan */
    for (int step = 0; step < T; ++step) {
        const int t = reverse ? (t1 - 1 - step) : (t0 + step);
        const double dtt = dt[(size_t)t * H + h];
        const double decay = exp(dtt * A[h]);
        const double *Bt = B + ((size_t)t * G + g) * N;
        const double *xt = x + ((size_t)t * H + h) * P;
        const double *prev = step ? hs + (size_t)(step - 1) * sz : NULL;
        double *cur = hs + (size_t)step * sz;
        for (int p = 0; p < P; ++p)
            for (int n = 0; n < N; ++n)
                cur[(size_t)p * N + n] = (prev ? decay * prev[(size_t)p * N + n] : 0.0) +
                                         dtt * Bt[n] * xt[p];
    }
    /* backward sweep */
    for (int step = T - 1; step >= 0; --step) {
        const int t = reverse ? (t1 - 1 - step) : (t0 + step);
        const double dtt = dt[(size_t)t * H + h];
        const double decay = exp(dtt * A[h]);
        const double *Bt = B + ((size_t)t * G + g) * N;
        const double *Ct = C + ((size_t)t * G + g) * N;
        const double *xt = x + ((size_t)t * H + h) * P;
        const double *dyt = dy + ((size_t)t * H + h) * P;
        const double *cur = hs + (size_t)step * sz;
        const double *prev = step ? hs + (size_t)(step - 1) * sz : NULL;
        double *dBt = dB + ((size_t)t * G + g) * N;
        double *dCt = dC + ((size_t)t * G + g) * N;
        double q = 0.0, r = 0.0, xdy = 0.0;
        for (int p = 0; p < P; ++p) {
            double *gp = gs + (size_t)p * N;
            double gb = 0.0;
            for (int n = 0; n < N; ++n) {
                gp[n] += Ct[n] * dyt[p];
                dCt[n] += cur[(size_t)p * N + n] * dyt[p];
                gb += gp[n] * Bt[n];
                dBt[n] += dtt * gp[n] * xt[p];
                if (prev)
                    q += gp[n] * prev[(size_t)p * N + n];
                r += gp[n] * Bt[n] * xt[p];
            }
            dx[((size_t)t * H + h) * P + p] = Dh * dyt[p] + dtt * gb;
            xdy += xt[p] * dyt[p];
        }
        ddt[(size_t)t * H + h] = r + A[h] * decay * q;
        *dA += dtt * decay * q;
        *dD += xdy;
        for (size_t i = 0; i < sz; ++i)
            gs[i] *= decay;
    }
    free(hs);
    free(gs);
    return 0;
}

/*
 * Gradients of oracle_bissd_f64's y with respect to every input of both
 * directions, given dy [batch][L][H][P]. gf and gb each point to six output
 * arrays, in this order: dx [batch][L][H][P], ddt [batch][L][H], dA [H],
 * dB [batch][L][G][N], dC [batch][L][G][N], dD [H] (all overwritten; gb and
 * the reverse inputs may be NULL for the forward stream alone). No initial
 * state. Returns 0, or -1 on inconsistent arguments or allocation failure.
 */
int oracle_bissd_bwd_f64(int batch, int L, int H, int P, int N, int G,
                         const double *xf, const double *dtf, const double *Af,
                         const double *Bf, const double *Cf, const double *Df,
                         const double *xb, const double *dtb, const double *Ab,
                         const double *Bb, const double *Cb, const double *Db,
                         const int32_t *cu_seqlens, int nseq, const double *dy,
                         double *const *gf, double *const *gb)
{
    if (batch < 0 || L < 0 || H <= 0 || P <= 0 || N <= 0 || G <= 0 || H % G)
        return -1;
    if (cu_seqlens && (batch != 1 || nseq < 0 || cu_seqlens[0] != 0 ||
                       cu_seqlens[nseq] != L))
        return -1;
    if (cu_seqlens)
        for (int i = 0; i < nseq; ++i)
            if (cu_seqlens[i + 1] < cu_seqlens[i])
                return -1;
    const int ndir = xb ? 2 : 1;
    const int nunits = cu_seqlens ? nseq : batch;
    const size_t nx = (size_t)batch * L * H * P, nt = (size_t)batch * L * H;
    const size_t nb = (size_t)batch * L * G * N;
    double *const *gr[2] = {gf, gb};
    for (int d = 0; d < ndir; ++d) {
        memset(gr[d][0], 0, sizeof(double) * nx);
        memset(gr[d][1], 0, sizeof(double) * nt);
        memset(gr[d][3], 0, sizeof(double) * nb);
        memset(gr[d][4], 0, sizeof(double) * nb);
    }
    /* per-unit partial sums of dA and dD, added up in unit order at the end */
    double *part = (double *)calloc((size_t)ndir * (nunits > 0 ? nunits : 1) * H * 2, sizeof(double));
    if (!part)
        return -1;
    int failed = 0;
    /* one unit (row or packed sequence) per task: its heads run in order,
     * so the group sums of dB and dC never race */
    #pragma omp parallel for schedule(dynamic) reduction(|:failed)
    for (int u = 0; u < nunits; ++u) {
        const int row = cu_seqlens ? 0 : u;
        const int t0 = cu_seqlens ? cu_seqlens[u] : 0;
        const int t1 = cu_seqlens ? cu_seqlens[u + 1] : L;
        const size_t xo = (size_t)row * L * H * P, to = (size_t)row * L * H;
        const size_t bo = (size_t)row * L * G * N;
        for (int d = 0; d < ndir; ++d) {
            const double *x = d ? xb : xf, *dt = d ? dtb : dtf, *A = d ? Ab : Af;
            const double *B = d ? Bb : Bf, *C = d ? Cb : Cf, *D = d ? Db : Df;
            for (int h = 0; h < H; ++h) {
                double *pa = part + (((size_t)d * nunits + u) * H + h) * 2;
                failed |= adjoint_one_head(d, t0, t1, h, H, P, N, G, x + xo, dt + to, A,
                                           B + bo, C + bo, D, dy + xo,
                                           gr[d][0] + xo, gr[d][1] + to,
                                           gr[d][3] + bo, gr[d][4] + bo, pa, pa + 1) != 0;
            }
        }
    }
    for (int d = 0; d < ndir; ++d)
        for (int h = 0; h < H; ++h) {
            double sa = 0.0, sd = 0.0;
            for (int u = 0; u < nunits; ++u) {
                sa += part[(((size_t)d * nunits + u) * H + h) * 2];
                sd += part[(((size_t)d * nunits + u) * H + h) * 2 + 1];
            }
            gr[d][2][h] = sa;
            gr[d][5][h] = sd;
        }
    free(part);
    return failed ? -1 : 0;
}

/* Largest P*N the oracle's per-unit state buffer holds. */
int oracle_max_state_elems(void) { return 128 * 128; }

/* Number of OpenMP threads a parallel region would use here. */
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
