/*
 * TEST INFRASTRUCTURE ONLY.  The plain, slow, fp64 CPU definition of the selective
 * state-space scan (S6) and of its single-token recurrent step.  It exists to check
 * the GPU library against; only the tests, the package's smoke check and the
 * benchmark's CPU-baseline leg call it.  It shares no code, header or constant with
 * the GPU path.
 *
 * What it computes, and where the pages state it:
 *  - continuous model h'(t) = A h(t) + B x(t), y(t) = C h(t) + D x(t)
 *      (yapayzekasozluk.tr "Temel Matematiksel Cerceve"; shakilmahmud.com section 1)
 *  - discretisation: ZOH for the state matrix, dA = exp(delta * A), exact for a diagonal A
 *      (yapayzekasozluk.tr "Temel Matematiksel Cerceve" names ZOH / A_bar, B_bar);
 *    the input term is taken in its simplified form delta * B_t * u_t (the pages give no
 *    B_bar formula)
 *  - selection: B_t, C_t and delta_t vary per token, delta_t = softplus(linear(x_t)),
 *    A stays fixed (azimuth.plus/paper/mamba, "selection" section, the three bullets and
 *    the remark that A alone stays fixed)
 *  - the recurrence h_t = A_bar_t h_{t-1} + B_bar_t x_t
 *      (azimuth.plus/paper/mamba, hardware-aware algorithm section, "parallel scan" bullet)
 *  - the gate branch multiplies the SSM branch elementwise after SiLU
 *      (azimuth.plus/paper/mamba, block architecture section)
 *  - the recurrent (inference) form: constant memory, one state update per token
 *      (shakilmahmud.com section 3; urworte.de "Methodische Grundlagen")
 *
 * Readings where the pages are silent: the scan starts from h = 0; the step size is
 * softplus(delta_in + delta_bias) when the flag is set, else delta_in + delta_bias;
 * B_t and C_t are one N-vector per (sequence, token), shared by every channel; the skip
 * term D*u is inside the gate: y = (C.h + D u) * silu(z).
 *
 * Arithmetic is IEEE fp64 throughout, in the order written; build with
 * -ffp-contract=off so that no multiply-add is fused.
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>

#define ORACLE_MAX_N 256

int ssm_oracle_max_n(void) { return ORACLE_MAX_N; }

/* softplus(x) = log(1 + e^x), written so that neither branch overflows. */
static double oracle_softplus(double x) {
    if (x > 0.0) return x + log1p(exp(-x));
    return log1p(exp(x));
}

/* silu(z) = z * sigmoid(z) = z / (1 + e^-z). */
static double oracle_silu(double z) { return z / (1.0 + exp(-z)); }

/*
 * Scan over one batch of sequences, continuing from the state h0 (the recurrent form
 * carries the state from one stretch of tokens to the next: shakilmahmud.com section 3).
 *   u, delta, z, y : [bsz][L][D]      B, C : [bsz][L][N]
 *   A : [D][N]     Dv, delta_bias : [D]   (Dv, z, delta_bias may be NULL)
 *   h0, last_state : [bsz][D][N] or NULL (h0 NULL: start from zero)
 * Channels (b, d) are independent; they are spread over `nthreads` OpenMP threads,
 * each walking its channel's tokens in order.  Returns 0, or -1 if N is too large.
 */
int ssm_oracle_scan_from(int64_t bsz, int64_t L, int64_t D, int64_t N, const double *h0,
                         const double *u, const double *delta, const double *A,
                         const double *B, const double *C, const double *Dv,
                         const double *z, const double *delta_bias, int softplus_flag,
                         double *y, double *last_state, int nthreads) {
    if (N > ORACLE_MAX_N || N < 1) return -1;
    int64_t nch = bsz * D;
#pragma omp parallel for schedule(dynamic, 1) num_threads(nthreads)
    for (int64_t ch = 0; ch < nch; ++ch) {
        int64_t b = ch / D, d = ch % D;
        double h[ORACLE_MAX_N];
        for (int64_t n = 0; n < N; ++n) h[n] = h0 ? h0[(b * D + d) * N + n] : 0.0;
        for (int64_t t = 0; t < L; ++t) {
            int64_t i = (b * L + t) * D + d;       /* (b, t, d) */
            const double *Bt = B + (b * L + t) * N;
            const double *Ct = C + (b * L + t) * N;
            double x = delta[i];
            if (delta_bias) x = x + delta_bias[d];
            double dt = softplus_flag ? oracle_softplus(x) : x;
            double ut = u[i];
            for (int64_t n = 0; n < N; ++n) {
                double dA = exp(dt * A[d * N + n]);
                h[n] = dA * h[n] + dt * Bt[n] * ut;
            }
            double acc = 0.0;
            for (int64_t n = 0; n < N; ++n) acc = acc + Ct[n] * h[n];
            double yt = acc;
            if (Dv) yt = yt + Dv[d] * ut;
            if (z) yt = yt * oracle_silu(z[i]);
            y[i] = yt;
        }
        if (last_state)
            for (int64_t n = 0; n < N; ++n) last_state[(b * D + d) * N + n] = h[n];
    }
    return 0;
}

/* The scan from h = 0 (the scan of a whole sequence). */
int ssm_oracle_scan(int64_t bsz, int64_t L, int64_t D, int64_t N,
                    const double *u, const double *delta, const double *A,
                    const double *B, const double *C, const double *Dv,
                    const double *z, const double *delta_bias, int softplus_flag,
                    double *y, double *last_state, int nthreads) {
    return ssm_oracle_scan_from(bsz, L, D, N, NULL, u, delta, A, B, C, Dv, z, delta_bias, softplus_flag,
                                y, last_state, nthreads);
}

/*
 * One recurrent step for S independent sequences; `state` is updated in place.
 *   state : [S][D][N]   u, delta, z, y : [S][D]   B, C : [S][N]   A : [D][N]   Dv : [D]
 * delta arrives already activated (no bias, no softplus).  The per-element arithmetic is
 * the scan's, in the same order, so L steps from a zero state reproduce the scan.
 */
int ssm_oracle_step(int64_t S, int64_t D, int64_t N, double *state,
                    const double *u, const double *delta, const double *A,
                    const double *B, const double *C, const double *Dv,
                    const double *z, double *y, int nthreads) {
    if (N > ORACLE_MAX_N || N < 1) return -1;
    int64_t nch = S * D;
#pragma omp parallel for schedule(static) num_threads(nthreads)
    for (int64_t ch = 0; ch < nch; ++ch) {
        int64_t s = ch / D, d = ch % D;
        double *h = state + (s * D + d) * N;
        const double *Bs = B + s * N;
        const double *Cs = C + s * N;
        double dt = delta[ch];
        double ut = u[ch];
        for (int64_t n = 0; n < N; ++n) {
            double dA = exp(dt * A[d * N + n]);
            h[n] = dA * h[n] + dt * Bs[n] * ut;
        }
        double acc = 0.0;
        for (int64_t n = 0; n < N; ++n) acc = acc + Cs[n] * h[n];
        double yt = acc;
        if (Dv) yt = yt + Dv[d] * ut;
        if (z) yt = yt * oracle_silu(z[ch]);
        y[ch] = yt;
    }
    return 0;
}
