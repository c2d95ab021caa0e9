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
 *    B_bar formula); with the exact-ZOH flag it is B_bar = (exp(delta A) - 1) / A * B, the
 *    zero-order hold of the same diagonal system (delta * B in the limit A = 0), under
 *    which Theorem 1's gated recurrence holds exactly (azimuth.plus/paper/mamba, Theorem 1)
 *  - selection: B_t, C_t and delta_t vary per token, delta_t = softplus(linear(x_t)),
 *    A stays fixed (azimuth.plus/paper/mamba, "selection" section, the three bullets and
 *    the remark that A alone stays fixed)
 *  - the recurrence h_t = A_bar_t h_{t-1} + B_bar_t x_t
 *      (azimuth.plus/paper/mamba, hardware-aware algorithm section, "parallel scan" bullet)
 *  - the gate branch multiplies the SSM branch elementwise after SiLU
 *      (azimuth.plus/paper/mamba, block architecture section)
 *  - the recurrent (inference) form: constant memory, one state update per token
 *      (shakilmahmud.com section 3; urworte.de "Methodische Grundlagen")
 *  - the short causal convolution and SiLU that produce the scan's input in the block's
 *      main branch (azimuth.plus/paper/mamba, block architecture section)
 *  - Mamba-2's state space dual layer: a scalar state matrix per head, whose sequence map
 *      is a 1-semiseparable matrix (mugbit.ir, Mamba-2 / structured state space duality)
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
#include <stdlib.h>
#include <string.h>

#define ORACLE_MAX_N 256

int ssm_oracle_max_n(void) { return ORACLE_MAX_N; }

/* softplus(x) = log(1 + e^x), written so that neither branch overflows. */
static double oracle_softplus(double x) {
    if (x > 0.0) return x + log1p(exp(-x));
    return log1p(exp(x));
}

/* silu(z) = z * sigmoid(z) = z / (1 + e^-z). */
/* Bits of `flags`: the step size is softplus(delta + bias); the input term uses the
 * exact zero-order-hold B_bar. */
#define ORACLE_SOFTPLUS 1
#define ORACLE_EXACT_ZOH 2

/* B_bar / B for one state under exact ZOH: (exp(dt a) - 1) / a, and dt when a = 0. */
static double oracle_zoh_coef(double dt, double a) { return a != 0.0 ? expm1(dt * a) / a : dt; }

/* d/da of the exact-ZOH coefficient (exp(dt a) - 1) / a: (dt exp(dt a) - (exp(dt a) - 1) / a) / a,
 * which tends to dt^2 / 2 at a = 0.  Where |dt a| < 1e-3 the closed form loses digits to
 * cancellation, and the power series of the same function is used instead:
 * dt^2 (1/2 + x/3 + x^2/8 + x^3/30 + x^4/144), x = dt a (term k: (k+1) x^k / (k+2)!). */
static double oracle_zoh_coef_da(double dt, double a) {
    double x = dt * a;
    if (fabs(x) < 1e-3)
        return dt * dt * (0.5 + x * (1.0 / 3.0 + x * (1.0 / 8.0 + x * (1.0 / 30.0 + x / 144.0))));
    return (dt * exp(x) - expm1(x) / a) / a;
}

static double oracle_silu(double z) { return z / (1.0 + exp(-z)); }

/* sigmoid(x) = 1 / (1 + e^-x), written so that e^x is only taken of x <= 0. */
static double oracle_sigmoid(double x) {
    if (x >= 0.0) return 1.0 / (1.0 + exp(-x));
    double e = exp(x);
    return e / (1.0 + e);
}

/*
 * Scan over one batch of sequences, continuing from the state h0 (the recurrent form
 * carries the state from one stretch of tokens to the next: shakilmahmud.com section 3).
 *   u, delta, z, y : [bsz][L][D]      B, C : [bsz][L][N]
 *   A : [D][N]     Dv, delta_bias : [D]   (Dv, z, delta_bias may be NULL)
 *   h0, last_state : [bsz][D][N] or NULL (h0 NULL: start from zero)
 *   flags: ORACLE_SOFTPLUS | ORACLE_EXACT_ZOH
 * Channels (b, d) are independent; they are spread over `nthreads` OpenMP threads,
 * each walking its channel's tokens in order.  Returns 0, or -1 if N is too large.
 */
int ssm_oracle_scan_from(int64_t bsz, int64_t L, int64_t D, int64_t N, const double *h0,
                         const double *u, const double *delta, const double *A,
                         const double *B, const double *C, const double *Dv,
                         const double *z, const double *delta_bias, int flags,
                         double *y, double *last_state, int nthreads) {
    if (N > ORACLE_MAX_N || N < 1) return -1;
    const int softplus_flag = flags & ORACLE_SOFTPLUS;
    const int zoh = flags & ORACLE_EXACT_ZOH;
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
            if (zoh) {
                for (int64_t n = 0; n < N; ++n) {
                    double a = A[d * N + n];
                    h[n] = exp(dt * a) * h[n] + oracle_zoh_coef(dt, a) * Bt[n] * ut;
                }
            } else {
                for (int64_t n = 0; n < N; ++n) {
                    double dA = exp(dt * A[d * N + n]);
                    h[n] = dA * h[n] + dt * Bt[n] * ut;
                }
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
                    const double *z, const double *delta_bias, int flags,
                    double *y, double *last_state, int nthreads) {
    return ssm_oracle_scan_from(bsz, L, D, N, NULL, u, delta, A, B, C, Dv, z, delta_bias, flags,
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

/*
 * Gradients of the scan from h0 (reverse mode of the recurrence, written out): given
 * dy = dLoss/dy and dlast = dLoss/d(last_state) (NULL = 0), returns the gradients with
 * respect to every input.  Per channel the forward states h_t are kept, then the tokens
 * are walked backwards with the adjoint G = dLoss/dh_t carried from token t+1
 * (G <- dA_t * lambda_t), where lambda_t = C_t dp_t + G is the full gradient w.r.t. h_t and
 * dp_t = dy_t silu(z_t) the gradient w.r.t. the ungated output:
 *   du_t     = D dp_t + sum_n lambda_t[n] m_t[n] B_t[n]
 *   ddelta_t = (sum_n lambda_t[n] (A[n] dA_t[n] h_{t-1}[n] + m'_t[n] B_t[n] u_t)) * softplus'(x_t)
 *   dA[n]   += lambda_t[n] (delta_t dA_t[n] h_{t-1}[n] + dm_t[n]/dA[n] B_t[n] u_t)
 *   dB_t[n] += lambda_t[n] m_t[n] u_t,   dC_t[n] += dp_t h_t[n]   (summed over channels)
 *   dD      += dp_t u_t,  ddelta_bias += ddelta_t,  dz_t = dy_t p_t silu'(z_t)
 *   dh0      = the adjoint left after token 0
 * with softplus'(x) = sigmoid(x) and silu'(z) = sigmoid(z) (1 + z (1 - sigmoid(z))).  m is
 * the input term's coefficient: delta itself (m' = 1, dm/dA = 0), or under the exact ZOH
 * (exp(delta A) - 1) / A (m' = exp(delta A) = dA_t, dm/dA = oracle_zoh_coef_da).
 * Shapes and flags as ssm_oracle_scan_from; du, ddelta, dz [bsz][L][D]; dA [D][N]; dB, dC
 * [bsz][L][N]; dD, dbias [D]; dh0 [bsz][D][N].  Every output is overwritten; dz, dD,
 * dbias, dh0 may be NULL (not wanted).  Channels d are spread over the threads (each
 * thread owns dA, dD, dbias of its channels); dB and dC are summed over channels from
 * per-thread buffers.  Returns 0, or -1 if N is too large or memory is short.
 */
int ssm_oracle_scan_bwd(int64_t bsz, int64_t L, int64_t D, int64_t N, const double *h0,
                        const double *u, const double *delta, const double *A,
                        const double *B, const double *C, const double *Dv,
                        const double *z, const double *delta_bias, int flags,
                        const double *dy, const double *dlast,
                        double *du, double *ddelta, double *dA, double *dB, double *dC,
                        double *dD, double *dz, double *dbias, double *dh0, int nthreads) {
    if (N > ORACLE_MAX_N || N < 1) return -1;
    const int softplus_flag = flags & ORACLE_SOFTPLUS;
    const int zoh = flags & ORACLE_EXACT_ZOH;
    const int64_t nbt = bsz * L * N;
    memset(dB, 0, sizeof(double) * (size_t)nbt);
    memset(dC, 0, sizeof(double) * (size_t)nbt);
    int fail = 0;
#pragma omp parallel num_threads(nthreads)
    {
        double *hist = malloc(sizeof(double) * (size_t)((L > 0 ? L : 1) * N));   /* h_t */
        double *decay = malloc(sizeof(double) * (size_t)((L > 0 ? L : 1) * N));  /* dA_t */
        double *coef = malloc(sizeof(double) * (size_t)((L > 0 ? L : 1) * N));   /* m_t */
        double *dt = malloc(sizeof(double) * (size_t)(L > 0 ? L : 1));
        double *dBl = calloc((size_t)(nbt > 0 ? nbt : 1), sizeof(double));
        double *dCl = calloc((size_t)(nbt > 0 ? nbt : 1), sizeof(double));
        const int have = hist && decay && coef && dt && dBl && dCl;
#pragma omp for schedule(static)
        for (int64_t d = 0; d < D; ++d) {
            if (!have) {
#pragma omp atomic write
                fail = 1;
                continue;
            }
            double dD_d = 0.0, dbias_d = 0.0;
            for (int64_t n = 0; n < N; ++n) dA[d * N + n] = 0.0;
            for (int64_t b = 0; b < bsz; ++b) {
                /* forward, keeping every state */
                double h[ORACLE_MAX_N], hinit[ORACLE_MAX_N], G[ORACLE_MAX_N];
                for (int64_t n = 0; n < N; ++n) {
                    hinit[n] = h0 ? h0[(b * D + d) * N + n] : 0.0;
                    h[n] = hinit[n];
                }
                for (int64_t t = 0; t < L; ++t) {
                    int64_t i = (b * L + t) * D + d;
                    const double *Bt = B + (b * L + t) * N;
                    double x = delta[i];
                    if (delta_bias) x = x + delta_bias[d];
                    dt[t] = softplus_flag ? oracle_softplus(x) : x;
                    for (int64_t n = 0; n < N; ++n) {
                        double a = exp(dt[t] * A[d * N + n]);
                        double m = zoh ? oracle_zoh_coef(dt[t], A[d * N + n]) : dt[t];
                        h[n] = a * h[n] + m * Bt[n] * u[i];
                        decay[t * N + n] = a;
                        coef[t * N + n] = m;
                        hist[t * N + n] = h[n];
                    }
                }
                /* backward */
                for (int64_t n = 0; n < N; ++n) G[n] = dlast ? dlast[(b * D + d) * N + n] : 0.0;
                for (int64_t t = L - 1; t >= 0; --t) {
                    int64_t i = (b * L + t) * D + d;
                    const double *Bt = B + (b * L + t) * N;
                    const double *Ct = C + (b * L + t) * N;
                    double ut = u[i];
                    double p = 0.0;
                    for (int64_t n = 0; n < N; ++n) p = p + Ct[n] * hist[t * N + n];
                    if (Dv) p = p + Dv[d] * ut;
                    double g = z ? oracle_silu(z[i]) : 1.0;
                    double dp = dy[i] * g;
                    if (dz) {
                        if (z) {
                            double sg = oracle_sigmoid(z[i]);
                            dz[i] = dy[i] * p * (sg * (1.0 + z[i] * (1.0 - sg)));
                        } else {
                            dz[i] = 0.0;
                        }
                    }
                    dD_d = dD_d + dp * ut;
                    double du_t = Dv ? Dv[d] * dp : 0.0;
                    double dd = 0.0;
                    for (int64_t n = 0; n < N; ++n) {
                        double lam = Ct[n] * dp + G[n];
                        double hprev = t > 0 ? hist[(t - 1) * N + n] : hinit[n];
                        double a = decay[t * N + n];
                        double m = coef[t * N + n];
                        double dm_ddt = zoh ? a : 1.0;   /* d m / d delta */
                        dCl[(b * L + t) * N + n] += dp * hist[t * N + n];
                        dBl[(b * L + t) * N + n] += lam * m * ut;
                        du_t = du_t + lam * m * Bt[n];
                        dd = dd + lam * (A[d * N + n] * a * hprev + dm_ddt * Bt[n] * ut);
                        dA[d * N + n] += lam * dt[t] * a * hprev;
                        if (zoh) dA[d * N + n] += lam * oracle_zoh_coef_da(dt[t], A[d * N + n]) * Bt[n] * ut;
                        G[n] = a * lam;
                    }
                    double x = delta[i];
                    if (delta_bias) x = x + delta_bias[d];
                    double dx = softplus_flag ? dd * oracle_sigmoid(x) : dd;
                    du[i] = du_t;
                    ddelta[i] = dx;
                    dbias_d = dbias_d + dx;
                }
                if (dh0)
                    for (int64_t n = 0; n < N; ++n) dh0[(b * D + d) * N + n] = G[n];
            }
            if (dD) dD[d] = dD_d;
            if (dbias) dbias[d] = dbias_d;
        }
        if (have) {
#pragma omp critical
            {
                for (int64_t k = 0; k < nbt; ++k) {
                    dB[k] += dBl[k];
                    dC[k] += dCl[k];
                }
            }
        }
        free(hist);
        free(decay);
        free(coef);
        free(dt);
        free(dBl);
        free(dCl);
    }
    return fail ? -1 : 0;
}

/*
 * The causal depthwise convolution of the block's main branch, then optionally SiLU:
 * the input of the selective scan comes from a short 1-D convolution over time (kernel
 * size 4) followed by SiLU (azimuth.plus/paper/mamba, block architecture section).
 * Depthwise: every channel has its own filter of `width` taps; causal: token t sees only
 * tokens t-width+1 .. t, with the inputs before token 0 taken from `state` (zeros if NULL).
 *   x, out       : [bsz][L][D]
 *   w            : [D][width], tap k multiplying x[t - (width-1) + k]
 *   bias         : [D] or NULL (= 0)
 *   state        : [bsz][width-1][D], the width-1 inputs before token 0, oldest first, or NULL
 *   silu         : nonzero = out = silu(pre-activation)
 *   state_out    : [bsz][width-1][D], the last width-1 inputs of (state, x), or NULL
 * Returns 0, or -1 for a width outside 1..16 or a failed allocation.
 */
int ssm_oracle_conv1d(int64_t bsz, int64_t L, int64_t D, int64_t width, const double *x,
                      const double *w, const double *bias, const double *state, int silu,
                      double *out, double *state_out) {
    if (width < 1 || width > 16) return -1;
    const int64_t H = width - 1;           /* history rows before token 0 */
    double *hist = malloc(sizeof(double) * (size_t)(H + L > 0 ? H + L : 1));
    if (!hist) return -1;
    for (int64_t b = 0; b < bsz; ++b) {
        for (int64_t d = 0; d < D; ++d) {
            /* the channel's inputs in time order: the state rows, then x */
            for (int64_t r = 0; r < H; ++r) hist[r] = state ? state[(b * H + r) * D + d] : 0.0;
            for (int64_t t = 0; t < L; ++t) hist[H + t] = x[(b * L + t) * D + d];
            for (int64_t t = 0; t < L; ++t) {
                double acc = bias ? bias[d] : 0.0;
                for (int64_t k = 0; k < width; ++k) acc = acc + w[d * width + k] * hist[t + k];
                out[(b * L + t) * D + d] = silu ? oracle_silu(acc) : acc;
            }
            if (state_out)
                for (int64_t r = 0; r < H; ++r) state_out[(b * H + r) * D + d] = hist[L + r];
        }
    }
    free(hist);
    return 0;
}

/*
 * Gradients of ssm_oracle_conv1d given dout = dLoss/dout.  The pages give the forward only
 * (a short causal convolution over time, then SiLU: azimuth.plus/paper/mamba, block
 * architecture section); its backward is the chain rule through that definition, written
 * out per channel with the same history array as the forward:
 *   pre[t]   = bias + sum_k w[k] hist[t+k]            (hist = the state rows, then x)
 *   g[t]     = dout[t] * silu'(pre[t])  with silu'(p) = s (1 + p (1 - s)), s = sigmoid(p);
 *              g[t] = dout[t] without SiLU
 *   dhist[j] = sum over (t, k) with t + k = j of w[k] g[t]
 *   dx[t]    = dhist[H + t],   dstate[r] = dhist[r]   (H = width - 1)
 *   dw[k]    = sum over sequences and tokens of g[t] hist[t+k],   dbias = sum of g[t]
 *   dx           : [bsz][L][D]            dw : [D][width]
 *   dbias        : [D] or NULL            dstate : [bsz][width-1][D] or NULL
 * (the final-window output state_out is taken to carry no gradient).  Returns 0, or -1 for
 * a width outside 1..16 or a failed allocation.
 */
int ssm_oracle_conv1d_bwd(int64_t bsz, int64_t L, int64_t D, int64_t width, const double *x,
                          const double *w, const double *bias, const double *state, int silu,
                          const double *dout, double *dx, double *dw, double *dbias, double *dstate) {
    if (width < 1 || width > 16) return -1;
    const int64_t H = width - 1;
    const int64_t n = H + L > 0 ? H + L : 1;
    double *hist = malloc(sizeof(double) * (size_t)n);
    double *dhist = malloc(sizeof(double) * (size_t)n);
    double *g = malloc(sizeof(double) * (size_t)(L > 0 ? L : 1));
    if (!hist || !dhist || !g) {
        free(hist);
        free(dhist);
        free(g);
        return -1;
    }
    for (int64_t d = 0; d < D; ++d) {
        for (int64_t k = 0; k < width; ++k) dw[d * width + k] = 0.0;
        if (dbias) dbias[d] = 0.0;
    }
    for (int64_t b = 0; b < bsz; ++b) {
        for (int64_t d = 0; d < D; ++d) {
            for (int64_t r = 0; r < H; ++r) hist[r] = state ? state[(b * H + r) * D + d] : 0.0;
            for (int64_t t = 0; t < L; ++t) hist[H + t] = x[(b * L + t) * D + d];
            /* dLoss/dpre at every token */
            for (int64_t t = 0; t < L; ++t) {
                double pre = bias ? bias[d] : 0.0;
                for (int64_t k = 0; k < width; ++k) pre = pre + w[d * width + k] * hist[t + k];
                const double go = dout[(b * L + t) * D + d];
                if (silu) {
                    const double s = oracle_sigmoid(pre);
                    g[t] = go * (s * (1.0 + pre * (1.0 - s)));
                } else {
                    g[t] = go;
                }
            }
            /* through the taps: to the inputs, the filter and the bias */
            for (int64_t j = 0; j < H + L; ++j) dhist[j] = 0.0;
            for (int64_t t = 0; t < L; ++t) {
                for (int64_t k = 0; k < width; ++k) {
                    dhist[t + k] = dhist[t + k] + w[d * width + k] * g[t];
                    dw[d * width + k] = dw[d * width + k] + g[t] * hist[t + k];
                }
                if (dbias) dbias[d] = dbias[d] + g[t];
            }
            for (int64_t t = 0; t < L; ++t) dx[(b * L + t) * D + d] = dhist[H + t];
            if (dstate)
                for (int64_t r = 0; r < H; ++r) dstate[(b * H + r) * D + d] = dhist[r];
        }
    }
    free(hist);
    free(dhist);
    free(g);
    return 0;
}

/*
 * The state space dual layer (SSD) of Mamba-2 (mugbit.ir, the Mamba-2 / structured state
 * space duality section): the selective scan with a scalar state matrix per head, so that
 * the sequence map is a 1-semiseparable matrix.  Per head h (P channels, group g = h / (H/G)
 * of the B / C projections) the state is a P x N matrix:
 *   dt_t      = softplus(dt_in[t,h] + dt_bias[h]) with the softplus flag, else dt_in + dt_bias
 *   S_t[p,n]  = exp(dt_t A[h]) S_{t-1}[p,n] + dt_t x_t[p] B_t[g,n]
 *   y_t[p]    = (sum_n C_t[g,n] S_t[p,n] + D[h] x_t[p]) * silu(z_t[p])      (z optional)
 *   x, z, y    : [bsz][L][H][P]     dt_in : [bsz][L][H]     A, dt_bias, D : [H]
 *   B, C       : [bsz][L][G][N]     h0, last_state : [bsz][H][P][N] (h0 NULL = zero)
 * Channels (b, h, p) are independent; spread over `nthreads` threads.  Returns 0, or -1 for
 * N too large or H not a multiple of G.
 */
int ssm_oracle_ssd(int64_t bsz, int64_t L, int64_t H, int64_t P, int64_t G, int64_t N,
                   const double *h0, const double *x, const double *dt_in, const double *A,
                   const double *B, const double *C, const double *Dv, const double *z,
                   const double *dt_bias, int flags, double *y, double *last_state, int nthreads) {
    if (N > ORACLE_MAX_N || N < 1 || G < 1 || H % G != 0) return -1;
    const int softplus_flag = flags & ORACLE_SOFTPLUS;
    const int64_t hpg = H / G;
    int64_t nch = bsz * H * P;
#pragma omp parallel for schedule(dynamic, 1) num_threads(nthreads)
    for (int64_t ch = 0; ch < nch; ++ch) {
        int64_t b = ch / (H * P), h = (ch / P) % H, p = ch % P, g = h / hpg;
        double s[ORACLE_MAX_N];
        for (int64_t n = 0; n < N; ++n) s[n] = h0 ? h0[((b * H + h) * P + p) * N + n] : 0.0;
        for (int64_t t = 0; t < L; ++t) {
            double v = dt_in[(b * L + t) * H + h];
            if (dt_bias) v = v + dt_bias[h];
            double dt = softplus_flag ? oracle_softplus(v) : v;
            double dA = exp(dt * A[h]);
            int64_t i = ((b * L + t) * H + h) * P + p;   /* (b, t, h, p) */
            const double *Bt = B + ((b * L + t) * G + g) * N;
            const double *Ct = C + ((b * L + t) * G + g) * N;
            double acc = 0.0;
            for (int64_t n = 0; n < N; ++n) {
                s[n] = dA * s[n] + dt * x[i] * Bt[n];
                acc = acc + Ct[n] * s[n];
            }
            double yt = acc;
            if (Dv) yt = yt + Dv[h] * x[i];
            if (z) yt = yt * oracle_silu(z[i]);
            y[i] = yt;
        }
        if (last_state)
            for (int64_t n = 0; n < N; ++n) last_state[((b * H + h) * P + p) * N + n] = s[n];
    }
    return 0;
}
