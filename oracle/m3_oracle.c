/*
 * m3_oracle.c -- TEST INFRASTRUCTURE ONLY.
 *
 * A plain, slow, sequential fp64 CPU implementation of the Mamba-3 SSM scan.
 * Only tests/, the smoke check and the benchmark's cpu_baseline leg may load
 * it.  It shares no code, header or constant with the HIP library.
 *
 * What it computes (per batch b and head h, group g = h / (H/G), tokens t = 1..L):
 *
 *   U_t   = B_t X_t                       B_t in R^{N x R}, X_t in R^{R x P}
 *           -- MIMO rank-R input: "Mamba-3 paper note" (docsaid.org),
 *              section "Solution 3: MIMO" (R input/output branches, rank-R write).
 *   alpha_t = exp(dt_t * A_h)
 *   beta_t  = (1 - lambda_t) * dt_t * alpha_t
 *   gamma_t = lambda_t * dt_t
 *           -- same note, section "Solution 1: a more expressive discretisation",
 *              exponential-trapezoidal recurrence and its alpha/beta/gamma.
 *   M_t   = block-diagonal of 2x2 counter-clockwise rotations by theta_{t,k}
 *           acting on the pair of state rows (2k, 2k+1)
 *           -- same note, section "Solution 2: a complex state that rotates"
 *              (complex SSM == real SSM of twice the size whose transition is the
 *              decay times a block-diagonal of 2x2 rotations; the rotation matrix
 *              of the parity example fixes the direction).
 *   h_t   = alpha_t M_t h_{t-1} + beta_t M_t U_{t-1} + gamma_t U_t
 *           (the complex transition multiplies the beta term as well: beta_t
 *            carries exp(dt_t * A_t) with complex A_t, so the rotation rides along)
 *   Y_t   = C_t^T h_t + D_h X_t           (R x P outputs)
 *           -- output equation y = C h + D x: IBM "What is a Mamba model?",
 *              section on the state and output equations.
 *
 * Per-token decay rate (m3o_scan_ex with a_per_token): the note writes A_t per
 * token in the discretisation; with a_per_token set, A is (batch, L, H) and
 * alpha_t = exp(dt_t * A_t) -- the same recurrence with the per-head A replaced.
 *
 * Start of a scan: h_0 and the previous input (B_0, X_0) come from the optional
 * state_in; absent, both are zero.  state_out is (h_L, B_L, X_L).
 *
 * Reduced-precision state (m3o_scan_rounded): a state kept in bf16 between
 * steps is the same recurrence with h_t replaced by its nearest bf16 value
 * (round to nearest, ties to even) after every token t flagged in round_after,
 * once Y_t has been formed from the unrounded h_t.  A decode step that reads
 * and writes a bf16 state rounds after every token; a prefill that only writes
 * its final state in bf16 rounds after its last token.
 *
 * All inputs and outputs are fp64 arrays (fp32 and bf16 values are exact in
 * fp64, so the kernels' inputs pass through unchanged).
 *
 * Layouts (contiguous, row-major, last index fastest):
 *   x, y  (batch, L, H, R, P)      dt, lambda (batch, L, H)      A, D (H)
 *   theta (batch, L, G, N/2)       B, C (batch, L, G, R, N)
 *   h0, h_out (batch, H, N, P)     b_last (batch, G, R, N)       x_last (batch, H, R, P)
 *
 * Pins: every function here is checked by tests/test_oracle_pins.py against
 * special cases, a brute-force matrix form, an independent complex-number
 * formulation, an ODE convergence order and the worked parity example printed
 * on the Mamba-3 note; no function is "parity unpinned".
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

typedef struct {
    int64_t batch, seqlen, nheads, ngroups, headdim, dstate, rank;
} m3o_dims;

#define IDX5(a, b, c, d, e, B_, C_, D_, E_) ((((((a) * (B_) + (b)) * (C_) + (c)) * (D_) + (d)) * (E_)) + (e))

/* Nearest bf16 value (8 significant bits, fp32's exponent range), ties to even.
 * v = m 2^e with 0.5 <= |m| < 1; keep 8 bits of m with the default rounding
 * mode of nearbyint (to nearest, ties to even).  Values below fp32's smallest
 * normal number keep fp32's absolute spacing there, 2^-133 at bf16 precision. */
double m3o_round_bf16(double v) {
    if (v == 0.0 || isnan(v) || isinf(v)) return v;
    int e;
    const double m = frexp(v, &e);
    if (e < -125) return ldexp(nearbyint(ldexp(v, 133)), -133);
    const double r = ldexp(nearbyint(ldexp(m, 8)), e - 8);
    return fabs(r) > 3.3895313892515355e38 ? copysign(INFINITY, v) : r;
}

/* Scan one (batch b, head h) slice through all L tokens. */
static void scan_slice(const m3o_dims* dm, int64_t b, int64_t h,
                       const double* x, const double* dt, const double* A, int a_per_token,
                       const double* lam, const double* theta, const double* B,
                       const double* C, const double* D,
                       const double* h0, const double* b_last, const double* x_last,
                       const unsigned char* round_after,
                       double* y, double* h_out, double* hs, double* U, double* Uprev) {
    const int64_t L = dm->seqlen, H = dm->nheads, G = dm->ngroups;
    const int64_t P = dm->headdim, N = dm->dstate, R = dm->rank, K = N / 2;
    const int64_t g = h / (H / G);

    /* h_0 */
    for (int64_t i = 0; i < N * P; ++i) hs[i] = h0 ? h0[(b * H + h) * N * P + i] : 0.0;
    /* U_0 = B_0 X_0 (the previous token's input term) */
    for (int64_t n = 0; n < N; ++n)
        for (int64_t p = 0; p < P; ++p) {
            double u = 0.0;
            if (b_last && x_last)
                for (int64_t r = 0; r < R; ++r)
                    u += b_last[((b * G + g) * R + r) * N + n] *
                         x_last[((b * H + h) * R + r) * P + p];
            Uprev[n * P + p] = u;
        }

    for (int64_t t = 0; t < L; ++t) {
        const double dtv = dt[(b * L + t) * H + h];
        const double lv = lam[(b * L + t) * H + h];
        const double a_th = a_per_token ? A[(b * L + t) * H + h] : A[h];
        const double alpha = exp(dtv * a_th);
        const double beta = (1.0 - lv) * dtv * alpha;
        const double gamma = lv * dtv;

        /* U_t = B_t X_t : U[n][p] = sum_r B[n][r] X[r][p] */
        for (int64_t n = 0; n < N; ++n)
            for (int64_t p = 0; p < P; ++p) {
                double u = 0.0;
                for (int64_t r = 0; r < R; ++r)
                    u += B[IDX5(b, t, g, r, n, L, G, R, N)] *
                         x[IDX5(b, t, h, r, p, L, H, R, P)];
                U[n * P + p] = u;
            }

        /* h_t = alpha M h + beta M U_{t-1} + gamma U_t, M rotating pairs (2k, 2k+1) */
        for (int64_t k = 0; k < K; ++k) {
            const double th = theta[((b * L + t) * G + g) * K + k];
            const double c = cos(th), s = sin(th);
            double* h0r = hs + (2 * k) * P;
            double* h1r = hs + (2 * k + 1) * P;
            const double* u0p = Uprev + (2 * k) * P;
            const double* u1p = Uprev + (2 * k + 1) * P;
            const double* u0 = U + (2 * k) * P;
            const double* u1 = U + (2 * k + 1) * P;
            for (int64_t p = 0; p < P; ++p) {
                const double mh0 = c * h0r[p] - s * h1r[p];   /* M h     */
                const double mh1 = s * h0r[p] + c * h1r[p];
                const double mu0 = c * u0p[p] - s * u1p[p];   /* M U_{t-1} */
                const double mu1 = s * u0p[p] + c * u1p[p];
                h0r[p] = alpha * mh0 + beta * mu0 + gamma * u0[p];
                h1r[p] = alpha * mh1 + beta * mu1 + gamma * u1[p];
            }
        }

        /* Y_t = C_t^T h_t + D X_t */
        for (int64_t r = 0; r < R; ++r)
            for (int64_t p = 0; p < P; ++p) {
                double acc = 0.0;
                for (int64_t n = 0; n < N; ++n)
                    acc += C[IDX5(b, t, g, r, n, L, G, R, N)] * hs[n * P + p];
                const int64_t xi = IDX5(b, t, h, r, p, L, H, R, P);
                y[xi] = acc + D[h] * x[xi];
            }

        if (round_after && round_after[t])
            for (int64_t i = 0; i < N * P; ++i) hs[i] = m3o_round_bf16(hs[i]);

        memcpy(Uprev, U, sizeof(double) * N * P);
    }
    if (h_out) memcpy(h_out + (b * H + h) * N * P, hs, sizeof(double) * N * P);
}

/*
 * Full scan.  Returns 0 on success, -1 on a shape error (N odd, H % G != 0,
 * non-positive sizes, y NULL), -2 if scratch memory cannot be allocated.
 * nthreads <= 0 uses the OpenMP default.  h_out may be NULL.
 * (b_last, x_last) are used only when both are non-NULL.  round_after is NULL
 * (full-precision state) or one flag per token (length L, shared by all slices).
 */
int m3o_scan_ex(const m3o_dims* dm, const double* x, const double* dt, const double* A,
                int a_per_token, const double* lam, const double* theta, const double* B,
                const double* C, const double* D, const double* h0, const double* b_last,
                const double* x_last, const unsigned char* round_after, double* y,
                double* h_out, int nthreads) {
    if (!dm || !y || dm->batch < 0 || dm->seqlen < 0 || dm->nheads <= 0 || dm->ngroups <= 0 ||
        dm->headdim <= 0 || dm->dstate <= 0 || dm->rank <= 0)
        return -1;
    if (dm->dstate % 2 != 0 || dm->nheads % dm->ngroups != 0) return -1;
    const int64_t NP = dm->dstate * dm->headdim;
    const int64_t nslices = dm->batch * dm->nheads;
    int err = 0;
#ifdef _OPENMP
    if (nthreads > 0) omp_set_num_threads(nthreads);
#else
    (void)nthreads;
#endif
#pragma omp parallel
    {
        double* scratch = (double*)malloc(sizeof(double) * 3 * (size_t)NP);
        if (!scratch) {
#pragma omp atomic write
            err = -2;
        }
#pragma omp for schedule(dynamic, 1)
        for (int64_t s = 0; s < nslices; ++s) {
            if (!scratch) continue;
            const int64_t b = s / dm->nheads, h = s % dm->nheads;
            scan_slice(dm, b, h, x, dt, A, a_per_token, lam, theta, B, C, D, h0, b_last, x_last,
                       round_after, y, h_out, scratch, scratch + NP, scratch + 2 * NP);
        }
        free(scratch);
    }
    return err;
}

/* The scan with one decay rate A per head (H), optionally rounding the state. */
int m3o_scan_rounded(const m3o_dims* dm, const double* x, const double* dt, const double* A,
                     const double* lam, const double* theta, const double* B, const double* C,
                     const double* D, const double* h0, const double* b_last,
                     const double* x_last, const unsigned char* round_after, double* y,
                     double* h_out, int nthreads) {
    return m3o_scan_ex(dm, x, dt, A, 0, lam, theta, B, C, D, h0, b_last, x_last, round_after, y,
                       h_out, nthreads);
}

/* The scan with a full-precision state (no rounding). */
int m3o_scan(const m3o_dims* dm, const double* x, const double* dt, const double* A,
             const double* lam, const double* theta, const double* B, const double* C,
             const double* D, const double* h0, const double* b_last, const double* x_last,
             double* y, double* h_out, int nthreads) {
    return m3o_scan_rounded(dm, x, dt, A, lam, theta, B, C, D, h0, b_last, x_last, NULL, y,
                            h_out, nthreads);
}

/* Number of OpenMP threads a parallel region would use (for reporting). */
int m3o_max_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/*
 * Backward pass (reverse-mode derivative) of the scan, for training.
 *
 * Given output cotangents dy (batch, L, H, R, P) and, optionally, a cotangent
 * dh_out (batch, H, N, P) of the final state, returns the gradient of
 *     Lsum = sum_t <dy_t, Y_t> + <dh_out, h_L>
 * with respect to every input of m3o_scan: dx, ddt, dlambda (shapes of their
 * inputs), dA and dD (H), dtheta (batch, L, G, N/2), dB and dC (batch, L, G, R, N)
 * (summed over the heads of a group, which share B, C and theta), dh0, and the
 * carried previous input db_last / dx_last when a carry is given.
 *
 * It is the same recurrence run backwards (adjoint method), written from the
 * forward definition above: with g_t = dLsum/dh_t and q_t = M_t^T g_t,
 *   g_t     = sum_r C_t[:,r] dy_t[r,:]^T + alpha_{t+1} q_{t+1}
 *   dU_t    = gamma_t g_t + beta_{t+1} q_{t+1}                 (U_t feeds h_t and h_{t+1})
 *   dalpha_t = <q_t, h_{t-1}>,  dbeta_t = <q_t, U_{t-1}>,  dgamma_t = <g_t, U_t>
 *   dtheta_{t,k} = sum_p ( q_t[2k+1,p] v_t[2k,p] - q_t[2k,p] v_t[2k+1,p] ),
 *                  v_t = alpha_t h_{t-1} + beta_t U_{t-1}     (derivative of the 2x2 rotation)
 *   dC_t[:,r] = h_t dy_t[r,:],  dB_t[:,r] = dU_t X_t[r,:],  dX_t[r,:] = D dy_t[r,:] + B_t[:,r]^T dU_t
 *   dD = sum_t <dy_t, X_t>,  dh0 = alpha_1 q_1,  dU_0 = beta_1 q_1 (the carried input)
 * and the chain rule through alpha = exp(dt A), beta = (1 - lambda) dt alpha,
 * gamma = lambda dt for ddt, dlambda and dA.  With a per-token decay rate
 * (a_per_token: A is (batch, L, H), the A_t of the discretisation) A is read at
 * each token and its gradient is written per token to dA_tok instead of summed
 * per head.
 *
 * The forward states are recomputed and kept for the whole slice (fp64, L + 1
 * states of N x P), which suits the small sizes it is used at.
 * Returns 0, -1 on a shape error, -2 if memory cannot be allocated.
 */
static int backward_batch(const m3o_dims* dm, int64_t b,
                          const double* x, const double* dt, const double* A, int a_per_token,
                          double* dA_tok, const double* lam,
                          const double* theta, const double* B, const double* C, const double* D,
                          const double* h0, const double* b_last, const double* x_last,
                          const double* dy, const double* dh_out,
                          double* dx, double* ddt, double* dA_b, double* dlam, double* dtheta,
                          double* dB, double* dC, double* dD_b, double* dh0, double* db_last,
                          double* dx_last) {
    const int64_t L = dm->seqlen, H = dm->nheads, G = dm->ngroups;
    const int64_t P = dm->headdim, N = dm->dstate, R = dm->rank, K = N / 2, NP = N * P;
    const int carry = (b_last && x_last);
    double* hall = (double*)malloc(sizeof(double) * (size_t)(L + 1) * NP);
    double* work = (double*)malloc(sizeof(double) * 6 * (size_t)NP);
    if (!hall || !work) {
        free(hall);
        free(work);
        return -2;
    }
    double *U = work, *Up = work + NP, *g = work + 2 * NP, *q = work + 3 * NP, *qn = work + 4 * NP,
           *dU = work + 5 * NP;

    for (int64_t h = 0; h < H; ++h) {
        const int64_t gi = h / (H / G);
        /* forward states h_0 .. h_L of this slice (index t + 1 holds h after token t) */
        for (int64_t i = 0; i < NP; ++i) hall[i] = h0 ? h0[(b * H + h) * NP + i] : 0.0;
        for (int64_t n = 0; n < N; ++n)
            for (int64_t p = 0; p < P; ++p) {
                double u = 0.0;
                if (carry)
                    for (int64_t r = 0; r < R; ++r)
                        u += b_last[((b * G + gi) * R + r) * N + n] * x_last[((b * H + h) * R + r) * P + p];
                Up[n * P + p] = u;
            }
        for (int64_t t = 0; t < L; ++t) {
            const double dtv = dt[(b * L + t) * H + h], lv = lam[(b * L + t) * H + h];
            const double a_th = a_per_token ? A[(b * L + t) * H + h] : A[h];
            const double alpha = exp(dtv * a_th), beta = (1.0 - lv) * dtv * alpha, gamma = lv * dtv;
            for (int64_t n = 0; n < N; ++n)
                for (int64_t p = 0; p < P; ++p) {
                    double u = 0.0;
                    for (int64_t r = 0; r < R; ++r)
                        u += B[IDX5(b, t, gi, r, n, L, G, R, N)] * x[IDX5(b, t, h, r, p, L, H, R, P)];
                    U[n * P + p] = u;
                }
            const double* hp = hall + t * NP;
            double* hn = hall + (t + 1) * NP;
            for (int64_t k = 0; k < K; ++k) {
                const double th = theta[((b * L + t) * G + gi) * K + k], c = cos(th), s = sin(th);
                for (int64_t p = 0; p < P; ++p) {
                    const double v0 = alpha * hp[(2 * k) * P + p] + beta * Up[(2 * k) * P + p];
                    const double v1 = alpha * hp[(2 * k + 1) * P + p] + beta * Up[(2 * k + 1) * P + p];
                    hn[(2 * k) * P + p] = c * v0 - s * v1 + gamma * U[(2 * k) * P + p];
                    hn[(2 * k + 1) * P + p] = s * v0 + c * v1 + gamma * U[(2 * k + 1) * P + p];
                }
            }
            memcpy(Up, U, sizeof(double) * NP);
        }

        /* reverse sweep; the final-state cotangent enters as a token after the last one
           with alpha = 1, beta = 0 and no rotation */
        for (int64_t i = 0; i < NP; ++i) qn[i] = dh_out ? dh_out[(b * H + h) * NP + i] : 0.0;
        double beta_next = 0.0, alpha_next = 1.0;
        double dA_h = 0.0, dD_h = 0.0;
        for (int64_t t = L - 1; t >= 0; --t) {
            const double dtv = dt[(b * L + t) * H + h], lv = lam[(b * L + t) * H + h];
            const double a_th = a_per_token ? A[(b * L + t) * H + h] : A[h];
            const double alpha = exp(dtv * a_th), beta = (1.0 - lv) * dtv * alpha, gamma = lv * dtv;
            const double* ht = hall + (t + 1) * NP;
            const double* hp = hall + t * NP;
            /* g_t = alpha_{t+1} q_{t+1} + C_t dy_t^T */
            for (int64_t n = 0; n < N; ++n)
                for (int64_t p = 0; p < P; ++p) {
                    double a = alpha_next * qn[n * P + p];
                    for (int64_t r = 0; r < R; ++r)
                        a += C[IDX5(b, t, gi, r, n, L, G, R, N)] * dy[IDX5(b, t, h, r, p, L, H, R, P)];
                    g[n * P + p] = a;
                }
            /* output side: dC, dD, the skip part of dX */
            for (int64_t r = 0; r < R; ++r) {
                for (int64_t n = 0; n < N; ++n) {
                    double a = 0.0;
                    for (int64_t p = 0; p < P; ++p) a += ht[n * P + p] * dy[IDX5(b, t, h, r, p, L, H, R, P)];
                    dC[IDX5(b, t, gi, r, n, L, G, R, N)] += a;
                }
                for (int64_t p = 0; p < P; ++p) {
                    const int64_t xi = IDX5(b, t, h, r, p, L, H, R, P);
                    dD_h += dy[xi] * x[xi];
                    dx[xi] = D[h] * dy[xi];
                }
            }
            /* U_t, U_{t-1} */
            for (int64_t n = 0; n < N; ++n)
                for (int64_t p = 0; p < P; ++p) {
                    double u = 0.0, up = 0.0;
                    for (int64_t r = 0; r < R; ++r) {
                        u += B[IDX5(b, t, gi, r, n, L, G, R, N)] * x[IDX5(b, t, h, r, p, L, H, R, P)];
                        if (t > 0)
                            up += B[IDX5(b, t - 1, gi, r, n, L, G, R, N)] * x[IDX5(b, t - 1, h, r, p, L, H, R, P)];
                        else if (carry)
                            up += b_last[((b * G + gi) * R + r) * N + n] * x_last[((b * H + h) * R + r) * P + p];
                    }
                    U[n * P + p] = u;
                    Up[n * P + p] = up;
                }
            /* dU_t = gamma_t g_t + beta_{t+1} q_{t+1};  dgamma_t = <g_t, U_t> */
            double dgam = 0.0;
            for (int64_t i = 0; i < NP; ++i) {
                dU[i] = gamma * g[i] + beta_next * qn[i];
                dgam += g[i] * U[i];
            }
            /* q_t = M_t^T g_t; dalpha, dbeta, dtheta */
            double dal = 0.0, dbe = 0.0;
            for (int64_t k = 0; k < K; ++k) {
                const double th = theta[((b * L + t) * G + gi) * K + k], c = cos(th), s = sin(th);
                double dth = 0.0;
                for (int64_t p = 0; p < P; ++p) {
                    const double g0 = g[(2 * k) * P + p], g1 = g[(2 * k + 1) * P + p];
                    const double q0 = c * g0 + s * g1, q1 = -s * g0 + c * g1;
                    q[(2 * k) * P + p] = q0;
                    q[(2 * k + 1) * P + p] = q1;
                    const double h0v = hp[(2 * k) * P + p], h1v = hp[(2 * k + 1) * P + p];
                    const double u0 = Up[(2 * k) * P + p], u1 = Up[(2 * k + 1) * P + p];
                    dal += q0 * h0v + q1 * h1v;
                    dbe += q0 * u0 + q1 * u1;
                    const double v0 = alpha * h0v + beta * u0, v1 = alpha * h1v + beta * u1;
                    dth += q1 * v0 - q0 * v1;
                }
                dtheta[((b * L + t) * G + gi) * K + k] += dth;
            }
            /* dB_t, dX_t from dU_t */
            for (int64_t r = 0; r < R; ++r) {
                for (int64_t n = 0; n < N; ++n) {
                    double a = 0.0;
                    for (int64_t p = 0; p < P; ++p) a += dU[n * P + p] * x[IDX5(b, t, h, r, p, L, H, R, P)];
                    dB[IDX5(b, t, gi, r, n, L, G, R, N)] += a;
                }
                for (int64_t p = 0; p < P; ++p) {
                    double a = 0.0;
                    for (int64_t n = 0; n < N; ++n) a += B[IDX5(b, t, gi, r, n, L, G, R, N)] * dU[n * P + p];
                    dx[IDX5(b, t, h, r, p, L, H, R, P)] += a;
                }
            }
            /* scalars through alpha = exp(dt A), beta = (1 - lambda) dt alpha, gamma = lambda dt */
            ddt[(b * L + t) * H + h] = dal * a_th * alpha + dbe * (1.0 - lv) * (alpha + dtv * a_th * alpha) + dgam * lv;
            dlam[(b * L + t) * H + h] = -dbe * dtv * alpha + dgam * dtv;
            const double dA_t = dal * dtv * alpha + dbe * (1.0 - lv) * dtv * dtv * alpha;
            if (a_per_token)
                dA_tok[(b * L + t) * H + h] = dA_t;
            else
                dA_h += dA_t;
            memcpy(qn, q, sizeof(double) * NP);
            alpha_next = alpha;
            beta_next = beta;
        }
        /* h_0 and the carried previous input (with no token, h_L is h_0 itself and the
           final-state cotangent passes through) */
        if (dh0)
            for (int64_t i = 0; i < NP; ++i) dh0[(b * H + h) * NP + i] = alpha_next * qn[i];
        if (carry && (db_last || dx_last)) {
            for (int64_t i = 0; i < NP; ++i) dU[i] = beta_next * qn[i];
            for (int64_t r = 0; r < R; ++r) {
                if (db_last)
                    for (int64_t n = 0; n < N; ++n) {
                        double a = 0.0;
                        for (int64_t p = 0; p < P; ++p) a += dU[n * P + p] * x_last[((b * H + h) * R + r) * P + p];
                        db_last[((b * G + gi) * R + r) * N + n] += a;
                    }
                if (dx_last)
                    for (int64_t p = 0; p < P; ++p) {
                        double a = 0.0;
                        for (int64_t n = 0; n < N; ++n) a += b_last[((b * G + gi) * R + r) * N + n] * dU[n * P + p];
                        dx_last[((b * H + h) * R + r) * P + p] = a;
                    }
            }
        } else if (dx_last) {
            for (int64_t r = 0; r < R; ++r)
                for (int64_t p = 0; p < P; ++p) dx_last[((b * H + h) * R + r) * P + p] = 0.0;
        }
        dA_b[h] += dA_h;
        dD_b[h] += dD_h;
    }
    free(hall);
    free(work);
    return 0;
}

/* Backward of m3o_scan_ex (see backward_batch).  Group-shared gradients (dtheta,
 * dB, dC, db_last) and the per-head sums dA (per-head A), dD are accumulated, so
 * each batch element is handled by one thread; the outputs are overwritten, not
 * added to.  With a_per_token, A and dA are (batch, L, H).  dh_out, dh0, db_last
 * and dx_last may be NULL. */
int m3o_scan_backward_ex(const m3o_dims* dm, const double* x, const double* dt, const double* A,
                         int a_per_token, const double* lam, const double* theta, const double* B,
                         const double* C, const double* D, const double* h0, const double* b_last,
                         const double* x_last, const double* dy, const double* dh_out, double* dx,
                         double* ddt, double* dA, double* dlam, double* dtheta, double* dB, double* dC,
                         double* dD, double* dh0, double* db_last, double* dx_last, int nthreads) {
    if (!dm || !dy || !dx || !ddt || !dA || !dlam || !dtheta || !dB || !dC || !dD || dm->batch < 0 ||
        dm->seqlen < 0 || dm->nheads <= 0 || dm->ngroups <= 0 || dm->headdim <= 0 || dm->dstate <= 0 ||
        dm->rank <= 0 || dm->dstate % 2 != 0 || dm->nheads % dm->ngroups != 0)
        return -1;
    const int64_t b_ = dm->batch, L = dm->seqlen, H = dm->nheads, G = dm->ngroups;
    const int64_t N = dm->dstate, R = dm->rank;
    memset(dtheta, 0, sizeof(double) * (size_t)(b_ * L * G * (N / 2)));
    memset(dB, 0, sizeof(double) * (size_t)(b_ * L * G * R * N));
    memset(dC, 0, sizeof(double) * (size_t)(b_ * L * G * R * N));
    if (db_last) memset(db_last, 0, sizeof(double) * (size_t)(b_ * G * R * N));
    double* partial = (double*)calloc((size_t)(2 * b_ * H + 1), sizeof(double));   /* dA, dD per batch */
    if (!partial) return -2;
    int err = 0;
#ifdef _OPENMP
    if (nthreads > 0) omp_set_num_threads(nthreads);
#else
    (void)nthreads;
#endif
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t b = 0; b < b_; ++b) {
        const int rc = backward_batch(dm, b, x, dt, A, a_per_token, dA, lam, theta, B, C, D, h0, b_last, x_last, dy,
                                      dh_out, dx, ddt, partial + b * H, dlam, dtheta, dB, dC,
                                      partial + (b_ + b) * H, dh0, db_last, dx_last);
        if (rc) {
#pragma omp atomic write
            err = rc;
        }
    }
    for (int64_t h = 0; h < H; ++h) {
        double a = 0.0, d = 0.0;
        for (int64_t b = 0; b < b_; ++b) {   /* fixed order: the result does not depend on threads */
            a += partial[b * H + h];
            d += partial[(b_ + b) * H + h];
        }
        if (!a_per_token) dA[h] = a;
        dD[h] = d;
    }
    free(partial);
    return err;
}

/* m3o_scan_backward_ex with one decay rate per head. */
int m3o_scan_backward(const m3o_dims* dm, const double* x, const double* dt, const double* A,
                      const double* lam, const double* theta, const double* B, const double* C,
                      const double* D, const double* h0, const double* b_last, const double* x_last,
                      const double* dy, const double* dh_out, double* dx, double* ddt, double* dA,
                      double* dlam, double* dtheta, double* dB, double* dC, double* dD, double* dh0,
                      double* db_last, double* dx_last, int nthreads) {
    return m3o_scan_backward_ex(dm, x, dt, A, 0, lam, theta, B, C, D, h0, b_last, x_last, dy, dh_out, dx, ddt,
                                dA, dlam, dtheta, dB, dC, dD, dh0, db_last, dx_last, nthreads);
}
