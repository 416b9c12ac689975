/*
 * mdn_oracle.c -- fp64 CPU oracle of the Momentum DeltaNet (MDN) recurrence.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the plain, slow, obviously correct
 * definition that the HIP path is checked against.  Only the test suite, the
 * smoke check and the CPU-baseline leg of the benchmark may load it.  It
 * shares no code, header or constant with the HIP library.
 *
 * What it computes (source: "MDN: Parallelizing Stepwise Momentum for Delta
 * Linear Attention", paper summary at paper.rainbus.top, method walk-through
 * step 1; the same two update equations appear in the ijyty.com article on
 * MDN, section 3), per (batch, head) and token t = 1..T:
 *
 *     p_t      = alpha_t k_t
 *     vtilde_t = v_t - S_{t-1}^T p_t          (uses the previous state)
 *     M_t      = mu_t M_{t-1} - eta_t k_t vtilde_t^T
 *     S_t      = alpha_t S_{t-1} - beta_t M_t (uses the new momentum)
 *     o_t      = S_t^T q_t                    (read-out after the update)
 *
 * S and M are dk x dv matrices stored row-major ([dk][dv], dv contiguous).
 * All arithmetic is IEEE double; nothing is reordered or fused beyond the
 * loops written here.  Heads are independent, so (batch, head) pairs run in
 * parallel under OpenMP; each head's loop is sequential in t.
 *
 * Layouts (all contiguous, fp64):
 *   q, k : [BH][T][dk]     v, O, Vt : [BH][T][dv]
 *   alpha, mu, beta, eta : [BH][T]
 *   S0, M0, ST, MT : [BH][dk][dv]; S0 or M0 may be NULL (= zero state).
 */
#include <stdlib.h>
#include <string.h>

/* One token of the recurrence on one head, in place on S and M.
 * Writes vtilde (length dv) and o (length dv). */
static void mdn_token(long dk, long dv, double* S, double* M,
                      const double* q, const double* k, const double* v,
                      double alpha, double mu, double beta, double eta,
                      double* vtilde, double* o)
{
    /* vtilde = v - S_{t-1}^T (alpha k) */
    for (long j = 0; j < dv; ++j) {
        double acc = 0.0;
        for (long i = 0; i < dk; ++i) acc += S[i * dv + j] * (alpha * k[i]);
        vtilde[j] = v[j] - acc;
    }
    /* M_t = mu M_{t-1} - eta k vtilde^T ;  S_t = alpha S_{t-1} - beta M_t */
    for (long i = 0; i < dk; ++i) {
        for (long j = 0; j < dv; ++j) {
            double m = mu * M[i * dv + j] - eta * k[i] * vtilde[j];
            M[i * dv + j] = m;
            S[i * dv + j] = alpha * S[i * dv + j] - beta * m;
        }
    }
    /* o_t = S_t^T q */
    for (long j = 0; j < dv; ++j) {
        double acc = 0.0;
        for (long i = 0; i < dk; ++i) acc += S[i * dv + j] * q[i];
        o[j] = acc;
    }
}

/* Whole-sequence forward: returns O, the final states and every vtilde. */
void mdn_oracle_fwd(long BH, long T, long dk, long dv,
                    const double* q, const double* k, const double* v,
                    const double* alpha, const double* mu,
                    const double* beta, const double* eta,
                    const double* S0, const double* M0,
                    double* O, double* ST, double* MT, double* Vt)
{
    long bh;
#pragma omp parallel for schedule(dynamic, 1)
    for (bh = 0; bh < BH; ++bh) {
        double* S = ST + bh * dk * dv;
        double* M = MT + bh * dk * dv;
        if (S0) memcpy(S, S0 + bh * dk * dv, sizeof(double) * dk * dv);
        else memset(S, 0, sizeof(double) * dk * dv);
        if (M0) memcpy(M, M0 + bh * dk * dv, sizeof(double) * dk * dv);
        else memset(M, 0, sizeof(double) * dk * dv);
        for (long t = 0; t < T; ++t) {
            long row = bh * T + t;
            mdn_token(dk, dv, S, M, q + row * dk, k + row * dk, v + row * dv,
                      alpha[row], mu[row], beta[row], eta[row],
                      Vt + row * dv, O + row * dv);
        }
    }
}

/* One decode step for every head: S, M updated in place, o written.
 * q, k : [BH][dk]; v, o : [BH][dv]; gates : [BH]. */
void mdn_oracle_step(long BH, long dk, long dv,
                     const double* q, const double* k, const double* v,
                     const double* alpha, const double* mu,
                     const double* beta, const double* eta,
                     double* S, double* M, double* o, double* vtilde)
{
    long bh;
#pragma omp parallel for schedule(static)
    for (bh = 0; bh < BH; ++bh) {
        mdn_token(dk, dv, S + bh * dk * dv, M + bh * dk * dv,
                  q + bh * dk, k + bh * dk, v + bh * dv,
                  alpha[bh], mu[bh], beta[bh], eta[bh],
                  vtilde + bh * dv, o + bh * dv);
    }
}

/* Set the number of OpenMP threads for the following calls (n >= 1). */
void mdn_oracle_set_threads(int n)
{
#ifdef _OPENMP
    extern void omp_set_num_threads(int);
    if (n >= 1) omp_set_num_threads(n);
#else
    (void)n;
#endif
}

/* Number of OpenMP threads the oracle will use (for reporting). */
int mdn_oracle_threads(void)
{
    int n = 1;
#pragma omp parallel
    {
#pragma omp single
        {
#ifdef _OPENMP
            extern int omp_get_num_threads(void);
            n = omp_get_num_threads();
#endif
        }
    }
    return n;
}
