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

/* ---------------------------------------------------------------------------
 * Reverse mode of the recurrence above (the gradient of a scalar loss L that
 * depends on O, S_T and M_T), by the chain rule applied to the four update
 * equations of one token, last token first.  Sh and Mh are dL/dS_t and
 * dL/dM_t, accumulated over every use of S_t and M_t:
 *
 *   o_t = S_t^T q_t                 : Sh += q_t do_t^T ;  dq_t = S_t do_t
 *   S_t = alpha S_{t-1} - beta M_t  : dalpha = <S_{t-1}, Sh> ; dbeta = -<M_t, Sh>
 *                                     Mh += -beta Sh ;  Sh_{t-1} = alpha Sh (+ below)
 *   M_t = mu M_{t-1} - eta k vt^T   : dmu = <M_{t-1}, Mh> ; deta = -k^T Mh vt
 *                                     dk = -eta Mh vt ; dvt = -eta Mh^T k
 *                                     Mh_{t-1} = mu Mh
 *   vt = v - S_{t-1}^T (alpha k)    : dv = dvt ; Sh_{t-1} += -(alpha k) dvt^T
 *                                     dp = -S_{t-1} dvt ; dalpha += k^T dp ;
 *                                     dk += alpha dp
 *
 * (<X, Y> is the sum of the elementwise products.)  The states S_{t-1}, M_{t-1}
 * are replayed forward from checkpoints taken every SEG tokens, so memory is
 * O((T/SEG + SEG) dk dv) per head; the arithmetic is that of the recurrence.
 * ------------------------------------------------------------------------- */
#define SEG 64

static void mdn_token_bwd(long dk, long dv, const double* Sp, const double* Mp,
                          const double* Sn, const double* Mn,
                          const double* q, const double* k, const double* vt,
                          double alpha, double mu, double beta, double eta,
                          const double* dout, double* Sh, double* Mh,
                          double* dq, double* dk_out, double* dv_out, double* dgate)
{
    double da = 0.0, db = 0.0, dm = 0.0, de = 0.0;
    /* read-out: Sh += q do^T ; dq = S_t do */
    for (long i = 0; i < dk; ++i)
        for (long j = 0; j < dv; ++j) Sh[i * dv + j] += q[i] * dout[j];
    for (long i = 0; i < dk; ++i) {
        double acc = 0.0;
        for (long j = 0; j < dv; ++j) acc += Sn[i * dv + j] * dout[j];
        dq[i] = acc;
    }
    /* S_t = alpha S_{t-1} - beta M_t */
    for (long i = 0; i < dk * dv; ++i) {
        da += Sp[i] * Sh[i];
        db -= Mn[i] * Sh[i];
    }
    for (long i = 0; i < dk * dv; ++i) Mh[i] -= beta * Sh[i];
    /* M_t = mu M_{t-1} - eta k vt^T */
    for (long i = 0; i < dk * dv; ++i) dm += Mp[i] * Mh[i];
    for (long i = 0; i < dk; ++i) {
        double acc = 0.0;
        for (long j = 0; j < dv; ++j) acc += Mh[i * dv + j] * vt[j];
        de -= k[i] * acc;
        dk_out[i] = -eta * acc;
    }
    for (long j = 0; j < dv; ++j) {
        double acc = 0.0;
        for (long i = 0; i < dk; ++i) acc += Mh[i * dv + j] * k[i];
        dv_out[j] = -eta * acc;              /* dvt, which is also dv */
    }
    /* vt = v - S_{t-1}^T (alpha k) */
    for (long i = 0; i < dk; ++i) {
        double acc = 0.0;
        for (long j = 0; j < dv; ++j) acc += Sp[i * dv + j] * dv_out[j];
        const double dp = -acc;
        da += k[i] * dp;
        dk_out[i] += alpha * dp;
    }
    /* adjoints of S_{t-1}, M_{t-1} */
    for (long i = 0; i < dk; ++i)
        for (long j = 0; j < dv; ++j)
            Sh[i * dv + j] = alpha * Sh[i * dv + j] - alpha * k[i] * dv_out[j];
    for (long i = 0; i < dk * dv; ++i) Mh[i] *= mu;
    dgate[0] = da; dgate[1] = dm; dgate[2] = db; dgate[3] = de;
}

/* Gradients of L = sum(dO * O) + sum(dST * S_T) + sum(dMT * M_T) with
 * respect to every input of mdn_oracle_fwd.  dST, dMT may be NULL (zero).
 * Outputs: dq, dk [BH][T][dk]; dv [BH][T][dv]; dalpha, dmu, dbeta, deta
 * [BH][T]; dS0, dM0 [BH][dk][dv] (the gradient with respect to the initial
 * state, whether or not S0/M0 were given). */
void mdn_oracle_bwd(long BH, long T, long dk, long dv,
                    const double* q, const double* k, const double* v,
                    const double* alpha, const double* mu,
                    const double* beta, const double* eta,
                    const double* S0, const double* M0,
                    const double* dO, const double* dST, const double* dMT,
                    double* dq, double* dk_out, double* dv_out,
                    double* dalpha, double* dmu, double* dbeta, double* deta,
                    double* dS0, double* dM0)
{
    const long nseg = (T + SEG - 1) / SEG;
    const long dd = dk * dv;
    long bh;
#pragma omp parallel for schedule(dynamic, 1)
    for (bh = 0; bh < BH; ++bh) {
        double* ck = (double*)malloc(sizeof(double) * 2 * dd * (nseg + 1));   /* checkpoints */
        double* St = (double*)malloc(sizeof(double) * 2 * dd * (SEG + 1));   /* replayed states */
        double* vt = (double*)malloc(sizeof(double) * dv * SEG);
        double* o = (double*)malloc(sizeof(double) * dv);
        double* Sh = dS0 + bh * dd;
        double* Mh = dM0 + bh * dd;
        double* S = ck;
        double* M = ck + dd;
        if (S0) memcpy(S, S0 + bh * dd, sizeof(double) * dd); else memset(S, 0, sizeof(double) * dd);
        if (M0) memcpy(M, M0 + bh * dd, sizeof(double) * dd); else memset(M, 0, sizeof(double) * dd);
        /* forward: checkpoint the states at every segment start */
        for (long sg = 0; sg < nseg; ++sg) {
            double* Sc = ck + 2 * dd * sg;
            double* Sx = ck + 2 * dd * (sg + 1);
            memcpy(Sx, Sc, sizeof(double) * 2 * dd);
            for (long t = sg * SEG; t < T && t < (sg + 1) * SEG; ++t) {
                const long row = bh * T + t;
                mdn_token(dk, dv, Sx, Sx + dd, q + row * dk, k + row * dk, v + row * dv,
                          alpha[row], mu[row], beta[row], eta[row], vt, o);
            }
        }
        /* the adjoints start from dL/dS_T, dL/dM_T */
        if (dST) memcpy(Sh, dST + bh * dd, sizeof(double) * dd); else memset(Sh, 0, sizeof(double) * dd);
        if (dMT) memcpy(Mh, dMT + bh * dd, sizeof(double) * dd); else memset(Mh, 0, sizeof(double) * dd);
        for (long sg = nseg - 1; sg >= 0; --sg) {
            const long t0 = sg * SEG, t1 = (sg + 1) * SEG < T ? (sg + 1) * SEG : T;
            /* replay the segment: St[s] = (S, M) after s tokens of the segment */
            memcpy(St, ck + 2 * dd * sg, sizeof(double) * 2 * dd);
            for (long t = t0; t < t1; ++t) {
                const long row = bh * T + t, s = t - t0;
                memcpy(St + 2 * dd * (s + 1), St + 2 * dd * s, sizeof(double) * 2 * dd);
                mdn_token(dk, dv, St + 2 * dd * (s + 1), St + 2 * dd * (s + 1) + dd,
                          q + row * dk, k + row * dk, v + row * dv,
                          alpha[row], mu[row], beta[row], eta[row], vt + s * dv, o);
            }
            for (long t = t1 - 1; t >= t0; --t) {
                const long row = bh * T + t, s = t - t0;
                double g[4];
                mdn_token_bwd(dk, dv, St + 2 * dd * s, St + 2 * dd * s + dd,
                              St + 2 * dd * (s + 1), St + 2 * dd * (s + 1) + dd,
                              q + row * dk, k + row * dk, vt + s * dv,
                              alpha[row], mu[row], beta[row], eta[row], dO + row * dv, Sh, Mh,
                              dq + row * dk, dk_out + row * dk, dv_out + row * dv, g);
                dalpha[row] = g[0]; dmu[row] = g[1]; dbeta[row] = g[2]; deta[row] = g[3];
            }
        }
        free(ck); free(St); free(vt); free(o);
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
