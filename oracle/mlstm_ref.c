/*
 * mlstm_ref.c -- float64 reference of the xLSTM mLSTM cell forward pass.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the oracle that the HIP library is
 * checked against.  Only the tests, the smoke check and the benchmark's CPU
 * baseline may load it; the library never calls it, and the two share no
 * source, header, helper or constant.
 *
 * What it computes (xLSTM note, "mLSTM (matrix LSTM)" and "sLSTM" sections:
 * exponential gates, the log-space stabilizer, the matrix-memory and
 * normalizer updates and the normalized, output-gated read-out), for every
 * independent (batch, head) pair, one token after another -- the plain
 * sequential recurrence, with no chunking and no reordering:
 *
 *   m_t  = max(f~_t + m_{t-1}, i~_t)                       stabilizer
 *   f'_t = exp(f~_t + m_{t-1} - m_t),  i'_t = exp(i~_t - m_t)
 *   C_t  = f'_t C_{t-1} + i'_t k_t v_t^T                   (d_qk x d_v)
 *   n_t  = f'_t n_{t-1} + i'_t k_t
 *   h_t  = sigmoid(o~_t) * (C_t^T q_t) / max(|n_t . q_t|, exp(-m_t))
 *
 * The states are kept in the stabilized variables (C_t, n_t above equal the
 * unstabilized matrix memory and normalizer times exp(-m_t)).  Dividing the
 * note's floor of one by the same factor gives exp(-m_t), so h_t is exactly
 * the note's unstabilized read-out C q / max(|n^T q|, 1).  The matrix memory
 * is stored d_qk x d_v (key index first, as the note states its shape) and
 * read out with its transpose; the note's value-first outer product read out
 * as C q is the same number.
 *
 * Readings where the pages are silent: f~ is the log forget gate (the cell
 * applies exp to it and nothing else); o~ gets an elementwise sigmoid; an
 * absent initial state means C = 0, n = 0, m = 0.
 *
 * Layouts (C order, float64): q, k [P, T, d_qk]; v, o_pre, h [P, T, d_v];
 * i_pre, f_pre [P, T]; C [P, d_qk, d_v]; n [P, d_qk]; m [P].  P is the number
 * of independent pairs.
 *
 * mlstm_ref_backward: reverse mode of the same recurrence for a loss whose
 * gradient with respect to h is given (dh).  Derivation: in the unstabilized
 * variables the read-out is C q / max(|n^T q|, 1) and the stabilizer does not
 * appear, so m is not differentiated; every gradient is then carried in the
 * stabilized variables.  With a_t = dh_t * sigmoid(o~_t) / den_t and
 * beta_t = -sign(n_t.q_t) (a_t . C_t^T q_t) / den_t when |n_t.q_t| is above
 * the floor exp(-m_t) (zero when the floor is active), the memory gradients
 * run backwards in time with the forward's own decay factors:
 *   dC*_t = q_t a_t^T + f'_{t+1} dC*_{t+1},   dn*_t = q_t beta_t + f'_{t+1} dn*_{t+1}
 * (dC*_t is the unstabilized memory gradient times exp(m_t)), and
 *   dq_t  = C_t a_t + n_t beta_t
 *   dk_t  = i'_t (dC*_t v_t + dn*_t),     dv_t = i'_t dC*_t^T k_t
 *   di~_t = i'_t (k_t^T dC*_t v_t + k_t . dn*_t)
 *   df~_t = f'_t (<dC*_t, C_{t-1}> + dn*_t . n_{t-1})
 *   do~_t = dh_t * (C_t^T q_t) / den_t * sigmoid'(o~_t)
 *   dC0 = f'_0 dC*_0,  dn0 = f'_0 dn*_0,  dm0 = <dC0, C0> + dn0 . n0.
 */
#include <math.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* logistic function, written so that neither branch overflows */
static double sigmoid(double x)
{
    if (x >= 0.0)
        return 1.0 / (1.0 + exp(-x));
    double e = exp(x);
    return e / (1.0 + e);
}

/* T sequential steps of one pair; C (d_qk*d_v), n (d_qk), *m are updated in
 * place and start as the initial state; num is d_v doubles of scratch. */
static void run_pair(const double *q, const double *k, const double *v,
                     const double *ig, const double *fg, const double *og,
                     double *C, double *n, double *m_io, double *h,
                     long T, long dk, long dv, double *num)
{
    double m = *m_io;
    for (long t = 0; t < T; ++t) {
        const double *qt = q + t * dk;
        const double *kt = k + t * dk;
        const double *vt = v + t * dv;
        const double *ot = og + t * dv;
        double *ht = h + t * dv;

        double m_new = fmax(fg[t] + m, ig[t]);
        double fp = exp(fg[t] + m - m_new);
        double ip = exp(ig[t] - m_new);

        for (long a = 0; a < dk; ++a) {
            double *row = C + a * dv;
            for (long b = 0; b < dv; ++b)
                row[b] = fp * row[b] + ip * kt[a] * vt[b];
            n[a] = fp * n[a] + ip * kt[a];
        }
        m = m_new;

        for (long b = 0; b < dv; ++b)
            num[b] = 0.0;
        double nq = 0.0;
        for (long a = 0; a < dk; ++a) {
            const double *row = C + a * dv;
            for (long b = 0; b < dv; ++b)
                num[b] += row[b] * qt[a];
            nq += n[a] * qt[a];
        }
        double den = fmax(fabs(nq), exp(-m));
        for (long b = 0; b < dv; ++b)
            ht[b] = sigmoid(ot[b]) * num[b] / den;
    }
    *m_io = m;
}

/*
 * Run the recurrence over P independent pairs of T tokens each.
 * C0, n0, m0: the initial state, or all NULL for the zero state.
 * C_T, n_T, m_T: the final state, or NULL when not wanted.
 * threads: OpenMP threads over pairs (<= 0: the runtime's default).
 * Returns 0, or -1 on bad sizes, -2 when only part of the initial state is
 * given, -3 when out of memory.
 */
int mlstm_ref_forward(const double *q, const double *k, const double *v,
                      const double *i_pre, const double *f_pre, const double *o_pre,
                      const double *C0, const double *n0, const double *m0,
                      double *h, double *C_T, double *n_T, double *m_T,
                      long P, long T, long dk, long dv, int threads)
{
    if (P < 0 || T < 0 || dk <= 0 || dv <= 0)
        return -1;
    int have0 = (C0 != NULL) + (n0 != NULL) + (m0 != NULL);
    if (have0 != 0 && have0 != 3)
        return -2;
    int fail = 0;
#ifdef _OPENMP
    if (threads <= 0)
        threads = omp_get_max_threads();
#pragma omp parallel for schedule(dynamic, 1) num_threads(threads) reduction(| : fail)
#endif
    for (long p = 0; p < P; ++p) {
        double *C = malloc(sizeof(double) * (size_t)(dk * dv));
        double *n = malloc(sizeof(double) * (size_t)dk);
        double *num = malloc(sizeof(double) * (size_t)dv);
        if (!C || !n || !num) {
            fail = 1;
        } else {
            double m = 0.0;
            if (have0) {
                memcpy(C, C0 + p * dk * dv, sizeof(double) * (size_t)(dk * dv));
                memcpy(n, n0 + p * dk, sizeof(double) * (size_t)dk);
                m = m0[p];
            } else {
                memset(C, 0, sizeof(double) * (size_t)(dk * dv));
                memset(n, 0, sizeof(double) * (size_t)dk);
            }
            run_pair(q + p * T * dk, k + p * T * dk, v + p * T * dv,
                     i_pre + p * T, f_pre + p * T, o_pre + p * T * dv,
                     C, n, &m, h + p * T * dv, T, dk, dv, num);
            if (C_T)
                memcpy(C_T + p * dk * dv, C, sizeof(double) * (size_t)(dk * dv));
            if (n_T)
                memcpy(n_T + p * dk, n, sizeof(double) * (size_t)dk);
            if (m_T)
                m_T[p] = m;
        }
        free(C);
        free(n);
        free(num);
    }
    return fail ? -3 : 0;
}

/* Reverse mode of one pair: a forward sweep keeps every C_t, n_t (t = -1 ..
 * T-1), the stabilizer factors and the read-out, then a backward sweep runs
 * the memory gradients from the last token to the first.  C, n, m: the
 * initial state (C, n are read, not written).  Gradient outputs may be NULL
 * except dq, dk, dv, di, df, do_. */
static int bwd_pair(const double *q, const double *k, const double *v,
                    const double *ig, const double *fg, const double *og, const double *dh,
                    const double *C0, const double *n0, double m0,
                    double *dq, double *dkk, double *dvv, double *di, double *df, double *dog,
                    double *dC0, double *dn0, double *dm0, long T, long dk, long dv)
{
    const long S = dk * dv;
    double *Cs = malloc(sizeof(double) * (size_t)((T + 1) * S));   /* C_{t-1} at index t */
    double *ns = malloc(sizeof(double) * (size_t)((T + 1) * dk));
    double *num = malloc(sizeof(double) * (size_t)(T * dv));
    double *nq = malloc(sizeof(double) * (size_t)T);
    double *den = malloc(sizeof(double) * (size_t)T);
    double *mm = malloc(sizeof(double) * (size_t)T);
    double *fpv = malloc(sizeof(double) * (size_t)(T + 1));
    double *ipv = malloc(sizeof(double) * (size_t)T);
    double *dCs = calloc((size_t)S, sizeof(double));
    double *dns = calloc((size_t)dk, sizeof(double));
    double *a = malloc(sizeof(double) * (size_t)dv);
    if (!Cs || !ns || !num || !nq || !den || !mm || !fpv || !ipv || !dCs || !dns || !a) {
        free(Cs); free(ns); free(num); free(nq); free(den); free(mm); free(fpv); free(ipv);
        free(dCs); free(dns); free(a);
        return 1;
    }
    /* forward sweep (as run_pair) */
    if (C0) {
        memcpy(Cs, C0, sizeof(double) * (size_t)S);
        memcpy(ns, n0, sizeof(double) * (size_t)dk);
    } else {
        memset(Cs, 0, sizeof(double) * (size_t)S);
        memset(ns, 0, sizeof(double) * (size_t)dk);
    }
    double m = m0;
    for (long t = 0; t < T; ++t) {
        const double *Cp = Cs + t * S, *np = ns + t * dk;
        double *C = Cs + (t + 1) * S, *n = ns + (t + 1) * dk;
        const double *qt = q + t * dk, *kt = k + t * dk, *vt = v + t * dv;
        const double mt = fmax(fg[t] + m, ig[t]);
        fpv[t] = exp(fg[t] + m - mt);
        ipv[t] = exp(ig[t] - mt);
        for (long r = 0; r < dk; ++r) {
            for (long b = 0; b < dv; ++b)
                C[r * dv + b] = fpv[t] * Cp[r * dv + b] + ipv[t] * kt[r] * vt[b];
            n[r] = fpv[t] * np[r] + ipv[t] * kt[r];
        }
        m = mt;
        mm[t] = m;
        double s = 0.0;
        for (long b = 0; b < dv; ++b)
            num[t * dv + b] = 0.0;
        for (long r = 0; r < dk; ++r) {
            for (long b = 0; b < dv; ++b)
                num[t * dv + b] += C[r * dv + b] * qt[r];
            s += n[r] * qt[r];
        }
        nq[t] = s;
        den[t] = fmax(fabs(s), exp(-m));
    }
    fpv[T] = 0.0; /* no token after the last */
    /* backward sweep */
    for (long t = T - 1; t >= 0; --t) {
        const double *qt = q + t * dk, *kt = k + t * dk, *vt = v + t * dv;
        const double *C = Cs + (t + 1) * S, *n = ns + (t + 1) * dk;
        const double *Cp = Cs + t * S, *np = ns + t * dk;
        const double *g = dh + t * dv, *nt = num + t * dv;
        double an = 0.0;
        for (long b = 0; b < dv; ++b) {
            double sg = sigmoid(og[t * dv + b]);
            a[b] = g[b] * sg / den[t];
            dog[t * dv + b] = g[b] * nt[b] / den[t] * sg * (1.0 - sg);
            an += a[b] * nt[b];
        }
        double beta = 0.0;
        if (fabs(nq[t]) > exp(-mm[t]))
            beta = -(nq[t] > 0.0 ? 1.0 : -1.0) * an / den[t];
        /* dC*_t, dn*_t from dC*_{t+1}, dn*_{t+1} */
        for (long r = 0; r < dk; ++r) {
            for (long b = 0; b < dv; ++b)
                dCs[r * dv + b] = qt[r] * a[b] + fpv[t + 1] * dCs[r * dv + b];
            dns[r] = qt[r] * beta + fpv[t + 1] * dns[r];
        }
        double sdi = 0.0, sdf = 0.0;
        for (long r = 0; r < dk; ++r) {
            double cq = 0.0, dcv = 0.0;
            for (long b = 0; b < dv; ++b) {
                cq += C[r * dv + b] * a[b];
                dcv += dCs[r * dv + b] * vt[b];
                sdf += dCs[r * dv + b] * Cp[r * dv + b];
            }
            dq[t * dk + r] = cq + n[r] * beta;
            dkk[t * dk + r] = ipv[t] * (dcv + dns[r]);
            sdi += kt[r] * (dcv + dns[r]);
            sdf += dns[r] * np[r];
        }
        for (long b = 0; b < dv; ++b) {
            double s = 0.0;
            for (long r = 0; r < dk; ++r)
                s += dCs[r * dv + b] * kt[r];
            dvv[t * dv + b] = ipv[t] * s;
        }
        di[t] = ipv[t] * sdi;
        df[t] = fpv[t] * sdf;
    }
    /* initial state: C0 enters as exp(m0) C0 */
    double f0 = T > 0 ? fpv[0] : 1.0, s0 = 0.0;
    for (long r = 0; r < dk; ++r) {
        for (long b = 0; b < dv; ++b) {
            double g0 = f0 * dCs[r * dv + b];
            if (dC0) dC0[r * dv + b] = g0;
            s0 += g0 * Cs[r * dv + b];
        }
        double g1 = f0 * dns[r];
        if (dn0) dn0[r] = g1;
        s0 += g1 * ns[r];
    }
    if (dm0) *dm0 = s0;
    free(Cs); free(ns); free(num); free(nq); free(den); free(mm); free(fpv); free(ipv);
    free(dCs); free(dns); free(a);
    return 0;
}

/*
 * Gradients of sum(dh * h) over P independent pairs (see the header).
 * C0, n0, m0: the initial state, or all NULL for the zero state.  dC0, dn0,
 * dm0: gradients of the initial state, or NULL when not wanted.
 * Returns 0, or -1 on bad sizes, -2 when only part of the initial state is
 * given, -3 when out of memory.
 */
int mlstm_ref_backward(const double *q, const double *k, const double *v,
                       const double *i_pre, const double *f_pre, const double *o_pre,
                       const double *C0, const double *n0, const double *m0, const double *dh,
                       double *dq, double *dk_out, double *dv_out, double *di, double *df, double *dog,
                       double *dC0, double *dn0, double *dm0,
                       long P, long T, long dk, long dv, int threads)
{
    if (P < 0 || T < 0 || dk <= 0 || dv <= 0)
        return -1;
    int have0 = (C0 != NULL) + (n0 != NULL) + (m0 != NULL);
    if (have0 != 0 && have0 != 3)
        return -2;
    int fail = 0;
#ifdef _OPENMP
    if (threads <= 0)
        threads = omp_get_max_threads();
#pragma omp parallel for schedule(dynamic, 1) num_threads(threads) reduction(| : fail)
#endif
    for (long p = 0; p < P; ++p) {
        fail |= bwd_pair(q + p * T * dk, k + p * T * dk, v + p * T * dv, i_pre + p * T, f_pre + p * T,
                         o_pre + p * T * dv, dh + p * T * dv,
                         have0 ? C0 + p * dk * dv : NULL, have0 ? n0 + p * dk : NULL, have0 ? m0[p] : 0.0,
                         dq + p * T * dk, dk_out + p * T * dk, dv_out + p * T * dv, di + p * T, df + p * T,
                         dog + p * T * dv, dC0 ? dC0 + p * dk * dv : NULL, dn0 ? dn0 + p * dk : NULL,
                         dm0 ? dm0 + p : NULL, T, dk, dv);
    }
    return fail ? -3 : 0;
}
