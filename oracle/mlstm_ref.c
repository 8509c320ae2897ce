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
