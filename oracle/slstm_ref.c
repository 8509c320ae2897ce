/*
 * slstm_ref.c -- float64 reference of the xLSTM sLSTM cell forward pass.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the oracle that the HIP library's
 * sLSTM kernel is checked against.  Only the tests, the smoke check and the
 * benchmark's CPU baseline may load it; the library never calls it, and the
 * two share no source, header, helper or constant.
 *
 * The xLSTM note (section "sLSTM") gives the sLSTM as an LSTM with
 * exponential input and forget gates, f = exp(f~) and i = exp(i~), kept
 * finite by the log-space stabilizer
 *     m_t = max(f~_t + m_{t-1}, i~_t),
 *     f'_t = exp(f~_t + m_{t-1} - m_t),  i'_t = exp(i~_t - m_t),
 * combined with a normalization; the summary page adds that it has a scalar
 * memory, a scalar update and memory mixing.  Readings where the pages are
 * silent (each also listed with the design notes):
 *   - every one of the d scalar cells of a head has its own gates and its own
 *     stabilizer (the formula above, elementwise);
 *   - the scalar update is the matrix memory's with the outer product replaced
 *     by the cell input: c_t = f' c_{t-1} + i' z_t with z_t = tanh(z~_t), and
 *     the normalizer is the key-free analogue n_t = f' n_{t-1} + i';
 *   - the read-out is h_t = sigmoid(o~_t) * c_t / n_t;
 *   - memory mixing: each gate's pre-activation adds a recurrent term R_g
 *     h_{t-1}, with R_g a d x d matrix per head (cells mix within their head,
 *     heads stay independent); row j of R_g feeds cell j;
 *   - the input part of every pre-activation (W_g x_t + b_g) is given;
 *   - an absent initial state means c = n = m = h = 0.
 * The states are kept stabilized (c_t, n_t equal the unstabilized ones times
 * exp(-m_t)), which leaves c_t / n_t, and so h_t, unchanged.
 *
 * Layouts (C order, float64): gx [P, T, 4, d] with gate order z, i, f, o;
 * R [P, 4, d, d] (one copy per group: the caller repeats a head's matrices
 * for each batch row); h [P, T, d]; states c, n, m, h0 [P, d].
 */
#include <math.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

static double sigmoid(double x) {
    if (x >= 0.0) return 1.0 / (1.0 + exp(-x));
    const double e = exp(x);
    return e / (1.0 + e);
}

/* one group of d cells over T tokens; returns 0, or -2 when out of memory */
static int run_group(const double *gx, const double *R, const double *c0, const double *n0,
                     const double *m0, const double *h0, double *h, double *cT, double *nT,
                     double *mT, double *hT, long T, long d) {
    double *c = calloc((size_t)d, sizeof(double));
    double *n = calloc((size_t)d, sizeof(double));
    double *m = calloc((size_t)d, sizeof(double));
    double *hp = calloc((size_t)d, sizeof(double));     /* h_{t-1} */
    double *pre = malloc((size_t)(4 * d) * sizeof(double));
    if (!c || !n || !m || !hp || !pre) {
        free(c);
        free(n);
        free(m);
        free(hp);
        free(pre);
        return -2;
    }
    if (c0) {
        memcpy(c, c0, (size_t)d * sizeof(double));
        memcpy(n, n0, (size_t)d * sizeof(double));
        memcpy(m, m0, (size_t)d * sizeof(double));
        memcpy(hp, h0, (size_t)d * sizeof(double));
    }
    for (long t = 0; t < T; ++t) {
        const double *g = gx + (size_t)t * 4 * d;
        /* every pre-activation from h_{t-1}, before any cell moves on */
        for (long gi = 0; gi < 4; ++gi)
            for (long j = 0; j < d; ++j) {
                const double *row = R + ((size_t)gi * d + j) * d;
                double s = g[gi * d + j];
                for (long k = 0; k < d; ++k) s += row[k] * hp[k];
                pre[gi * d + j] = s;
            }
        double *ht = h + (size_t)t * d;
        for (long j = 0; j < d; ++j) {
            const double zt = tanh(pre[j]);
            const double it = pre[d + j], ft = pre[2 * d + j], ot = pre[3 * d + j];
            const double mnew = fmax(ft + m[j], it);
            const double ip = exp(it - mnew);
            const double fp = exp(ft + m[j] - mnew);
            c[j] = fp * c[j] + ip * zt;
            n[j] = fp * n[j] + ip;
            m[j] = mnew;
            ht[j] = sigmoid(ot) * c[j] / n[j];
        }
        memcpy(hp, ht, (size_t)d * sizeof(double));
    }
    if (cT) {
        memcpy(cT, c, (size_t)d * sizeof(double));
        memcpy(nT, n, (size_t)d * sizeof(double));
        memcpy(mT, m, (size_t)d * sizeof(double));
        memcpy(hT, hp, (size_t)d * sizeof(double));
    }
    free(c);
    free(n);
    free(m);
    free(hp);
    free(pre);
    return 0;
}

/* Returns 0, -1 on bad sizes, -2 when out of memory.  The state arguments
 * come in complete sets: all of c0, n0, m0, h0 or none; all of cT, nT, mT,
 * hT or none.  threads > 0 sets the number of threads of this call only
 * (0: the OpenMP default); the process-wide setting is left alone. */
int slstm_ref_forward(const double *gx, const double *R, const double *c0, const double *n0,
                      const double *m0, const double *h0, double *h, double *cT, double *nT,
                      double *mT, double *hT, long P, long T, long d, int threads) {
    if (P < 0 || T < 0 || d <= 0) return -1;
    int fail = 0;
#ifdef _OPENMP
    if (threads <= 0) threads = omp_get_max_threads();
#pragma omp parallel for schedule(dynamic, 1) num_threads(threads) reduction(| : fail)
#endif
    for (long p = 0; p < P; ++p) {
        const size_t sd = (size_t)p * d;
        fail |= run_group(gx + (size_t)p * T * 4 * d, R + (size_t)p * 4 * d * d, c0 ? c0 + sd : NULL,
                          n0 ? n0 + sd : NULL, m0 ? m0 + sd : NULL, h0 ? h0 + sd : NULL,
                          h + (size_t)p * T * d, cT ? cT + sd : NULL, nT ? nT + sd : NULL,
                          mT ? mT + sd : NULL, hT ? hT + sd : NULL, T, d) != 0;
    }
    (void)threads;
    return fail ? -2 : 0;
}
