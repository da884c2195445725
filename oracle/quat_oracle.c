/*
 * quat_oracle.c -- plain float64 CPU oracle for the quaternion cumulative
 * product scan and its vector-Jacobian product.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may link, load or
 * call this file; only the tests, the smoke check and the benchmark's CPU
 * baseline leg use it.  It shares no code with the device library.
 *
 * Source of the definitions: the burn-mamba source page
 * "burn_mamba/mamba3/quat_scan/backward.rs", module documentation, section
 * "Gradient math":
 *   - scan:       cum[t] = q_t (x) cum[t-1],  cum[-1] = init
 *                 (equivalently cum[t] = P_t (x) init, P_t = q_t (x) ... (x) q_0)
 *   - per-factor VJP of o = a (x) b with cotangent g (real inner product):
 *                 grad_a = g (x) conj(b),  grad_b = conj(a) (x) g
 *   - reverse recurrence for the total cotangent reaching cum[t]:
 *                 G[t] = d_cum[t] + conj(q_{t+1}) (x) G[t+1]
 *   - closed form stated there for unit quaternions:
 *                 S[t] = sum_{u>=t} conj(P_u) (x) d_cum[u],  G[t] = P_t (x) S[t],
 *                 d_q[t] = G[t] (x) conj(cum[t-1]),  d_init = S[0]
 *
 * The page does not define the product itself.  Reading taken here: scalar
 * first (w, x, y, z) with Hamilton's rules i^2 = j^2 = k^2 = ijk = -1.  The
 * product is written as a 4x4 left-multiplication matrix applied to the right
 * operand.
 *
 * Layout: q, cum, d_cum, d_q are [b][s][m][4] row-major float64 (m = h*j);
 * init and d_init are [b][m][4].
 *
 * Everything is sequential over the sequence axis; OpenMP only splits the
 * independent columns (one column = one (batch, h*j) index).
 */
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* a (x) b = Lmat(a) * b, with Lmat(a) the left-multiplication matrix of a. */
static void lmat(const double a[4], double L[4][4]) {
    const double w = a[0], x = a[1], y = a[2], z = a[3];
    L[0][0] = w;  L[0][1] = -x; L[0][2] = -y; L[0][3] = -z;
    L[1][0] = x;  L[1][1] = w;  L[1][2] = -z; L[1][3] = y;
    L[2][0] = y;  L[2][1] = z;  L[2][2] = w;  L[2][3] = -x;
    L[3][0] = z;  L[3][1] = -y; L[3][2] = x;  L[3][3] = w;
}

static void qmul(const double a[4], const double b[4], double out[4]) {
    double L[4][4], r[4];
    lmat(a, L);
    for (int i = 0; i < 4; ++i) {
        double acc = 0.0;
        for (int k = 0; k < 4; ++k) acc += L[i][k] * b[k];
        r[i] = acc;
    }
    memcpy(out, r, sizeof r);
}

static void qconj(const double a[4], double out[4]) {
    out[0] = a[0]; out[1] = -a[1]; out[2] = -a[2]; out[3] = -a[3];
}

static double qnorm2(const double a[4]) {
    return a[0] * a[0] + a[1] * a[1] + a[2] * a[2] + a[3] * a[3];
}

static int set_threads(int nthreads) {
#ifdef _OPENMP
    if (nthreads <= 0) nthreads = omp_get_max_threads();
    return nthreads;
#else
    (void)nthreads;
    return 1;
#endif
}

/* Exposed for the tests: out = a (x) b. */
void oracle_qmul(const double* a, const double* b, double* out) { qmul(a, b, out); }

/* Number of threads a call with this request would use. */
int oracle_threads(int nthreads) { return set_threads(nthreads); }

#define IDX(bi, t, c) ((((size_t)(bi) * (size_t)s + (size_t)(t)) * (size_t)m + (size_t)(c)) * 4)
#define CIDX(bi, c) (((size_t)(bi) * (size_t)m + (size_t)(c)) * 4)

/* Forward scan: cum[t] = q_t (x) cum[t-1], cum[-1] = init. */
void oracle_fwd(const double* q, const double* init, double* cum,
                int64_t b, int64_t s, int64_t m, int nthreads) {
    const int64_t ncol = b * m;
    const int nt = set_threads(nthreads);
    (void)nt;
#pragma omp parallel for num_threads(nt) schedule(static)
    for (int64_t col = 0; col < ncol; ++col) {
        const int64_t bi = col / m, c = col % m;
        double carry[4];
        memcpy(carry, init + CIDX(bi, c), sizeof carry);
        for (int64_t t = 0; t < s; ++t) {
            qmul(q + IDX(bi, t, c), carry, carry);
            memcpy(cum + IDX(bi, t, c), carry, sizeof carry);
        }
    }
}

/*
 * Exact VJP by the reverse recurrence (valid for all quaternions):
 *   G[s-1] = d_cum[s-1];  G[t] = d_cum[t] + conj(q_{t+1}) (x) G[t+1]
 *   d_q[t] = G[t] (x) conj(cum[t-1])     (per-factor rule, left factor q_t)
 *   d_init = conj(q_0) (x) G[0]          (per-factor rule, right factor init)
 * Either output pointer may be NULL.  Returns 0, or -1 if scratch memory
 * could not be allocated.
 */
int oracle_bwd(const double* q, const double* init, const double* d_cum,
               double* d_q, double* d_init,
               int64_t b, int64_t s, int64_t m, int nthreads) {
    const int64_t ncol = b * m;
    const int nt = set_threads(nthreads);
    int failed = 0;
#pragma omp parallel num_threads(nt)
    {
        double* cum = (double*)malloc((size_t)s * 4 * sizeof(double));
        if (!cum) {
#pragma omp atomic write
            failed = 1;
        }
#pragma omp for schedule(static)
        for (int64_t col = 0; col < ncol; ++col) {
            if (!cum) continue;
            const int64_t bi = col / m, c = col % m;
            const double* ini = init + CIDX(bi, c);
            double carry[4];
            memcpy(carry, ini, sizeof carry);
            for (int64_t t = 0; t < s; ++t) {
                qmul(q + IDX(bi, t, c), carry, carry);
                memcpy(cum + 4 * t, carry, sizeof carry);
            }
            double G[4], tmp[4], cj[4];
            memcpy(G, d_cum + IDX(bi, s - 1, c), sizeof G);
            for (int64_t t = s - 1; t >= 0; --t) {
                if (t < s - 1) {
                    qconj(q + IDX(bi, t + 1, c), cj);
                    qmul(cj, G, tmp);
                    const double* d = d_cum + IDX(bi, t, c);
                    for (int k = 0; k < 4; ++k) G[k] = d[k] + tmp[k];
                }
                if (d_q) {
                    qconj(t > 0 ? cum + 4 * (t - 1) : ini, cj);
                    qmul(G, cj, d_q + IDX(bi, t, c));
                }
            }
            if (d_init) {
                qconj(q + IDX(bi, 0, c), cj);
                qmul(cj, G, d_init + CIDX(bi, c));
            }
        }
        free(cum);
    }
    return failed ? -1 : 0;
}

/*
 * The closed form exactly as the page states it (prefix product P, suffix sum
 * S, G = P (x) S, d_q = G (x) conj(cum_prev), d_init = S[0]).  With
 * normalise != 0, G[t] is divided by |P_t|^2, which makes the closed form the
 * exact VJP for any invertible steps (telescoping the reverse recurrence with
 * conj(q) = |q|^2 q^-1).  Used by the tests to show where the page's form
 * holds; the reference answer is oracle_bwd.
 */
int oracle_bwd_closed_form(const double* q, const double* init, const double* d_cum,
                           double* d_q, double* d_init,
                           int64_t b, int64_t s, int64_t m, int normalise, int nthreads) {
    const int64_t ncol = b * m;
    const int nt = set_threads(nthreads);
    int failed = 0;
#pragma omp parallel num_threads(nt)
    {
        double* P = (double*)malloc((size_t)s * 4 * sizeof(double));
        double* S = (double*)malloc((size_t)s * 4 * sizeof(double));
        if (!P || !S) {
#pragma omp atomic write
            failed = 1;
        }
#pragma omp for schedule(static)
        for (int64_t col = 0; col < ncol; ++col) {
            if (!P || !S) continue;
            const int64_t bi = col / m, c = col % m;
            const double* ini = init + CIDX(bi, c);
            double acc[4] = {1.0, 0.0, 0.0, 0.0}, cj[4], x[4];
            for (int64_t t = 0; t < s; ++t) {          /* P_t = q_t (x) P_{t-1} */
                qmul(q + IDX(bi, t, c), acc, acc);
                memcpy(P + 4 * t, acc, sizeof acc);
            }
            double run[4] = {0.0, 0.0, 0.0, 0.0};
            for (int64_t t = s - 1; t >= 0; --t) {     /* S = reverse cumsum */
                qconj(P + 4 * t, cj);
                qmul(cj, d_cum + IDX(bi, t, c), x);
                for (int k = 0; k < 4; ++k) run[k] += x[k];
                memcpy(S + 4 * t, run, sizeof run);
            }
            if (d_q) {
                for (int64_t t = 0; t < s; ++t) {
                    double G[4], prev[4];
                    qmul(P + 4 * t, S + 4 * t, G);
                    if (normalise) {
                        const double n2 = qnorm2(P + 4 * t);
                        for (int k = 0; k < 4; ++k) G[k] /= n2;
                    }
                    if (t == 0) memcpy(prev, ini, sizeof prev);
                    else qmul(P + 4 * (t - 1), ini, prev);   /* cum[t-1] = P_{t-1} (x) init */
                    qconj(prev, cj);
                    qmul(G, cj, d_q + IDX(bi, t, c));
                }
            }
            if (d_init) memcpy(d_init + CIDX(bi, c), S, 4 * sizeof(double));
        }
        free(P);
        free(S);
    }
    return failed ? -1 : 0;
}
