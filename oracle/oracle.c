/*
 * oracle.c -- fp64 CPU oracle for linear-attention state caching.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the library path may call, link or
 * load this file; only the test-suite, the smoke check and the CPU-baseline
 * leg of the benchmark use it.  It shares no code, header, table or helper
 * with the GPU library.
 *
 * Everything here is the plain definition, token by token, in double
 * precision, with no blocking, chunking or reordering:
 *
 *   recurrence        S_i = T_i S_{i-1} + u_i            (HYPIC reading notes,
 *                                                          ch.1 sec.2, Eq. (2))
 *   transition family T_i, u_i per rule and gate         (ch.2 sec.3, Table 1)
 *   segment pair      T_C = T_m ... T_1,  S_{C|0} = end state from S_0 = 0
 *                     built with two runs of the same recurrence: one from
 *                     S_0 = 0 with the writes, one from S_0 = I with u = 0
 *                                                         (ch.2 secs.2 and 4)
 *   composition       S <- T_C S + S_{C|0} per segment in prompt order
 *                                                         (ch.2 sec.2, Eq. (6))
 *   causal conv       depthwise, width W, history = previous W-1 raw rows
 *                                                         (ch.2 sec.6)
 *   rotary shift      x <- R(delta) x, pairs of entries turned by delta theta_i
 *                                                         (ch.2 sec.6, Eqs. (7)-(8))
 *
 * Families (rule, gate):
 *   decay, scalar : T_i = g_i I,                 u_i = k_i v_i^T    (RetNet, Mamba2)
 *   decay, diag   : T_i = diag(g_i),             u_i = k_i v_i^T    (GLA)
 *   delta, scalar : T_i = g_i (I - b_i k_i k_i^T), u_i = b_i k_i v_i^T (GDN; DeltaNet g=1)
 *   delta, diag   : T_i = (I - b_i k_i k_i^T) diag(g_i), u_i = b_i k_i v_i^T (KDA)
 * The delta transitions are applied in their rank-one form, which is the
 * same product written without forming T_i.
 *
 * Layouts: row-major.  A state S is d_k x d_v; a transition is d_k x d_k.
 * Per-token arrays are addressed as base + off[unit] + t * ld.
 */
#include <math.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

enum { ORC_DECAY = 0, ORC_DELTA = 1 };
enum { ORC_GATE_SCALAR = 0, ORC_GATE_DIAG = 1 };

int orc_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* Worker threads of the batched calls (the CPU baseline times 1 and all). */
void orc_set_threads(int n)
{
#ifdef _OPENMP
    if (n > 0) omp_set_num_threads(n);
#else
    (void)n;
#endif
}

/* One token: S <- T_t S + u_t, S is dk x dv.  v == NULL means u_t = 0
 * (the transition-only run).  p is scratch of length dv. */
static void orc_step(int rule, int gate, int dk, int dv,
                     const double *k, const double *v, double b, const double *g,
                     double *S, double *p)
{
    int i, j;
    if (gate == ORC_GATE_SCALAR) {
        for (i = 0; i < dk * dv; ++i) S[i] *= g[0];
    } else {
        for (i = 0; i < dk; ++i)
            for (j = 0; j < dv; ++j) S[i * dv + j] *= g[i];
    }
    if (rule == ORC_DELTA) {
        /* (I - b k k^T) applied to the gated state: S -= b k (k^T S) */
        for (j = 0; j < dv; ++j) {
            double acc = 0.0;
            for (i = 0; i < dk; ++i) acc += k[i] * S[i * dv + j];
            p[j] = acc;
        }
        for (i = 0; i < dk; ++i)
            for (j = 0; j < dv; ++j) S[i * dv + j] -= b * k[i] * p[j];
        if (v)
            for (i = 0; i < dk; ++i)
                for (j = 0; j < dv; ++j) S[i * dv + j] += b * k[i] * v[j];
    } else {
        if (v)
            for (i = 0; i < dk; ++i)
                for (j = 0; j < dv; ++j) S[i * dv + j] += k[i] * v[j];
    }
}

/* Read-out o = q^T S (post-update state, Eq. (2)). */
static void orc_readout(int dk, int dv, const double *q, const double *S, double *o)
{
    int i, j;
    for (j = 0; j < dv; ++j) {
        double acc = 0.0;
        for (i = 0; i < dk; ++i) acc += q[i] * S[i * dv + j];
        o[j] = acc;
    }
}

/*
 * Run the recurrence over m[u] tokens for n_units independent units.
 * S: [n_units][dk][dv], holds the initial state on entry and the end state
 * on exit.  v == NULL: no writes (u = 0).  beta is read only for the delta
 * rule.  g is a scalar per token (gate == SCALAR; ldg may be 0 for a
 * per-head constant) or a dk-vector per token (gate == DIAG).
 * q/o optional (both NULL or both set): o_t = q_t^T S_t.
 */
void orc_recur_batch(int rule, int gate, int n_units, int dk, int dv,
                     const double *k, const long *off_k, long ldk,
                     const double *v, const long *off_v, long ldv,
                     const double *beta, const long *off_b, long ldb,
                     const double *g, const long *off_g, long ldg,
                     const double *q, const long *off_q, long ldq,
                     double *o, const long *off_o, long ldo,
                     const int *m, double *S)
{
    long u;
#pragma omp parallel for schedule(dynamic, 1)
    for (u = 0; u < n_units; ++u) {
        double *p = (double *)malloc(sizeof(double) * (size_t)dv);
        double *Su = S + u * (long)dk * dv;
        int t;
        for (t = 0; t < m[u]; ++t) {
            const double *kt = k + off_k[u] + (long)t * ldk;
            const double *vt = v ? v + off_v[u] + (long)t * ldv : NULL;
            double bt = (rule == ORC_DELTA) ? beta[off_b[u] + (long)t * ldb] : 0.0;
            const double *gt = g + off_g[u] + (long)t * ldg;
            orc_step(rule, gate, dk, dv, kt, vt, bt, gt, Su, p);
            if (q && o)
                orc_readout(dk, dv, q + off_q[u] + (long)t * ldq, Su,
                            o + off_o[u] + (long)t * ldo);
        }
        free(p);
    }
}

/*
 * Segment pair per unit, by the two-run construction: S_{C|0} is the end
 * state from S_0 = 0 with the writes; T_C is the end "state" of the same
 * recurrence started from S_0 = I (a dk x dk accumulator) with u = 0.
 * T: [n_units][dk][dk], S0: [n_units][dk][dv] (both overwritten).
 */
void orc_build_batch(int rule, int gate, int n_units, int dk, int dv,
                     const double *k, const long *off_k, long ldk,
                     const double *v, const long *off_v, long ldv,
                     const double *beta, const long *off_b, long ldb,
                     const double *g, const long *off_g, long ldg,
                     const int *m, double *T, double *S0)
{
    long u;
    int i;
    memset(S0, 0, sizeof(double) * (size_t)n_units * dk * dv);
    memset(T, 0, sizeof(double) * (size_t)n_units * dk * dk);
    for (u = 0; u < n_units; ++u)
        for (i = 0; i < dk; ++i) T[u * (long)dk * dk + (long)i * dk + i] = 1.0;
    orc_recur_batch(rule, gate, n_units, dk, dv, k, off_k, ldk, v, off_v, ldv,
                    beta, off_b, ldb, g, off_g, ldg, NULL, NULL, 0, NULL, NULL, 0, m, S0);
    orc_recur_batch(rule, gate, n_units, dk, dk, k, off_k, ldk, NULL, NULL, 0,
                    beta, off_b, ldb, g, off_g, ldg, NULL, NULL, 0, NULL, NULL, 0, m, T);
}

/*
 * One composition step per unit: S <- T S + S0 (Eq. (6) applied one segment
 * at a time).  T: [n_units][dk][dk] dense, S0 and S: [n_units][dk][dv].
 */
void orc_apply_pair_batch(int n_units, int dk, int dv,
                          const double *T, const double *S0, double *S)
{
    long u;
#pragma omp parallel for schedule(static)
    for (u = 0; u < n_units; ++u) {
        const double *Tu = T + u * (long)dk * dk;
        const double *S0u = S0 + u * (long)dk * dv;
        double *Su = S + u * (long)dk * dv;
        double *tmp = (double *)malloc(sizeof(double) * (size_t)dk * dv);
        int i, j, l;
        for (i = 0; i < dk; ++i)
            for (j = 0; j < dv; ++j) {
                double acc = 0.0;
                for (l = 0; l < dk; ++l) acc += Tu[i * dk + l] * Su[l * dv + j];
                tmp[i * dv + j] = acc + S0u[i * dv + j];
            }
        memcpy(Su, tmp, sizeof(double) * (size_t)dk * dv);
        free(tmp);
    }
}

/*
 * Depthwise causal convolution over n rows of C channels, width W:
 *   y[t][c] = sum_{j=0}^{W-1} w[c][j] * x[t - (W-1) + j][c]
 * where rows before the first are taken from hist (W-1 rows, oldest first,
 * i.e. hist[W-2] is the row just before x[0]); hist == NULL means zeros.
 */
void orc_causal_conv(int n, int C, int W, const double *x, long ldx,
                     const double *hist, long ldh, const double *w, double *y, long ldy)
{
    int t, c, j;
    for (t = 0; t < n; ++t)
        for (c = 0; c < C; ++c) {
            double acc = 0.0;
            for (j = 0; j < W; ++j) {
                int src = t - (W - 1) + j;
                double xv;
                if (src >= 0)
                    xv = x[(long)src * ldx + c];
                else
                    xv = hist ? hist[(long)(W - 1 + src) * ldh + c] : 0.0;
                acc += w[(long)c * W + j] * xv;
            }
            y[(long)t * ldy + c] = acc;
        }
}

/* Scale each of n rows of length d to unit Euclidean norm (zero rows stay 0). */
void orc_l2norm_rows(long n, int d, double *x, long ld)
{
    long r;
    int i;
    for (r = 0; r < n; ++r) {
        double s = 0.0;
        for (i = 0; i < d; ++i) s += x[r * ld + i] * x[r * ld + i];
        if (s > 0.0) {
            double inv = 1.0 / sqrt(s);
            for (i = 0; i < d; ++i) x[r * ld + i] *= inv;
        }
    }
}

/*
 * Rotary re-rotation x <- R(delta_r) x of n row vectors of length d (row r at
 * x + r * d).  The leading rot_dim entries form rot_dim / 2 pairs, pair i being
 * entries (i, i + rot_dim/2) (pairing 0) or (2i, 2i + 1) (pairing 1); pair i is
 * turned by the angle delta_r * theta_i, theta_i = base^(-2i / rot_dim):
 *   (x1, x2) <- (x1 cos - x2 sin, x1 sin + x2 cos).
 * Entries past rot_dim are unchanged.  Moving cached keys from start position
 * a to b is delta = b - a (K_b = R(b - a) K_a, ch.2 sec.6, Eq. (8)).
 */
void orc_rope_rows(long n, int d, int rot_dim, int pairing, double base, const double *delta, double *x)
{
    long r;
    int half = rot_dim / 2;
    for (r = 0; r < n; ++r) {
        double *v = x + r * d;
        int i;
        for (i = 0; i < half; ++i) {
            double th = delta[r] * pow(base, -2.0 * (double)i / (double)rot_dim);
            double c = cos(th), sn = sin(th);
            int a = pairing == 0 ? i : 2 * i;
            int b = pairing == 0 ? i + half : 2 * i + 1;
            double x1 = v[a], x2 = v[b];
            v[a] = x1 * c - x2 * sn;
            v[b] = x1 * sn + x2 * c;
        }
    }
}
