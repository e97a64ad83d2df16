/*
 * emulate.c -- precision-emulating model of tiled online-softmax attention and
 * of baseline attention (TEST INFRASTRUCTURE ONLY; not the oracle of parity).
 *
 * Golden et al., "Is Flash Attention Stable?", sec. III, measure numerical
 * deviation with a microbenchmark that runs the flash algorithm and baseline
 * attention with their intermediate values held in a chosen numerical format,
 * and compares both with an fp64 "golden value" (sec. IV-A, Figs. 3-6).  This
 * file is such a model, written from that description: every arithmetic step
 * is done in fp64 and its result rounded to the format the step is assigned.
 * Formats are (p, emin, emax): p significant bits (with the implicit one),
 * normal exponents emin..emax, gradual underflow, round to nearest even,
 * overflow to infinity.  p = 0 means "no rounding" (plain fp64).
 *
 * Flash model (the blocked algorithm of the yadro-code tutorial "How
 * FlashAttention reduces GPU memory traffic", online-merge paragraphs, with
 * the -inf guard of this project's oracle):
 *   s_j   = R_acc(scale * dot_acc(q, k_j))                 dot: R_acc per add
 *   m'    = max(m, max_tile s_j)
 *   alpha = R_acc(exp(m - m'))                             (0 when m = -inf)
 *   l     = R_acc(alpha * l),  acc_c = R_acc(alpha * acc_c)
 *   P_j   = R_p(R_acc(exp(R_acc(s_j - m'))))
 *   l     = R_acc(l + P_j),    acc_c = R_acc(acc_c + P_j * v_jc)   (one rounding)
 *   between key tiles, when the state is stored: l = R_state(l), acc = R_state(acc)
 *   o_c   = R_out(R_acc(acc_c / l))
 * The Q-outer nest keeps each row's state across all its tiles; the KV-outer
 * nest walks tiles outermost and keeps every row's state in arrays, rounding
 * it to the state format between tiles (the state would live in memory).
 *
 * Baseline model (Golden et al., sec. II-A: S, softmax(S), then P V, with S
 * and P materialised):
 *   S_j = R_store(R_acc(scale * dot_acc(q, k_j)));  m = max_j S_j
 *   e_j = R_acc(exp(R_acc(S_j - m)));  z = sum_acc e_j
 *   P_j = R_store(R_acc(e_j / z));     o_c = R_out(sum_acc R_acc(P_j * v_jc))
 *
 * Layout: q, k, v are [B][H][N][d] fp64 holding the (already rounded) input
 * values; rows[] are flat row indices (b*H + h)*N + i; o_rows is [nrows][d].
 * No masking here except the causal prefix.  Return 0, or -1 on bad arguments.
 */
#include <math.h>
#include <stdlib.h>

typedef struct emu_fmt {
    int p;       /* significant bits; 0 = no rounding */
    int emin;    /* smallest normal exponent */
    int emax;    /* largest exponent */
} emu_fmt;

typedef struct emu_cfg {
    emu_fmt acc;     /* arithmetic of dot products, sums and the running state */
    emu_fmt pfmt;    /* P as fed to P.V and to l */
    emu_fmt state;   /* l and acc between key tiles when stored (KV-outer) */
    emu_fmt out;     /* output storage */
    long bc;         /* keys per tile */
    int order;       /* 0 ascending tiles, 1 descending */
    int kv_outer;    /* 0 Q-outer nest, 1 KV-outer nest (state rounded between tiles) */
} emu_cfg;

double emu_round(double x, int p, int emin, int emax)
{
    if (p <= 0 || x == 0.0 || !isfinite(x)) return x;
    int e;
    (void)frexp(x, &e);                 /* |x| in [2^(e-1), 2^e) */
    int E = e - 1;
    if (E < emin) E = emin;             /* subnormal range: fixed quantum */
    const double quantum = ldexp(1.0, E - (p - 1));
    const double r = nearbyint(x / quantum) * quantum;
    const double maxv = ldexp(2.0 - ldexp(1.0, 1 - p), emax);
    if (fabs(r) > maxv) return copysign(INFINITY, x);
    return r;
}

static double R(double x, const emu_fmt* f) { return emu_round(x, f->p, f->emin, f->emax); }

static double dot_acc(const double* a, const double* b, long d, const emu_fmt* f)
{
    double s = 0.0;
    for (long c = 0; c < d; ++c) s = R(s + a[c] * b[c], f);
    return s;
}

static void tile_range(long t, long bc, long N, long* j0, long* j1)
{
    *j0 = t * bc;
    *j1 = (t + 1) * bc < N ? (t + 1) * bc : N;
}

/* One step of the online merge for one row and one tile. */
static void merge_tile(const double* qi, const double* K, const double* V, long i, long j0, long j1,
                       long d, double scale, int causal, const emu_cfg* cfg,
                       double* m, double* l, double* acc, double* s)
{
    double mt = -INFINITY;
    for (long j = j0; j < j1; ++j) {
        if (causal && j > i) { s[j - j0] = -INFINITY; continue; }
        s[j - j0] = R(scale * dot_acc(qi, K + j * d, d, &cfg->acc), &cfg->acc);
        if (s[j - j0] > mt) mt = s[j - j0];
    }
    const double m_new = *m > mt ? *m : mt;
    if (m_new == -INFINITY) return;                         /* nothing visible yet */
    const double alpha = (*m == -INFINITY) ? 0.0 : R(exp(*m - m_new), &cfg->acc);
    *l = R(alpha * *l, &cfg->acc);
    for (long c = 0; c < d; ++c) acc[c] = R(alpha * acc[c], &cfg->acc);
    for (long j = j0; j < j1; ++j) {
        if (s[j - j0] == -INFINITY) continue;
        const double pj = R(R(exp(R(s[j - j0] - m_new, &cfg->acc)), &cfg->acc), &cfg->pfmt);
        *l = R(*l + pj, &cfg->acc);
        const double* vj = V + j * d;
        for (long c = 0; c < d; ++c) acc[c] = R(acc[c] + pj * vj[c], &cfg->acc);
    }
    *m = m_new;
}

static void finish_row(double m, double l, const double* acc, long d, const emu_cfg* cfg, double* o)
{
    (void)m;
    for (long c = 0; c < d; ++c)
        o[c] = (l > 0.0) ? R(R(acc[c] / l, &cfg->acc), &cfg->out) : 0.0;
}

int emu_flash_rows(const double* q, const double* k, const double* v, long B, long H, long N, long d,
                   double scale, int causal, const emu_cfg* cfg, const long* rows, long nrows,
                   double* o_rows)
{
    if (B < 0 || H < 0 || N < 0 || d <= 0 || !cfg || cfg->bc <= 0 || nrows < 0 || (nrows && (!rows || !o_rows)))
        return -1;
    const long nt = (N + cfg->bc - 1) / cfg->bc;
    for (long t = 0; t < nrows; ++t)
        if (rows[t] < 0 || rows[t] >= B * H * N) return -1;
    if (!cfg->kv_outer) {
#pragma omp parallel
        {
            double* s = (double*)malloc(sizeof(double) * (size_t)cfg->bc);
            double* acc = (double*)malloc(sizeof(double) * (size_t)d);
#pragma omp for schedule(dynamic, 4)
            for (long t = 0; t < nrows; ++t) {
                const long r = rows[t], i = r % N, bh = r / N;
                const double* K = k + bh * N * d;
                const double* V = v + bh * N * d;
                double m = -INFINITY, l = 0.0;
                for (long c = 0; c < d; ++c) acc[c] = 0.0;
                for (long u = 0; u < nt; ++u) {
                    long j0, j1;
                    tile_range(cfg->order ? nt - 1 - u : u, cfg->bc, N, &j0, &j1);
                    merge_tile(q + r * d, K, V, i, j0, j1, d, scale, causal, cfg, &m, &l, acc, s);
                }
                finish_row(m, l, acc, d, cfg, o_rows + t * d);
            }
            free(s);
            free(acc);
        }
        return 0;
    }
    /* KV-outer: tiles outermost, every row's state in arrays between tiles */
    double* M = (double*)malloc(sizeof(double) * (size_t)(nrows ? nrows : 1));
    double* L = (double*)malloc(sizeof(double) * (size_t)(nrows ? nrows : 1));
    double* A = (double*)malloc(sizeof(double) * (size_t)(nrows ? nrows : 1) * (size_t)d);
    if (!M || !L || !A) { free(M); free(L); free(A); return -1; }
    for (long t = 0; t < nrows; ++t) {
        M[t] = -INFINITY; L[t] = 0.0;
        for (long c = 0; c < d; ++c) A[t * d + c] = 0.0;
    }
    for (long u = 0; u < nt; ++u) {
        long j0, j1;
        tile_range(cfg->order ? nt - 1 - u : u, cfg->bc, N, &j0, &j1);
#pragma omp parallel
        {
            double* s = (double*)malloc(sizeof(double) * (size_t)cfg->bc);
#pragma omp for schedule(dynamic, 4)
            for (long t = 0; t < nrows; ++t) {
                const long r = rows[t], i = r % N, bh = r / N;
                merge_tile(q + r * d, k + bh * N * d, v + bh * N * d, i, j0, j1, d, scale, causal, cfg,
                           &M[t], &L[t], A + t * d, s);
                L[t] = R(L[t], &cfg->state);
                for (long c = 0; c < d; ++c) A[t * d + c] = R(A[t * d + c], &cfg->state);
            }
            free(s);
        }
    }
    for (long t = 0; t < nrows; ++t) finish_row(M[t], L[t], A + t * d, d, cfg, o_rows + t * d);
    free(M); free(L); free(A);
    return 0;
}

int emu_baseline_rows(const double* q, const double* k, const double* v, long B, long H, long N, long d,
                      double scale, int causal, const emu_fmt* acc, const emu_fmt* store, const emu_fmt* out,
                      const long* rows, long nrows, double* o_rows)
{
    if (B < 0 || H < 0 || N < 0 || d <= 0 || !acc || !store || !out || nrows < 0 || (nrows && (!rows || !o_rows)))
        return -1;
    for (long t = 0; t < nrows; ++t)
        if (rows[t] < 0 || rows[t] >= B * H * N) return -1;
#pragma omp parallel
    {
        double* S = (double*)malloc(sizeof(double) * (size_t)(N ? N : 1));
        double* P = (double*)malloc(sizeof(double) * (size_t)(N ? N : 1));
#pragma omp for schedule(dynamic, 4)
        for (long t = 0; t < nrows; ++t) {
            const long r = rows[t], i = r % N, bh = r / N;
            const double* qi = q + r * d;
            const long jn = causal ? i + 1 : N;
            double m = -INFINITY;
            for (long j = 0; j < jn; ++j) {
                S[j] = R(R(scale * dot_acc(qi, k + (bh * N + j) * d, d, acc), acc), store);
                if (S[j] > m) m = S[j];
            }
            double z = 0.0;
            for (long j = 0; j < jn; ++j) {
                P[j] = R(exp(R(S[j] - m, acc)), acc);
                z = R(z + P[j], acc);
            }
            for (long j = 0; j < jn; ++j) P[j] = R(R(P[j] / z, acc), store);
            double* o = o_rows + t * d;
            for (long c = 0; c < d; ++c) {
                double a = 0.0;
                for (long j = 0; j < jn; ++j) a = R(a + P[j] * v[(bh * N + j) * d + c], acc);
                o[c] = R(a, out);
            }
        }
        free(S);
        free(P);
    }
    return 0;
}
