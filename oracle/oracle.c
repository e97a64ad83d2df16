/*
 * oracle.c -- plain, slow, obviously correct fp64 CPU oracle for exact attention.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may include, link, load
 * or call this file.  Only tests/, __graft_entry__.smoke() and the cpu_baseline
 * leg of bench.py use it.  It shares no code, header, helper or table with the
 * HIP library; its one input is plain fp64 arrays that the caller has widened
 * exactly from the values stored on the device.
 *
 * What it computes (sources are the three pages this project follows):
 *
 *   [Golden et al., "Is Flash Attention Stable?", sec. II-A]
 *       Attention(Q,K,V) = softmax(Q K^T / sqrt(d_k)) V, with Q, K, V of shape
 *       N x d and an N x N score matrix.  Here the factor 1/sqrt(d_k) is the
 *       caller's `scale` (any positive value).  The fp64 evaluation of this
 *       definition is the "golden value" of that paper's sec. IV-A.
 *
 *   [yadro-code tutorial "How FlashAttention reduces GPU memory traffic",
 *    safe-softmax and online-merge paragraphs]
 *       A row's weights are exp(s_j - max s); subtracting the maximum leaves the
 *       ratio unchanged and keeps every exponent <= 0.  The blocked form keeps a
 *       running maximum m, a running sum l of exponentials and an unnormalised
 *       weighted vector a; a block with a larger maximum M first multiplies l
 *       and a by exp(m - M), then adds its own terms taken relative to M; the
 *       result is a / l, formed once at the end.
 *
 *   [same tutorial, self-checking program and the paragraph after it]
 *       The causal mask is the visible prefix j <= i of row i.  A row with no
 *       visible position has to be given a meaning of its own; this library's
 *       reading is output 0 and log-sum-exp -inf (nothing visible, empty sum).
 *
 *   Key padding (not on the pages): mask[b*N + j] != 0 removes key j of batch
 *   b from every row of that batch.  Log-sum-exp (not on the pages): the
 *   natural log of the sum over visible j of exp(s_j), i.e. m + log(l).
 *
 * Every function below is a direct transcription of one of these statements,
 * with no blocking, fusion or reordering beyond what the statement itself has.
 * Dot products and sums run over ascending index.
 *
 * Layout: q, k, v, o are [B][H][N][d] row-major; lse is [B][H][N]; mask is
 * [B][N] bytes or NULL.  All sizes are >= 0; the functions return 0 on success
 * and -1 on a bad argument (negative size, non-positive width, NULL output).
 */
#include <math.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* Visibility of key j to query row i of batch b. */
static int visible(long b, long i, long j, long N, int causal, const unsigned char* mask)
{
    if (causal && j > i) return 0;
    if (mask && mask[b * N + j] != 0) return 0;
    return 1;
}

/* Score s_ij = scale * sum_c q[i][c] * k[j][c]  (Golden et al., sec. II-A). */
static double score(const double* qi, const double* kj, long d, double scale)
{
    double acc = 0.0;
    for (long c = 0; c < d; ++c) acc += qi[c] * kj[c];
    return scale * acc;
}

/*
 * One query row of the plain definition.  `s` is caller scratch of length N.
 * Writes o_row[0..d) and *lse_row.
 */
static void plain_row(const double* q, const double* k, const double* v,
                      long b, long h, long i, long H, long N, long d,
                      double scale, int causal, const unsigned char* mask,
                      double* s, double* o_row, double* lse_row)
{
    const long base = (b * H + h) * N;
    const double* qi = q + (base + i) * d;
    int any = 0;
    double m = -INFINITY;
    for (long j = 0; j < N; ++j) {
        if (!visible(b, i, j, N, causal, mask)) continue;
        s[j] = score(qi, k + (base + j) * d, d, scale);
        if (!any || s[j] > m) m = s[j];
        any = 1;
    }
    if (!any) {                       /* fully masked row: output 0, lse -inf */
        for (long c = 0; c < d; ++c) o_row[c] = 0.0;
        *lse_row = -INFINITY;
        return;
    }
    double l = 0.0;                    /* safe softmax: weights exp(s - max) */
    for (long c = 0; c < d; ++c) o_row[c] = 0.0;
    for (long j = 0; j < N; ++j) {
        if (!visible(b, i, j, N, causal, mask)) continue;
        const double w = exp(s[j] - m);
        l += w;
        const double* vj = v + (base + j) * d;
        for (long c = 0; c < d; ++c) o_row[c] += w * vj[c];
    }
    for (long c = 0; c < d; ++c) o_row[c] /= l;
    *lse_row = m + log(l);
}

static int bad_sizes(long B, long H, long N, long d)
{
    return B < 0 || H < 0 || N < 0 || d < 0;
}

/* Full tensor, plain definition. */
int oracle_attn_f64(const double* q, const double* k, const double* v,
                    double* o, double* lse, long B, long H, long N, long d,
                    double scale, int causal, const unsigned char* mask)
{
    if (bad_sizes(B, H, N, d) || !o) return -1;
    const long rows = B * H * N;
    if (rows == 0) return 0;
#pragma omp parallel
    {
        double* s = (double*)malloc(sizeof(double) * (size_t)(N > 0 ? N : 1));
#pragma omp for schedule(dynamic, 16)
        for (long r = 0; r < rows; ++r) {
            const long i = r % N, bh = r / N, h = bh % H, b = bh / H;
            double dummy;
            plain_row(q, k, v, b, h, i, H, N, d, scale, causal, mask, s,
                      o + r * d, lse ? lse + r : &dummy);
        }
        free(s);
    }
    return 0;
}

/*
 * Selected rows only, plain definition.  rows[t] is a flat row index
 * (b*H + h)*N + i; results go to o_rows[t][0..d) and lse_rows[t].
 */
int oracle_attn_rows_f64(const double* q, const double* k, const double* v,
                         long B, long H, long N, long d, double scale, int causal,
                         const unsigned char* mask, const long* rows, long nrows,
                         double* o_rows, double* lse_rows)
{
    if (bad_sizes(B, H, N, d) || nrows < 0 || !o_rows || !lse_rows) return -1;
    for (long t = 0; t < nrows; ++t)
        if (rows[t] < 0 || rows[t] >= B * H * N) return -1;
#pragma omp parallel
    {
        double* s = (double*)malloc(sizeof(double) * (size_t)(N > 0 ? N : 1));
#pragma omp for schedule(dynamic, 1)
        for (long t = 0; t < nrows; ++t) {
            const long r = rows[t];
            const long i = r % N, bh = r / N, h = bh % H, b = bh / H;
            plain_row(q, k, v, b, h, i, H, N, d, scale, causal, mask, s,
                      o_rows + t * d, lse_rows + t);
        }
        free(s);
    }
    return 0;
}

/*
 * Block-sparse visibility (the yadro-code tutorial names a block-sparse
 * variant of FlashAttention without describing it; this library's reading):
 * on top of causal and key-padding visibility, the pair (i, j) is visible only
 * if bmask[((b*H + h)*nqb + i/bs)*nkb + j/bs] != 0, with blocks of bs x bs
 * and nqb = nkb = ceil(N / bs).  Plain definition otherwise, as
 * oracle_attn_f64 (rows with nothing visible give 0 and -inf).
 */
int oracle_attn_blockmask_f64(const double* q, const double* k, const double* v,
                              double* o, double* lse, long B, long H, long N, long d,
                              double scale, int causal, const unsigned char* mask,
                              const unsigned char* bmask, long bs)
{
    if (bad_sizes(B, H, N, d) || !o || !lse || !bmask || bs <= 0) return -1;
    const long nb = (N + bs - 1) / bs;
    const long rows = B * H * N;
#pragma omp parallel
    {
        double* s = (double*)malloc(sizeof(double) * (size_t)(N > 0 ? N : 1));
#pragma omp for schedule(dynamic, 8)
        for (long r = 0; r < rows; ++r) {
            const long i = r % N, bh = r / N, b = bh / H;
            const double* qi = q + r * d;
            const unsigned char* brow = bmask + (bh * nb + i / bs) * nb;
            double m = -INFINITY;
            int any = 0;
            for (long j = 0; j < N; ++j) {
                if (!visible(b, i, j, N, causal, mask) || !brow[j / bs]) { s[j] = -INFINITY; continue; }
                s[j] = score(qi, k + (bh * N + j) * d, d, scale);
                if (!any || s[j] > m) m = s[j];
                any = 1;
            }
            double* orow = o + r * d;
            for (long c = 0; c < d; ++c) orow[c] = 0.0;
            if (!any) { lse[r] = -INFINITY; continue; }
            double l = 0.0;
            for (long j = 0; j < N; ++j) {
                if (s[j] == -INFINITY) continue;
                const double w = exp(s[j] - m);
                l += w;
                for (long c = 0; c < d; ++c) orow[c] += w * v[(bh * N + j) * d + c];
            }
            for (long c = 0; c < d; ++c) orow[c] /= l;
            lse[r] = m + log(l);
        }
        free(s);
    }
    return 0;
}

/*
 * Gradient of the plain definition (reverse mode of softmax(scale q k^T) v),
 * written out from the definition with the chain rule: for one (b, h), with
 * P the row softmax over visible keys and O = P V,
 *     dV = P^T dO,   dP = dO V^T,   dS_ij = P_ij (dP_ij - sum_c dO_ic O_ic),
 *     dQ = scale dS K,   dK = scale dS^T Q.
 * Masked pairs have P = 0 and contribute nothing; a row with no visible key
 * has O = 0 and contributes nothing.  All [B][H][N][d]; fp64 throughout.
 */
int oracle_attn_bwd_f64(const double* q, const double* k, const double* v, const double* dout,
                        double* dq, double* dk, double* dv, long B, long H, long N, long d,
                        double scale, int causal, const unsigned char* mask)
{
    if (bad_sizes(B, H, N, d) || !dq || !dk || !dv) return -1;
    const long BH = B * H;
#pragma omp parallel for schedule(dynamic, 1)
    for (long bh = 0; bh < BH; ++bh) {
        const long b = bh / H;
        const double* Q = q + bh * N * d;
        const double* K = k + bh * N * d;
        const double* V = v + bh * N * d;
        const double* dO = dout + bh * N * d;
        double* dQ = dq + bh * N * d;
        double* dK = dk + bh * N * d;
        double* dV = dv + bh * N * d;
        for (long t = 0; t < N * d; ++t) { dQ[t] = 0.0; dK[t] = 0.0; dV[t] = 0.0; }
        double* P = (double*)malloc(sizeof(double) * (size_t)(N > 0 ? N : 1));
        double* orow = (double*)malloc(sizeof(double) * (size_t)(d > 0 ? d : 1));
        for (long i = 0; i < N; ++i) {
            /* forward for row i: P_i. and O_i */
            double m = -INFINITY;
            int any = 0;
            for (long j = 0; j < N; ++j) {
                if (!visible(b, i, j, N, causal, mask)) { P[j] = -INFINITY; continue; }
                P[j] = score(Q + i * d, K + j * d, d, scale);
                if (!any || P[j] > m) m = P[j];
                any = 1;
            }
            if (!any) continue;
            double l = 0.0;
            for (long j = 0; j < N; ++j) {
                P[j] = (P[j] == -INFINITY) ? 0.0 : exp(P[j] - m);
                l += P[j];
            }
            for (long c = 0; c < d; ++c) orow[c] = 0.0;
            for (long j = 0; j < N; ++j) {
                P[j] /= l;
                for (long c = 0; c < d; ++c) orow[c] += P[j] * V[j * d + c];
            }
            double Di = 0.0;                       /* sum_c dO_ic O_ic */
            for (long c = 0; c < d; ++c) Di += dO[i * d + c] * orow[c];
            for (long j = 0; j < N; ++j) {
                if (P[j] == 0.0) continue;
                double dPij = 0.0;
                for (long c = 0; c < d; ++c) dPij += dO[i * d + c] * V[j * d + c];
                const double dSij = P[j] * (dPij - Di);
                for (long c = 0; c < d; ++c) {
                    dV[j * d + c] += P[j] * dO[i * d + c];
                    dQ[i * d + c] += scale * dSij * K[j * d + c];
                    dK[j * d + c] += scale * dSij * Q[i * d + c];
                }
            }
        }
        free(P);
        free(orow);
    }
    return 0;
}

/*
 * Query block against a longer key/value sequence, plain definition (the
 * tutorial's remark that prompt processing and step-by-step generation with a
 * key/value cache have different matrix shapes: here Nq query rows meet Nk
 * cached keys).  q, o are [B][H][Nq][d], k, v are [B][H][Nk][d], lse is
 * [B][H][Nq], mask is [B][Nk] or NULL.  Causal visibility is aligned to the
 * end of the cache: query row i sits at position Nk - Nq + i and sees keys
 * j <= Nk - Nq + i (with Nq = Nk this is the j <= i prefix).
 */
int oracle_attn_kv_f64(const double* q, const double* k, const double* v,
                       double* o, double* lse, long B, long H, long Nq, long Nk, long d,
                       double scale, int causal, const unsigned char* mask)
{
    if (B < 0 || H < 0 || Nq < 0 || Nk < 0 || d < 0 || !o || !lse) return -1;
    const long rows = B * H * Nq;
#pragma omp parallel
    {
        double* s = (double*)malloc(sizeof(double) * (size_t)(Nk > 0 ? Nk : 1));
#pragma omp for schedule(dynamic, 4)
        for (long r = 0; r < rows; ++r) {
            const long i = r % Nq, bh = r / Nq, b = bh / H;
            const double* qi = q + r * d;
            const double* kb = k + bh * Nk * d;
            const double* vb = v + bh * Nk * d;
            const long last = causal ? Nk - Nq + i : Nk - 1;    /* last visible key */
            double m = -INFINITY;
            int any = 0;
            for (long j = 0; j < Nk; ++j) {
                if (j > last || (mask && mask[b * Nk + j] != 0)) continue;
                s[j] = score(qi, kb + j * d, d, scale);
                if (!any || s[j] > m) m = s[j];
                any = 1;
            }
            double* orow = o + r * d;
            for (long c = 0; c < d; ++c) orow[c] = 0.0;
            if (!any) { lse[r] = -INFINITY; continue; }
            double l = 0.0;
            for (long j = 0; j < Nk; ++j) {
                if (j > last || (mask && mask[b * Nk + j] != 0)) continue;
                const double w = exp(s[j] - m);
                l += w;
                for (long c = 0; c < d; ++c) orow[c] += w * vb[j * d + c];
            }
            for (long c = 0; c < d; ++c) orow[c] /= l;
            lse[r] = m + log(l);
        }
        free(s);
    }
    return 0;
}

/*
 * Running state of the online merge for one row: maximum m, sum of
 * exponentials l, unnormalised weighted vector a[0..d).
 */
typedef struct { double m, l; double* a; } row_state;

/*
 * Fold one block of (score, value-row) pairs into a row state, following the
 * tutorial's online-merge paragraph: block maximum, new maximum, rescale the
 * old sum and vector by exp(m - M), then add each term exp(s - M).
 *
 * Guard, which the tutorial's own program lacks because it assumes at least
 * one visible element: a block in which nothing is visible and nothing was
 * visible before it leaves the state untouched, instead of evaluating
 * exp(-inf - (-inf)).  `rescale` = 0 is a deliberately wrong variant (the
 * tutorial's exercise) used only by the mutation test.
 */
static void fold_block(row_state* st, const double* s, const double* const* vals,
                       const unsigned char* vis, long n, long d, int rescale)
{
    double mt = -INFINITY;
    for (long t = 0; t < n; ++t)
        if (vis[t] && s[t] > mt) mt = s[t];
    const double m_new = st->m > mt ? st->m : mt;
    if (m_new == -INFINITY) return;            /* nothing visible yet */
    if (rescale) {
        const double alpha = exp(st->m - m_new);   /* exp(-inf) = 0 when m = -inf */
        st->l *= alpha;
        for (long c = 0; c < d; ++c) st->a[c] *= alpha;
    }
    for (long t = 0; t < n; ++t) {
        if (!vis[t]) continue;
        const double w = exp(s[t] - m_new);
        st->l += w;
        for (long c = 0; c < d; ++c) st->a[c] += w * vals[t][c];
    }
    st->m = m_new;
}

/* Final normalisation a / l, once, at the end; empty sum -> (0, -inf). */
static void finish_row(const row_state* st, long d, double* o_row, double* lse_row)
{
    if (st->l == 0.0) {
        for (long c = 0; c < d; ++c) o_row[c] = 0.0;
        *lse_row = -INFINITY;
        return;
    }
    for (long c = 0; c < d; ++c) o_row[c] = st->a[c] / st->l;
    *lse_row = st->m + log(st->l);
}

/*
 * Score-level API, as in the tutorial's program: one row of n scores s[0..n)
 * with value rows vals[j][0..dv) (row-major n x dv).
 */
int oracle_row_softmax_f64(const double* s, const double* vals, long n, long dv,
                           double* out, double* lse)
{
    if (n < 0 || dv < 0 || !out || !lse) return -1;
    if (n == 0) {
        for (long c = 0; c < dv; ++c) out[c] = 0.0;
        *lse = -INFINITY;
        return 0;
    }
    double m = s[0];
    for (long j = 1; j < n; ++j) if (s[j] > m) m = s[j];
    double l = 0.0;
    for (long c = 0; c < dv; ++c) out[c] = 0.0;
    for (long j = 0; j < n; ++j) {
        const double w = exp(s[j] - m);
        l += w;
        for (long c = 0; c < dv; ++c) out[c] += w * vals[j * dv + c];
    }
    for (long c = 0; c < dv; ++c) out[c] /= l;
    *lse = m + log(l);
    return 0;
}

/*
 * Blocked online form at score level: blocks [t*width, min(n,(t+1)*width)),
 * visited in ascending (order = 0) or descending (order = 1) t.  `vis` may be
 * NULL (everything visible).  `rescale` = 1 is the correct algorithm.
 */
int oracle_row_blocked_f64(const double* s, const double* vals, const unsigned char* vis,
                           long n, long dv, long width, int order, int rescale,
                           double* out, double* lse)
{
    if (n < 0 || dv < 0 || width <= 0 || !out || !lse) return -1;
    double* a = (double*)calloc((size_t)(dv > 0 ? dv : 1), sizeof(double));
    const double** vp = (const double**)malloc(sizeof(double*) * (size_t)(width));
    unsigned char* vb = (unsigned char*)malloc((size_t)width);
    if (!a || !vp || !vb) { free(a); free(vp); free(vb); return -1; }
    row_state st = { -INFINITY, 0.0, a };
    const long nblk = (n + width - 1) / width;
    for (long u = 0; u < nblk; ++u) {
        const long t = order ? nblk - 1 - u : u;
        const long j0 = t * width, j1 = (j0 + width < n) ? j0 + width : n;
        for (long j = j0; j < j1; ++j) {
            vp[j - j0] = vals + j * dv;
            vb[j - j0] = vis ? vis[j] : 1;
        }
        fold_block(&st, s + j0, vp, vb, j1 - j0, dv, rescale);
    }
    finish_row(&st, dv, out, lse);
    free(a); free(vp); free(vb);
    return 0;
}

/*
 * Full tensor, blocked online form, query-row outer loop: each row folds the
 * key tiles [t*bc, min(N,(t+1)*bc)) in ascending (order 0) or descending
 * (order 1) t.
 */
int oracle_attn_blocked_f64(const double* q, const double* k, const double* v,
                            double* o, double* lse, long B, long H, long N, long d,
                            double scale, int causal, const unsigned char* mask,
                            long bc, int order)
{
    if (bad_sizes(B, H, N, d) || bc <= 0 || !o) return -1;
    const long rows = B * H * N;
    if (rows == 0) return 0;
    const long nblk = (N + bc - 1) / bc;
#pragma omp parallel
    {
        double* a = (double*)calloc((size_t)(d > 0 ? d : 1), sizeof(double));
        double* s = (double*)malloc(sizeof(double) * (size_t)bc);
        const double** vp = (const double**)malloc(sizeof(double*) * (size_t)bc);
        unsigned char* vb = (unsigned char*)malloc((size_t)bc);
#pragma omp for schedule(dynamic, 16)
        for (long r = 0; r < rows; ++r) {
            const long i = r % N, bh = r / N, h = bh % H, b = bh / H;
            const long base = (b * H + h) * N;
            for (long c = 0; c < d; ++c) a[c] = 0.0;
            row_state st = { -INFINITY, 0.0, a };
            for (long u = 0; u < nblk; ++u) {
                const long t = order ? nblk - 1 - u : u;
                const long j0 = t * bc, j1 = (j0 + bc < N) ? j0 + bc : N;
                for (long j = j0; j < j1; ++j) {
                    vb[j - j0] = (unsigned char)visible(b, i, j, N, causal, mask);
                    s[j - j0] = vb[j - j0] ? score(q + (base + i) * d, k + (base + j) * d, d, scale)
                                           : -INFINITY;
                    vp[j - j0] = v + (base + j) * d;
                }
                fold_block(&st, s, vp, vb, j1 - j0, d, 1);
            }
            double dummy;
            finish_row(&st, d, o + r * d, lse ? lse + r : &dummy);
        }
        free(a); free(s); free(vp); free(vb);
    }
    return 0;
}

/*
 * Full tensor, blocked online form with the loop nest swapped: the key tile
 * is the outer loop and every row of a (b, h) updates its own state for that
 * tile before the next tile starts.  Each row sees exactly the same sequence
 * of operations as in oracle_attn_blocked_f64.
 */
int oracle_attn_blocked_kvouter_f64(const double* q, const double* k, const double* v,
                                    double* o, double* lse, long B, long H, long N, long d,
                                    double scale, int causal, const unsigned char* mask,
                                    long bc, int order)
{
    if (bad_sizes(B, H, N, d) || bc <= 0 || !o) return -1;
    if (B * H * N == 0) return 0;
    const long nblk = (N + bc - 1) / bc;
#pragma omp parallel for schedule(dynamic, 1)
    for (long bh = 0; bh < B * H; ++bh) {
        const long b = bh / H;
        const long base = bh * N;
        row_state* st = (row_state*)malloc(sizeof(row_state) * (size_t)N);
        double* acc = (double*)calloc((size_t)(N * (d > 0 ? d : 1)), sizeof(double));
        double* s = (double*)malloc(sizeof(double) * (size_t)bc);
        const double** vp = (const double**)malloc(sizeof(double*) * (size_t)bc);
        unsigned char* vb = (unsigned char*)malloc((size_t)bc);
        for (long i = 0; i < N; ++i) { st[i].m = -INFINITY; st[i].l = 0.0; st[i].a = acc + i * d; }
        for (long u = 0; u < nblk; ++u) {
            const long t = order ? nblk - 1 - u : u;
            const long j0 = t * bc, j1 = (j0 + bc < N) ? j0 + bc : N;
            for (long i = 0; i < N; ++i) {
                for (long j = j0; j < j1; ++j) {
                    vb[j - j0] = (unsigned char)visible(b, i, j, N, causal, mask);
                    s[j - j0] = vb[j - j0] ? score(q + (base + i) * d, k + (base + j) * d, d, scale)
                                           : -INFINITY;
                    vp[j - j0] = v + (base + j) * d;
                }
                fold_block(&st[i], s, vp, vb, j1 - j0, d, 1);
            }
        }
        for (long i = 0; i < N; ++i) {
            double dummy;
            finish_row(&st[i], d, o + (base + i) * d, lse ? lse + base + i : &dummy);
        }
        free(st); free(acc); free(s); free(vp); free(vb);
    }
    return 0;
}

/* Number of OpenMP threads a parallel region would use (for reports). */
int oracle_num_threads(void)
{
    int n = 1;
#pragma omp parallel
    {
#pragma omp single
        {
#ifdef _OPENMP
            n = omp_get_num_threads();
#endif
        }
    }
    return n;
}

/* Threads of the parallel loops that follow (only for timing the oracle on
 * one thread; the arithmetic of every routine is the same for any count). */
void oracle_set_threads(int n)
{
#ifdef _OPENMP
    if (n > 0) omp_set_num_threads(n);
#else
    (void)n;
#endif
}
