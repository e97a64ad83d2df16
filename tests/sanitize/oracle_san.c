/*
 * oracle_san.c -- the fp64 oracle and the precision model (oracle/oracle.c,
 * oracle/emulate.c) built with gcc under AddressSanitizer and
 * UndefinedBehaviorSanitizer and driven over small ragged shapes, masks that
 * empty whole rows, every blocked form and the argument errors.  Besides the
 * sanitizers' own checks it asserts properties that hold by construction:
 * a row that sees one key returns that key's value row exactly, rows with
 * nothing visible give 0 and -inf, the two blocked loop nests agree bit for
 * bit, and the blocked forms, the row API, the cache form and the model with
 * rounding switched off agree with the plain definition.  Exit status 0 when
 * every check holds.
 */
#include <math.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

/* the oracle's exported functions (liboracle.so) */
int oracle_attn_f64(const double*, const double*, const double*, double*, double*, long, long, long, long,
                    double, int, const unsigned char*);
int oracle_attn_rows_f64(const double*, const double*, const double*, long, long, long, long, double, int,
                         const unsigned char*, const long*, long, double*, double*);
int oracle_attn_blockmask_f64(const double*, const double*, const double*, double*, double*, long, long, long,
                              long, double, int, const unsigned char*, const unsigned char*, long);
int oracle_attn_bwd_f64(const double*, const double*, const double*, const double*, double*, double*, double*,
                        long, long, long, long, double, int, const unsigned char*);
int oracle_attn_kv_f64(const double*, const double*, const double*, double*, double*, long, long, long, long,
                       long, double, int, const unsigned char*);
int oracle_row_softmax_f64(const double*, const double*, long, long, double*, double*);
int oracle_row_blocked_f64(const double*, const double*, const unsigned char*, long, long, long, int, int,
                           double*, double*);
int oracle_attn_blocked_f64(const double*, const double*, const double*, double*, double*, long, long, long,
                            long, double, int, const unsigned char*, long, int);
int oracle_attn_blocked_kvouter_f64(const double*, const double*, const double*, double*, double*, long, long,
                                    long, long, double, int, const unsigned char*, long, int);
int oracle_num_threads(void);
void oracle_set_threads(int);

/* the precision model's argument structs, as emulate.c lays them out */
typedef struct { int p, emin, emax; } emu_fmt;
typedef struct { emu_fmt acc, pfmt, state, out; long bc; int order; int kv_outer; } emu_cfg;
double emu_round(double, int, int, int);
int emu_flash_rows(const double*, const double*, const double*, long, long, long, long, double, int,
                   const emu_cfg*, const long*, long, double*);
int emu_baseline_rows(const double*, const double*, const double*, long, long, long, long, double, int,
                      const emu_fmt*, const emu_fmt*, const emu_fmt*, const long*, long, double*);

static int failures = 0;
#define CHECK(c)                                                                    \
    do {                                                                            \
        if (!(c)) {                                                                 \
            fprintf(stderr, "%s:%d: check failed: %s\n", __FILE__, __LINE__, #c);   \
            ++failures;                                                             \
        }                                                                           \
    } while (0)

static unsigned long long rng = 0x9e3779b97f4a7c15ULL;
static double uniform(void) /* in [-1, 1) */
{
    rng = rng * 6364136223846793005ULL + 1442695040888963407ULL;
    return (double)(rng >> 11) / 4503599627370496.0 - 1.0;
}

static double* randn(long n)
{
    double* a = (double*)malloc(sizeof(double) * (size_t)(n > 0 ? n : 1));
    for (long i = 0; i < n; ++i) a[i] = uniform();
    return a;
}

static double maxdiff(const double* a, const double* b, long n)
{
    double m = 0.0;
    for (long i = 0; i < n; ++i) {
        if (isinf(a[i]) || isinf(b[i])) {
            if (a[i] != b[i]) return INFINITY;
            continue;
        }
        const double e = fabs(a[i] - b[i]);
        if (!(e <= m)) m = e;
    }
    return m;
}

int main(void)
{
    const long B = 2, H = 2, N = 37, d = 16;
    const long rows = B * H * N, n = rows * d;
    const double scale = 0.25;
    double *q = randn(n), *k = randn(n), *v = randn(n);
    unsigned char mask[2 * 37];
    for (long j = 0; j < N; ++j) {
        mask[j] = (unsigned char)(j % 5 == 3);   /* nonzero = padded; batch 0: some keys, key 0 visible */
        mask[N + j] = 1;                        /* batch 1: every key padded */
    }
    double* o = (double*)malloc(sizeof(double) * n);
    double* lse = (double*)malloc(sizeof(double) * rows);
    double* o2 = (double*)malloc(sizeof(double) * n);
    double* lse2 = (double*)malloc(sizeof(double) * rows);

    oracle_set_threads(2);
    CHECK(oracle_num_threads() >= 1);

    /* plain definition, causal with padding */
    CHECK(oracle_attn_f64(q, k, v, o, lse, B, H, N, d, scale, 1, mask) == 0);
    for (long h = 0; h < H; ++h) {
        const long r0 = (0 * H + h) * N;                  /* batch 0, row 0: sees key 0 only */
        CHECK(memcmp(o + r0 * d, v + r0 * d, sizeof(double) * d) == 0);
        double s = 0.0;
        for (long c = 0; c < d; ++c) s += q[r0 * d + c] * k[r0 * d + c];
        CHECK(lse[r0] == s * scale);
        for (long i = 0; i < N; ++i) {                    /* batch 1: nothing visible */
            const long r = (1 * H + h) * N + i;
            CHECK(isinf(lse[r]) && lse[r] < 0);
            for (long c = 0; c < d; ++c) CHECK(o[r * d + c] == 0.0 && !signbit(o[r * d + c]));
        }
    }

    /* selected rows: the same plain definition */
    long sel[5] = {0, 1, 36, 40, rows - 1};
    double orow[5 * 16], lrow[5];
    CHECK(oracle_attn_rows_f64(q, k, v, B, H, N, d, scale, 1, mask, sel, 5, orow, lrow) == 0);
    for (int t = 0; t < 5; ++t) {
        CHECK(memcmp(orow + t * d, o + sel[t] * d, sizeof(double) * d) == 0);
        CHECK(lrow[t] == lse[sel[t]] || (isinf(lrow[t]) && isinf(lse[sel[t]])));
    }
    long bad_row = rows;
    CHECK(oracle_attn_rows_f64(q, k, v, B, H, N, d, scale, 1, mask, &bad_row, 1, orow, lrow) == -1);

    /* blocked forms: both nests bit for bit, ragged tiles, both orders */
    for (int order = 0; order < 2; ++order)
        for (long bc = 1; bc <= 9; bc += 4) {
            CHECK(oracle_attn_blocked_f64(q, k, v, o2, lse2, B, H, N, d, scale, 1, mask, bc, order) == 0);
            double* o3 = (double*)malloc(sizeof(double) * n);
            double* l3 = (double*)malloc(sizeof(double) * rows);
            CHECK(oracle_attn_blocked_kvouter_f64(q, k, v, o3, l3, B, H, N, d, scale, 1, mask, bc, order) == 0);
            CHECK(memcmp(o2, o3, sizeof(double) * n) == 0);
            CHECK(maxdiff(lse2, l3, rows) == 0.0);
            CHECK(maxdiff(o2, o, n) < 1e-13);
            CHECK(maxdiff(lse2, lse, rows) < 1e-13);
            free(o3);
            free(l3);
        }

    /* block flags all set: the plain definition */
    const long bs = 8, nb = (N + bs - 1) / bs;
    unsigned char* bm = (unsigned char*)malloc((size_t)(B * H * nb * nb));
    memset(bm, 1, (size_t)(B * H * nb * nb));
    CHECK(oracle_attn_blockmask_f64(q, k, v, o2, lse2, B, H, N, d, scale, 1, mask, bm, bs) == 0);
    CHECK(maxdiff(o2, o, n) < 1e-14 && maxdiff(lse2, lse, rows) < 1e-14);
    /* only the diagonal blocks: row 0 of every head still sees key 0 */
    memset(bm, 0, (size_t)(B * H * nb * nb));
    for (long bh = 0; bh < B * H; ++bh)
        for (long t = 0; t < nb; ++t) bm[(bh * nb + t) * nb + t] = 1;
    CHECK(oracle_attn_blockmask_f64(q, k, v, o2, lse2, B, H, N, d, scale, 1, NULL, bm, bs) == 0);
    CHECK(memcmp(o2, v, sizeof(double) * d) == 0);
    CHECK(oracle_attn_blockmask_f64(q, k, v, o2, lse2, B, H, N, d, scale, 1, NULL, bm, 0) == -1);
    free(bm);

    /* cache form with Nq = Nk is the full causal form; Nq < Nk shifts the diagonal */
    CHECK(oracle_attn_kv_f64(q, k, v, o2, lse2, B, H, N, N, d, scale, 1, mask) == 0);
    CHECK(maxdiff(o2, o, n) < 1e-14 && maxdiff(lse2, lse, rows) < 1e-14);
    {
        const long Nq = 3;
        double* qs = randn(B * H * Nq * d);
        double* os = (double*)malloc(sizeof(double) * B * H * Nq * d);
        double* ls = (double*)malloc(sizeof(double) * B * H * Nq);
        CHECK(oracle_attn_kv_f64(qs, k, v, os, ls, B, H, Nq, N, d, scale, 1, NULL) == 0);
        for (long i = 0; i < B * H * Nq; ++i) CHECK(isfinite(ls[i]));
        CHECK(oracle_attn_kv_f64(qs, k, v, os, ls, B, H, Nq, 0, d, scale, 1, NULL) == 0);   /* empty cache */
        for (long i = 0; i < B * H * Nq; ++i) CHECK(isinf(ls[i]) && os[i * d] == 0.0);
        free(qs);
        free(os);
        free(ls);
    }

    /* gradient: finite; with every key padded it is exactly zero */
    {
        double* dout = randn(n);
        double *dq = (double*)malloc(sizeof(double) * n), *dk = (double*)malloc(sizeof(double) * n),
               *dv = (double*)malloc(sizeof(double) * n);
        CHECK(oracle_attn_bwd_f64(q, k, v, dout, dq, dk, dv, B, H, N, d, scale, 1, mask) == 0);
        for (long i = 0; i < n; ++i) CHECK(isfinite(dq[i]) && isfinite(dk[i]) && isfinite(dv[i]));
        for (long i = H * N * d; i < n; ++i) CHECK(dq[i] == 0.0 && dk[i] == 0.0 && dv[i] == 0.0);
        CHECK(oracle_attn_bwd_f64(q, k, v, dout, NULL, dk, dv, B, H, N, d, scale, 1, mask) == -1);
        free(dout);
        free(dq);
        free(dk);
        free(dv);
    }

    /* score-level API: empty row, and the blocked fold at every width */
    {
        double s[7], vals[7 * 3], out[3], l0, out2[3], l2;
        for (int j = 0; j < 7; ++j) s[j] = 3.0 * uniform();
        for (int j = 0; j < 21; ++j) vals[j] = uniform();
        CHECK(oracle_row_softmax_f64(s, vals, 0, 3, out, &l0) == 0);
        CHECK(out[0] == 0.0 && isinf(l0));
        CHECK(oracle_row_softmax_f64(s, vals, 7, 3, out, &l0) == 0);
        for (long w = 1; w <= 8; ++w)
            for (int order = 0; order < 2; ++order) {
                CHECK(oracle_row_blocked_f64(s, vals, NULL, 7, 3, w, order, 1, out2, &l2) == 0);
                CHECK(maxdiff(out, out2, 3) < 1e-15 && fabs(l2 - l0) < 1e-15);
            }
        unsigned char none[7] = {0};
        CHECK(oracle_row_blocked_f64(s, vals, none, 7, 3, 3, 0, 1, out2, &l2) == 0);
        CHECK(out2[0] == 0.0 && isinf(l2));
        CHECK(oracle_row_blocked_f64(s, vals, NULL, 7, 3, 0, 0, 1, out2, &l2) == -1);
    }

    /* precision model: rounding of special values, and rounding switched off */
    CHECK(emu_round(1.0 + ldexp(1.0, -8), 8, -126, 127) == 1.0);                       /* tie to even */
    CHECK(emu_round(1.0 + 3 * ldexp(1.0, -8), 8, -126, 127) == 1.0 + ldexp(1.0, -6));  /* tie to even */
    CHECK(isinf(emu_round(1e39, 8, -126, 127)));
    CHECK(emu_round(ldexp(1.0, -133), 8, -126, 127) == ldexp(1.0, -133));              /* smallest subnormal */
    CHECK(emu_round(ldexp(1.0, -135), 8, -126, 127) == 0.0);
    CHECK(emu_round(0.1, 0, 0, 0) == 0.1);
    {
        const emu_fmt off = {0, 0, 0}, bf = {8, -126, 127};
        emu_cfg cfg = {off, off, off, off, 5, 0, 0};
        long r5[4] = {0, 17, 36, 100};
        double e1[4 * 16], e2[4 * 16], ref[4 * 16], lref[4];
        CHECK(oracle_attn_rows_f64(q, k, v, B, H, N, d, scale, 1, NULL, r5, 4, ref, lref) == 0);
        for (int kv = 0; kv < 2; ++kv) {
            cfg.kv_outer = kv;
            CHECK(emu_flash_rows(q, k, v, B, H, N, d, scale, 1, &cfg, r5, 4, e1) == 0);
            CHECK(maxdiff(e1, ref, 4 * d) < 1e-13);
        }
        CHECK(emu_baseline_rows(q, k, v, B, H, N, d, scale, 1, &off, &off, &off, r5, 4, e2) == 0);
        CHECK(maxdiff(e2, ref, 4 * d) < 1e-13);
        cfg.pfmt = bf;
        cfg.out = bf;
        cfg.order = 1;
        CHECK(emu_flash_rows(q, k, v, B, H, N, d, scale, 1, &cfg, r5, 4, e1) == 0);
        CHECK(maxdiff(e1, ref, 4 * d) < 2e-2);
        CHECK(emu_baseline_rows(q, k, v, B, H, N, d, scale, 1, &off, &bf, &bf, r5, 4, e2) == 0);
        CHECK(maxdiff(e2, ref, 4 * d) < 2e-2);
        cfg.bc = 0;
        CHECK(emu_flash_rows(q, k, v, B, H, N, d, scale, 1, &cfg, r5, 4, e1) == -1);
    }

    /* empty and invalid sizes touch nothing */
    CHECK(oracle_attn_f64(NULL, NULL, NULL, o, NULL, 0, 4, 8, 16, scale, 0, NULL) == 0);
    CHECK(oracle_attn_f64(q, k, v, o, lse, -1, H, N, d, scale, 0, NULL) == -1);
    CHECK(oracle_attn_blocked_f64(NULL, NULL, NULL, o, NULL, B, H, 0, d, scale, 0, NULL, 4, 0) == 0);
    CHECK(oracle_attn_blocked_kvouter_f64(NULL, NULL, NULL, o, NULL, B, 0, N, d, scale, 0, NULL, 4, 0) == 0);

    free(q);
    free(k);
    free(v);
    free(o);
    free(lse);
    free(o2);
    free(lse2);
    if (failures) {
        fprintf(stderr, "oracle_san: %d check(s) failed\n", failures);
        return 1;
    }
    printf("oracle_san: all oracle checks passed\n");
    return 0;
}
