/*
 * Host driver for the fp64 oracle built with AddressSanitizer and
 * UndefinedBehaviorSanitizer: runs every oracle entry on small inputs that
 * reach its edge cases (n = 1, M > n, M = 1, ties and signed zeros, negative
 * head weights, a subset of rows, a ragged decode batch with a length-1
 * sequence) and checks the selection invariants.  Values are not compared
 * here (the pins do that); this run is about memory and UB.  A sanitizer
 * report aborts the process; a broken invariant exits 1.
 */
#include <math.h>
#include <stdio.h>
#include <stdlib.h>

void oracle_index_scores(int T, int HI, int dI, const double *qI, const double *w, const double *kI,
                         long kstride, double *scores);
int oracle_topm(int T, const double *scores, int M, int *idx_out);
int oracle_sparse_given_sets(int U, int Hq, int Hkv, int d, int M, double scale, const double *q,
                             const double *kv_k, const double *kv_v, const long *row0, const int *idx,
                             const double *z, const double *olin, double *out, double *osp, int nthreads);
int oracle_prefill(int B, int n, int Hq, int Hkv, int d, int HI, int dI, int M, double scale,
                   const double *q, const double *k, const double *v, const double *qI, const double *kI,
                   const double *w, const double *z, const double *S0, const int *rows, int nrows,
                   double *out, double *state_out, int *idx, double *osp, double *olin, int nthreads);
int oracle_decode(int B, const long *cu, int Hq, int Hkv, int d, int HI, int dI, int M, double scale,
                  const double *q, const double *kc, const double *vc, const double *qI, const double *kIc,
                  const double *w, const double *z, const double *state_in, double *out, double *state_out,
                  int *idx, double *osp, double *olin, int nthreads);

static unsigned long long lcg = 88172645463325252ull;
static double uni(void) { /* xorshift64, uniform in [-1, 1) */
    lcg ^= lcg << 13;
    lcg ^= lcg >> 7;
    lcg ^= lcg << 17;
    return (double)(lcg >> 11) / 4503599627370496.0 - 1.0;
}
static double *vec(long n) {
    double *x = malloc(sizeof(double) * (size_t)(n > 0 ? n : 1));
    for (long i = 0; i < n; ++i) x[i] = uni();
    return x;
}

static int bad = 0;

/* every set: min(M, T) ascending distinct entries in [0, T), then -1 */
static void check_set(const int *set, int T, int M) {
    int m = T < M ? T : M;
    for (int i = 0; i < M; ++i) {
        if (i < m && (set[i] < 0 || set[i] >= T || (i > 0 && set[i] <= set[i - 1]))) bad = 1;
        if (i >= m && set[i] != -1) bad = 1;
    }
}

static void prefill_case(int B, int n, int Hq, int Hkv, int d, int HI, int dI, int M, int signed_w,
                         int with_state, int nrows) {
    int G = Hkv;
    double *q = vec((long)B * n * Hq * d), *k = vec((long)B * n * Hkv * d), *v = vec((long)B * n * Hkv * d);
    double *qI = vec((long)B * n * G * HI * dI), *kI = vec((long)B * n * G * dI), *w = vec((long)B * n * G * HI);
    double *z = vec((long)B * n * Hq), *S0 = with_state ? vec((long)B * Hq * d * d) : NULL;
    for (long i = 0; i < (long)B * n * G * HI; ++i) w[i] = signed_w ? w[i] : fabs(w[i]);
    /* ties: every fifth key repeats the first one; signed zeros in q_idx */
    for (long r = 5; r < (long)B * n * G; r += 5)
        for (int c = 0; c < dI; ++c) kI[r * dI + c] = kI[c];
    for (long i = 0; i < (long)B * n * G * HI * dI; i += 7) qI[i] = (i & 8) ? -0.0 : 0.0;
    int *rows = NULL;
    int R = n;
    if (nrows > 0 && nrows < n) {
        rows = malloc(sizeof(int) * (size_t)nrows);
        for (int i = 0; i < nrows; ++i) rows[i] = (int)((long)i * n / nrows);
        R = nrows;
    }
    long orow = (long)B * R * Hq * d;
    double *out = malloc(sizeof(double) * (size_t)orow), *osp = malloc(sizeof(double) * (size_t)orow);
    double *olin = malloc(sizeof(double) * (size_t)orow), *st = malloc(sizeof(double) * (size_t)B * Hq * d * d);
    int *idx = malloc(sizeof(int) * (size_t)B * R * G * M);
    oracle_prefill(B, n, Hq, Hkv, d, HI, dI, M, 0.0, q, k, v, qI, kI, w, z, S0, rows, rows ? R : 0, out, st, idx,
                   osp, olin, 2);
    for (int b = 0; b < B; ++b)
        for (int r = 0; r < R; ++r)
            for (int g = 0; g < G; ++g) check_set(idx + (((long)b * R + r) * G + g) * M, (rows ? rows[r] : r) + 1, M);
    /* the sparse branch again on the oracle's own sets, unit per (b, row) */
    long U = (long)B * R;
    double *qs = malloc(sizeof(double) * (size_t)orow), *zs = malloc(sizeof(double) * (size_t)U * Hq);
    long *row0 = malloc(sizeof(long) * (size_t)U);
    for (long u = 0; u < U; ++u) {
        long b = u / R, t = rows ? rows[u % R] : u % R;
        row0[u] = b * n;
        for (int i = 0; i < Hq * d; ++i) qs[u * Hq * d + i] = q[(b * n + t) * Hq * d + i];
        for (int h = 0; h < Hq; ++h) zs[u * Hq + h] = z[(b * n + t) * Hq + h];
    }
    double *out2 = malloc(sizeof(double) * (size_t)orow), *osp2 = malloc(sizeof(double) * (size_t)orow);
    oracle_sparse_given_sets((int)U, Hq, Hkv, d, M, 0.0, qs, k, v, row0, idx, zs, olin, out2, osp2, 2);
    free(q); free(k); free(v); free(qI); free(kI); free(w); free(z); free(S0); free(rows);
    free(out); free(osp); free(olin); free(st); free(idx); free(qs); free(zs); free(row0); free(out2); free(osp2);
}

static void decode_case(int B, const long *L, int Hq, int Hkv, int d, int HI, int dI, int M) {
    int G = Hkv;
    long *cu = malloc(sizeof(long) * (size_t)(B + 1));
    cu[0] = 0;
    for (int b = 0; b < B; ++b) cu[b + 1] = cu[b] + L[b];
    long tot = cu[B];
    double *q = vec((long)B * Hq * d), *kc = vec(tot * Hkv * d), *vc = vec(tot * Hkv * d);
    double *qI = vec((long)B * G * HI * dI), *kIc = vec(tot * G * dI), *w = vec((long)B * G * HI);
    double *z = vec((long)B * Hq), *S = vec((long)B * Hq * d * d);
    double *out = malloc(sizeof(double) * (size_t)B * Hq * d), *osp = malloc(sizeof(double) * (size_t)B * Hq * d);
    double *olin = malloc(sizeof(double) * (size_t)B * Hq * d), *st = malloc(sizeof(double) * (size_t)B * Hq * d * d);
    int *idx = malloc(sizeof(int) * (size_t)B * G * M);
    oracle_decode(B, cu, Hq, Hkv, d, HI, dI, M, 0.0, q, kc, vc, qI, kIc, w, z, S, out, st, idx, osp, olin, 2);
    for (int b = 0; b < B; ++b)
        for (int g = 0; g < G; ++g) check_set(idx + ((long)b * G + g) * M, (int)L[b], M);
    free(cu); free(q); free(kc); free(vc); free(qI); free(kIc); free(w); free(z); free(S);
    free(out); free(osp); free(olin); free(st); free(idx);
}

int main(void) {
    prefill_case(1, 1, 2, 1, 8, 2, 4, 4, 0, 0, 0);          /* n = 1 */
    prefill_case(2, 37, 4, 2, 8, 3, 8, 64, 1, 1, 0);        /* M > n, batch of two, state in */
    prefill_case(1, 90, 6, 3, 16, 4, 8, 1, 1, 0, 0);        /* M = 1 */
    prefill_case(1, 120, 4, 2, 8, 2, 8, 12, 1, 1, 17);      /* a subset of rows */
    prefill_case(1, 70, 2, 2, 8, 8, 16, 9, 0, 0, 0);        /* 8 indexer heads, ties */
    {
        double sc[6] = {0.0, -0.0, 1.0, -2.0, 1.0, 0.0};
        int set[8];
        oracle_topm(6, sc, 8, set);
        check_set(set, 6, 8);
        oracle_topm(0, sc, 3, set);
        for (int i = 0; i < 3; ++i) bad |= set[i] != -1;
        double qI[4] = {1, 0, 0, 1}, wI[2] = {-1, 0.5}, kI[4] = {1, 1, -1, 2}, out[2];
        oracle_index_scores(2, 2, 2, qI, wI, kI, 2, out);
    }
    const long L1[4] = {1, 40, 3, 129};
    decode_case(4, L1, 4, 2, 8, 2, 8, 16);                   /* ragged, a length-1 sequence */
    const long L2[2] = {300, 2};
    decode_case(2, L2, 2, 1, 16, 4, 8, 256);                 /* M above every length */
    printf(bad ? "broken invariant\n" : "ok\n");
    return bad;
}
