/*
 * lisa_oracle.c -- plain fp64 CPU oracle of the LISA layer forward pass.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may call, link or
 * load this file or the library built from it; only the tests, the smoke
 * check and the CPU-baseline leg of the benchmark use it.  It shares no code
 * with the HIP implementation.
 *
 * What it computes (LISA: Linear-Indexed Sparse Attention, arXiv 2607.19358):
 *   - arxivdaily page for 2607.19358, English abstract: two branches run in
 *     parallel inside the layer -- a linear-attention module (long-range
 *     memory, O(n)) and a Lightning Indexer that picks the top-M tokens of
 *     the full context for a sparse self-attention -- and a gate fuses them.
 *   - gptget.net analysis of 2607.19358, method-details section: the linear
 *     branch uses the identity feature map and a state matrix S_t updated in
 *     O(1) per step; the indexer scores tokens with query/key projections and
 *     a ReLU'd dot product; a learned gate parameter g mixes the branches.
 *   - same page, experiment-design section: M = 256.
 * The pages print no formulas; the readings used here (one indexer per KV
 * group with keys shared across indexer heads, per-head weights w, causal
 * candidates 0..t including t, lowest index wins ties, softmax scale
 * 1/sqrt(d), S_t including the current token, sigmoid gate on a logit z,
 * GQA head h -> group h*Hkv/Hq) are listed with their reasons in the design
 * notes of this repository and in include/lisa.h.
 *
 * Everything is fp64, sequential in the order the definitions state.  The
 * only parallelism is OpenMP over independent output rows; no step is
 * blocked, chunked, fused or reordered.
 *
 * Layouts (row-major, fp64):
 *   prefill  q [B,n,Hq,d]  k,v [B,n,Hkv,d]  qI [B,n,G,HI,dI]  kI [B,n,G,dI]
 *            w [B,n,G,HI]  z [B,n,Hq]  S0/state_out [B,Hq,d,d] (row = key dim)
 *   decode   q [B,Hq,d]  kc,vc [sumL,Hkv,d]  qI [B,G,HI,dI]  kIc [sumL,G,dI]
 *            w [B,G,HI]  z [B,Hq]  state [B,Hq,d,d]; cu [B+1] row offsets.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* ---- step (1): Lightning Indexer score --------------------------------- */
/* I(s) = sum_j w_j * max(0, qI_j . kI_s)   for s = 0..T-1.
 * qI: [HI][dI] for the query; w: [HI]; key s at kI + s*kstride. */
void oracle_index_scores(int T, int HI, int dI, const double *qI, const double *w,
                         const double *kI, long kstride, double *scores) {
    for (int s = 0; s < T; ++s) {
        const double *ks = kI + (long)s * kstride;
        double total = 0.0;
        for (int j = 0; j < HI; ++j) {
            double dot = 0.0;
            for (int c = 0; c < dI; ++c) dot += qI[j * dI + c] * ks[c];
            double relu = dot > 0.0 ? dot : 0.0;
            total += w[j] * relu;
        }
        scores[s] = total;
    }
}

/* ---- step (2): top-M selection ----------------------------------------- */
typedef struct { double score; int index; } cand_t;

/* Order: higher score first; on equal scores the lower index first.
 * -0.0 and +0.0 compare equal under C's floating-point comparison. */
static int cand_order(const void *a, const void *b) {
    const cand_t *x = (const cand_t *)a, *y = (const cand_t *)b;
    if (x->score > y->score) return -1;
    if (x->score < y->score) return 1;
    return (x->index > y->index) - (x->index < y->index);
}

static int int_ascending(const void *a, const void *b) {
    int x = *(const int *)a, y = *(const int *)b;
    return (x > y) - (x < y);
}

/* Writes the min(M, T) selected indices in ascending order, then -1 up to M.
 * Returns the number selected. */
int oracle_topm(int T, const double *scores, int M, int *idx_out) {
    int m = T < M ? T : M;
    if (T > 0) {
        cand_t *c = (cand_t *)malloc(sizeof(cand_t) * (size_t)T);
        for (int s = 0; s < T; ++s) { c[s].score = scores[s]; c[s].index = s; }
        qsort(c, (size_t)T, sizeof(cand_t), cand_order);
        for (int i = 0; i < m; ++i) idx_out[i] = c[i].index;
        free(c);
        qsort(idx_out, (size_t)m, sizeof(int), int_ascending);
    }
    for (int i = m; i < M; ++i) idx_out[i] = -1;
    return m;
}

/* ---- step (3): softmax attention over the selected rows ---------------- */
/* o = sum_{s in set} softmax_s(scale * q . k_s) * v_s ; set entries < 0 are
 * padding.  Key s at krow(s) = kv + s*kvstride, same for v. */
static void sparse_one_head(int d, double scale, const double *q, const double *kbase,
                            const double *vbase, long kvstride, const int *set, int M,
                            double *o) {
    double *a = (double *)malloc(sizeof(double) * (size_t)(M > 0 ? M : 1));
    double amax = -INFINITY;
    int cnt = 0;
    for (int i = 0; i < M; ++i) {
        if (set[i] < 0) continue;
        const double *ks = kbase + (long)set[i] * kvstride;
        double dot = 0.0;
        for (int c = 0; c < d; ++c) dot += q[c] * ks[c];
        a[i] = scale * dot;
        if (a[i] > amax) amax = a[i];
        ++cnt;
    }
    for (int c = 0; c < d; ++c) o[c] = 0.0;
    if (cnt == 0) { free(a); return; }
    double denom = 0.0;
    for (int i = 0; i < M; ++i) {
        if (set[i] < 0) continue;
        a[i] = exp(a[i] - amax);
        denom += a[i];
    }
    for (int i = 0; i < M; ++i) {
        if (set[i] < 0) continue;
        const double *vs = vbase + (long)set[i] * kvstride;
        double p = a[i] / denom;
        for (int c = 0; c < d; ++c) o[c] += p * vs[c];
    }
    free(a);
}

/* ---- step (4) gate ------------------------------------------------------ */
/* g = 1/(1+exp(-z)); o = g*o_sparse + (1-g)*o_linear. */
static void gate_mix(int d, double z, const double *osp, const double *olin, double *o) {
    double g = 1.0 / (1.0 + exp(-z));
    for (int c = 0; c < d; ++c) o[c] = g * osp[c] + (1.0 - g) * olin[c];
}

static int group_of(int h, int Hq, int Hkv) { return (int)(((long)h * Hkv) / Hq); }

static void set_threads(int nthreads) {
#ifdef _OPENMP
    if (nthreads > 0) omp_set_num_threads(nthreads);
#else
    (void)nthreads;
#endif
}

/*
 * Sparse branch plus gate for a list of query units, given the index sets.
 * Unit u: query vectors q[u][Hq][d], gate logits z[u][Hq], linear-branch
 * output olin[u][Hq][d], index sets idx[u][G][M] (token positions relative to
 * the unit's first key row), K/V rows of the unit's sequence start at
 * row0[u] in kv[rows][Hkv][d].  Writes out[u][Hq][d] and, if non-null,
 * osp[u][Hq][d].
 */
int oracle_sparse_given_sets(int U, int Hq, int Hkv, int d, int M, double scale,
                             const double *q, const double *kv_k, const double *kv_v,
                             const long *row0, const int *idx, const double *z,
                             const double *olin, double *out, double *osp, int nthreads) {
    if (scale <= 0.0) scale = 1.0 / sqrt((double)d);
    set_threads(nthreads);
    long kvstride = (long)Hkv * d;
#pragma omp parallel for schedule(dynamic, 4)
    for (long uh = 0; uh < (long)U * Hq; ++uh) {
        long u = uh / Hq;
        int h = (int)(uh % Hq);
        int g = group_of(h, Hq, Hkv);
        double *tmp = (double *)malloc(sizeof(double) * (size_t)d);
        const double *kb = kv_k + row0[u] * kvstride + (long)g * d;
        const double *vb = kv_v + row0[u] * kvstride + (long)g * d;
        sparse_one_head(d, scale, q + uh * d, kb, vb, kvstride, idx + (u * Hkv + g) * (long)M,
                        M, tmp);
        if (osp) memcpy(osp + uh * d, tmp, sizeof(double) * (size_t)d);
        gate_mix(d, z[uh], tmp, olin + uh * d, out + uh * d);
        free(tmp);
    }
    return 0;
}

/*
 * Full prefill of one layer.  rows/nrows select which query positions t are
 * evaluated (rows == NULL: all n, in order); per-row outputs are compact:
 * out/osp/olin [B][nrows][Hq][d], idx [B][nrows][G][M].  state_out gets S_{n-1}
 * (the state after the last token) for every head.  S0 may be NULL (zero).
 */
int oracle_prefill(int B, int n, int Hq, int Hkv, int d, int HI, int dI, int M, double scale,
                   const double *q, const double *k, const double *v, const double *qI,
                   const double *kI, const double *w, const double *z, const double *S0,
                   const int *rows, int nrows, double *out, double *state_out, int *idx,
                   double *osp, double *olin, int nthreads) {
    if (scale <= 0.0) scale = 1.0 / sqrt((double)d);
    if (!rows) nrows = n;
    set_threads(nthreads);
    const int G = Hkv;
    double *lin = (double *)malloc(sizeof(double) * (size_t)B * nrows * Hq * d + 1);
    double *sp = (double *)malloc(sizeof(double) * (size_t)B * nrows * Hq * d + 1);

    /* Linear branch, recurrent form, one head at a time:
     * S_t = S_{t-1} + k_t v_t^T (S_{-1} = S0), o_lin[t] = q_t^T S_t. */
#pragma omp parallel for schedule(dynamic, 1)
    for (long bh = 0; bh < (long)B * Hq; ++bh) {
        int b = (int)(bh / Hq), h = (int)(bh % Hq), g = group_of(h, Hq, Hkv);
        double *S = (double *)malloc(sizeof(double) * (size_t)d * d);
        if (S0) memcpy(S, S0 + bh * d * d, sizeof(double) * (size_t)d * d);
        else memset(S, 0, sizeof(double) * (size_t)d * d);
        int next = 0; /* rows[] is ascending; next = first row not yet written */
        for (int t = 0; t < n; ++t) {
            const double *kt = k + (((long)b * n + t) * Hkv + g) * d;
            const double *vt = v + (((long)b * n + t) * Hkv + g) * d;
            for (int i = 0; i < d; ++i)
                for (int j = 0; j < d; ++j) S[i * d + j] += kt[i] * vt[j];
            const double *qt = q + (((long)b * n + t) * Hq + h) * d;
            for (;;) {
                int r;
                if (!rows) r = t;
                else if (next < nrows && rows[next] == t) r = next++;
                else break;
                double *o = lin + (((long)b * nrows + r) * Hq + h) * d;
                for (int j = 0; j < d; ++j) {
                    double acc = 0.0;
                    for (int i = 0; i < d; ++i) acc += qt[i] * S[i * d + j];
                    o[j] = acc;
                }
                if (!rows) break;
            }
        }
        if (state_out) memcpy(state_out + bh * d * d, S, sizeof(double) * (size_t)d * d);
        free(S);
    }

    /* Indexer, selection and sparse attention for each (b, row, group). */
#pragma omp parallel for schedule(dynamic, 1)
    for (long brg = 0; brg < (long)B * nrows * G; ++brg) {
        int g = (int)(brg % G);
        long br = brg / G;
        int b = (int)(br / nrows), r = (int)(br % nrows);
        int t = rows ? rows[r] : r;
        double *sc = (double *)malloc(sizeof(double) * (size_t)(t + 1));
        const double *qIt = qI + ((((long)b * n + t) * G + g) * HI) * dI;
        const double *wt = w + (((long)b * n + t) * G + g) * HI;
        const double *kIb = kI + ((long)b * n * G + g) * dI;
        oracle_index_scores(t + 1, HI, dI, qIt, wt, kIb, (long)G * dI, sc);
        int *set = idx + (((long)b * nrows + r) * G + g) * M;
        oracle_topm(t + 1, sc, M, set);
        free(sc);
        const double *kb = k + ((long)b * n * Hkv + g) * d;
        const double *vb = v + ((long)b * n * Hkv + g) * d;
        for (int h = 0; h < Hq; ++h) {
            if (group_of(h, Hq, Hkv) != g) continue;
            const double *qt = q + (((long)b * n + t) * Hq + h) * d;
            sparse_one_head(d, scale, qt, kb, vb, (long)Hkv * d, set, M,
                            sp + (((long)b * nrows + r) * Hq + h) * d);
        }
    }

    /* Gate. */
    for (long brh = 0; brh < (long)B * nrows * Hq; ++brh) {
        long br = brh / Hq;
        int h = (int)(brh % Hq);
        int b = (int)(br / nrows), r = (int)(br % nrows);
        int t = rows ? rows[r] : r;
        double zz = z[((long)b * n + t) * Hq + h];
        gate_mix(d, zz, sp + brh * d, lin + brh * d, out + brh * d);
    }
    if (osp) memcpy(osp, sp, sizeof(double) * (size_t)B * nrows * Hq * d);
    if (olin) memcpy(olin, lin, sizeof(double) * (size_t)B * nrows * Hq * d);
    free(lin);
    free(sp);
    return 0;
}

/*
 * One decode step.  Sequence b owns cache rows [cu[b], cu[b+1]); its last row
 * is the new token (already appended).  With t = L_b - 1:
 *   S_t = S_{t-1} + k_t v_t^T (state updated in place into state_out),
 *   o_lin = q^T S_t, the indexer scores rows 0..t, top-M, sparse attention,
 *   gate.  out [B][Hq][d], idx [B][G][M].
 */
int oracle_decode(int B, const long *cu, int Hq, int Hkv, int d, int HI, int dI, int M,
                  double scale, const double *q, const double *kc, const double *vc,
                  const double *qI, const double *kIc, const double *w, const double *z,
                  const double *state_in, double *out, double *state_out, int *idx,
                  double *osp, double *olin, int nthreads) {
    if (scale <= 0.0) scale = 1.0 / sqrt((double)d);
    set_threads(nthreads);
    const int G = Hkv;
    double *lin = (double *)malloc(sizeof(double) * (size_t)B * Hq * d + 1);
    double *sp = (double *)malloc(sizeof(double) * (size_t)B * Hq * d + 1);

#pragma omp parallel for schedule(dynamic, 1)
    for (long bh = 0; bh < (long)B * Hq; ++bh) {
        int b = (int)(bh / Hq), h = (int)(bh % Hq), g = group_of(h, Hq, Hkv);
        long t_row = cu[b + 1] - 1;
        const double *kt = kc + (t_row * Hkv + g) * d;
        const double *vt = vc + (t_row * Hkv + g) * d;
        const double *Sin = state_in + bh * d * d;
        double *S = state_out + bh * d * d;
        for (int i = 0; i < d; ++i)
            for (int j = 0; j < d; ++j) S[i * d + j] = Sin[i * d + j] + kt[i] * vt[j];
        const double *qb = q + bh * d;
        for (int j = 0; j < d; ++j) {
            double acc = 0.0;
            for (int i = 0; i < d; ++i) acc += qb[i] * S[i * d + j];
            lin[bh * d + j] = acc;
        }
    }

#pragma omp parallel for schedule(dynamic, 1)
    for (long bg = 0; bg < (long)B * G; ++bg) {
        int b = (int)(bg / G), g = (int)(bg % G);
        long L = cu[b + 1] - cu[b];
        double *sc = (double *)malloc(sizeof(double) * (size_t)(L > 0 ? L : 1));
        oracle_index_scores((int)L, HI, dI, qI + bg * HI * dI, w + bg * HI,
                            kIc + (cu[b] * G + g) * dI, (long)G * dI, sc);
        int *set = idx + bg * M;
        oracle_topm((int)L, sc, M, set);
        free(sc);
        const double *kb = kc + (cu[b] * Hkv + g) * d;
        const double *vb = vc + (cu[b] * Hkv + g) * d;
        for (int h = 0; h < Hq; ++h) {
            if (group_of(h, Hq, Hkv) != g) continue;
            sparse_one_head(d, scale, q + ((long)b * Hq + h) * d, kb, vb, (long)Hkv * d, set,
                            M, sp + ((long)b * Hq + h) * d);
        }
    }

    for (long bh = 0; bh < (long)B * Hq; ++bh)
        gate_mix(d, z[bh], sp + bh * d, lin + bh * d, out + bh * d);
    if (osp) memcpy(osp, sp, sizeof(double) * (size_t)B * Hq * d);
    if (olin) memcpy(olin, lin, sizeof(double) * (size_t)B * Hq * d);
    free(lin);
    free(sp);
    return 0;
}
