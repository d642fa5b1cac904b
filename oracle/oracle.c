/*
 * oracle.c -- plain, slow, fp64 CPU reference for exact attention.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the oracle that the GPU kernels are
 * checked against.  Only the test suite, the smoke check and the benchmark's
 * CPU-baseline leg may load it.  It shares no code, header, table or helper
 * with the GPU library, and the GPU library never calls it.
 *
 * What it computes (all in double precision, straight from the definitions):
 *
 *   Forward -- "standard attention" as the blog post "Gemini 3 Flash的注意力
 *   内核重写：算子融合如何实现亚毫秒级推理" (hotdry blog) lays it out in its
 *   section on the memory-bandwidth bottleneck of traditional attention: three
 *   passes per query row,
 *       pass 1  S_ij = scale * <q_i, k_j>               (causal: S_ij = -inf for j > pos_i)
 *       pass 2  P_ij = exp(S_ij - m_i) / l_i,  m_i = max_j S_ij,  l_i = sum_j exp(S_ij - m_i)
 *               (max-shifted softmax, as in the stable_softmax example of the
 *               snabindia page, section 2.2)
 *       pass 3  O_i  = sum_j P_ij v_j
 *   plus lse_i = m_i + ln l_i (natural log of the scaled logits), the single
 *   per-row statistic the backward recomputation needs (the blog's section 4
 *   keeps the per-row maximum and normaliser; m + ln l carries both).
 *   A row with no visible key has O_i = 0 and lse_i = -inf.
 *
 *   Online validator -- the blog's section 3 ("在线softmax算法"): m = -inf,
 *   l = 0; for every block of keys take the block maximum, raise the running
 *   maximum, rescale the running sum AND the partial output when the maximum
 *   grew, add the block's exponentials to the sum and their weighted values to
 *   the partial output; finally O = acc / l.  (The page's snippet rescales only
 *   the sum; its prose says the partial output is updated too, and exactness
 *   needs both.)  Used only to check that the block-wise recurrence equals the
 *   three-pass definition.
 *
 *   Backward -- the gradient of O = softmax(scale * Q K^T [+ mask]) V with
 *   respect to Q, K, V by ordinary matrix calculus (the pages give only the
 *   recomputation idea, blog section 4, and a softmax vector-Jacobian product
 *   whose printed form on the snabindia page, section 3.2, is garbled):
 *       dV = P^T dO
 *       dP = dO V^T
 *       D_i = sum_j P_ij dP_ij
 *       dS = P o (dP - D)          (o = elementwise product)
 *       dQ = scale * dS K
 *       dK = scale * dS^T Q
 *
 * Masks: causal, an optional sliding window and an optional block mask, with
 * query rows placed at key positions qpos (see visible()); rectangular
 * n_q != n_k shapes align the rows to the end of the key sequence.  Variable-length batches are handled
 * by the Python wrapper, one sequence at a time.
 *
 * Layout: every array is a batch of G independent heads, row-major
 * [G, rows, d] (lse: [G, rows]).  Rows are processed one at a time, so the
 * N x N score matrix is never held in memory; OpenMP spreads rows over cores.
 * Summation order is plain index order.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

static double dot(const double* a, const double* b, int64_t d) {
    double s = 0.0;
    for (int64_t c = 0; c < d; ++c) s += a[c] * b[c];
    return s;
}

/*
 * Which keys a query row sees.  The row sits at key position pos (for equal
 * query and key lengths pos is the row index; for n_q != n_k the rows are
 * aligned to the end of the key sequence, pos = i + n_k - n_q).  Key j is
 * visible iff
 *     (causal: j <= pos)                    -- the causal call of the snabindia
 *                                              page's chapter 1 skips the upper triangle
 *     and (wl < 0 or j >= pos - wl)         -- sliding window to the left
 *     and (wr < 0 or j <= pos + wr)         -- sliding window to the right
 * (a local window of the kind the yunthe article's hybrid local/global block
 * uses).  wl = wr = -1 means no window.  With a block mask (the all-zero-block
 * skipping of the snabindia page's chapter 1 and section 3.1, here as an
 * explicit mask), head g additionally needs
 *     bm[g][pos / bq][j / bk] != 0
 * -- the (query block, key block) pair takes part; bm is [G, nqb, nkb] bytes,
 * nqb * bq >= largest position + 1, nkb * bk >= n_k.  bm = NULL: no block mask.
 */
typedef struct {
    int causal;
    int64_t wl, wr;
    const uint8_t* bm;
    int64_t bq, bk, nqb, nkb;
} mask_t;

static int visible(mask_t mk, int64_t g, int64_t j, int64_t pos) {
    if (mk.causal && j > pos) return 0;
    if (mk.wl >= 0 && j < pos - mk.wl) return 0;
    if (mk.wr >= 0 && j > pos + mk.wr) return 0;
    if (mk.bm && !mk.bm[(g * mk.nqb + pos / mk.bq) * mk.nkb + j / mk.bk]) return 0;
    return 1;
}

/*
 * Forward, three passes per query row.
 *   q: [G, nq, d]   k, v: [G, nk, d]   qpos: [nq] sequence position of each query row
 *   causal, wl, wr, bm, bq, bk, nqb, nkb: the mask (see visible())
 *   o: [G, nq, d]   lse: [G, nq]
 * Returns 0, or -1 if a work buffer cannot be allocated.
 */
int oracle_attn_fwd(int64_t G, int64_t nq, int64_t nk, int64_t d,
                    const double* q, const double* k, const double* v,
                    const int64_t* qpos, int causal, int64_t wl, int64_t wr,
                    const uint8_t* bm, int64_t bq, int64_t bk, int64_t nqb, int64_t nkb, double scale,
                    double* o, double* lse) {
    const mask_t mk = {causal, wl, wr, bm, bq, bk, nqb, nkb};
    int failed = 0;
#pragma omp parallel
    {
        double* s = (double*)malloc(sizeof(double) * (size_t)(nk > 0 ? nk : 1));
        if (!s) {
#pragma omp atomic write
            failed = 1;
        }
#pragma omp for schedule(dynamic, 4)
        for (int64_t r = 0; r < G * nq; ++r) {
            if (!s) continue;
            int64_t g = r / nq, i = r % nq;
            const double* qi = q + (g * nq + i) * d;
            const double* kg = k + g * nk * d;
            const double* vg = v + g * nk * d;
            double* oi = o + (g * nq + i) * d;
            /* pass 1: scores */
            for (int64_t j = 0; j < nk; ++j)
                s[j] = visible(mk, g, j, qpos[i]) ? scale * dot(qi, kg + j * d, d) : -INFINITY;
            /* pass 2: max-shifted softmax */
            double m = -INFINITY;
            for (int64_t j = 0; j < nk; ++j) if (s[j] > m) m = s[j];
            for (int64_t c = 0; c < d; ++c) oi[c] = 0.0;
            if (m == -INFINITY) { /* no visible key */
                lse[g * nq + i] = -INFINITY;
                continue;
            }
            double l = 0.0;
            for (int64_t j = 0; j < nk; ++j) {
                s[j] = (s[j] == -INFINITY) ? 0.0 : exp(s[j] - m);
                l += s[j];
            }
            for (int64_t j = 0; j < nk; ++j) s[j] /= l;
            /* pass 3: weighted sum of values */
            for (int64_t j = 0; j < nk; ++j) {
                if (s[j] == 0.0) continue;
                const double* vj = vg + j * d;
                for (int64_t c = 0; c < d; ++c) oi[c] += s[j] * vj[c];
            }
            lse[g * nq + i] = m + log(l);
        }
        free(s);
    }
    return failed ? -1 : 0;
}

/*
 * Online (block-wise) forward: the running-max recurrence, keys visited in
 * blocks of `block` keys.  Same arguments and outputs as oracle_attn_fwd.
 */
int oracle_attn_fwd_online(int64_t G, int64_t nq, int64_t nk, int64_t d,
                           const double* q, const double* k, const double* v,
                           const int64_t* qpos, int causal, int64_t wl, int64_t wr,
                           const uint8_t* bm, int64_t bq, int64_t bk, int64_t nqb, int64_t nkb, double scale,
                           int64_t block, double* o, double* lse) {
    const mask_t mk = {causal, wl, wr, bm, bq, bk, nqb, nkb};
    if (block < 1) return -2;
    int failed = 0;
#pragma omp parallel
    {
        double* s = (double*)malloc(sizeof(double) * (size_t)block);
        double* acc = (double*)malloc(sizeof(double) * (size_t)(d > 0 ? d : 1));
        if (!s || !acc) {
#pragma omp atomic write
            failed = 1;
        }
#pragma omp for schedule(dynamic, 4)
        for (int64_t r = 0; r < G * nq; ++r) {
            if (!s || !acc) continue;
            int64_t g = r / nq, i = r % nq;
            const double* qi = q + (g * nq + i) * d;
            const double* kg = k + g * nk * d;
            const double* vg = v + g * nk * d;
            double m = -INFINITY, l = 0.0;
            for (int64_t c = 0; c < d; ++c) acc[c] = 0.0;
            for (int64_t j0 = 0; j0 < nk; j0 += block) {
                int64_t nb = (nk - j0 < block) ? nk - j0 : block;
                /* block scores and block maximum */
                double m_local = -INFINITY;
                for (int64_t t = 0; t < nb; ++t) {
                    int64_t j = j0 + t;
                    s[t] = visible(mk, g, j, qpos[i]) ? scale * dot(qi, kg + j * d, d) : -INFINITY;
                    if (s[t] > m_local) m_local = s[t];
                }
                if (m_local == -INFINITY) continue; /* nothing visible in this block */
                double m_new = m_local > m ? m_local : m;
                if (m_new > m) { /* the maximum grew: rescale sum and partial output */
                    double alpha = exp(m - m_new); /* exp(-inf) = 0 on the first block */
                    l *= alpha;
                    for (int64_t c = 0; c < d; ++c) acc[c] *= alpha;
                    m = m_new;
                }
                for (int64_t t = 0; t < nb; ++t) {
                    if (s[t] == -INFINITY) continue;
                    double p = exp(s[t] - m);
                    l += p;
                    const double* vj = vg + (j0 + t) * d;
                    for (int64_t c = 0; c < d; ++c) acc[c] += p * vj[c];
                }
            }
            double* oi = o + (g * nq + i) * d;
            if (m == -INFINITY) {
                for (int64_t c = 0; c < d; ++c) oi[c] = 0.0;
                lse[g * nq + i] = -INFINITY;
            } else {
                for (int64_t c = 0; c < d; ++c) oi[c] = acc[c] / l;
                lse[g * nq + i] = m + log(l);
            }
        }
        free(s);
        free(acc);
    }
    return failed ? -1 : 0;
}

/*
 * Backward.  q, dout: [G, nq, d]; k, v: [G, nk, d]; qpos: [nq] key position
 * of each query row (see visible()).  Outputs only the requested rows:
 *   dq: [G, nrows, d] for query rows rows[0..nrows)   (rows == NULL: all nq rows)
 *   dk, dv: [G, nkeys, d] for key rows keys[0..nkeys) (keys == NULL: all nk keys)
 * Row statistics m_i, l_i and D_i are computed for every query row that
 * contributes (all rows when any dk/dv is requested), then
 *   dq_i = scale * sum_j P_ij (dP_ij - D_i) k_j
 *   dv_j = sum_i P_ij dO_i
 *   dk_j = scale * sum_i P_ij (dP_ij - D_i) q_i
 * with P_ij = exp(S_ij - m_i) / l_i over visible keys (0 elsewhere) and
 * dP_ij = <dO_i, v_j>.  A row that sees no key has P = 0 and contributes
 * nothing.  Returns 0, -1 on allocation failure.
 */
int oracle_attn_bwd(int64_t G, int64_t nq, int64_t nk, int64_t d,
                    const double* q, const double* k, const double* v, const double* dout,
                    const int64_t* qpos, int causal, int64_t wl, int64_t wr,
                    const uint8_t* bm, int64_t bq, int64_t bk, int64_t nqb, int64_t nkb, double scale,
                    const int64_t* rows, int64_t nrows, double* dq,
                    const int64_t* keys, int64_t nkeys, double* dk, double* dv) {
    const mask_t mk = {causal, wl, wr, bm, bq, bk, nqb, nkb};
    if (rows == NULL) nrows = nq;
    if (keys == NULL) nkeys = nk;
    /* Which query rows need statistics: all of them if any key gradient is asked for. */
    int need_all = nkeys > 0;
    int64_t nstat = need_all ? nq : nrows;
    size_t ns = (size_t)(G * nq > 0 ? G * nq : 1);
    double* m = (double*)malloc(sizeof(double) * ns);
    double* l = (double*)malloc(sizeof(double) * ns);
    double* D = (double*)malloc(sizeof(double) * ns);
    if (!m || !l || !D) { free(m); free(l); free(D); return -1; }
    int failed = 0;

    /* Phase 1: per query row, the softmax statistics and D_i = sum_j P_ij dP_ij. */
#pragma omp parallel
    {
        double* s = (double*)malloc(sizeof(double) * (size_t)(nk > 0 ? nk : 1));
        double* dp = (double*)malloc(sizeof(double) * (size_t)(nk > 0 ? nk : 1));
        if (!s || !dp) {
#pragma omp atomic write
            failed = 1;
        }
#pragma omp for schedule(dynamic, 4)
        for (int64_t r = 0; r < G * nstat; ++r) {
            if (!s || !dp) continue;
            int64_t g = r / nstat, ii = r % nstat;
            int64_t i = (need_all || rows == NULL) ? ii : rows[ii];
            const double* qi = q + (g * nq + i) * d;
            const double* doi = dout + (g * nq + i) * d;
            const double* kg = k + g * nk * d;
            const double* vg = v + g * nk * d;
            double mi = -INFINITY;
            for (int64_t j = 0; j < nk; ++j) {
                s[j] = visible(mk, g, j, qpos[i]) ? scale * dot(qi, kg + j * d, d) : -INFINITY;
                if (s[j] > mi) mi = s[j];
            }
            double li = 0.0, Di = 0.0;
            if (mi != -INFINITY) {
                for (int64_t j = 0; j < nk; ++j) {
                    s[j] = (s[j] == -INFINITY) ? 0.0 : exp(s[j] - mi);
                    li += s[j];
                }
                for (int64_t j = 0; j < nk; ++j) {
                    s[j] /= li; /* P_ij */
                    dp[j] = (s[j] == 0.0) ? 0.0 : dot(doi, vg + j * d, d);
                    Di += s[j] * dp[j];
                }
            }
            m[g * nq + i] = mi;
            l[g * nq + i] = li;
            D[g * nq + i] = Di;
        }
        free(s);
        free(dp);
    }
    if (failed) { free(m); free(l); free(D); return -1; }

    /* Phase 2: dq for the requested query rows. */
#pragma omp parallel for schedule(dynamic, 4)
    for (int64_t r = 0; r < G * nrows; ++r) {
        int64_t g = r / nrows, ii = r % nrows;
        int64_t i = rows ? rows[ii] : ii;
        const double* qi = q + (g * nq + i) * d;
        const double* doi = dout + (g * nq + i) * d;
        const double* kg = k + g * nk * d;
        const double* vg = v + g * nk * d;
        double* dqi = dq + (g * nrows + ii) * d;
        for (int64_t c = 0; c < d; ++c) dqi[c] = 0.0;
        if (m[g * nq + i] == -INFINITY) continue; /* the row sees no key */
        for (int64_t j = 0; j < nk; ++j) {
            if (!visible(mk, g, j, qpos[i])) continue;
            double p = exp(scale * dot(qi, kg + j * d, d) - m[g * nq + i]) / l[g * nq + i];
            double ds = p * (dot(doi, vg + j * d, d) - D[g * nq + i]);
            for (int64_t c = 0; c < d; ++c) dqi[c] += scale * ds * kg[j * d + c];
        }
    }

    /* Phase 3: dk, dv for the requested key rows. */
#pragma omp parallel for schedule(dynamic, 4)
    for (int64_t r = 0; r < G * nkeys; ++r) {
        int64_t g = r / nkeys, jj = r % nkeys;
        int64_t j = keys ? keys[jj] : jj;
        const double* kj = k + (g * nk + j) * d;
        const double* vj = v + (g * nk + j) * d;
        double* dkj = dk + (g * nkeys + jj) * d;
        double* dvj = dv + (g * nkeys + jj) * d;
        for (int64_t c = 0; c < d; ++c) { dkj[c] = 0.0; dvj[c] = 0.0; }
        for (int64_t i = 0; i < nq; ++i) {
            if (!visible(mk, g, j, qpos[i])) continue;
            const double* qi = q + (g * nq + i) * d;
            const double* doi = dout + (g * nq + i) * d;
            double p = exp(scale * dot(qi, kj, d) - m[g * nq + i]) / l[g * nq + i];
            double ds = p * (dot(doi, vj, d) - D[g * nq + i]);
            for (int64_t c = 0; c < d; ++c) {
                dvj[c] += p * doi[c];
                dkj[c] += scale * ds * qi[c];
            }
        }
    }
    free(m);
    free(l);
    free(D);
    return 0;
}

/* Number of OpenMP threads a parallel region of the oracle uses. */
int oracle_num_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
