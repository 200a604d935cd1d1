/*
 * fa_oracle.c -- plain, slow CPU reference for the attention forward pass.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may link, load or
 * call this file; it exists so that tests, the smoke check and the CPU
 * baseline of the benchmark have an independent answer to compare with.  It
 * shares no code, header, table or constant with the GPU library.
 *
 * Sources (cited by page title and section):
 *   [impl] "FlashAttention-2实现与优化：高效注意力机制详解"
 *          §3.1 (PyTorch forward), §3.2 (Triton forward), §4.2-4.3.
 *   [evo]  "FlashAttention技术演进全景图" §2.1 (matmul -> softmax -> matmul),
 *          §2.3 (max-subtracted softmax).
 *   [mem]  "解释FlashAttention的显存优化原理" §一.1 (standard attention).
 *
 * Everything is computed in IEEE double precision, one query row at a time.
 * Inputs arrive as double arrays (bf16 and fp32 values are exact in double).
 * Layout: q [B,H,Nq,D], k and v [B,H,Nk,D], o [B,H,Nq,D], lse [B,H,Nq], all
 * contiguous row-major.  "rows" optionally restricts the computation to a
 * list of flat row ids r = (b*H + h)*Nq + i; then o is [nrows,D] and lse is
 * [nrows], in list order.
 *
 * Readings of the pages that this file adopts:
 *   - the valid key set of row i is { j < Nk : !causal || j <= i } (global
 *     indices from 0, "top-left" alignment), so a causal row never sees a
 *     later key and every row sees at least key 0 when Nk >= 1;
 *   - masked keys are excluded from the softmax (the pages' -1e6 fill gives
 *     the same numbers once a row has one valid key, see fa_oracle_online);
 *   - keys j >= Nk never exist: a ragged last tile is cut at Nk;
 *   - lse uses the natural logarithm: L = m + ln(l).
 *
 * Parity status: pinned (see tests/test_oracle_pins.py).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

enum { ORACLE_OK = 0, ORACLE_EINVAL = 1, ORACLE_ENOMEM = 2 };

/* Number of OpenMP threads a parallel region will use (1 without OpenMP). */
int fa_oracle_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* Sets the OpenMP threads of later parallel regions (no effect without
   OpenMP); returns the previous setting. */
int fa_oracle_set_threads(int n)
{
#ifdef _OPENMP
    const int prev = omp_get_max_threads();
    if (n >= 1)
        omp_set_num_threads(n);
    return prev;
#else
    (void)n;
    return 1;
#endif
}

static int bad_shape(int64_t B, int64_t H, int64_t Nq, int64_t Nk, int64_t D)
{
    return B < 1 || H < 1 || Nq < 1 || Nk < 1 || D < 1;
}

/* Number of keys row i may attend to: all Nk, or keys 0..i when causal. */
static int64_t valid_keys(int64_t i, int64_t Nk, int causal)
{
    if (!causal)
        return Nk;
    return (i + 1 < Nk) ? i + 1 : Nk;
}

/*
 * Two-pass attention, the plain definition ([evo] §2.1, §2.3; [mem] §一.1;
 * output conventions from [impl] §3.1/§3.2):
 *     s_j = scale * <q_i, k_j>               for j in the valid set
 *     m   = max_j s_j
 *     w_j = exp(s_j - m),  l = sum_j w_j
 *     o_i = (sum_j w_j v_j) / l
 *     L_i = m + ln l
 */
int fa_oracle_attention(const double *q, const double *k, const double *v,
                        double *o, double *lse,
                        int64_t B, int64_t H, int64_t Nq, int64_t Nk, int64_t D,
                        double scale, int causal,
                        const int64_t *rows, int64_t nrows)
{
    if (!q || !k || !v || !o || !lse || bad_shape(B, H, Nq, Nk, D))
        return ORACLE_EINVAL;
    const int64_t total = B * H * Nq;
    const int64_t count = rows ? nrows : total;
    if (rows) {
        for (int64_t t = 0; t < nrows; ++t)
            if (rows[t] < 0 || rows[t] >= total)
                return ORACLE_EINVAL;
    }
    int failed = 0;

#pragma omp parallel
    {
        double *w = (double *)malloc((size_t)Nk * sizeof(double));
        if (!w) {
#pragma omp atomic write
            failed = 1;
        }
#pragma omp for schedule(dynamic, 8)
        for (int64_t t = 0; t < count; ++t) {
            if (!w)
                continue;
            const int64_t r = rows ? rows[t] : t;
            const int64_t bh = r / Nq;
            const int64_t i = r % Nq;
            const double *qi = q + r * D;
            const double *kb = k + bh * Nk * D;
            const double *vb = v + bh * Nk * D;
            const int64_t n = valid_keys(i, Nk, causal);

            /* pass 1: scores and their maximum */
            double m = -INFINITY;
            for (int64_t j = 0; j < n; ++j) {
                double dot = 0.0;
                for (int64_t d = 0; d < D; ++d)
                    dot += qi[d] * kb[j * D + d];
                w[j] = scale * dot;
                if (w[j] > m)
                    m = w[j];
            }
            /* pass 2: max-subtracted exponentials and their sum */
            double l = 0.0;
            for (int64_t j = 0; j < n; ++j) {
                w[j] = exp(w[j] - m);
                l += w[j];
            }
            /* weighted sum of values, normalised by l */
            double *oi = o + t * D;
            for (int64_t d = 0; d < D; ++d)
                oi[d] = 0.0;
            for (int64_t j = 0; j < n; ++j)
                for (int64_t d = 0; d < D; ++d)
                    oi[d] += w[j] * vb[j * D + d];
            for (int64_t d = 0; d < D; ++d)
                oi[d] /= l;
            lse[t] = m + log(l);
        }
        free(w);
    }
    return failed ? ORACLE_ENOMEM : ORACLE_OK;
}

/*
 * The tiled online-softmax recurrence of [impl] §3.1 (the running statistics
 * m, l and an unnormalised accumulator, updated once per key tile), in double
 * precision, used only to show that the recurrence reaches the two-pass
 * result.  Query rows are grouped in tiles of bq rows and keys in tiles of bk
 * keys; the last tile of each is cut at Nq / Nk.  Causally hidden keys inside
 * a visited tile get the pages' fill value -1e6 ([impl] §3.1, §4.3); every key
 * tile is visited, as on the pages (no tile skipping).  Per key tile:
 *     m' = max(m, max_j s_j)
 *     p_j = exp(s_j - m')
 *     l  = exp(m - m') * l + sum_j p_j
 *     acc = exp(m - m') * acc + sum_j p_j v_j
 * and at the end o = acc / l, L = m + ln l ([impl] §3.1).
 */
int fa_oracle_online(const double *q, const double *k, const double *v,
                     double *o, double *lse,
                     int64_t B, int64_t H, int64_t Nq, int64_t Nk, int64_t D,
                     double scale, int causal, int64_t bq, int64_t bk)
{
    if (!q || !k || !v || !o || !lse || bad_shape(B, H, Nq, Nk, D) || bq < 1 ||
        bk < 1)
        return ORACLE_EINVAL;
    const int64_t ntiles_q = (Nq + bq - 1) / bq;
    int failed = 0;

#pragma omp parallel
    {
        double *s = (double *)malloc((size_t)(bq * bk) * sizeof(double));
        double *m = (double *)malloc((size_t)bq * sizeof(double));
        double *l = (double *)malloc((size_t)bq * sizeof(double));
        double *acc = (double *)malloc((size_t)(bq * D) * sizeof(double));
        const int ok = s && m && l && acc;
        if (!ok) {
#pragma omp atomic write
            failed = 1;
        }
#pragma omp for collapse(2) schedule(dynamic, 1)
        for (int64_t bh = 0; bh < B * H; ++bh) {
            for (int64_t tq = 0; tq < ntiles_q; ++tq) {
                if (!ok)
                    continue;
                const int64_t i0 = tq * bq;
                const int64_t ni = (i0 + bq <= Nq) ? bq : Nq - i0;
                const double *kb = k + bh * Nk * D;
                const double *vb = v + bh * Nk * D;
                for (int64_t r = 0; r < ni; ++r) {
                    m[r] = -INFINITY;
                    l[r] = 0.0;
                    for (int64_t d = 0; d < D; ++d)
                        acc[r * D + d] = 0.0;
                }
                for (int64_t j0 = 0; j0 < Nk; j0 += bk) {
                    const int64_t nj = (j0 + bk <= Nk) ? bk : Nk - j0;
                    for (int64_t r = 0; r < ni; ++r) {
                        const int64_t i = i0 + r;
                        const double *qi = q + (bh * Nq + i) * D;
                        double *sr = s + r * bk;
                        double tmax = -INFINITY;
                        for (int64_t c = 0; c < nj; ++c) {
                            const int64_t j = j0 + c;
                            double dot = 0.0;
                            for (int64_t d = 0; d < D; ++d)
                                dot += qi[d] * kb[j * D + d];
                            sr[c] = scale * dot;
                            if (causal && !(i >= j))
                                sr[c] = -1e6;
                            if (sr[c] > tmax)
                                tmax = sr[c];
                        }
                        const double mnew = (m[r] > tmax) ? m[r] : tmax;
                        const double alpha = exp(m[r] - mnew);
                        double psum = 0.0;
                        for (int64_t c = 0; c < nj; ++c) {
                            sr[c] = exp(sr[c] - mnew);
                            psum += sr[c];
                        }
                        l[r] = alpha * l[r] + psum;
                        double *ar = acc + r * D;
                        for (int64_t d = 0; d < D; ++d) {
                            double pv = 0.0;
                            for (int64_t c = 0; c < nj; ++c)
                                pv += sr[c] * vb[(j0 + c) * D + d];
                            ar[d] = alpha * ar[d] + pv;
                        }
                        m[r] = mnew;
                    }
                }
                for (int64_t r = 0; r < ni; ++r) {
                    const int64_t row = bh * Nq + i0 + r;
                    for (int64_t d = 0; d < D; ++d)
                        o[row * D + d] = acc[r * D + d] / l[r];
                    lse[row] = m[r] + log(l[r]);
                }
            }
        }
        free(s);
        free(m);
        free(l);
        free(acc);
    }
    return failed ? ORACLE_ENOMEM : ORACLE_OK;
}

/*
 * Gradients of the attention forward pass, the plain chain rule in double
 * precision.  Page "解释FlashAttention的显存优化原理" §一.2(2) (and page
 * "FlashAttention技术演进全景图" §2.2, item 3) describe the backward pass as
 * recomputing the forward quantities instead of storing them; page
 * "FlashAttention-2实现与优化：高效注意力机制详解" §3.1 keeps q, k, v, o and L
 * for it and lists the backward pass among its extensions (§7).  The pages
 * print no formula for it, so this routine is the derivative of the
 * definition in fa_oracle_attention, with the upstream gradient dO of O:
 *
 *     P_ij  = exp(s_ij - m_i) / l_i            (the softmax of row i)
 *     dV_j  = sum_i P_ij dO_i
 *     dP_ij = <dO_i, v_j>
 *     D_i   = sum_j P_ij dP_ij                 (softmax Jacobian, row term)
 *     dS_ij = P_ij (dP_ij - D_i)
 *     dQ_i  = scale * sum_j dS_ij k_j
 *     dK_j  = scale * sum_i dS_ij q_i
 *
 * with sums over the visible pairs only (same key set as the forward).
 * Optional "magnitude" outputs bq, bk, bv (same shapes as dq, dk, dv, may be
 * NULL) hold the same sums taken over absolute values,
 *
 *     bv_j = sum_i P_ij |dO_i|
 *     bq_i = scale * sum_j (|dS_ij| + P_ij E_i) |k_j|
 *     bk_j = scale * sum_i (|dS_ij| + P_ij E_i) |q_i|,
 *     E_i  = sum_d |dO_id| sum_j P_ij |v_jd|
 *
 * which bound the effect of rounding one factor of every product to a short
 * floating-point type.  E_i bounds the row term's sensitivity to its O: a
 * GPU forms D_i as <dO_i, O_i> from the forward's stored O, whose error from
 * rounding P is at most a unit roundoff times sum_j P_ij |v_jd| per element
 * (which also covers rounding O itself, since |O_id| is no larger).  Tests
 * derive their tolerances from these sums.
 *
 * qrows / krows optionally restrict dq (and bq) to a list of flat query rows
 * (b*H + h)*Nq + i and dk, dv (and bk, bv) to flat key rows (b*H + h)*Nk + j;
 * the outputs are then [nq, D] / [nk, D] in list order.  Row statistics are
 * computed for every row of each (b, h) slice that holds a requested row,
 * since a key's gradient needs all of them.
 */
int fa_oracle_attention_bwd(const double *q, const double *k, const double *v,
                            const double *dout,
                            double *dq, double *dk, double *dv,
                            double *bq, double *bk, double *bv,
                            int64_t B, int64_t H, int64_t Nq, int64_t Nk, int64_t D,
                            double scale, int causal,
                            const int64_t *qrows, int64_t nq,
                            const int64_t *krows, int64_t nk)
{
    if (!q || !k || !v || !dout || !dq || !dk || !dv || bad_shape(B, H, Nq, Nk, D))
        return ORACLE_EINVAL;
    const int64_t totq = B * H * Nq, totk = B * H * Nk;
    if (qrows)
        for (int64_t t = 0; t < nq; ++t)
            if (qrows[t] < 0 || qrows[t] >= totq)
                return ORACLE_EINVAL;
    if (krows)
        for (int64_t t = 0; t < nk; ++t)
            if (krows[t] < 0 || krows[t] >= totk)
                return ORACLE_EINVAL;
    const int64_t cq = qrows ? nq : totq;
    const int64_t ck = krows ? nk : totk;
    const int magn = bq && bk && bv;

    /* per-row statistics: max m, normaliser l, row term D, and E
       (o below holds sum_j P_ij |v_j|, the magnitude of row i of O) */
    double *m = (double *)malloc((size_t)totq * sizeof(double));
    double *l = (double *)malloc((size_t)totq * sizeof(double));
    double *rd = (double *)malloc((size_t)totq * sizeof(double));
    double *re = (double *)malloc((size_t)totq * sizeof(double));
    if (!m || !l || !rd || !re) {
        free(m);
        free(l);
        free(rd);
        free(re);
        return ORACLE_ENOMEM;
    }
    /* slices (b, h) that hold a requested row: only their statistics are
       needed */
    unsigned char *need = (unsigned char *)calloc((size_t)(B * H), 1);
    if (!need) {
        free(m);
        free(l);
        free(rd);
        free(re);
        return ORACLE_ENOMEM;
    }
    if (!qrows || !krows)
        memset(need, 1, (size_t)(B * H));
    else {
        for (int64_t t = 0; t < nq; ++t)
            need[qrows[t] / Nq] = 1;
        for (int64_t t = 0; t < nk; ++t)
            need[krows[t] / Nk] = 1;
    }
    int failed = 0;

#pragma omp parallel
    {
        double *s = (double *)malloc((size_t)Nk * sizeof(double));
        double *o = (double *)malloc((size_t)D * sizeof(double));
        if (!s || !o) {
#pragma omp atomic write
            failed = 1;
        }
        /* pass 1, every query row: scores, m, l, then P, dP, D_i and E_i */
#pragma omp for schedule(dynamic, 8)
        for (int64_t r = 0; r < totq; ++r) {
            if (!s || !o || !need[r / Nq])
                continue;
            const int64_t bh = r / Nq, i = r % Nq;
            const double *qi = q + r * D, *gi = dout + r * D;
            const double *kb = k + bh * Nk * D, *vb = v + bh * Nk * D;
            const int64_t n = valid_keys(i, Nk, causal);
            double mx = -INFINITY;
            for (int64_t j = 0; j < n; ++j) {
                double dot = 0.0;
                for (int64_t d = 0; d < D; ++d)
                    dot += qi[d] * kb[j * D + d];
                s[j] = scale * dot;
                if (s[j] > mx)
                    mx = s[j];
            }
            double sum = 0.0;
            for (int64_t j = 0; j < n; ++j)
                sum += exp(s[j] - mx);
            double acc = 0.0;
            for (int64_t d = 0; d < D; ++d)
                o[d] = 0.0;
            for (int64_t j = 0; j < n; ++j) {
                const double p = exp(s[j] - mx) / sum;
                double dp = 0.0;
                for (int64_t d = 0; d < D; ++d) {
                    dp += gi[d] * vb[j * D + d];
                    o[d] += p * fabs(vb[j * D + d]);
                }
                acc += p * dp;
            }
            double e = 0.0;
            for (int64_t d = 0; d < D; ++d)
                e += fabs(gi[d]) * o[d];
            m[r] = mx;
            l[r] = sum;
            rd[r] = acc;
            re[r] = e;
        }
        /* implicit barrier: every row's statistics are ready */

        /* pass 2, the requested query rows: dQ_i */
#pragma omp for schedule(dynamic, 8)
        for (int64_t t = 0; t < cq; ++t) {
            const int64_t r = qrows ? qrows[t] : t;
            const int64_t bh = r / Nq, i = r % Nq;
            const double *qi = q + r * D, *gi = dout + r * D;
            const double *kb = k + bh * Nk * D, *vb = v + bh * Nk * D;
            const int64_t n = valid_keys(i, Nk, causal);
            double *gq = dq + t * D;
            double *mq = magn ? bq + t * D : NULL;
            for (int64_t d = 0; d < D; ++d) {
                gq[d] = 0.0;
                if (mq)
                    mq[d] = 0.0;
            }
            for (int64_t j = 0; j < n; ++j) {
                double dot = 0.0, dp = 0.0;
                for (int64_t d = 0; d < D; ++d) {
                    dot += qi[d] * kb[j * D + d];
                    dp += gi[d] * vb[j * D + d];
                }
                const double p = exp(scale * dot - m[r]) / l[r];
                const double ds = p * (dp - rd[r]);
                const double w = fabs(ds) + p * re[r];
                for (int64_t d = 0; d < D; ++d) {
                    gq[d] += ds * kb[j * D + d];
                    if (mq)
                        mq[d] += w * fabs(kb[j * D + d]);
                }
            }
            for (int64_t d = 0; d < D; ++d) {
                gq[d] *= scale;
                if (mq)
                    mq[d] *= fabs(scale);
            }
        }

        /* pass 3, the requested key rows: dK_j and dV_j */
#pragma omp for schedule(dynamic, 8)
        for (int64_t t = 0; t < ck; ++t) {
            const int64_t c = krows ? krows[t] : t;
            const int64_t bh = c / Nk, j = c % Nk;
            const double *kj = k + c * D, *vj = v + c * D;
            double *gk = dk + t * D, *gv = dv + t * D;
            double *mk = magn ? bk + t * D : NULL, *mv = magn ? bv + t * D : NULL;
            for (int64_t d = 0; d < D; ++d) {
                gk[d] = gv[d] = 0.0;
                if (magn)
                    mk[d] = mv[d] = 0.0;
            }
            /* rows that see key j: all rows, or i >= j when causal */
            for (int64_t i = causal ? j : 0; i < Nq; ++i) {
                const int64_t r = bh * Nq + i;
                const double *qi = q + r * D, *gi = dout + r * D;
                double dot = 0.0, dp = 0.0;
                for (int64_t d = 0; d < D; ++d) {
                    dot += qi[d] * kj[d];
                    dp += gi[d] * vj[d];
                }
                const double p = exp(scale * dot - m[r]) / l[r];
                const double ds = p * (dp - rd[r]);
                const double w = fabs(ds) + p * re[r];
                for (int64_t d = 0; d < D; ++d) {
                    gv[d] += p * gi[d];
                    gk[d] += ds * qi[d];
                    if (magn) {
                        mv[d] += p * fabs(gi[d]);
                        mk[d] += w * fabs(qi[d]);
                    }
                }
            }
            for (int64_t d = 0; d < D; ++d) {
                gk[d] *= scale;
                if (magn)
                    mk[d] *= fabs(scale);
            }
        }
        free(s);
        free(o);
    }
    free(need);
    free(m);
    free(l);
    free(rd);
    free(re);
    return failed ? ORACLE_ENOMEM : ORACLE_OK;
}

/*
 * Attention under a local-window + global-token mask, the plain definition
 * in double precision.  Page "FlashAttention-2实现与优化：高效注意力机制详解"
 * §7 names sparse attention combining local windows and global tokens as an
 * extension, and page "解释FlashAttention的显存优化原理" §二 (case 2) uses
 * local blocks plus global key points; neither defines the pattern, so this
 * file reads it as: key j (j < Nk) is visible to query i iff
 *
 *     (causal ? 0 <= i - j < window : |i - j| < window)      local band
 *  or (j < nglobal || i < nglobal) && (!causal || j <= i)     global tokens
 *
 * (indices from 0 in both sequences; window >= 1, nglobal >= 0).  Over the
 * visible keys the row is the two-pass softmax of fa_oracle_attention.  A
 * row with no visible key (possible only when Nq > Nk) gets O = 0 and
 * L = -inf.  "rows" as in fa_oracle_attention.
 */
static int visible_masked(int64_t i, int64_t j, int causal, int64_t window, int64_t nglobal)
{
    const int64_t d = i - j;
    const int local = causal ? (d >= 0 && d < window) : (d > -window && d < window);
    const int global = (j < nglobal || i < nglobal) && (!causal || j <= i);
    return local || global;
}

int fa_oracle_attention_masked(const double *q, const double *k, const double *v,
                               double *o, double *lse,
                               int64_t B, int64_t H, int64_t Nq, int64_t Nk, int64_t D,
                               double scale, int causal, int64_t window, int64_t nglobal,
                               const int64_t *rows, int64_t nrows)
{
    if (!q || !k || !v || !o || !lse || bad_shape(B, H, Nq, Nk, D) || window < 1 ||
        nglobal < 0)
        return ORACLE_EINVAL;
    const int64_t total = B * H * Nq;
    const int64_t count = rows ? nrows : total;
    if (rows)
        for (int64_t t = 0; t < nrows; ++t)
            if (rows[t] < 0 || rows[t] >= total)
                return ORACLE_EINVAL;
    int failed = 0;

#pragma omp parallel
    {
        double *w = (double *)malloc((size_t)Nk * sizeof(double));
        int64_t *idx = (int64_t *)malloc((size_t)Nk * sizeof(int64_t));
        if (!w || !idx) {
#pragma omp atomic write
            failed = 1;
        }
#pragma omp for schedule(dynamic, 8)
        for (int64_t t = 0; t < count; ++t) {
            if (!w || !idx)
                continue;
            const int64_t r = rows ? rows[t] : t;
            const int64_t bh = r / Nq, i = r % Nq;
            const double *qi = q + r * D;
            const double *kb = k + bh * Nk * D, *vb = v + bh * Nk * D;
            double *oi = o + t * D;
            int64_t n = 0;
            for (int64_t j = 0; j < Nk; ++j)
                if (visible_masked(i, j, causal, window, nglobal))
                    idx[n++] = j;
            for (int64_t d = 0; d < D; ++d)
                oi[d] = 0.0;
            if (n == 0) {
                lse[t] = -INFINITY;
                continue;
            }
            double m = -INFINITY;
            for (int64_t c = 0; c < n; ++c) {
                double dot = 0.0;
                for (int64_t d = 0; d < D; ++d)
                    dot += qi[d] * kb[idx[c] * D + d];
                w[c] = scale * dot;
                if (w[c] > m)
                    m = w[c];
            }
            double l = 0.0;
            for (int64_t c = 0; c < n; ++c) {
                w[c] = exp(w[c] - m);
                l += w[c];
            }
            for (int64_t c = 0; c < n; ++c)
                for (int64_t d = 0; d < D; ++d)
                    oi[d] += w[c] * vb[idx[c] * D + d];
            for (int64_t d = 0; d < D; ++d)
                oi[d] /= l;
            lse[t] = m + log(l);
        }
        free(w);
        free(idx);
    }
    return failed ? ORACLE_ENOMEM : ORACLE_OK;
}

/*
 * Gradients of fa_oracle_attention_masked (the local-window + global-token
 * mask), the chain rule in double precision over the visible pairs only:
 * with P_ij the softmax of row i over its visible keys,
 *     dV_j = sum_i P_ij dO_i,  dP_ij = <dO_i, v_j>,  D_i = sum_j P_ij dP_ij,
 *     dS_ij = P_ij (dP_ij - D_i),
 *     dQ_i = scale sum_j dS_ij k_j,  dK_j = scale sum_i dS_ij q_i.
 * Rows with no visible key contribute nothing (dQ_i = 0).  The magnitude
 * sums bq, bk, bv (may be NULL) and the row lists qrows / krows are those of
 * fa_oracle_attention_bwd, with every sum over the visible pairs: they bound
 * the effect of rounding one factor of every product, and the row lists
 * restrict the outputs to sampled rows (statistics are computed for every
 * row of each (b, h) slice that holds a requested row).
 */
int fa_oracle_attention_bwd_masked(const double *q, const double *k, const double *v,
                                   const double *dout, double *dq, double *dk, double *dv,
                                   double *bq, double *bk, double *bv,
                                   int64_t B, int64_t H, int64_t Nq, int64_t Nk, int64_t D,
                                   double scale, int causal, int64_t window, int64_t nglobal,
                                   const int64_t *qrows, int64_t nq,
                                   const int64_t *krows, int64_t nk)
{
    if (!q || !k || !v || !dout || !dq || !dk || !dv || bad_shape(B, H, Nq, Nk, D) ||
        window < 1 || nglobal < 0)
        return ORACLE_EINVAL;
    const int64_t totq = B * H * Nq, totk = B * H * Nk;
    if (qrows)
        for (int64_t t = 0; t < nq; ++t)
            if (qrows[t] < 0 || qrows[t] >= totq)
                return ORACLE_EINVAL;
    if (krows)
        for (int64_t t = 0; t < nk; ++t)
            if (krows[t] < 0 || krows[t] >= totk)
                return ORACLE_EINVAL;
    const int64_t cq = qrows ? nq : totq;
    const int64_t ck = krows ? nk : totk;
    const int magn = bq && bk && bv;
    double *m = (double *)malloc((size_t)totq * sizeof(double));
    double *l = (double *)malloc((size_t)totq * sizeof(double));
    double *rd = (double *)malloc((size_t)totq * sizeof(double));
    double *re = (double *)malloc((size_t)totq * sizeof(double));
    unsigned char *need = (unsigned char *)calloc((size_t)(B * H), 1);
    if (!m || !l || !rd || !re || !need) {
        free(m);
        free(l);
        free(rd);
        free(re);
        free(need);
        return ORACLE_ENOMEM;
    }
    if (!qrows || !krows)
        memset(need, 1, (size_t)(B * H));
    else {
        for (int64_t t = 0; t < nq; ++t)
            need[qrows[t] / Nq] = 1;
        for (int64_t t = 0; t < nk; ++t)
            need[krows[t] / Nk] = 1;
    }
    int failed = 0;

#pragma omp parallel
    {
        double *o = (double *)malloc((size_t)D * sizeof(double));
        if (!o) {
#pragma omp atomic write
            failed = 1;
        }
        /* pass 1, every query row of the needed slices: max m, normaliser l,
           row term D_i and E_i = sum_d |dO_id| sum_j P_ij |v_jd| */
#pragma omp for schedule(dynamic, 8)
        for (int64_t r = 0; r < totq; ++r) {
            if (!o || !need[r / Nq])
                continue;
            const int64_t bh = r / Nq, i = r % Nq;
            const double *qi = q + r * D, *gi = dout + r * D;
            const double *kb = k + bh * Nk * D, *vb = v + bh * Nk * D;
            double mx = -INFINITY;
            for (int64_t j = 0; j < Nk; ++j) {
                if (!visible_masked(i, j, causal, window, nglobal))
                    continue;
                double dot = 0.0;
                for (int64_t d = 0; d < D; ++d)
                    dot += qi[d] * kb[j * D + d];
                if (scale * dot > mx)
                    mx = scale * dot;
            }
            double sum = 0.0;
            for (int64_t j = 0; j < Nk; ++j) {
                if (!visible_masked(i, j, causal, window, nglobal))
                    continue;
                double dot = 0.0;
                for (int64_t d = 0; d < D; ++d)
                    dot += qi[d] * kb[j * D + d];
                sum += exp(scale * dot - mx);
            }
            double acc = 0.0;
            for (int64_t d = 0; d < D; ++d)
                o[d] = 0.0;
            for (int64_t j = 0; j < Nk && sum > 0.0; ++j) {
                if (!visible_masked(i, j, causal, window, nglobal))
                    continue;
                double dot = 0.0, dp = 0.0;
                for (int64_t d = 0; d < D; ++d) {
                    dot += qi[d] * kb[j * D + d];
                    dp += gi[d] * vb[j * D + d];
                }
                const double p = exp(scale * dot - mx) / sum;
                for (int64_t d = 0; d < D; ++d)
                    o[d] += p * fabs(vb[j * D + d]);
                acc += p * dp;
            }
            double e = 0.0;
            for (int64_t d = 0; d < D; ++d)
                e += fabs(gi[d]) * o[d];
            m[r] = mx;
            l[r] = sum;
            rd[r] = acc;
            re[r] = e;
        }
        /* implicit barrier: every needed row's statistics are ready */

        /* pass 2, the requested query rows: dQ_i (and bq_i) */
#pragma omp for schedule(dynamic, 8)
        for (int64_t t = 0; t < cq; ++t) {
            const int64_t r = qrows ? qrows[t] : t;
            const int64_t bh = r / Nq, i = r % Nq;
            const double *qi = q + r * D, *gi = dout + r * D;
            const double *kb = k + bh * Nk * D, *vb = v + bh * Nk * D;
            double *aq = dq + t * D;
            double *mq = magn ? bq + t * D : NULL;
            for (int64_t d = 0; d < D; ++d) {
                aq[d] = 0.0;
                if (mq)
                    mq[d] = 0.0;
            }
            for (int64_t j = 0; j < Nk && l[r] > 0.0; ++j) {
                if (!visible_masked(i, j, causal, window, nglobal))
                    continue;
                double dot = 0.0, dp = 0.0;
                for (int64_t d = 0; d < D; ++d) {
                    dot += qi[d] * kb[j * D + d];
                    dp += gi[d] * vb[j * D + d];
                }
                const double p = exp(scale * dot - m[r]) / l[r];
                const double ds = p * (dp - rd[r]);
                const double w = fabs(ds) + p * re[r];
                for (int64_t d = 0; d < D; ++d) {
                    aq[d] += ds * kb[j * D + d];
                    if (mq)
                        mq[d] += w * fabs(kb[j * D + d]);
                }
            }
            for (int64_t d = 0; d < D; ++d) {
                aq[d] *= scale;
                if (mq)
                    mq[d] *= fabs(scale);
            }
        }

        /* pass 3, the requested key rows: dK_j and dV_j (and bk_j, bv_j) */
#pragma omp for schedule(dynamic, 8)
        for (int64_t t = 0; t < ck; ++t) {
            const int64_t c = krows ? krows[t] : t;
            const int64_t bh = c / Nk, j = c % Nk;
            const double *kc = k + c * D, *vc = v + c * D;
            double *ak = dk + t * D, *av = dv + t * D;
            double *mk = magn ? bk + t * D : NULL, *mv = magn ? bv + t * D : NULL;
            for (int64_t d = 0; d < D; ++d) {
                ak[d] = av[d] = 0.0;
                if (magn)
                    mk[d] = mv[d] = 0.0;
            }
            for (int64_t i = 0; i < Nq; ++i) {
                if (!visible_masked(i, j, causal, window, nglobal))
                    continue;
                const int64_t r = bh * Nq + i;
                const double *qi = q + r * D, *gi = dout + r * D;
                double dot = 0.0, dp = 0.0;
                for (int64_t d = 0; d < D; ++d) {
                    dot += qi[d] * kc[d];
                    dp += gi[d] * vc[d];
                }
                const double p = exp(scale * dot - m[r]) / l[r];
                const double ds = p * (dp - rd[r]);
                const double w = fabs(ds) + p * re[r];
                for (int64_t d = 0; d < D; ++d) {
                    av[d] += p * gi[d];
                    ak[d] += ds * qi[d];
                    if (magn) {
                        mv[d] += p * fabs(gi[d]);
                        mk[d] += w * fabs(qi[d]);
                    }
                }
            }
            for (int64_t d = 0; d < D; ++d) {
                ak[d] *= scale;
                if (magn)
                    mk[d] *= fabs(scale);
            }
        }
        free(o);
    }
    free(m);
    free(l);
    free(rd);
    free(re);
    free(need);
    return failed ? ORACLE_ENOMEM : ORACLE_OK;
}
