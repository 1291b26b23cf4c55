/*
 * attn_oracle.c -- plain fp64 CPU oracle for exact (causal) softmax attention
 * and its analytic gradients.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path links, loads or calls
 * this file: only the test suite, the package smoke check and the CPU-baseline
 * leg of the benchmark do.  It shares no source, header, table or helper with
 * the HIP library.
 *
 * What it computes is the textbook definition, materialised one query row at a
 * time (a row of P is held as S doubles; nothing S x S is ever resident):
 *
 *   CS336 Assignment 2 handout (videobook.pages.dev, "Stanford-CS336 A2"),
 *   section 4.2 "FlashAttention-2", Eq. 4-6 (forward), Eq. 12 (logsumexp),
 *   Eq. 7-11 (standard backward) and Eq. 13-19 (backward with the row
 *   statistic D = rowsum(O o dO)).
 *
 *   s_ij  = scale * <Q_i, K_j>                       (Eq. 4, scale = 1/sqrt(d) by default)
 *   P_ij  = exp(s_ij - m_i) / l_i  over allowed j    (Eq. 5, row softmax)
 *   O_i   = sum_j P_ij V_j                           (Eq. 6)
 *   L_i   = m_i + ln l_i = ln sum_j exp(s_ij)        (Eq. 12, natural log of scaled scores)
 *   dV_j  = sum_i P_ij dO_i                          (Eq. 7 / 15)
 *   dP_ij = <dO_i, V_j>                              (Eq. 8 / 16)
 *   Delta_i = sum_j P_ij dP_ij  (= <dO_i, O_i>)      (handout text before Eq. 13)
 *   dS_ij = P_ij (dP_ij - Delta_i)                   (Eq. 9 / 17)
 *   dQ_i  = scale * sum_j dS_ij K_j                  (Eq. 10 / 18)
 *   dK_j  = scale * sum_i dS_ij Q_i                  (Eq. 11 / 19)
 *
 * Causal masking: key j is allowed for query i iff j <= i (0-based, diagonal
 * included, both sequences starting at position 0), as in the handout's
 * flash_forward part (c) and the lecture notes' online-attention sketch;
 * excluded keys get P_ij = 0 exactly.
 *
 * Layout: every tensor is one contiguous block of BH heads, each [Sq or Sk][D]
 * row-major doubles.  Q/O/dO/dQ have Sq rows per head, K/V/dK/dV Sk rows.
 * lse and delta are [BH][Sq].
 *
 * Parallelism is OpenMP over heads (and over rows where rows are independent);
 * it changes no arithmetic order inside a head's reduction.
 */
#include <math.h>
#include <stddef.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

static double dot(const double *a, const double *b, long n)
{
    double s = 0.0;
    for (long t = 0; t < n; ++t)
        s += a[t] * b[t];
    return s;
}

/* Number of keys query i may attend to. */
static long n_allowed(long i, long Sk, int causal)
{
    if (!causal)
        return Sk;
    return (i + 1 < Sk) ? i + 1 : Sk;
}

/*
 * One query row of the forward definition (Eq. 4-6, 12).
 * p (scratch, Sk doubles) receives the normalised probabilities P_i. (zeros
 * for excluded keys).  Writes o[D] and *lse.
 */
static void row_forward(const double *qi, const double *k, const double *v,
                        long Sk, long D, double scale, long nkeys,
                        double *p, double *o, double *lse)
{
    double m = -INFINITY;
    for (long j = 0; j < nkeys; ++j) {
        p[j] = scale * dot(qi, k + j * D, D);        /* s_ij */
        if (p[j] > m)
            m = p[j];
    }
    double l = 0.0;
    for (long j = 0; j < nkeys; ++j) {
        p[j] = exp(p[j] - m);
        l += p[j];
    }
    for (long j = 0; j < nkeys; ++j)
        p[j] /= l;                                   /* P_ij */
    for (long j = nkeys; j < Sk; ++j)
        p[j] = 0.0;
    for (long d = 0; d < D; ++d)
        o[d] = 0.0;
    for (long j = 0; j < nkeys; ++j) {
        const double *vj = v + j * D;
        for (long d = 0; d < D; ++d)
            o[d] += p[j] * vj[d];                    /* O_i = sum_j P_ij V_j */
    }
    *lse = m + log(l);                               /* L_i = m_i + ln l_i */
}

/* Forward: O [BH][Sq][D], lse [BH][Sq]. */
void oracle_fwd(const double *q, const double *k, const double *v,
                double *o, double *lse, long BH, long Sq, long Sk, long D,
                double scale, int causal, int nthreads)
{
#ifdef _OPENMP
    if (nthreads > 0)
        omp_set_num_threads(nthreads);
#endif
#pragma omp parallel
    {
        double *p = (double *)malloc(sizeof(double) * (size_t)(Sk > 0 ? Sk : 1));
#pragma omp for collapse(2) schedule(dynamic, 16)
        for (long h = 0; h < BH; ++h)
            for (long i = 0; i < Sq; ++i) {
                const double *qh = q + h * Sq * D, *kh = k + h * Sk * D, *vh = v + h * Sk * D;
                row_forward(qh + i * D, kh, vh, Sk, D, scale, n_allowed(i, Sk, causal), p,
                            o + (h * Sq + i) * D, lse + h * Sq + i);
            }
        free(p);
    }
}

/*
 * Full backward of one head from the definition (Eq. 7-11 with the Delta
 * simplification of Eq. 13-19).  Recomputes each row of P from scratch.
 * Outputs dq [Sq][D], dk/dv [Sk][D] (overwritten), o [Sq][D], lse [Sq],
 * delta_p [Sq] = sum_j P_ij dP_ij and delta_o [Sq] = <dO_i, O_i>.
 */
static void head_backward(const double *q, const double *k, const double *v,
                          const double *dout, double *dq, double *dk, double *dv,
                          double *o, double *lse, double *delta_p, double *delta_o,
                          long Sq, long Sk, long D, double scale, int causal)
{
    double *p = (double *)malloc(sizeof(double) * (size_t)(Sk > 0 ? Sk : 1));
    double *dp = (double *)malloc(sizeof(double) * (size_t)(Sk > 0 ? Sk : 1));
    memset(dk, 0, sizeof(double) * (size_t)(Sk * D));
    memset(dv, 0, sizeof(double) * (size_t)(Sk * D));
    for (long i = 0; i < Sq; ++i) {
        const double *qi = q + i * D, *doi = dout + i * D;
        double *oi = o + i * D, *dqi = dq + i * D;
        long nk = n_allowed(i, Sk, causal);
        row_forward(qi, k, v, Sk, D, scale, nk, p, oi, lse + i);
        double dsum = 0.0;
        for (long j = 0; j < nk; ++j) {
            dp[j] = dot(doi, v + j * D, D);             /* dP_ij = <dO_i, V_j> */
            dsum += p[j] * dp[j];
        }
        delta_p[i] = dsum;                               /* Delta_i = sum_j P_ij dP_ij */
        delta_o[i] = dot(doi, oi, D);                    /* Delta_i = <dO_i, O_i> */
        for (long d = 0; d < D; ++d)
            dqi[d] = 0.0;
        for (long j = 0; j < nk; ++j) {
            double ds = p[j] * (dp[j] - dsum);           /* dS_ij */
            const double *kj = k + j * D;
            double *dkj = dk + j * D, *dvj = dv + j * D;
            for (long d = 0; d < D; ++d) {
                dqi[d] += scale * ds * kj[d];            /* dQ_i = scale sum_j dS_ij K_j */
                dkj[d] += scale * ds * qi[d];            /* dK_j = scale sum_i dS_ij Q_i */
                dvj[d] += p[j] * doi[d];                 /* dV_j = sum_i P_ij dO_i */
            }
        }
    }
    free(p);
    free(dp);
}

/* Backward for all heads; also returns O, lse and both forms of Delta. */
void oracle_bwd(const double *q, const double *k, const double *v, const double *dout,
                double *dq, double *dk, double *dv, double *o, double *lse,
                double *delta_p, double *delta_o, long BH, long Sq, long Sk, long D,
                double scale, int causal, int nthreads)
{
#ifdef _OPENMP
    if (nthreads > 0)
        omp_set_num_threads(nthreads);
#endif
#pragma omp parallel for schedule(dynamic, 1)
    for (long h = 0; h < BH; ++h)
        head_backward(q + h * Sq * D, k + h * Sk * D, v + h * Sk * D, dout + h * Sq * D,
                      dq + h * Sq * D, dk + h * Sk * D, dv + h * Sk * D, o + h * Sq * D,
                      lse + h * Sq, delta_p + h * Sq, delta_o + h * Sq, Sq, Sk, D, scale,
                      causal);
}

/*
 * Materialised probabilities of one head, P [Sq][Sk] (small shapes only; used
 * to check the softmax invariants).
 */
void oracle_probs(const double *q, const double *k, double *P, long Sq, long Sk, long D,
                  double scale, int causal)
{
    double *o = (double *)malloc(sizeof(double) * (size_t)(D > 0 ? D : 1));
    double *vz = (double *)calloc((size_t)(Sk * D > 0 ? Sk * D : 1), sizeof(double));
    for (long i = 0; i < Sq; ++i) {
        double lse;
        row_forward(q + i * D, k, vz, Sk, D, scale, n_allowed(i, Sk, causal), P + i * Sk, o,
                    &lse);
    }
    free(o);
    free(vz);
}

/*
 * Sampled evaluation of one head (for shapes where the full backward is too
 * slow on the host).
 *
 * oracle_head_stats: for every query row i of the head, L_i and
 *   Delta_i = <dO_i, O_i> with O_i the oracle's own fp64 output.
 * oracle_rows: for the listed query rows, O_i, L_i and dQ_i
 *   (each needs only row i of P, dP and dS).
 * oracle_cols: for the listed keys j, dK_j and dV_j, given the head's full L
 *   and Delta (P_ij = exp(s_ij - L_i), Eq. 14; dS_ij = P_ij (dP_ij - Delta_i),
 *   Eq. 17; dK_j = scale sum_i dS_ij Q_i, Eq. 19; dV_j = sum_i P_ij dO_i, Eq. 15).
 */
void oracle_head_stats(const double *q, const double *k, const double *v, const double *dout,
                       double *lse, double *delta, long S, long D, double scale, int causal,
                       int nthreads)
{
#ifdef _OPENMP
    if (nthreads > 0)
        omp_set_num_threads(nthreads);
#endif
#pragma omp parallel
    {
        double *p = (double *)malloc(sizeof(double) * (size_t)(S > 0 ? S : 1));
        double *o = (double *)malloc(sizeof(double) * (size_t)(D > 0 ? D : 1));
#pragma omp for schedule(dynamic, 8)
        for (long i = 0; i < S; ++i) {
            row_forward(q + i * D, k, v, S, D, scale, n_allowed(i, S, causal), p, o, lse + i);
            delta[i] = dot(dout + i * D, o, D);
        }
        free(p);
        free(o);
    }
}

void oracle_rows(const double *q, const double *k, const double *v, const double *dout,
                 const long *rows, long nrows, double *o, double *lse, double *dq, long S,
                 long D, double scale, int causal, int nthreads)
{
#ifdef _OPENMP
    if (nthreads > 0)
        omp_set_num_threads(nthreads);
#endif
#pragma omp parallel
    {
        double *p = (double *)malloc(sizeof(double) * (size_t)(S > 0 ? S : 1));
        double *dp = (double *)malloc(sizeof(double) * (size_t)(S > 0 ? S : 1));
#pragma omp for schedule(dynamic, 1)
        for (long r = 0; r < nrows; ++r) {
            long i = rows[r];
            long nk = n_allowed(i, S, causal);
            const double *qi = q + i * D, *doi = dout + i * D;
            double *oi = o + r * D, *dqi = dq + r * D;
            row_forward(qi, k, v, S, D, scale, nk, p, oi, lse + r);
            double dsum = dot(doi, oi, D);                 /* Delta_i = <dO_i, O_i> */
            for (long d = 0; d < D; ++d)
                dqi[d] = 0.0;
            for (long j = 0; j < nk; ++j) {
                dp[j] = dot(doi, v + j * D, D);
                double ds = p[j] * (dp[j] - dsum);
                const double *kj = k + j * D;
                for (long d = 0; d < D; ++d)
                    dqi[d] += scale * ds * kj[d];
            }
        }
        free(p);
        free(dp);
    }
}

void oracle_cols(const double *q, const double *k, const double *v, const double *dout,
                 const double *lse, const double *delta, const long *cols, long ncols,
                 double *dk, double *dv, long S, long D, double scale, int causal, int nthreads)
{
#ifdef _OPENMP
    if (nthreads > 0)
        omp_set_num_threads(nthreads);
#endif
#pragma omp parallel for schedule(dynamic, 1)
    for (long c = 0; c < ncols; ++c) {
        long j = cols[c];
        const double *kj = k + j * D, *vj = v + j * D;
        double *dkj = dk + c * D, *dvj = dv + c * D;
        for (long d = 0; d < D; ++d) {
            dkj[d] = 0.0;
            dvj[d] = 0.0;
        }
        for (long i = causal ? j : 0; i < S; ++i) {
            const double *qi = q + i * D, *doi = dout + i * D;
            double pij = exp(scale * dot(qi, kj, D) - lse[i]);   /* Eq. 14 */
            double ds = pij * (dot(doi, vj, D) - delta[i]);     /* Eq. 16-17 */
            for (long d = 0; d < D; ++d) {
                dkj[d] += scale * ds * qi[d];
                dvj[d] += pij * doi[d];
            }
        }
    }
}


/*
 * Forward with the queries shifted against the keys (queries and keys of
 * different lengths, e.g. one shard of a sequence against another):
 * query i sits q_offset positions after key 0, so under the causal mask key j
 * is allowed iff j <= i + q_offset.  A row that allows no key has no softmax;
 * it gets O_i = 0 and L_i = -inf (the empty sum), the values that leave any
 * merge with other key sets unchanged.  Same equations as oracle_fwd
 * (handout Eq. 4-6, 12).
 */
void oracle_fwd_offset(const double *q, const double *k, const double *v,
                       double *o, double *lse, long BH, long Sq, long Sk, long D,
                       double scale, int causal, long q_offset, int nthreads)
{
#ifdef _OPENMP
    if (nthreads > 0)
        omp_set_num_threads(nthreads);
#endif
#pragma omp parallel
    {
        double *p = (double *)malloc(sizeof(double) * (size_t)(Sk > 0 ? Sk : 1));
#pragma omp for collapse(2) schedule(dynamic, 16)
        for (long h = 0; h < BH; ++h)
            for (long i = 0; i < Sq; ++i) {
                const double *qh = q + h * Sq * D, *kh = k + h * Sk * D, *vh = v + h * Sk * D;
                long nkeys = Sk;
                if (causal) {
                    nkeys = i + 1 + q_offset;
                    if (nkeys < 0)
                        nkeys = 0;
                    if (nkeys > Sk)
                        nkeys = Sk;
                }
                double *oi = o + (h * Sq + i) * D;
                if (nkeys == 0) {
                    for (long d = 0; d < D; ++d)
                        oi[d] = 0.0;
                    lse[h * Sq + i] = -INFINITY;
                    continue;
                }
                row_forward(qh + i * D, kh, vh, Sk, D, scale, nkeys, p, oi, lse + h * Sq + i);
            }
        free(p);
    }
}

/*
 * Merge of attention results over disjoint key sets (the ring-attention
 * blog "[Attention]FlashAttention/Ring-Attention/混合序列并行的统一原理",
 * section "online attention": the softmax numerators and denominators of
 * the two halves are rescaled to the common maximum and added).  With each
 * part's result given as its normalised output o_r and logsumexp L_r
 * (denominator B_r e^{m_r} = e^{L_r}), the merged row is
 *   M = max_r L_r,  w_r = e^{L_r - M},  O = sum_r w_r o_r / sum_r w_r,
 *   L = M + ln sum_r w_r,
 * and a row that is empty in every part stays O = 0, L = -inf.
 * o_parts [n][rows][D], lse_parts [n][rows]; o [rows][D], lse [rows].
 */
void oracle_merge(const double *o_parts, const double *lse_parts, long n, double *o,
                  double *lse, long rows, long D)
{
#pragma omp parallel for schedule(static)
    for (long i = 0; i < rows; ++i) {
        double M = -INFINITY;
        for (long r = 0; r < n; ++r)
            if (lse_parts[r * rows + i] > M)
                M = lse_parts[r * rows + i];
        double *oi = o + i * D;
        for (long d = 0; d < D; ++d)
            oi[d] = 0.0;
        if (M == -INFINITY) {
            lse[i] = -INFINITY;
            continue;
        }
        double wsum = 0.0;
        for (long r = 0; r < n; ++r) {
            const double w = exp(lse_parts[r * rows + i] - M);
            wsum += w;
            const double *pr = o_parts + (r * rows + i) * D;
            for (long d = 0; d < D; ++d)
                oi[d] += w * pr[d];
        }
        for (long d = 0; d < D; ++d)
            oi[d] /= wsum;
        lse[i] = M + log(wsum);
    }
}


/*
 * Gradient contributions of one key set, given the row statistics L and
 * Delta of the full attention (over every key set).  With P_ij = exp(s_ij -
 * L_i) (handout Eq. 14, with the full L), the backward equations Eq. 15-19
 * are sums over keys, so they split exactly over disjoint key sets: this set
 * contributes dQ_i += scale sum_{j in set} dS_ij K_j and owns dK_j, dV_j of its
 * keys summed over these queries.  Key j is allowed for query i iff
 * j <= i + q_offset (causal); a row with L_i = -inf has no probability mass
 * and contributes nothing.  Outputs are overwritten:
 * dq [BH][Sq][D], dk/dv [BH][Sk][D].
 */
void oracle_bwd_partial(const double *q, const double *k, const double *v, const double *dout,
                        const double *lse, const double *delta, double *dq, double *dk,
                        double *dv, long BH, long Sq, long Sk, long D, double scale, int causal,
                        long q_offset, int nthreads)
{
#ifdef _OPENMP
    if (nthreads > 0)
        omp_set_num_threads(nthreads);
#endif
#pragma omp parallel for schedule(dynamic, 1)
    for (long h = 0; h < BH; ++h) {
        const double *qh = q + h * Sq * D, *kh = k + h * Sk * D, *vh = v + h * Sk * D;
        const double *doh = dout + h * Sq * D;
        double *dqh = dq + h * Sq * D, *dkh = dk + h * Sk * D, *dvh = dv + h * Sk * D;
        memset(dqh, 0, sizeof(double) * (size_t)(Sq * D));
        memset(dkh, 0, sizeof(double) * (size_t)(Sk * D));
        memset(dvh, 0, sizeof(double) * (size_t)(Sk * D));
        for (long i = 0; i < Sq; ++i) {
            const double L = lse[h * Sq + i], Dl = delta[h * Sq + i];
            if (L == -INFINITY)
                continue;
            long nk = Sk;
            if (causal) {
                nk = i + 1 + q_offset;
                if (nk < 0)
                    nk = 0;
                if (nk > Sk)
                    nk = Sk;
            }
            const double *qi = qh + i * D, *doi = doh + i * D;
            double *dqi = dqh + i * D;
            for (long j = 0; j < nk; ++j) {
                const double pij = exp(scale * dot(qi, kh + j * D, D) - L);   /* Eq. 13-14 */
                const double dpij = dot(doi, vh + j * D, D);                   /* Eq. 16 */
                const double ds = pij * (dpij - Dl);                           /* Eq. 17 */
                const double *kj = kh + j * D;
                double *dkj = dkh + j * D, *dvj = dvh + j * D;
                for (long d = 0; d < D; ++d) {
                    dqi[d] += scale * ds * kj[d];                              /* Eq. 18 */
                    dkj[d] += scale * ds * qi[d];                              /* Eq. 19 */
                    dvj[d] += pij * doi[d];                                    /* Eq. 15 */
                }
            }
        }
    }
}
