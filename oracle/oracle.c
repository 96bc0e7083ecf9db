/*
 * oracle.c -- plain fp64 CPU exact attention.  TEST INFRASTRUCTURE ONLY.
 *
 * This file is the parity oracle for the HIP library.  Only the test suite,
 * the smoke check and the CPU-baseline leg of the benchmark may load it; the
 * product path never calls it, and it shares no source with the HIP code.
 *
 * What it computes, row by row, with every input bf16 value widened exactly
 * to double:
 *
 *   1. a full row of scores S_ij = scale * (q_i . k_j) for every visible key
 *      j, and -inf for every masked key (the masked dot product is skipped:
 *      its value is -inf by definition).  This is the scaled-logit matrix of
 *      the dense definition (mdooai.com "어텐션 최적화: FlashAttention과 희소
 *      어텐션", the key-formula section; the -inf convention for keys outside
 *      the allowed set is the sparse-attention formula of the same page);
 *   2. with the ALiBi flag, a distance bias on visible scores:
 *      S <- S - slope_h * |i - j| for query head h (a bias added before the
 *      softmax that grows with the query-key distance, aegloslab "3.7
 *      어텐션 II" section 3.7.5; the per-head slopes are an input);
 *   3. the soft cap, on visible scores only: S <- c * tanh(S / c) (a kernel
 *      flag in the same section; the order scale -> bias -> mask -> cap is
 *      the reading stated in the design notes);
 *   4. the row softmax P_ij = exp(S_ij - m_i) / sum_j exp(S_ij - m_i) with
 *      m_i = max_j S_ij (llm-systems-engineering "Attention 최적화가 어려운
 *      이유", sections on the computation flow and on the remaining scores);
 *   5. O_i = sum_j P_ij v_j and LSE_i = m_i + ln sum_j exp(S_ij - m_i), the
 *      natural-log form of the row statistics m and l that the forward pass
 *      keeps for the backward pass (youngju.dev "FlashAttention 논문 분석",
 *      section "Recomputation 전략").
 *   6. A row with no visible key gives O_i = 0 and LSE_i = -inf.
 *
 * Visibility of key j for query i in batch row b:
 *   CAUSAL : j <= i
 *   WINDOW : i - window_left <= j <= i + window_right (inclusive; the
 *            symmetric |i-j| <= w window of the sliding-window score_mod in
 *            it-trends-board "PyTorch FlexAttention 도입 분석", section 2)
 *   DOCS   : doc(b,i) == doc(b,j), documents given as cumulative boundaries
 *            (aegloslab "3.7 어텐션 II" section 3.7.6)
 *   flags combine by AND.  Decode: j < lens[b] (section 3.7.4 of the same
 *   textbook chapter: one new query against the cached keys).
 *
 * GQA: query head h reads KV head h / (Hq / Hkv) (contiguous groups; the
 * same chapter, section 3.7.5).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORACLE_CAUSAL 1
#define ORACLE_WINDOW 2
#define ORACLE_DOCS 4
#define ORACLE_SOFTCAP 8
#define ORACLE_ALIBI 16

static double widen_bf16(uint16_t bits)
{
    uint32_t u = (uint32_t)bits << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

typedef struct {
    const uint16_t *q, *k, *v;
    const int64_t *qs, *ks, *vs; /* element strides of b, h, n; d stride 1 */
    int B, Hq, Hkv, N, d;
    int flags;
    int64_t wl, wr;
    double softcap;
    const int32_t *doc_offsets; /* [B][doc_stride], padded with N */
    int doc_stride;
    double scale;
    const double *alibi_slopes; /* [Hq], with ORACLE_ALIBI */
} fwd_problem;

/* Index of the document holding token i: the number of interior boundaries
 * at or below i. */
static int doc_of(const fwd_problem *p, int b, int i)
{
    const int32_t *off = p->doc_offsets + (int64_t)b * p->doc_stride;
    int t, n = 0;
    for (t = 1; t < p->doc_stride; ++t)
        if (off[t] <= i)
            ++n;
    return n;
}

static int visible(const fwd_problem *p, int b, int i, int j)
{
    if ((p->flags & ORACLE_CAUSAL) && j > i)
        return 0;
    if ((p->flags & ORACLE_WINDOW) &&
        ((int64_t)j < (int64_t)i - p->wl || (int64_t)j > (int64_t)i + p->wr))
        return 0;
    if ((p->flags & ORACLE_DOCS) && doc_of(p, b, i) != doc_of(p, b, j))
        return 0;
    return 1;
}

/* Steps 3-5 on one materialised score row s[0..n). */
static void softmax_and_mix(const double *s, int n, const uint16_t *vbase,
                            int64_t vrow_stride, int d, double *o, double *lse,
                            double *prow)
{
    double m = -INFINITY, sum = 0.0;
    int j, t;
    for (j = 0; j < n; ++j)
        if (s[j] > m)
            m = s[j];
    for (t = 0; t < d; ++t)
        o[t] = 0.0;
    if (m == -INFINITY) {
        *lse = -INFINITY;
        if (prow)
            for (j = 0; j < n; ++j)
                prow[j] = 0.0;
        return;
    }
    for (j = 0; j < n; ++j)
        sum += exp(s[j] - m);
    for (j = 0; j < n; ++j) {
        double pj = exp(s[j] - m) / sum;
        if (prow)
            prow[j] = pj;
        if (pj != 0.0) {
            const uint16_t *vj = vbase + (int64_t)j * vrow_stride;
            for (t = 0; t < d; ++t)
                o[t] += pj * widen_bf16(vj[t]);
        }
    }
    *lse = m + log(sum);
}

static void fwd_row(const fwd_problem *p, int b, int h, int i, double *srow,
                    double *o, double *lse, double *prow)
{
    int hk = h / (p->Hq / p->Hkv);
    const uint16_t *qi = p->q + b * p->qs[0] + h * p->qs[1] + (int64_t)i * p->qs[2];
    const uint16_t *kb = p->k + b * p->ks[0] + hk * p->ks[1];
    const uint16_t *vb = p->v + b * p->vs[0] + hk * p->vs[1];
    int j, t;
    for (j = 0; j < p->N; ++j) {
        if (!visible(p, b, i, j)) {
            srow[j] = -INFINITY;
            continue;
        }
        const uint16_t *kj = kb + (int64_t)j * p->ks[2];
        double dot = 0.0;
        for (t = 0; t < p->d; ++t)
            dot += widen_bf16(qi[t]) * widen_bf16(kj[t]);
        double sc = p->scale * dot;
        if (p->flags & ORACLE_ALIBI)
            sc -= p->alibi_slopes[h] * fabs((double)i - (double)j);
        if (p->flags & ORACLE_SOFTCAP)
            sc = p->softcap * tanh(sc / p->softcap);
        srow[j] = sc;
    }
    softmax_and_mix(srow, p->N, vb, p->vs[2], p->d, o, lse, prow);
}

int oracle_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/*
 * Forward attention on selected rows.
 *   rows: nrows triples (b, h, i); NULL means every row in (b, h, i) order.
 *   out_o [nrows][d], out_lse [nrows], out_p [nrows][N] (may be NULL).
 * Returns 0, or -1 on invalid arguments.
 */
int oracle_fwd(const uint16_t *q, const int64_t *q_strides, const uint16_t *k,
               const int64_t *k_strides, const uint16_t *v,
               const int64_t *v_strides, int B, int Hq, int Hkv, int N, int d,
               int flags, int64_t window_left, int64_t window_right,
               double softcap, const int32_t *doc_offsets, int doc_stride,
               double scale, int64_t nrows, const int32_t *rows, double *out_o,
               double *out_lse, double *out_p, const double *alibi_slopes)
{
    fwd_problem p;
    int64_t total = (int64_t)B * Hq * N;
    if (B < 0 || Hq <= 0 || Hkv <= 0 || Hq % Hkv || N < 0 || d <= 0)
        return -1;
    if ((flags & ORACLE_DOCS) && (!doc_offsets || doc_stride < 2))
        return -1;
    if ((flags & ORACLE_SOFTCAP) && !(softcap > 0.0))
        return -1;
    if ((flags & ORACLE_ALIBI) && !alibi_slopes)
        return -1;
    if (!rows)
        nrows = total;
    p.alibi_slopes = alibi_slopes;
    p.q = q; p.k = k; p.v = v;
    p.qs = q_strides; p.ks = k_strides; p.vs = v_strides;
    p.B = B; p.Hq = Hq; p.Hkv = Hkv; p.N = N; p.d = d;
    p.flags = flags; p.wl = window_left; p.wr = window_right;
    p.softcap = softcap; p.doc_offsets = doc_offsets; p.doc_stride = doc_stride;
    p.scale = scale;

#pragma omp parallel
    {
        double *srow = (double *)malloc(sizeof(double) * (size_t)(N > 0 ? N : 1));
        int64_t r;
#pragma omp for schedule(dynamic, 4)
        for (r = 0; r < nrows; ++r) {
            int b, h, i;
            if (rows) {
                b = rows[3 * r]; h = rows[3 * r + 1]; i = rows[3 * r + 2];
            } else {
                b = (int)(r / ((int64_t)Hq * N));
                h = (int)((r / N) % Hq);
                i = (int)(r % N);
            }
            fwd_row(&p, b, h, i, srow, out_o + r * d, out_lse + r,
                    out_p ? out_p + r * (int64_t)N : NULL);
        }
        free(srow);
    }
    return 0;
}

/*
 * Decode: one query per (b, hq) against keys j < lens[b] of the cache.
 *   q [B][Hq][d] contiguous; caches with element strides (b, h, t).
 *   out_o [B][Hq][d], out_lse [B][Hq].
 */
int oracle_decode(const uint16_t *q, const uint16_t *kc, const int64_t *k_strides,
                  const uint16_t *vc, const int64_t *v_strides,
                  const int32_t *lens, int B, int Hq, int Hkv, int T, int d,
                  double scale, double *out_o, double *out_lse)
{
    int64_t r;
    if (B < 0 || Hq <= 0 || Hkv <= 0 || Hq % Hkv || T < 0 || d <= 0)
        return -1;
    for (r = 0; r < B; ++r)
        if (lens[r] < 0 || lens[r] > T)
            return -1;
#pragma omp parallel
    {
        double *srow = (double *)malloc(sizeof(double) * (size_t)(T > 0 ? T : 1));
#pragma omp for schedule(dynamic, 1)
        for (r = 0; r < (int64_t)B * Hq; ++r) {
            int b = (int)(r / Hq), h = (int)(r % Hq);
            int hk = h / (Hq / Hkv);
            const uint16_t *qi = q + r * d;
            const uint16_t *kb = kc + b * k_strides[0] + hk * k_strides[1];
            const uint16_t *vb = vc + b * v_strides[0] + hk * v_strides[1];
            int n = lens[b], j, t;
            for (j = 0; j < n; ++j) {
                const uint16_t *kj = kb + (int64_t)j * k_strides[2];
                double dot = 0.0;
                for (t = 0; t < d; ++t)
                    dot += widen_bf16(qi[t]) * widen_bf16(kj[t]);
                srow[j] = scale * dot;
            }
            softmax_and_mix(srow, n, vb, v_strides[2], d, out_o + r * d,
                            out_lse + r, NULL);
        }
        free(srow);
    }
    return 0;
}

/*
 * Backward of the forward above (gradients of a loss through O), fp64.
 * For every query row i of (b, h), with the row's scores s (scaled, masked,
 * soft-capped) and probabilities P recomputed from q, k, v:
 *   dP_ij = dO_i . v_j,  D_i = sum_j P_ij dP_ij  (= dO_i . O_i),
 *   dS_ij = P_ij (dP_ij - D_i)                   (softmax backward),
 *   dU_ij = dS_ij * (1 - (s_ij / c)^2)           (soft cap: d c tanh(u/c) / du;
 *                                                 dU = dS without a cap),
 *   dq_i += scale * sum_j dU_ij k_j,
 *   dk_j += scale * dU_ij q_i,   dv_j += P_ij dO_i,
 * where k_j, v_j belong to KV head h / (Hq / Hkv), so the dk and dv of a KV
 * head sum over its query heads.  These are the gradients the recomputation
 * strategy of youngju.dev "FlashAttention 논문 분석" (section "Recomputation
 * 전략") evaluates from the saved row statistics; here they follow from the
 * definition directly (the chain rule through softmax and the matrix
 * products).  Masked keys have P = 0, hence zero gradient.
 *   dout [B][Hq][N][d] contiguous bf16 bits; outputs contiguous fp64:
 *   out_dq [B][Hq][N][d], out_dk / out_dv [B][Hkv][N][d].
 * Returns 0, or -1 on invalid arguments.
 */
int oracle_bwd(const uint16_t *q, const int64_t *q_strides, const uint16_t *k,
               const int64_t *k_strides, const uint16_t *v,
               const int64_t *v_strides, const uint16_t *dout, int B, int Hq,
               int Hkv, int N, int d, int flags, int64_t window_left,
               int64_t window_right, double softcap,
               const int32_t *doc_offsets, int doc_stride, double scale,
               double *out_dq, double *out_dk, double *out_dv)
{
    fwd_problem p;
    int64_t unit;
    if (B < 0 || Hq <= 0 || Hkv <= 0 || Hq % Hkv || N < 0 || d <= 0)
        return -1;
    if ((flags & ORACLE_DOCS) && (!doc_offsets || doc_stride < 2))
        return -1;
    if ((flags & ORACLE_SOFTCAP) && !(softcap > 0.0))
        return -1;
    p.q = q; p.k = k; p.v = v;
    p.qs = q_strides; p.ks = k_strides; p.vs = v_strides;
    p.B = B; p.Hq = Hq; p.Hkv = Hkv; p.N = N; p.d = d;
    p.flags = flags; p.wl = window_left; p.wr = window_right;
    p.softcap = softcap; p.doc_offsets = doc_offsets; p.doc_stride = doc_stride;
    p.scale = scale;
    p.alibi_slopes = NULL;
    if (flags & ORACLE_ALIBI)
        return -1; /* the gradient oracle covers the forward without the bias */
    memset(out_dq, 0, sizeof(double) * (size_t)B * Hq * N * d);
    memset(out_dk, 0, sizeof(double) * (size_t)B * Hkv * N * d);
    memset(out_dv, 0, sizeof(double) * (size_t)B * Hkv * N * d);

    /* One work unit per (b, KV head): it owns that head's dk and dv. */
#pragma omp parallel
    {
        size_t nn = (size_t)(N > 0 ? N : 1);
        double *srow = (double *)malloc(sizeof(double) * nn);
        double *prow = (double *)malloc(sizeof(double) * nn);
        double *o = (double *)malloc(sizeof(double) * (size_t)d);
#pragma omp for schedule(dynamic, 1)
        for (unit = 0; unit < (int64_t)B * Hkv; ++unit) {
            int b = (int)(unit / Hkv), hk = (int)(unit % Hkv);
            int group = Hq / Hkv, h, i, j, t;
            const uint16_t *kb = k + b * k_strides[0] + hk * k_strides[1];
            const uint16_t *vb = v + b * v_strides[0] + hk * v_strides[1];
            double *dkb = out_dk + ((int64_t)b * Hkv + hk) * N * d;
            double *dvb = out_dv + ((int64_t)b * Hkv + hk) * N * d;
            for (h = hk * group; h < (hk + 1) * group; ++h) {
                for (i = 0; i < N; ++i) {
                    double lse, dsum = 0.0;
                    const uint16_t *qi = q + b * q_strides[0] + h * q_strides[1] + (int64_t)i * q_strides[2];
                    const uint16_t *doi = dout + (((int64_t)b * Hq + h) * N + i) * d;
                    double *dqi = out_dq + (((int64_t)b * Hq + h) * N + i) * d;
                    fwd_row(&p, b, h, i, srow, o, &lse, prow);
                    if (lse == -INFINITY)
                        continue; /* no visible key: O = 0 does not depend on the inputs */
                    for (t = 0; t < d; ++t)
                        dsum += widen_bf16(doi[t]) * o[t];
                    for (j = 0; j < N; ++j) {
                        double dp = 0.0, du;
                        const uint16_t *kj = kb + (int64_t)j * k_strides[2];
                        const uint16_t *vj = vb + (int64_t)j * v_strides[2];
                        if (prow[j] == 0.0)
                            continue;
                        for (t = 0; t < d; ++t)
                            dp += widen_bf16(doi[t]) * widen_bf16(vj[t]);
                        du = prow[j] * (dp - dsum);
                        if (flags & ORACLE_SOFTCAP) {
                            double r = srow[j] / softcap;
                            du *= 1.0 - r * r;
                        }
                        for (t = 0; t < d; ++t) {
                            dqi[t] += scale * du * widen_bf16(kj[t]);
                            dkb[(int64_t)j * d + t] += scale * du * widen_bf16(qi[t]);
                            dvb[(int64_t)j * d + t] += prow[j] * widen_bf16(doi[t]);
                        }
                    }
                }
            }
        }
        free(srow);
        free(prow);
        free(o);
    }
    return 0;
}
