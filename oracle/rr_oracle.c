/*
 * rr_oracle.c -- CPU oracle for the RRAttention sparse-prefill path.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may link, load or
 * call this file; only the test suite, the smoke check and the CPU-baseline
 * leg of the benchmark do.  It shares no code, header, table or helper with
 * the GPU library.
 *
 * Plain loops in IEEE double precision, no fast-math, no FMA contraction
 * (built with -ffp-contract=off).  Every sum runs in ascending index order.
 * OpenMP only distributes independent rows; each row is written by exactly
 * one thread, so results do not depend on the thread count.
 *
 * Sources (the web pages on RRAttention and on XAttention):
 *  [RR-sum]  RRAttention summary page (research.elamur.ai), "Summary" and
 *            "Key points": one query is scored in each stride of S tokens,
 *            the sampled offset rotates from head to head, scores are pooled
 *            per stride (O(L^2/S^2) estimation), blocks are kept by an
 *            adaptive Top-tau rule; defaults B=128, S=8; stride-level softmax.
 *  [RR-abs]  RRAttention abstract (arXiv 2602.05853, quoted on the digest and
 *            citation-map pages): rotating query positions across heads
 *            within each stride, stride-level aggregation, Top-tau selection,
 *            block-sparse attention over the kept blocks.
 *  [RR-dig]  RRAttention digest page, "method details", framework steps 1-4:
 *            split into strides, heads take turns sampling, attention between
 *            sampled queries and keys, aggregation per stride.
 *  [XA-tb]   XAttention review page, section "threshold block selection",
 *            formal definition of find_blocks: the smallest set of blocks
 *            whose summed attention probability reaches tau; its steps 1-2
 *            (antidiagonal sums per S x S sub-block, softmax over the sums).
 *  [RBS-abs] RBS-Attention page, abstract and method summary: centroid base
 *            branch, rescue branch from the maximum key-block radius,
 *            independent thresholds, masks combined.
 *  [XA-is]   XAttention review page, "importance prediction": elements are
 *            picked along the antidiagonal of each sub-block with stride S
 *            and their sum stands for the block's importance.
 *
 * Readings where the pages are silent (each is also listed in the design
 * notes of the repository):
 *  - key side of a stride: the mean of its S keys (E1);
 *  - rotation: query head h samples offset h mod S inside every stride (E2);
 *  - stride-level causality: stride i sees strides j <= i (E3);
 *  - scale 1/sqrt(d) (E2, E6);
 *  - stride -> block pooling: sum of the stride probabilities (E4);
 *  - Top-tau per (query head, query block-row), ">=" not ">", ties broken
 *    by the smaller key-block index, tau >= 1 keeps every causal block (E5);
 *  - query head h reads kv-head h / (Hq/Hkv) (E2, E6).
 *
 * Pins: every function here is checked by tests that do not re-type its
 * formula: S=1 reduction to exact block attention mass, constant-key closed
 * form, stride-mean construction, sampled-row probing, brute-force subset
 * enumeration, and scaled_dot_product_attention in float64.
 *
 * Layouts: Q [L][Hq][d], K and V [L][Hkv][d], as bf16 bit patterns (uint16).
 * L % S == 0 and B % S == 0 are required; L % B may be nonzero (the last
 * block is short).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* Error codes of the oracle entry points. */
#define RRO_OK 0
#define RRO_E_ARG 1
#define RRO_E_NOMEM 2

/* Exact widening of a bf16 bit pattern to double. */
static double bf16_value(uint16_t bits)
{
    uint32_t u = (uint32_t)bits << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

static int shape_ok(int L, int Hq, int Hkv, int d, int B, int S)
{
    if (L <= 0 || Hq <= 0 || Hkv <= 0 || d <= 0 || B <= 0 || S <= 0) return 0;
    if (Hq % Hkv != 0) return 0;
    if (B % S != 0) return 0;
    if (L % S != 0) return 0;
    return 1;
}

void rro_set_threads(int n)
{
#ifdef _OPENMP
    if (n > 0) omp_set_num_threads(n);
#else
    (void)n;
#endif
}

int rro_get_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/*
 * E1 -- stride key pooling [RR-sum "scores are pooled per stride"; RR-abs
 * "stride-level aggregation"].  Kbar[g][j][k] = (1/S) sum_{t<S} K[jS+t][g][k]
 * for every stride j < L/S.  Reading: the pooled key of a stride is the mean
 * of its S keys, so q.Kbar_j is the mean of the S token logits of stride j.
 */
int rro_pool_keys(const uint16_t *K, int L, int Hkv, int d, int S, double *Kbar)
{
    if (!K || !Kbar || L <= 0 || Hkv <= 0 || d <= 0 || S <= 0 || L % S) return RRO_E_ARG;
    int ns = L / S;
    for (int g = 0; g < Hkv; ++g)
        for (int j = 0; j < ns; ++j)
            for (int k = 0; k < d; ++k) {
                double sum = 0.0;
                for (int t = 0; t < S; ++t)
                    sum += bf16_value(K[((size_t)(j * S + t) * Hkv + g) * d + k]);
                Kbar[((size_t)g * ns + j) * d + k] = sum / (double)S;
            }
    return RRO_OK;
}

/*
 * E2 -- round-robin sampled scoring for one stride row [RR-sum: one query per
 * stride, offset rotating with the head; RR-dig step 2: heads take turns].
 * Query head h uses token i*S + (h mod S) of stride i.  For j <= i:
 *   s[j] = (1/sqrt(d)) * sum_k Q[iS + h mod S][h][k] * Kbar[g(h)][j][k].
 * Each s[j] is accumulated over k in ascending order (the loop over k is
 * outermost so that the pass over j is a plain scaled vector add).
 * KbarT is the pooled key of kv-head g(h) stored transposed, [k][ns].
 */
static void stride_scores(const uint16_t *Q, const double *KbarT, int ns, int Hq,
                          int d, int S, int h, int i, double *s)
{
    int t = i * S + (h % S);
    const uint16_t *q = Q + ((size_t)t * Hq + h) * d;
    for (int j = 0; j <= i; ++j) s[j] = 0.0;
    for (int k = 0; k < d; ++k) {
        double qk = bf16_value(q[k]);
        const double *col = KbarT + (size_t)k * ns;
        for (int j = 0; j <= i; ++j) s[j] += qk * col[j];
    }
    double sigma = 1.0 / sqrt((double)d);
    for (int j = 0; j <= i; ++j) s[j] *= sigma;
}

/*
 * E3 -- causal stride-level softmax [RR-sum "Key points": the method's
 * softmax granularity is the stride].  p[j] = exp(s[j]-m) / sum_{j'<=i}
 * exp(s[j']-m), m = max_{j<=i} s[j]; strides after i get no probability.
 */
static void causal_softmax(double *s, int i)
{
    double m = s[0];
    for (int j = 1; j <= i; ++j)
        if (s[j] > m) m = s[j];
    double z = 0.0;
    for (int j = 0; j <= i; ++j) {
        s[j] = exp(s[j] - m);
        z += s[j];
    }
    for (int j = 0; j <= i; ++j) s[j] /= z;
}

/* Pooled keys of every kv-head transposed to [g][k][ns] for stride_scores. */
static double *pooled_keys_transposed(const uint16_t *K, int L, int Hkv, int d, int S)
{
    int ns = L / S;
    double *Kbar = (double *)malloc(sizeof(double) * (size_t)Hkv * ns * d);
    double *KbarT = (double *)malloc(sizeof(double) * (size_t)Hkv * ns * d);
    if (!Kbar || !KbarT) {
        free(Kbar);
        free(KbarT);
        return NULL;
    }
    rro_pool_keys(K, L, Hkv, d, S, Kbar);
    for (int g = 0; g < Hkv; ++g)
        for (int j = 0; j < ns; ++j)
            for (int k = 0; k < d; ++k)
                KbarT[((size_t)g * d + k) * ns + j] = Kbar[((size_t)g * ns + j) * d + k];
    free(Kbar);
    return KbarT;
}

/*
 * E2 alone, for tests: raw scores s[0..i] of stride row i of head h.
 */
int rro_stride_scores(const uint16_t *Q, const uint16_t *K, int L, int Hq, int Hkv,
                      int d, int S, int h, int i, double *s)
{
    if (!Q || !K || !s || !shape_ok(L, Hq, Hkv, d, S, S)) return RRO_E_ARG;
    int ns = L / S, G = Hq / Hkv;
    if (h < 0 || h >= Hq || i < 0 || i >= ns) return RRO_E_ARG;
    double *KbarT = pooled_keys_transposed(K, L, Hkv, d, S);
    if (!KbarT) return RRO_E_NOMEM;
    stride_scores(Q, KbarT + (size_t)(h / G) * d * ns, ns, Hq, d, S, h, i, s);
    free(KbarT);
    return RRO_OK;
}

/*
 * E2 for a list of stride rows, for tests: rows holds nrows pairs (h, i);
 * the scores s[0..i] of row r are written to out + sum_{r' < r} (i_r' + 1).
 * Same arithmetic as rro_stride_scores; the pooled keys are formed once.
 */
int rro_stride_score_rows(const uint16_t *Q, const uint16_t *K, int L, int Hq, int Hkv,
                          int d, int S, const int32_t *rows, int nrows, double *out)
{
    if (!Q || !K || !rows || !out || nrows < 0 || !shape_ok(L, Hq, Hkv, d, S, S)) return RRO_E_ARG;
    int ns = L / S, G = Hq / Hkv;
    size_t *off = (size_t *)malloc(sizeof(size_t) * (size_t)(nrows + 1));
    if (!off) return RRO_E_NOMEM;
    off[0] = 0;
    for (int r = 0; r < nrows; ++r) {
        int h = rows[2 * r], i = rows[2 * r + 1];
        if (h < 0 || h >= Hq || i < 0 || i >= ns) {
            free(off);
            return RRO_E_ARG;
        }
        off[r + 1] = off[r] + (size_t)i + 1;
    }
    double *KbarT = pooled_keys_transposed(K, L, Hkv, d, S);
    if (!KbarT) {
        free(off);
        return RRO_E_NOMEM;
    }
#pragma omp parallel for schedule(dynamic, 1)
    for (int r = 0; r < nrows; ++r) {
        int h = rows[2 * r], i = rows[2 * r + 1];
        stride_scores(Q, KbarT + (size_t)(h / G) * d * ns, ns, Hq, d, S, h, i, out + off[r]);
    }
    free(KbarT);
    free(off);
    return RRO_OK;
}

/*
 * E1-E4 -- block scores for a list of (head, query block-row) pairs
 * [RR-dig step 4 and RR-abs "stride-level aggregation"; B from RR-sum
 * "Key points"].  With c = B/S strides per block and c_I strides in block I
 * (c_I < c only for a short last block):
 *   A[h][I][J] = sum_{a < c_I} sum_{b < c, Jc+b <= Ic+a} P[h][Ic+a][Jc+b]
 * where P is the causal stride softmax of the sampled scores.  Each block-row
 * therefore sums to c_I.  rows holds nrows pairs (h, I); A is [nrows][nb]
 * with zeros for J > I.
 */
int rro_block_scores(const uint16_t *Q, const uint16_t *K, int L, int Hq, int Hkv,
                     int d, int B, int S, const int32_t *rows, int nrows, double *A)
{
    if (!Q || !K || !rows || !A || nrows < 0 || !shape_ok(L, Hq, Hkv, d, B, S)) return RRO_E_ARG;
    int ns = L / S, c = B / S, nb = (L + B - 1) / B, G = Hq / Hkv;
    for (int r = 0; r < nrows; ++r)
        if (rows[2 * r] < 0 || rows[2 * r] >= Hq || rows[2 * r + 1] < 0 || rows[2 * r + 1] >= nb)
            return RRO_E_ARG;
    double *KbarT = pooled_keys_transposed(K, L, Hkv, d, S);
    if (!KbarT) return RRO_E_NOMEM;
    int err = RRO_OK;
#pragma omp parallel
    {
        double *p = (double *)malloc(sizeof(double) * (size_t)ns);
        if (!p) {
#pragma omp atomic write
            err = RRO_E_NOMEM;
        }
#pragma omp for schedule(dynamic, 1)
        for (int r = 0; r < nrows; ++r) {
            if (!p) continue;
            int h = rows[2 * r], I = rows[2 * r + 1];
            double *Arow = A + (size_t)r * nb;
            for (int J = 0; J < nb; ++J) Arow[J] = 0.0;
            for (int a = 0; a < c; ++a) {
                int i = I * c + a;
                if (i >= ns) break;
                stride_scores(Q, KbarT + (size_t)(h / G) * d * ns, ns, Hq, d, S, h, i, p);
                causal_softmax(p, i);
                for (int j = 0; j <= i; ++j) Arow[j / c] += p[j];
            }
        }
        free(p);
    }
    free(KbarT);
    return err;
}

/*
 * X1 -- XAttention's antidiagonal stride scoring [XA-is: XAttention review
 * page, "importance prediction", and "threshold block selection" step 1].
 * Inside every S x S sub-block of the attention map the elements on the
 * antidiagonal (lower-left to upper-right) are summed as the sub-block's
 * importance.  Sub-block (i, j) spans query tokens iS..iS+S-1 and key tokens
 * jS..jS+S-1, so its antidiagonal pairs query iS+t with key jS+S-1-t.
 * Reading: the elements summed are the scaled logits (1/sqrt(d)) q.k (the
 * next step applies the softmax to the sums).  For j <= i:
 *   x[j] = (1/sqrt(d)) * sum_{t<S} sum_k Q[iS+t][h][k] * K[jS+S-1-t][g(h)][k]
 * summed over t, then k, in ascending order.  With average != 0 the sum is
 * divided by S (the mean antidiagonal logit, which keeps the softmax at the
 * temperature of single tokens), an alternative reading of the same step.
 * Kd is K widened to double, [L][Hkv][d]; qrow receives the S query rows of
 * stride i.
 */
static void xattn_stride_scores(const uint16_t *Q, const double *Kd, int Hq, int Hkv, int d,
                                int S, int average, int h, int i, double *qrow, double *x)
{
    int g = h / (Hq / Hkv);
    double sc = 1.0 / sqrt((double)d);
    if (average) sc /= (double)S;
    for (int t = 0; t < S; ++t)
        for (int k = 0; k < d; ++k)
            qrow[(size_t)t * d + k] = bf16_value(Q[((size_t)(i * S + t) * Hq + h) * d + k]);
    for (int j = 0; j <= i; ++j) {
        double acc = 0.0;
        for (int t = 0; t < S; ++t) {
            const double *kk = Kd + ((size_t)(j * S + S - 1 - t) * Hkv + g) * d;
            const double *q = qrow + (size_t)t * d;
            for (int k = 0; k < d; ++k) acc += q[k] * kk[k];
        }
        x[j] = sc * acc;
    }
}

static double *widen_keys(const uint16_t *K, int L, int Hkv, int d)
{
    size_t n = (size_t)L * Hkv * d;
    double *Kd = (double *)malloc(sizeof(double) * n);
    if (!Kd) return NULL;
    for (size_t e = 0; e < n; ++e) Kd[e] = bf16_value(K[e]);
    return Kd;
}

/* X1 alone, for tests: antidiagonal scores x[0..i] of stride row i, head h. */
int rro_xattn_stride_scores(const uint16_t *Q, const uint16_t *K, int L, int Hq, int Hkv,
                            int d, int S, int average, int h, int i, double *x)
{
    if (!Q || !K || !x || !shape_ok(L, Hq, Hkv, d, S, S)) return RRO_E_ARG;
    int ns = L / S;
    if (h < 0 || h >= Hq || i < 0 || i >= ns) return RRO_E_ARG;
    double *Kd = widen_keys(K, L, Hkv, d);
    double *qrow = (double *)malloc(sizeof(double) * (size_t)S * d);
    if (!Kd || !qrow) {
        free(Kd);
        free(qrow);
        return RRO_E_NOMEM;
    }
    xattn_stride_scores(Q, Kd, Hq, Hkv, d, S, average, h, i, qrow, x);
    free(Kd);
    free(qrow);
    return RRO_OK;
}

/*
 * X1 + E3 + E4 -- XAttention block scores [XA-tb steps 1-2: antidiagonal
 * sums, then a softmax over them; pooled to B x B blocks as for E4].  The
 * softmax runs over the causal strides j <= i of stride row i (E3) and its
 * probabilities are summed over the c x c sub-blocks of each block (E4), so
 * each block-row again sums to c_I.  Same row list and output layout as
 * rro_block_scores.
 */
int rro_xattn_block_scores(const uint16_t *Q, const uint16_t *K, int L, int Hq, int Hkv,
                           int d, int B, int S, int average, const int32_t *rows, int nrows,
                           double *A)
{
    if (!Q || !K || !rows || !A || nrows < 0 || !shape_ok(L, Hq, Hkv, d, B, S)) return RRO_E_ARG;
    int ns = L / S, c = B / S, nb = (L + B - 1) / B;
    for (int r = 0; r < nrows; ++r)
        if (rows[2 * r] < 0 || rows[2 * r] >= Hq || rows[2 * r + 1] < 0 || rows[2 * r + 1] >= nb)
            return RRO_E_ARG;
    double *Kd = widen_keys(K, L, Hkv, d);
    if (!Kd) return RRO_E_NOMEM;
    int err = RRO_OK;
#pragma omp parallel
    {
        double *p = (double *)malloc(sizeof(double) * (size_t)ns);
        double *qrow = (double *)malloc(sizeof(double) * (size_t)S * d);
        if (!p || !qrow) {
#pragma omp atomic write
            err = RRO_E_NOMEM;
        }
#pragma omp for schedule(dynamic, 1)
        for (int r = 0; r < nrows; ++r) {
            if (!p || !qrow) continue;
            int h = rows[2 * r], I = rows[2 * r + 1];
            double *Arow = A + (size_t)r * nb;
            for (int J = 0; J < nb; ++J) Arow[J] = 0.0;
            for (int a = 0; a < c; ++a) {
                int i = I * c + a;
                if (i >= ns) break;
                xattn_stride_scores(Q, Kd, Hq, Hkv, d, S, average, h, i, qrow, p);
                causal_softmax(p, i);
                for (int j = 0; j <= i; ++j) Arow[j / c] += p[j];
            }
        }
        free(p);
        free(qrow);
    }
    free(Kd);
    return err;
}

/*
 * R1 -- RBS-Attention's rescue branch [RBS-abs: RBS-Attention page, abstract
 * and method summary: a block centroid can hide one highly relevant key
 * among many irrelevant ones ("mean dilution"); a rescue branch uses the
 * maximum key-block radius to flag blocks at risk of underestimation, is
 * thresholded independently of the base branch, and its mask is combined
 * with the base mask].  Reading (the page gives no formula): with the
 * centroid kc_J of the keys of block J (kv-head g(h)), its radius
 * r_J = max_{n in J} ||K[n] - kc_J||_2, and the mean query qc_I of block I
 * (head h), the rescue logit is the largest logit qc_I can reach against a
 * key of block J (Cauchy-Schwarz):
 *   u[h][I][J] = (1/sqrt(d)) * (qc_I . kc_J + ||qc_I||_2 * r_J),  J <= I,
 * and the rescue scores are its softmax over J <= I (each row sums to 1),
 * ready for the same Top-tau rule (E5) with the rescue branch's own tau.
 * A short last block averages its real tokens only.  Out: A [Hq][nb][nb],
 * zeros for J > I.
 */
int rro_rescue_scores(const uint16_t *Q, const uint16_t *K, int L, int Hq, int Hkv, int d,
                      int B, double *A)
{
    if (!Q || !K || !A || !shape_ok(L, Hq, Hkv, d, B, 1)) return RRO_E_ARG;
    int nb = (L + B - 1) / B, G = Hq / Hkv;
    double *kc = (double *)calloc((size_t)Hkv * nb * d, sizeof(double));
    double *rad = (double *)calloc((size_t)Hkv * nb, sizeof(double));
    double *qc = (double *)calloc((size_t)Hq * nb * d, sizeof(double));
    if (!kc || !rad || !qc) {
        free(kc);
        free(rad);
        free(qc);
        return RRO_E_NOMEM;
    }
    for (int g = 0; g < Hkv; ++g)
        for (int J = 0; J < nb; ++J) {
            int n0 = J * B, n1 = (J + 1) * B < L ? (J + 1) * B : L;
            double *c = kc + ((size_t)g * nb + J) * d;
            for (int n = n0; n < n1; ++n)
                for (int k = 0; k < d; ++k) c[k] += bf16_value(K[((size_t)n * Hkv + g) * d + k]);
            for (int k = 0; k < d; ++k) c[k] /= (double)(n1 - n0);
            double r = 0.0;
            for (int n = n0; n < n1; ++n) {
                double s2 = 0.0;
                for (int k = 0; k < d; ++k) {
                    double e = bf16_value(K[((size_t)n * Hkv + g) * d + k]) - c[k];
                    s2 += e * e;
                }
                if (sqrt(s2) > r) r = sqrt(s2);
            }
            rad[(size_t)g * nb + J] = r;
        }
    for (int h = 0; h < Hq; ++h)
        for (int I = 0; I < nb; ++I) {
            int t0 = I * B, t1 = (I + 1) * B < L ? (I + 1) * B : L;
            double *c = qc + ((size_t)h * nb + I) * d;
            for (int t = t0; t < t1; ++t)
                for (int k = 0; k < d; ++k) c[k] += bf16_value(Q[((size_t)t * Hq + h) * d + k]);
            for (int k = 0; k < d; ++k) c[k] /= (double)(t1 - t0);
        }
    double sigma = 1.0 / sqrt((double)d);
#pragma omp parallel for schedule(dynamic, 1)
    for (int r = 0; r < Hq * nb; ++r) {
        int h = r / nb, I = r % nb, g = h / G;
        const double *q = qc + (size_t)r * d;
        double qn = 0.0;
        for (int k = 0; k < d; ++k) qn += q[k] * q[k];
        qn = sqrt(qn);
        double *Arow = A + (size_t)r * nb;
        double m = -INFINITY;
        for (int J = 0; J < nb; ++J) {
            if (J > I) {
                Arow[J] = 0.0;
                continue;
            }
            const double *c = kc + ((size_t)g * nb + J) * d;
            double dot = 0.0;
            for (int k = 0; k < d; ++k) dot += q[k] * c[k];
            Arow[J] = sigma * (dot + qn * rad[(size_t)g * nb + J]);
            if (Arow[J] > m) m = Arow[J];
        }
        double z = 0.0;
        for (int J = 0; J <= I; ++J) {
            Arow[J] = exp(Arow[J] - m);
            z += Arow[J];
        }
        for (int J = 0; J <= I; ++J) Arow[J] /= z;
    }
    free(kc);
    free(rad);
    free(qc);
    return RRO_OK;
}

/* Ordering of E5: larger block score first, then smaller block index. */
typedef struct {
    double a;
    int j;
} scored_block;

static int by_score_desc_then_index(const void *x, const void *y)
{
    const scored_block *u = (const scored_block *)x, *v = (const scored_block *)y;
    if (u->a > v->a) return -1;
    if (u->a < v->a) return 1;
    return (u->j > v->j) - (u->j < v->j);
}

/*
 * E5 -- adaptive Top-tau [RR-sum "Summary": blocks kept by a Top-tau rule;
 * XA-tb: the smallest set whose summed probability is at least tau].
 * For each row (block-row I of some head) with causal blocks J = 0..I:
 *   W = sum_J A[J]; order the blocks by (A desc, J asc) as pi_0, pi_1, ...;
 *   C_k = A[pi_0] + ... + A[pi_k];
 *   tau >= 1: keep every J <= I;
 *   else K* = min{k : C_k >= tau*W} (none: keep all); keep pi_0..pi_K*.
 * A greedy largest-first prefix reaches any mass with the fewest blocks, so
 * this is a minimum-cardinality set with mass >= tau*W.
 * Outputs per row: keep[nb] (1 = kept), count, and optionally
 * cbefore[nb] = (mass of the blocks ordered before J) / W for J <= I
 * (-1 for J > I), used to classify near-threshold differences.
 */
int rro_select(const double *A, const int32_t *Irow, int nrows, int nb, double tau,
               uint8_t *keep, int32_t *count, double *cbefore)
{
    if (!A || !Irow || !keep || !count || nrows < 0 || nb <= 0) return RRO_E_ARG;
    if (!(tau > 0.0)) return RRO_E_ARG;
    for (int r = 0; r < nrows; ++r)
        if (Irow[r] < 0 || Irow[r] >= nb) return RRO_E_ARG;
    int err = RRO_OK;
#pragma omp parallel
    {
        scored_block *ord = (scored_block *)malloc(sizeof(scored_block) * (size_t)nb);
        if (!ord) {
#pragma omp atomic write
            err = RRO_E_NOMEM;
        }
#pragma omp for schedule(dynamic, 16)
        for (int r = 0; r < nrows; ++r) {
            if (!ord) continue;
            const double *a = A + (size_t)r * nb;
            uint8_t *kp = keep + (size_t)r * nb;
            double *cb = cbefore ? cbefore + (size_t)r * nb : NULL;
            int n = Irow[r] + 1;
            double W = 0.0;
            for (int J = 0; J < n; ++J) W += a[J];
            for (int J = 0; J < nb; ++J) {
                kp[J] = 0;
                if (cb) cb[J] = -1.0;
            }
            for (int J = 0; J < n; ++J) {
                ord[J].a = a[J];
                ord[J].j = J;
            }
            qsort(ord, (size_t)n, sizeof(scored_block), by_score_desc_then_index);
            int kstar = -1;
            double C = 0.0;
            for (int k = 0; k < n; ++k) {
                if (cb) cb[ord[k].j] = C / W;
                C += ord[k].a;
                if (kstar < 0 && C >= tau * W) kstar = k;
            }
            if (tau >= 1.0 || kstar < 0) kstar = n - 1;
            for (int k = 0; k <= kstar; ++k) kp[ord[k].j] = 1;
            count[r] = kstar + 1;
        }
        free(ord);
    }
    return err;
}

/*
 * E6 -- causal block-sparse attention with GQA [RR-abs: attention computed
 * only on the kept blocks; scaled dot-product attention of "Attention is all
 * you need" (reference list of the RRAttention summary page); GQA: query
 * head h reads kv-head h / (Hq/Hkv)].  For token t in block I = t/B and head h:
 *   N = { n <= t : mask[h][I][n/B] };  l_n = (1/sqrt(d)) Q[t][h].K[n][g(h)];
 *   O[t][h] = sum_{n in N} softmax(l)_n V[n][g(h)].
 * mask is [Hq][nb][nb] (1 = keep).  toks holds n pairs (h, t); O is [n][d].
 * A query whose set N is empty gets a zero row (cannot happen for masks
 * produced by E5, which keep at least one causal block).
 */
int rro_attention(const uint16_t *Q, const uint16_t *K, const uint16_t *V, int L, int Hq,
                  int Hkv, int d, int B, const uint8_t *mask, const int32_t *toks, int n,
                  double *O)
{
    if (!Q || !K || !V || !mask || !toks || !O || n < 0) return RRO_E_ARG;
    if (L <= 0 || Hq <= 0 || Hkv <= 0 || d <= 0 || B <= 0 || Hq % Hkv) return RRO_E_ARG;
    for (int r = 0; r < n; ++r)
        if (toks[2 * r] < 0 || toks[2 * r] >= Hq || toks[2 * r + 1] < 0 || toks[2 * r + 1] >= L)
            return RRO_E_ARG;
    int nb = (L + B - 1) / B, G = Hq / Hkv;
    double sigma = 1.0 / sqrt((double)d);
    int err = RRO_OK;
#pragma omp parallel
    {
        double *l = (double *)malloc(sizeof(double) * (size_t)L);
        double *q = (double *)malloc(sizeof(double) * (size_t)d);
        if (!l || !q) {
#pragma omp atomic write
            err = RRO_E_NOMEM;
        }
#pragma omp for schedule(dynamic, 4)
        for (int r = 0; r < n; ++r) {
            if (!l || !q) continue;
            int h = toks[2 * r], t = toks[2 * r + 1], g = h / G, I = t / B;
            const uint8_t *mrow = mask + ((size_t)h * nb + I) * nb;
            double *o = O + (size_t)r * d;
            for (int k = 0; k < d; ++k) {
                q[k] = bf16_value(Q[((size_t)t * Hq + h) * d + k]);
                o[k] = 0.0;
            }
            double m = -INFINITY;
            for (int nn = 0; nn <= t; ++nn) {
                if (!mrow[nn / B]) continue;
                const uint16_t *kr = K + ((size_t)nn * Hkv + g) * d;
                double dot = 0.0;
                for (int k = 0; k < d; ++k) dot += q[k] * bf16_value(kr[k]);
                l[nn] = sigma * dot;
                if (l[nn] > m) m = l[nn];
            }
            if (m == -INFINITY) continue;
            double z = 0.0;
            for (int nn = 0; nn <= t; ++nn) {
                if (!mrow[nn / B]) continue;
                double p = exp(l[nn] - m);
                z += p;
                const uint16_t *vr = V + ((size_t)nn * Hkv + g) * d;
                for (int k = 0; k < d; ++k) o[k] += p * bf16_value(vr[k]);
            }
            for (int k = 0; k < d; ++k) o[k] /= z;
        }
        free(l);
        free(q);
    }
    return err;
}
