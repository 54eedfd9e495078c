/*
 * Drives every entry point of oracle/rr_oracle.c on small seeded inputs
 * (ragged L, several S, B, d and G) and through its argument checks, for a
 * build under AddressSanitizer and UndefinedBehaviorSanitizer.  Prints "ok"
 * and exits 0 when every call returns the expected status and the results
 * satisfy their basic invariants; any sanitizer report aborts the run.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

int rro_pool_keys(const uint16_t *K, int L, int Hkv, int d, int S, double *Kbar);
int rro_stride_scores(const uint16_t *Q, const uint16_t *K, int L, int Hq, int Hkv, int d, int S,
                      int h, int i, double *s);
int rro_stride_score_rows(const uint16_t *Q, const uint16_t *K, int L, int Hq, int Hkv, int d,
                          int S, const int32_t *rows, int nrows, double *out);
int rro_block_scores(const uint16_t *Q, const uint16_t *K, int L, int Hq, int Hkv, int d, int B,
                     int S, const int32_t *rows, int nrows, double *A);
int rro_xattn_stride_scores(const uint16_t *Q, const uint16_t *K, int L, int Hq, int Hkv, int d,
                            int S, int average, int h, int i, double *x);
int rro_xattn_block_scores(const uint16_t *Q, const uint16_t *K, int L, int Hq, int Hkv, int d,
                           int B, int S, int average, const int32_t *rows, int nrows, double *A);
int rro_rescue_scores(const uint16_t *Q, const uint16_t *K, int L, int Hq, int Hkv, int d, int B,
                      double *A);
int rro_select(const double *A, const int32_t *Irow, int nrows, int nb, double tau, uint8_t *keep,
               int32_t *count, double *cbefore);
int rro_attention(const uint16_t *Q, const uint16_t *K, const uint16_t *V, int L, int Hq, int Hkv,
                  int d, int B, const uint8_t *mask, const int32_t *toks, int n, double *O);

static uint64_t state = 0x9E3779B97F4A7C15ull;
static double uniform(void) {
    state ^= state << 13;
    state ^= state >> 7;
    state ^= state << 17;
    return (double)(state >> 11) / 9007199254740992.0;
}
/* bf16 pattern of a value in [-2, 2) (truncated, enough for inputs). */
static uint16_t bf16_of(double x) {
    float f = (float)x;
    uint32_t u;
    memcpy(&u, &f, 4);
    return (uint16_t)(u >> 16);
}
static uint16_t *random_bf16(size_t n) {
    uint16_t *p = malloc(n * sizeof(uint16_t));
    for (size_t i = 0; i < n; ++i) p[i] = bf16_of(4.0 * uniform() - 2.0);
    return p;
}

static int failures = 0;
#define CHECK(cond)                                                        \
    do {                                                                   \
        if (!(cond)) {                                                     \
            fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #cond); \
            ++failures;                                                    \
        }                                                                  \
    } while (0)

static void run_shape(int L, int Hq, int Hkv, int d, int B, int S) {
    const int nb = (L + B - 1) / B, ns = L / S, c = B / S;
    uint16_t *Q = random_bf16((size_t)L * Hq * d), *K = random_bf16((size_t)L * Hkv * d);
    uint16_t *V = random_bf16((size_t)L * Hkv * d);

    double *Kbar = malloc(sizeof(double) * (size_t)Hkv * ns * d);
    CHECK(rro_pool_keys(K, L, Hkv, d, S, Kbar) == 0);

    double *s = malloc(sizeof(double) * ns);
    CHECK(rro_stride_scores(Q, K, L, Hq, Hkv, d, S, Hq - 1, ns - 1, s) == 0);
    int32_t rows2[4] = {0, 0, Hq - 1, ns - 1};
    double *s2 = malloc(sizeof(double) * (1 + ns));
    CHECK(rro_stride_score_rows(Q, K, L, Hq, Hkv, d, S, rows2, 2, s2) == 0);
    CHECK(memcmp(s2 + 1, s, sizeof(double) * ns) == 0);

    const int nrows = Hq * nb;
    int32_t *rows = malloc(sizeof(int32_t) * 2 * nrows), *Irow = malloc(sizeof(int32_t) * nrows);
    for (int h = 0; h < Hq; ++h)
        for (int I = 0; I < nb; ++I) {
            rows[2 * (h * nb + I)] = h;
            rows[2 * (h * nb + I) + 1] = I;
            Irow[h * nb + I] = I;
        }
    double *A = malloc(sizeof(double) * (size_t)nrows * nb);
    CHECK(rro_block_scores(Q, K, L, Hq, Hkv, d, B, S, rows, nrows, A) == 0);
    for (int r = 0; r < nrows; ++r) {
        const int I = Irow[r];
        const int cI = (I == nb - 1) ? ns - I * c : c;
        double w = 0.0;
        for (int J = 0; J < nb; ++J) w += A[(size_t)r * nb + J];
        CHECK(fabs(w - cI) < 1e-9 * cI);
    }
    uint8_t *keep = malloc((size_t)nrows * nb);
    int32_t *count = malloc(sizeof(int32_t) * nrows);
    double *cb = malloc(sizeof(double) * (size_t)nrows * nb);
    CHECK(rro_select(A, Irow, nrows, nb, 0.9, keep, count, cb) == 0);
    for (int r = 0; r < nrows; ++r) CHECK(count[r] >= 1 && count[r] <= Irow[r] + 1);

    if (c >= 8 && c <= 32) {
        double *x = malloc(sizeof(double) * ns);
        CHECK(rro_xattn_stride_scores(Q, K, L, Hq, Hkv, d, S, 1, 0, ns - 1, x) == 0);
        CHECK(rro_xattn_block_scores(Q, K, L, Hq, Hkv, d, B, S, 0, rows, nrows, A) == 0);
        free(x);
    }
    double *Ar = malloc(sizeof(double) * (size_t)Hq * nb * nb);
    CHECK(rro_rescue_scores(Q, K, L, Hq, Hkv, d, B, Ar) == 0);

    int32_t toks[6] = {0, 0, Hq - 1, L - 1, Hq / 2, L / 2};
    double *O = malloc(sizeof(double) * 3 * d);
    CHECK(rro_attention(Q, K, V, L, Hq, Hkv, d, B, keep, toks, 3, O) == 0);
    for (int i = 0; i < 3 * d; ++i) CHECK(isfinite(O[i]));

    /* Argument checks: each must fail cleanly. */
    CHECK(rro_pool_keys(NULL, L, Hkv, d, S, Kbar) != 0);
    if (S > 1) CHECK(rro_pool_keys(K, L + 1, Hkv, d, S, Kbar) != 0);         /* L % S */
    CHECK(rro_stride_scores(Q, K, L, Hq, Hkv, d, S, Hq, 0, s) != 0);
    CHECK(rro_stride_scores(Q, K, L, Hq, Hkv, d, S, 0, ns, s) != 0);
    int32_t bad[2] = {0, ns};
    CHECK(rro_stride_score_rows(Q, K, L, Hq, Hkv, d, S, bad, 1, s2) != 0);
    int32_t badrow[2] = {Hq, 0};
    CHECK(rro_block_scores(Q, K, L, Hq, Hkv, d, B, S, badrow, 1, A) != 0);
    if (Hkv > 1) CHECK(rro_block_scores(Q, K, L, Hq + 1, Hkv, d, B, S, rows, 1, A) != 0);  /* Hq % Hkv */
    int32_t badtok[2] = {0, L};
    CHECK(rro_attention(Q, K, V, L, Hq, Hkv, d, B, keep, badtok, 1, O) != 0);

    free(Q); free(K); free(V); free(Kbar); free(s); free(s2); free(rows); free(Irow); free(A);
    free(keep); free(count); free(cb); free(Ar); free(O);
}

int main(void) {
    run_shape(192, 4, 2, 16, 64, 8);    /* ragged: 3 blocks, the last one full */
    run_shape(200, 4, 1, 16, 64, 8);    /* short last block (8 tokens) */
    run_shape(136, 6, 3, 32, 64, 4);    /* G = 2, ragged */
    run_shape(256, 7, 1, 16, 128, 16);  /* G = 7 */
    run_shape(96, 2, 2, 8, 32, 1);      /* S = 1 */
    run_shape(128, 2, 1, 16, 64, 64);   /* one stride per block */
    if (failures) {
        fprintf(stderr, "%d checks failed\n", failures);
        return 1;
    }
    printf("ok\n");
    return 0;
}
