/* Sanitizer driver for the CPU oracle (test infrastructure): runs every
 * oracle entry point on small seeded inputs -- ragged and empty sequences,
 * partial last blocks, top-k above the number of past blocks, both key-conv
 * modes, the BLASST skip, the row-sampled variants and the backward -- so
 * an AddressSanitizer / UBSan / ThreadSanitizer build reports any
 * out-of-bounds access, use of freed memory, undefined behaviour or data
 * race.  Numerical results are checked elsewhere; here every call must
 * return 0 and every output must be finite where it is defined. */
#include <math.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

int moba_oracle_key_conv(const float *k, const float *w, int H, int d, int W, int mode,
                         int round_bf16, const int *cu, int nseq, float *out, int nthreads);
int moba_oracle_total_blocks(const int *cu, int nseq, int B);
int moba_oracle_centroids(const float *k, int H, int d, int B, const int *cu, int nseq,
                          float *cent, int nthreads);
int moba_oracle_route(const float *q, const float *cent, int H, int d, int B, int K,
                      const int *cu, int nseq, int *idx, double *gap_a, double *gap_b,
                      unsigned char *exempt, int nthreads);
int moba_oracle_attend(const float *q, const float *k, const float *v, const int *idx, int H,
                       int d, int B, int K, const int *cu, int nseq, double scale, double *o,
                       double *lse, int nthreads);
int moba_oracle_attend_blasst(const float *q, const float *k, const float *v, const int *idx,
                              int H, int d, int B, int K, const int *cu, int nseq, double scale,
                              double log_lambda, const unsigned char *keep,
                              const unsigned long long *flip, double tau, double *o,
                              double *lse, unsigned long long *near, unsigned char *keep_out,
                              int nthreads);
int moba_oracle_route_rows(const float *q, const float *cent, int H, int d, int B, int K,
                           const int *cu, int nseq, const long long *rows, int nrows, int *idx,
                           double *gap_a, double *gap_b, unsigned char *exempt);
int moba_oracle_route_scores(const float *q, const float *cent, int H, int d, int B,
                             const int *cu, int nseq, const long long *rows, int nrows,
                             int nmax, double *scores);
int moba_oracle_attend_rows(const float *q, const float *k, const float *v, const int *idx,
                            int H, int d, int B, int K, const int *cu, int nseq, double scale,
                            const long long *rows, int nrows, double *o, double *lse);
int moba_oracle_attend_bwd(const float *q, const float *k, const float *v, const int *idx,
                           const unsigned char *keep, const float *dout, int H, int d, int B, int K, const int *cu,
                           int nseq, double scale, const unsigned char *qsel,
                           const unsigned char *kbsel, double *dq, double *dk, double *dv,
                           int nthreads);
int moba_oracle_key_conv_bwd(const float *k, const float *w, const float *g, int H, int d,
                             int W, int mode, const int *cu, int nseq, double *dk, double *dw,
                             int nthreads);

static unsigned long long rng_state = 88172645463325252ull;
static float urand(void)
{
    rng_state ^= rng_state << 13;
    rng_state ^= rng_state >> 7;
    rng_state ^= rng_state << 17;
    return (float)((rng_state >> 11) * (1.0 / 9007199254740992.0)) * 2.0f - 1.0f;
}
static float *fill(size_t n)
{
    float *p = (float *)malloc(sizeof(float) * (n ? n : 1));
    for (size_t i = 0; i < n; ++i) p[i] = urand();
    return p;
}
static int fails = 0;
#define CHECK(call)                                                              \
    do {                                                                         \
        int rc_ = (call);                                                        \
        if (rc_ != 0) { fprintf(stderr, "FAIL %s -> %d\n", #call, rc_); ++fails; } \
    } while (0)

static void finite_or_fail(const double *x, size_t n, const char *what)
{
    for (size_t i = 0; i < n; ++i)
        if (!isfinite(x[i])) { fprintf(stderr, "FAIL non-finite %s[%zu]\n", what, i); ++fails; return; }
}

static void run_case(const int *cu, int nseq, int H, int d, int B, int K, int W, int nthreads)
{
    const int T = cu[nseq];
    const size_t rows = (size_t)T * H;
    float *q = fill(rows * d), *k = fill(rows * d), *v = fill(rows * d), *g = fill(rows * d);
    float *w = fill((size_t)W * H * d);
    float *kc = (float *)malloc(sizeof(float) * (rows * d + 1));
    for (int mode = 0; mode < 2; ++mode)
        CHECK(moba_oracle_key_conv(k, w, H, d, W, mode, mode, cu, nseq, kc, nthreads));
    double *dk = (double *)malloc(sizeof(double) * (rows * d + 1));
    double *dw = (double *)malloc(sizeof(double) * ((size_t)W * H * d + 1));
    for (int mode = 0; mode < 2; ++mode)
        CHECK(moba_oracle_key_conv_bwd(k, w, g, H, d, W, mode, cu, nseq, dk, dw, nthreads));

    const int nb = moba_oracle_total_blocks(cu, nseq, B);
    float *cent = (float *)malloc(sizeof(float) * ((size_t)nb * H * d + 1));
    CHECK(moba_oracle_centroids(kc, H, d, B, cu, nseq, cent, nthreads));
    int *idx = (int *)malloc(sizeof(int) * (rows * K + 1));
    double *ga = (double *)malloc(sizeof(double) * (rows + 1));
    double *gb = (double *)malloc(sizeof(double) * (rows + 1));
    unsigned char *ex = (unsigned char *)malloc(rows + 1);
    CHECK(moba_oracle_route(q, cent, H, d, B, K, cu, nseq, idx, ga, gb, ex, nthreads));

    double *o = (double *)malloc(sizeof(double) * (rows * d + 1));
    double *lse = (double *)malloc(sizeof(double) * (rows + 1));
    CHECK(moba_oracle_attend(q, kc, v, idx, H, d, B, K, cu, nseq, 0.0, o, lse, nthreads));
    finite_or_fail(o, rows * d, "o");

    /* BLASST: a mid lambda, an explicit keep mask, and flips of near decisions */
    unsigned char *keep = (unsigned char *)malloc(rows * K + 1);
    unsigned long long *flip = (unsigned long long *)calloc(rows + 1, sizeof(unsigned long long));
    unsigned long long *near = (unsigned long long *)malloc(sizeof(unsigned long long) * (rows + 1));
    for (size_t i = 0; i < rows * K; ++i) keep[i] = (unsigned char)(i % 3 != 1);
    for (size_t i = 0; i < rows; ++i) flip[i] = (i % 5 == 0) ? ~0ull : 0ull;
    unsigned char *kept = (unsigned char *)malloc(rows * K + 1);
    CHECK(moba_oracle_attend_blasst(q, kc, v, idx, H, d, B, K, cu, nseq, 0.0, log(0.01), NULL,
                                    NULL, 1e-4, o, lse, near, kept, nthreads));
    CHECK(moba_oracle_attend_blasst(q, kc, v, idx, H, d, B, K, cu, nseq, 0.0, log(0.5), keep,
                                    flip, 1e-2, o, lse, near, NULL, nthreads));

    /* row-sampled variants: every third (token, head) row */
    long long *rs = (long long *)malloc(sizeof(long long) * (rows + 1));
    int nr = 0;
    for (size_t r = 0; r < rows; r += 3) rs[nr++] = (long long)r;
    int nmax = 1;
    for (int s = 0; s < nseq; ++s) {
        int n = (cu[s + 1] - cu[s] + B - 1) / B;
        if (n > nmax) nmax = n;
    }
    /* route_rows / attend_rows write full-size arrays at the listed rows */
    int *idx2 = (int *)malloc(sizeof(int) * (rows * K + 1));
    memcpy(idx2, idx, sizeof(int) * rows * K);
    double *sc = (double *)malloc(sizeof(double) * ((size_t)nr * nmax + 1));
    CHECK(moba_oracle_route_rows(q, cent, H, d, B, K, cu, nseq, rs, nr, idx2, ga, gb, ex));
    CHECK(moba_oracle_route_scores(q, cent, H, d, B, cu, nseq, rs, nr, nmax, sc));
    CHECK(moba_oracle_attend_rows(q, kc, v, idx2, H, d, B, K, cu, nseq, 0.0, rs, nr, o, lse));

    /* backward on every row and on a selection of query rows / key blocks */
    double *dq = (double *)malloc(sizeof(double) * (rows * d + 1));
    double *dk2 = (double *)malloc(sizeof(double) * (rows * d + 1));
    double *dv = (double *)malloc(sizeof(double) * (rows * d + 1));
    CHECK(moba_oracle_attend_bwd(q, kc, v, idx, NULL, g, H, d, B, K, cu, nseq, 0.0, NULL, NULL,
                                 dq, dk2, dv, nthreads));
    finite_or_fail(dq, rows * d, "dq");
    unsigned char *qsel = (unsigned char *)malloc(rows + 1);
    unsigned char *kbsel = (unsigned char *)malloc((size_t)nb * H + 1);
    for (size_t i = 0; i < rows; ++i) qsel[i] = (unsigned char)(i % 2);
    for (size_t i = 0; i < (size_t)nb * H; ++i) kbsel[i] = (unsigned char)(i % 3 == 0);
    CHECK(moba_oracle_attend_bwd(q, kc, v, idx, NULL, g, H, d, B, K, cu, nseq, 0.5, qsel, kbsel,
                                 dq, dk2, dv, nthreads));
    /* the BLASST backward on the decisions of the lambda = 0.01 forward, and
       on a mask that drops every block of some rows */
    CHECK(moba_oracle_attend_bwd(q, kc, v, idx, kept, g, H, d, B, K, cu, nseq, 0.0, NULL, NULL,
                                 dq, dk2, dv, nthreads));
    finite_or_fail(dq, rows * d, "dq (blasst)");
    for (size_t i = 0; i < rows * K; ++i) keep[i] = (unsigned char)(i % 7 != 0 && i % 5 != 2);
    for (size_t i = 0; i < rows * K && i < 4 * (size_t)K; ++i) keep[i] = 0;
    CHECK(moba_oracle_attend_bwd(q, kc, v, idx, keep, g, H, d, B, K, cu, nseq, 0.0, NULL, NULL,
                                 dq, dk2, dv, nthreads));
    finite_or_fail(dq, rows * d, "dq (dropped rows)");

    free(q); free(k); free(v); free(g); free(w); free(kc); free(dk); free(dw); free(cent);
    free(idx); free(ga); free(gb); free(ex); free(o); free(lse); free(keep); free(flip);
    free(near); free(kept); free(rs); free(idx2); free(sc); free(dq); free(dk2); free(dv); free(qsel);
    free(kbsel);
}

int main(int argc, char **argv)
{
    const int nthreads = argc > 1 ? atoi(argv[1]) : 3;
    /* one sequence, a partial last block, k above the past blocks early on */
    const int cu1[2] = {0, 77};
    run_case(cu1, 1, 2, 8, 16, 4, 3, nthreads);
    /* ragged varlen with an empty and a one-token sequence */
    const int cu2[6] = {0, 40, 40, 41, 100, 133};
    run_case(cu2, 5, 3, 16, 8, 3, 2, nthreads);
    /* k = 1 (own block only) and W = 1 */
    const int cu3[3] = {0, 64, 96};
    run_case(cu3, 2, 1, 8, 16, 1, 1, nthreads);
    /* long enough for every rank of k = 8 and near-ties in the BLASST pass */
    const int cu4[2] = {0, 300};
    run_case(cu4, 1, 2, 16, 16, 8, 4, nthreads);
    if (fails) { fprintf(stderr, "%d failures\n", fails); return 1; }
    printf("ok\n");
    return 0;
}
