/*
 * moba_oracle.c -- plain, slow, obviously-correct CPU reference of the
 * Mixture of Block Attention (MoBA) forward pass and of the gradients of its
 * attention step.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may link, load or
 * call this file; only the tests, the package's smoke check and the
 * benchmark's CPU-baseline leg do.  It shares no code, header or table with
 * the HIP library.
 *
 * Source of every step: "Optimizing Mixture of Block Attention" (Xiao, Guo,
 * Mazaheri, Han), summary pages:
 *   - task definition ("Definizione del Compito"): O = softmax(QK^T/sqrt(d))V
 *     restricted to the selected blocks; N keys split into n = N/B blocks;
 *     each query keeps its top-k blocks;
 *   - statistical model ("Architettura del Modello Statistico", router score
 *     equation): block score s_j = q . kbar_j, kbar_j the mean of the keys of
 *     block j;
 *   - key convolution ("Progettazione della Convoluzione delle Chiavi
 *     (Appendice B)", formal-form equation): depthwise causal conv over the
 *     sequence, one filter per channel, left padding; the page's form adds
 *     the input back after a SiLU.
 * Causal rules not on the pages (own block always kept, future blocks
 * masked, token-causal inside the own block, lower block index wins ties) are
 * the plainest reading of a decoder model and are stated at each step.
 *
 * Precision: all sums and dot products accumulate in fp64, sequentially, in
 * the order written.  Exception (a quantised result): the key convolution's
 * output is rounded to the I/O dtype, so it is computed in fp32 with fmaf in
 * a fixed order (taps from the oldest to the newest token) exactly as the
 * kernel computes it, and both sides take the rounding decision in the same
 * precision.  Build with -ffp-contract=off and without -ffast-math.
 *
 * Tensors are fp32 arrays [tokens][heads][d] holding the exact values of the
 * I/O dtype (bf16 inputs are decoded to fp32 by the caller).  Sequences are
 * given as cu[0..nseq] over the token axis; each sequence is independent.
 *
 * Parity status: every function here is pinned by CPU tests (see the
 * oracle tests): conv against a library conv1d in fp64 and special cases,
 * centroids against a library mean, routing against brute-force argsort and
 * hand-computed integer cases, attention against library SDPA (dense and
 * explicit-mask) and closed-form special cases, the attention backward
 * against the library's autograd of explicit-mask SDPA, central differences
 * of the forward, and closed-form invariants.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* ---------- bf16 round-to-nearest-even (IEEE definition) ---------- */
static float round_to_bf16(float x)
{
    uint32_t u;
    memcpy(&u, &x, 4);
    if ((u & 0x7f800000u) == 0x7f800000u) {          /* inf / nan */
        if (u & 0x007fffffu) u |= 0x00400000u;        /* quiet nan */
        u &= 0xffff0000u;
    } else {
        uint32_t lsb = (u >> 16) & 1u;
        u = (u + 0x7fffu + lsb) & 0xffff0000u;
    }
    float r;
    memcpy(&r, &u, 4);
    return r;
}

/* ---------- a tiny work-sharing pool over (sequence, head) jobs ---------- */
typedef void (*job_fn)(void *ctx, int job);
typedef struct {
    job_fn fn;
    void *ctx;
    int njobs;
    volatile int next;
    pthread_mutex_t mu;
} pool_t;

static void *pool_worker(void *arg)
{
    pool_t *p = (pool_t *)arg;
    for (;;) {
        pthread_mutex_lock(&p->mu);
        int j = p->next++;
        pthread_mutex_unlock(&p->mu);
        if (j >= p->njobs) break;
        p->fn(p->ctx, j);
    }
    return NULL;
}

static void run_jobs(job_fn fn, void *ctx, int njobs, int nthreads)
{
    if (nthreads < 1) nthreads = 1;
    if (nthreads > njobs) nthreads = njobs;
    pool_t p;
    p.fn = fn;
    p.ctx = ctx;
    p.njobs = njobs;
    p.next = 0;
    pthread_mutex_init(&p.mu, NULL);
    if (nthreads <= 1) {
        pool_worker(&p);
    } else {
        pthread_t *th = (pthread_t *)malloc(sizeof(pthread_t) * (size_t)nthreads);
        for (int i = 0; i < nthreads; ++i) pthread_create(&th[i], NULL, pool_worker, &p);
        for (int i = 0; i < nthreads; ++i) pthread_join(th[i], NULL);
        free(th);
    }
    pthread_mutex_destroy(&p.mu);
}

static int ceil_div(int a, int b) { return (a + b - 1) / b; }

/* =====================================================================
 * Step 1: key convolution (summary page, Appendice B, formal form).
 *   conv_t = sum_{l=0}^{W-1} w[h][c][l] * k_{t-l}   (zero before the
 *            sequence start: causal, left padded, per sequence)
 *   mode 0 ("plain"):        k'_t = conv_t
 *   mode 1 (page's form):    k'_t = k_t + SiLU(conv_t)
 * The tap sum is fp32 fmaf from the oldest tap (l = W-1) to l = 0, started
 * at +0; taps before the sequence start are skipped.  k' is rounded to the
 * I/O dtype (bf16 RNE when round_bf16 != 0).
 * ===================================================================== */
typedef struct {
    const float *k, *w;
    float *out;
    const int *cu;
    int H, d, W, mode, round_bf16;
} conv_ctx;

static void conv_job(void *vctx, int job)
{
    conv_ctx *c = (conv_ctx *)vctx;
    int s = job / c->H, h = job % c->H;
    int t0 = c->cu[s], t1 = c->cu[s + 1];
    for (int t = t0; t < t1; ++t) {
        for (int ch = 0; ch < c->d; ++ch) {
            const float *wv = c->w + ((size_t)h * c->d + ch) * c->W;
            float acc = 0.0f;
            for (int l = c->W - 1; l >= 0; --l) {
                if (t - l < t0) continue;
                float x = c->k[((size_t)(t - l) * c->H + h) * c->d + ch];
                acc = fmaf(wv[l], x, acc);
            }
            float r;
            if (c->mode == 0) {
                r = acc;
            } else {
                double a = (double)acc;
                double silu = a / (1.0 + exp(-a));
                r = (float)((double)c->k[((size_t)t * c->H + h) * c->d + ch] + silu);
            }
            if (c->round_bf16) r = round_to_bf16(r);
            c->out[((size_t)t * c->H + h) * c->d + ch] = r;
        }
    }
}

int moba_oracle_key_conv(const float *k, const float *w, int H, int d, int W,
                         int mode, int round_bf16, const int *cu, int nseq,
                         float *out, int nthreads)
{
    if (W < 1 || (mode != 0 && mode != 1)) return 1;
    conv_ctx c = {k, w, out, cu, H, d, W, mode, round_bf16};
    run_jobs(conv_job, &c, nseq * H, nthreads);
    return 0;
}

/* =====================================================================
 * Step 2: block centroids (summary page, statistical model, router-score
 * equation: kbar_j = (1/B) sum_{k in block j} k).
 * Block j of a sequence covers local tokens [jB, min((j+1)B, L)); a final
 * partial block is averaged over the keys it holds.  The sum is fp64 in
 * token order, divided once, rounded once to fp32.
 * Output rows are [global block][H][d] with blocks sequence-major.
 * ===================================================================== */
typedef struct {
    const float *k;
    float *cent;
    const int *cu;
    const int *boff;
    int H, d, B;
} cent_ctx;

static void cent_job(void *vctx, int job)
{
    cent_ctx *c = (cent_ctx *)vctx;
    int s = job / c->H, h = job % c->H;
    int t0 = c->cu[s], L = c->cu[s + 1] - c->cu[s];
    int n = ceil_div(L, c->B);
    double *acc = (double *)malloc(sizeof(double) * (size_t)c->d);
    for (int j = 0; j < n; ++j) {
        int a = j * c->B, b = (j + 1) * c->B < L ? (j + 1) * c->B : L;
        for (int ch = 0; ch < c->d; ++ch) acc[ch] = 0.0;
        for (int u = a; u < b; ++u)
            for (int ch = 0; ch < c->d; ++ch)
                acc[ch] += (double)c->k[((size_t)(t0 + u) * c->H + h) * c->d + ch];
        float *dst = c->cent + ((size_t)(c->boff[s] + j) * c->H + h) * c->d;
        for (int ch = 0; ch < c->d; ++ch) dst[ch] = (float)(acc[ch] / (double)(b - a));
    }
    free(acc);
}

static int *block_offsets(const int *cu, int nseq, int B)
{
    int *boff = (int *)malloc(sizeof(int) * (size_t)(nseq + 1));
    boff[0] = 0;
    for (int s = 0; s < nseq; ++s) boff[s + 1] = boff[s] + ceil_div(cu[s + 1] - cu[s], B);
    return boff;
}

int moba_oracle_total_blocks(const int *cu, int nseq, int B)
{
    int tot = 0;
    for (int s = 0; s < nseq; ++s) tot += ceil_div(cu[s + 1] - cu[s], B);
    return tot;
}

int moba_oracle_centroids(const float *k, int H, int d, int B, const int *cu,
                          int nseq, float *cent, int nthreads)
{
    if (B < 1) return 1;
    int *boff = block_offsets(cu, nseq, B);
    cent_ctx c = {k, cent, cu, boff, H, d, B};
    run_jobs(cent_job, &c, nseq * H, nthreads);
    free(boff);
    return 0;
}

/* =====================================================================
 * Step 3-4: router scores and causal top-k selection.
 *   s_{t,j} = q_t . kbar_j  (router-score equation), fp64, sequential over
 *   channels, for the past blocks j < i = floor(t_local / B) only (future
 *   blocks are masked).  The own block i is always kept and does not
 *   compete.  Of the i past blocks, the first m = min(k-1, i) in the total
 *   order (score descending, block index ascending) are kept.
 *   Output row: ascending block ids (local to the sequence), own block
 *   included, padded with -1 to length k.
 *   Near-tie record (for i >= k): a = (k-1)-th best past score, b = k-th
 *   best; exempt = |a-b| <= 1e-5 * max(|a|,|b|,1e-30).
 * ===================================================================== */
typedef struct {
    const float *q, *cent;
    int *idx;
    double *gap_a, *gap_b;
    unsigned char *exempt;
    const int *cu, *boff;
    int H, d, B, K;
} route_ctx;

/* strict "a ranks before b": higher score first, lower index on ties */
static int ranks_before(double sa, int ja, double sb, int jb)
{
    if (sa > sb) return 1;
    if (sa < sb) return 0;
    return ja < jb;
}

static int cmp_int(const void *a, const void *b)
{
    int x = *(const int *)a, y = *(const int *)b;
    return (x > y) - (x < y);
}

/* router scores of one query (token t_local `tl` of sequence s, head h)
 * against its i past blocks, written to sc[0..i-1]; returns i */
static int score_past(const route_ctx *c, int s, int h, int tl, double *sc)
{
    size_t t = (size_t)(c->cu[s] + tl);
    int i = tl / c->B;
    const float *qv = c->q + (t * c->H + h) * c->d;
    for (int j = 0; j < i; ++j) {
        const float *cv = c->cent + ((size_t)(c->boff[s] + j) * c->H + h) * c->d;
        double acc = 0.0;
        for (int ch = 0; ch < c->d; ++ch) acc = acc + (double)qv[ch] * (double)cv[ch];
        sc[j] = acc;
    }
    return i;
}

/* one query: token t_local `tl` of sequence s, head h; sc/order scratch of
 * n doubles/ints, row scratch of K ints */
static void route_one(route_ctx *c, int s, int h, int tl, double *sc, int *order, int *row)
{
    int t0 = c->cu[s];
    size_t t = (size_t)(t0 + tl);
    int i = score_past(c, s, h, tl, sc);
    /* selection sort of the first m+1 places in the total order */
    int m = (c->K - 1) < i ? (c->K - 1) : i;
    int need = (m + 1) < i ? (m + 1) : i;
    for (int j = 0; j < i; ++j) order[j] = j;
    for (int p = 0; p < need; ++p) {
        int best = p;
        for (int r = p + 1; r < i; ++r)
            if (ranks_before(sc[order[r]], order[r], sc[order[best]], order[best])) best = r;
        int tmp = order[p]; order[p] = order[best]; order[best] = tmp;
    }
    for (int p = 0; p < m; ++p) row[p] = order[p];
    row[m] = i;
    qsort(row, (size_t)(m + 1), sizeof(int), cmp_int);
    for (int p = m + 1; p < c->K; ++p) row[p] = -1;
    int *dst = c->idx + (t * c->H + h) * c->K;
    for (int p = 0; p < c->K; ++p) dst[p] = row[p];
    size_t r = t * c->H + h;
    if (c->gap_a) {
        if (i >= c->K && c->K >= 2) {
            double a = sc[order[c->K - 2]], b = sc[order[c->K - 1]];
            double mx = fabs(a) > fabs(b) ? fabs(a) : fabs(b);
            if (mx < 1e-30) mx = 1e-30;
            c->gap_a[r] = a;
            c->gap_b[r] = b;
            c->exempt[r] = (fabs(a - b) <= 1e-5 * mx) ? 1 : 0;
        } else {
            c->gap_a[r] = NAN;
            c->gap_b[r] = NAN;
            c->exempt[r] = 0;
        }
    }
}

static void route_job(void *vctx, int job)
{
    route_ctx *c = (route_ctx *)vctx;
    int s = job / c->H, h = job % c->H;
    int L = c->cu[s + 1] - c->cu[s];
    int n = ceil_div(L, c->B);
    double *sc = (double *)malloc(sizeof(double) * (size_t)(n > 0 ? n : 1));
    int *order = (int *)malloc(sizeof(int) * (size_t)(n > 0 ? n : 1));
    int *row = (int *)malloc(sizeof(int) * (size_t)c->K);
    for (int tl = 0; tl < L; ++tl) route_one(c, s, h, tl, sc, order, row);
    free(sc);
    free(order);
    free(row);
}

int moba_oracle_route(const float *q, const float *cent, int H, int d, int B,
                      int K, const int *cu, int nseq, int *idx, double *gap_a,
                      double *gap_b, unsigned char *exempt, int nthreads)
{
    if (B < 1 || K < 1) return 1;
    int *boff = block_offsets(cu, nseq, B);
    route_ctx c = {q, cent, idx, gap_a, gap_b, exempt, cu, boff, H, d, B, K};
    run_jobs(route_job, &c, nseq * H, nthreads);
    free(boff);
    return 0;
}

/* =====================================================================
 * Step 5: attention over the selected blocks (task definition:
 * O = softmax(QK^T / sqrt(d)) V restricted to the selected blocks).
 *   Key set of query t (block i): every key of each listed past block
 *   j (0 <= j < i) plus the keys u <= t of its own block i (token-causal).
 *   Entries equal to -1 are padding; entries > i are ignored (future).
 *   z_u = scale * (q_t . k_u) in fp64; M = max z; l = sum exp(z - M);
 *   O_t = sum exp(z_u - M) v_u / l;  LSE_t = M + ln l.
 * The own block is always attended, listed or not.
 * ===================================================================== */
typedef struct {
    const float *q, *k, *v;
    const int *idx;
    double *o, *lse;
    const int *cu;
    int H, d, B, K;
    double scale;
} attn_ctx;

static void attend_one(attn_ctx *c, int s, int h, int tl, double *z, int *keys)
{
    int t0 = c->cu[s], L = c->cu[s + 1] - c->cu[s];
    size_t t = (size_t)(t0 + tl);
    int i = tl / c->B;
    const int *row = c->idx + (t * c->H + h) * c->K;
    int nk = 0;
    /* listed past blocks, in row order */
    for (int p = 0; p < c->K; ++p) {
        int j = row[p];
        if (j < 0 || j >= i) continue;
        for (int u = j * c->B; u < (j + 1) * c->B && u < L; ++u) keys[nk++] = u;
    }
    /* own block, causal */
    for (int u = i * c->B; u <= tl; ++u) keys[nk++] = u;
    const float *qv = c->q + (t * c->H + h) * c->d;
    double M = -INFINITY;
    for (int e = 0; e < nk; ++e) {
        const float *kv = c->k + ((size_t)(t0 + keys[e]) * c->H + h) * c->d;
        double acc = 0.0;
        for (int ch = 0; ch < c->d; ++ch) acc = acc + (double)qv[ch] * (double)kv[ch];
        z[e] = c->scale * acc;
        if (z[e] > M) M = z[e];
    }
    double l = 0.0;
    for (int e = 0; e < nk; ++e) l += exp(z[e] - M);
    double *ov = c->o + (t * c->H + h) * c->d;
    for (int ch = 0; ch < c->d; ++ch) ov[ch] = 0.0;
    for (int e = 0; e < nk; ++e) {
        double p = exp(z[e] - M);
        const float *vv = c->v + ((size_t)(t0 + keys[e]) * c->H + h) * c->d;
        for (int ch = 0; ch < c->d; ++ch) ov[ch] += p * (double)vv[ch];
    }
    for (int ch = 0; ch < c->d; ++ch) ov[ch] /= l;
    if (c->lse) c->lse[t * c->H + h] = M + log(l);
}

static void attn_job(void *vctx, int job)
{
    attn_ctx *c = (attn_ctx *)vctx;
    int s = job / c->H, h = job % c->H;
    int L = c->cu[s + 1] - c->cu[s];
    int maxkeys = c->K * c->B + c->B;
    double *z = (double *)malloc(sizeof(double) * (size_t)maxkeys);
    int *keys = (int *)malloc(sizeof(int) * (size_t)maxkeys);
    for (int tl = 0; tl < L; ++tl) attend_one(c, s, h, tl, z, keys);
    free(z);
    free(keys);
}

int moba_oracle_attend(const float *q, const float *k, const float *v,
                       const int *idx, int H, int d, int B, int K,
                       const int *cu, int nseq, double scale, double *o,
                       double *lse, int nthreads)
{
    if (B < 1 || K < 1) return 1;
    if (!(scale > 0.0)) scale = 1.0 / sqrt((double)d);
    attn_ctx c = {q, k, v, idx, o, lse, cu, H, d, B, K, scale};
    run_jobs(attn_job, &c, nseq * H, nthreads);
    return 0;
}

/* =====================================================================
 * Step 5, BLASST variant ("BLASST: Dynamic BLocked Attention Sparsity via
 * Softmax Thresholding", section "Meccanismo di Pruning"): the query's
 * blocks are visited in ascending order, as an online softmax visits its
 * key blocks, with a running maximum M of the attended scores; a block
 * whose own maximum m~ satisfies m~ - M < ln(lambda), 0 <= lambda <= 1, is
 * skipped -- its keys take no part in the softmax.  The first block is
 * never skipped.  Blocks: the listed past blocks (0 <= j < i, ascending, as in
 * step 5), then the own block i with its causal keys u <= t.
 *   log_lambda = -inf keeps every block (step 5 exactly).
 *   keep (optional, uint8 [rows][K]): instead of the rule, block of slot p
 *   is attended iff keep[row][p] != 0; the own block is slot p with
 *   idx == i, or kept when no slot lists it.
 *   near (optional, uint64 per row): bit b set where the decision on the
 *   b-th visited block lies within tau * max(1, |M|) of the threshold (a
 *   decision that a different rounding of the scores may take the other
 *   way); flip (optional, uint64 per row): such near decisions whose bit is
 *   set are taken the other way (the later ones still follow the rule).
 *   keep_out (optional, uint8 [rows][K]): the decisions taken, per slot:
 *   1 where the slot's block was attended (the own block's slot included),
 *   0 for skipped blocks and for slots that name no block of the row.
 * ===================================================================== */
typedef struct {
    attn_ctx a;
    double log_lambda, tau;
    const unsigned char *keep;
    const unsigned long long *flip;
    unsigned long long *near;
    unsigned char *keep_out;
} blasst_ctx;

static void blasst_one(blasst_ctx *c, int s, int h, int tl, double *z, int *keys,
                       int *kept, int *bstart, int *bslot)
{
    attn_ctx *a = &c->a;
    int t0 = a->cu[s], L = a->cu[s + 1] - a->cu[s];
    size_t t = (size_t)(t0 + tl);
    size_t r = t * a->H + h;
    int i = tl / a->B;
    const int *row = a->idx + r * a->K;
    /* blocks in visiting order with their key ranges in keys[] */
    int nb = 0, nk = 0, own_slot = -1;
    for (int p = 0; p < a->K; ++p) {
        int j = row[p];
        if (j == i) own_slot = p;
        if (j < 0 || j >= i) continue;
        bstart[nb] = nk;
        bslot[nb++] = p;
        for (int u = j * a->B; u < (j + 1) * a->B && u < L; ++u) keys[nk++] = u;
    }
    bstart[nb] = nk;
    bslot[nb++] = own_slot;
    for (int u = i * a->B; u <= tl; ++u) keys[nk++] = u;
    bstart[nb] = nk;
    const float *qv = a->q + r * a->d;
    for (int e = 0; e < nk; ++e) {
        const float *kv = a->k + ((size_t)(t0 + keys[e]) * a->H + h) * a->d;
        double acc = 0.0;
        for (int ch = 0; ch < a->d; ++ch) acc = acc + (double)qv[ch] * (double)kv[ch];
        z[e] = a->scale * acc;
    }
    /* block maxima and the skip decisions, in visiting order */
    double M = -INFINITY;
    unsigned long long near = 0;
    const unsigned long long flip = c->flip ? c->flip[r] : 0;
    for (int b = 0; b < nb; ++b) {
        double m = -INFINITY;
        for (int e = bstart[b]; e < bstart[b + 1]; ++e) if (z[e] > m) m = z[e];
        int kb;
        if (c->keep) {
            kb = bslot[b] < 0 ? 1 : c->keep[r * a->K + bslot[b]] != 0;
        } else {
            kb = 1;
            if (M > -INFINITY && m - M < c->log_lambda) kb = 0;
            if (M > -INFINITY && c->log_lambda > -INFINITY) {
                double mx = fabs(M) > 1.0 ? fabs(M) : 1.0;
                if (fabs(m - M - c->log_lambda) <= c->tau * mx) {
                    near |= 1ull << b;
                    if ((flip >> b) & 1ull) kb = !kb;
                }
            }
        }
        /* the running maximum is that of the attended scores */
        if (kb && m > M) M = m;
        kept[b] = kb;
    }
    if (c->near) c->near[r] = near;
    if (c->keep_out) {
        unsigned char *ko = c->keep_out + r * a->K;
        for (int p = 0; p < a->K; ++p) ko[p] = 0;
        for (int b = 0; b < nb; ++b)
            if (bslot[b] >= 0) ko[bslot[b]] = (unsigned char)(kept[b] != 0);
    }
    /* softmax over the kept blocks' keys */
    double Mk = -INFINITY;
    for (int b = 0; b < nb; ++b) {
        if (!kept[b]) continue;
        for (int e = bstart[b]; e < bstart[b + 1]; ++e) if (z[e] > Mk) Mk = z[e];
    }
    double l = 0.0;
    double *ov = a->o + r * a->d;
    for (int ch = 0; ch < a->d; ++ch) ov[ch] = 0.0;
    for (int b = 0; b < nb; ++b) {
        if (!kept[b]) continue;
        for (int e = bstart[b]; e < bstart[b + 1]; ++e) {
            double p = exp(z[e] - Mk);
            l += p;
            const float *vv = a->v + ((size_t)(t0 + keys[e]) * a->H + h) * a->d;
            for (int ch = 0; ch < a->d; ++ch) ov[ch] += p * (double)vv[ch];
        }
    }
    for (int ch = 0; ch < a->d; ++ch) ov[ch] /= l;
    if (a->lse) a->lse[r] = Mk + log(l);
}

static void blasst_job(void *vctx, int job)
{
    blasst_ctx *c = (blasst_ctx *)vctx;
    int s = job / c->a.H, h = job % c->a.H;
    int L = c->a.cu[s + 1] - c->a.cu[s];
    int maxkeys = c->a.K * c->a.B + c->a.B;
    double *z = (double *)malloc(sizeof(double) * (size_t)maxkeys);
    int *keys = (int *)malloc(sizeof(int) * (size_t)maxkeys);
    int *kept = (int *)malloc(sizeof(int) * (size_t)(c->a.K + 2));
    int *bstart = (int *)malloc(sizeof(int) * (size_t)(c->a.K + 3));
    int *bslot = (int *)malloc(sizeof(int) * (size_t)(c->a.K + 2));
    for (int tl = 0; tl < L; ++tl) blasst_one(c, s, h, tl, z, keys, kept, bstart, bslot);
    free(z);
    free(keys);
    free(kept);
    free(bstart);
    free(bslot);
}

int moba_oracle_attend_blasst(const float *q, const float *k, const float *v,
                              const int *idx, int H, int d, int B, int K,
                              const int *cu, int nseq, double scale, double log_lambda,
                              const unsigned char *keep, const unsigned long long *flip,
                              double tau, double *o, double *lse, unsigned long long *near,
                              unsigned char *keep_out, int nthreads)
{
    if (B < 1 || K < 1 || K > 63) return 1;
    if (!(scale > 0.0)) scale = 1.0 / sqrt((double)d);
    blasst_ctx c = {{q, k, v, idx, o, lse, cu, H, d, B, K, scale}, log_lambda, tau, keep, flip,
                    near, keep_out};
    run_jobs(blasst_job, &c, nseq * H, nthreads);
    return 0;
}

/* =====================================================================
 * Row subsets (for sampled checks at sizes where the full oracle is too
 * slow): the same steps 3-4 / 5 for the listed (token, head) rows only.
 * rows[r] = token * H + head (global token index).  Outputs are written at
 * the rows' usual places in idx / o / lse; other rows are untouched.
 * ===================================================================== */
static int seq_of_token(const int *cu, int nseq, int t)
{
    int s = 0;
    while (s + 1 < nseq && cu[s + 1] <= t) ++s;
    return s;
}

/* Steps 3-4 for the listed rows only (row = token * H + head).  idx,
 * gap_a, gap_b and exempt are full-size ([tokens * H] rows) and only the
 * listed rows are written. */
int moba_oracle_route_rows(const float *q, const float *cent, int H, int d, int B,
                           int K, const int *cu, int nseq, const long long *rows,
                           int nrows, int *idx, double *gap_a, double *gap_b,
                           unsigned char *exempt)
{
    if (B < 1 || K < 1) return 1;
    int *boff = block_offsets(cu, nseq, B);
    route_ctx c = {q, cent, idx, gap_a, gap_b, exempt, cu, boff, H, d, B, K};
    int nmax = 1;
    for (int s = 0; s < nseq; ++s) {
        int n = ceil_div(cu[s + 1] - cu[s], B);
        if (n > nmax) nmax = n;
    }
    double *sc = (double *)malloc(sizeof(double) * (size_t)nmax);
    int *order = (int *)malloc(sizeof(int) * (size_t)nmax);
    int *row = (int *)malloc(sizeof(int) * (size_t)K);
    for (int r = 0; r < nrows; ++r) {
        int t = (int)(rows[r] / H), h = (int)(rows[r] % H);
        int s = seq_of_token(cu, nseq, t);
        route_one(&c, s, h, t - cu[s], sc, order, row);
    }
    free(sc);
    free(order);
    free(row);
    free(boff);
    return 0;
}

/* Step 3 alone for the listed rows: the fp64 router score of every past
 * block, scores[r * nmax + j] for j < i (the row's own block index), NaN
 * for j >= i.  nmax must be at least the longest sequence's block count.
 * Lets a test check that a selection differing from this oracle's is still
 * a valid tolerant top-(k-1) of the same scores. */
int moba_oracle_route_scores(const float *q, const float *cent, int H, int d, int B,
                             const int *cu, int nseq, const long long *rows, int nrows,
                             int nmax, double *scores)
{
    if (B < 1) return 1;
    int *boff = block_offsets(cu, nseq, B);
    route_ctx c = {q, cent, NULL, NULL, NULL, NULL, cu, boff, H, d, B, 1};
    for (int s = 0; s < nseq; ++s)
        if (ceil_div(cu[s + 1] - cu[s], B) > nmax) { free(boff); return 2; }
    for (int r = 0; r < nrows; ++r) {
        int t = (int)(rows[r] / H), h = (int)(rows[r] % H);
        int s = seq_of_token(cu, nseq, t);
        double *out = scores + (size_t)r * (size_t)nmax;
        int i = score_past(&c, s, h, t - cu[s], out);
        for (int j = i; j < nmax; ++j) out[j] = NAN;
    }
    free(boff);
    return 0;
}

/* Step 5 for the listed rows only: idx, o and lse are full-size ([tokens *
 * H] rows); only the listed rows of o and lse are written. */
int moba_oracle_attend_rows(const float *q, const float *k, const float *v,
                            const int *idx, int H, int d, int B, int K,
                            const int *cu, int nseq, double scale,
                            const long long *rows, int nrows, double *o,
                            double *lse)
{
    if (B < 1 || K < 1) return 1;
    if (!(scale > 0.0)) scale = 1.0 / sqrt((double)d);
    attn_ctx c = {q, k, v, idx, o, lse, cu, H, d, B, K, scale};
    int maxkeys = K * B + B;
    double *z = (double *)malloc(sizeof(double) * (size_t)maxkeys);
    int *keys = (int *)malloc(sizeof(int) * (size_t)maxkeys);
    for (int r = 0; r < nrows; ++r) {
        int t = (int)(rows[r] / H), h = (int)(rows[r] % H);
        int s = seq_of_token(cu, nseq, t);
        attend_one(&c, s, h, t - cu[s], z, keys);
    }
    free(z);
    free(keys);
    return 0;
}

/* =====================================================================
 * Backward of step 5: gradients of O with respect to q, k and v for a
 * fixed selection (summary page, "Backward Pass: Ricalcolo (Algoritmo 5)":
 * FlashAttention-2 style, the scores and probabilities are recomputed from
 * q and k instead of being stored).  The gradients are those of softmax
 * attention over the row's key set (listed past blocks + own block
 * causally, exactly as in step 5), with dO the gradient of the output:
 *   z_tu  = scale q_t . k_u,   P_tu = exp(z_tu - LSE_t)
 *   dv_u += P_tu dO_t
 *   dP_tu = dO_t . v_u
 *   D_t   = sum_u P_tu dP_tu
 *   dS_tu = P_tu (dP_tu - D_t)
 *   dq_t  = scale sum_u dS_tu k_u
 *   dk_u += scale dS_tu q_t
 * The block selection is piecewise constant in q and k, so nothing flows
 * through the router (its gradient is zero almost everywhere).
 * Subsets, for sampled checks at sizes where the whole backward is too
 * slow: qsel (uint8 per row t*H+h, NULL = all) picks the rows whose dq is
 * written; kbsel (uint8 per (global block, head), NULL = all) picks the key
 * blocks whose dk / dv are written.  Unpicked outputs are left untouched;
 * picked dk / dv are overwritten with the sum over every row.
 * keep (optional, uint8 [rows][K]): the backward of the BLASST variant of
 * step 5 for fixed decisions (BLASST page, "Meccanismo di Pruning", and its
 * sparsity-aware training): slot p's block is in the key set iff
 * keep[row][p] != 0, the own block included (its slot is the one with
 * idx == i; a row that lists no own block keeps it), as in the BLASST
 * forward with an explicit keep.  The skip decisions are piecewise constant
 * in q and k, so, as for the router, nothing flows through them.
 * ===================================================================== */
typedef struct {
    const float *q, *k, *v, *dout;
    const int *idx;
    const unsigned char *keep;
    const unsigned char *qsel, *kbsel;
    double *dq, *dk, *dv;
    const int *cu, *boff;
    int H, d, B, K;
    double scale;
} bwd_ctx;

static void bwd_job(void *vctx, int job)
{
    bwd_ctx *c = (bwd_ctx *)vctx;
    int s = job / c->H, h = job % c->H;
    int t0 = c->cu[s], L = c->cu[s + 1] - t0;
    int d = c->d, H = c->H;
    int maxkeys = c->K * c->B + c->B;
    double *z = (double *)malloc(sizeof(double) * (size_t)maxkeys);
    double *dp = (double *)malloc(sizeof(double) * (size_t)maxkeys);
    int *keys = (int *)malloc(sizeof(int) * (size_t)maxkeys);
    /* the picked key rows of this (sequence, head) start from zero */
    for (int u = 0; u < L; ++u) {
        int g = c->boff[s] + u / c->B;
        if (c->kbsel && !c->kbsel[(size_t)g * H + h]) continue;
        double *dkr = c->dk + ((size_t)(t0 + u) * H + h) * d;
        double *dvr = c->dv + ((size_t)(t0 + u) * H + h) * d;
        for (int ch = 0; ch < d; ++ch) { dkr[ch] = 0.0; dvr[ch] = 0.0; }
    }
    for (int tl = 0; tl < L; ++tl) {
        size_t t = (size_t)(t0 + tl);
        int i = tl / c->B;
        const int *row = c->idx + (t * H + h) * c->K;
        const unsigned char *kp = c->keep ? c->keep + (t * H + h) * c->K : NULL;
        int nk = 0, own = 1;
        for (int p = 0; p < c->K; ++p) {
            int j = row[p];
            if (kp && j == i) own = kp[p] != 0;
            if (j < 0 || j >= i || (kp && !kp[p])) continue;
            for (int u = j * c->B; u < (j + 1) * c->B && u < L; ++u) keys[nk++] = u;
        }
        if (own)
            for (int u = i * c->B; u <= tl; ++u) keys[nk++] = u;
        /* is this row needed at all? */
        int want_q = !c->qsel || c->qsel[t * H + h];
        int want_k = 0;
        for (int e = 0; e < nk && !want_k; ++e)
            want_k = !c->kbsel || c->kbsel[(size_t)(c->boff[s] + keys[e] / c->B) * H + h];
        if (!want_q && !want_k) continue;
        if (nk == 0) {                           /* every block dropped: no keys, no gradient */
            double *dqr = c->dq + (t * H + h) * d;
            for (int ch = 0; ch < d; ++ch) dqr[ch] = 0.0;
            continue;
        }
        const float *qv = c->q + (t * H + h) * d;
        const float *dov = c->dout + (t * H + h) * d;
        double M = -INFINITY;
        for (int e = 0; e < nk; ++e) {
            const float *kv = c->k + ((size_t)(t0 + keys[e]) * H + h) * d;
            double acc = 0.0;
            for (int ch = 0; ch < d; ++ch) acc = acc + (double)qv[ch] * (double)kv[ch];
            z[e] = c->scale * acc;
            if (z[e] > M) M = z[e];
        }
        double l = 0.0;
        for (int e = 0; e < nk; ++e) l += exp(z[e] - M);
        double lse = M + log(l);
        double Dt = 0.0;
        for (int e = 0; e < nk; ++e) {
            const float *vv = c->v + ((size_t)(t0 + keys[e]) * H + h) * d;
            double acc = 0.0;
            for (int ch = 0; ch < d; ++ch) acc = acc + (double)dov[ch] * (double)vv[ch];
            dp[e] = acc;
            z[e] = exp(z[e] - lse);              /* z now holds P */
            Dt += z[e] * dp[e];
        }
        double *dqr = want_q ? c->dq + (t * H + h) * d : NULL;
        if (dqr)
            for (int ch = 0; ch < d; ++ch) dqr[ch] = 0.0;
        for (int e = 0; e < nk; ++e) {
            double P = z[e];
            double dS = P * (dp[e] - Dt);
            size_t ku = (size_t)(t0 + keys[e]) * H + h;
            if (dqr) {
                const float *kv = c->k + ku * d;
                for (int ch = 0; ch < d; ++ch) dqr[ch] += c->scale * dS * (double)kv[ch];
            }
            if (!c->kbsel || c->kbsel[(size_t)(c->boff[s] + keys[e] / c->B) * H + h]) {
                double *dkr = c->dk + ku * d;
                double *dvr = c->dv + ku * d;
                for (int ch = 0; ch < d; ++ch) {
                    dkr[ch] += c->scale * dS * (double)qv[ch];
                    dvr[ch] += P * (double)dov[ch];
                }
            }
        }
    }
    free(z);
    free(dp);
    free(keys);
}

int moba_oracle_attend_bwd(const float *q, const float *k, const float *v,
                           const int *idx, const unsigned char *keep, const float *dout,
                           int H, int d, int B, int K, const int *cu, int nseq, double scale,
                           const unsigned char *qsel, const unsigned char *kbsel,
                           double *dq, double *dk, double *dv, int nthreads)
{
    if (B < 1 || K < 1) return 1;
    if (!(scale > 0.0)) scale = 1.0 / sqrt((double)d);
    int *boff = block_offsets(cu, nseq, B);
    bwd_ctx c = {q, k, v, dout, idx, keep, qsel, kbsel, dq, dk, dv, cu, boff, H, d, B, K, scale};
    run_jobs(bwd_job, &c, nseq * H, nthreads);
    free(boff);
    return 0;
}

/* =====================================================================
 * Backward of step 1 (key convolution, Appendice B formal form): given
 * g = dL/dk', the gradients with respect to k and to the filter w, in fp64.
 *   u_t  = sum_l w_l k_{t-l}                    (the conv, taps inside the
 *                                                sequence only)
 *   mode 0:  e_t = g_t                          (k' = u)
 *   mode 1:  e_t = g_t * s'(u_t),               (k' = k + SiLU(u))
 *            s'(u) = sig(u) (1 + u (1 - sig(u))), sig(u) = 1/(1+exp(-u))
 *   dk_t = [mode 1: g_t] + sum_l w_l e_{t+l}    (t+l inside the sequence)
 *   dw_l = sum over sequences and t of e_t k_{t-l}   (t-l inside it)
 * per (head, channel).  One job per head (dw sums over every sequence).
 * ===================================================================== */
typedef struct {
    const float *k, *w, *g;
    double *dk, *dw;
    const int *cu;
    int nseq, H, d, W, mode;
} convb_ctx;

static void convb_job(void *vctx, int h)
{
    convb_ctx *c = (convb_ctx *)vctx;
    int H = c->H, d = c->d, W = c->W;
    for (int ch = 0; ch < d; ++ch) {
        const float *wv = c->w + ((size_t)h * d + ch) * W;
        double *dwv = c->dw + ((size_t)h * d + ch) * W;
        for (int l = 0; l < W; ++l) dwv[l] = 0.0;
        for (int s = 0; s < c->nseq; ++s) {
            int t0 = c->cu[s], t1 = c->cu[s + 1];
            for (int t = t0; t < t1; ++t) {
                size_t row = ((size_t)t * H + h) * d + ch;
                double acc = (c->mode == 1) ? (double)c->g[row] : 0.0;
                for (int l = 0; l < W; ++l) {
                    int tt = t + l;
                    if (tt >= t1) break;
                    size_t r2 = ((size_t)tt * H + h) * d + ch;
                    double e = (double)c->g[r2];
                    if (c->mode == 1) {
                        double u = 0.0;
                        for (int m = 0; m < W; ++m)
                            if (tt - m >= t0)
                                u += (double)c->w[((size_t)h * d + ch) * W + m] *
                                     (double)c->k[((size_t)(tt - m) * H + h) * d + ch];
                        double sg = 1.0 / (1.0 + exp(-u));
                        e *= sg * (1.0 + u * (1.0 - sg));
                    }
                    acc += (double)wv[l] * e;
                    /* dw_l gets e_{tt} k_{tt-l} = e_{t+l} k_t */
                    dwv[l] += e * (double)c->k[row];
                }
                c->dk[row] = acc;
            }
        }
    }
}

int moba_oracle_key_conv_bwd(const float *k, const float *w, const float *g, int H,
                             int d, int W, int mode, const int *cu, int nseq,
                             double *dk, double *dw, int nthreads)
{
    if (W < 1 || (mode != 0 && mode != 1)) return 1;
    convb_ctx c = {k, w, g, dk, dw, cu, nseq, H, d, W, mode};
    run_jobs(convb_job, &c, H, nthreads);
    return 0;
}
