/* Sanitizer driver for the host side of the C ABI (test infrastructure):
 * calls every entry point that needs no GPU -- sizes, block counts, status
 * strings -- on valid, ragged, many-sequence and oversized shapes, and the
 * compute entry points with arguments that validation refuses before any
 * device work (null, misaligned or short buffers, bad shapes).  Run under
 * AddressSanitizer and UBSan; every refusal must carry the documented
 * status. */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

#include "moba.h"

static int fails = 0;
#define EXPECT(cond)                                                  \
    do {                                                              \
        if (!(cond)) { fprintf(stderr, "FAIL line %d: %s\n", __LINE__, #cond); ++fails; } \
    } while (0)

static moba_shape shape(int b, int n, int H, int d, int B, int K, int dtype, const int32_t *cu,
                        int nseq)
{
    moba_shape s;
    s.batch = b; s.seq = n; s.heads = H; s.head_dim = d; s.cu_seqlens = cu;
    s.num_seqs = nseq; s.block_size = B; s.top_k = K; s.dtype = dtype;
    return s;
}

static void sizes(const moba_shape *s)
{
    (void)moba_total_blocks(s);
    (void)moba_attn_fwd_workspace_bytes(s);
    (void)moba_attn_bwd_workspace_bytes(s);
    (void)moba_route_topk_workspace_bytes(s);
    for (int W = 0; W <= 9; ++W) (void)moba_key_conv_bwd_workspace_bytes(s, W);
}

/* compute entry points with a refused argument: a null or misaligned data
 * pointer (refused whatever the shape), aliased buffers, a null workspace;
 * with a refused shape (want_shape), a call whose other arguments would
 * pass.  No call here reaches device work. */
static void refused(const moba_shape *s, moba_status want_shape)
{
    void *p = (void *)(uintptr_t)(1u << 20);           /* never dereferenced */
    void *odd = (void *)(uintptr_t)((1u << 20) + 4);
    float *fp = (float *)p;
    int32_t *ip = (int32_t *)p;
    const size_t big = (size_t)1 << 40;
    EXPECT(moba_centroids(s, NULL, fp, NULL) != MOBA_OK);
    EXPECT(moba_centroids(s, odd, fp, NULL) != MOBA_OK);
    EXPECT(moba_route_topk(s, NULL, fp, ip, p, big, NULL) != MOBA_OK);
    EXPECT(moba_route_topk(s, odd, fp, ip, p, big, NULL) != MOBA_OK);
    EXPECT(moba_attn_fwd(s, NULL, p, p, ip, 0.0f, p, NULL, p, big, NULL) != MOBA_OK);
    EXPECT(moba_attn_index(s, NULL, p, big, NULL) != MOBA_OK);
    EXPECT(moba_attn_fwd_blasst(s, NULL, p, p, ip, 0.0f, 0.5f, p, NULL, NULL, p, big, NULL) != MOBA_OK);
    EXPECT(moba_attn_fwd_blasst(s, p, p, p, ip, 0.0f, 0.5f, p, NULL, ip, p, big, NULL) != MOBA_OK);
    EXPECT(moba_attn_fwd_blasst(s, p, p, p, ip, 0.0f, 0.5f, p, NULL, (int32_t *)odd, p, big,
                                NULL) != MOBA_OK);
    EXPECT(moba_attn_fwd_blasst(s, p, p, p, ip, 0.0f, 1.5f, p, NULL, NULL, p, big, NULL) != MOBA_OK);
    EXPECT(moba_attn_bwd(s, NULL, p, p, ip, 0.0f, p, fp, p, p, p, p, p, big, NULL) != MOBA_OK);
    EXPECT(moba_attn_bwd_blasst(s, NULL, p, p, ip, 0.0f, p, fp, p, p, p, p, p, big, NULL) != MOBA_OK);
    EXPECT(moba_key_conv(s, p, fp, 3, 0, p, NULL, NULL) != MOBA_OK);   /* k' aliases k */
    if (want_shape != MOBA_OK) {
        EXPECT(moba_route_topk(s, p, fp, ip, p, big, NULL) == want_shape);
        EXPECT(moba_total_blocks(s) == -1);
        EXPECT(moba_attn_fwd_workspace_bytes(s) == 0);
    }
}

int main(void)
{
    EXPECT(moba_abi_version() > 0);
    {
        uint32_t f = 7u;      /* the release library has no bounds checks */
        EXPECT(moba_debug_violations(&f) == MOBA_ERR_UNSUPPORTED && f == 7u);
    }
    for (int c = -3; c < 16; ++c) EXPECT(moba_status_string((moba_status)c) != NULL);

    /* uniform batches over every supported block size, k and dtype */
    const int Bs[4] = {64, 128, 256, 512};
    for (int bi = 0; bi < 4; ++bi)
        for (int K = 1; K <= 8; ++K)
            for (int dt = 0; dt < 2; ++dt) {
                moba_shape s = shape(2, 1000 + 37 * K, 3, 64, Bs[bi], K, dt, NULL, 0);
                sizes(&s);
                refused(&s, MOBA_OK);
            }
    {
        moba_shape s = shape(1, 4096, 2, 128, 128, 16, MOBA_BF16, NULL, 0);
        sizes(&s);
        refused(&s, MOBA_OK);
    }
    /* varlen: ragged, empty and one-token sequences; 1, 64, 65 and 200 of them */
    const int ns[4] = {1, 64, 65, 200};
    for (int a = 0; a < 4; ++a) {
        int32_t *cu = (int32_t *)malloc(sizeof(int32_t) * (size_t)(ns[a] + 1));
        cu[0] = 0;
        for (int i = 0; i < ns[a]; ++i) cu[i + 1] = cu[i] + (37 * i) % 301;
        moba_shape s = shape(1, cu[ns[a]], 2, 64, 64, 4, MOBA_BF16, cu, ns[a]);
        sizes(&s);
        EXPECT(moba_total_blocks(&s) >= 0);
        refused(&s, MOBA_OK);
        free(cu);
    }
    /* refused shapes */
    {
        moba_shape s = shape(2, 1000, 3, 96, 64, 4, MOBA_BF16, NULL, 0);
        sizes(&s); refused(&s, MOBA_ERR_UNSUPPORTED);
        s = shape(2, 1000, 3, 64, 32, 4, MOBA_BF16, NULL, 0);
        sizes(&s); refused(&s, MOBA_ERR_UNSUPPORTED);
        s = shape(2, 1000, 3, 64, 64, 0, MOBA_BF16, NULL, 0);
        sizes(&s); refused(&s, MOBA_ERR_INVALID_ARG);
        s = shape(2, 1000, 0, 64, 64, 4, MOBA_BF16, NULL, 0);
        sizes(&s); refused(&s, MOBA_ERR_INVALID_ARG);
        s = shape(-1, 1000, 3, 64, 64, 4, MOBA_BF16, NULL, 0);
        sizes(&s); refused(&s, MOBA_ERR_INVALID_ARG);
        s = shape(2, 1 << 26, 2, 64, 64, 4, MOBA_BF16, NULL, 0);    /* 2^27 token-heads */
        sizes(&s); refused(&s, MOBA_ERR_UNSUPPORTED);
        s = shape(1, 16384 * 64 + 1, 1, 64, 64, 4, MOBA_BF16, NULL, 0);  /* 16385 blocks */
        sizes(&s); refused(&s, MOBA_ERR_UNSUPPORTED);
        const int32_t bad1[3] = {0, 10, 5};
        s = shape(1, 10, 2, 64, 64, 4, MOBA_BF16, bad1, 2);
        sizes(&s); refused(&s, MOBA_ERR_INVALID_ARG);
        const int32_t bad2[2] = {1, 10};
        s = shape(1, 10, 2, 64, 64, 4, MOBA_BF16, bad2, 1);
        sizes(&s); refused(&s, MOBA_ERR_INVALID_ARG);
        s = shape(1, 10, 2, 64, 64, 4, 7, NULL, 0);
        sizes(&s); refused(&s, MOBA_ERR_INVALID_ARG);
        /* decreasing offsets beyond the first group of 64 sequences */
        int32_t cu[201];
        cu[0] = 0;
        for (int i = 0; i < 200; ++i) cu[i + 1] = cu[i] + 10;
        cu[150] = cu[149] - 3;
        s = shape(1, cu[200], 2, 64, 64, 4, MOBA_BF16, cu, 200);
        sizes(&s); refused(&s, MOBA_ERR_INVALID_ARG);
    }
    EXPECT(moba_total_blocks(NULL) == -1);
    EXPECT(moba_attn_fwd_workspace_bytes(NULL) == 0);
    if (fails) { fprintf(stderr, "%d failures\n", fails); return 1; }
    printf("ok\n");
    return 0;
}
