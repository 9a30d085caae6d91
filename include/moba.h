/*
 * moba.h -- C ABI of the MI355X (gfx950) Mixture of Block Attention forward
 * and of its attention backward.
 *
 * The method is the one of "Optimizing Mixture of Block Attention" (Xiao,
 * Guo, Mazaheri, Han), as summarised on its summary pages:
 *   - task definition ("Definizione del Compito"): N keys split into
 *     n = N/B blocks; each query attends, with O = softmax(QK^T/sqrt(d))V,
 *     to its top-k blocks only;
 *   - router score ("Architettura del Modello Statistico", router-score
 *     equation): s_j = q . kbar_j with kbar_j the mean key of block j;
 *   - key convolution ("Appendice B", formal-form equation): a depthwise,
 *     causal, left-padded conv over the sequence, one filter per channel.
 * Causal rules (not spelled out on the pages, plainest decoder reading): the
 * query's own block is always kept and attended token-causally (u <= t), and
 * does not compete for the other k-1 places; future blocks are never
 * selected; equal scores go to the lower block index.  k counts the own
 * block (k = 8 of n = 64 blocks is the pages' "7/8 sparsity").
 *
 * Conventions shared by every call
 *   - All tensor pointers are DEVICE pointers owned by the caller.  The
 *     library never allocates, frees or synchronises; every call only
 *     enqueues kernels on `stream` (a hipStream_t; NULL = default stream)
 *     and returns.  Inputs are never modified; outputs are fully written.
 *   - q, k, v, k_out, o: [batch][seq][heads][head_dim], contiguous,
 *     head_dim fastest, dtype `shape->dtype`.  Varlen: batch == 1, seq ==
 *     total tokens, and `cu_seqlens` (HOST array of num_seqs+1 int32,
 *     cu[0] = 0, non-decreasing, cu[num_seqs] = seq) splits the token axis
 *     into independent sequences.  A uniform batch is the same as num_seqs =
 *     batch sequences of length seq.
 *   - Blocks restart at every sequence start; block j of a sequence holds
 *     its tokens [jB, min((j+1)B, L)).  Block ids in `idx` are local to the
 *     sequence.  "total blocks" = sum over sequences of ceil(L/B); centroid
 *     rows are ordered sequence-major, then block.
 *   - Errors: arguments are validated on the host before any launch:
 *     MOBA_ERR_INVALID_ARG (null pointer, misaligned pointer -- 16 bytes
 *     required --, inconsistent shape), MOBA_ERR_UNSUPPORTED (outside the
 *     support matrix below), MOBA_ERR_WORKSPACE_TOO_SMALL.  A failed launch
 *     returns MOBA_ERR_HIP.  Device faults surface at the caller's next sync.
 *     Nothing is printed, nothing throws.
 *   - Non-finite inputs: a NaN or infinity in a query row leaves that row's
 *     selection and output unspecified and every other row as it would be
 *     without it; one in k, v or a centroid leaves the rows that read it
 *     unspecified.  In every case the calls touch only the buffers they are
 *     given (block ids outside [0, own block) in idx are ignored by the
 *     attention calls).
 *   - Calls are stateless and may be issued from several host threads.
 *   - A call over more sequences than one launch table holds
 *     (MOBA_MAX_SEQS, a varlen batch or a uniform batch of more rows) runs
 *     them as consecutive groups of MOBA_MAX_SEQS sequences, each with its
 *     pointers advanced to its first token / block (sequences are
 *     independent): the results are those of one call.  The attention
 *     workspaces then hold one region per group, back to back.
 *
 * Support matrix: head_dim 64 or 128; block_size 64, 128, 256 or 512
 * (256 / 512: top_k <= 8, the summary page's MoBA-256 / MoBA-512 variants,
 * "Configurazione MoBA"); top_k 1..32; conv width 1..8; dtype bf16 (fast
 * path) or fp32 (correctness path; block_size <= 256); any number of
 * sequences; at most 16384 blocks per sequence; tokens * heads < 2^27 per
 * call.  The attention kernels work on blocks of up to 128 keys, 64 for
 * fp32 at head_dim 128; top_k times the number of such sub-blocks per
 * block must not exceed 32 (fp32, head_dim 128, block_size 128: top_k <=
 * 16).
 * Larger blocks: routing (centroids, scores, top-k) works on the blocks as
 * given; the attention calls attend a selected block as its sub-blocks
 * (the same key set, so the same result), with the query's own block split
 * into the sub-blocks before its own sub-block and its own sub-block
 * (token-causal).
 */
#ifndef MOBA_H_
#define MOBA_H_

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MOBA_ABI_VERSION 3
/* sequences per launch group (a call with more runs several groups) */
#define MOBA_MAX_SEQS 64

typedef enum {
    MOBA_OK = 0,
    MOBA_ERR_INVALID_ARG = 1,
    MOBA_ERR_UNSUPPORTED = 2,
    MOBA_ERR_WORKSPACE_TOO_SMALL = 3,
    MOBA_ERR_HIP = 4
} moba_status;

typedef enum { MOBA_F32 = 0, MOBA_BF16 = 1 } moba_dtype;

typedef enum {
    MOBA_CONV_PLAIN = 0,          /* k'_t = sum_l w_l * k_{t-l}                 */
    MOBA_CONV_SILU_RESIDUAL = 1   /* k'_t = k_t + SiLU(sum_l w_l * k_{t-l})     */
} moba_conv_mode;

typedef struct {
    int32_t batch;                /* uniform batches; 1 when cu_seqlens is set    */
    int32_t seq;                  /* tokens per batch row (varlen: total tokens)  */
    int32_t heads;
    int32_t head_dim;
    const int32_t *cu_seqlens;    /* HOST pointer or NULL; read during the call   */
    int32_t num_seqs;             /* entries of cu_seqlens minus one (varlen)     */
    int32_t block_size;           /* B                                            */
    int32_t top_k;                /* k, counting the query's own block            */
    int32_t dtype;                /* moba_dtype of q, k, v, k', o                 */
} moba_shape;

/*
 * moba_key_conv -- key convolution (Appendice B, formal form).
 *   w: fp32 [heads][head_dim][width]; w[h][c][l] multiplies k_{t-l} of
 *      channel (h, c) (l = 0 is the current token).  Zero before each
 *      sequence start.
 *   The tap sum is fp32 fmaf from the oldest tap to the newest, started at
 *   +0; MOBA_CONV_SILU_RESIDUAL then forms k_t + conv/(1+exp(-conv)) as if
 *   in fp64 and rounds it to fp32 (bf16 output: a fast fp32 evaluation is
 *   used wherever its error bound proves the same bf16 result, the fp64
 *   formula elsewhere).
 *   k_out (same layout and dtype as k) is rounded to the dtype (bf16:
 *   round-to-nearest-even).  k_out must not alias k.
 *   If `cent` is not NULL, the block centroids of k_out are also written to
 *   it (same contract as moba_centroids), in the same pass.
 */
moba_status moba_key_conv(const moba_shape *shape, const void *k,
                          const float *w, int32_t width, int32_t mode,
                          void *k_out, float *cent, hipStream_t stream);

/*
 * moba_key_conv_bwd -- gradients of moba_key_conv (Appendice B, formal form)
 * given dk_out = dL/dk' (same layout and dtype as k):
 *   e_t  = dk_out_t                 (MOBA_CONV_PLAIN)
 *        = dk_out_t * s'(u_t)       (MOBA_CONV_SILU_RESIDUAL; u_t the tap sum,
 *                                    s'(u) = sig(u) (1 + u (1 - sig(u))))
 *   dk_t = [SiLU form: dk_out_t] + sum_l w_l e_{t+l}   (t+l in the sequence)
 *   dw[h][c][l] = sum over all tokens t of e_t k_{t-l}  (t-l in the sequence)
 *   dk: same layout and dtype as k (fp32 sums, rounded once); must not alias
 *   k or dk_out.  dw: fp32 [heads][head_dim][width], fully written; the sum
 *   over tokens is fp32 per key block and fp64 across blocks, in a fixed
 *   order (deterministic).
 *   workspace: at least moba_key_conv_bwd_workspace_bytes() (one fp32
 *   partial of dw per key block), 256-byte aligned, scratch on exit.
 *   Same validation and errors as moba_key_conv.
 */
moba_status moba_key_conv_bwd(const moba_shape *shape, const void *k,
                              const float *w, int32_t width, int32_t mode,
                              const void *dk_out, void *dk, float *dw,
                              void *workspace, size_t workspace_bytes,
                              hipStream_t stream);

/* Bytes of workspace moba_key_conv_bwd needs (0 on invalid shape / width). */
size_t moba_key_conv_bwd_workspace_bytes(const moba_shape *shape,
                                         int32_t width);

/*
 * moba_centroids -- block means kbar_j (router-score equation).
 *   cent: fp32 [total_blocks][heads][head_dim].  Each mean is the exact
 *   fp64 sum of the block's keys, divided by the block's key count and
 *   rounded once to fp32; a final partial block is averaged over the keys
 *   it holds.
 */
moba_status moba_centroids(const moba_shape *shape, const void *k,
                           float *cent, hipStream_t stream);

/*
 * moba_route_topk -- router scores and causal top-k selection.
 *   For query t in block i of its sequence: scores s_j = q_t . cent_j for the
 *   past blocks j < i; keep the first min(k-1, i) in the order (score
 *   descending, block id ascending), add the own block i.
 *   idx: int32 [batch][seq][heads][top_k]; each row ascending, own block
 *   included, padded with -1 at the end.
 *   The selection is exact with respect to scores computed in fp64: the
 *   kernel scores in fp32 with a rigorous error bound and re-scores in fp64
 *   any query whose k-1-th and k-th scores are closer than that bound.
 *   workspace: device memory of at least moba_route_topk_workspace_bytes(),
 *   256-byte aligned (bf16 queries: the centroids split into bf16 high and
 *   low parts and their squared norms, written by the call; fp32 queries do
 *   not use it); contents on entry ignored, scratch on exit.  NULL or
 *   misaligned -> MOBA_ERR_INVALID_ARG, too small ->
 *   MOBA_ERR_WORKSPACE_TOO_SMALL.  A moba_attn_fwd workspace of at least
 *   this size may be reused (calls stream-ordered).
 */
moba_status moba_route_topk(const moba_shape *shape, const void *q,
                            const float *cent, int32_t *idx,
                            void *workspace, size_t workspace_bytes,
                            hipStream_t stream);

/* Bytes of workspace moba_route_topk needs for `shape` (0 on invalid shape). */
size_t moba_route_topk_workspace_bytes(const moba_shape *shape);

/*
 * moba_route_topk_noalloc -- moba_route_topk for callers that cannot
 * allocate device memory (code under stream capture, tight serving loops,
 * harnesses that forbid allocation): the same selection, with the routing
 * workspace taken from a fixed buffer of MOBA_ROUTE_SCRATCH_BYTES inside
 * the library (one per GPU, held until the process ends) instead of a
 * caller's workspace.  It makes no allocation of its own.
 *   bf16 queries need 4 * head_dim + 4 bytes per (block, head) centroid
 *   row, so the buffer covers about 129 000 rows at head_dim 64 and 65 000
 *   at 128 (one 512K-token sequence of 16 heads at B = 128 takes 16 MiB);
 *   a larger shape (moba_route_topk_workspace_bytes() above
 *   MOBA_ROUTE_SCRATCH_BYTES) returns MOBA_ERR_WORKSPACE_TOO_SMALL before
 *   any launch.  fp32 queries do not use the buffer.
 *   Every call on one GPU uses that GPU's one buffer: calls that may
 *   overlap on a GPU (several streams, several host threads) race and must
 *   be ordered by the caller.  Nothing in the buffer needs to start at zero;
 *   each call rewrites what it reads.  Other arguments and errors as
 *   moba_route_topk.
 */
#define MOBA_ROUTE_SCRATCH_BYTES (32u << 20)
moba_status moba_route_topk_noalloc(const moba_shape *shape, const void *q,
                                    const float *cent, int32_t *idx,
                                    hipStream_t stream);

/*
 * moba_attn_fwd -- attention over the selected blocks (task definition).
 *   For query t in block i: keys = all keys of each listed past block
 *   (0 <= idx < i) plus the keys u <= t of block i.  -1 entries are padding;
 *   listed entries >= i are ignored (the own block is always attended).
 *   Listed past blocks must be distinct.  With top_k == 1 only the own
 *   block is attended (a row has no room for a routed block).
 *   z_u = scale * q_t . k_u; O_t = softmax(z) V; LSE_t = max z + ln sum
 *   exp(z - max z) (natural log).
 *   softmax_scale <= 0 selects 1/sqrt(head_dim).
 *   o: same layout/dtype as q.  lse: NULL or fp32 [batch][seq][heads].
 *   workspace: device memory of at least moba_attn_fwd_workspace_bytes(),
 *   256-byte aligned; its contents on entry are ignored and on exit are
 *   scratch.  Calls that share a workspace must be stream-ordered.
 *   Internally: build, for every (sequence, head, block j), the list of
 *   (query, slot) pairs that routed to j; attend each list's gathered
 *   queries against block j densely (bf16 MFMA, fp32 softmax), keeping one
 *   (o, lse) partial per pair; then the own block causally and the merge of
 *   the partials per query.
 */
moba_status moba_attn_fwd(const moba_shape *shape, const void *q,
                          const void *k, const void *v, const int32_t *idx,
                          float softmax_scale, void *o, float *lse,
                          void *workspace, size_t workspace_bytes,
                          hipStream_t stream);

/*
 * moba_attn_fwd_blasst -- moba_attn_fwd with the BLASST block skip ("BLASST:
 * Dynamic BLocked Attention Sparsity via Softmax Thresholding", section
 * "Meccanismo di Pruning") applied to each query's selected blocks: the
 * blocks are visited in ascending order, the own block last, keeping a
 * running maximum M of the kept blocks' scores; a block whose maximum
 * score m satisfies m - M < ln(blasst_lambda) is skipped (its keys take no
 * part in the softmax).  The first block is always kept.
 *   blasst_lambda in [0, 1] (else MOBA_ERR_INVALID_ARG); 0 keeps every
 *   block (moba_attn_fwd's result).  o and lse are those of the softmax
 *   over the kept blocks' keys.  Shapes whose blocks the attention
 *   kernels take whole only (block size 64 or 128, not fp32 at head_dim
 *   128 with 128-key blocks; others: MOBA_ERR_UNSUPPORTED).  Block maxima are taken from the fp32 scores;
 *   a decision within rounding of the threshold may go either way.
 *   The key-block-major order computes every selected (query, block) pair
 *   before any query's running maximum is known, so the skip is decided in
 *   the merge of the per-block partials: it saves the merge's reads of the
 *   skipped partials, not their computation.
 *   kept_idx: NULL, or int32 [batch][seq][heads][top_k], 16-byte aligned,
 *   not idx: receives the attended selection -- idx's past blocks that were
 *   kept, then the own block if it was kept, ascending, -1 padded (with
 *   lambda = 0: idx itself).  It is the selection moba_attn_bwd_blasst takes.
 *   Same workspace (moba_attn_fwd_workspace_bytes), other arguments and
 *   errors as moba_attn_fwd.
 */
moba_status moba_attn_fwd_blasst(const moba_shape *shape, const void *q,
                                 const void *k, const void *v,
                                 const int32_t *idx, float softmax_scale,
                                 float blasst_lambda, void *o, float *lse,
                                 int32_t *kept_idx, void *workspace,
                                 size_t workspace_bytes, hipStream_t stream);

/* The three stages of moba_attn_fwd, in order, for stage timing: the
 * index inversion, the routed (past-block) attention, and the own-block
 * attention plus merge.  Running them in order on one stream with one
 * workspace is exactly moba_attn_fwd.  Same arguments and errors. */
moba_status moba_attn_index(const moba_shape *shape, const int32_t *idx,
                            void *workspace, size_t workspace_bytes,
                            hipStream_t stream);
moba_status moba_attn_routed(const moba_shape *shape, const void *q,
                             const void *k, const void *v, float softmax_scale,
                             void *workspace, size_t workspace_bytes,
                             hipStream_t stream);
moba_status moba_attn_combine(const moba_shape *shape, const void *q,
                              const void *k, const void *v,
                              const int32_t *idx, float softmax_scale,
                              void *o, float *lse, void *workspace,
                              size_t workspace_bytes, hipStream_t stream);

/*
 * moba_attn_bwd -- gradients of moba_attn_fwd's O with respect to q, k and v
 * for the fixed selection idx (summary page, "Backward Pass: Ricalcolo
 * (Algoritmo 5)": recompute the scores and probabilities FlashAttention-2
 * style, parallel over key blocks, gathering each block's queries as the
 * forward does).  The selection is piecewise constant in q and k, so no
 * gradient flows through the router; the gradient of k flows into k' only
 * (the key convolution's input is the caller's business).
 *   q, k, v, idx, softmax_scale: exactly as given to moba_attn_fwd.
 *   o, lse: that call's outputs (lse is required here).
 *   dout: dL/dO, same layout and dtype as o.
 *   dq, dk, dv: outputs, same layout and dtype as q; fully written; must
 *   not alias any input or each other.
 *   For query t with key set U_t (as in moba_attn_fwd), with
 *   P_tu = exp(scale q_t.k_u - lse_t) and D_t = dout_t . o_t:
 *     dv_u = sum_t P_tu dout_t,  dS_tu = P_tu (dout_t . v_u - D_t),
 *     dq_t = scale sum_u dS_tu k_u,  dk_u = scale sum_t dS_tu q_t.
 *   bf16: P and dS enter the matrix products as bf16, every sum is fp32,
 *   outputs are rounded once.  fp32 (a plain recompute path, for exactness
 *   rather than speed): every product and sum in fp32, in a fixed order.
 *   workspace: at least moba_attn_bwd_workspace_bytes(), 256-byte aligned,
 *   scratch on exit; it holds the inverted lists and (bf16) one fp32 dq
 *   piece per routed (query, slot) pair.  No atomics on results: dq, dk and
 *   dv are bitwise repeatable (dk / dv for sequences of up to 4096 blocks;
 *   longer ones may differ between runs by fp32 summation order).
 *   Same error behaviour as moba_attn_fwd.
 */
moba_status moba_attn_bwd(const moba_shape *shape, const void *q,
                          const void *k, const void *v, const int32_t *idx,
                          float softmax_scale, const void *o, const float *lse,
                          const void *dout, void *dq, void *dk, void *dv,
                          void *workspace, size_t workspace_bytes,
                          hipStream_t stream);

/*
 * moba_attn_bwd_blasst -- gradients of moba_attn_fwd_blasst's O (BLASST
 * page, "Meccanismo di Pruning", and the page's sparsity-aware training):
 * for the skip decisions that call took, the gradients of softmax attention
 * over the kept blocks' keys.  The decisions are piecewise constant in q and
 * k, so, as for the router, no gradient flows through them.
 *   kept_idx: the forward's kept_idx output (rows ascending, -1 padded; a
 *   row lists its own block only if the own block was kept, and attends it
 *   causally then).  o, lse: that forward's outputs.  Other arguments,
 *   workspace (moba_attn_bwd_workspace_bytes), repeatability and errors as
 *   moba_attn_bwd; the shapes moba_attn_fwd_blasst takes (others:
 *   MOBA_ERR_UNSUPPORTED).  A row that lists no block has no keys: its dq is
 *   zero and it adds nothing to dk, dv.
 */
moba_status moba_attn_bwd_blasst(const moba_shape *shape, const void *q,
                                 const void *k, const void *v,
                                 const int32_t *kept_idx, float softmax_scale,
                                 const void *o, const float *lse,
                                 const void *dout, void *dq, void *dk,
                                 void *dv, void *workspace,
                                 size_t workspace_bytes, hipStream_t stream);

/* Bytes of workspace moba_attn_bwd (and moba_attn_bwd_blasst) needs for
 * `shape` (0 on invalid shape). */
size_t moba_attn_bwd_workspace_bytes(const moba_shape *shape);

/* Bytes of workspace moba_attn_fwd needs for `shape` (0 on invalid shape). */
size_t moba_attn_fwd_workspace_bytes(const moba_shape *shape);

/* Total number of blocks (centroid rows) of `shape`; -1 on invalid shape. */
int64_t moba_total_blocks(const moba_shape *shape);

/* Text of a status value; any int is accepted ("unknown status" outside
 * the enum).  The returned string is static. */
const char *moba_status_string(int32_t status);
int32_t moba_abi_version(void);

/*
 * moba_debug_violations -- for the bounds-checking debug build of this
 * library (libmoba_amd_debug.so, compiled with MOBA_DEBUG_BOUNDS), where the
 * kernels check every index they take from data (list entries, list
 * positions, work items) against the region it addresses and skip an
 * access that would leave it.  Writes to *flags the OR of the violations
 * seen on the current device since the last call (0: none; bits 0..7: the
 * check that failed, in the order routed item, routed entry, merge
 * position, backward list, backward entry, dq position, index-pass
 * position, fp32 backward entry; bit 31: the flags could not be read) and
 * clears them.  Synchronous (waits for the device).  The release library
 * returns MOBA_ERR_UNSUPPORTED and writes nothing; a null flags pointer is
 * MOBA_ERR_INVALID_ARG.  For tests of the kernels' indexing, not for use
 * while other calls run.
 */
moba_status moba_debug_violations(uint32_t *flags);

#ifdef __cplusplus
}
#endif

#endif /* MOBA_H_ */
