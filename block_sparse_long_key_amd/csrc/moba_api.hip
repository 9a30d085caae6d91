// moba_api.hip -- the C ABI of include/moba.h: argument validation,
// sequence/block tables, workspace carving and kernel launches.  No
// allocation, no synchronisation, no printing.
#include <math.h>
#include <algorithm>
#include <string.h>

#include "moba_internal.h"

using namespace moba;

namespace {

constexpr int64_t kMaxRows = (int64_t)1 << 27;   // tokens * heads (entry encoding)

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

int ceil_div(int a, int b) { return (a + b - 1) / b; }

// Validate the shape and fill the launch description.
moba_status make_launch(const moba_shape* sh, Launch* L, hipStream_t stream)
{
    if (!sh) return MOBA_ERR_INVALID_ARG;
    if (sh->heads < 1 || sh->seq < 0 || sh->batch < 1) return MOBA_ERR_INVALID_ARG;
    if (sh->dtype != MOBA_F32 && sh->dtype != MOBA_BF16) return MOBA_ERR_INVALID_ARG;
    if (sh->head_dim != 64 && sh->head_dim != 128) return MOBA_ERR_UNSUPPORTED;
    if (sh->block_size != 64 && sh->block_size != 128 && sh->block_size != 256 &&
        sh->block_size != 512)
        return MOBA_ERR_UNSUPPORTED;
    if (sh->top_k < 1) return MOBA_ERR_INVALID_ARG;
    if (sh->top_k > 32) return MOBA_ERR_UNSUPPORTED;
    // the MFMA router takes top_k <= 8 with blocks of 256 / 512 keys
    if (sh->block_size > 128 && sh->top_k > 8) return MOBA_ERR_UNSUPPORTED;
    // blocks larger than the attention kernels' are attended as their
    // sub-blocks: the expanded selection must fit 32 slots
    const int ab = att_block(sh->dtype, sh->head_dim, sh->block_size);
    if (sh->top_k * (sh->block_size / ab) > 32) return MOBA_ERR_UNSUPPORTED;
    // the fp32 router runs one thread per query of a block (<= 256)
    if (sh->dtype == MOBA_F32 && sh->block_size > 256) return MOBA_ERR_UNSUPPORTED;

    memset(L, 0, sizeof(*L));
    SegTable& st = L->st;
    st.H = sh->heads;
    st.B = sh->block_size;
    st.K = sh->top_k;
    int64_t tokens;
    if (sh->cu_seqlens) {
        if (sh->batch != 1) return MOBA_ERR_INVALID_ARG;
        if (sh->num_seqs < 1) return MOBA_ERR_INVALID_ARG;
        if (sh->num_seqs > kMaxSeqs) return MOBA_ERR_UNSUPPORTED;
        const int32_t* cu = sh->cu_seqlens;
        if (cu[0] != 0 || cu[sh->num_seqs] != sh->seq) return MOBA_ERR_INVALID_ARG;
        for (int s = 0; s < sh->num_seqs; ++s)
            if (cu[s + 1] < cu[s]) return MOBA_ERR_INVALID_ARG;
        st.nseq = sh->num_seqs;
        for (int s = 0; s <= st.nseq; ++s) st.cu[s] = cu[s];
        tokens = sh->seq;
    } else {
        if (sh->batch > kMaxSeqs) return MOBA_ERR_UNSUPPORTED;
        st.nseq = sh->batch;
        tokens = (int64_t)sh->batch * sh->seq;
        if (tokens * sh->heads >= kMaxRows) return MOBA_ERR_UNSUPPORTED;
        for (int s = 0; s <= st.nseq; ++s) st.cu[s] = s * sh->seq;
    }
    if (tokens * sh->heads >= kMaxRows) return MOBA_ERR_UNSUPPORTED;

    const int K1 = st.K - 1;
    int maxn = 0;
    for (int s = 0; s < st.nseq; ++s) maxn = std::max(maxn, ceil_div(st.cu[s + 1] - st.cu[s], st.B));
    // (measured, index pass: 4096 blocks 1.03 -> 0.77 ms with 1/16 of the
    // blocks per chunk, 0.93 with 1/32, 1.26 with 1/8; at 1024 blocks 32 per
    // chunk stays best)
    st.chunk = kInvChunkBlocks;
    if (maxn > 1024)
        while (st.chunk * 16 < maxn) st.chunk *= 2;
    st.item_rows = item_rows_for(sh->dtype, sh->head_dim);
    st.boff[0] = 0;
    st.cbase[0] = 0;
    st.cmbase[0] = 0;
    st.ebase[0] = 0;
    st.ibase[0] = 0;
    for (int s = 0; s < st.nseq; ++s) {
        const int Ls = st.cu[s + 1] - st.cu[s];
        const int n = ceil_div(Ls, st.B);
        if (n > kMaxBlocksPerSeq) return MOBA_ERR_UNSUPPORTED;
        const int nch = ceil_div(n, st.chunk);
        st.boff[s + 1] = st.boff[s] + n;
        st.cbase[s + 1] = st.cbase[s] + nch;
        st.cmbase[s + 1] = st.cmbase[s] + (int64_t)st.H * nch * n;
        // lists are sized for K entries per row so that any idx row (even one
        // that omits its own block) stays in bounds
        st.ebase[s + 1] = st.ebase[s] + (int64_t)st.H * Ls * st.K;
        const int64_t cap = (int64_t)Ls * st.K / st.item_rows + n;
        st.ibase[s + 1] = st.ibase[s] + (int64_t)st.H * cap;
    }
    st.total_blocks = st.boff[st.nseq];
    st.total_chunks = st.cbase[st.nseq];
    st.total_items = K1 > 0 ? st.ibase[st.nseq] : 0;
    L->D = sh->head_dim;
    L->dtype = sh->dtype;
    L->tokens = (int)tokens;
    L->stream = stream;
    return MOBA_OK;
}

// bwd: the backward's workspace (index + its own buffers, no forward partials)
// expand: the selection is re-expressed in the attention kernels' blocks
// first (block sizes 256 / 512; 128 in fp32 at d = 128); L is then the
// attention launch
WsLayout layout(const Launch& L, bool bwd = false, bool expand = false)
{
    WsLayout w;
    memset(&w, 0, sizeof(w));
    const SegTable& st = L.st;
    const size_t esz = L.dtype == MOBA_BF16 ? 2 : 4;
    const size_t rows = (size_t)L.tokens * st.H;
    if (st.K > 1) {
        w.cmat_bytes = (size_t)st.cmbase[st.nseq] * 4;
        w.items_bytes = (size_t)st.total_items * sizeof(Item);
        w.ent_bytes = (size_t)st.ebase[st.nseq] * 4;
        w.rev_bytes = rows * st.K * 4;
        w.lst_bytes = (size_t)st.total_blocks * st.H * 8;
        if (!bwd) {
            // partials are indexed like the entries (list order)
            w.po_bytes = (size_t)st.ebase[st.nseq] * L.D * esz;
            w.pl_bytes = (size_t)st.ebase[st.nseq] * 4;
            w.pm_bytes = (size_t)st.ebase[st.nseq] * 8;
        }
    }
    if (bwd) {
        w.rs_bytes = rows * 8;
        const size_t ent_rows = st.K > 1 ? (size_t)st.ebase[st.nseq] : 0;
        w.pq_bytes = (ent_rows + rows) * L.D * 4;
        w.own_bytes = rows;
    }
    if (expand) w.px_bytes = rows * st.K * 4;
    size_t off = 0;
    w.cmat_off = off;  off += align256(w.cmat_bytes);
    w.items_off = off; off += align256(w.items_bytes);
    w.ent_off = off;   off += align256(w.ent_bytes);
    w.rev_off = off;   off += align256(w.rev_bytes);
    w.po_off = off;    off += align256(w.po_bytes);
    w.pl_off = off;    off += align256(w.pl_bytes);
    w.pm_off = off;    off += align256(w.pm_bytes);
    w.lst_off = off;   off += align256(w.lst_bytes);
    w.rs_off = off;    off += align256(w.rs_bytes);
    w.pq_off = off;    off += align256(w.pq_bytes);
    w.px_off = off;    off += align256(w.px_bytes);
    w.own_off = off;   off += align256(w.own_bytes);
    w.total = off;
    return w;
}

moba_status hip_status(hipError_t e) { return e == hipSuccess ? MOBA_OK : MOBA_ERR_HIP; }

bool ptr_ok(const void* p) { return p != nullptr && aligned16(p); }
// idx and lse of a later sequence group start at a row offset: 4-byte
// aligned (the caller's own pointers are checked for 16 bytes)
bool idx_ok(const void* p) { return p != nullptr && ((uintptr_t)p & 3u) == 0; }


// The attention entry points work on att_block()-key blocks when the
// shape's blocks are larger: Ll is the shape's own launch (routing
// granularity), La the one the attention kernels run with (block ab,
// top_k * B / ab slots).
moba_status attn_launch(const moba_shape* sh, hipStream_t stream, Launch* Ll, Launch* La)
{
    moba_status st = make_launch(sh, Ll, stream);
    if (st != MOBA_OK) return st;
    const int ab = att_block(sh->dtype, sh->head_dim, sh->block_size);
    if (sh->block_size <= ab) {
        *La = *Ll;
        return MOBA_OK;
    }
    moba_shape p = *sh;
    p.block_size = ab;
    p.top_k = sh->top_k * (sh->block_size / ab);
    return make_launch(&p, La, stream);
}

bool expands(const Launch& Ll) { return Ll.st.B > att_block(Ll.dtype, Ll.D, Ll.st.B); }

moba_status check_ws(const Launch& L, const void* ws, size_t bytes, WsLayout* out, bool bwd = false,
                     bool expand = false)
{
    *out = layout(L, bwd, expand);
    if (out->total > 0) {
        if (!ws || ((uintptr_t)ws & 255u) != 0) return MOBA_ERR_INVALID_ARG;
        if (bytes < out->total) return MOBA_ERR_WORKSPACE_TOO_SMALL;
    }
    return MOBA_OK;
}

float resolve_scale(float scale, int D)
{
    return scale > 0.f ? scale : (float)(1.0 / sqrt((double)D));
}

// ---------------------------------------------------------------------
// Calls over more sequences than one launch table holds (kMaxSeqs) run as
// consecutive groups of at most kMaxSeqs sequences, each a shape of its own
// with every pointer advanced to its first token or block: sequences are
// independent, so the results are those of one call.  Workspaces hold one
// region per group (the stages of one call find their group's lists in
// place); the routing workspace is reused group after group.
struct Groups {
    int n = 0;                     // number of groups
    int nseq = 0;                  // sequences over all groups
    moba_shape base;               // the caller's shape
    const int32_t* cu = nullptr;   // caller's cu_seqlens (null: uniform batch)
};

struct Group {
    moba_shape sh;
    int32_t cu[kMaxSeqs + 1];
    int64_t tok0 = 0;              // first token of the group (over the call)
    int64_t blk0 = 0;              // first block of the group (shape's block size)
};

int64_t ceil_div64(int64_t a, int64_t b) { return (a + b - 1) / b; }

// validates what spans groups (cu_seqlens as a whole, the token x head
// limit); everything else is checked per group by make_launch
moba_status split(const moba_shape* sh, Groups* G)
{
    if (!sh) return MOBA_ERR_INVALID_ARG;
    if (sh->heads < 1 || sh->seq < 0 || sh->batch < 1 || sh->block_size < 1)
        return MOBA_ERR_INVALID_ARG;
    G->base = *sh;
    if (sh->cu_seqlens) {
        if (sh->batch != 1 || sh->num_seqs < 1) return MOBA_ERR_INVALID_ARG;
        const int32_t* cu = sh->cu_seqlens;
        if (cu[0] != 0 || cu[sh->num_seqs] != sh->seq) return MOBA_ERR_INVALID_ARG;
        for (int q = 0; q < sh->num_seqs; ++q)
            if (cu[q + 1] < cu[q]) return MOBA_ERR_INVALID_ARG;
        G->cu = cu;
        G->nseq = sh->num_seqs;
    } else {
        G->nseq = sh->batch;
    }
    const int64_t tokens = sh->cu_seqlens ? (int64_t)sh->seq : (int64_t)sh->batch * sh->seq;
    if (tokens * sh->heads >= kMaxRows) return MOBA_ERR_UNSUPPORTED;
    G->n = (G->nseq + kMaxSeqs - 1) / kMaxSeqs;
    return MOBA_OK;
}

void group(const Groups& G, int g, Group* out)
{
    const int s0 = g * kMaxSeqs;
    const int n = std::min(kMaxSeqs, G.nseq - s0);
    out->sh = G.base;
    if (G.cu) {
        const int32_t c0 = G.cu[s0];
        for (int q = 0; q <= n; ++q) out->cu[q] = G.cu[s0 + q] - c0;
        out->sh.cu_seqlens = out->cu;
        out->sh.num_seqs = n;
        out->sh.seq = G.cu[s0 + n] - c0;
        out->tok0 = c0;
        int64_t b = 0;
        for (int q = 0; q < s0; ++q) b += ceil_div64(G.cu[q + 1] - G.cu[q], G.base.block_size);
        out->blk0 = b;
    } else {
        out->sh.batch = n;
        out->tok0 = (int64_t)s0 * G.base.seq;
        out->blk0 = (int64_t)s0 * ceil_div64(G.base.seq, G.base.block_size);
    }
}

moba_status check_groups(const Groups& G)
{
    for (int g = 0; g < G.n; ++g) {
        Group gr;
        group(G, g, &gr);
        Launch L;
        const moba_status st = make_launch(&gr.sh, &L, nullptr);
        if (st != MOBA_OK) return st;
    }
    return MOBA_OK;
}

size_t esize(const moba_shape* sh) { return sh->dtype == MOBA_BF16 ? 2 : 4; }

// element offsets of a group: token rows of q/k/v/o, idx rows, lse, centroids
template <typename P>
P* at(P* p, int64_t rows, size_t bytes_per_row)
{
    return p ? (P*)((char*)const_cast<void*>((const void*)p) + rows * (int64_t)bytes_per_row) : p;
}

}  // namespace

namespace one {
int64_t total_blocks_one(const moba_shape* shape)
{
    Launch L;
    if (make_launch(shape, &L, nullptr) != MOBA_OK) return -1;
    return L.st.total_blocks;
}

size_t attn_fwd_workspace_bytes_one(const moba_shape* shape)
{
    Launch Ll, La;
    if (attn_launch(shape, nullptr, &Ll, &La) != MOBA_OK) return 0;
    return layout(La, false, expands(Ll)).total;
}

size_t attn_bwd_workspace_bytes_one(const moba_shape* shape)
{
    Launch Ll, La;
    if (attn_launch(shape, nullptr, &Ll, &La) != MOBA_OK) return 0;
    return layout(La, true, expands(Ll)).total;
}

moba_status key_conv_one(const moba_shape* shape, const void* k, const float* w, int32_t width,
                          int32_t mode, void* k_out, float* cent, hipStream_t stream)
{
    Launch L;
    moba_status st = make_launch(shape, &L, stream);
    if (st != MOBA_OK) return st;
    if (mode != MOBA_CONV_PLAIN && mode != MOBA_CONV_SILU_RESIDUAL) return MOBA_ERR_INVALID_ARG;
    if (width < 1) return MOBA_ERR_INVALID_ARG;
    if (width > 8) return MOBA_ERR_UNSUPPORTED;
    if (!ptr_ok(k) || !ptr_ok(w) || !ptr_ok(k_out)) return MOBA_ERR_INVALID_ARG;
    if (cent && !aligned16(cent)) return MOBA_ERR_INVALID_ARG;
    if (k == k_out) return MOBA_ERR_INVALID_ARG;
    if (L.tokens == 0) return MOBA_OK;
    return hip_status(launch_conv_pool(L, k, w, width, mode, k_out, cent));
}

size_t key_conv_bwd_workspace_bytes_one(const moba_shape* shape, int32_t width)
{
    Launch L;
    if (make_launch(shape, &L, nullptr) != MOBA_OK || width < 1 || width > 8) return 0;
    return align256((size_t)L.st.total_blocks * L.st.H * L.D * width * 4);
}

moba_status key_conv_bwd_one(const moba_shape* shape, const void* k, const float* w, int32_t width,
                              int32_t mode, const void* dk_out, void* dk, float* dw, void* workspace,
                              size_t workspace_bytes, hipStream_t stream)
{
    Launch L;
    moba_status st = make_launch(shape, &L, stream);
    if (st != MOBA_OK) return st;
    if (mode != MOBA_CONV_PLAIN && mode != MOBA_CONV_SILU_RESIDUAL) return MOBA_ERR_INVALID_ARG;
    if (width < 1) return MOBA_ERR_INVALID_ARG;
    if (width > 8) return MOBA_ERR_UNSUPPORTED;
    if (!ptr_ok(k) || !ptr_ok(w) || !ptr_ok(dk_out) || !ptr_ok(dk) || !ptr_ok(dw))
        return MOBA_ERR_INVALID_ARG;
    if (dk == k || dk == dk_out) return MOBA_ERR_INVALID_ARG;
    const size_t need = key_conv_bwd_workspace_bytes_one(shape, width);
    if (!workspace || ((uintptr_t)workspace & 255u) != 0) return MOBA_ERR_INVALID_ARG;
    if (workspace_bytes < need) return MOBA_ERR_WORKSPACE_TOO_SMALL;
    return hip_status(launch_conv_bwd(L, k, w, width, mode, dk_out, dk, (float*)workspace));
}

moba_status centroids_one(const moba_shape* shape, const void* k, float* cent, hipStream_t stream)
{
    Launch L;
    moba_status st = make_launch(shape, &L, stream);
    if (st != MOBA_OK) return st;
    if (!ptr_ok(k) || !ptr_ok(cent)) return MOBA_ERR_INVALID_ARG;
    if (L.tokens == 0) return MOBA_OK;
    return hip_status(launch_conv_pool(L, k, nullptr, 0, 0, nullptr, cent));
}

size_t route_topk_workspace_bytes_one(const moba_shape* shape)
{
    Launch L;
    if (make_launch(shape, &L, nullptr) != MOBA_OK) return 0;
    return std::max(route_ws_bytes(L), (size_t)256);
}

// every check of moba_route_topk on one group, without launching
moba_status route_topk_ok(const moba_shape* shape, const void* q, const float* cent,
                          const int32_t* idx, const void* workspace, size_t workspace_bytes)
{
    Launch L;
    moba_status st = make_launch(shape, &L, nullptr);
    if (st != MOBA_OK) return st;
    if (!ptr_ok(q) || !ptr_ok(cent) || !idx_ok(idx)) return MOBA_ERR_INVALID_ARG;
    if (!workspace || ((uintptr_t)workspace & 255u) != 0) return MOBA_ERR_INVALID_ARG;
    if (workspace_bytes < std::max(route_ws_bytes(L), (size_t)256)) return MOBA_ERR_WORKSPACE_TOO_SMALL;
    return MOBA_OK;
}

moba_status route_topk_one(const moba_shape* shape, const void* q, const float* cent, int32_t* idx,
                            void* workspace, size_t workspace_bytes, hipStream_t stream)
{
    moba_status st = route_topk_ok(shape, q, cent, idx, workspace, workspace_bytes);
    if (st != MOBA_OK) return st;
    Launch L;
    st = make_launch(shape, &L, stream);
    if (st != MOBA_OK) return st;
    if (L.tokens == 0) return MOBA_OK;
    return hip_status(launch_route(L, q, cent, workspace, idx));
}

// whether one group's routing workspace fits the fixed scratch buffer
moba_status route_noalloc_fits(const moba_shape* shape)
{
    Launch L;
    const moba_status st = make_launch(shape, &L, nullptr);
    if (st != MOBA_OK) return st;
    if (L.dtype == MOBA_BF16 && route_ws_bytes(L) > (size_t)MOBA_ROUTE_SCRATCH_BYTES)
        return MOBA_ERR_WORKSPACE_TOO_SMALL;
    return MOBA_OK;
}

moba_status route_topk_noalloc_one(const moba_shape* shape, const void* q, const float* cent,
                                    int32_t* idx, hipStream_t stream)
{
    Launch L;
    moba_status st = make_launch(shape, &L, stream);
    if (st != MOBA_OK) return st;
    if (!ptr_ok(q) || !ptr_ok(cent) || !idx_ok(idx)) return MOBA_ERR_INVALID_ARG;
    st = route_noalloc_fits(shape);
    if (st != MOBA_OK) return st;
    if (L.tokens == 0) return MOBA_OK;
    void* ws = nullptr;
    hipError_t e = route_scratch(&ws);
    if (e != hipSuccess) return MOBA_ERR_HIP;
    return hip_status(launch_route(L, q, cent, ws, idx));
}

// the index pass on the (possibly expanded) selection
hipError_t run_index(const Launch& Ll, const Launch& La, const WsLayout& ws, char* wsp,
                     const int32_t* idx, bool det = false)
{
    if (expands(Ll)) {
        int32_t* px = (int32_t*)(wsp + ws.px_off);
        hipError_t e = launch_expand_idx(Ll, La.st.B, La.st.K, idx, px);
        if (e != hipSuccess) return e;
        idx = px;
    }
    return launch_inv(La, ws, wsp, idx, det);
}

moba_status attn_index_one(const moba_shape* shape, const int32_t* idx, void* workspace,
                            size_t workspace_bytes, hipStream_t stream)
{
    Launch Ll, L;
    moba_status st = attn_launch(shape, stream, &Ll, &L);
    if (st != MOBA_OK) return st;
    if (!idx_ok(idx)) return MOBA_ERR_INVALID_ARG;
    WsLayout ws;
    st = check_ws(L, workspace, workspace_bytes, &ws, false, expands(Ll));
    if (st != MOBA_OK) return st;
    if (L.tokens == 0) return MOBA_OK;
    return hip_status(run_index(Ll, L, ws, (char*)workspace, idx));
}

moba_status attn_routed_one(const moba_shape* shape, const void* q, const void* k, const void* v,
                             float softmax_scale, void* workspace, size_t workspace_bytes,
                             hipStream_t stream)
{
    Launch Ll, L;
    moba_status st = attn_launch(shape, stream, &Ll, &L);
    if (st != MOBA_OK) return st;
    if (!ptr_ok(q) || !ptr_ok(k) || !ptr_ok(v)) return MOBA_ERR_INVALID_ARG;
    WsLayout ws;
    st = check_ws(L, workspace, workspace_bytes, &ws, false, expands(Ll));
    if (st != MOBA_OK) return st;
    if (L.tokens == 0) return MOBA_OK;
    return hip_status(launch_routed_attn(L, ws, (char*)workspace, q, k, v,
                                         resolve_scale(softmax_scale, L.D)));
}

moba_status attn_combine_one(const moba_shape* shape, const void* q, const void* k, const void* v,
                              const int32_t* idx, float softmax_scale, void* o, float* lse,
                              void* workspace, size_t workspace_bytes, hipStream_t stream)
{
    Launch Ll, L;
    moba_status st = attn_launch(shape, stream, &Ll, &L);
    if (st != MOBA_OK) return st;
    if (!ptr_ok(q) || !ptr_ok(k) || !ptr_ok(v) || !idx_ok(idx) || !ptr_ok(o))
        return MOBA_ERR_INVALID_ARG;
    if (lse && ((uintptr_t)lse & 3u)) return MOBA_ERR_INVALID_ARG;
    WsLayout ws;
    st = check_ws(L, workspace, workspace_bytes, &ws, false, expands(Ll));
    if (st != MOBA_OK) return st;
    if (L.tokens == 0) return MOBA_OK;
    return hip_status(launch_diag_combine(L, ws, (char*)workspace, q, k, v, idx,
                                          resolve_scale(softmax_scale, L.D), o, lse));
}

moba_status attn_fwd_one(const moba_shape* shape, const void* q, const void* k, const void* v,
                          const int32_t* idx, float softmax_scale, void* o, float* lse,
                          void* workspace, size_t workspace_bytes, hipStream_t stream)
{
    moba_status st = attn_index_one(shape, idx, workspace, workspace_bytes, stream);
    if (st != MOBA_OK) return st;
    st = attn_routed_one(shape, q, k, v, softmax_scale, workspace, workspace_bytes, stream);
    if (st != MOBA_OK) return st;
    return attn_combine_one(shape, q, k, v, idx, softmax_scale, o, lse, workspace,
                             workspace_bytes, stream);
}

moba_status attn_fwd_blasst_one(const moba_shape* shape, const void* q, const void* k, const void* v,
                                const int32_t* idx, float softmax_scale, float blasst_lambda, void* o,
                                float* lse, int32_t* kept, void* workspace, size_t workspace_bytes,
                                hipStream_t stream)
{
    Launch Ll, L;
    moba_status st = attn_launch(shape, stream, &Ll, &L);
    if (st != MOBA_OK) return st;
    if (!(blasst_lambda >= 0.f && blasst_lambda <= 1.f)) return MOBA_ERR_INVALID_ARG;
    if (expands(Ll)) return MOBA_ERR_UNSUPPORTED;
    if (!ptr_ok(q) || !ptr_ok(k) || !ptr_ok(v) || !idx_ok(idx) || !ptr_ok(o)) return MOBA_ERR_INVALID_ARG;
    if (lse && ((uintptr_t)lse & 3u)) return MOBA_ERR_INVALID_ARG;
    if (kept && (!idx_ok(kept) || kept == idx)) return MOBA_ERR_INVALID_ARG;
    WsLayout ws;
    st = check_ws(L, workspace, workspace_bytes, &ws, false, false);
    if (st != MOBA_OK) return st;
    if (L.tokens == 0) return MOBA_OK;
    char* wsp = (char*)workspace;
    const float scale = resolve_scale(softmax_scale, L.D);
    hipError_t e = run_index(Ll, L, ws, wsp, idx);
    if (e == hipSuccess) e = launch_routed_attn(L, ws, wsp, q, k, v, scale, blasst_lambda > 0.f);
    if (e == hipSuccess) e = launch_diag_combine(L, ws, wsp, q, k, v, idx, scale, o, lse, blasst_lambda, kept);
    return hip_status(e);
}

// own_listed: the own block is attended only where idx lists it (the
// kept selection of a BLASST forward); otherwise always, as in the forward
moba_status attn_bwd_one(const moba_shape* shape, const void* q, const void* k, const void* v,
                          const int32_t* idx, float softmax_scale, const void* o, const float* lse,
                          const void* dout, void* dq, void* dk, void* dv, void* workspace,
                          size_t workspace_bytes, hipStream_t stream, bool own_listed = false)
{
    Launch Ll, L;
    moba_status st = attn_launch(shape, stream, &Ll, &L);
    if (st != MOBA_OK) return st;
    if (own_listed && expands(Ll)) return MOBA_ERR_UNSUPPORTED;
    if (!ptr_ok(q) || !ptr_ok(k) || !ptr_ok(v) || !idx_ok(idx) || !ptr_ok(o) || !ptr_ok(lse) ||
        !ptr_ok(dout) || !ptr_ok(dq) || !ptr_ok(dk) || !ptr_ok(dv))
        return MOBA_ERR_INVALID_ARG;
    const void* ins[] = {q, k, v, o, dout, (const void*)lse, (const void*)idx};
    const void* outs[] = {dq, dk, dv};
    for (const void* a : outs) {
        for (const void* b : ins)
            if (a == b) return MOBA_ERR_INVALID_ARG;
    }
    if (dq == dk || dq == dv || dk == dv) return MOBA_ERR_INVALID_ARG;
    WsLayout ws;
    st = check_ws(L, workspace, workspace_bytes, &ws, true, expands(Ll));
    if (st != MOBA_OK) return st;
    if (L.tokens == 0) return MOBA_OK;
    // repeatable list order: dK / dV sum each list's rows in that order
    hipError_t e = run_index(Ll, L, ws, (char*)workspace, idx, true);
    if (e != hipSuccess) return MOBA_ERR_HIP;
    uint8_t* own = nullptr;
    if (own_listed) {
        own = (uint8_t*)workspace + ws.own_off;
        e = launch_own_flags(L, idx, own);
        if (e != hipSuccess) return MOBA_ERR_HIP;
    }
    const float scale = resolve_scale(softmax_scale, L.D);
    if (L.dtype == MOBA_F32) {
        const int32_t* ia = expands(Ll) ? (const int32_t*)((char*)workspace + ws.px_off) : idx;
        return hip_status(launch_attn_bwd_f32(L, ws, (char*)workspace, ia, q, k, v, o, lse, dout, scale,
                                              dq, dk, dv, own));
    }
    return hip_status(launch_attn_bwd(L, ws, (char*)workspace, q, k, v, o, lse, dout, scale, dq, dk, dv,
                                      own));
}

}  // namespace one

extern "C" {

int32_t moba_abi_version(void) { return MOBA_ABI_VERSION; }

moba_status moba_debug_violations(uint32_t* flags)
{
#ifdef MOBA_DEBUG_BOUNDS
    if (!flags) return MOBA_ERR_INVALID_ARG;
    *flags = dbg_take_attn() | dbg_take_attn_bwd() | dbg_take_attn_bwd_f32() | dbg_take_invert();
    return MOBA_OK;
#else
    (void)flags;
    return MOBA_ERR_UNSUPPORTED;
#endif
}

// (an int: a C caller may pass any value, which a C++ enum parameter of
// this range could not hold without undefined behaviour)
const char* moba_status_string(int32_t s)
{
    switch (s) {
        case MOBA_OK: return "ok";
        case MOBA_ERR_INVALID_ARG: return "invalid argument";
        case MOBA_ERR_UNSUPPORTED: return "unsupported shape or parameter";
        case MOBA_ERR_WORKSPACE_TOO_SMALL: return "workspace too small";
        case MOBA_ERR_HIP: return "HIP launch error";
    }
    return "unknown status";
}

// ---------------------------------------------------------------- groups --
#define MOBA_GROUPS(shape)                      \
    Groups G;                                   \
    {                                           \
        moba_status st_ = split(shape, &G);     \
        if (st_ == MOBA_OK) st_ = check_groups(G); \
        if (st_ != MOBA_OK) return st_;         \
    }

int64_t moba_total_blocks(const moba_shape* shape)
{
    Groups G;
    if (split(shape, &G) != MOBA_OK) return -1;
    int64_t n = 0;
    for (int g = 0; g < G.n; ++g) {
        Group gr;
        group(G, g, &gr);
        const int64_t b = one::total_blocks_one(&gr.sh);
        if (b < 0) return -1;
        n += b;
    }
    return n;
}

size_t moba_attn_fwd_workspace_bytes(const moba_shape* shape)
{
    Groups G;
    if (split(shape, &G) != MOBA_OK) return 0;
    size_t n = 0;
    for (int g = 0; g < G.n; ++g) {
        Group gr;
        group(G, g, &gr);
        Launch Ll, La;
        if (attn_launch(&gr.sh, nullptr, &Ll, &La) != MOBA_OK) return 0;
        n += one::attn_fwd_workspace_bytes_one(&gr.sh);
    }
    return n;
}

size_t moba_attn_bwd_workspace_bytes(const moba_shape* shape)
{
    Groups G;
    if (split(shape, &G) != MOBA_OK) return 0;
    size_t n = 0;
    for (int g = 0; g < G.n; ++g) {
        Group gr;
        group(G, g, &gr);
        Launch Ll, La;
        if (attn_launch(&gr.sh, nullptr, &Ll, &La) != MOBA_OK) return 0;
        n += one::attn_bwd_workspace_bytes_one(&gr.sh);
    }
    return n;
}

moba_status moba_key_conv(const moba_shape* shape, const void* k, const float* w, int32_t width,
                          int32_t mode, void* k_out, float* cent, hipStream_t stream)
{
    MOBA_GROUPS(shape);
    const size_t row = (size_t)shape->heads * shape->head_dim;
    for (int g = 0; g < G.n; ++g) {
        Group gr;
        group(G, g, &gr);
        moba_status st = one::key_conv_one(&gr.sh, at(k, gr.tok0, row * esize(shape)), w, width, mode,
                                           at(k_out, gr.tok0, row * esize(shape)),
                                           at(cent, gr.blk0, row * 4), stream);
        if (st != MOBA_OK) return st;
    }
    return MOBA_OK;
}

size_t moba_key_conv_bwd_workspace_bytes(const moba_shape* shape, int32_t width)
{
    const int64_t nb = moba_total_blocks(shape);
    if (nb < 0 || width < 1 || width > 8) return 0;
    return align256((size_t)nb * shape->heads * shape->head_dim * width * 4);
}

moba_status moba_key_conv_bwd(const moba_shape* shape, const void* k, const float* w, int32_t width,
                              int32_t mode, const void* dk_out, void* dk, float* dw, void* workspace,
                              size_t workspace_bytes, hipStream_t stream)
{
    MOBA_GROUPS(shape);
    if (mode != MOBA_CONV_PLAIN && mode != MOBA_CONV_SILU_RESIDUAL) return MOBA_ERR_INVALID_ARG;
    if (width < 1) return MOBA_ERR_INVALID_ARG;
    if (width > 8) return MOBA_ERR_UNSUPPORTED;
    if (!ptr_ok(k) || !ptr_ok(w) || !ptr_ok(dk_out) || !ptr_ok(dk) || !ptr_ok(dw))
        return MOBA_ERR_INVALID_ARG;
    if (dk == k || dk == dk_out) return MOBA_ERR_INVALID_ARG;
    const size_t need = moba_key_conv_bwd_workspace_bytes(shape, width);
    if (!workspace || ((uintptr_t)workspace & 255u) != 0) return MOBA_ERR_INVALID_ARG;
    if (workspace_bytes < need) return MOBA_ERR_WORKSPACE_TOO_SMALL;
    const size_t row = (size_t)shape->heads * shape->head_dim;
    const size_t part = row * (size_t)width;            // dw partial floats per block
    // every group's pass first (dk and per-block dw partials), then one fixed-order sum
    for (int g = 0; g < G.n; ++g) {
        Group gr;
        group(G, g, &gr);
        moba_status st = one::key_conv_bwd_one(&gr.sh, at(k, gr.tok0, row * esize(shape)), w, width, mode,
                                               at(dk_out, gr.tok0, row * esize(shape)),
                                               at(dk, gr.tok0, row * esize(shape)), dw,
                                               at(workspace, gr.blk0, part * 4),
                                               workspace_bytes - (size_t)gr.blk0 * part * 4, stream);
        if (st != MOBA_OK) return st;
    }
    return hip_status(launch_conv_dw_reduce(stream, (int)moba_total_blocks(shape), (int)part,
                                            (const float*)workspace, dw));
}

moba_status moba_centroids(const moba_shape* shape, const void* k, float* cent, hipStream_t stream)
{
    MOBA_GROUPS(shape);
    const size_t row = (size_t)shape->heads * shape->head_dim;
    for (int g = 0; g < G.n; ++g) {
        Group gr;
        group(G, g, &gr);
        moba_status st = one::centroids_one(&gr.sh, at(k, gr.tok0, row * esize(shape)),
                                            at(cent, gr.blk0, row * 4), stream);
        if (st != MOBA_OK) return st;
    }
    return MOBA_OK;
}

size_t moba_route_topk_workspace_bytes(const moba_shape* shape)
{
    Groups G;
    if (split(shape, &G) != MOBA_OK) return 0;
    size_t n = 0;
    for (int g = 0; g < G.n; ++g) {
        Group gr;
        group(G, g, &gr);
        const size_t b = one::route_topk_workspace_bytes_one(&gr.sh);
        if (b == 0) return 0;
        n = std::max(n, b);
    }
    return n;
}

moba_status moba_route_topk(const moba_shape* shape, const void* q, const float* cent, int32_t* idx,
                            void* workspace, size_t workspace_bytes, hipStream_t stream)
{
    MOBA_GROUPS(shape);
    if (!ptr_ok(idx)) return MOBA_ERR_INVALID_ARG;
    const size_t row = (size_t)shape->heads * shape->head_dim;
    const size_t irow = (size_t)shape->heads * (shape->top_k > 0 ? shape->top_k : 0) * 4;
    // every group is checked (arguments, workspace size) before the first launch
    for (int g = 0; g < G.n; ++g) {
        Group gr;
        group(G, g, &gr);
        const moba_status st = one::route_topk_ok(&gr.sh, at(q, gr.tok0, row * esize(shape)),
                                                  at(cent, gr.blk0, row * 4), at(idx, gr.tok0, irow),
                                                  workspace, workspace_bytes);
        if (st != MOBA_OK) return st;
    }
    for (int g = 0; g < G.n; ++g) {
        Group gr;
        group(G, g, &gr);
        moba_status st = one::route_topk_one(&gr.sh, at(q, gr.tok0, row * esize(shape)),
                                             at(cent, gr.blk0, row * 4), at(idx, gr.tok0, irow),
                                             workspace, workspace_bytes, stream);
        if (st != MOBA_OK) return st;
    }
    return MOBA_OK;
}

moba_status moba_route_topk_noalloc(const moba_shape* shape, const void* q, const float* cent,
                                    int32_t* idx, hipStream_t stream)
{
    MOBA_GROUPS(shape);
    if (!ptr_ok(idx)) return MOBA_ERR_INVALID_ARG;
    // every group must fit the scratch buffer before the first launch
    for (int g = 0; g < G.n; ++g) {
        Group gr;
        group(G, g, &gr);
        const moba_status st = one::route_noalloc_fits(&gr.sh);
        if (st != MOBA_OK) return st;
    }
    const size_t row = (size_t)shape->heads * shape->head_dim;
    const size_t irow = (size_t)shape->heads * (shape->top_k > 0 ? shape->top_k : 0) * 4;
    for (int g = 0; g < G.n; ++g) {
        Group gr;
        group(G, g, &gr);
        moba_status st = one::route_topk_noalloc_one(&gr.sh, at(q, gr.tok0, row * esize(shape)),
                                                     at(cent, gr.blk0, row * 4), at(idx, gr.tok0, irow),
                                                     stream);
        if (st != MOBA_OK) return st;
    }
    return MOBA_OK;
}

#define MOBA_ATTN_GROUPS(bwd_)                                                           \
    const size_t row = (size_t)shape->heads * shape->head_dim;                          \
    const size_t irow = (size_t)shape->heads * (shape->top_k > 0 ? shape->top_k : 0) * 4; \
    const size_t lrow = (size_t)shape->heads * 4;                                       \
    (void)row; (void)irow; (void)lrow;                                                  \
    const size_t need_ = (bwd_) ? moba_attn_bwd_workspace_bytes(shape)                   \
                                : moba_attn_fwd_workspace_bytes(shape);                  \
    if (G.n > 1 && need_ > 0 && (!workspace || ((uintptr_t)workspace & 255u) != 0))    \
        return MOBA_ERR_INVALID_ARG;                                                    \
    if (G.n > 1 && workspace_bytes < need_) return MOBA_ERR_WORKSPACE_TOO_SMALL;        \
    size_t wsoff = 0;

moba_status moba_attn_index(const moba_shape* shape, const int32_t* idx, void* workspace,
                            size_t workspace_bytes, hipStream_t stream)
{
    MOBA_GROUPS(shape);
    if (!ptr_ok(idx)) return MOBA_ERR_INVALID_ARG;
    MOBA_ATTN_GROUPS(false);
    for (int g = 0; g < G.n; ++g) {
        Group gr;
        group(G, g, &gr);
        const size_t wsz = one::attn_fwd_workspace_bytes_one(&gr.sh);
        moba_status st = one::attn_index_one(&gr.sh, at(idx, gr.tok0, irow), at(workspace, (int64_t)wsoff, 1),
                                             G.n > 1 ? wsz : workspace_bytes, stream);
        if (st != MOBA_OK) return st;
        wsoff += wsz;
    }
    return MOBA_OK;
}

moba_status moba_attn_routed(const moba_shape* shape, const void* q, const void* k, const void* v,
                             float softmax_scale, void* workspace, size_t workspace_bytes,
                             hipStream_t stream)
{
    MOBA_GROUPS(shape);
    MOBA_ATTN_GROUPS(false);
    const size_t er = row * esize(shape);
    for (int g = 0; g < G.n; ++g) {
        Group gr;
        group(G, g, &gr);
        const size_t wsz = one::attn_fwd_workspace_bytes_one(&gr.sh);
        moba_status st = one::attn_routed_one(&gr.sh, at(q, gr.tok0, er), at(k, gr.tok0, er),
                                              at(v, gr.tok0, er), softmax_scale,
                                              at(workspace, (int64_t)wsoff, 1),
                                              G.n > 1 ? wsz : workspace_bytes, stream);
        if (st != MOBA_OK) return st;
        wsoff += wsz;
    }
    return MOBA_OK;
}

moba_status moba_attn_combine(const moba_shape* shape, const void* q, const void* k, const void* v,
                              const int32_t* idx, float softmax_scale, void* o, float* lse,
                              void* workspace, size_t workspace_bytes, hipStream_t stream)
{
    MOBA_GROUPS(shape);
    if (!ptr_ok(idx)) return MOBA_ERR_INVALID_ARG;
    if (lse && !aligned16(lse)) return MOBA_ERR_INVALID_ARG;
    MOBA_ATTN_GROUPS(false);
    const size_t er = row * esize(shape);
    for (int g = 0; g < G.n; ++g) {
        Group gr;
        group(G, g, &gr);
        const size_t wsz = one::attn_fwd_workspace_bytes_one(&gr.sh);
        moba_status st = one::attn_combine_one(&gr.sh, at(q, gr.tok0, er), at(k, gr.tok0, er),
                                               at(v, gr.tok0, er), at(idx, gr.tok0, irow), softmax_scale,
                                               at(o, gr.tok0, er), at(lse, gr.tok0, lrow),
                                               at(workspace, (int64_t)wsoff, 1),
                                               G.n > 1 ? wsz : workspace_bytes, stream);
        if (st != MOBA_OK) return st;
        wsoff += wsz;
    }
    return MOBA_OK;
}

moba_status moba_attn_fwd(const moba_shape* shape, const void* q, const void* k, const void* v,
                          const int32_t* idx, float softmax_scale, void* o, float* lse,
                          void* workspace, size_t workspace_bytes, hipStream_t stream)
{
    moba_status st = moba_attn_index(shape, idx, workspace, workspace_bytes, stream);
    if (st != MOBA_OK) return st;
    st = moba_attn_routed(shape, q, k, v, softmax_scale, workspace, workspace_bytes, stream);
    if (st != MOBA_OK) return st;
    return moba_attn_combine(shape, q, k, v, idx, softmax_scale, o, lse, workspace,
                             workspace_bytes, stream);
}

moba_status moba_attn_fwd_blasst(const moba_shape* shape, const void* q, const void* k, const void* v,
                                 const int32_t* idx, float softmax_scale, float blasst_lambda, void* o,
                                 float* lse, int32_t* kept_idx, void* workspace, size_t workspace_bytes,
                                 hipStream_t stream)
{
    MOBA_GROUPS(shape);
    if (!ptr_ok(idx)) return MOBA_ERR_INVALID_ARG;
    if (lse && !aligned16(lse)) return MOBA_ERR_INVALID_ARG;
    if (kept_idx && (!aligned16(kept_idx) || kept_idx == idx)) return MOBA_ERR_INVALID_ARG;
    MOBA_ATTN_GROUPS(false);
    const size_t er = row * esize(shape);
    for (int g = 0; g < G.n; ++g) {
        Group gr;
        group(G, g, &gr);
        const size_t wsz = one::attn_fwd_workspace_bytes_one(&gr.sh);
        moba_status st = one::attn_fwd_blasst_one(&gr.sh, at(q, gr.tok0, er), at(k, gr.tok0, er),
                                                  at(v, gr.tok0, er), at(idx, gr.tok0, irow), softmax_scale,
                                                  blasst_lambda, at(o, gr.tok0, er), at(lse, gr.tok0, lrow),
                                                  at(kept_idx, gr.tok0, irow), at(workspace, (int64_t)wsoff, 1),
                                                  G.n > 1 ? wsz : workspace_bytes, stream);
        if (st != MOBA_OK) return st;
        wsoff += wsz;
    }
    return MOBA_OK;
}

static moba_status attn_bwd_groups(const moba_shape* shape, const void* q, const void* k, const void* v,
                                   const int32_t* idx, float softmax_scale, const void* o, const float* lse,
                                   const void* dout, void* dq, void* dk, void* dv, void* workspace,
                                   size_t workspace_bytes, hipStream_t stream, bool own_listed)
{
    MOBA_GROUPS(shape);
    if (!ptr_ok(idx) || !ptr_ok(lse)) return MOBA_ERR_INVALID_ARG;
    MOBA_ATTN_GROUPS(true);
    const size_t er = row * esize(shape);
    for (int g = 0; g < G.n; ++g) {
        Group gr;
        group(G, g, &gr);
        const size_t wsz = one::attn_bwd_workspace_bytes_one(&gr.sh);
        moba_status st = one::attn_bwd_one(&gr.sh, at(q, gr.tok0, er), at(k, gr.tok0, er), at(v, gr.tok0, er),
                                           at(idx, gr.tok0, irow), softmax_scale, at(o, gr.tok0, er),
                                           at(lse, gr.tok0, lrow), at(dout, gr.tok0, er), at(dq, gr.tok0, er),
                                           at(dk, gr.tok0, er), at(dv, gr.tok0, er),
                                           at(workspace, (int64_t)wsoff, 1),
                                           G.n > 1 ? wsz : workspace_bytes, stream, own_listed);
        if (st != MOBA_OK) return st;
        wsoff += wsz;
    }
    return MOBA_OK;
}

moba_status moba_attn_bwd(const moba_shape* shape, const void* q, const void* k, const void* v,
                          const int32_t* idx, float softmax_scale, const void* o, const float* lse,
                          const void* dout, void* dq, void* dk, void* dv, void* workspace,
                          size_t workspace_bytes, hipStream_t stream)
{
    return attn_bwd_groups(shape, q, k, v, idx, softmax_scale, o, lse, dout, dq, dk, dv, workspace,
                           workspace_bytes, stream, false);
}

moba_status moba_attn_bwd_blasst(const moba_shape* shape, const void* q, const void* k, const void* v,
                                 const int32_t* kept_idx, float softmax_scale, const void* o,
                                 const float* lse, const void* dout, void* dq, void* dk, void* dv,
                                 void* workspace, size_t workspace_bytes, hipStream_t stream)
{
    return attn_bwd_groups(shape, q, k, v, kept_idx, softmax_scale, o, lse, dout, dq, dk, dv, workspace,
                           workspace_bytes, stream, true);
}

}  // extern "C"
