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
    // blocks of 256 / 512 keys are attended as 2 / 4 blocks of 128: the
    // expanded selection must fit 32 slots
    if (sh->block_size > 128 && sh->top_k > 8) return MOBA_ERR_UNSUPPORTED;
    // the fp32 router runs one thread per query of a block (<= 256)
    if (sh->dtype == MOBA_F32 && sh->block_size > 256) return MOBA_ERR_UNSUPPORTED;
    // fp32 keeps a whole (128-key) block of K and V in LDS: B * d <= 8192
    const int att_b = sh->block_size < 128 ? sh->block_size : 128;
    if (sh->dtype == MOBA_F32 && sh->head_dim * att_b > 8192) return MOBA_ERR_UNSUPPORTED;

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
        const int64_t cap = (int64_t)Ls * st.K / kItemRows + n;
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
// expand: the selection is re-expressed in 128-key blocks first (block
// sizes 256 / 512); L is then the 128-key launch
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
        }
    }
    if (bwd) {
        w.rs_bytes = rows * 8;
        const size_t ent_rows = st.K > 1 ? (size_t)st.ebase[st.nseq] : 0;
        w.pq_bytes = (ent_rows + rows) * L.D * 4;
    }
    if (expand) w.px_bytes = rows * st.K * 4;
    size_t off = 0;
    w.cmat_off = off;  off += align256(w.cmat_bytes);
    w.items_off = off; off += align256(w.items_bytes);
    w.ent_off = off;   off += align256(w.ent_bytes);
    w.rev_off = off;   off += align256(w.rev_bytes);
    w.po_off = off;    off += align256(w.po_bytes);
    w.pl_off = off;    off += align256(w.pl_bytes);
    w.lst_off = off;   off += align256(w.lst_bytes);
    w.rs_off = off;    off += align256(w.rs_bytes);
    w.pq_off = off;    off += align256(w.pq_bytes);
    w.px_off = off;    off += align256(w.px_bytes);
    w.total = off;
    return w;
}

moba_status hip_status(hipError_t e) { return e == hipSuccess ? MOBA_OK : MOBA_ERR_HIP; }

bool ptr_ok(const void* p) { return p != nullptr && aligned16(p); }

// The attention entry points work on 128-key blocks when the shape's blocks
// are larger: Ll is the shape's own launch (routing granularity), La the
// one the attention kernels run with (block 128, top_k * B / 128 slots).
moba_status attn_launch(const moba_shape* sh, hipStream_t stream, Launch* Ll, Launch* La)
{
    moba_status st = make_launch(sh, Ll, stream);
    if (st != MOBA_OK) return st;
    if (sh->block_size <= 128) {
        *La = *Ll;
        return MOBA_OK;
    }
    moba_shape p = *sh;
    p.block_size = 128;
    p.top_k = sh->top_k * (sh->block_size / 128);
    return make_launch(&p, La, stream);
}

bool expands(const Launch& Ll) { return Ll.st.B > 128; }

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

}  // namespace

extern "C" {

int32_t moba_abi_version(void) { return MOBA_ABI_VERSION; }

const char* moba_status_string(moba_status s)
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

int64_t moba_total_blocks(const moba_shape* shape)
{
    Launch L;
    if (make_launch(shape, &L, nullptr) != MOBA_OK) return -1;
    return L.st.total_blocks;
}

size_t moba_attn_fwd_workspace_bytes(const moba_shape* shape)
{
    Launch Ll, La;
    if (attn_launch(shape, nullptr, &Ll, &La) != MOBA_OK) return 0;
    return layout(La, false, expands(Ll)).total;
}

size_t moba_attn_bwd_workspace_bytes(const moba_shape* shape)
{
    Launch Ll, La;
    if (attn_launch(shape, nullptr, &Ll, &La) != MOBA_OK) return 0;
    return layout(La, true, expands(Ll)).total;
}

moba_status moba_key_conv(const moba_shape* shape, const void* k, const float* w, int32_t width,
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

size_t moba_key_conv_bwd_workspace_bytes(const moba_shape* shape, int32_t width)
{
    Launch L;
    if (make_launch(shape, &L, nullptr) != MOBA_OK || width < 1 || width > 8) return 0;
    return align256((size_t)L.st.total_blocks * L.st.H * L.D * width * 4);
}

moba_status moba_key_conv_bwd(const moba_shape* shape, const void* k, const float* w, int32_t width,
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
    const size_t need = moba_key_conv_bwd_workspace_bytes(shape, width);
    if (!workspace || ((uintptr_t)workspace & 255u) != 0) return MOBA_ERR_INVALID_ARG;
    if (workspace_bytes < need) return MOBA_ERR_WORKSPACE_TOO_SMALL;
    return hip_status(launch_conv_bwd(L, k, w, width, mode, dk_out, dk, dw, (float*)workspace));
}

moba_status moba_centroids(const moba_shape* shape, const void* k, float* cent, hipStream_t stream)
{
    Launch L;
    moba_status st = make_launch(shape, &L, stream);
    if (st != MOBA_OK) return st;
    if (!ptr_ok(k) || !ptr_ok(cent)) return MOBA_ERR_INVALID_ARG;
    if (L.tokens == 0) return MOBA_OK;
    return hip_status(launch_conv_pool(L, k, nullptr, 0, 0, nullptr, cent));
}

size_t moba_route_topk_workspace_bytes(const moba_shape* shape)
{
    Launch L;
    if (make_launch(shape, &L, nullptr) != MOBA_OK) return 0;
    return std::max(route_ws_bytes(L), (size_t)256);
}

moba_status moba_route_topk(const moba_shape* shape, const void* q, const float* cent, int32_t* idx,
                            void* workspace, size_t workspace_bytes, hipStream_t stream)
{
    Launch L;
    moba_status st = make_launch(shape, &L, stream);
    if (st != MOBA_OK) return st;
    if (!ptr_ok(q) || !ptr_ok(cent) || !ptr_ok(idx)) return MOBA_ERR_INVALID_ARG;
    if (!workspace || ((uintptr_t)workspace & 255u) != 0) return MOBA_ERR_INVALID_ARG;
    if (workspace_bytes < std::max(route_ws_bytes(L), (size_t)256)) return MOBA_ERR_WORKSPACE_TOO_SMALL;
    if (L.tokens == 0) return MOBA_OK;
    return hip_status(launch_route(L, q, cent, workspace, idx));
}

// the index pass on the (possibly expanded) selection
hipError_t run_index(const Launch& Ll, const Launch& La, const WsLayout& ws, char* wsp,
                     const int32_t* idx, bool det = false)
{
    if (expands(Ll)) {
        int32_t* px = (int32_t*)(wsp + ws.px_off);
        hipError_t e = launch_expand_idx(Ll, La.st.K, idx, px);
        if (e != hipSuccess) return e;
        idx = px;
    }
    return launch_inv(La, ws, wsp, idx, det);
}

moba_status moba_attn_index(const moba_shape* shape, const int32_t* idx, void* workspace,
                            size_t workspace_bytes, hipStream_t stream)
{
    Launch Ll, L;
    moba_status st = attn_launch(shape, stream, &Ll, &L);
    if (st != MOBA_OK) return st;
    if (!ptr_ok(idx)) return MOBA_ERR_INVALID_ARG;
    WsLayout ws;
    st = check_ws(L, workspace, workspace_bytes, &ws, false, expands(Ll));
    if (st != MOBA_OK) return st;
    if (L.tokens == 0) return MOBA_OK;
    return hip_status(run_index(Ll, L, ws, (char*)workspace, idx));
}

moba_status moba_attn_routed(const moba_shape* shape, const void* q, const void* k, const void* v,
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

moba_status moba_attn_combine(const moba_shape* shape, const void* q, const void* k, const void* v,
                              const int32_t* idx, float softmax_scale, void* o, float* lse,
                              void* workspace, size_t workspace_bytes, hipStream_t stream)
{
    Launch Ll, L;
    moba_status st = attn_launch(shape, stream, &Ll, &L);
    if (st != MOBA_OK) return st;
    if (!ptr_ok(q) || !ptr_ok(k) || !ptr_ok(v) || !ptr_ok(idx) || !ptr_ok(o))
        return MOBA_ERR_INVALID_ARG;
    if (lse && !aligned16(lse)) return MOBA_ERR_INVALID_ARG;
    WsLayout ws;
    st = check_ws(L, workspace, workspace_bytes, &ws, false, expands(Ll));
    if (st != MOBA_OK) return st;
    if (L.tokens == 0) return MOBA_OK;
    return hip_status(launch_diag_combine(L, ws, (char*)workspace, q, k, v, idx,
                                          resolve_scale(softmax_scale, L.D), o, lse));
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

moba_status moba_attn_bwd(const moba_shape* shape, const void* q, const void* k, const void* v,
                          const int32_t* idx, float softmax_scale, const void* o, const float* lse,
                          const void* dout, void* dq, void* dk, void* dv, void* workspace,
                          size_t workspace_bytes, hipStream_t stream)
{
    Launch Ll, L;
    moba_status st = attn_launch(shape, stream, &Ll, &L);
    if (st != MOBA_OK) return st;
    if (!ptr_ok(q) || !ptr_ok(k) || !ptr_ok(v) || !ptr_ok(idx) || !ptr_ok(o) || !ptr_ok(lse) ||
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
    const float scale = resolve_scale(softmax_scale, L.D);
    if (L.dtype == MOBA_F32) {
        const int32_t* ia = expands(Ll) ? (const int32_t*)((char*)workspace + ws.px_off) : idx;
        return hip_status(launch_attn_bwd_f32(L, ws, (char*)workspace, ia, q, k, v, o, lse, dout, scale,
                                              dq, dk, dv));
    }
    return hip_status(launch_attn_bwd(L, ws, (char*)workspace, q, k, v, o, lse, dout, scale, dq, dk, dv));
}

}  // extern "C"
