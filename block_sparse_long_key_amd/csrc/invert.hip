// invert.hip -- query-major block selections -> key-block-major query lists.
//
// "Optimizing Mixture of Block Attention", summary page, section "Tre Kernel
// Fusi": the top-k stage ends by turning the per-query block ids into a
// varlen layout indexed by key block, which the gather-and-densify forward
// consumes.  This is that step, written as a counting sort with no global
// atomics:
//   count   -- one workgroup per (sequence, head, chunk of query blocks):
//              LDS histogram of the routed past blocks; row of the count
//              matrix cm[chunk][j] for the lists j this chunk can reach;
//   scan    -- one workgroup per (sequence, head): list totals, list offsets,
//              per-chunk positions (in place), the work items (runs of
//              <= item_rows entries of one list) for the routed attention,
//              and the (first entry, count) of every whole list;
//   scatter -- same grid as count: entries (token << 5 | slot) written at the
//              chunk's positions with LDS cursors, and the reverse map
//              (query, slot) -> list position (-1 where nothing is routed),
//              stored head-major [H][tokens][K] so both its writer and its
//              reader (one query block of one head) touch contiguous runs.
// The own block is not listed (the own-block kernel handles it); -1 and
// out-of-range ids are skipped.  Order inside a list: the forward's fast
// placement depends on wave timing, which the routed attention does not
// depend on (each row of a tile is computed independently); the backward
// asks for a placement that depends only on idx (see inv_scatter_kernel).
#include "moba_internal.h"

namespace moba {
namespace {

constexpr int kThreads = 256;
constexpr int kScanThreads = 1024;
constexpr int kBatch = 16;        // idx words loaded ahead per thread
// largest blocks per sequence for the repeatable scatter (4 x 4 B of LDS
// cursors per block: 64 KB)
constexpr int kDetMaxBlocks = 4096;

// entry e -> token row e / K by a multiply-high with M = ceil(2^32 / K):
// e M / 2^32 exceeds e / K by less than e / 2^32, and the fractional part of
// e / K is at most (K-1) / K, so the floor is exact for e < 2^32 / K (every
// entry index of a chunk is below 2^18); token -> block by a shift (B is a
// power of two)
struct Div {
    uint32_t m;
    int lb;
    __device__ __forceinline__ Div(int K, int B)
        : m(0xffffffffu / (uint32_t)K + 1u), lb(31 - __builtin_clz((unsigned)B)) {}
    __device__ __forceinline__ int row(int e) const { return (int)__umulhi((uint32_t)e, m); }
    __device__ __forceinline__ int block(int t) const { return t >> lb; }
};

__device__ __forceinline__ int32_t* cm_base(const SegTable& st, int32_t* cmat, int s, int h)
{
    return cmat + st.cmbase[s] + (int64_t)h * seq_nchunk(st, s) * seq_nblk(st, s);
}

__global__ __launch_bounds__(kThreads) void inv_count_kernel(SegTable st, const int32_t* __restrict__ idx,
                                                            int32_t* __restrict__ cmat)
{
    extern __shared__ int32_t hist[];
    const int c = blockIdx.x, h = blockIdx.y;
    const int s = seq_of_chunk(st, c);
    const int cl = c - st.cbase[s];
    const int n = seq_nblk(st, s), L = seq_len(st, s), t0 = st.cu[s];
    const int B = st.B, K = st.K, H = st.H;
    const int ib0 = cl * st.chunk, ib1 = min(n, ib0 + st.chunk);
    const int nl = ib1;                       // lists reachable: j < ib1
    for (int j = threadIdx.x; j < nl; j += kThreads) hist[j] = 0;
    __syncthreads();
    const int tl0 = ib0 * B, tl1 = min(L, ib1 * B);
    const int nent = (tl1 - tl0) * K;
    const int32_t* src = idx + ((size_t)(t0 + tl0) * H + h) * K;
    const Div div(K, B);
    if ((K & 3) == 0) {
        // k a multiple of 4: four slots of one row per 16-byte load (a
        // row's K words start 16-byte aligned), kBatch / 4 loads in flight
        constexpr int QB = kBatch / 4;
        const int nq4 = nent >> 2;
        for (int q0 = threadIdx.x; q0 < nq4; q0 += kThreads * QB) {
            int4 jv[QB];
#pragma unroll
            for (int u = 0; u < QB; ++u) {
                const int e = 4 * (q0 + u * kThreads);
                const int r = div.row(e), slot = e - r * K;
                jv[u] = e < nent ? *(const int4*)(src + (size_t)r * H * K + slot) : make_int4(-1, -1, -1, -1);
            }
#pragma unroll
            for (int u = 0; u < QB; ++u) {
                const int e = 4 * (q0 + u * kThreads);
                const int i = div.block(tl0 + div.row(e));
                if (jv[u].x >= 0 && jv[u].x < i) atomicAdd(&hist[jv[u].x], 1);
                if (jv[u].y >= 0 && jv[u].y < i) atomicAdd(&hist[jv[u].y], 1);
                if (jv[u].z >= 0 && jv[u].z < i) atomicAdd(&hist[jv[u].z], 1);
                if (jv[u].w >= 0 && jv[u].w < i) atomicAdd(&hist[jv[u].w], 1);
            }
        }
    } else
    // kBatch loads in flight per thread before their LDS updates
    for (int e0 = threadIdx.x; e0 < nent; e0 += kThreads * kBatch) {
        int jv[kBatch];
#pragma unroll
        for (int u = 0; u < kBatch; ++u) {
            const int e = e0 + u * kThreads;
            const int r = div.row(e), slot = e - r * K;
            jv[u] = e < nent ? src[(size_t)r * H * K + slot] : -1;
        }
#pragma unroll
        for (int u = 0; u < kBatch; ++u) {
            const int e = e0 + u * kThreads;
            const int i = div.block(tl0 + div.row(e));
            if (jv[u] >= 0 && jv[u] < i) atomicAdd(&hist[jv[u]], 1);
        }
    }
    __syncthreads();
    int32_t* dst = cm_base(st, cmat, s, h) + (int64_t)cl * n;
    for (int j = threadIdx.x; j < nl; j += kThreads) dst[j] = hist[j];
}

__global__ __launch_bounds__(kScanThreads) void inv_scan_kernel(SegTable st, int32_t* __restrict__ cmat,
                                                               Item* __restrict__ items,
                                                               int2* __restrict__ lst)
{
    extern __shared__ int32_t lds[];
    const int s = blockIdx.x, h = blockIdx.y;
    const int n = seq_nblk(st, s), nch = seq_nchunk(st, s);
    int32_t* tot = lds;               // [n] list totals -> entry offsets
    int32_t* ioff = lds + n;          // [n] item offsets
    __shared__ int32_t part_e[kScanThreads], part_i[kScanThreads];
    int32_t* cm = cm_base(st, cmat, s, h);
    const int64_t ib = st.ibase[s] + (int64_t)h * seq_item_cap(st, s);
    const int64_t cap = seq_item_cap(st, s);

    // list totals (chunk c reaches list j iff j < (c+1)*chunk)
    for (int j = threadIdx.x; j < n; j += kScanThreads) {
        int t = 0;
        for (int c = j / st.chunk; c < nch; ++c) t += cm[(int64_t)c * n + j];
        tot[j] = t;
    }
    __syncthreads();
    // block scan over contiguous ranges
    const int per = (n + kScanThreads - 1) / kScanThreads;
    const int j0 = threadIdx.x * per, j1 = min(n, j0 + per);
    int se = 0, si = 0;
    const int IR = st.item_rows;
    for (int j = j0; j < j1; ++j) { se += tot[j]; si += (tot[j] + IR - 1) / IR; }
    part_e[threadIdx.x] = se;
    part_i[threadIdx.x] = si;
    __syncthreads();
    for (int off = 1; off < kScanThreads; off <<= 1) {
        int ve = threadIdx.x >= off ? part_e[threadIdx.x - off] : 0;
        int vi = threadIdx.x >= off ? part_i[threadIdx.x - off] : 0;
        __syncthreads();
        part_e[threadIdx.x] += ve;
        part_i[threadIdx.x] += vi;
        __syncthreads();
    }
    int be = part_e[threadIdx.x] - se, bi = part_i[threadIdx.x] - si;   // exclusive
    const int n_items = part_i[kScanThreads - 1];
    for (int j = j0; j < j1; ++j) {
        const int t = tot[j];
        tot[j] = be;
        ioff[j] = bi;
        be += t;
        bi += (t + IR - 1) / IR;
        // keep the list total in the scan result: ioff/tot of j+1 give it
    }
    __syncthreads();
    // per-chunk positions (in place) and items, coalesced over j
    const int g0 = st.boff[s];
    for (int j = threadIdx.x; j < n; j += kScanThreads) {
        const int beg = tot[j];
        int run = beg;
        for (int c = j / st.chunk; c < nch; ++c) {
            const int v = cm[(int64_t)c * n + j];
            cm[(int64_t)c * n + j] = run;
            run += v;
        }
        const int total = run - beg;
        lst[(int64_t)h * st.total_blocks + g0 + j] = make_int2(beg, total);
        const int nit = (total + IR - 1) / IR;
        for (int r = 0; r < nit; ++r) {
            Item it;
            it.begin = beg + r * IR;
            it.count = min(IR, total - r * IR);
            it.g = g0 + j;
            it.h = h;
            items[ib + ioff[j] + r] = it;
        }
    }
    // unused capacity: empty items
    for (int64_t r = n_items + threadIdx.x; r < cap; r += kScanThreads) {
        Item it;
        it.begin = 0; it.count = 0; it.g = 0; it.h = h;
        items[ib + r] = it;
    }
}

// DET = false: LDS cursors shared by the 4 waves (entries of one list land
// in an order that depends on wave timing; the forward does not depend on
// it).  DET = true: each wave owns a contiguous quarter of the chunk's
// tokens and its own cursors, based at the chunk position plus the counts of
// the earlier waves (a counting pass first), so every entry's position
// depends only on the idx contents -- the backward sums its list-ordered
// rows into dK / dV, which are then bitwise repeatable.
template <bool DET>
__global__ __launch_bounds__(kThreads) void inv_scatter_kernel(SegTable st, const int32_t* __restrict__ idx,
                                                              const int32_t* __restrict__ cmat,
                                                              uint32_t* __restrict__ entries,
                                                              int32_t* __restrict__ rev)
{
    extern __shared__ int32_t cur[];
    const int c = blockIdx.x, h = blockIdx.y;
    const int s = seq_of_chunk(st, c);
    const int cl = c - st.cbase[s];
    const int n = seq_nblk(st, s), L = seq_len(st, s), t0 = st.cu[s];
    const int B = st.B, K = st.K, H = st.H;
    const int ib0 = cl * st.chunk, ib1 = min(n, ib0 + st.chunk);
    const int32_t* pos = cm_base(st, const_cast<int32_t*>(cmat), s, h) + (int64_t)cl * n;
    uint32_t* ent = entries + st.ebase[s] + (int64_t)h * L * K;
    const int tl0 = ib0 * B, tl1 = min(L, ib1 * B);
    const int nent = (tl1 - tl0) * K;
    const int32_t* src = idx + ((size_t)(t0 + tl0) * H + h) * K;
    // reverse map is head-major, [H][tokens][K]: this chunk's records are
    // one contiguous run, written in order
    int32_t* rv = rev + ((size_t)h * st.cu[st.nseq] + t0 + tl0) * K;
    const Div div(K, B);
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    // DET: wave w takes entries [e_lo, e_hi) (whole tokens), lanes stride 64
    const int ntok = tl1 - tl0, tpw = (ntok + 3) / 4;
    const int e_lo = DET ? min(ntok, wave * tpw) * K : 0;
    const int e_hi = DET ? min(ntok, (wave + 1) * tpw) * K : nent;
    const int first = DET ? e_lo + lane : threadIdx.x;
    constexpr int STEP = DET ? 64 : kThreads;
    int32_t* wc = DET ? cur + wave * ib1 : cur;        // this wave's cursors
    if constexpr (DET) {
        for (int j = threadIdx.x; j < 4 * ib1; j += kThreads) cur[j] = 0;
        __syncthreads();
        for (int e0 = first; e0 < e_hi; e0 += STEP * kBatch) {
            int jv[kBatch];
#pragma unroll
            for (int u = 0; u < kBatch; ++u) {
                const int e = e0 + u * STEP;
                const int r = div.row(e), slot = e - r * K;
                jv[u] = e < e_hi ? src[(size_t)r * H * K + slot] : -1;
            }
#pragma unroll
            for (int u = 0; u < kBatch; ++u) {
                const int e = e0 + u * STEP;
                const int i = div.block(tl0 + div.row(e));
                if (e < e_hi && jv[u] >= 0 && jv[u] < i) atomicAdd(&wc[jv[u]], 1);
            }
        }
        __syncthreads();
        // cursors: chunk position + counts of the earlier waves
        for (int j = threadIdx.x; j < ib1; j += kThreads) {
            int run = pos[j];
#pragma unroll
            for (int w = 0; w < 4; ++w) {
                const int t = cur[w * ib1 + j];
                cur[w * ib1 + j] = run;
                run += t;
            }
        }
    } else {
        for (int j = threadIdx.x; j < ib1; j += kThreads) cur[j] = pos[j];
    }
    __syncthreads();
    if (!DET && (K & 3) == 0) {
        // k a multiple of 4: four slots of one row per 16-byte load and per
        // 16-byte reverse-map store
        constexpr int QB = kBatch / 4;
        const int nq4 = e_hi >> 2;
        for (int q0 = threadIdx.x; q0 < nq4; q0 += kThreads * QB) {
            int4 jv[QB];
#pragma unroll
            for (int u = 0; u < QB; ++u) {
                const int e = 4 * (q0 + u * kThreads);
                const int r = div.row(e), slot = e - r * K;
                jv[u] = e < e_hi ? *(const int4*)(src + (size_t)r * H * K + slot) : make_int4(-1, -1, -1, -1);
            }
            int4 pv[QB];
#pragma unroll
            for (int u = 0; u < QB; ++u) {
                const int e = 4 * (q0 + u * kThreads);
                const int i = div.block(tl0 + div.row(e));
                pv[u].x = (jv[u].x >= 0 && jv[u].x < i) ? atomicAdd(&wc[jv[u].x], 1) : -1;
                pv[u].y = (jv[u].y >= 0 && jv[u].y < i) ? atomicAdd(&wc[jv[u].y], 1) : -1;
                pv[u].z = (jv[u].z >= 0 && jv[u].z < i) ? atomicAdd(&wc[jv[u].z], 1) : -1;
                pv[u].w = (jv[u].w >= 0 && jv[u].w < i) ? atomicAdd(&wc[jv[u].w], 1) : -1;
            }
#pragma unroll
            for (int u = 0; u < QB; ++u) {
                const int e = 4 * (q0 + u * kThreads);
                if (e >= e_hi) continue;
                const int r = div.row(e), slot = e - r * K;
                const uint32_t tok = (uint32_t)(t0 + tl0 + r) << 5;
                // (debug builds: positions inside the (sequence, head) region)
                if (pv[u].x >= 0 && MOBA_INBOUNDS(pv[u].x < L * K, kDbgScatter)) ent[pv[u].x] = tok | (uint32_t)slot;
                if (pv[u].y >= 0 && MOBA_INBOUNDS(pv[u].y < L * K, kDbgScatter)) ent[pv[u].y] = tok | (uint32_t)(slot + 1);
                if (pv[u].z >= 0 && MOBA_INBOUNDS(pv[u].z < L * K, kDbgScatter)) ent[pv[u].z] = tok | (uint32_t)(slot + 2);
                if (pv[u].w >= 0 && MOBA_INBOUNDS(pv[u].w < L * K, kDbgScatter)) ent[pv[u].w] = tok | (uint32_t)(slot + 3);
                *(int4*)(rv + e) = pv[u];
            }
        }
        return;
    }
    for (int e0 = first; e0 < e_hi; e0 += STEP * kBatch) {
        int jv[kBatch];
#pragma unroll
        for (int u = 0; u < kBatch; ++u) {
            const int e = e0 + u * STEP;
            const int r = div.row(e), slot = e - r * K;
            jv[u] = e < e_hi ? src[(size_t)r * H * K + slot] : -1;
        }
        // all LDS cursor bumps of the batch first, then the stores
        int pv[kBatch];
#pragma unroll
        for (int u = 0; u < kBatch; ++u) {
            const int e = e0 + u * STEP;
            const int i = div.block(tl0 + div.row(e));
            pv[u] = (e < e_hi && jv[u] >= 0 && jv[u] < i) ? atomicAdd(&wc[jv[u]], 1) : -1;
        }
#pragma unroll
        for (int u = 0; u < kBatch; ++u) {
            const int e = e0 + u * STEP;
            const int r = div.row(e), slot = e - r * K;
            if (pv[u] >= 0 && MOBA_INBOUNDS(pv[u] < L * K, kDbgScatter))
                ent[pv[u]] = ((uint32_t)(t0 + tl0 + r) << 5) | (uint32_t)slot;
            // every slot is written, so each query's K positions form one
            // contiguous, fully written record
            if (e < e_hi) rv[e] = pv[u];
        }
    }
}

// Blocks larger than the attention kernels' (128 keys; 64 for fp32 at
// d = 128): a selected block of B = r * ab keys is the union of its r
// sub-blocks of ab keys, and the query's own block splits into the
// sub-blocks before its own sub-block (every key of which precedes the
// query) and its own sub-block (token-causal).  Attention over the selection
// is therefore attention over ab-key blocks with this expanded list, which
// the ab-key kernels run unchanged.  One thread per (token, head) row.
__global__ __launch_bounds__(kThreads) void expand_idx_kernel(SegTable stl, int r, int lab, int Kp,
                                                             const int32_t* __restrict__ idx,
                                                             int32_t* __restrict__ pidx, int64_t rows)
{
    const int64_t row = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    if (row >= rows) return;
    const int H = stl.H, K = stl.K;
    const int t = (int)(row / H);
    int s = 0;
    {
        int lo = 0, hi = stl.nseq - 1;          // last s with cu[s] <= t
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (stl.cu[mid] <= t) lo = mid; else hi = mid - 1;
        }
        s = lo;
    }
    const int tl = t - stl.cu[s];
    const int il = tl / stl.B;                   // logical own block
    const int pt = tl >> lab;                    // physical own block
    const int32_t* in = idx + row * K;
    int32_t* out = pidx + row * Kp;
    int n = 0;
    for (int p = 0; p < K; ++p) {
        const int j = in[p];
        if (j < 0 || j >= il) continue;
        for (int c = 0; c < r && n < Kp; ++c) out[n++] = j * r + c;
    }
    for (int pb = il * r; pb < pt && n < Kp; ++pb) out[n++] = pb;
    for (; n < Kp; ++n) out[n] = -1;
}

}  // namespace

uint32_t dbg_take_invert()
{
#ifdef MOBA_DEBUG_BOUNDS
    return dbg_take_local();
#else
    return 0u;
#endif
}

hipError_t launch_expand_idx(const Launch& Ll, int ab, int Kp, const int32_t* idx, int32_t* pidx)
{
    const int64_t rows = (int64_t)Ll.tokens * Ll.st.H;
    if (rows == 0) return hipSuccess;
    const int r = Ll.st.B / ab;
    const int lab = 31 - __builtin_clz((unsigned)ab);
    hipLaunchKernelGGL(expand_idx_kernel, dim3((unsigned)((rows + kThreads - 1) / kThreads)), dim3(kThreads), 0,
                       Ll.stream, Ll.st, r, lab, Kp, idx, pidx, rows);
    return hipGetLastError();
}

hipError_t launch_inv(const Launch& L, const WsLayout& ws, char* wsp, const int32_t* idx, bool det)
{
    const SegTable& st = L.st;
    if (st.K <= 1 || st.total_chunks == 0) return hipSuccess;
    int32_t* cmat = (int32_t*)(wsp + ws.cmat_off);
    Item* items = (Item*)(wsp + ws.items_off);
    uint32_t* ent = (uint32_t*)(wsp + ws.ent_off);
    int32_t* rev = (int32_t*)(wsp + ws.rev_off);
    int2* lst = (int2*)(wsp + ws.lst_off);
    int maxn = 0;
    for (int s = 0; s < st.nseq; ++s) maxn = maxn > seq_nblk(st, s) ? maxn : seq_nblk(st, s);
    dim3 gc(st.total_chunks, st.H);
    hipLaunchKernelGGL(inv_count_kernel, gc, dim3(kThreads), (size_t)maxn * 4, L.stream, st, idx, cmat);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(inv_scan_kernel, dim3(st.nseq, st.H), dim3(kScanThreads), (size_t)maxn * 8,
                       L.stream, st, cmat, items, lst);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    // the repeatable placement keeps 4 cursor sets in LDS
    if (det && maxn <= kDetMaxBlocks)
        hipLaunchKernelGGL(inv_scatter_kernel<true>, gc, dim3(kThreads), (size_t)maxn * 16, L.stream, st, idx,
                           cmat, ent, rev);
    else
        hipLaunchKernelGGL(inv_scatter_kernel<false>, gc, dim3(kThreads), (size_t)maxn * 4, L.stream, st, idx,
                           cmat, ent, rev);
    return hipGetLastError();
}

}  // namespace moba
