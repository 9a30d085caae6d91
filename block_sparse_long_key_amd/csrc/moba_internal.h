// moba_internal.h -- shared definitions of the gfx950 MoBA forward kernels.
//
// Sequences, blocks and heads are addressed through a SegTable that the host
// fills from the shape and passes to every kernel by value (no device
// allocation, no host<->device copy).  Token rows are [tokens][heads][d].
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/moba.h"

namespace moba {

constexpr int kMaxSeqs = MOBA_MAX_SEQS;
// most queries per routed-attention work item (looped in tiles of 128);
// SegTable::item_rows holds the launch's value: this one, or twice it for
// bf16 at d = 128 (routed attention at 64K x 16 heads: d = 128 items of
// 4096 rows 1.823 -> 1.767 ms, against d = 64 items of 2048 rows 0.839 vs
// 0.851 ms with 4096 and 0.865 with 1024).  Kernels that copy an item's
// entries to LDS (fp32, and d = 64 with 64-key blocks) size the copy by
// this constant and always get it.
constexpr int kItemRows = 2048;
inline int item_rows_for(int dtype, int head_dim)
{
    return (dtype == MOBA_BF16 && head_dim == 128) ? 2 * kItemRows : kItemRows;
}
// query blocks per inversion chunk (one workgroup of the count/scatter
// passes): this many, or for sequences of more than 1024 blocks the power of
// two reaching 1/16 of the longest one's blocks, so a chunk's entries still
// land in runs of several entries per list when there are thousands of lists
constexpr int kInvChunkBlocks = 32;
// largest number of blocks of one sequence (LDS histogram of the inversion)
constexpr int kMaxBlocksPerSeq = 16384;

// Keys per block of the attention kernels: the shape's block size up to
// 128; fp32 at d = 128 attends 64-key blocks (a block of K and V^T in fp32
// must fit LDS: B * d <= 8192).  Larger blocks are attended as the union of
// their sub-blocks of this size.
inline int att_block(int dtype, int head_dim, int block_size)
{
    const int cap = (dtype == MOBA_F32 && head_dim == 128) ? 64 : 128;
    return block_size < cap ? block_size : cap;
}

struct SegTable {
    int32_t nseq;       // number of independent sequences
    int32_t H;          // heads
    int32_t B;          // block size
    int32_t K;          // top_k (own block included)
    int32_t total_blocks;
    int32_t total_chunks;   // inversion chunks over all sequences (per head)
    int32_t chunk;          // query blocks per inversion chunk
    int64_t total_items;    // routed-attention item capacity over all (seq, head)
    int32_t item_rows;      // most entries per item
    int32_t cu[kMaxSeqs + 1];     // token start of sequence s
    int32_t boff[kMaxSeqs + 1];   // first global block of sequence s
    int32_t cbase[kMaxSeqs + 1];  // first inversion chunk of sequence s
    int64_t cmbase[kMaxSeqs + 1]; // count-matrix base of (s, h=0); + h * nch * nblk
    int64_t ebase[kMaxSeqs + 1];  // entries base of (s, h=0); + h * L * K
    int64_t ibase[kMaxSeqs + 1];  // item base of (s, h=0); + h * cap(s)
};

__host__ __device__ inline int seq_len(const SegTable& st, int s) { return st.cu[s + 1] - st.cu[s]; }
__host__ __device__ inline int seq_nblk(const SegTable& st, int s) { return st.boff[s + 1] - st.boff[s]; }
__host__ __device__ inline int seq_nchunk(const SegTable& st, int s) { return st.cbase[s + 1] - st.cbase[s]; }
__host__ __device__ inline int64_t seq_item_cap(const SegTable& st, int s) {
    // a row lists at most K blocks (K-1 when it holds its own block, as it should)
    return (int64_t)seq_len(st, s) * st.K / st.item_rows + seq_nblk(st, s);
}

// sequence holding global block g (boff is non-decreasing; empty sequences
// have boff[s] == boff[s+1] and are skipped)
__device__ inline int seq_of_block(const SegTable& st, int g) {
    int lo = 0, hi = st.nseq - 1;
    while (lo < hi) {               // last s with boff[s] <= g and nonempty
        int mid = (lo + hi + 1) >> 1;
        if (st.boff[mid] <= g) lo = mid; else hi = mid - 1;
    }
    while (lo > 0 && st.boff[lo] > g) --lo;
    return lo;
}
// sequence holding token t (the last s with cu[s] <= t: with empty
// sequences sharing a start, the nonempty one that follows them)
__device__ inline int seq_of_token(const SegTable& st, int t) {
    int lo = 0, hi = st.nseq - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (st.cu[mid] <= t) lo = mid; else hi = mid - 1;
    }
    return lo;
}
__device__ inline int seq_of_chunk(const SegTable& st, int c) {
    int lo = 0, hi = st.nseq - 1;
    while (lo < hi) {
        int mid = (lo + hi + 1) >> 1;
        if (st.cbase[mid] <= c) lo = mid; else hi = mid - 1;
    }
    return lo;
}

// ------------------------------------------------------ bounds checks --
// Debug builds (-DMOBA_DEBUG_BOUNDS, libmoba_amd_debug.so) check every
// index that kernels take from data -- list entries, list positions, work
// items -- against the region it addresses before the access; a failed
// check sets a bit in this source file's violation word and the kernel
// skips or clamps the access instead of leaving its buffers.  Release
// builds compile MOBA_INBOUNDS to true (the condition is not evaluated), so
// their code is unchanged.  Bits:
enum : unsigned {
    kDbgItem = 1u,         // routed item outside its (sequence, head) list region
    kDbgEntry = 2u,        // routed list entry: token outside the list's sequence, or slot >= K
    kDbgMergePos = 4u,     // merge: list position outside the region
    kDbgBwdList = 8u,      // backward: a list's (first, count) outside the region
    kDbgBwdEntry = 16u,    // backward: list entry token outside the sequence, or slot >= K
    kDbgDqPos = 32u,       // dq merge: list position outside the region
    kDbgScatter = 64u,     // index pass: list position outside the region
    kDbgKvEntry = 128u,    // fp32 backward (dk, dv): list entry outside the sequence
};
#ifdef MOBA_DEBUG_BOUNDS
namespace {
__device__ unsigned int g_dbg_violations = 0u;   // one per source file
// this source file's violation word on the current device, then cleared
// (a synchronous copy on the null stream)
inline uint32_t dbg_take_local()
{
    uint32_t v = 0u;
    const uint32_t z = 0u;
    if (hipMemcpyFromSymbol(&v, HIP_SYMBOL(g_dbg_violations), sizeof(v), 0, hipMemcpyDeviceToHost) != hipSuccess)
        return 0x80000000u;
    if (hipMemcpyToSymbol(HIP_SYMBOL(g_dbg_violations), &z, sizeof(z), 0, hipMemcpyHostToDevice) != hipSuccess)
        return 0x80000000u;
    return v;
}
}  // namespace
#define MOBA_INBOUNDS(cond, bit) ((cond) || (atomicOr(&g_dbg_violations, (unsigned)(bit)), false))
#else
#define MOBA_INBOUNDS(cond, bit) true
#endif
// each source file's violation word (0 in release builds)
uint32_t dbg_take_attn();
uint32_t dbg_take_attn_bwd();
uint32_t dbg_take_attn_bwd_f32();
uint32_t dbg_take_invert();

// ------------------------------------------------------------ bf16 ------
// bf16 is carried as its 16-bit pattern.  Rounding is IEEE round to nearest,
// ties to even, done by the hardware conversion (v_cvt_pk_bf16_f32).
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
    return __uint_as_float(((uint32_t)b) << 16);
}
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
    return __builtin_bit_cast(uint16_t, (__bf16)f);
}
// two floats -> packed bf16 pair (a in the low half)
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
    const f32x2_t x = {a, b};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(x, bf16x2_t));
}
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

template <typename T> struct IO;
template <> struct IO<float> {
    static __device__ __forceinline__ float load(const float* p) { return *p; }
    static __device__ __forceinline__ float round(float x) { return x; }
    static __device__ __forceinline__ void store(float* p, float x) { *p = x; }
};
template <> struct IO<uint16_t> {
    static __device__ __forceinline__ float load(const uint16_t* p) { return bf16_to_f32(*p); }
    static __device__ __forceinline__ float round(float x) { return bf16_to_f32(f32_to_bf16(x)); }
    static __device__ __forceinline__ void store(uint16_t* p, float x) { *p = f32_to_bf16(x); }
};

// ------------------------------------------------------------ MFMA ------
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint16_t u16x8_t __attribute__((ext_vector_type(8)));
typedef uint16_t u16x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

// routed-attention work item: a run of <= item_rows entries of one list
struct Item {
    int32_t begin;   // first entry, relative to the (seq, head) entries base
    int32_t count;   // 0 = empty slot
    int32_t g;       // global key block
    int32_t h;       // head
};

// ----------------------------------------------------- workspace layout --
struct WsLayout {
    size_t cmat_off, cmat_bytes;     // int32 count / position matrix
    size_t items_off, items_bytes;   // Item[total_items]
    size_t ent_off, ent_bytes;       // uint32 entries (t << 5 | slot), list order
    size_t rev_off, rev_bytes;       // int32 [H][tokens][K]: list position of (t, slot), -1 if none
    size_t po_off, po_bytes;         // partial o rows, list order (I/O dtype, D per row)
    size_t pl_off, pl_bytes;         // partial lse, list order, fp32 (log2 units)
    size_t pm_off, pm_bytes;         // BLASST: (partial lse, block maximum) fp32 pairs, list order (log2 units)
    size_t lst_off, lst_bytes;       // int2 [H][total blocks]: (first entry, count) of each list
    size_t rs_off, rs_bytes;         // backward: float2 [tokens][H] (lse in log2 units, dO . O)
    size_t pq_off, pq_bytes;         // backward: fp32 dq pieces, list order, then own-block rows
    size_t px_off, px_bytes;         // block sizes > 128: int32 [tokens][H][K'] selection in 128-key blocks
    size_t own_off, own_bytes;       // backward: uint8 [tokens][H], 1 where the row attends its own block
    size_t total;
};

// ----------------------------------------------------------- launchers --
struct Launch {
    SegTable st;
    int D;
    int dtype;          // moba_dtype
    int tokens;         // total tokens over all sequences
    hipStream_t stream;
};

hipError_t launch_conv_pool(const Launch& L, const void* k, const float* w, int W,
                            int mode, void* k_out, float* cent);
hipError_t launch_conv_bwd(const Launch& L, const void* k, const float* w, int W, int mode,
                           const void* gk, void* dk, float* dwp);
hipError_t launch_conv_dw_reduce(hipStream_t stream, int nblk, int n, const float* dwp, float* dw);
// The router's workspace: the centroids split for the MFMA scores (bf16 high
// and low parts, [block][head][d] like the centroids) and their squared
// norms ([block][head]).
struct RouteWs {
    uint16_t* hi;
    uint16_t* lo;
    float* n2;
};
inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }
size_t route_ws_bytes(const Launch& L);
// address of this device's fixed routing scratch (MOBA_ROUTE_SCRATCH_BYTES)
hipError_t route_scratch(void** out);
RouteWs route_ws(const Launch& L, void* workspace);
// bf16 queries use the workspace; fp32 queries do not read it
hipError_t launch_route(const Launch& L, const void* q, const float* cent, void* workspace,
                        int32_t* idx);
// det: place each list's entries in an order that depends only on idx
hipError_t launch_inv(const Launch& L, const WsLayout& ws, char* wsp, const int32_t* idx,
                      bool det = false);
// ab: the attention launch's block size (a divisor of Ll's)
hipError_t launch_expand_idx(const Launch& Ll, int ab, int Kp, const int32_t* idx, int32_t* pidx);
hipError_t launch_routed_attn(const Launch& L, const WsLayout& ws, char* wsp,
                              const void* q, const void* k, const void* v, float scale,
                              bool block_max = false);
// own (nullable, uint8 per (token, head)): rows with own[row] == 0 leave
// their own block out of the key set (a BLASST selection); null: every row
// attends its own block
hipError_t launch_attn_bwd(const Launch& L, const WsLayout& ws, char* wsp, const void* q,
                           const void* k, const void* v, const void* o, const float* lse,
                           const void* dout, float scale, void* dq, void* dk, void* dv,
                           const uint8_t* own = nullptr);
// fp32 inputs; idx: the selection in the launch's blocks (expanded for B > 128)
hipError_t launch_attn_bwd_f32(const Launch& L, const WsLayout& ws, char* wsp, const int32_t* idx,
                               const void* q, const void* k, const void* v, const void* o,
                               const float* lse, const void* dout, float scale, void* dq, void* dk,
                               void* dv, const uint8_t* own = nullptr);
// own[row] = 1 where idx's row lists the row's own block, else 0
hipError_t launch_own_flags(const Launch& L, const int32_t* idx, uint8_t* own);
// blasst_lambda > 0: the BLASST skip over the partials' block maxima
// (which the routed pass must have stored, block_max = true)
hipError_t launch_diag_combine(const Launch& L, const WsLayout& ws, char* wsp,
                               const void* q, const void* k, const void* v,
                               const int32_t* idx, float scale, void* o, float* lse,
                               float blasst_lambda = 0.f, int32_t* kept = nullptr);

}  // namespace moba
