// router.hip -- router scores and causal top-k block selection (gfx950).
//
// "Optimizing Mixture of Block Attention", summary page: section
// "Architettura del Modello Statistico" (router-score equation
// s_j = q . kbar_j) and section "Definizione del Compito" (each query keeps
// its top-k blocks).  The causal rules -- own block always kept and not
// competing, future blocks masked, equal scores to the lower block id -- are
// the plainest decoder reading.
//
// Exactness.  The selection must equal the one made on fp64 scores.  Scores
// are computed here in fp32 (fmaf, sequential over channels) whose error is
// at most E = gamma_d * |q| * max_j |kbar_j| (gamma_d = d u / (1 - d u),
// u = 2^-24, Cauchy-Schwarz on sum |q_c kbar_c|).  If the (k-1)-th and k-th
// best fp32 scores are more than 2E apart, the fp32 top-(k-1) set is the
// exact one (any swap would need two scores to move by more than E each).
// Otherwise the query is re-scored in fp64, sequentially over channels --
// products of bf16/fp32 values are exact in fp64, so the fp64 scores are the
// correctly-ordered sums -- and selected again.  That happens for a small
// fraction of queries (near-ties).
//
// fp32 queries (VALU kernel): one workgroup = one query block (B threads,
// one query each) of one head; the centroids of the past blocks stream
// through LDS in tiles of 32 and are read by all threads as broadcasts.
// bf16 queries use the MFMA kernel below.
#include <mutex>
#include <type_traits>

#include "moba_internal.h"

namespace moba {
namespace {

constexpr int kTile = 32;
// idx slot-0 markers between the two router kernels: row awaiting the full
// fp64 re-selection; row carrying a hint (finalists and a bound)
constexpr int32_t kPending = (int32_t)0x80000000;
constexpr int32_t kHint = (int32_t)0x80000001;
constexpr int kHintMinK = 6;           // F = 2K-4 finalists: at least K+2
constexpr int kHintNone = 0xffff;      // empty finalist slot; block ids stay below

template <int KMAX>
__device__ __forceinline__ void insert_desc(float (&sc)[KMAX], int (&ix)[KMAX], int K,
                                            float sv, int j)
{
    // list sorted by (score desc, index asc); new j is larger than every
    // listed index, so it goes after equal scores
#pragma unroll
    for (int p = KMAX - 1; p >= 1; --p) {
        if (p < K) {
            if (sc[p - 1] < sv) { sc[p] = sc[p - 1]; ix[p] = ix[p - 1]; }
            else if (sc[p] < sv) { sc[p] = sv; ix[p] = j; }
        }
    }
    if (sc[0] < sv) { sc[0] = sv; ix[0] = j; }
}

template <int KMAX>
__device__ __forceinline__ void insert_desc64(double (&sc)[KMAX], int (&ix)[KMAX], int K,
                                              double sv, int j)
{
#pragma unroll
    for (int p = KMAX - 1; p >= 1; --p) {
        if (p < K) {
            if (sc[p - 1] < sv) { sc[p] = sc[p - 1]; ix[p] = ix[p - 1]; }
            else if (sc[p] < sv) { sc[p] = sv; ix[p] = j; }
        }
    }
    if (sc[0] < sv) { sc[0] = sv; ix[0] = j; }
}

template <int KMAX>
__device__ __forceinline__ float pick(const float (&a)[KMAX], int p)
{
    float r = a[0];
#pragma unroll
    for (int e = 1; e < KMAX; ++e) if (e == p) r = a[e];
    return r;
}

// ascending sort of the first n entries (others must be INT_MAX): a bitonic
// sorting network over KMAX (a power of two) entries, every index fixed at
// compile time (KMAX/2 * log2(KMAX) * (log2(KMAX) + 1) / 2 compare-exchanges)
template <int KMAX>
__device__ __forceinline__ void sort_asc(int (&x)[KMAX])
{
    static_assert((KMAX & (KMAX - 1)) == 0, "KMAX must be a power of two");
#pragma unroll
    for (int k = 2; k <= KMAX; k <<= 1)
#pragma unroll
        for (int j = k >> 1; j > 0; j >>= 1)
#pragma unroll
            for (int p = 0; p < KMAX; ++p) {
                const int l = p ^ j;
                if (l > p) {
                    const int lo = min(x[p], x[l]);
                    const int hi = max(x[p], x[l]);
                    const bool up = (p & k) == 0;
                    x[p] = up ? lo : hi;
                    x[l] = up ? hi : lo;
                }
            }
}

template <typename T, int D, int KMAX>
__global__ __launch_bounds__(256) void route_kernel(SegTable st, const T* __restrict__ q,
                                                   const float* __restrict__ cent,
                                                   int32_t* __restrict__ idx)
{
    __shared__ float cs[kTile][D];
    __shared__ float cn[kTile];

    const int g = blockIdx.x;
    const int h = blockIdx.y;
    const int H = st.H;
    const int K = st.K;
    const int s = seq_of_block(st, g);
    const int i = g - st.boff[s];
    const int L = seq_len(st, s);
    const int tl = i * st.B + threadIdx.x;
    const bool valid = threadIdx.x < st.B && tl < L;
    const size_t row = (size_t)(st.cu[s] + tl) * H + h;
    int32_t* out = idx + row * K;
    const float* cbase = cent + (size_t)st.boff[s] * H * D + (size_t)h * D;

    if (K == 1) {
        // only the own block
        if (valid) out[0] = i;
        return;
    }
    if (i <= K - 1) {
        // every past block is kept: 0..i, then padding
        if (valid)
            for (int p = 0; p < K; ++p) out[p] = p <= i ? p : -1;
        return;
    }

    float qv[D];
    float qn2 = 0.f;
    if (valid) {
        const T* qp = q + row * D;
#pragma unroll
        for (int c = 0; c < D; ++c) {
            qv[c] = IO<T>::load(qp + c);
            qn2 = __builtin_fmaf(qv[c], qv[c], qn2);
        }
    } else {
#pragma unroll
        for (int c = 0; c < D; ++c) qv[c] = 0.f;
    }

    float sc[KMAX];
    int ix[KMAX];
#pragma unroll
    for (int p = 0; p < KMAX; ++p) { sc[p] = -INFINITY; ix[p] = -1; }
    float thr = -INFINITY;       // = sc[K-1]
    float cmax = 0.f;            // max centroid norm seen

    for (int j0 = 0; j0 < i; j0 += kTile) {
        const int nt = min(kTile, i - j0);
        __syncthreads();
        for (int e = threadIdx.x; e < nt * D; e += blockDim.x) {
            int jj = e / D, c = e % D;
            cs[jj][c] = cbase[(size_t)(j0 + jj) * H * D + c];
        }
        __syncthreads();
        if (threadIdx.x < nt) {
            float n2 = 0.f;
            for (int c = 0; c < D; ++c) n2 = __builtin_fmaf(cs[threadIdx.x][c], cs[threadIdx.x][c], n2);
            cn[threadIdx.x] = sqrtf(n2);
        }
        __syncthreads();
        for (int jj = 0; jj < nt; ++jj) {
            float sv = 0.f;
#pragma unroll
            for (int c = 0; c < D; ++c) sv = __builtin_fmaf(qv[c], cs[jj][c], sv);
            cmax = fmaxf(cmax, cn[jj]);
            if (sv > thr) {
                insert_desc<KMAX>(sc, ix, K, sv, j0 + jj);
                thr = pick<KMAX>(sc, K - 1);
            }
        }
    }
    if (!valid) return;

    // separation test of the (k-1)-th and k-th best scores
    const float u = 5.9604645e-08f;                       // 2^-24
    const float gam = (float)D * u / (1.0f - (float)D * u);
    const float E = gam * sqrtf(qn2) * cmax * 1.01f + 1e-30f;
    const float a = pick<KMAX>(sc, K - 2);
    const float b = thr;
    int sel[KMAX];
    if (a - b > 2.0f * E) {
#pragma unroll
        for (int p = 0; p < KMAX; ++p) sel[p] = (p < K - 1) ? ix[p] : 0x7fffffff;
    } else {
        // exact re-scoring in fp64
        double s64[KMAX];
        int ix64[KMAX];
#pragma unroll
        for (int p = 0; p < KMAX; ++p) { s64[p] = -INFINITY; ix64[p] = -1; }
        const int K1 = K - 1;
        for (int j = 0; j < i; ++j) {
            const float* cp = cbase + (size_t)j * H * D;
            double acc = 0.0;
            for (int c = 0; c < D; ++c) acc = __builtin_fma((double)qv[c], (double)cp[c], acc);
            double last = s64[0];
#pragma unroll
            for (int e = 1; e < KMAX; ++e) if (e == K1 - 1) last = s64[e];
            if (acc > last) insert_desc64<KMAX>(s64, ix64, K1, acc, j);
        }
#pragma unroll
        for (int p = 0; p < KMAX; ++p) sel[p] = (p < K - 1) ? ix64[p] : 0x7fffffff;
    }
    sort_asc<KMAX>(sel);
#pragma unroll
    for (int p = 0; p < KMAX; ++p)
        if (p < K - 1) out[p] = sel[p];
    out[K - 1] = i;
}

// ------------------------------------------------------------------------
// bf16 queries: MFMA scoring.  Each centroid c (fp32) is split into two bf16
// terms, hi = rne(c), lo = rne(c - hi), so c = hi + lo + r with
// |r| <= 2^-16 |c|; q is exact in bf16, every product q*hi, q*lo is exact in
// fp32 and v_mfma_f32_16x16x32_bf16 accumulates in fp32.  Bounding each of
// the (2d + 16) accumulation steps by one fp32 ulp gives
//   |s_mfma - s| <= (2^-16 + (2d + 16) 2^-23) * sum_c |q_c c_c|
//                <= (2^-16 + (2d + 16) 2^-23) * |q| * max_j |c_j|  =: E,
// and the separation test / fp64 re-scoring work as in the VALU kernel.
//
// route_prep_kernel splits every centroid once (hi, lo, |c|^2).  Workgroup
// = one query block of one head, B/32 waves of 32 queries (two 16-query
// sub-tiles); the hi / lo rows are copied into LDS in tiles of 64 blocks.
// S^T = C Q^T puts 4 blocks x 1 query in each lane.
//
// Selection without branches: a score s of block j becomes a float key whose
// low LB mantissa bits hold j, |key - s| <= 2^(LB-23) |s|.  Keys are unique
// and decode back to their block; how they order equal scores does not
// matter, since two keys within 2E of each other at the selection boundary
// send the row to the exact fp64 path, and inside the selection order is
// irrelevant (the output is sorted by block).  A lane keeps its LL best keys
// in a descending list, and inserting a key x is one v_med3_f32 per slot,
// a[p] = med3(a[p-1], a[p], x).  The key error is added to E in the
// separation test.  The 4 lanes of a query merge their lists by shuffles.
//
// Near-ties (the separation test fails) are finished by route_fix_kernel,
// which runs right after: when the query's K best keys are provably the only
// blocks that can still be selected, the row carries them (K fp64
// re-scorings); otherwise, for k >= 6, it carries its best 2K-4 blocks and a
// bound on every other block (2K-4 fp64 re-scorings, enough unless one lane
// held nearly all of the top k); only the rest are re-scored in fp64
// against every past block.
__device__ __forceinline__ bool ranks_before64(double sa, int ja, double sb, int jb)
{
    return sa > sb || (sa == sb && ja < jb);
}

// insert (sv, j) into a descending list; j exceeds every listed index, so it
// goes after equal scores; the last slot falls off
template <int KMAX, typename F>
__device__ __forceinline__ void insert_tail(F (&sc)[KMAX], int (&ix)[KMAX], F sv, int j)
{
#pragma unroll
    for (int p = KMAX - 1; p >= 1; --p) {
        if (sc[p - 1] < sv) { sc[p] = sc[p - 1]; ix[p] = ix[p - 1]; }
        else if (sc[p] < sv) { sc[p] = sv; ix[p] = j; }
    }
    if (sc[0] < sv) { sc[0] = sv; ix[0] = j; }
}

// max / min of non-NaN floats as one v_med3_f32 each: med3(a, b, +inf) is
// max(a, b).  The infinity comes from a register the compiler cannot see
// through; with a literal it rewrites the med3 as fmaxf, which first
// canonicalises both operands (two more instructions).
__device__ __forceinline__ float opaque_inf()
{
    float r;
    asm volatile("v_mov_b32 %0, 0x7f800000" : "=v"(r));
    return r;
}
__device__ __forceinline__ float fmax2(float a, float b, float inf) { return __builtin_amdgcn_fmed3f(a, b, inf); }
__device__ __forceinline__ float fmin2(float a, float b, float inf) { return __builtin_amdgcn_fmed3f(a, b, -inf); }

// block id carried in the low bits of a selection key
__device__ __forceinline__ int key_block(float k, uint32_t lmask)
{
    return (int)(__float_as_uint(k) & lmask);
}

// Top N of two descending lists x and y, sorted, into x: c[p] = max(x[p],
// y[N-1-p]) is bitonic and holds the top N of both; a bitonic clean sorts it.
template <int N>
__device__ __forceinline__ void top_of_two(float (&x)[N], const float (&y)[N], float inf)
{
#pragma unroll
    for (int p = 0; p < N; ++p) x[p] = fmax2(x[p], y[N - 1 - p], inf);
#pragma unroll
    for (int st2 = N / 2; st2 >= 1; st2 >>= 1)
#pragma unroll
        for (int p = 0; p < N; ++p)
            if ((p & st2) == 0) {
                const float hi = fmax2(x[p], x[p + st2], inf);
                const float lo = fmin2(x[p], x[p + st2], inf);
                x[p] = hi;
                x[p + st2] = lo;
            }
}

// Sorted (descending) top-N merge of the lists of lanes l, l^16, l^32, l^48.
// The first NIN entries of x are the lane's own sorted list (the rest -INF).
template <int N, int NIN>
__device__ __forceinline__ void merge_lanes(float (&x)[N])
{
    const float inf = opaque_inf();
#pragma unroll
    for (int m = 16; m <= 32; m <<= 1) {
        float y[N];
#pragma unroll
        for (int p = 0; p < N; ++p) y[p] = (m == 16 && p >= NIN) ? -INFINITY : __shfl_xor(x[p], m);
        top_of_two<N>(x, y, inf);
    }
}

// Split of the fp32 centroids for the MFMA scores, once per (block, head):
// hi = bf16(c), lo = bf16(c - hi) (c - hi is exact in fp32), and |c|^2 in
// fp32.  Eight channels per thread; the D/8 threads of a row sum its norm.
template <int D>
__global__ __launch_bounds__(256) void route_prep_kernel(int64_t rows, const float* __restrict__ cent,
                                                         uint16_t* __restrict__ chg, uint16_t* __restrict__ clg,
                                                         float* __restrict__ cng)
{
    constexpr int TPR = D / 8;                     // threads per centroid row
    const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t row = t / TPR;
    const int c8 = (int)(t % TPR);
    float x[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    if (row < rows) {
        const float4 a = *(const float4*)(cent + row * D + 8 * c8);
        const float4 b = *(const float4*)(cent + row * D + 8 * c8 + 4);
        x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
        x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
    }
    u32x4_t hi, lo;
    float n2 = 0.f;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const uint32_t h = pack_bf16x2(x[2 * e], x[2 * e + 1]);
        hi[e] = h;
        lo[e] = pack_bf16x2(x[2 * e] - bf16_lo(h), x[2 * e + 1] - bf16_hi(h));
        n2 = __builtin_fmaf(x[2 * e], x[2 * e], n2);
        n2 = __builtin_fmaf(x[2 * e + 1], x[2 * e + 1], n2);
    }
#pragma unroll
    for (int m = 1; m < TPR; m <<= 1) n2 += __shfl_xor(n2, m);
    if (row < rows) {
        *(u32x4_t*)(chg + row * D + 8 * c8) = hi;
        *(u32x4_t*)(clg + row * D + 8 * c8) = lo;
        if (c8 == 0) cng[row] = n2;
    }
}

// (query block g, head h) of workgroup blockIdx.x in a 1-D grid of
// total_blocks * H: head-major, each head's blocks from the last (the longest
// scan) to the first, so the long workgroups start early and short ones fill
// the tail.
__device__ __forceinline__ void route_item(const SegTable& st, int& g, int& h)
{
    const int w = blockIdx.x;
    h = w / st.total_blocks;
    g = st.total_blocks - 1 - (w - h * st.total_blocks);
}

template <int D, int BLK, int KMAX>
// (d = 64 with short lists fits 128 VGPRs: ask for 4 waves per SIMD)
__global__ __launch_bounds__(2 * BLK, ((D == 64 && KMAX <= 8) ? 4 : 1)) void route_mfma_kernel(SegTable st, const uint16_t* __restrict__ q,
                                                             const uint16_t* __restrict__ chg,
                                                             const uint16_t* __restrict__ clg,
                                                             const float* __restrict__ cng,
                                                             int32_t* __restrict__ idx)
{
    constexpr int TB = 64;                 // centroid rows per LDS tile
    constexpr int CS = D + 8;              // LDS row stride (bf16 elements)
    constexpr int NKS = D / 32;            // MFMA k-steps
    constexpr int NT = 2 * BLK;
    constexpr int NW = NT / 64;
    __shared__ __align__(16) uint16_t chi[TB * CS];
    __shared__ __align__(16) uint16_t clo[TB * CS];
    __shared__ float red[NW];

    int g, h;
    route_item(st, g, h);
    const int H = st.H, K = st.K;
    const int s = seq_of_block(st, g);
    const int i = g - st.boff[s];
    const int L = seq_len(st, s);
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int l16 = lane & 15, g4 = lane >> 4;
    const size_t cofs = (size_t)st.boff[s] * H * D + (size_t)h * D;
    const uint16_t* hbase = chg + cofs;
    const uint16_t* lbase = clg + cofs;
    const float* nbase = cng + (size_t)st.boff[s] * H + h;

    int tl[2];
    bool valid[2];
#pragma unroll
    for (int sb = 0; sb < 2; ++sb) {
        tl[sb] = i * BLK + 32 * wave + 16 * sb + l16;
        valid[sb] = tl[sb] < L;
    }
    if (K == 1 || i <= K - 1) {
        // only the own block, or every past block: no scoring
        if (g4 == 0) {
#pragma unroll
            for (int sb = 0; sb < 2; ++sb) {
                if (!valid[sb]) continue;
                int32_t* out = idx + ((size_t)(st.cu[s] + tl[sb]) * H + h) * K;
                if (K == 1) out[0] = i;
                else for (int p = 0; p < K; ++p) out[p] = p <= i ? p : -1;
            }
        }
        return;
    }

    // query fragments (B operand) and |q|^2 (bf16 pair dot products; |q|
    // only scales the error bound E, which carries a 2 % margin)
    u16x8_t qb[2][NKS];
    float qn2[2];
#pragma unroll
    for (int sb = 0; sb < 2; ++sb) {
        float acc = 0.f;
        const uint16_t* qp = q + ((size_t)(st.cu[s] + tl[sb]) * H + h) * D;
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) {
            u16x8_t z = {0, 0, 0, 0, 0, 0, 0, 0};
            qb[sb][ks] = valid[sb] ? *(const u16x8_t*)(qp + 32 * ks + 8 * g4) : z;
            const u32x4_t qw = __builtin_bit_cast(u32x4_t, qb[sb][ks]);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const bf16x2_t x2 = __builtin_bit_cast(bf16x2_t, qw[e]);
                acc = __builtin_amdgcn_fdot2_f32_bf16(x2, x2, acc, false);
            }
        }
        acc += __shfl_xor(acc, 16);
        acc += __shfl_xor(acc, 32);
        qn2[sb] = acc;
    }

    // per-lane key lists (descending); the low LB mantissa bits of a key
    // carry the block id j < i.  A lane keeps LL < KMAX keys (slots LL..
    // KMAX - 1 stay -inf): the query's top K is exact unless one lane holds
    // more than LL of it, which the merge detects (a lane's last kept key
    // above the merged K-th) and sends to the fp64 path.
    // (measured: with k = 8 every slot pays for itself -- 6 slots send too
    // many rows to fp64; with k = 16 a lane holds 11 of the query's top 15
    // rarely enough (about 4 rows in 10^4) that 11 slots route 1024 blocks
    // 12 % faster than 15 and 4 % faster than 13, while 10 slots are slower)
    constexpr int LL = KMAX >= 16 ? KMAX - 5 : KMAX - 1;
    float key[2][KMAX];
#pragma unroll
    for (int sb = 0; sb < 2; ++sb)
#pragma unroll
        for (int p = 0; p < KMAX; ++p) key[sb][p] = -INFINITY;
    // the last, partial group of 16 writes ids up to the next multiple of
    // 16 (its blocks j >= i carry the lowest finite score), so the id field
    // has at least 4 bits: every id then decodes to itself, and a masked
    // block's id stays >= i wherever keys are turned back into block ids
    const int LB = max(4, 32 - __builtin_clz((unsigned)(i - 1) | 1u));
    const uint32_t lmask = (1u << LB) - 1u;
    float cmax2 = 0.f;                      // max |c|^2 over the past blocks

    // score one group of 16 blocks (LDS rows 16*bt..) against both sub-tiles
    // and insert the keys.  In the partial group, blocks j >= i get the
    // lowest finite score, below every real key (-inf would turn into a NaN
    // once j is written into its mantissa); that is a select, not a branch,
    // so every MFMA result is first read in the block that produced it.
    const float pinf = opaque_inf();
    auto group = [&](int bt, int jb, auto partial) {
        u16x8_t ah[NKS], al[NKS];
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) {
            ah[ks] = *(const u16x8_t*)(chi + (16 * bt + l16) * CS + 32 * ks + 8 * g4);
            al[ks] = *(const u16x8_t*)(clo + (16 * bt + l16) * CS + 32 * ks + 8 * g4);
        }
#pragma unroll
        for (int sb = 0; sb < 2; ++sb) {
            f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < NKS; ++ks) {
                acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, ah[ks]),
                                                              __builtin_bit_cast(bf16x8_t, qb[sb][ks]),
                                                              acc, 0, 0, 0);
                acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, al[ks]),
                                                              __builtin_bit_cast(bf16x8_t, qb[sb][ks]),
                                                              acc, 0, 0, 0);
            }
            // lane holds blocks jb + 4*g4 + r for query l16 of sub-tile sb
            if constexpr (decltype(partial)::value) {
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    acc[r] = (jb + 4 * g4 + r < i) ? acc[r] : -__FLT_MAX__;
            }
            // keys: the scores with their low LB mantissa bits replaced by j.
            // Every key runs through the med3 chain in every lane: one at or
            // below the lane's last kept key leaves the list as it was, so
            // no per-key mask is needed (at these list lengths nearly every
            // wave has a passing lane for every key, and a mask only adds
            // the compare and the exec updates)
            float x[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const uint32_t j = (uint32_t)(jb + 4 * g4 + r);
                x[r] = __uint_as_float((__float_as_uint(acc[r]) & ~lmask) | j);
            }
#pragma unroll
            for (int r = 0; r < 4; ++r) {
#pragma unroll
                for (int p = LL - 1; p >= 1; --p)
                    key[sb][p] = __builtin_amdgcn_fmed3f(key[sb][p - 1], key[sb][p], x[r]);
                key[sb][0] = fmax2(key[sb][0], x[r], pinf);
            }
        }
    };

    // tile staging: a thread's 16-byte chunks of a 64-block tile; rows past
    // the scan are clamped to block i - 1 (always inside the sequence), so
    // every load is in bounds and the partial group's extra rows hold real
    // centroids, whose scores are replaced before selection.  The next
    // tile's loads are in flight while the current tile is scored when that
    // takes few registers (d = 64 with 128-query blocks or larger).
    constexpr int NCH = TB * (D / 8);               // 16-byte chunks of a tile
    constexpr int NIT = (NCH + NT - 1) / NT;
    constexpr bool kPrefetch = NIT <= 2;
    u32x4_t xh[NIT], xl[NIT];
    float cn = 0.f;
    auto fetch = [&](int j0) {
#pragma unroll
        for (int it = 0; it < NIT; ++it) {
            const int e = threadIdx.x + it * NT;
            if (NCH % NT == 0 || e < NCH) {
                const int r = e / (D / 8), c8 = e % (D / 8);
                const size_t off = (size_t)min(j0 + r, i - 1) * H * D + 8 * c8;
                xh[it] = *(const u32x4_t*)(hbase + off);
                xl[it] = *(const u32x4_t*)(lbase + off);
            }
        }
        if (threadIdx.x < TB) cn = nbase[(size_t)min(j0 + (int)threadIdx.x, i - 1) * H];
    };
    if constexpr (kPrefetch) fetch(0);
    for (int j0 = 0; j0 < i; j0 += TB) {
        __syncthreads();                            // the previous tile is consumed
        if constexpr (!kPrefetch) fetch(j0);
#pragma unroll
        for (int it = 0; it < NIT; ++it) {
            const int e = threadIdx.x + it * NT;
            if (NCH % NT == 0 || e < NCH) {
                const int r = e / (D / 8), c8 = e % (D / 8);
                *(u32x4_t*)(chi + r * CS + 8 * c8) = xh[it];
                *(u32x4_t*)(clo + r * CS + 8 * c8) = xl[it];
            }
        }
        cmax2 = fmaxf(cmax2, cn);
        __syncthreads();
        if constexpr (kPrefetch)
            if (j0 + TB < i) fetch(j0 + TB);
        for (int bt = 0; bt < TB / 16; ++bt) {
            const int jb = j0 + 16 * bt;
            if (jb + 16 > i) break;                 // full groups here
            group(bt, jb, std::false_type{});
        }
    }
    // the last, partial group of 16 blocks is still in LDS
    if (i & 15) {
        const int jb = i & ~15;
        group((jb % TB) / 16, jb, std::true_type{});
    }
    // max centroid norm over the workgroup
#pragma unroll
    for (int m = 1; m < 64; m <<= 1) cmax2 = fmaxf(cmax2, __shfl_xor(cmax2, m));
    if (lane == 0) red[wave] = cmax2;
    __syncthreads();
    float cm2 = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w) cm2 = fmaxf(cm2, red[w]);
    const float cmax = sqrtf(cm2);
    const float E0 = (1.52587890625e-05f + (float)(2 * D + 16) * 1.1920929e-07f) * 1.02f;

    // Both sub-tiles are merged in one pass.  In the first exchange (lanes
    // l, l^16) a lane keeps the list of the sub-tile ps = g4 & 1 it finishes
    // and sends its partner the other one, so even lane groups merge
    // sub-tile 0 and odd ones sub-tile 1; the second exchange (l, l^32)
    // pairs lanes of the same parity.  Afterwards every lane holds the sorted
    // top KMAX keys of query l16 of sub-tile ps.
    const int ps = g4 & 1;
    float mk[KMAX];
    {
        float y[KMAX];
#pragma unroll
        for (int p = 0; p < KMAX; ++p) {
            mk[p] = ps ? key[1][p] : key[0][p];
            y[p] = __shfl_xor(ps ? key[0][p] : key[1][p], 16);
        }
        top_of_two<KMAX>(mk, y, pinf);
#pragma unroll
        for (int p = 0; p < KMAX; ++p) y[p] = __shfl_xor(mk[p], 32);
        top_of_two<KMAX>(mk, y, pinf);
    }
    float a = mk[0], b = mk[0];
#pragma unroll
    for (int p = 1; p < KMAX; ++p) {
        a = (p == K - 2) ? mk[p] : a;
        b = (p == K - 1) ? mk[p] : b;
    }
    // a lane whose last kept key is above b may have dropped one of the top
    // K: then nothing here is trusted (overflow -> fp64 path)
    float lastmax = fmaxf(ps ? key[1][LL - 1] : key[0][LL - 1],
                          __shfl_xor(ps ? key[0][LL - 1] : key[1][LL - 1], 16));
    lastmax = fmaxf(lastmax, __shfl_xor(lastmax, 32));
    const bool overflow = lastmax > b;
    // keys are within 2^(LB-23)|s| of the MFMA scores
    const float dk = ldexpf(fmaxf(fabsf(a), fabsf(b)), LB - 23) * 1.02f;
    const float Er = E0 * sqrtf(ps ? qn2[1] : qn2[0]) * cmax + 1e-30f;   // MFMA score vs fp64 score
    const float E = Er + dk;
    const bool vp = ps ? valid[1] : valid[0];
    const bool flag = overflow || !(a - b > 2.0f * E);
    if (g4 < 2 && vp && !flag) {
        int sel[KMAX];
#pragma unroll
        for (int p = 0; p < KMAX; ++p) sel[p] = p < K - 1 ? key_block(mk[p], lmask) : 0x7fffffff;
        sort_asc<KMAX>(sel);
        int32_t* out = idx + ((size_t)(st.cu[s] + (ps ? tl[1] : tl[0])) * H + h) * K;
#pragma unroll
        for (int p = 0; p < KMAX; ++p)
            if (p < K - 1) out[p] = sel[p];
        out[K - 1] = i;
    }
    const uint64_t flagged = __ballot(vp && flag);
    if (!flagged) return;

#pragma unroll
    for (int sb = 0; sb < 2; ++sb) {
        // sub-tile sb's rows were finished by the lane groups of parity sb
        if (!(flagged & (0x0000FFFF0000FFFFull << (16 * sb)))) continue;
        const int src = l16 + 16 * sb;
        const float as = __shfl(a, src), Es = __shfl(E, src), Ers = __shfl(Er, src);
        const float lms = __shfl(lastmax, src);
        const bool fls = __shfl((int)flag, src) != 0;
        const bool ovs = __shfl((int)overflow, src) != 0;

        constexpr int MW = 2 * KMAX;
        float wk[MW];
#pragma unroll
        for (int p = 0; p < MW; ++p) wk[p] = p < KMAX ? key[sb][p] : -INFINITY;
        merge_lanes<MW, KMAX>(wk);
        // near-tie: every block that can still be selected has a key >= a - 2E
        // (its exact score is >= a - E), and b is one of them.  If the
        // (K+1)-th key of the query is below a - 2E and no lane dropped a key
        // that high, the K best keys are exactly the candidates: hand them to
        // route_fix_kernel in the row (slot p = -(j + 2)), which re-scores
        // them in fp64 and drops the worst.
        // Otherwise (k >= 6, ids of 16 bits) the row becomes a hint: the
        // blocks of its F = 2K-4 best keys (two ids per slot) and an upper
        // bound ub on the fp64 score of every other block -- its key is at
        // most kn = max(wk[F], lastmax), its MFMA score at most kn plus the id
        // bits, its fp64 score at most that plus Er.  route_fix_kernel scores
        // the F in fp64; if the (K-1)-th of them is above ub they hold the
        // selection.  Failing that (or with no room for a hint) the row is
        // marked for a full fp64 re-selection.
        const float tlow = as - 2.0f * Es;
        float next = wk[0];
#pragma unroll
        for (int p = 1; p < MW; ++p) next = (p == K) ? wk[p] : next;
        const bool cands = !ovs && next < tlow && lms < tlow;
        if (g4 == 0 && valid[sb] && fls) {
            int32_t* out = idx + ((size_t)(st.cu[s] + tl[sb]) * H + h) * K;
            if (cands) {
#pragma unroll
                for (int p = 0; p < KMAX; ++p)
                    if (p < K) out[p] = -(key_block(wk[p], lmask) + 2);
            } else if (K >= kHintMinK && i <= kHintNone) {
                const int F = 2 * K - 4;
                float kf = wk[0];
#pragma unroll
                for (int p = 1; p < MW; ++p) kf = (p == F) ? wk[p] : kf;
                const float kn = fmaxf(kf, lms);
                const float ub = kn == -INFINITY ? -INFINITY
                                                 : (kn + ldexpf(fabsf(kn), LB - 22)) + Ers;
                out[0] = kHint;
                out[1] = __float_as_int(ub);
#pragma unroll
                for (int p = 0; p + 2 < KMAX; ++p) {
                    if (p + 2 < K) {
                        uint32_t w = 0;
#pragma unroll
                        for (int u = 0; u < 2; ++u) {
                            const float kk = wk[2 * p + u];
                            const int j = key_block(kk, lmask);
                            const uint32_t id = (kk > -INFINITY && j < i) ? (uint32_t)j : (uint32_t)kHintNone;
                            w |= id << (16 * u);
                        }
                        out[2 + p] = (int32_t)w;
                    }
                }
            } else {
                out[0] = kPending;
            }
        }
    }
}

// ------------------------------------------------------------------------
// Exact re-selection of the near-tie rows the MFMA kernel left.  Scores are
// fp64, summed sequentially over channels (products of bf16 by fp32 are
// exact in fp64), ties to the lower block id.
//
// Candidate rows (slot p = -(j + 2) for the K best keys): the candidate
// rows of a 64-row chunk are taken 64/KMAX at a time, one lane per (row,
// candidate): the lane re-scores its candidate, ranks it against the row's
// others by shuffles, and the K-1 best are written in ascending block order,
// the own block last.
// fp64 score of a bf16 query row against an fp32 centroid row, summed
// sequentially over the channels (every product is exact in fp64)
template <int D>
__device__ __forceinline__ double score64(const uint16_t* qp, const float* crow)
{
    const float4* cp = (const float4*)crow;
    double acc = 0.0;
#pragma unroll
    for (int c8 = 0; c8 < D / 8; ++c8) {
        const u32x4_t qw = *(const u32x4_t*)(qp + 8 * c8);
        const float4 c0 = cp[2 * c8], c1 = cp[2 * c8 + 1];
        acc = __builtin_fma((double)bf16_lo(qw[0]), (double)c0.x, acc);
        acc = __builtin_fma((double)bf16_hi(qw[0]), (double)c0.y, acc);
        acc = __builtin_fma((double)bf16_lo(qw[1]), (double)c0.z, acc);
        acc = __builtin_fma((double)bf16_hi(qw[1]), (double)c0.w, acc);
        acc = __builtin_fma((double)bf16_lo(qw[2]), (double)c1.x, acc);
        acc = __builtin_fma((double)bf16_hi(qw[2]), (double)c1.y, acc);
        acc = __builtin_fma((double)bf16_lo(qw[3]), (double)c1.z, acc);
        acc = __builtin_fma((double)bf16_hi(qw[3]), (double)c1.w, acc);
    }
    return acc;
}

template <int D, int BLK, int KMAX>
__device__ __forceinline__ void fix_candidate_rows(const SegTable& st, const uint16_t* __restrict__ q,
                                                   const float* cbase, int32_t* __restrict__ idx,
                                                   int s, int i, int h, int r0, int32_t s0)
{
    constexpr int RPW = 64 / KMAX;               // rows per pass
    const int H = st.H, K = st.K;
    const int lane = threadIdx.x & 63;
    const int grp = lane / KMAX, p = lane % KMAX;
    {
        uint64_t cm = __ballot(s0 != kPending && s0 != kHint && s0 <= -2);
        while (cm) {
            // this group's row: the grp-th set bit of cm
            uint64_t m = cm;
            for (int t = 0; t < grp; ++t) m &= m - 1;
            const int src = m ? __builtin_ctzll(m) : -1;
            for (int t = 0; t < RPW; ++t) cm &= cm - 1;
            double sc = -INFINITY;
            int j = 0x7fffffff;
            int32_t* row = nullptr;
            if (src >= 0) row = idx + ((size_t)(st.cu[s] + i * BLK + r0 + src) * H + h) * K;
            // (a candidate is a past block whenever the scores are finite;
            // the check keeps the centroid read inside the sequence's rows
            // when a query or centroid holds a NaN)
            if (src >= 0 && p < K && -row[p] - 2 >= 0 && -row[p] - 2 < i) {
                j = -row[p] - 2;
                sc = score64<D>(q + ((size_t)(st.cu[s] + i * BLK + r0 + src) * H + h) * D,
                                cbase + (size_t)j * H * D);
            }
            // rank against the row's candidates; the last-ranked is dropped
            int rank = 0, pos = 0;
#pragma unroll
            for (int e = 0; e < KMAX; ++e) {
                const double os = __shfl(sc, grp * KMAX + e);
                const int oj = __shfl(j, grp * KMAX + e);
                rank += ranks_before64(os, oj, sc, j) ? 1 : 0;
            }
            const bool keep = src >= 0 && p < K && rank < K - 1;
#pragma unroll
            for (int e = 0; e < KMAX; ++e) {
                const int oj = __shfl(j, grp * KMAX + e);
                const int ok = __shfl(keep ? 1 : 0, grp * KMAX + e);
                pos += (ok && oj < j) ? 1 : 0;
            }
            if (keep) row[pos] = j;
            if (src >= 0 && p == 0) row[K - 1] = i;
        }
    }
}

// Hint rows (slot 0 = kHint; slot 1 = ub as float bits; slots 2.. = the
// block ids of the row's best F = 2K-4 keys, two per slot, kHintNone for
// none): the hint rows of a 64-row chunk are taken 64/(2 KMAX) at a time,
// one lane per (row, finalist).  A lane scores its finalist in fp64 and
// ranks it against the row's others by (score desc, id asc); if the
// (K-1)-th score is above ub, no other block can reach it and the K-1 best
// finalists are written in ascending block order, the own block last.
// Returns the rows (bits of the chunk) whose bound failed.
template <int D, int BLK, int KMAX>
__device__ __forceinline__ uint64_t fix_hint_rows(const SegTable& st, const uint16_t* __restrict__ q,
                                                  const float* cbase, int32_t* __restrict__ idx,
                                                  int s, int i, int h, int r0, int32_t s0)
{
    constexpr int FP = 2 * KMAX;                 // lanes per row (F <= FP)
    constexpr int RPW = 64 / FP;                 // rows per pass
    const int H = st.H, K = st.K, F = 2 * K - 4;
    const int lane = threadIdx.x & 63;
    const int grp = lane / FP, p = lane % FP;
    uint64_t failed = 0;
    uint64_t cm = __ballot(s0 == kHint);
    while (cm) {
        // this group's row: the grp-th set bit of cm
        uint64_t m = cm;
        for (int t = 0; t < grp; ++t) m &= m - 1;
        const int src = m ? __builtin_ctzll(m) : -1;
        for (int t = 0; t < RPW; ++t) cm &= cm - 1;
        double sc = -INFINITY;
        int j = 0x7fffffff;
        float ub = INFINITY;
        int32_t* row = nullptr;
        if (src >= 0) {
            row = idx + ((size_t)(st.cu[s] + i * BLK + r0 + src) * H + h) * K;
            ub = __int_as_float(row[1]);
            if (p < F) {
                const uint32_t w = (uint32_t)row[2 + p / 2];
                const int id = (int)((p & 1) ? (w >> 16) : (w & 0xffffu));
                if (id != kHintNone) {
                    j = id;
                    sc = score64<D>(q + ((size_t)(st.cu[s] + i * BLK + r0 + src) * H + h) * D,
                                    cbase + (size_t)j * H * D);
                }
            }
        }
        const bool real = j != 0x7fffffff;
        int rank = 0;
#pragma unroll
        for (int e = 0; e < FP; ++e) {
            const double os = __shfl(sc, grp * FP + e);
            const int oj = __shfl(j, grp * FP + e);
            rank += ranks_before64(os, oj, sc, j) ? 1 : 0;
        }
        const bool keep = real && rank < K - 1;
        // the (K-1)-th score of the row (-inf with fewer real finalists)
        double t = (real && rank == K - 2) ? sc : -INFINITY;
#pragma unroll
        for (int e = 1; e < FP; e <<= 1) t = fmax(t, __shfl_xor(t, e));
        const bool exact = src >= 0 && t > (double)ub;
        int pos = 0;
#pragma unroll
        for (int e = 0; e < FP; ++e) {
            const int oj = __shfl(j, grp * FP + e);
            const int ok = __shfl(keep ? 1 : 0, grp * FP + e);
            pos += (ok && oj < j) ? 1 : 0;
        }
        if (exact && keep) row[pos] = j;
        if (exact && p == 0) row[K - 1] = i;
        if (src >= 0 && !exact && p == 0) row[0] = kPending;
#pragma unroll
        for (int g = 0; g < RPW; ++g) {
            const int gs = __shfl(src, g * FP);
            const int ge = __shfl(exact ? 1 : 0, g * FP);
            if (gs >= 0 && !ge) failed |= 1ull << gs;
        }
    }
    return failed;
}

// orders one wave's LDS writes before its later reads by other lanes
__device__ __forceinline__ void wave_lds_sync()
{
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Marked rows (slot 0 = kPending), rare: lanes score past blocks j = lane,
// lane + 64, ... and keep their best KMAX by (score desc, index asc) in a
// sorted list; K-1 rounds of a wave-wide argmax over the list heads then
// give the selection in rank order.
template <int D, int BLK, int KMAX>
__device__ __forceinline__ void fix_marked_rows(const SegTable& st, const uint16_t* __restrict__ q,
                                                const float* cbase, int32_t* __restrict__ idx,
                                                float* qstage, int s, int i, int h, int r0, int32_t s0,
                                                uint64_t more)
{
    const int H = st.H, K = st.K;
    const int lane = threadIdx.x & 63;
    {
        // rows marked by the MFMA kernel, and hint rows whose bound failed
        uint64_t fm = __ballot(s0 == kPending) | more;
        while (fm) {
            const int src = __builtin_ctzll(fm);
            fm &= fm - 1;
            const int tq = i * BLK + r0 + src;
            const uint16_t* qp = q + ((size_t)(st.cu[s] + tq) * H + h) * D;
            for (int c = lane; c < D; c += 64) qstage[c] = bf16_to_f32(qp[c]);
            wave_lds_sync();
            double sc[KMAX];
            int jx[KMAX];
#pragma unroll
            for (int p = 0; p < KMAX; ++p) { sc[p] = -INFINITY; jx[p] = 0x7fffffff; }
            const float4* qs = (const float4*)qstage;
            for (int j = lane; j < i; j += 64) {
                const float4* cp = (const float4*)(cbase + (size_t)j * H * D);
                double acc = 0.0;
#pragma unroll 4
                for (int c4 = 0; c4 < D / 4; ++c4) {
                    const float4 cv = cp[c4], qv = qs[c4];
                    acc = __builtin_fma((double)qv.x, (double)cv.x, acc);
                    acc = __builtin_fma((double)qv.y, (double)cv.y, acc);
                    acc = __builtin_fma((double)qv.z, (double)cv.z, acc);
                    acc = __builtin_fma((double)qv.w, (double)cv.w, acc);
                }
                // j grows, so an equal score stays behind the listed ones
                if (acc > sc[KMAX - 1]) insert_tail<KMAX>(sc, jx, acc, j);
            }
            int head = 0;
            int rsel[KMAX];
#pragma unroll
            for (int p = 0; p < KMAX; ++p) rsel[p] = 0x7fffffff;
            for (int r = 0; r < K - 1; ++r) {
                double bs = -INFINITY;
                int bj = 0x7fffffff;
#pragma unroll
                for (int p = 0; p < KMAX; ++p)
                    if (p == head) { bs = sc[p]; bj = jx[p]; }
                const int myj = bj;
#pragma unroll
                for (int m = 1; m < 64; m <<= 1) {
                    const double os = __shfl_xor(bs, m);
                    const int oj = __shfl_xor(bj, m);
                    if (ranks_before64(os, oj, bs, bj)) { bs = os; bj = oj; }
                }
                head += (myj == bj) ? 1 : 0;
#pragma unroll
                for (int p = 0; p < KMAX; ++p)
                    if (p == r) rsel[p] = bj;
            }
            sort_asc<KMAX>(rsel);
            if (lane == 0) {
                int32_t* out = idx + ((size_t)(st.cu[s] + tq) * H + h) * K;
#pragma unroll
                for (int p = 0; p < KMAX; ++p)
                    if (p < K - 1) out[p] = rsel[p];
                out[K - 1] = i;
            }
            wave_lds_sync();
        }
    }
}

// One workgroup per (query block, head), in the MFMA kernel's order, and one
// wave per 64-row chunk of the block: one look at its rows, then its
// candidate, hint and (rare) marked rows.  The waves share nothing (each has
// its own LDS staging row) and never wait for one another.
template <int D, int BLK, int KMAX>
__global__ __launch_bounds__(BLK) void route_fix_kernel(SegTable st, const uint16_t* __restrict__ q,
                                                                      const float* __restrict__ cent,
                                                                      int32_t* __restrict__ idx)
{
    // one wave per 64-row chunk of the query block; the waves share nothing
    __shared__ __align__(16) float qstage[BLK / 64][D];
    int g, h;
    route_item(st, g, h);
    const int H = st.H, K = st.K;
    const int s = seq_of_block(st, g);
    const int i = g - st.boff[s];
    if (K == 1 || i <= K - 1) return;                  // no scoring happened here
    const int L = seq_len(st, s);
    const int lane = threadIdx.x & 63;
    const float* cbase = cent + (size_t)st.boff[s] * H * D + (size_t)h * D;
    const int wave = threadIdx.x >> 6;
    const int r0 = 64 * wave;
    const int tl = i * BLK + r0 + lane;
    int32_t s0 = 0;
    if (tl < L) s0 = idx[((size_t)(st.cu[s] + tl) * H + h) * K];
    fix_candidate_rows<D, BLK, KMAX>(st, q, cbase, idx, s, i, h, r0, s0);
    const uint64_t failed = fix_hint_rows<D, BLK, KMAX>(st, q, cbase, idx, s, i, h, r0, s0);
    fix_marked_rows<D, BLK, KMAX>(st, q, cbase, idx, qstage[wave], s, i, h, r0, s0, failed);
}

template <typename T, int D>
hipError_t launch_d(const Launch& L, const void* q, const float* cent, int32_t* idx)
{
    dim3 grid(L.st.total_blocks, L.st.H);
    dim3 block(L.st.B);
    const int K = L.st.K;
    if (K <= 8)
        hipLaunchKernelGGL((route_kernel<T, D, 8>), grid, block, 0, L.stream, L.st,
                           (const T*)q, cent, idx);
    else if (K <= 16)
        hipLaunchKernelGGL((route_kernel<T, D, 16>), grid, block, 0, L.stream, L.st,
                           (const T*)q, cent, idx);
    else
        hipLaunchKernelGGL((route_kernel<T, D, 32>), grid, block, 0, L.stream, L.st,
                           (const T*)q, cent, idx);
    return hipGetLastError();
}

}  // namespace

template <int D, int BLK, int KMAX>
hipError_t launch_mfma_k(const Launch& L, const uint16_t* q, const float* cent, const RouteWs& w,
                         int32_t* idx)
{
    const dim3 grid((unsigned)L.st.total_blocks * L.st.H);
    hipLaunchKernelGGL((route_mfma_kernel<D, BLK, KMAX>), grid, dim3(2 * BLK), 0, L.stream, L.st, q, w.hi,
                       w.lo, w.n2, idx);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((route_fix_kernel<D, BLK, KMAX>), grid, dim3(BLK), 0, L.stream, L.st, q, cent, idx);
    return hipGetLastError();
}

template <int D, int BLK>
hipError_t launch_mfma(const Launch& L, const void* q, const float* cent, const RouteWs& w, int32_t* idx)
{
    const int K = L.st.K;
    const uint16_t* qq = (const uint16_t*)q;
    const int64_t rows = (int64_t)L.st.total_blocks * L.st.H;
    const int64_t threads = rows * (D / 8);
    hipLaunchKernelGGL((route_prep_kernel<D>), dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, L.stream,
                       rows, cent, w.hi, w.lo, w.n2);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (K <= 8) return launch_mfma_k<D, BLK, 8>(L, qq, cent, w, idx);
    if constexpr (BLK <= 128) {
        // (blocks of 256 / 512 keys are limited to top_k <= 8 by the API)
        if (K <= 16) return launch_mfma_k<D, BLK, 16>(L, qq, cent, w, idx);
        return launch_mfma_k<D, BLK, 32>(L, qq, cent, w, idx);
    }
    return hipErrorInvalidValue;
}

template <int D>
hipError_t launch_mfma_b(const Launch& L, const void* q, const float* cent, const RouteWs& w, int32_t* idx)
{
    switch (L.st.B) {
        case 64: return launch_mfma<D, 64>(L, q, cent, w, idx);
        case 128: return launch_mfma<D, 128>(L, q, cent, w, idx);
        case 256: return launch_mfma<D, 256>(L, q, cent, w, idx);
        case 512: return launch_mfma<D, 512>(L, q, cent, w, idx);
    }
    return hipErrorInvalidValue;
}

RouteWs route_ws(const Launch& L, void* workspace)
{
    const size_t rows = (size_t)L.st.total_blocks * L.st.H;
    const size_t half = align256(rows * L.D * sizeof(uint16_t));
    char* p = (char*)workspace;
    return RouteWs{(uint16_t*)p, (uint16_t*)(p + half), (float*)(p + 2 * half)};
}

size_t route_ws_bytes(const Launch& L)
{
    const size_t rows = (size_t)L.st.total_blocks * L.st.H;
    return 2 * align256(rows * L.D * sizeof(uint16_t)) + align256(rows * sizeof(float));
}

hipError_t launch_route(const Launch& L, const void* q, const float* cent, void* workspace, int32_t* idx)
{
    if (L.st.total_blocks == 0) return hipSuccess;
    if (L.dtype == MOBA_BF16) {
        const RouteWs w = route_ws(L, workspace);
        return L.D == 64 ? launch_mfma_b<64>(L, q, cent, w, idx) : launch_mfma_b<128>(L, q, cent, w, idx);
    }
    return L.D == 64 ? launch_d<float, 64>(L, q, cent, idx)
                     : launch_d<float, 128>(L, q, cent, idx);
}

// ------------------------------------------------------------------------
// The fixed routing scratch of moba_route_topk_noalloc: one copy per GPU,
// held while the process runs.  Host code never passes `scratch` itself (a
// host-side stand-in for the device symbol): it asks for the symbol's
// address on the current device once, and passes that.
}  // namespace moba

static __device__ __align__(256) char scratch[MOBA_ROUTE_SCRATCH_BYTES];

namespace moba {
namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];
}  // namespace

hipError_t route_scratch(void** out)
{
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (!p) return hipErrorInvalidSymbol;
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return hipSuccess;
}

}  // namespace moba
