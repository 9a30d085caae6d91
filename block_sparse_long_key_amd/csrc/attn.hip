// attn.hip -- block-sparse attention of the MoBA forward (gfx950).
//
// "Optimizing Mixture of Block Attention", summary page:
//   - section "Definizione del Compito": O = softmax(QK^T/sqrt(d))V over
//     the selected blocks only;
//   - section "Tre Kernel Fusi", forward "gather-and-densify": for a key
//     block, gather the queries that selected it, keep them on chip and run
//     dense products against the block's keys and values.
// The pages' kernel targets another GPU; here the design is CDNA4-first:
//
// routed kernel -- one workgroup (4 waves) per work item = one key block j
//   of one (sequence, head) and up to 128 of the queries that routed to it.
//   K_j goes to LDS row-major, V_j to LDS transposed (so both MFMA operands
//   are contiguous 16-byte / 8-byte LDS reads).  Each wave gathers 32 query
//   rows straight from HBM into registers and computes, per 16-query
//   sub-tile, S^T = K_j Q^T with v_mfma_f32_16x16x32_bf16 (fp32 accumulate),
//   the row max / exp2 / row sum in fp32, then O^T = V_j^T P^T with the same
//   MFMA: the S^T accumulator layout (4 consecutive keys x 1 query per lane)
//   is exactly the B-operand layout of the second product once keys are
//   paired as {4g..4g+3, 16+4g..16+4g+3}, so P never leaves registers.
//   Output: one normalised partial o (I/O dtype) and its log2-sum-exp per
//   (query, slot).
// own-block kernel -- one workgroup per (query block i, head): the causal
//   tile Q_i K_i^T (u <= t), same MFMA scheme, skipping key tiles that are
//   fully masked, then the merge of that result with the query's routed
//   partials (log-sum-exp weights, fp32), writing O and LSE.
// fp32 I/O uses v_mfma_f32_16x16x4_f32 on the same skeleton (correctness
// path); bf16 rounds P to bf16 for the PV product and normalises by the sum
// of the rounded weights, so each output row is a convex combination of V
// rows with the weights used (fp32 accumulation); the log-sum-exp uses the
// unrounded fp32 weights.
#include "moba_internal.h"

namespace moba {
namespace {

__device__ __forceinline__ f32x4_t mfma_bf16(const u16x8_t& a, const u16x8_t& b, const f32x4_t& c)
{
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                   __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}
__device__ __forceinline__ f32x4_t mfma_f32(float a, float b, const f32x4_t& c)
{
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ float wave_max16(float x)
{
    x = fmaxf(x, __shfl_xor(x, 16));
    x = fmaxf(x, __shfl_xor(x, 32));
    return x;
}
__device__ __forceinline__ float wave_sum16(float x)
{
    x += __shfl_xor(x, 16);
    x += __shfl_xor(x, 32);
    return x;
}

template <typename T, int D, int BLK>
struct Smem {
    static constexpr bool BF = sizeof(T) == 2;
    static constexpr int KS = BF ? D + 8 : D + 4;      // K row stride (elements)
    static constexpr int VS = BF ? BLK + 8 : BLK + 4;  // V^T row stride
    T k[BLK * KS];
    T vt[D * VS];
};

// Load rows [0, nrows) of a key block (rows >= nrows are zero) into LDS:
// K row-major, V transposed.  row u of the block is global row (row0 + u*H).
template <typename T, int D, int BLK, int NT>
__device__ __forceinline__ void load_kv(Smem<T, D, BLK>& sm, const T* __restrict__ k,
                                        const T* __restrict__ v, size_t row0, int H, int nrows)
{
    using S = Smem<T, D, BLK>;
    constexpr int EPC = 16 / sizeof(T);      // elements per 16-byte chunk
    constexpr int CPR = D / EPC;             // chunks per row
    for (int e = threadIdx.x; e < BLK * CPR; e += NT) {
        const int u = e / CPR, c = e % CPR;
        u32x4_t val = {0u, 0u, 0u, 0u};
        if (u < nrows) val = *(const u32x4_t*)(k + (row0 + (size_t)u * H) * D + c * EPC);
        *(u32x4_t*)(sm.k + u * S::KS + c * EPC) = val;
    }
    if constexpr (S::BF) {
        // two rows per thread so V^T is written as 32-bit words
        for (int e = threadIdx.x; e < (BLK / 2) * CPR; e += NT) {
            const int p = e % (BLK / 2), c = e / (BLK / 2);
            const int u = 2 * p;
            u16x8_t v0 = {0, 0, 0, 0, 0, 0, 0, 0}, v1 = v0;
            if (u < nrows) v0 = *(const u16x8_t*)(v + (row0 + (size_t)u * H) * D + c * 8);
            if (u + 1 < nrows) v1 = *(const u16x8_t*)(v + (row0 + (size_t)(u + 1) * H) * D + c * 8);
#pragma unroll
            for (int r = 0; r < 8; ++r) {
                const uint32_t word = (uint32_t)v0[r] | ((uint32_t)v1[r] << 16);
                *(uint32_t*)(sm.vt + (c * 8 + r) * S::VS + u) = word;
            }
        }
    } else {
        for (int e = threadIdx.x; e < BLK * CPR; e += NT) {
            const int u = e % BLK, c = e / BLK;
            float4 val = make_float4(0.f, 0.f, 0.f, 0.f);
            if (u < nrows) val = *(const float4*)((const float*)v + (row0 + (size_t)u * H) * D + c * 4);
            float* dst = (float*)sm.vt + (c * 4) * S::VS + u;
            dst[0] = val.x;
            dst[S::VS] = val.y;
            dst[2 * S::VS] = val.z;
            dst[3 * S::VS] = val.w;
        }
    }
}

// Per-wave tile state for NSB sub-tiles of 16 queries against BLK keys.
template <typename T, int D, int BLK>
struct WaveTile {
    static constexpr bool BF = sizeof(T) == 2;
    static constexpr int NKT = BLK / 16;          // key tiles
    static constexpr int NDT = D / 16;            // dim tiles
    static constexpr int QREG = BF ? D / 32 : D / 4;
    // query fragments: bf16 -> QREG x 8 bf16; fp32 -> QREG floats
    u16x8_t qb[BF ? QREG : 1];
    float qf[BF ? 1 : QREG];
    f32x4_t s[NKT];
    f32x4_t o[NDT];

    // B-operand fragment of query row `qrow` (null -> zero)
    __device__ __forceinline__ void load_q(const T* qrow, int g4)
    {
        if constexpr (BF) {
#pragma unroll
            for (int ks = 0; ks < QREG; ++ks) {
                u16x8_t z = {0, 0, 0, 0, 0, 0, 0, 0};
                qb[ks] = qrow ? *(const u16x8_t*)(qrow + 32 * ks + 8 * g4) : z;
            }
        } else {
            // k-slot g4 of k-step ks <-> dim g4*(D/4) + ks (contiguous per lane)
#pragma unroll
            for (int ks = 0; ks < QREG; ks += 4) {
                float4 z = make_float4(0.f, 0.f, 0.f, 0.f);
                float4 x = qrow ? *(const float4*)((const float*)qrow + g4 * (D / 4) + ks) : z;
                qf[ks] = x.x; qf[ks + 1] = x.y; qf[ks + 2] = x.z; qf[ks + 3] = x.w;
            }
        }
    }

    // S^T tiles kt <= ktmax (others left at zero)
    __device__ __forceinline__ void scores(const Smem<T, D, BLK>& sm, int l16, int g4, int ktmax)
    {
        using S = Smem<T, D, BLK>;
#pragma unroll
        for (int kt = 0; kt < NKT; ++kt) {
            s[kt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
            if (kt > ktmax) continue;
            if constexpr (BF) {
#pragma unroll
                for (int ks = 0; ks < QREG; ++ks) {
                    const u16x8_t a = *(const u16x8_t*)(sm.k + (16 * kt + l16) * S::KS + 32 * ks + 8 * g4);
                    s[kt] = mfma_bf16(a, qb[ks], s[kt]);
                }
            } else {
                const float* kr = (const float*)sm.k + (16 * kt + l16) * S::KS + g4 * (D / 4);
#pragma unroll
                for (int ks = 0; ks < QREG; ++ks) s[kt] = mfma_f32(kr[ks], qf[ks], s[kt]);
            }
        }
    }

    // O^T += V^T P^T over key tiles kt <= ktmax; s[] holds P
    __device__ __forceinline__ void pv(const Smem<T, D, BLK>& sm, int l16, int g4, int ktmax)
    {
        using S = Smem<T, D, BLK>;
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) o[dt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        if constexpr (BF) {
#pragma unroll
            for (int ks2 = 0; ks2 < NKT / 2; ++ks2) {
                if (2 * ks2 > ktmax) continue;
                u16x8_t pb;
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    pb[r] = f32_to_bf16(s[2 * ks2][r]);
                    pb[4 + r] = f32_to_bf16(s[2 * ks2 + 1][r]);
                }
#pragma unroll
                for (int dt = 0; dt < NDT; ++dt) {
                    const uint16_t* vp = sm.vt + (16 * dt + l16) * S::VS + 32 * ks2 + 4 * g4;
                    const u16x4_t lo = *(const u16x4_t*)vp;
                    const u16x4_t hi = *(const u16x4_t*)(vp + 16);
                    const u16x8_t a = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
                    o[dt] = mfma_bf16(a, pb, o[dt]);
                }
            }
        } else {
#pragma unroll
            for (int kt = 0; kt < NKT; ++kt) {
                if (kt > ktmax) continue;
#pragma unroll
                for (int dt = 0; dt < NDT; ++dt) {
                    const float* vp = (const float*)sm.vt + (16 * dt + l16) * S::VS + 16 * kt + 4 * g4;
#pragma unroll
                    for (int r = 0; r < 4; ++r) o[dt] = mfma_f32(vp[r], s[kt][r], o[dt]);
                }
            }
        }
    }
};

template <typename T>
__device__ __forceinline__ void store4(T* p, const float (&x)[4])
{
    if constexpr (sizeof(T) == 2) {
        u32x2_t w;
        w[0] = (uint32_t)f32_to_bf16(x[0]) | ((uint32_t)f32_to_bf16(x[1]) << 16);
        w[1] = (uint32_t)f32_to_bf16(x[2]) | ((uint32_t)f32_to_bf16(x[3]) << 16);
        *(u32x2_t*)p = w;
    } else {
        *(float4*)p = make_float4(x[0], x[1], x[2], x[3]);
    }
}
template <typename T>
__device__ __forceinline__ void load4(const T* p, float (&x)[4])
{
    if constexpr (sizeof(T) == 2) {
        const u32x2_t w = *(const u32x2_t*)p;
        x[0] = __uint_as_float(w[0] << 16);
        x[1] = __uint_as_float(w[0] & 0xffff0000u);
        x[2] = __uint_as_float(w[1] << 16);
        x[3] = __uint_as_float(w[1] & 0xffff0000u);
    } else {
        const float4 v = *(const float4*)p;
        x[0] = v.x; x[1] = v.y; x[2] = v.z; x[3] = v.w;
    }
}

// ------------------------------------------------------------------------
// routed attention: one item = (key block j, <= 128 gathered queries)
template <typename T, int D, int BLK>
__global__ __launch_bounds__(256) void routed_attn_kernel(
    SegTable st, const Item* __restrict__ items, const uint32_t* __restrict__ entries,
    const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v, float sl2,
    T* __restrict__ po, float* __restrict__ pl, int64_t nitems, int64_t per_xcd)
{
    __shared__ __align__(16) Smem<T, D, BLK> sm;
    // the hardware deals workgroups round-robin over the 8 XCDs; give each
    // XCD a contiguous run of items so one (sequence, head) stays in one L2
    const int64_t w = blockIdx.x;
    const int64_t item = (w & 7) * per_xcd + (w >> 3);
    if (item >= nitems) return;
    const Item it = items[item];
    if (it.count <= 0) return;

    const int H = st.H, K = st.K, h = it.h;
    const int s = seq_of_block(st, it.g);
    const int j = it.g - st.boff[s];
    const int t0 = st.cu[s];
    const int L = seq_len(st, s);
    load_kv<T, D, BLK, 256>(sm, k, v, (size_t)(t0 + j * BLK) * H + h, H, BLK);
    __syncthreads();

    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int l16 = lane & 15, g4 = lane >> 4;
    if (32 * wave >= it.count) return;
    const uint32_t* ent = entries + st.ebase[s] + (int64_t)h * L * K + it.begin;

#pragma unroll
    for (int sb = 0; sb < 2; ++sb) {
        const int r = 32 * wave + 16 * sb + l16;
        const bool ok = r < it.count;
        uint32_t e = ok ? ent[r] : 0u;
        const int tq = (int)(e >> 5), slot = (int)(e & 31u);
        WaveTile<T, D, BLK> wt;
        wt.load_q(ok ? q + ((size_t)tq * H + h) * D : nullptr, g4);
        wt.scores(sm, l16, g4, BLK / 16 - 1);
        float mx = -INFINITY;
#pragma unroll
        for (int kt = 0; kt < BLK / 16; ++kt)
#pragma unroll
            for (int r4 = 0; r4 < 4; ++r4) mx = fmaxf(mx, wt.s[kt][r4]);
        const float m2 = wave_max16(mx) * sl2;
        // sum: exact fp32 weights (for the log-sum-exp); sumr: the weights
        // actually used by the PV product (bf16-rounded), for normalising
        float sum = 0.f, sumr = 0.f;
#pragma unroll
        for (int kt = 0; kt < BLK / 16; ++kt)
#pragma unroll
            for (int r4 = 0; r4 < 4; ++r4) {
                const float p = exp2f(__builtin_fmaf(wt.s[kt][r4], sl2, -m2));
                const float pr = (sizeof(T) == 2) ? bf16_to_f32(f32_to_bf16(p)) : p;
                wt.s[kt][r4] = pr;
                sum += p;
                sumr += pr;
            }
        sum = wave_sum16(sum);
        sumr = wave_sum16(sumr);
        wt.pv(sm, l16, g4, BLK / 16 - 1);
        if (ok) {
            const float inv = 1.0f / sumr;
            const size_t prow = ((size_t)tq * H + h) * K + slot;
            T* dst = po + prow * D + 4 * g4;
#pragma unroll
            for (int dt = 0; dt < D / 16; ++dt) {
                float x[4];
#pragma unroll
                for (int r4 = 0; r4 < 4; ++r4) x[r4] = wt.o[dt][r4] * inv;
                store4<T>(dst + 16 * dt, x);
            }
            if (g4 == 0) pl[prow] = m2 + __log2f(sum);
        }
    }
}

// ------------------------------------------------------------------------
// own block (causal) + merge of the routed partials
template <typename T, int D, int BLK>
__global__ __launch_bounds__(2 * BLK) void diag_combine_kernel(
    SegTable st, const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v,
    const int32_t* __restrict__ idx, const T* __restrict__ po, const float* __restrict__ pl,
    float sl2, T* __restrict__ o, float* __restrict__ lse)
{
    __shared__ __align__(16) Smem<T, D, BLK> sm;
    const int g = blockIdx.x, h = blockIdx.y;
    const int H = st.H, K = st.K;
    const int s = seq_of_block(st, g);
    const int i = g - st.boff[s];
    const int t0 = st.cu[s];
    const int L = seq_len(st, s);
    const int nq = min(BLK, L - i * BLK);
    const size_t row0 = (size_t)(t0 + i * BLK) * H + h;
    load_kv<T, D, BLK, 2 * BLK>(sm, k, v, row0, H, nq);
    __syncthreads();

    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int l16 = lane & 15, g4 = lane >> 4;
    if (32 * wave >= nq) return;

#pragma unroll
    for (int sb = 0; sb < 2; ++sb) {
        const int r = 32 * wave + 16 * sb + l16;        // query row in the block
        const bool ok = r < nq;
        const int ktmax = 2 * wave + sb;                // last key tile touching rows of this sub-tile
        const size_t qrow = row0 + (size_t)r * H;
        WaveTile<T, D, BLK> wt;
        wt.load_q(ok ? q + qrow * D : nullptr, g4);
        wt.scores(sm, l16, g4, ktmax);
        float mx = -INFINITY;
#pragma unroll
        for (int kt = 0; kt < BLK / 16; ++kt)
#pragma unroll
            for (int r4 = 0; r4 < 4; ++r4) {
                const int u = 16 * kt + 4 * g4 + r4;
                if (kt > ktmax || u > r) wt.s[kt][r4] = -INFINITY;
                mx = fmaxf(mx, wt.s[kt][r4]);
            }
        const float m2 = wave_max16(mx) * sl2;
        // sum: exact fp32 weights (for the log-sum-exp); sumr: the weights
        // actually used by the PV product (bf16-rounded), for normalising
        float sum = 0.f, sumr = 0.f;
#pragma unroll
        for (int kt = 0; kt < BLK / 16; ++kt)
#pragma unroll
            for (int r4 = 0; r4 < 4; ++r4) {
                const float p = exp2f(__builtin_fmaf(wt.s[kt][r4], sl2, -m2));
                const float pr = (sizeof(T) == 2) ? bf16_to_f32(f32_to_bf16(p)) : p;
                wt.s[kt][r4] = pr;
                sum += p;
                sumr += pr;
            }
        sum = wave_sum16(sum);
        sumr = wave_sum16(sumr);
        wt.pv(sm, l16, g4, ktmax);
        if (!ok) continue;

        // merge: running (M, wsum, acc) in log2 units, own block first
        float acc[D / 16][4];
        const float inv = 1.0f / sumr;
#pragma unroll
        for (int dt = 0; dt < D / 16; ++dt)
#pragma unroll
            for (int r4 = 0; r4 < 4; ++r4) acc[dt][r4] = wt.o[dt][r4] * inv;
        float M = m2 + __log2f(sum);
        float wsum = 1.0f;
        const int32_t* irow = idx + qrow * K;
        for (int p = 0; p < K; ++p) {
            const int jj = irow[p];
            if (jj < 0 || jj >= i) continue;
            const size_t prow = qrow * K + p;
            const float lp = pl[prow];
            if (lp > M) {
                const float f = exp2f(M - lp);
#pragma unroll
                for (int dt = 0; dt < D / 16; ++dt)
#pragma unroll
                    for (int r4 = 0; r4 < 4; ++r4) acc[dt][r4] *= f;
                wsum *= f;
                M = lp;
            }
            const float wgt = exp2f(lp - M);
            wsum += wgt;
            const T* src = po + prow * D + 4 * g4;
#pragma unroll
            for (int dt = 0; dt < D / 16; ++dt) {
                float x[4];
                load4<T>(src + 16 * dt, x);
#pragma unroll
                for (int r4 = 0; r4 < 4; ++r4) acc[dt][r4] = __builtin_fmaf(wgt, x[r4], acc[dt][r4]);
            }
        }
        const float winv = 1.0f / wsum;
        T* dst = o + qrow * D + 4 * g4;
#pragma unroll
        for (int dt = 0; dt < D / 16; ++dt) {
            float x[4];
#pragma unroll
            for (int r4 = 0; r4 < 4; ++r4) x[r4] = acc[dt][r4] * winv;
            store4<T>(dst + 16 * dt, x);
        }
        if (lse && g4 == 0) lse[qrow] = (M + __log2f(wsum)) * 0.69314718055994531f;
    }
}

template <typename T, int D, int BLK>
hipError_t routed_t(const Launch& L, const WsLayout& ws, char* wsp, const void* q, const void* k,
                    const void* v, float sl2)
{
    const int64_t nitems = L.st.total_items;
    if (nitems == 0) return hipSuccess;
    const int64_t per_xcd = (nitems + 7) / 8;
    const int64_t grid = per_xcd * 8;
    hipLaunchKernelGGL((routed_attn_kernel<T, D, BLK>), dim3((unsigned)grid), dim3(256), 0, L.stream,
                       L.st, (const Item*)(wsp + ws.items_off), (const uint32_t*)(wsp + ws.ent_off),
                       (const T*)q, (const T*)k, (const T*)v, sl2, (T*)(wsp + ws.po_off),
                       (float*)(wsp + ws.pl_off), nitems, per_xcd);
    return hipGetLastError();
}

template <typename T, int D, int BLK>
hipError_t diag_t(const Launch& L, const WsLayout& ws, char* wsp, const void* q, const void* k,
                  const void* v, const int32_t* idx, float sl2, void* o, float* lse)
{
    if (L.st.total_blocks == 0) return hipSuccess;
    hipLaunchKernelGGL((diag_combine_kernel<T, D, BLK>), dim3(L.st.total_blocks, L.st.H),
                       dim3(2 * BLK), 0, L.stream, L.st, (const T*)q, (const T*)k, (const T*)v, idx,
                       (const T*)(wsp + ws.po_off), (const float*)(wsp + ws.pl_off), sl2, (T*)o, lse);
    return hipGetLastError();
}

}  // namespace

#define MOBA_DISPATCH(FN, ...)                                                        \
    do {                                                                              \
        const int B_ = L.st.B;                                                        \
        if (L.dtype == MOBA_BF16) {                                                   \
            if (L.D == 64 && B_ == 64) return FN<uint16_t, 64, 64>(__VA_ARGS__);      \
            if (L.D == 64 && B_ == 128) return FN<uint16_t, 64, 128>(__VA_ARGS__);    \
            if (L.D == 128 && B_ == 64) return FN<uint16_t, 128, 64>(__VA_ARGS__);    \
            if (L.D == 128 && B_ == 128) return FN<uint16_t, 128, 128>(__VA_ARGS__);  \
        } else {                                                                      \
            if (L.D == 64 && B_ == 64) return FN<float, 64, 64>(__VA_ARGS__);         \
            if (L.D == 64 && B_ == 128) return FN<float, 64, 128>(__VA_ARGS__);       \
            if (L.D == 128 && B_ == 64) return FN<float, 128, 64>(__VA_ARGS__);       \
        }                                                                             \
        return hipErrorInvalidValue;                                                  \
    } while (0)

hipError_t launch_routed_attn(const Launch& L, const WsLayout& ws, char* wsp, const void* q,
                              const void* k, const void* v, float scale)
{
    if (L.st.K <= 1) return hipSuccess;
    const float sl2 = scale * 1.4426950408889634f;
    MOBA_DISPATCH(routed_t, L, ws, wsp, q, k, v, sl2);
}

hipError_t launch_diag_combine(const Launch& L, const WsLayout& ws, char* wsp, const void* q,
                               const void* k, const void* v, const int32_t* idx, float scale,
                               void* o, float* lse)
{
    const float sl2 = scale * 1.4426950408889634f;
    MOBA_DISPATCH(diag_t, L, ws, wsp, q, k, v, idx, sl2, o, lse);
}

}  // namespace moba
