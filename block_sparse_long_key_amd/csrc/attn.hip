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
//   of one (sequence, head) and up to 2048 of the queries that routed to it,
//   taken in tiles of 128.
//   K_j goes to LDS row-major, V_j to LDS transposed (so both MFMA operands
//   are contiguous 16-byte / 8-byte LDS reads).  Each wave gathers 32 query
//   rows straight from HBM into registers and computes, per 16-query
//   sub-tile, S^T = K_j Q^T with v_mfma_f32_16x16x32_bf16 (fp32 accumulate),
//   the row max / exp2 / row sum in fp32, then O^T = V_j^T P^T with the same
//   MFMA: the S^T accumulator layout (4 consecutive keys x 1 query per lane)
//   is exactly the B-operand layout of the second product once keys are
//   paired as {4g..4g+3, 16+4g..16+4g+3}, so P never leaves registers.
//   Output: one normalised partial o (I/O dtype) and its log2-sum-exp per
//   (query, slot), stored in list order so each tile's writes are one
//   contiguous run of full rows (scattered partial-line writes cost far
//   more than the MFMA work); bf16 rows are staged in LDS and stored whole.
// own-block kernel -- one workgroup per (query block i, head): the causal
//   tile Q_i K_i^T (u <= t), same MFMA scheme, skipping key tiles that are
//   fully masked (bf16 d = 128: V_i^T staged over K_i after the scores),
//   then the merge of that result with the query's routed partials
//   (log-sum-exp weights, fp32), writing O and LSE.
// fp32 I/O uses v_mfma_f32_16x16x4_f32 on the same skeleton (correctness
// path); bf16 rounds P to bf16 for the PV product and normalises by the sum
// of the rounded weights, so each output row is a convex combination of V
// rows with the weights used (fp32 accumulation); the log-sum-exp uses the
// unrounded fp32 weights.  Normalisations multiply by the hardware
// reciprocal (1 ulp: far below the bf16 rounding that follows; x * rcp(x)
// stays within 2^-23 of 1, so V = 1 still gives exactly 1).
#include <math.h>
#include <type_traits>

#include "moba_internal.h"

namespace moba {
namespace {

// waves of a routed-attention workgroup (32 gathered rows each per tile)
constexpr int kRoutedWaves = 4;

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
    // row strides (elements): the MFMA fragment reads of 8 lanes (b128, K)
    // or 16 lanes (b64, V^T) then hit distinct LDS banks -- K rows step 4
    // banks, V^T rows 2 banks
    static constexpr int KS = BF ? D + 8 : D + 4;      // K row stride
    static constexpr int VS = BLK + 4;                 // V^T row stride
    T k[BLK * KS];
    T vt[D * VS];
};

// The same strides with V^T over K's storage: a kernel loads V^T only after
// its last read of K (halves the LDS of one key block's stage).
template <typename T, int D, int BLK>
struct SmemOne {
    static constexpr bool BF = sizeof(T) == 2;
    static constexpr int KS = Smem<T, D, BLK>::KS;
    static constexpr int VS = Smem<T, D, BLK>::VS;
    static constexpr int N = BLK * KS > D * VS ? BLK * KS : D * VS;
    union {
        T k[N];
        T vt[N];
    };
};

// Load rows [0, nrows) of a key block (rows >= nrows are zero) into LDS:
// K row-major (load_k), V transposed (load_vt).  Row u of the block is
// global row (row0 + u*H).
template <typename T, int D, int BLK, int NT, typename SM>
__device__ __forceinline__ void load_k(SM& sm, const T* __restrict__ k, size_t row0, int H, int nrows)
{
    constexpr int EPC = 16 / sizeof(T);      // elements per 16-byte chunk
    constexpr int CPR = D / EPC;             // chunks per row
    for (int e = threadIdx.x; e < BLK * CPR; e += NT) {
        const int u = e / CPR, c = e % CPR;
        u32x4_t val = {0u, 0u, 0u, 0u};
        if (u < nrows) val = *(const u32x4_t*)(k + (row0 + (size_t)u * H) * D + c * EPC);
        *(u32x4_t*)(sm.k + u * SM::KS + c * EPC) = val;
    }
}

template <typename T, int D, int BLK, int NT, typename SM>
__device__ __forceinline__ void load_vt(SM& sm, const T* __restrict__ v, size_t row0, int H, int nrows)
{
    constexpr int EPC = 16 / sizeof(T);
    constexpr int CPR = D / EPC;
    if constexpr (SM::BF) {
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
                *(uint32_t*)(sm.vt + (c * 8 + r) * SM::VS + u) = word;
            }
        }
    } else {
        for (int e = threadIdx.x; e < BLK * CPR; e += NT) {
            const int u = e % BLK, c = e / BLK;
            float4 val = make_float4(0.f, 0.f, 0.f, 0.f);
            if (u < nrows) val = *(const float4*)((const float*)v + (row0 + (size_t)u * H) * D + c * 4);
            float* dst = (float*)sm.vt + (c * 4) * SM::VS + u;
            dst[0] = val.x;
            dst[SM::VS] = val.y;
            dst[2 * SM::VS] = val.z;
            dst[3 * SM::VS] = val.w;
        }
    }
}

template <typename T, int D, int BLK, int NT>
__device__ __forceinline__ void load_kv(Smem<T, D, BLK>& sm, const T* __restrict__ k,
                                        const T* __restrict__ v, size_t row0, int H, int nrows)
{
    load_k<T, D, BLK, NT>(sm, k, row0, H, nrows);
    load_vt<T, D, BLK, NT>(sm, v, row0, H, nrows);
}

// Per-wave tile state: two sub-tiles of 16 queries each against BLK keys.
// Both sub-tiles share every K / V operand fragment read from LDS.
template <typename T, int D, int BLK>
struct Wave2 {
    static constexpr bool BF = sizeof(T) == 2;
    static constexpr int NKT = BLK / 16;          // key tiles
    static constexpr int NDT = D / 16;            // dim tiles
    static constexpr int QREG = BF ? D / 32 : D / 4;
    u16x8_t qb[2][BF ? QREG : 1];                 // bf16: B operand per k-step
    float qf[2][BF ? 1 : QREG];                   // fp32: one k-slot per k-step
    f32x4_t s[2][NKT];
    f32x4_t o[2][NDT];
    uint32_t pk[2][BF ? NKT * 2 : 1];             // bf16: P packed in pairs (PV B operand)
    f32x4_t osum[2];                              // bf16: row sums of the rounded P (MFMA)

    // B-operand fragments of query row `qrow` for sub-tile sb (null -> zero)
    __device__ __forceinline__ void load_q(int sb, const T* qrow, int g4)
    {
        if constexpr (BF) {
#pragma unroll
            for (int ks = 0; ks < QREG; ++ks) {
                u16x8_t z = {0, 0, 0, 0, 0, 0, 0, 0};
                qb[sb][ks] = qrow ? *(const u16x8_t*)(qrow + 32 * ks + 8 * g4) : z;
            }
        } else {
            // k-slot g4 of k-step ks <-> dim g4*(D/4) + ks (contiguous per lane)
#pragma unroll
            for (int ks = 0; ks < QREG; ks += 4) {
                float4 z = make_float4(0.f, 0.f, 0.f, 0.f);
                float4 x = qrow ? *(const float4*)((const float*)qrow + g4 * (D / 4) + ks) : z;
                qf[sb][ks] = x.x; qf[sb][ks + 1] = x.y; qf[sb][ks + 2] = x.z; qf[sb][ks + 3] = x.w;
            }
        }
    }

    // S^T tiles: sub-tile sb computes key tiles kt <= km[sb] (others zero).
    // The K fragments of tile kt+1 are read from LDS while tile kt's MFMAs
    // run; the scheduling fences keep the compiler from hoisting every
    // fragment load (which would double the register footprint).
    template <typename S>
    __device__ __forceinline__ void scores(const S& sm, int l16, int g4, int km0, int km1)
    {
        const int km = km0 > km1 ? km0 : km1;
#pragma unroll
        for (int kt = 0; kt < NKT; ++kt) {
            s[0][kt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
            s[1][kt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        }
        if constexpr (BF) {
            u16x8_t a[QREG], an[QREG];
#pragma unroll
            for (int ks = 0; ks < QREG; ++ks)
                a[ks] = *(const u16x8_t*)(sm.k + l16 * S::KS + 32 * ks + 8 * g4);
#pragma unroll
            for (int kt = 0; kt < NKT; ++kt) {
                if (kt > km) break;
                if (kt + 1 < NKT) {
#pragma unroll
                    for (int ks = 0; ks < QREG; ++ks)
                        an[ks] = *(const u16x8_t*)(sm.k + (16 * (kt + 1) + l16) * S::KS + 32 * ks + 8 * g4);
                }
#pragma unroll
                for (int ks = 0; ks < QREG; ++ks) {
                    if (kt <= km0) s[0][kt] = mfma_bf16(a[ks], qb[0][ks], s[0][kt]);
                    if (kt <= km1) s[1][kt] = mfma_bf16(a[ks], qb[1][ks], s[1][kt]);
                }
#pragma unroll
                for (int ks = 0; ks < QREG; ++ks) a[ks] = an[ks];
                __builtin_amdgcn_sched_barrier(0);
            }
        } else {
#pragma unroll
            for (int kt = 0; kt < NKT; ++kt) {
                if (kt > km) break;
                const float* kr = (const float*)sm.k + (16 * kt + l16) * S::KS + g4 * (D / 4);
#pragma unroll
                for (int ks = 0; ks < QREG; ++ks) {
                    const float a = kr[ks];
                    if (kt <= km0) s[0][kt] = mfma_f32(a, qf[0][ks], s[0][kt]);
                    if (kt <= km1) s[1][kt] = mfma_f32(a, qf[1][ks], s[1][kt]);
                }
                __builtin_amdgcn_sched_barrier(0);
            }
        }
    }

    // O^T = V^T P^T over key tiles kt <= km[sb]; s[] holds P.  One key step
    // (32 keys) at a time, fenced like scores().
    template <typename S>
    __device__ __forceinline__ void pv(const S& sm, int l16, int g4, int km0, int km1)
    {
        const int km = km0 > km1 ? km0 : km1;
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) {
            o[0][dt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
            o[1][dt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        }
        if constexpr (BF) {
            // an all-ones A operand turns one more MFMA per key step into the
            // row sums of the bf16 weights, accumulated exactly like O
            osum[0] = f32x4_t{0.f, 0.f, 0.f, 0.f};
            osum[1] = f32x4_t{0.f, 0.f, 0.f, 0.f};
            const u16x8_t ones = {0x3f80, 0x3f80, 0x3f80, 0x3f80, 0x3f80, 0x3f80, 0x3f80, 0x3f80};
#pragma unroll
            for (int ks2 = 0; ks2 < NKT / 2; ++ks2) {
                if (2 * ks2 > km) break;
                u16x8_t pb[2];
#pragma unroll
                for (int sb = 0; sb < 2; ++sb) {
                    u32x4_t w = {pk[sb][4 * ks2], pk[sb][4 * ks2 + 1], pk[sb][4 * ks2 + 2], pk[sb][4 * ks2 + 3]};
                    pb[sb] = __builtin_bit_cast(u16x8_t, w);
                }
#pragma unroll
                for (int dt = 0; dt < NDT; ++dt) {
                    const uint16_t* vp = sm.vt + (16 * dt + l16) * S::VS + 32 * ks2 + 4 * g4;
                    const u16x4_t lo = *(const u16x4_t*)vp;
                    const u16x4_t hi = *(const u16x4_t*)(vp + 16);
                    const u16x8_t a = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
                    if (2 * ks2 <= km0) o[0][dt] = mfma_bf16(a, pb[0], o[0][dt]);
                    if (2 * ks2 <= km1) o[1][dt] = mfma_bf16(a, pb[1], o[1][dt]);
                }
                if (2 * ks2 <= km0) osum[0] = mfma_bf16(ones, pb[0], osum[0]);
                if (2 * ks2 <= km1) osum[1] = mfma_bf16(ones, pb[1], osum[1]);
                __builtin_amdgcn_sched_barrier(0);
            }
        } else {
#pragma unroll
            for (int kt = 0; kt < NKT; ++kt) {
                if (kt > km) break;
#pragma unroll
                for (int dt = 0; dt < NDT; ++dt) {
                    const float* vp = (const float*)sm.vt + (16 * dt + l16) * S::VS + 16 * kt + 4 * g4;
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const float a = vp[r];
                        if (kt <= km0) o[0][dt] = mfma_f32(a, s[0][kt][r], o[0][dt]);
                        if (kt <= km1) o[1][dt] = mfma_f32(a, s[1][kt][r], o[1][dt]);
                    }
                }
                __builtin_amdgcn_sched_barrier(0);
            }
        }
    }

    // softmax of sub-tile sb in log2 units; key u > ulim masked when MASK.
    // Returns m2 and the sum of the exact fp32 weights (for the log-sum-exp);
    // bf16 packs P for the PV product.
    template <bool MASK>
    __device__ __forceinline__ void softmax(int sb, float sl2, int g4, int km, int ulim,
                                            float& m2, float& sum)
    {
        float mx = -INFINITY;
#pragma unroll
        for (int kt = 0; kt < NKT; ++kt)
#pragma unroll
            for (int r4 = 0; r4 < 4; ++r4) {
                if constexpr (MASK) {
                    const int u = 16 * kt + 4 * g4 + r4;
                    if (kt > km || u > ulim) s[sb][kt][r4] = -INFINITY;
                }
                mx = fmaxf(mx, s[sb][kt][r4]);
            }
        m2 = wave_max16(mx) * sl2;
        float a0 = 0.f, a1 = 0.f;
#pragma unroll
        for (int kt = 0; kt < NKT; ++kt)
#pragma unroll
            for (int r4 = 0; r4 < 4; ++r4) {
                const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(s[sb][kt][r4], sl2, -m2));
                s[sb][kt][r4] = p;
                if (r4 & 1) a1 += p; else a0 += p;
            }
        if constexpr (BF) {
            // key tiles 2c and 2c+1 form the 8-key group of PV step c
#pragma unroll
            for (int kt = 0; kt < NKT; ++kt)
#pragma unroll
                for (int h2 = 0; h2 < 2; ++h2)
                    pk[sb][4 * (kt / 2) + 2 * (kt % 2) + h2] =
                        pack_bf16x2(s[sb][kt][2 * h2], s[sb][kt][2 * h2 + 1]);
        }
        sum = wave_sum16(a0 + a1);
    }

    // sum of the weights the PV product used (call after pv)
    __device__ __forceinline__ float used_sum(int sb, float sum) const
    {
        if constexpr (BF) return osum[sb][0];
        else return sum;
    }
};

// A partial-output row is stored permuted so that each lane's values are
// contiguous: dim 16*dt + 4*g + r (the O^T accumulator layout) lives at
// g*(D/4) + 4*dt + r.  Lane g reads / writes D/4 consecutive elements.
template <typename T, int NDT>
__device__ __forceinline__ void store_lane_row(T* p, const float (&x)[NDT][4])
{
    if constexpr (sizeof(T) == 2) {
#pragma unroll
        for (int c = 0; c < NDT / 2; ++c) {
            u32x4_t w;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int dt = 2 * c + e / 2, r = 2 * (e % 2);
                w[e] = pack_bf16x2(x[dt][r], x[dt][r + 1]);
            }
            *(u32x4_t*)(p + 8 * c) = w;
        }
    } else {
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) {
            *(f32x4_t*)(p + 4 * dt) = f32x4_t{x[dt][0], x[dt][1], x[dt][2], x[dt][3]};
        }
    }
}

template <typename T, int NDT>
struct LaneRow {
    // packed copy of one lane's D/4 elements of a partial row
    u32x4_t w[sizeof(T) == 2 ? NDT / 2 : NDT];
    __device__ __forceinline__ void load(const T* p)
    {
#pragma unroll
        for (int c = 0; c < (sizeof(T) == 2 ? NDT / 2 : NDT); ++c) w[c] = *(const u32x4_t*)(p + (16 / sizeof(T)) * c);
    }
    __device__ __forceinline__ float get(int dt, int r) const
    {
        if constexpr (sizeof(T) == 2) {
            const uint32_t word = w[dt / 2][2 * (dt % 2) + r / 2];
            return __uint_as_float((r & 1) ? (word & 0xffff0000u) : (word << 16));
        } else {
            return __uint_as_float(w[dt][r]);
        }
    }
};

// O (row-contiguous dims) store of one lane's O^T values
template <typename T>
__device__ __forceinline__ void store4(T* p, const float (&x)[4])
{
    if constexpr (sizeof(T) == 2) {
        u32x2_t w;
        w[0] = pack_bf16x2(x[0], x[1]);
        w[1] = pack_bf16x2(x[2], x[3]);
        *(u32x2_t*)p = w;
    } else {
        *(float4*)p = make_float4(x[0], x[1], x[2], x[3]);
    }
}

// ------------------------------------------------------------------------
// routed attention: one item = (key block j, <= item_rows gathered queries),
// processed in tiles of 128 queries (4 waves x 2 sub-tiles x 16) while K_j
// and V_j stay in LDS
template <typename T, int D, int BLK>
// (bf16 d = 64: at most 128 VGPRs, 4 waves per SIMD)
__global__ __launch_bounds__(64 * kRoutedWaves, (sizeof(T) == 2 && D == 64 ? 4 : 1)) void routed_attn_kernel(
    SegTable st, const Item* __restrict__ items, const uint32_t* __restrict__ entries,
    const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v, float sl2,
    T* __restrict__ po, float* __restrict__ pl, float* __restrict__ pm, int64_t nitems,
    int64_t per_xcd)
{
    __shared__ __align__(16) Smem<T, D, BLK> sm;
    // bf16: entries are read from global memory (L2) a tile ahead instead of
    // from an LDS copy, and partial rows are staged 8 at a time, so LDS
    // allows 4 workgroups per CU at d = 64 (3 with the copy: routed kernel
    // -10 % at B = 128) and 2 at d = 128 (1 with 16 staged rows).  With
    // 64-key blocks LDS never limits and the LDS copy is kept.
    constexpr bool LDS_ENT = sizeof(T) != 2 || (D == 64 && BLK == 64);
    __shared__ uint32_t sent[LDS_ENT ? kItemRows : 1];
    constexpr int NDT = D / 16;
    using W = Wave2<T, D, BLK>;
    // bf16: each wave stages its 16 partial rows of a sub-tile in LDS and
    // stores them as whole contiguous 16-byte chunks (64 lanes = 1 KB per
    // instruction) instead of half rows; rows padded by 16 B so the 8-lane
    // b128 writes hit distinct banks
    constexpr bool STAGE = sizeof(T) == 2;
    constexpr int RB = D * (int)sizeof(T);            // partial row bytes
    constexpr int RS = RB + 16;                       // staged row stride
    constexpr int SR = LDS_ENT ? 16 : 8;              // rows staged per pass
    __shared__ __align__(16) char ostage[STAGE ? kRoutedWaves * SR * RS : 16];
    constexpr int NT = 64 * kRoutedWaves;             // threads
    constexpr int TR = 32 * kRoutedWaves;             // rows per tile
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
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int l16 = lane & 15, g4 = lane >> 4;
    // (debug builds: the item lies inside its (sequence, head) list region)
    if (!MOBA_INBOUNDS(it.g >= 0 && it.g < st.total_blocks && h >= 0 && h < H && j < seq_nblk(st, s) &&
                       it.begin >= 0 && (int64_t)it.begin + it.count <= (int64_t)L * K, kDbgItem))
        return;

    // the item's (query, slot) entries go to LDS once; its partials are
    // written at the same (list-order) positions, so every tile writes one
    // contiguous run of full rows
    const int64_t e0 = st.ebase[s] + (int64_t)h * L * K + it.begin;
    const uint32_t* ent = entries + e0;
    if constexpr (LDS_ENT)
        for (int r = threadIdx.x; r < it.count; r += NT) sent[r] = ent[r];

    // gathered query fragments of the first tile are requested before the
    // K / V staging so the two overlap
    W wt;
    u16x8_t qn[2][W::BF ? W::QREG : 1];
    float qfn[2][W::BF ? 1 : W::QREG];
    int base = 32 * wave;
    // the entries (query, slot) of a tile's two sub-tile rows of this lane
    auto tile_ent = [&](int b0, const uint32_t* src, uint32_t (&e)[2]) {
#pragma unroll
        for (int sb = 0; sb < 2; ++sb) {
            const int r = b0 + 16 * sb + l16;
            e[sb] = r < it.count ? src[r] : 0u;
        }
    };
    auto fetch_q = [&](int b0, u16x8_t (&qb)[2][W::BF ? W::QREG : 1], float (&qf)[2][W::BF ? 1 : W::QREG],
                       const uint32_t (&ev)[2]) {
#pragma unroll
        for (int sb = 0; sb < 2; ++sb) {
            const int r = b0 + 16 * sb + l16;
            const uint32_t e = ev[sb];
            const bool ok = r < it.count &&
                            MOBA_INBOUNDS((int)(e >> 5) >= t0 && (int)(e >> 5) < t0 + L && (int)(e & 31u) < K,
                                          kDbgEntry);
            const T* qrow = ok ? q + ((size_t)(e >> 5) * H + h) * D : nullptr;
            if constexpr (W::BF) {
#pragma unroll
                for (int ks = 0; ks < W::QREG; ++ks) {
                    u16x8_t z = {0, 0, 0, 0, 0, 0, 0, 0};
                    qb[sb][ks] = qrow ? *(const u16x8_t*)(qrow + 32 * ks + 8 * g4) : z;
                }
            } else {
#pragma unroll
                for (int ks = 0; ks < W::QREG; ks += 4) {
                    float4 z = make_float4(0.f, 0.f, 0.f, 0.f);
                    float4 x = qrow ? *(const float4*)((const float*)qrow + g4 * (D / 4) + ks) : z;
                    qf[sb][ks] = x.x; qf[sb][ks + 1] = x.y; qf[sb][ks + 2] = x.z; qf[sb][ks + 3] = x.w;
                }
            }
        }
    };
    uint32_t en[2];
    tile_ent(base, ent, en);
    if (base < it.count) fetch_q(base, qn, qfn, en);
    // entries from global memory are requested a tile before their rows, so
    // a row gather never waits for its entry
    if constexpr (!LDS_ENT) tile_ent(base + TR, ent, en);
    load_kv<T, D, BLK, NT>(sm, k, v, (size_t)(t0 + j * BLK) * H + h, H, BLK);
    __syncthreads();

    for (; base < it.count; base += TR) {
        // current tile's fragments; the next tile's are requested now and
        // arrive while this one computes
        bool ok[2];
#pragma unroll
        for (int sb = 0; sb < 2; ++sb) {
            const int r = base + 16 * sb + l16;
            ok[sb] = r < it.count;
            if constexpr (W::BF) {
#pragma unroll
                for (int ks = 0; ks < W::QREG; ++ks) wt.qb[sb][ks] = qn[sb][ks];
            } else {
#pragma unroll
                for (int ks = 0; ks < W::QREG; ++ks) wt.qf[sb][ks] = qfn[sb][ks];
            }
        }
        if (base + TR < it.count) {
            if constexpr (LDS_ENT) tile_ent(base + TR, sent, en);
            fetch_q(base + TR, qn, qfn, en);
            if constexpr (!LDS_ENT) tile_ent(base + 2 * TR, ent, en);
        }
        wt.scores(sm, l16, g4, BLK / 16 - 1, BLK / 16 - 1);
        float m2[2], sum[2];
#pragma unroll
        for (int sb = 0; sb < 2; ++sb)
            wt.template softmax<false>(sb, sl2, g4, BLK / 16 - 1, BLK, m2[sb], sum[sb]);
        wt.pv(sm, l16, g4, BLK / 16 - 1, BLK / 16 - 1);
#pragma unroll
        for (int sb = 0; sb < 2; ++sb) {
            const int row0 = base + 16 * sb;                  // first row of the sub-tile
            if (row0 >= it.count) continue;                   // wave-uniform
            const float inv = __builtin_amdgcn_rcpf(wt.used_sum(sb, sum[sb]));
            const size_t prow = (size_t)(e0 + row0 + l16);
            float x[NDT][4];
#pragma unroll
            for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
                for (int r4 = 0; r4 < 4; ++r4) x[dt][r4] = wt.o[sb][dt][r4] * inv;
            if constexpr (STAGE) {
                char* st_w = ostage + wave * SR * RS;
                constexpr int CPR = RB / 16;                  // 16-byte chunks per row
#pragma unroll
                for (int hp = 0; hp < 16 / SR; ++hp) {
                    // rows hp*SR .. hp*SR + SR-1 of the sub-tile
                    if (l16 / SR == hp)
                        store_lane_row<T, NDT>((T*)(st_w + (l16 % SR) * RS) + g4 * (D / 4), x);
                    // (LDS accesses of one wave complete in order)
#pragma unroll
                    for (int n = 0; n < SR * CPR / 64; ++n) {
                        const int qc = 64 * n + lane, r = qc / CPR, c = qc % CPR;
                        const int rr = hp * SR + r;
                        const u32x4_t w = *(const u32x4_t*)(st_w + r * RS + c * 16);
                        if (row0 + rr < it.count)
                            // whole rows, non-temporal: read back only by the
                            // merge kernel, much later; kept out of the way in
                            // L2 they leave room for the gathered query rows
                            // other lists reuse (routed reads 1.76 -> 1.40 GB
                            // at 2 x 64K)
                            __builtin_nontemporal_store(w, (u32x4_t*)((char*)po + (size_t)(e0 + row0 + rr) * RB + c * 16));
                    }
                }
            } else {
                // (64-byte pieces of rows: a non-temporal hint would skip the
                // L2 merge of the pieces -- measured 2x slower at d = 128)
                if (ok[sb]) store_lane_row<T, NDT>(po + prow * D + g4 * (D / 4), x);
            }
            if (ok[sb] && g4 == 0) {
                const float lv = m2[sb] + __builtin_amdgcn_logf(sum[sb]);
                if (pm) {
                    // BLASST: the log2-sum-exp and the block's maximum score
                    // (log2 units) side by side, so the merge's skip decision
                    // and its weight come from one 8-byte read
                    const f32x2_t lm = {lv, m2[sb]};
                    __builtin_nontemporal_store(lm, (f32x2_t*)pm + prow);
                } else if constexpr (STAGE) {
                    __builtin_nontemporal_store(lv, pl + prow);
                } else {
                    pl[prow] = lv;
                }
            }
        }
    }
}

// ------------------------------------------------------------------------
// own block (causal) + merge of the routed partials.
// Phase A: the causal tile on MFMA, as in the routed kernel.  Phase B: the
// own-block result goes to LDS (over the K rows, no longer needed) in the
// partials' lane-permuted layout.  Phase C: lanes are re-mapped to
// (query, 16-byte chunk); the query's list positions come from the reverse
// map built by the index pass, its partial rows are gathered as coalesced
// 16-byte chunks and merged with a running (max, sum) in log2 units.
// BL: the BLASST variant (skip decisions, the kept selection, the partials'
// (lse, maximum) pairs); the plain merge is compiled without that code.
template <typename T, int D, int BLK, bool BL>
__global__ __launch_bounds__(2 * BLK, (sizeof(T) == 2 && D == 64 ? 4 : 1)) void diag_combine_kernel(
    SegTable st, const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v,
    const int32_t* __restrict__ rev, const T* __restrict__ po, const float* __restrict__ pl,
    const float* __restrict__ pm, float log2lam, float sl2, T* __restrict__ o,
    float* __restrict__ lse, const int32_t* __restrict__ idx, int32_t* __restrict__ kept)
{
    // bf16 d = 128: V^T is loaded over K once the scores are done, so the
    // stage takes half the LDS and 3 workgroups fit a CU (2 otherwise)
    constexpr bool ONE = sizeof(T) == 2 && D == 128;
    using SM = std::conditional_t<ONE, SmemOne<T, D, BLK>, Smem<T, D, BLK>>;
    __shared__ __align__(16) SM sm;
    __shared__ float own_lse[BLK];
    __shared__ float own_max[BLK];            // BLASST: own block's maximum (log2 units)
    constexpr int NDT = D / 16;
    constexpr int CH = 16 / sizeof(T);        // elements per 16-byte chunk
    constexpr int NCH = D / CH;               // chunks per row
    constexpr int QPP = 64 / NCH;             // queries per wave pass
    constexpr int PF = 8;                     // slots loaded together
    static_assert(BLK * D <= BLK * SM::KS, "own rows fit over K");
    T* own = sm.k;                            // [BLK][D], lane-permuted rows

    const int g = blockIdx.x, h = blockIdx.y;
    const int H = st.H, K = st.K;
    const int s = seq_of_block(st, g);
    const int i = g - st.boff[s];
    const int t0 = st.cu[s];
    const int L = seq_len(st, s);
    const int nq = min(BLK, L - i * BLK);
    const size_t row0 = (size_t)(t0 + i * BLK) * H + h;
    load_k<T, D, BLK, 2 * BLK>(sm, k, row0, H, nq);
    if constexpr (!ONE) load_vt<T, D, BLK, 2 * BLK>(sm, v, row0, H, nq);
    __syncthreads();

    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int l16 = lane & 15, g4 = lane >> 4;
    const bool active = 32 * wave < nq;

    // ---- phase A
    Wave2<T, D, BLK> wt;
    float m2[2], sum[2];
    if (active) {
#pragma unroll
        for (int sb = 0; sb < 2; ++sb) {
            const int r = 32 * wave + 16 * sb + l16;
            wt.load_q(sb, r < nq ? q + (row0 + (size_t)r * H) * D : nullptr, g4);
        }
        const int km0 = 2 * wave, km1 = 2 * wave + 1;   // last key tile of each sub-tile
        wt.scores(sm, l16, g4, km0, km1);
#pragma unroll
        for (int sb = 0; sb < 2; ++sb)
            wt.template softmax<true>(sb, sl2, g4, sb ? km1 : km0, 32 * wave + 16 * sb + l16,
                                      m2[sb], sum[sb]);
    }
    if constexpr (ONE) {
        __syncthreads();                      // every wave is done with K
        load_vt<T, D, BLK, 2 * BLK>(sm, v, row0, H, nq);
        __syncthreads();
    }
    if (active) {
        const int km0 = 2 * wave, km1 = 2 * wave + 1;
        wt.pv(sm, l16, g4, km0, km1);
    }
    __syncthreads();
    // ---- phase B
    if (active) {
#pragma unroll
        for (int sb = 0; sb < 2; ++sb) {
            const int r = 32 * wave + 16 * sb + l16;
            const float inv = __builtin_amdgcn_rcpf(wt.used_sum(sb, sum[sb]));
            float x[NDT][4];
#pragma unroll
            for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
                for (int r4 = 0; r4 < 4; ++r4) x[dt][r4] = wt.o[sb][dt][r4] * inv;
            store_lane_row<T, NDT>(own + r * D + g4 * (D / 4), x);
            if (g4 == 0) {
                own_lse[r] = m2[sb] + __builtin_amdgcn_logf(sum[sb]);
                own_max[r] = m2[sb];
            }
        }
    }
    __syncthreads();
    if (!active) return;
    // ---- phase C
    const int c = lane % NCH, ql = lane / NCH;
    for (int pass = 0; pass < 32 / QPP; ++pass) {
        const int r = 32 * wave + pass * QPP + ql;
        if (r >= nq) break;
        const size_t qrow = row0 + (size_t)r * H;
        float acc[CH];
        {
            const u32x4_t w = *(const u32x4_t*)(own + r * D + c * CH);
            if constexpr (sizeof(T) == 2) {
#pragma unroll
                for (int e = 0; e < 4; ++e) { acc[2 * e] = bf16_lo(w[e]); acc[2 * e + 1] = bf16_hi(w[e]); }
            } else {
#pragma unroll
                for (int e = 0; e < 4; ++e) acc[e] = __uint_as_float(w[e]);
            }
        }
        // the query's K list positions (-1: nothing routed in that slot)
        const int32_t* rrow = rev + ((size_t)h * st.cu[st.nseq] + t0 + i * BLK + r) * K;
        const int64_t eb = st.ebase[s] + (int64_t)h * L * K;
        const int kmerge = K > 1 ? K : 0;      // K == 1: no routed partials exist
        // BLASST ("BLASST", summary page, "Meccanismo di Pruning"): blocks in
        // ascending order (the slot order), the own block last; a block whose
        // maximum is more than -log2(lambda) below the running maximum of the
        // kept blocks takes no part.  Without it every slot is kept.
        uint32_t keepm = 0xffffffffu;
        bool own_kept = true;
        if (BL && pm) {
            float Mr = -INFINITY;
            keepm = 0u;
            // PF slots' list positions, then their block maxima, are
            // requested together; the decisions then run in registers, in
            // slot order
            for (int p0 = 0; p0 < kmerge; p0 += PF) {
                int pos[PF];
                float mt[PF];
#pragma unroll
                for (int u = 0; u < PF; ++u) {
                    pos[u] = p0 + u < kmerge ? rrow[p0 + u] : -1;
                    if (pos[u] >= 0 && !MOBA_INBOUNDS(pos[u] < L * K, kDbgMergePos)) pos[u] = -1;
                }
#pragma unroll
                for (int u = 0; u < PF; ++u) mt[u] = pos[u] >= 0 ? ((const f32x2_t*)pm)[eb + pos[u]][1] : 0.f;
#pragma unroll
                for (int u = 0; u < PF; ++u) {
                    if (pos[u] < 0) continue;
                    if (!(Mr > -INFINITY && mt[u] - Mr < log2lam)) {
                        keepm |= 1u << (p0 + u);
                        Mr = fmaxf(Mr, mt[u]);
                    }
                }
            }
            own_kept = !(Mr > -INFINITY && own_max[r] - Mr < log2lam);
        }
        // the attended selection: idx's routed blocks that were kept, then
        // the own block if kept, ascending, -1 padded
        if (BL && kept && c == 0) {
            const int32_t* irow = idx + qrow * K;
            int32_t* krow = kept + qrow * K;
            int n = 0;
            for (int p = 0; p < kmerge; ++p) {
                const int j = irow[p];
                if (j >= 0 && j < i && rrow[p] >= 0 && ((keepm >> p) & 1u)) krow[n++] = j;
            }
            if (own_kept && n < K) krow[n++] = i;
            for (; n < K; ++n) krow[n] = -1;
        }
        float M = own_lse[r];
        float wsum = 1.0f;
        if (!own_kept) {
            M = -INFINITY;
            wsum = 0.f;
#pragma unroll
            for (int e = 0; e < CH; ++e) acc[e] = 0.f;
        }
        for (int p0 = 0; p0 < kmerge; p0 += PF) {
            int pos[PF];
#pragma unroll
            for (int u = 0; u < PF; ++u) {
                pos[u] = (p0 + u < kmerge && ((keepm >> (p0 + u)) & 1u)) ? rrow[p0 + u] : -1;
                if (pos[u] >= 0 && !MOBA_INBOUNDS(pos[u] < L * K, kDbgMergePos)) pos[u] = -1;
            }
            float lp[PF];
            u32x4_t xv[PF];
#pragma unroll
            for (int u = 0; u < PF; ++u) {
                if (pos[u] >= 0) {
                    const int64_t prow = eb + pos[u];
                    // (BLASST: the pair the decision just read, now cached)
                    lp[u] = (BL && pm) ? ((const f32x2_t*)pm)[prow][0] : pl[prow];
                    xv[u] = *(const u32x4_t*)(po + prow * D + c * CH);
                }
            }
#pragma unroll
            for (int u = 0; u < PF; ++u) {
                if (pos[u] < 0) continue;
                if (lp[u] > M) {
                    const float f = __builtin_amdgcn_exp2f(M - lp[u]);
#pragma unroll
                    for (int e = 0; e < CH; ++e) acc[e] *= f;
                    wsum *= f;
                    M = lp[u];
                }
                const float wgt = __builtin_amdgcn_exp2f(lp[u] - M);
                wsum += wgt;
                if constexpr (sizeof(T) == 2) {
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        acc[2 * e] = __builtin_fmaf(wgt, bf16_lo(xv[u][e]), acc[2 * e]);
                        acc[2 * e + 1] = __builtin_fmaf(wgt, bf16_hi(xv[u][e]), acc[2 * e + 1]);
                    }
                } else {
#pragma unroll
                    for (int e = 0; e < 4; ++e) acc[e] = __builtin_fmaf(wgt, __uint_as_float(xv[u][e]), acc[e]);
                }
            }
        }
        // stored position c*CH + e holds dim 16*dt + 4*gg + r4 with
        // gg = pos / (D/4), dt = (pos % (D/4)) / 4: runs of 4 consecutive dims
        const float winv = __builtin_amdgcn_rcpf(wsum);
#pragma unroll
        for (int e4 = 0; e4 < CH / 4; ++e4) {
            const int pos = c * CH + 4 * e4;
            const int dim = 16 * ((pos % (D / 4)) / 4) + 4 * (pos / (D / 4));
            float x[4];
#pragma unroll
            for (int r4 = 0; r4 < 4; ++r4) x[r4] = acc[4 * e4 + r4] * winv;
            store4<T>(o + qrow * D + dim, x);
        }
        if (lse && c == 0) lse[qrow] = (M + __builtin_amdgcn_logf(wsum)) * 0.69314718055994531f;
    }
}

template <typename T, int D, int BLK>
hipError_t routed_t(const Launch& L, const WsLayout& ws, char* wsp, const void* q, const void* k,
                    const void* v, float sl2, bool block_max)
{
    const int64_t nitems = L.st.total_items;
    if (nitems == 0) return hipSuccess;
    const int64_t per_xcd = (nitems + 7) / 8;
    const int64_t grid = per_xcd * 8;
    hipLaunchKernelGGL((routed_attn_kernel<T, D, BLK>), dim3((unsigned)grid), dim3(64 * kRoutedWaves), 0, L.stream,
                       L.st, (const Item*)(wsp + ws.items_off), (const uint32_t*)(wsp + ws.ent_off),
                       (const T*)q, (const T*)k, (const T*)v, sl2, (T*)(wsp + ws.po_off),
                       (float*)(wsp + ws.pl_off), block_max ? (float*)(wsp + ws.pm_off) : nullptr,
                       nitems, per_xcd);
    return hipGetLastError();
}

template <typename T, int D, int BLK>
hipError_t diag_t(const Launch& L, const WsLayout& ws, char* wsp, const void* q, const void* k,
                  const void* v, const int32_t* idx, float sl2, void* o, float* lse,
                  float blasst_lambda, int32_t* kept)
{
    if (L.st.total_blocks == 0) return hipSuccess;
    // the index pass turned idx into the reverse map; idx itself is read
    // only to write the kept selection
    const bool bl = blasst_lambda > 0.f || kept;
    auto kern = bl ? diag_combine_kernel<T, D, BLK, true> : diag_combine_kernel<T, D, BLK, false>;
    hipLaunchKernelGGL(kern, dim3(L.st.total_blocks, L.st.H),
                       dim3(2 * BLK), 0, L.stream, L.st, (const T*)q, (const T*)k, (const T*)v,
                       (const int32_t*)(wsp + ws.rev_off), (const T*)(wsp + ws.po_off),
                       (const float*)(wsp + ws.pl_off),
                       blasst_lambda > 0.f ? (const float*)(wsp + ws.pm_off) : nullptr,
                       blasst_lambda > 0.f ? log2f(blasst_lambda) : 0.f, sl2, (T*)o, lse,
                       idx, kept);
    return hipGetLastError();
}

}  // namespace

uint32_t dbg_take_attn()
{
#ifdef MOBA_DEBUG_BOUNDS
    return dbg_take_local();
#else
    return 0u;
#endif
}

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
                              const void* k, const void* v, float scale, bool block_max)
{
    if (L.st.K <= 1) return hipSuccess;
    const float sl2 = scale * 1.4426950408889634f;
    MOBA_DISPATCH(routed_t, L, ws, wsp, q, k, v, sl2, block_max);
}

hipError_t launch_diag_combine(const Launch& L, const WsLayout& ws, char* wsp, const void* q,
                               const void* k, const void* v, const int32_t* idx, float scale,
                               void* o, float* lse, float blasst_lambda, int32_t* kept)
{
    const float sl2 = scale * 1.4426950408889634f;
    MOBA_DISPATCH(diag_t, L, ws, wsp, q, k, v, idx, sl2, o, lse, blasst_lambda, kept);
}

}  // namespace moba
