// attn_bwd.hip -- gradients of the MoBA block-sparse attention (gfx950, bf16).
//
// "Optimizing Mixture of Block Attention", summary page, section "Backward
// Pass: Ricalcolo (Algoritmo 5)": FlashAttention-2 style recomputation,
// parallel over keys (one workgroup per key block), gathering the queries
// that selected the block as the forward does, and summing the per-query
// dQ pieces in a high-precision buffer.  The pages accumulate dQ with
// atomics; here every (query, slot) piece is written once, fp32, at its
// list position, and a query-major pass adds them in a fixed order, so the
// result is deterministic and no line is contended.
//
// prep kernel -- per (token, head): D_t = dO_t . O_t (fp32, from the
//   forward's O) and the forward's log-sum-exp in log2 units.
// list kernel -- one workgroup (4 waves) per (key block j, head): K_j and
//   V_j stay in LDS; tiles of 32 query rows (first the causal own-block
//   rows of block j, then the rows of j's routed list) are staged in LDS
//   and, with wave w owning keys [w*BLK/4, (w+1)*BLK/4):
//     S  = Q K_j^T, dP = dO V_j^T      (MFMA, A = rows, B = K/V rows)
//     P  = exp2(S log2e*scale - lse2), dS = P (dP - D)
//     dV_j^T += dO^T P, dK_j^T += Q^T dS   (A = LDS transpose reads of the
//                                           dO / Q tile, B = P / dS straight
//                                           from the S accumulators)
//     dQ^T = K_j^T dS^T                 (dS^T through LDS; both operands
//                                        are LDS transpose reads)
//   dK_j, dV_j leave once, in bf16; each tile's dQ rows (fp32, 4 dims per
//   lane) go to the row's list position (routed) or to the own-block area.
// combine kernel -- per (token, head): dq = scale * (own-block piece + the
//   routed pieces found through the reverse map), rounded to bf16.
//
// Operand layouts of v_mfma_f32_16x16x32_bf16 used below: A lane (row l16,
// k = 8*g4..8*g4+7), B lane (column l16, same k), C lane (column l16, rows
// 4*g4..4*g4+3).  ds_read_b64_tr_b16: within each 16-lane group, lane L
// names an 8-byte chunk; output lane l receives element l%4 of the chunks
// of lanes l/4, 4+l/4, 8+l/4, 12+l/4.  With lane L pointing at row
// r0 + L/4, columns c0 + 4*(L%4) of a row-major bf16 tile, lane l gets
// column c0 + l of rows r0..r0+3: a 4 x 16 tile read transposed.
#include <type_traits>

#include "moba_internal.h"

namespace moba {
namespace {

constexpr int kBwdThreads = 256;     // 4 waves
constexpr int kTileRows = 32;        // query rows per tile

typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4_t lds_s16x4_t;

__device__ __forceinline__ u16x4_t tr_read(const uint16_t* p)
{
    const s16x4_t r = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)p);
    return __builtin_bit_cast(u16x4_t, r);
}

__device__ __forceinline__ u16x8_t cat(const u16x4_t& a, const u16x4_t& b)
{
    return u16x8_t{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
}

__device__ __forceinline__ f32x4_t mfma(const u16x8_t& a, const u16x8_t& b, const f32x4_t& c)
{
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                   __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

__device__ __forceinline__ u16x8_t pack8(const f32x4_t& lo, const f32x4_t& hi)
{
    const u32x4_t w = {pack_bf16x2(lo[0], lo[1]), pack_bf16x2(lo[2], lo[3]),
                       pack_bf16x2(hi[0], hi[1]), pack_bf16x2(hi[2], hi[3])};
    return __builtin_bit_cast(u16x8_t, w);
}

// ------------------------------------------------------------------------
// D_t = dO_t . O_t and lse2_t = lse_t * log2(e), one row per D/8 lanes
template <int D>
__global__ __launch_bounds__(kBwdThreads) void bwd_prep_kernel(int64_t rows, const uint16_t* __restrict__ o,
                                                               const uint16_t* __restrict__ dout,
                                                               const float* __restrict__ lse,
                                                               float2* __restrict__ rowstat)
{
    constexpr int CPR = D / 8;
    const int64_t gid = (int64_t)blockIdx.x * kBwdThreads + threadIdx.x;
    const int64_t r = gid / CPR;
    const int c = (int)(gid % CPR);
    float acc = 0.f;
    if (r < rows) {
        const u32x4_t a = *(const u32x4_t*)(o + r * D + 8 * c);
        const u32x4_t b = *(const u32x4_t*)(dout + r * D + 8 * c);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            acc = __builtin_fmaf(bf16_lo(a[e]), bf16_lo(b[e]), acc);
            acc = __builtin_fmaf(bf16_hi(a[e]), bf16_hi(b[e]), acc);
        }
    }
#pragma unroll
    for (int m = 1; m < CPR; m <<= 1) acc += __shfl_xor(acc, m);
    if (r < rows && c == 0) rowstat[r] = make_float2(lse[r] * 1.4426950408889634f, acc);
}

// ------------------------------------------------------------------------
template <int D, int BLK>
struct BwdSmem {
    static constexpr int RS = D + 8;            // K / V / Q / dO row stride (elements)
    static constexpr int SS = kTileRows + 16;   // dS^T row stride (elements)
    uint16_t k[BLK * RS];
    uint16_t v[BLK * RS];
    uint16_t q[kTileRows * RS];
    uint16_t dout[kTileRows * RS];
    uint16_t dst[BLK * SS];                     // dS^T [key][query]
    float lse2[kTileRows];
    float dsum[kTileRows];
    int64_t dest[kTileRows];                    // dq piece row, -1 = none
};

// waves per list workgroup: d = 128 with 128-key blocks splits the keys over
// 8 waves (16 each) so the per-wave dK / dV accumulators fit 2 waves per SIMD
template <int D, int BLK>
constexpr int bwd_waves() { return (D == 128 && BLK == 128) ? 8 : 4; }

template <int D, int BLK>
__global__ __launch_bounds__((64 * bwd_waves<D, BLK>()), 2) void bwd_list_kernel(
    SegTable st, const int2* __restrict__ lst, const uint32_t* __restrict__ entries,
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    const uint16_t* __restrict__ dout, const float2* __restrict__ rowstat, float sl2, float scale,
    float* __restrict__ pq, int64_t diag_base, uint16_t* __restrict__ dk, uint16_t* __restrict__ dv,
    int64_t nlists, int64_t per_xcd, int routed, const uint8_t* __restrict__ own)
{
    using S = BwdSmem<D, BLK>;
    __shared__ __align__(16) S sm;
    constexpr int RS = S::RS, SS = S::SS;
    constexpr int NW = bwd_waves<D, BLK>();
    constexpr int NT = 64 * NW;
    constexpr int KPW = BLK / NW;               // keys per wave
    constexpr int NKS = KPW / 16;               // 16-key sub-blocks per wave
    constexpr int NDT = D / 16;                 // 16-dim blocks
    constexpr int CPR = D / 8;                  // 16-byte chunks per staged row
    constexpr int RPP = NT / CPR;               // staged rows per pass
    constexpr int NPASS = kTileRows / RPP;
    constexpr int NB = 2 * NDT / NW;            // dQ^T blocks per wave (of 2 * NDT)
    static_assert(NKS >= 1 && NPASS >= 1, "shape");

    // contiguous runs of lists per XCD (the hardware deals workgroups
    // round-robin over the 8 XCDs), so one head's rows stay in one L2
    const int64_t wg = blockIdx.x;
    const int64_t item = (wg & 7) * per_xcd + (wg >> 3);
    if (item >= nlists) return;
    const int H = st.H, K = st.K;
    const int h = (int)(item / st.total_blocks), g = (int)(item % st.total_blocks);
    const int s = seq_of_block(st, g);
    const int j = g - st.boff[s];
    const int t0 = st.cu[s];
    const int L = seq_len(st, s);
    const int nq = min(BLK, L - j * BLK);        // rows of block j
    int2 li = make_int2(0, 0);
    if (routed) li = lst[item];
    // (debug builds: the list lies inside its (sequence, head) region)
    if (!MOBA_INBOUNDS(li.x >= 0 && li.y >= 0 && (int64_t)li.x + li.y <= (int64_t)L * K, kDbgBwdList))
        li = make_int2(0, 0);
    const int64_t eb = st.ebase[s] + (int64_t)h * L * K;
    const int ndiag = (nq + kTileRows - 1) / kTileRows;
    const int ntiles = ndiag + (li.y + kTileRows - 1) / kTileRows;

    const int tid = threadIdx.x;
    const int wave = tid >> 6, lane = tid & 63;
    const int l16 = lane & 15, g4 = lane >> 4;
    const int kw0 = wave * KPW;

    // ---- K_j, V_j to LDS (rows >= nq zero)
    {
        const size_t row0 = (size_t)(t0 + j * BLK) * H + h;
        for (int e = tid; e < BLK * CPR; e += NT) {
            const int u = e / CPR, c = e % CPR;
            u32x4_t kk = {0u, 0u, 0u, 0u}, vv = kk;
            if (u < nq) {
                kk = *(const u32x4_t*)(k + (row0 + (size_t)u * H) * D + 8 * c);
                vv = *(const u32x4_t*)(v + (row0 + (size_t)u * H) * D + 8 * c);
            }
            *(u32x4_t*)(sm.k + u * RS + 8 * c) = kk;
            *(u32x4_t*)(sm.v + u * RS + 8 * c) = vv;
        }
    }

    // ---- staging of one tile's rows into registers
    const int sc = tid % CPR, sr = tid / CPR;
    u32x4_t pre_q[NPASS], pre_do[NPASS];
    float2 pre_stat[NPASS];
    int64_t pre_dest[NPASS];
    // a routed row's token comes from its list entry; entries are loaded
    // two tiles ahead and the rows one tile ahead, so the two dependent
    // global loads of a routed row never sit on one tile's critical path
    uint32_t pre_e[NPASS];
    auto fetch_ent = [&](int tile) {
        if (tile < ndiag || tile >= ntiles) return;
#pragma unroll
        for (int p = 0; p < NPASS; ++p) {
            const int rr = kTileRows * (tile - ndiag) + sr + RPP * p;
            pre_e[p] = rr < li.y ? entries[eb + li.x + rr] : 0u;
        }
    };
    auto fetch = [&](int tile) {
#pragma unroll
        for (int p = 0; p < NPASS; ++p) {
            const int r = sr + RPP * p;
            bool ok;
            int t;
            int64_t dest;
            if (tile < ndiag) {
                const int ql = kTileRows * tile + r;
                ok = ql < nq;
                t = t0 + j * BLK + ql;
                dest = diag_base + (int64_t)t * H + h;
            } else {
                const int rr = kTileRows * (tile - ndiag) + r;
                t = (int)(pre_e[p] >> 5);
                ok = rr < li.y &&
                     MOBA_INBOUNDS(t >= t0 && t < t0 + L && (int)(pre_e[p] & 31u) < K, kDbgBwdEntry);
                dest = eb + li.x + rr;
            }
            const size_t row = (size_t)t * H + h;
            u32x4_t z = {0u, 0u, 0u, 0u};
            pre_q[p] = ok ? *(const u32x4_t*)(q + row * D + 8 * sc) : z;
            pre_do[p] = ok ? *(const u32x4_t*)(dout + row * D + 8 * sc) : z;
            // a row that leaves its own block out (own[row] == 0) takes
            // part in the own-block tile with P = 0: no dK / dV share and a
            // zero dq piece
            const bool live = ok && !(own && tile < ndiag && !own[row]);
            pre_stat[p] = (live && sc == 0) ? rowstat[row] : make_float2(__builtin_inff(), 0.f);
            pre_dest[p] = ok ? dest : -1;
        }
    };
    fetch_ent(0);
    if (ntiles > 0) fetch(0);
    fetch_ent(1);

    // d = 64: the wave's K / V fragments (B operands of S and dP) and K^T
    // fragments (A operands of dQ^T) are the same for every tile; they are
    // read from LDS once and kept in registers
    constexpr bool KREG = D == 64;
    const int qs_w = wave / (NW / 2);            // this wave's dQ^T query sub-block
    u16x8_t kbr[KREG ? NKS : 1][KREG ? D / 32 : 1], vbr[KREG ? NKS : 1][KREG ? D / 32 : 1];
    u16x8_t kar[KREG ? NB : 1][KREG ? BLK / 32 : 1];
    auto kfrag = [&](int ks, int kk) -> u16x8_t {
        return *(const u16x8_t*)(sm.k + (kw0 + 16 * ks + l16) * RS + 32 * kk + 8 * g4);
    };
    auto vfrag = [&](int ks, int kk) -> u16x8_t {
        return *(const u16x8_t*)(sm.v + (kw0 + 16 * ks + l16) * RS + 32 * kk + 8 * g4);
    };
    auto ktfrag = [&](int b, int kk) -> u16x8_t {
        const int dt = (wave % (NW / 2)) * NB + b;
        const int r0 = 32 * kk + 8 * g4 + (l16 >> 2);
        return cat(tr_read(sm.k + r0 * RS + 16 * dt + 4 * (l16 & 3)),
                   tr_read(sm.k + (r0 + 4) * RS + 16 * dt + 4 * (l16 & 3)));
    };
    if constexpr (KREG) {
        __syncthreads();
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks)
#pragma unroll
            for (int kk = 0; kk < D / 32; ++kk) {
                kbr[ks][kk] = kfrag(ks, kk);
                vbr[ks][kk] = vfrag(ks, kk);
            }
#pragma unroll
        for (int b = 0; b < NB; ++b)
#pragma unroll
            for (int kk = 0; kk < BLK / 32; ++kk) kar[b][kk] = ktfrag(b, kk);
    }

    f32x4_t dvt[NDT][NKS], dkt[NDT][NKS];
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) {
            dvt[dt][ks] = f32x4_t{0.f, 0.f, 0.f, 0.f};
            dkt[dt][ks] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        }

    for (int tile = 0; tile < ntiles; ++tile) {
        // ---- staged rows to LDS
#pragma unroll
        for (int p = 0; p < NPASS; ++p) {
            const int r = sr + RPP * p;
            *(u32x4_t*)(sm.q + r * RS + 8 * sc) = pre_q[p];
            *(u32x4_t*)(sm.dout + r * RS + 8 * sc) = pre_do[p];
            if (sc == 0) {
                sm.lse2[r] = pre_stat[p].x;
                sm.dsum[r] = pre_stat[p].y;
                sm.dest[r] = pre_dest[p];
            }
        }
        __syncthreads();
        const int64_t mydest = sm.dest[16 * qs_w + l16];
        if (tile + 1 < ntiles) fetch(tile + 1);
        fetch_ent(tile + 2);

        // ---- S = Q K^T, dP = dO V^T over this wave's keys
        f32x4_t sacc[2][NKS], pacc[2][NKS];
#pragma unroll
        for (int qs = 0; qs < 2; ++qs)
#pragma unroll
            for (int ks = 0; ks < NKS; ++ks) {
                sacc[qs][ks] = f32x4_t{0.f, 0.f, 0.f, 0.f};
                pacc[qs][ks] = f32x4_t{0.f, 0.f, 0.f, 0.f};
            }
#pragma unroll
        for (int kk = 0; kk < D / 32; ++kk) {
            u16x8_t qa[2], da[2];
#pragma unroll
            for (int qs = 0; qs < 2; ++qs) {
                qa[qs] = *(const u16x8_t*)(sm.q + (16 * qs + l16) * RS + 32 * kk + 8 * g4);
                da[qs] = *(const u16x8_t*)(sm.dout + (16 * qs + l16) * RS + 32 * kk + 8 * g4);
            }
#pragma unroll
            for (int ks = 0; ks < NKS; ++ks) {
                u16x8_t kb, vb;
                if constexpr (KREG) { kb = kbr[ks][kk]; vb = vbr[ks][kk]; }
                else { kb = kfrag(ks, kk); vb = vfrag(ks, kk); }
#pragma unroll
                for (int qs = 0; qs < 2; ++qs) {
                    sacc[qs][ks] = mfma(qa[qs], kb, sacc[qs][ks]);
                    pacc[qs][ks] = mfma(da[qs], vb, pacc[qs][ks]);
                }
            }
        }
        // ---- P and dS (C layout: key kw0+16ks+l16, query 16qs+4g4+r); the
        // causal mask key <= query exists only in the own-block tiles
        auto softmax_grad = [&](auto masked) {
            constexpr bool MASK = decltype(masked)::value;
            const int qb = kTileRows * tile;
#pragma unroll
            for (int qs = 0; qs < 2; ++qs) {
                const float4 l2 = *(const float4*)(sm.lse2 + 16 * qs + 4 * g4);
                const float4 dd = *(const float4*)(sm.dsum + 16 * qs + 4 * g4);
                const float lr[4] = {l2.x, l2.y, l2.z, l2.w};
                const float dr[4] = {dd.x, dd.y, dd.z, dd.w};
#pragma unroll
                for (int ks = 0; ks < NKS; ++ks) {
                    const int key = kw0 + 16 * ks + l16;
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        float p = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[qs][ks][r], sl2, -lr[r]));
                        if constexpr (MASK) p = key > qb + 16 * qs + 4 * g4 + r ? 0.f : p;
                        sacc[qs][ks][r] = p;
                        pacc[qs][ks][r] = p * (pacc[qs][ks][r] - dr[r]);
                    }
                }
            }
        };
        if (tile < ndiag) softmax_grad(std::true_type{});
        else softmax_grad(std::false_type{});
        // ---- dV^T += dO^T P, dK^T += Q^T dS; dS^T to LDS
        u16x8_t pb[NKS], sb[NKS];
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) {
            pb[ks] = pack8(sacc[0][ks], sacc[1][ks]);
            sb[ks] = pack8(pacc[0][ks], pacc[1][ks]);
            const u32x4_t w = __builtin_bit_cast(u32x4_t, sb[ks]);
#pragma unroll
            for (int qs = 0; qs < 2; ++qs)
                *(u32x2_t*)(sm.dst + (kw0 + 16 * ks + l16) * SS + 16 * qs + 4 * g4) =
                    u32x2_t{w[2 * qs], w[2 * qs + 1]};
        }
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) {
            const int off_lo = (4 * g4 + (l16 >> 2)) * RS + 16 * dt + 4 * (l16 & 3);
            const int off_hi = off_lo + 16 * RS;
            const u16x8_t doa = cat(tr_read(sm.dout + off_lo), tr_read(sm.dout + off_hi));
            const u16x8_t qta = cat(tr_read(sm.q + off_lo), tr_read(sm.q + off_hi));
#pragma unroll
            for (int ks = 0; ks < NKS; ++ks) {
                dvt[dt][ks] = mfma(doa, pb[ks], dvt[dt][ks]);
                dkt[dt][ks] = mfma(qta, sb[ks], dkt[dt][ks]);
            }
        }
        __syncthreads();
        // ---- dQ^T = K^T dS^T for query sub-block qs_w, NB dim blocks
#pragma unroll
        for (int b = 0; b < NB; ++b) {
            const int dt = (wave % (NW / 2)) * NB + b;
            f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kk = 0; kk < BLK / 32; ++kk) {
                const int r0 = 32 * kk + 8 * g4 + (l16 >> 2);
                u16x8_t ka;
                if constexpr (KREG) ka = kar[b][kk];
                else ka = ktfrag(b, kk);
                const u16x8_t sbb = cat(tr_read(sm.dst + r0 * SS + 16 * qs_w + 4 * (l16 & 3)),
                                        tr_read(sm.dst + (r0 + 4) * SS + 16 * qs_w + 4 * (l16 & 3)));
                acc = mfma(ka, sbb, acc);
            }
            if (mydest >= 0)
                *(float4*)(pq + mydest * D + 16 * dt + 4 * g4) = make_float4(acc[0], acc[1], acc[2], acc[3]);
        }
    }

    // ---- dK_j = scale * dK^T, dV_j (lane: key kw0+16ks+l16, dims 16dt+4g4..+3)
    const size_t row0 = (size_t)(t0 + j * BLK) * H + h;
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
        const int u = kw0 + 16 * ks + l16;
        if (u >= nq) continue;
        const size_t row = row0 + (size_t)u * H;
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) {
            *(u32x2_t*)(dk + row * D + 16 * dt + 4 * g4) =
                u32x2_t{pack_bf16x2(dkt[dt][ks][0] * scale, dkt[dt][ks][1] * scale),
                        pack_bf16x2(dkt[dt][ks][2] * scale, dkt[dt][ks][3] * scale)};
            *(u32x2_t*)(dv + row * D + 16 * dt + 4 * g4) =
                u32x2_t{pack_bf16x2(dvt[dt][ks][0], dvt[dt][ks][1]),
                        pack_bf16x2(dvt[dt][ks][2], dvt[dt][ks][3])};
        }
    }
}

// ------------------------------------------------------------------------
// dq_t = scale * (own-block piece + routed pieces), D/4 lanes per row
template <int D>
__global__ __launch_bounds__(kBwdThreads) void dq_combine_kernel(SegTable st, int tokens,
                                                                 const int32_t* __restrict__ rev,
                                                                 const float* __restrict__ pq,
                                                                 int64_t diag_base, float scale,
                                                                 uint16_t* __restrict__ dq)
{
    constexpr int CPR = D / 4;
    constexpr int RPW = kBwdThreads / CPR;
    constexpr int PF = 8;
    const int h = blockIdx.y;
    const int t = blockIdx.x * RPW + threadIdx.x / CPR;
    const int c = threadIdx.x % CPR;
    if (t >= tokens) return;
    const int H = st.H, K = st.K;
    const int64_t own = diag_base + (int64_t)t * H + h;
    float4 acc = *(const float4*)(pq + own * D + 4 * c);
    if (K > 1) {
        const int s = seq_of_token(st, t);
        const int64_t eb = st.ebase[s] + (int64_t)h * seq_len(st, s) * K;
        const int32_t* rrow = rev + ((size_t)h * tokens + t) * K;
        for (int p0 = 0; p0 < K; p0 += PF) {
            int pos[PF];
#pragma unroll
            for (int u = 0; u < PF; ++u) {
                pos[u] = p0 + u < K ? rrow[p0 + u] : -1;
                if (pos[u] >= 0 && !MOBA_INBOUNDS(pos[u] < seq_len(st, s) * K, kDbgDqPos)) pos[u] = -1;
            }
            float4 x[PF];
#pragma unroll
            for (int u = 0; u < PF; ++u)
                x[u] = pos[u] >= 0 ? *(const float4*)(pq + (eb + pos[u]) * D + 4 * c)
                                   : make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
            for (int u = 0; u < PF; ++u) {
                acc.x += x[u].x; acc.y += x[u].y; acc.z += x[u].z; acc.w += x[u].w;
            }
        }
    }
    *(u32x2_t*)(dq + ((size_t)t * H + h) * D + 4 * c) =
        u32x2_t{pack_bf16x2(acc.x * scale, acc.y * scale), pack_bf16x2(acc.z * scale, acc.w * scale)};
}

// own[row] = 1 iff idx's row lists the row's own block (t - cu[s]) / B
__global__ __launch_bounds__(kBwdThreads) void own_flags_kernel(SegTable st, int64_t rows,
                                                                const int32_t* __restrict__ idx,
                                                                uint8_t* __restrict__ own)
{
    const int64_t row = (int64_t)blockIdx.x * kBwdThreads + threadIdx.x;
    if (row >= rows) return;
    const int t = (int)(row / st.H);
    const int s = seq_of_token(st, t);
    const int i = (t - st.cu[s]) / st.B;
    const int32_t* r = idx + row * st.K;
    bool f = false;
    for (int p = 0; p < st.K; ++p) f |= r[p] == i;
    own[row] = f ? 1 : 0;
}

template <int D, int BLK>
hipError_t bwd_t(const Launch& L, const WsLayout& ws, char* wsp, const void* q, const void* k,
                 const void* v, const void* o, const float* lse, const void* dout, float scale,
                 void* dq, void* dk, void* dv, const uint8_t* own)
{
    const SegTable& st = L.st;
    const int64_t rows = (int64_t)L.tokens * st.H;
    float2* rowstat = (float2*)(wsp + ws.rs_off);
    float* pq = (float*)(wsp + ws.pq_off);
    const int64_t diag_base = st.K > 1 ? st.ebase[st.nseq] : 0;
    {
        const int64_t thr = rows * (D / 8);
        const unsigned grid = (unsigned)((thr + kBwdThreads - 1) / kBwdThreads);
        hipLaunchKernelGGL((bwd_prep_kernel<D>), dim3(grid), dim3(kBwdThreads), 0, L.stream, rows,
                           (const uint16_t*)o, (const uint16_t*)dout, lse, rowstat);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    {
        const int64_t nlists = (int64_t)st.total_blocks * st.H;
        const int64_t per_xcd = (nlists + 7) / 8;
        hipLaunchKernelGGL((bwd_list_kernel<D, BLK>), dim3((unsigned)(per_xcd * 8)), dim3(64 * bwd_waves<D, BLK>()), 0,
                           L.stream, st, (const int2*)(wsp + ws.lst_off), (const uint32_t*)(wsp + ws.ent_off),
                           (const uint16_t*)q, (const uint16_t*)k, (const uint16_t*)v,
                           (const uint16_t*)dout, (const float2*)rowstat, scale * 1.4426950408889634f,
                           scale, pq, diag_base, (uint16_t*)dk, (uint16_t*)dv, nlists, per_xcd,
                           st.K > 1 ? 1 : 0, own);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    {
        constexpr int RPW = kBwdThreads / (D / 4);
        dim3 grid((unsigned)((L.tokens + RPW - 1) / RPW), (unsigned)st.H);
        hipLaunchKernelGGL((dq_combine_kernel<D>), grid, dim3(kBwdThreads), 0, L.stream, st, L.tokens,
                           (const int32_t*)(wsp + ws.rev_off), pq, diag_base, scale, (uint16_t*)dq);
    }
    return hipGetLastError();
}

}  // namespace

uint32_t dbg_take_attn_bwd()
{
#ifdef MOBA_DEBUG_BOUNDS
    return dbg_take_local();
#else
    return 0u;
#endif
}

hipError_t launch_attn_bwd(const Launch& L, const WsLayout& ws, char* wsp, const void* q,
                           const void* k, const void* v, const void* o, const float* lse,
                           const void* dout, float scale, void* dq, void* dk, void* dv,
                           const uint8_t* own)
{
    if (L.dtype != MOBA_BF16) return hipErrorInvalidValue;
    const int B = L.st.B;
    if (L.D == 64 && B == 64) return bwd_t<64, 64>(L, ws, wsp, q, k, v, o, lse, dout, scale, dq, dk, dv, own);
    if (L.D == 64 && B == 128) return bwd_t<64, 128>(L, ws, wsp, q, k, v, o, lse, dout, scale, dq, dk, dv, own);
    if (L.D == 128 && B == 64) return bwd_t<128, 64>(L, ws, wsp, q, k, v, o, lse, dout, scale, dq, dk, dv, own);
    if (L.D == 128 && B == 128)
        return bwd_t<128, 128>(L, ws, wsp, q, k, v, o, lse, dout, scale, dq, dk, dv, own);
    return hipErrorInvalidValue;
}

hipError_t launch_own_flags(const Launch& L, const int32_t* idx, uint8_t* own)
{
    const int64_t rows = (int64_t)L.tokens * L.st.H;
    if (rows == 0) return hipSuccess;
    hipLaunchKernelGGL(own_flags_kernel, dim3((unsigned)((rows + kBwdThreads - 1) / kBwdThreads)),
                       dim3(kBwdThreads), 0, L.stream, L.st, rows, idx, own);
    return hipGetLastError();
}

}  // namespace moba
