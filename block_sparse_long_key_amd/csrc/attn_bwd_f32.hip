// attn_bwd_f32.hip -- attention backward for fp32 inputs (gfx950): the plain
// recompute path, written for exactness and clarity (the bf16 path in
// attn_bwd.hip is the fast one).
//
// "Optimizing Mixture of Block Attention", summary page, section "Backward
// Pass: Ricalcolo (Algoritmo 5)": scores and probabilities are recomputed
// from q, k and the forward's LSE.  For query t with key set U_t (the listed
// past blocks and its own block up to t) and P_tu = exp(scale q_t.k_u -
// lse_t), D_t = dO_t . O_t:
//   dv_u = sum_t P_tu dO_t,   dS_tu = P_tu (dO_t . v_u - D_t),
//   dq_t = scale sum_u dS_tu k_u,   dk_u = scale sum_t dS_tu q_t.
//
// bwd_prep_f32_kernel -- lse in log2 units and D_t per (token, head).
// bwd_dq_f32_kernel   -- one wave per (token, head); lanes hold channels;
//   the two dot products of each key are wave sums (butterfly: every lane
//   gets the same total), dq accumulates over the row's blocks in idx order
//   and, inside a block, in key order.
// bwd_kv_f32_kernel   -- one wave per (key token, head); sums over the
//   block's list in the list's (repeatable) order, then the own-block rows
//   t >= u in token order.
// Every sum is fp32 in a fixed order: the results are bitwise repeatable.
#include "moba_internal.h"

namespace moba {
namespace {

constexpr int kPrepThreads = 256;

__device__ __forceinline__ float wave_total(float x)
{
#pragma unroll
    for (int m = 1; m < 64; m <<= 1) x += __shfl_xor(x, m);
    return x;
}

// rowstat[r] = {lse_r * log2(e), dO_r . O_r}; D/4 lanes per row
template <int D>
__global__ __launch_bounds__(kPrepThreads) void bwd_prep_f32_kernel(int64_t rows, const float* __restrict__ o,
                                                                   const float* __restrict__ dout,
                                                                   const float* __restrict__ lse,
                                                                   float2* __restrict__ rowstat)
{
    constexpr int CPR = D / 4;
    const int64_t gid = (int64_t)blockIdx.x * kPrepThreads + threadIdx.x;
    const int64_t r = gid / CPR;
    const int c = (int)(gid % CPR);
    float acc = 0.f;
    if (r < rows) {
        const float4 a = *(const float4*)(o + r * D + 4 * c);
        const float4 b = *(const float4*)(dout + r * D + 4 * c);
        acc = __builtin_fmaf(a.x, b.x, acc);
        acc = __builtin_fmaf(a.y, b.y, acc);
        acc = __builtin_fmaf(a.z, b.z, acc);
        acc = __builtin_fmaf(a.w, b.w, acc);
    }
#pragma unroll
    for (int m = 1; m < CPR; m <<= 1) acc += __shfl_xor(acc, m);
    if (r < rows && c == 0) rowstat[r] = make_float2(lse[r] * 1.4426950408889634f, acc);
}

template <int D>
__global__ __launch_bounds__(64) void bwd_dq_f32_kernel(SegTable st, const int32_t* __restrict__ idx,
                                                       const float* __restrict__ q, const float* __restrict__ k,
                                                       const float* __restrict__ v,
                                                       const float* __restrict__ dout,
                                                       const float2* __restrict__ rowstat, float sl2,
                                                       float scale, float* __restrict__ dq,
                                                       const uint8_t* __restrict__ own)
{
    constexpr int CPL = D / 64;                  // channels per lane: c = 64 e + lane
    const int t = blockIdx.x, h = blockIdx.y;
    const int H = st.H, K = st.K, B = st.B;
    const int lane = threadIdx.x;
    const int s = seq_of_token(st, t);
    const int tl = t - st.cu[s];
    const int i = tl / B;                        // own block
    const size_t row = (size_t)t * H + h;
    float qv[CPL], dov[CPL], acc[CPL];
#pragma unroll
    for (int e = 0; e < CPL; ++e) {
        qv[e] = q[row * D + 64 * e + lane];
        dov[e] = dout[row * D + 64 * e + lane];
        acc[e] = 0.f;
    }
    const float2 rs = rowstat[row];
    const int32_t* sel = idx + row * K;
    // the listed past blocks in idx order (entries >= i or < 0 skipped, as the
    // forward does), then the own block up to t (unless own[row] == 0)
    const int pend = (own && !own[row]) ? K - 1 : K;
    for (int p = 0; p <= pend; ++p) {
        int j = i;
        if (p < K) {
            j = sel[p];
            if (j < 0 || j >= i) continue;
        }
        const int u0 = j * B, u1 = p < K ? u0 + B : tl + 1;
        for (int u = u0; u < u1; ++u) {
            const size_t kr = ((size_t)(st.cu[s] + u) * H + h) * D;
            float sp = 0.f, dp = 0.f;
#pragma unroll
            for (int e = 0; e < CPL; ++e) {
                sp = __builtin_fmaf(qv[e], k[kr + 64 * e + lane], sp);
                dp = __builtin_fmaf(dov[e], v[kr + 64 * e + lane], dp);
            }
            sp = wave_total(sp);
            dp = wave_total(dp);
            const float pr = __builtin_amdgcn_exp2f(__builtin_fmaf(sp, sl2, -rs.x));
            const float ds = pr * (dp - rs.y);
#pragma unroll
            for (int e = 0; e < CPL; ++e) acc[e] = __builtin_fmaf(ds, k[kr + 64 * e + lane], acc[e]);
        }
    }
#pragma unroll
    for (int e = 0; e < CPL; ++e) dq[row * D + 64 * e + lane] = acc[e] * scale;
}

template <int D>
__global__ __launch_bounds__(64) void bwd_kv_f32_kernel(SegTable st, const int2* __restrict__ lst,
                                                       const uint32_t* __restrict__ entries,
                                                       const float* __restrict__ q, const float* __restrict__ k,
                                                       const float* __restrict__ v,
                                                       const float* __restrict__ dout,
                                                       const float2* __restrict__ rowstat, float sl2,
                                                       float scale, float* __restrict__ dk, float* __restrict__ dv,
                                                       const uint8_t* __restrict__ own)
{
    constexpr int CPL = D / 64;
    const int u = blockIdx.x, h = blockIdx.y;    // key token u (global), head h
    const int H = st.H, K = st.K, B = st.B;
    const int lane = threadIdx.x;
    const int s = seq_of_token(st, u);
    const int L = seq_len(st, s);
    const int ul = u - st.cu[s];
    const int j = ul / B;
    const size_t krow = (size_t)u * H + h;
    float kv[CPL], vv[CPL], ak[CPL], av[CPL];
#pragma unroll
    for (int e = 0; e < CPL; ++e) {
        kv[e] = k[krow * D + 64 * e + lane];
        vv[e] = v[krow * D + 64 * e + lane];
        ak[e] = 0.f;
        av[e] = 0.f;
    }
    auto add_row = [&](int t) {                  // query token t (global)
        const size_t row = (size_t)t * H + h;
        float qv[CPL], dov[CPL];
        float sp = 0.f, dp = 0.f;
#pragma unroll
        for (int e = 0; e < CPL; ++e) {
            qv[e] = q[row * D + 64 * e + lane];
            dov[e] = dout[row * D + 64 * e + lane];
            sp = __builtin_fmaf(qv[e], kv[e], sp);
            dp = __builtin_fmaf(dov[e], vv[e], dp);
        }
        sp = wave_total(sp);
        dp = wave_total(dp);
        const float2 rs = rowstat[row];
        const float pr = __builtin_amdgcn_exp2f(__builtin_fmaf(sp, sl2, -rs.x));
        const float ds = pr * (dp - rs.y);
#pragma unroll
        for (int e = 0; e < CPL; ++e) {
            av[e] = __builtin_fmaf(pr, dov[e], av[e]);
            ak[e] = __builtin_fmaf(ds, qv[e], ak[e]);
        }
    };
    // the queries that routed to block j, in list order
    if (K > 1) {
        int2 le = lst[(int64_t)h * st.total_blocks + st.boff[s] + j];
        if (!MOBA_INBOUNDS(le.x >= 0 && le.y >= 0 && (int64_t)le.x + le.y <= (int64_t)L * K, kDbgBwdList))
            le = make_int2(0, 0);
        const uint32_t* ent = entries + st.ebase[s] + (int64_t)h * L * K + le.x;
        for (int e = 0; e < le.y; ++e) {
            const int t = (int)(ent[e] >> 5);
            if (MOBA_INBOUNDS(t >= st.cu[s] && t < st.cu[s] + L, kDbgKvEntry)) add_row(t);
        }
    }
    // the own-block queries t >= u (those that attend their own block)
    const int tend = min((j + 1) * B, L);
    for (int tl = ul; tl < tend; ++tl)
        if (!own || own[(size_t)(st.cu[s] + tl) * H + h]) add_row(st.cu[s] + tl);
#pragma unroll
    for (int e = 0; e < CPL; ++e) {
        dk[krow * D + 64 * e + lane] = ak[e] * scale;
        dv[krow * D + 64 * e + lane] = av[e];
    }
}

template <int D>
hipError_t bwd_f32_t(const Launch& L, const WsLayout& ws, char* wsp, const int32_t* idx, const float* q,
                     const float* k,
                     const float* v, const float* o, const float* lse, const float* dout, float scale,
                     float* dq, float* dk, float* dv, const uint8_t* own)
{
    const SegTable& st = L.st;
    const int64_t rows = (int64_t)L.tokens * st.H;
    float2* rowstat = (float2*)(wsp + ws.rs_off);
    const float sl2 = scale * 1.4426950408889634f;
    {
        const int64_t thr = rows * (D / 4);
        hipLaunchKernelGGL((bwd_prep_f32_kernel<D>), dim3((unsigned)((thr + kPrepThreads - 1) / kPrepThreads)),
                           dim3(kPrepThreads), 0, L.stream, rows, o, dout, lse, rowstat);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    const dim3 grid((unsigned)L.tokens, (unsigned)st.H);
    hipLaunchKernelGGL((bwd_dq_f32_kernel<D>), grid, dim3(64), 0, L.stream, st, idx, q, k, v, dout,
                       (const float2*)rowstat, sl2, scale, dq, own);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((bwd_kv_f32_kernel<D>), grid, dim3(64), 0, L.stream, st,
                       (const int2*)(wsp + ws.lst_off), (const uint32_t*)(wsp + ws.ent_off), q, k, v, dout,
                       (const float2*)rowstat, sl2, scale, dk, dv, own);
    return hipGetLastError();
}

}  // namespace

uint32_t dbg_take_attn_bwd_f32()
{
#ifdef MOBA_DEBUG_BOUNDS
    return dbg_take_local();
#else
    return 0u;
#endif
}

hipError_t launch_attn_bwd_f32(const Launch& L, const WsLayout& ws, char* wsp, const int32_t* idx,
                               const void* q, const void* k, const void* v, const void* o,
                               const float* lse, const void* dout, float scale, void* dq, void* dk,
                               void* dv, const uint8_t* own)
{
    if (L.D == 64)
        return bwd_f32_t<64>(L, ws, wsp, idx, (const float*)q, (const float*)k, (const float*)v, (const float*)o,
                             lse, (const float*)dout, scale, (float*)dq, (float*)dk, (float*)dv, own);
    if (L.D == 128)
        return bwd_f32_t<128>(L, ws, wsp, idx, (const float*)q, (const float*)k, (const float*)v, (const float*)o,
                              lse, (const float*)dout, scale, (float*)dq, (float*)dk, (float*)dv, own);
    return hipErrorInvalidValue;
}

}  // namespace moba
