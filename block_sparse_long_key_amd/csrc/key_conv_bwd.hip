// key_conv_bwd.hip -- gradients of the key convolution (gfx950).
//
// "Optimizing Mixture of Block Attention", summary page, section
// "Progettazione della Convoluzione delle Chiavi (Appendice B)", formal-form
// equation: k'_t = sum_l w_l * k_{t-l} per channel (causal, zero left pad
// per sequence), or the page's k'_t = k_t + SiLU(u_t) with u_t that sum.
// Given g = dL/dk':
//   e_t  = g_t                           (plain)
//        = g_t * s'(u_t)                 (SiLU form; s'(u) = sig(u)(1 + u(1 - sig(u))))
//   dk_t = [SiLU form: g_t] + sum_l w_l e_{t+l}     (t+l inside the sequence)
//   dw_l = sum_t e_t k_{t-l}                         (t-l inside the sequence)
//
// conv_bwd_kernel -- one workgroup per (key block, 1024 channels), 4
//   channels per thread, like the forward conv: at a fixed token the
//   threads cover one contiguous row of heads*d elements.  The block's
//   tokens are walked from the last to the first, so both sliding windows
//   (e of the W-1 later tokens for dk, k of the W-1 earlier tokens for u and
//   dw) advance by one row per token; the W-1 tokens after the block are a
//   halo computed up front.  dw is summed per block in fp32 and written as
//   one partial per (block, channel, tap).
// conv_dw_reduce_kernel -- dw = sum of the block partials in fp64, in a
//   fixed order (deterministic), rounded once to fp32.
#include "moba_internal.h"

namespace moba {
namespace {

constexpr int kThreads = 256;
// N consecutive channels of one token row, unpacked to fp32 (N = 4 or 8)
template <typename T, int N> struct RowN;
template <int N> struct RowN<float, N> {
    static __device__ __forceinline__ void load(const float* p, float (&x)[N]) {
#pragma unroll
        for (int c = 0; c < N / 4; ++c) {
            const float4 v = *reinterpret_cast<const float4*>(p + 4 * c);
            x[4 * c] = v.x; x[4 * c + 1] = v.y; x[4 * c + 2] = v.z; x[4 * c + 3] = v.w;
        }
    }
    static __device__ __forceinline__ void store(float* p, const float (&x)[N]) {
#pragma unroll
        for (int c = 0; c < N / 4; ++c)
            *reinterpret_cast<float4*>(p + 4 * c) = make_float4(x[4 * c], x[4 * c + 1], x[4 * c + 2], x[4 * c + 3]);
    }
};
template <int N> struct RowN<uint16_t, N> {
    static __device__ __forceinline__ void load(const uint16_t* p, float (&x)[N]) {
        if constexpr (N == 8) {
            const uint4 v = *reinterpret_cast<const uint4*>(p);
            const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
            for (int e = 0; e < 4; ++e) { x[2 * e] = bf16_lo(w[e]); x[2 * e + 1] = bf16_hi(w[e]); }
        } else {
            const uint2 v = *reinterpret_cast<const uint2*>(p);
            x[0] = bf16_lo(v.x); x[1] = bf16_hi(v.x);
            x[2] = bf16_lo(v.y); x[3] = bf16_hi(v.y);
        }
    }
    static __device__ __forceinline__ void store(uint16_t* p, const float (&x)[N]) {
        if constexpr (N == 8) {
            uint4 v;
            v.x = pack_bf16x2(x[0], x[1]);
            v.y = pack_bf16x2(x[2], x[3]);
            v.z = pack_bf16x2(x[4], x[5]);
            v.w = pack_bf16x2(x[6], x[7]);
            *reinterpret_cast<uint4*>(p) = v;
        } else {
            uint2 v;
            v.x = pack_bf16x2(x[0], x[1]);
            v.y = pack_bf16x2(x[2], x[3]);
            *reinterpret_cast<uint2*>(p) = v;
        }
    }
};

// s'(u) of SiLU(u) = u * sig(u); sig on the hardware exp2 and reciprocal
// (a few fp32 ulp; the accurate expf and IEEE quotient cost 11 % of this
// pass in the SiLU mode)
__device__ __forceinline__ float silu_grad(float u)
{
    const float sg = __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-u * 1.4426950408889634f));
    return sg * (1.0f + u * (1.0f - sg));
}

// WK: the filter width, a compile-time constant (windows of WK registers,
// exactly WK fmas per tap loop, no per-tap selects).  NV: channels per
// thread, 8 where a workgroup then reads whole 2048-channel rows.
template <typename T, int MODE, int WK, int NV>
__global__ __launch_bounds__(kThreads) void conv_bwd_kernel(
    SegTable st, int HD, const T* __restrict__ k, const float* __restrict__ w,
    const T* __restrict__ gk, T* __restrict__ dk, float* __restrict__ dwp)
{
    const int gb = blockIdx.x;
    const int s = seq_of_block(st, gb);
    const int jb = gb - st.boff[s];
    const size_t t0 = (size_t)st.cu[s];
    const int L = seq_len(st, s);
    const int a = jb * st.B;
    const int b = min(a + st.B, L);
    const int ch = (blockIdx.y * kThreads + threadIdx.x) * NV;
    if (ch >= HD) return;

    float wr[NV][WK];
#pragma unroll
    for (int v = 0; v < NV; ++v)
#pragma unroll
        for (int l = 0; l < WK; ++l) wr[v][l] = w[(size_t)(ch + v) * WK + l];

    // u_tau from direct loads (halo tokens only)
    auto conv_at = [&](int tau, float (&u)[NV]) {
#pragma unroll
        for (int v = 0; v < NV; ++v) u[v] = 0.f;
#pragma unroll
        for (int m = WK - 1; m >= 0; --m) {
            if (tau - m >= 0) {
                float x[NV];
                RowN<T, NV>::load(k + (t0 + tau - m) * HD + ch, x);
#pragma unroll
                for (int v = 0; v < NV; ++v) u[v] = __builtin_fmaf(wr[v][m], x[v], u[v]);
            }
        }
    };

    // ewin[v][l] = e_{t+l} once e_t is shifted in, so before the first
    // (last-in-sequence-order) token ewin[v][m] holds e_{b+m}: the halo,
    // zero past the sequence end
    float ewin[NV][WK];
#pragma unroll
    for (int v = 0; v < NV; ++v)
#pragma unroll
        for (int l = 0; l < WK; ++l) ewin[v][l] = 0.f;
#pragma unroll
    for (int l = 1; l < WK; ++l) {
        const int tau = b - 1 + l;
        if (tau < L) {
            float gx[NV];
            RowN<T, NV>::load(gk + (t0 + tau) * HD + ch, gx);
            if constexpr (MODE == 1) {
                float u[NV];
                conv_at(tau, u);
#pragma unroll
                for (int v = 0; v < NV; ++v) gx[v] *= silu_grad(u[v]);
            }
#pragma unroll
            for (int v = 0; v < NV; ++v) ewin[v][l - 1] = gx[v];
        }
    }
    // kwin[v][m] = k_{t-m} (zero before the sequence start)
    float kwin[NV][WK];
#pragma unroll
    for (int v = 0; v < NV; ++v)
#pragma unroll
        for (int m = 0; m < WK; ++m) kwin[v][m] = 0.f;
#pragma unroll
    for (int m = 0; m < WK; ++m) {
        const int tau = b - 1 - m;
        if (tau >= 0) {
            float x[NV];
            RowN<T, NV>::load(k + (t0 + tau) * HD + ch, x);
#pragma unroll
            for (int v = 0; v < NV; ++v) kwin[v][m] = x[v];
        }
    }

    float dwa[NV][WK];
#pragma unroll
    for (int v = 0; v < NV; ++v)
#pragma unroll
        for (int l = 0; l < WK; ++l) dwa[v][l] = 0.f;

#pragma unroll 4
    for (int t = b - 1; t >= a; --t) {
        const size_t row = (t0 + t) * HD + ch;
        float gx[NV];
        RowN<T, NV>::load(gk + row, gx);
        // the k row that enters the window for the next (earlier) token
        float knext[NV] = {};
        if (t - WK >= 0) RowN<T, NV>::load(k + (t0 + t - WK) * HD + ch, knext);
        float out[NV];
#pragma unroll
        for (int v = 0; v < NV; ++v) {
            float e = gx[v];
            if constexpr (MODE == 1) {
                float u = 0.f;
#pragma unroll
                for (int m = WK - 1; m >= 0; --m)
                    u = __builtin_fmaf(wr[v][m], kwin[v][m], u);
                e *= silu_grad(u);
            }
#pragma unroll
            for (int l = WK - 1; l >= 1; --l) ewin[v][l] = ewin[v][l - 1];
            ewin[v][0] = e;
            float acc = MODE == 1 ? gx[v] : 0.f;
#pragma unroll
            for (int l = 0; l < WK; ++l)
                acc = __builtin_fmaf(wr[v][l], ewin[v][l], acc);
            out[v] = acc;
#pragma unroll
            for (int l = 0; l < WK; ++l)
                dwa[v][l] = __builtin_fmaf(e, kwin[v][l], dwa[v][l]);
#pragma unroll
            for (int m = 0; m < WK - 1; ++m) kwin[v][m] = kwin[v][m + 1];
            // the entering row is k_{t-W}, at index W-1 after the shift
            kwin[v][WK - 1] = knext[v];
        }
        RowN<T, NV>::store(dk + row, out);
    }
    float* dst = dwp + ((size_t)gb * HD + ch) * WK;
#pragma unroll
    for (int v = 0; v < NV; ++v)
#pragma unroll
        for (int l = 0; l < WK; ++l) dst[v * WK + l] = dwa[v][l];
}

// 16 waves x 64 columns per workgroup: wave r sums the blocks g = r mod 16
// (fp64), then the 16 partial sums are added in wave order -- the same
// order on every run
constexpr int kRedWaves = 16;
__global__ __launch_bounds__(64 * kRedWaves) void conv_dw_reduce_kernel(int nblk, int n,
                                                                        const float* __restrict__ dwp,
                                                                        float* __restrict__ dw)
{
    __shared__ double part[kRedWaves][64];
    const int col = threadIdx.x & 63, r = threadIdx.x >> 6;
    const int i = blockIdx.x * 64 + col;
    double acc = 0.0;
    if (i < n) {
#pragma unroll 4
        for (int g = r; g < nblk; g += kRedWaves) acc += (double)dwp[(size_t)g * n + i];
    }
    part[r][col] = acc;
    __syncthreads();
    if (r == 0 && i < n) {
        double t = 0.0;
        for (int q = 0; q < kRedWaves; ++q) t += part[q][col];
        dw[i] = (float)t;
    }
}

template <typename T, int MODE, int WK, int NV>
hipError_t conv_bwd_n(const Launch& L, const void* k, const float* w, const void* gk, void* dk,
                      float* dwp)
{
    const int HD = L.st.H * L.D;
    const int nblk = L.st.total_blocks;
    if (nblk > 0) {
        dim3 grid(nblk, (HD + kThreads * NV - 1) / (kThreads * NV));
        hipLaunchKernelGGL((conv_bwd_kernel<T, MODE, WK, NV>), grid, dim3(kThreads), 0, L.stream, L.st,
                           HD, (const T*)k, w, (const T*)gk, (T*)dk, dwp);
    }
    return hipGetLastError();
}

// 8 channels per thread for plain convs of up to 4 taps on rows of 2048
// channels or more (wider windows would not fit the registers)
template <typename T, int MODE, int WK>
hipError_t conv_bwd_w(const Launch& L, const void* k, const float* w, const void* gk, void* dk,
                      float* dwp)
{
    if constexpr (MODE == 0 && WK <= 4)
        if (L.st.H * L.D >= 2048) return conv_bwd_n<T, MODE, WK, 8>(L, k, w, gk, dk, dwp);
    return conv_bwd_n<T, MODE, WK, 4>(L, k, w, gk, dk, dwp);
}

template <typename T, int MODE>
hipError_t conv_bwd_t(const Launch& L, const void* k, const float* w, int W, const void* gk,
                      void* dk, float* dwp)
{
    switch (W) {
        case 1: return conv_bwd_w<T, MODE, 1>(L, k, w, gk, dk, dwp);
        case 2: return conv_bwd_w<T, MODE, 2>(L, k, w, gk, dk, dwp);
        case 3: return conv_bwd_w<T, MODE, 3>(L, k, w, gk, dk, dwp);
        case 4: return conv_bwd_w<T, MODE, 4>(L, k, w, gk, dk, dwp);
        case 5: return conv_bwd_w<T, MODE, 5>(L, k, w, gk, dk, dwp);
        case 6: return conv_bwd_w<T, MODE, 6>(L, k, w, gk, dk, dwp);
        case 7: return conv_bwd_w<T, MODE, 7>(L, k, w, gk, dk, dwp);
        case 8: return conv_bwd_w<T, MODE, 8>(L, k, w, gk, dk, dwp);
    }
    return hipErrorInvalidValue;
}

}  // namespace

// dk and the per-block dw partials (at dwp + block * H*d*W) of one launch
hipError_t launch_conv_bwd(const Launch& L, const void* k, const float* w, int W, int mode,
                           const void* gk, void* dk, float* dwp)
{
    if (L.dtype == MOBA_BF16)
        return mode == 0 ? conv_bwd_t<uint16_t, 0>(L, k, w, W, gk, dk, dwp)
                         : conv_bwd_t<uint16_t, 1>(L, k, w, W, gk, dk, dwp);
    return mode == 0 ? conv_bwd_t<float, 0>(L, k, w, W, gk, dk, dwp)
                     : conv_bwd_t<float, 1>(L, k, w, W, gk, dk, dwp);
}

// dw = the sum over nblk blocks of the partials (n = H*d*W values each)
hipError_t launch_conv_dw_reduce(hipStream_t stream, int nblk, int n, const float* dwp, float* dw)
{
    hipLaunchKernelGGL(conv_dw_reduce_kernel, dim3((n + 63) / 64), dim3(64 * kRedWaves), 0, stream,
                       nblk, n, dwp, dw);
    return hipGetLastError();
}

}  // namespace moba
