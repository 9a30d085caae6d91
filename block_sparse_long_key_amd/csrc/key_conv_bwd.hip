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
constexpr int kVec = 4;          // channels per thread
constexpr int kMaxW = 8;

template <typename T> struct Row4;
template <> struct Row4<float> {
    static __device__ __forceinline__ void load(const float* p, float (&x)[4]) {
        const float4 v = *reinterpret_cast<const float4*>(p);
        x[0] = v.x; x[1] = v.y; x[2] = v.z; x[3] = v.w;
    }
    static __device__ __forceinline__ void store(float* p, const float (&x)[4]) {
        *reinterpret_cast<float4*>(p) = make_float4(x[0], x[1], x[2], x[3]);
    }
};
template <> struct Row4<uint16_t> {
    static __device__ __forceinline__ void load(const uint16_t* p, float (&x)[4]) {
        const uint2 v = *reinterpret_cast<const uint2*>(p);
        x[0] = bf16_lo(v.x); x[1] = bf16_hi(v.x);
        x[2] = bf16_lo(v.y); x[3] = bf16_hi(v.y);
    }
    static __device__ __forceinline__ void store(uint16_t* p, const float (&x)[4]) {
        uint2 v;
        v.x = pack_bf16x2(x[0], x[1]);
        v.y = pack_bf16x2(x[2], x[3]);
        *reinterpret_cast<uint2*>(p) = v;
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

template <typename T, int MODE>
__global__ __launch_bounds__(kThreads) void conv_bwd_kernel(
    SegTable st, int HD, const T* __restrict__ k, const float* __restrict__ w, int W,
    const T* __restrict__ gk, T* __restrict__ dk, float* __restrict__ dwp)
{
    const int gb = blockIdx.x;
    const int s = seq_of_block(st, gb);
    const int jb = gb - st.boff[s];
    const size_t t0 = (size_t)st.cu[s];
    const int L = seq_len(st, s);
    const int a = jb * st.B;
    const int b = min(a + st.B, L);
    const int ch = (blockIdx.y * kThreads + threadIdx.x) * kVec;
    if (ch >= HD) return;

    float wr[kVec][kMaxW];
#pragma unroll
    for (int v = 0; v < kVec; ++v)
#pragma unroll
        for (int l = 0; l < kMaxW; ++l) wr[v][l] = l < W ? w[(size_t)(ch + v) * W + l] : 0.f;

    // u_tau from direct loads (halo tokens only)
    auto conv_at = [&](int tau, float (&u)[kVec]) {
#pragma unroll
        for (int v = 0; v < kVec; ++v) u[v] = 0.f;
#pragma unroll
        for (int m = kMaxW - 1; m >= 0; --m) {
            if (m < W && tau - m >= 0) {
                float x[4];
                Row4<T>::load(k + (t0 + tau - m) * HD + ch, x);
#pragma unroll
                for (int v = 0; v < kVec; ++v) u[v] = __builtin_fmaf(wr[v][m], x[v], u[v]);
            }
        }
    };

    // ewin[v][l] = e_{t+l} once e_t is shifted in, so before the first
    // (last-in-sequence-order) token ewin[v][m] holds e_{b+m}: the halo,
    // zero past the sequence end
    float ewin[kVec][kMaxW];
#pragma unroll
    for (int v = 0; v < kVec; ++v)
#pragma unroll
        for (int l = 0; l < kMaxW; ++l) ewin[v][l] = 0.f;
#pragma unroll
    for (int l = 1; l < kMaxW; ++l) {
        const int tau = b - 1 + l;
        if (l < W && tau < L) {
            float gx[4];
            Row4<T>::load(gk + (t0 + tau) * HD + ch, gx);
            if constexpr (MODE == 1) {
                float u[kVec];
                conv_at(tau, u);
#pragma unroll
                for (int v = 0; v < kVec; ++v) gx[v] *= silu_grad(u[v]);
            }
#pragma unroll
            for (int v = 0; v < kVec; ++v) ewin[v][l - 1] = gx[v];
        }
    }
    // kwin[v][m] = k_{t-m} (zero before the sequence start)
    float kwin[kVec][kMaxW];
#pragma unroll
    for (int v = 0; v < kVec; ++v)
#pragma unroll
        for (int m = 0; m < kMaxW; ++m) kwin[v][m] = 0.f;
#pragma unroll
    for (int m = 0; m < kMaxW; ++m) {
        const int tau = b - 1 - m;
        if (m < W && tau >= 0) {
            float x[4];
            Row4<T>::load(k + (t0 + tau) * HD + ch, x);
#pragma unroll
            for (int v = 0; v < kVec; ++v) kwin[v][m] = x[v];
        }
    }

    float dwa[kVec][kMaxW];
#pragma unroll
    for (int v = 0; v < kVec; ++v)
#pragma unroll
        for (int l = 0; l < kMaxW; ++l) dwa[v][l] = 0.f;

#pragma unroll 4
    for (int t = b - 1; t >= a; --t) {
        const size_t row = (t0 + t) * HD + ch;
        float gx[4];
        Row4<T>::load(gk + row, gx);
        // the k row that enters the window for the next (earlier) token
        float knext[4] = {0.f, 0.f, 0.f, 0.f};
        if (t - W >= 0) Row4<T>::load(k + (t0 + t - W) * HD + ch, knext);
        float out[4];
#pragma unroll
        for (int v = 0; v < kVec; ++v) {
            float e = gx[v];
            if constexpr (MODE == 1) {
                float u = 0.f;
#pragma unroll
                for (int m = kMaxW - 1; m >= 0; --m)
                    if (m < W) u = __builtin_fmaf(wr[v][m], kwin[v][m], u);
                e *= silu_grad(u);
            }
#pragma unroll
            for (int l = kMaxW - 1; l >= 1; --l) ewin[v][l] = ewin[v][l - 1];
            ewin[v][0] = e;
            float acc = MODE == 1 ? gx[v] : 0.f;
#pragma unroll
            for (int l = 0; l < kMaxW; ++l)
                if (l < W) acc = __builtin_fmaf(wr[v][l], ewin[v][l], acc);
            out[v] = acc;
#pragma unroll
            for (int l = 0; l < kMaxW; ++l)
                if (l < W) dwa[v][l] = __builtin_fmaf(e, kwin[v][l], dwa[v][l]);
#pragma unroll
            for (int m = 0; m < kMaxW - 1; ++m) kwin[v][m] = kwin[v][m + 1];
            kwin[v][kMaxW - 1] = 0.f;
            // the entering row is k_{t-W}, at index W-1 after the shift
#pragma unroll
            for (int m = 0; m < kMaxW; ++m)
                if (m == W - 1) kwin[v][m] = knext[v];
        }
        Row4<T>::store(dk + row, out);
    }
    float* dst = dwp + ((size_t)gb * HD + ch) * W;
#pragma unroll
    for (int v = 0; v < kVec; ++v)
#pragma unroll
        for (int l = 0; l < kMaxW; ++l)
            if (l < W) dst[v * W + l] = dwa[v][l];
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

template <typename T, int MODE>
hipError_t conv_bwd_t(const Launch& L, const void* k, const float* w, int W, const void* gk,
                      void* dk, float* dw, float* dwp)
{
    const int HD = L.st.H * L.D;
    const int nblk = L.st.total_blocks;
    if (nblk > 0) {
        dim3 grid(nblk, (HD + kThreads * kVec - 1) / (kThreads * kVec));
        hipLaunchKernelGGL((conv_bwd_kernel<T, MODE>), grid, dim3(kThreads), 0, L.stream, L.st, HD,
                           (const T*)k, w, W, (const T*)gk, (T*)dk, dwp);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    const int n = HD * W;
    hipLaunchKernelGGL(conv_dw_reduce_kernel, dim3((n + 63) / 64), dim3(64 * kRedWaves), 0,
                       L.stream, nblk, n, dwp, dw);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_conv_bwd(const Launch& L, const void* k, const float* w, int W, int mode,
                           const void* gk, void* dk, float* dw, float* dwp)
{
    if (L.dtype == MOBA_BF16)
        return mode == 0 ? conv_bwd_t<uint16_t, 0>(L, k, w, W, gk, dk, dw, dwp)
                         : conv_bwd_t<uint16_t, 1>(L, k, w, W, gk, dk, dw, dwp);
    return mode == 0 ? conv_bwd_t<float, 0>(L, k, w, W, gk, dk, dw, dwp)
                     : conv_bwd_t<float, 1>(L, k, w, W, gk, dk, dw, dwp);
}

}  // namespace moba
