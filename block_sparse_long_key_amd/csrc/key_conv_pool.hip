// key_conv_pool.hip -- key convolution and block mean pooling (gfx950).
//
// Key convolution: "Optimizing Mixture of Block Attention", summary page,
// section "Progettazione della Convoluzione delle Chiavi (Appendice B)",
// formal-form equation: a depthwise (one filter per channel), causal,
// left-padded conv1d over the sequence; the page's form is
// k'_t = k_t + SiLU(sum_l W_l * k_{t-l}); the plain form drops the residual
// and the activation.
// Block centroids: same pages, section "Architettura del Modello
// Statistico", router-score equation: kbar_j = mean of the keys of block j.
//
// One workgroup owns one key block (B tokens of one sequence) and 1024
// channels (heads x head_dim, 4 per thread).  At a fixed token the threads
// read/write one contiguous row of H*d elements, so every access is
// coalesced; the W-1 previous tokens live in registers (sliding window), so
// k is read once and k' written once; the pooled sum of the block is kept in
// fp64 registers and the centroid written at the end of the block.  HBM
// bound: 2 |K| bytes with the conv, |K| bytes for pooling alone.
#include "moba_internal.h"

namespace moba {
namespace {

constexpr int kThreads = 256;
constexpr int kVec = 4;          // channels per thread
constexpr int kMaxW = 8;

template <typename T> struct Vec4;
template <> struct Vec4<float> {
    static __device__ __forceinline__ void load(const float* p, float (&x)[4]) {
        float4 v = *reinterpret_cast<const float4*>(p);
        x[0] = v.x; x[1] = v.y; x[2] = v.z; x[3] = v.w;
    }
    static __device__ __forceinline__ void store(float* p, const float (&x)[4]) {
        *reinterpret_cast<float4*>(p) = make_float4(x[0], x[1], x[2], x[3]);
    }
};
template <> struct Vec4<uint16_t> {
    static __device__ __forceinline__ void load(const uint16_t* p, float (&x)[4]) {
        uint2 v = *reinterpret_cast<const uint2*>(p);
        x[0] = __uint_as_float(v.x << 16);
        x[1] = __uint_as_float(v.x & 0xffff0000u);
        x[2] = __uint_as_float(v.y << 16);
        x[3] = __uint_as_float(v.y & 0xffff0000u);
    }
    static __device__ __forceinline__ void store(uint16_t* p, const float (&x)[4]) {
        uint2 v;
        v.x = (uint32_t)f32_to_bf16(x[0]) | ((uint32_t)f32_to_bf16(x[1]) << 16);
        v.y = (uint32_t)f32_to_bf16(x[2]) | ((uint32_t)f32_to_bf16(x[3]) << 16);
        *reinterpret_cast<uint2*>(p) = v;
    }
};

// CONV: apply the key convolution (MODE 0 plain, 1 SiLU + residual) and
//       write k'.  POOL: write the block centroid of the (convolved) keys.
template <typename T, bool CONV, bool POOL, int MODE>
__global__ __launch_bounds__(kThreads) void conv_pool_kernel(
    SegTable st, int HD, const T* __restrict__ k, const float* __restrict__ w,
    int W, T* __restrict__ kout, float* __restrict__ cent)
{
    const int g = blockIdx.x;
    const int s = seq_of_block(st, g);
    const int jb = g - st.boff[s];
    const int t0 = st.cu[s];
    const int L = seq_len(st, s);
    const int a = jb * st.B;
    const int b = min(a + st.B, L);
    const int ch = (blockIdx.y * kThreads + threadIdx.x) * kVec;
    if (ch >= HD) return;

    float wr[kVec][kMaxW];
    float win[kVec][kMaxW];        // win[v][l] = x_{t-l} after the shift
#pragma unroll
    for (int v = 0; v < kVec; ++v)
#pragma unroll
        for (int l = 0; l < kMaxW; ++l) {
            wr[v][l] = 0.f;
            win[v][l] = 0.f;
        }
    if constexpr (CONV) {
#pragma unroll
        for (int v = 0; v < kVec; ++v)
#pragma unroll
            for (int l = 0; l < kMaxW; ++l)
                if (l < W) wr[v][l] = w[(size_t)(ch + v) * W + l];
        // before the first shift, win[m] holds x_{a-1-m}
#pragma unroll
        for (int m = 0; m < kMaxW - 1; ++m) {
            if (m < W - 1 && a - 1 - m >= 0) {
                float x[4];
                Vec4<T>::load(k + (size_t)(t0 + a - 1 - m) * HD + ch, x);
#pragma unroll
                for (int v = 0; v < kVec; ++v) win[v][m] = x[v];
            }
        }
    }

    double sum[kVec] = {0.0, 0.0, 0.0, 0.0};
    // (8 tokens in flight: plain conv / pooling 4-14 % faster than 4; the
    // SiLU mode is VALU-bound and keeps 4)
#pragma unroll (MODE == 1 ? 4 : 8)
    for (int tl = a; tl < b; ++tl) {
        const size_t row = (size_t)(t0 + tl) * HD + ch;
        float x[4];
        Vec4<T>::load(k + row, x);
        float y[4];
        if constexpr (CONV) {
#pragma unroll
            for (int v = 0; v < kVec; ++v) {
#pragma unroll
                for (int l = kMaxW - 1; l >= 1; --l) win[v][l] = win[v][l - 1];
                win[v][0] = x[v];
                float acc = 0.0f;
#pragma unroll
                for (int l = kMaxW - 1; l >= 0; --l)
                    if (l < W) acc = __builtin_fmaf(wr[v][l], win[v][l], acc);
                float r = acc;
                // SiLU(acc) = acc / (1 + e^-acc) on the hardware exp2 and
                // reciprocal (a few ulp in fp32; the accurate expf and
                // IEEE quotient made this mode VALU-bound, 1.5x slower).
                // Below acc = -87 the reciprocal's result is denormal and the
                // term (|.| < 1e-36) may come out as zero.
                if constexpr (MODE == 1)
                    r = x[v] + acc * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-acc * 1.4426950408889634f));
                y[v] = IO<T>::round(r);
            }
            Vec4<T>::store(kout + row, y);
        } else {
#pragma unroll
            for (int v = 0; v < kVec; ++v) y[v] = x[v];
        }
        if constexpr (POOL) {
#pragma unroll
            for (int v = 0; v < kVec; ++v) sum[v] += (double)y[v];
        }
    }
    if constexpr (POOL) {
        const double cnt = (double)(b - a);
        float* dst = cent + (size_t)g * HD + ch;
        float r[4];
#pragma unroll
        for (int v = 0; v < kVec; ++v) r[v] = (float)(sum[v] / cnt);
        *reinterpret_cast<float4*>(dst) = make_float4(r[0], r[1], r[2], r[3]);
    }
}

template <typename T, bool CONV, bool POOL, int MODE>
hipError_t launch_t(const Launch& L, const void* k, const float* w, int W, void* kout, float* cent)
{
    const int HD = L.st.H * L.D;
    dim3 grid(L.st.total_blocks, (HD + kThreads * kVec - 1) / (kThreads * kVec));
    if (grid.x == 0) return hipSuccess;
    hipLaunchKernelGGL((conv_pool_kernel<T, CONV, POOL, MODE>), grid, dim3(kThreads), 0,
                       L.stream, L.st, HD, (const T*)k, w, W, (T*)kout, cent);
    return hipGetLastError();
}

template <typename T>
hipError_t dispatch_t(const Launch& L, const void* k, const float* w, int W, int mode,
                      void* kout, float* cent)
{
    const bool conv = kout != nullptr;
    const bool pool = cent != nullptr;
    if (!conv) return launch_t<T, false, true, 0>(L, k, w, W, kout, cent);
    if (mode == 0)
        return pool ? launch_t<T, true, true, 0>(L, k, w, W, kout, cent)
                    : launch_t<T, true, false, 0>(L, k, w, W, kout, cent);
    return pool ? launch_t<T, true, true, 1>(L, k, w, W, kout, cent)
                : launch_t<T, true, false, 1>(L, k, w, W, kout, cent);
}

}  // namespace

// k_out == nullptr: pooling only (moba_centroids).  cent == nullptr: conv only.
hipError_t launch_conv_pool(const Launch& L, const void* k, const float* w, int W,
                            int mode, void* k_out, float* cent)
{
    if (L.dtype == MOBA_BF16) return dispatch_t<uint16_t>(L, k, w, W, mode, k_out, cent);
    return dispatch_t<float>(L, k, w, W, mode, k_out, cent);
}

}  // namespace moba
