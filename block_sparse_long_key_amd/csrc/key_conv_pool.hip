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

// N consecutive channels of one token row (N = 4: 8 / 16 bytes, N = 8: 16 /
// 32 bytes), unpacked to fp32
template <typename T, int N> struct VecIO;
template <int N> struct VecIO<float, N> {
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
template <> struct VecIO<uint16_t, 4> {
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
template <> struct VecIO<uint16_t, 8> {
    static __device__ __forceinline__ void load(const uint16_t* p, float (&x)[8]) {
        const uint4 v = *reinterpret_cast<const uint4*>(p);
        const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            x[2 * e] = __uint_as_float(w[e] << 16);
            x[2 * e + 1] = __uint_as_float(w[e] & 0xffff0000u);
        }
    }
    static __device__ __forceinline__ void store(uint16_t* p, const float (&x)[8]) {
        uint4 v;
        v.x = (uint32_t)f32_to_bf16(x[0]) | ((uint32_t)f32_to_bf16(x[1]) << 16);
        v.y = (uint32_t)f32_to_bf16(x[2]) | ((uint32_t)f32_to_bf16(x[3]) << 16);
        v.z = (uint32_t)f32_to_bf16(x[4]) | ((uint32_t)f32_to_bf16(x[5]) << 16);
        v.w = (uint32_t)f32_to_bf16(x[6]) | ((uint32_t)f32_to_bf16(x[7]) << 16);
        *reinterpret_cast<uint4*>(p) = v;
    }
};

// k + SiLU(acc) rounded to T, equal to the exact formula's result: the
// fp64 value v = k + acc / (1 + e^-acc), rounded to fp32 and then to T.
template <typename T>
__device__ __forceinline__ float silu_exact(float x, float acc)
{
    const double a = (double)acc;
    float f = (float)((double)x + a / (1.0 + exp(-a)));
    // the fp32 rounding stays a step of its own: folded into the dtype
    // conversion it would become one fp64 -> bf16 rounding, which differs
    // where the fp32 value is a bf16 tie
    asm volatile("" : "+v"(f));
    return IO<T>::round(f);
}

// The same for bf16 output from the hardware exp2 and reciprocal in fp32:
// |r - v| <= |silu| (|acc| + 8) 2^-23 + |r| 2^-24 (the exp2 argument's
// rounding costs |acc| 2^-23 relative, exp2, the reciprocal and the three
// roundings a few 2^-24 more) and fp32(v) is another |r| 2^-24 away.  When
// r is farther than twice that from the bf16 rounding midpoint next to it,
// every value in reach rounds to the same bf16: `safe`, and the result is
// exact; otherwise (about 1 element in 700) silu_exact decides.
__device__ __forceinline__ float silu_fast_bf16(float x, float acc, bool& safe)
{
    const float silu = acc * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-acc * 1.4426950408889634f));
    const float r = x + silu;
    const float rb = IO<uint16_t>::round(r);
    const uint32_t ex = __float_as_uint(r) & 0x7f800000u;
    // half a bf16 ulp in r's binade
    const float hu = __uint_as_float(ex - (8u << 23));
    const float delta = __builtin_fmaf(fabsf(silu), (fabsf(acc) + 8.0f) * 1.1920929e-07f,
                                       fabsf(r) * 5.9604645e-08f) + 1e-35f;
    safe = ex > (9u << 23) && hu - fabsf(r - rb) > 2.0f * delta;
    return rb;
}

// CONV: apply the key convolution (MODE 0 plain, 1 SiLU + residual) and
//       write k'.  POOL: write the block centroid of the (convolved) keys.
// WK: the filter width, a compile-time constant so that the sliding window
//     is WK registers per channel and each output is exactly WK fmas
//     (a run-time width would cost a select per possible tap: measured
//     VALU-bound at 63 % busy with W = 3).  1 when CONV is false.
// NV: channels per thread (4 or 8): a workgroup covers 256 * NV channels of
//     a token row, so rows of 2048 channels are read whole with 16-byte bf16
//     loads (plain conv C5-shaped 0.321 -> 0.234 ms; with 1024-channel rows
//     half the threads would idle, so 4 there).
template <typename T, bool CONV, bool POOL, int MODE, int WK, int NV>
__global__ __launch_bounds__(kThreads) void conv_pool_kernel(
    SegTable st, int HD, const T* __restrict__ k, const float* __restrict__ w,
    T* __restrict__ kout, float* __restrict__ cent)
{
    const int g = blockIdx.x;
    const int s = seq_of_block(st, g);
    const int jb = g - st.boff[s];
    const int t0 = st.cu[s];
    const int L = seq_len(st, s);
    const int a = jb * st.B;
    const int b = min(a + st.B, L);
    const int ch = (blockIdx.y * kThreads + threadIdx.x) * NV;
    if (ch >= HD) return;

    float wr[NV][WK];
    float win[NV][WK];           // win[v][l] = x_{t-l} after the shift
#pragma unroll
    for (int v = 0; v < NV; ++v)
#pragma unroll
        for (int l = 0; l < WK; ++l) {
            wr[v][l] = 0.f;
            win[v][l] = 0.f;
        }
    if constexpr (CONV) {
#pragma unroll
        for (int v = 0; v < NV; ++v)
#pragma unroll
            for (int l = 0; l < WK; ++l) wr[v][l] = w[(size_t)(ch + v) * WK + l];
        // before the first shift, win[m] holds x_{a-1-m}
#pragma unroll
        for (int m = 0; m < WK - 1; ++m) {
            if (a - 1 - m >= 0) {
                float x[NV];
                VecIO<T, NV>::load(k + (size_t)(t0 + a - 1 - m) * HD + ch, x);
#pragma unroll
                for (int v = 0; v < NV; ++v) win[v][m] = x[v];
            }
        }
    }

    // bf16 k + SiLU(conv): elements whose fast result is not proven are
    // queued (x, acc, fast result, position) and finished after the block
    // in fp64, so a wave runs the fp64 formula a few times per block instead
    // of at every token where one lane needs it; a full queue finishes an
    // element on the spot
    constexpr bool DEFER = CONV && MODE == 1 && sizeof(T) == 2;
    constexpr int kQ = 6;
    __shared__ float4 fq[DEFER ? kQ : 1][kThreads];
    int nq = 0;

    double sum[NV] = {};
    // (8 tokens in flight: plain conv / pooling 4-14 % faster than 4; the
    // SiLU mode is VALU-bound and keeps 4)
    constexpr int kUnroll = MODE == 1 ? 4 : 8;
#pragma unroll kUnroll
    for (int tl = a; tl < b; ++tl) {
        const size_t row = (size_t)(t0 + tl) * HD + ch;
        float x[NV];
        VecIO<T, NV>::load(k + row, x);
        float y[NV];
        if constexpr (CONV) {
#pragma unroll
            for (int v = 0; v < NV; ++v) {
#pragma unroll
                for (int l = WK - 1; l >= 1; --l) win[v][l] = win[v][l - 1];
                win[v][0] = x[v];
                // taps from the oldest token to the newest
                float acc = 0.0f;
#pragma unroll
                for (int l = WK - 1; l >= 0; --l) acc = __builtin_fmaf(wr[v][l], win[v][l], acc);
                if constexpr (DEFER) {
                    bool safe;
                    y[v] = silu_fast_bf16(x[v], acc, safe);
                    if (!safe) {
                        if (nq < kQ) {
                            fq[nq][threadIdx.x] = make_float4(x[v], acc, y[v],
                                                              __int_as_float(((tl - a) << 3) | v));
                            ++nq;
                        } else {
                            y[v] = silu_exact<T>(x[v], acc);
                        }
                    }
                } else if constexpr (MODE == 1) {
                    y[v] = silu_exact<T>(x[v], acc);
                } else {
                    y[v] = IO<T>::round(acc);
                }
            }
            VecIO<T, NV>::store(kout + row, y);
        } else {
#pragma unroll
            for (int v = 0; v < NV; ++v) y[v] = x[v];
        }
        if constexpr (POOL) {
#pragma unroll
            for (int v = 0; v < NV; ++v) sum[v] += (double)y[v];
        }
    }
    if constexpr (DEFER) {
        // finish the queued elements: the exact k' replaces the fast one in
        // k_out (this thread stored it) and in the block sum (an fp64 sum of
        // bf16 keys is exact, so the order of its terms does not matter)
        for (int e = 0; e < nq; ++e) {
            const float4 f = fq[e][threadIdx.x];
            const int pos = __float_as_int(f.w);
            const int tl = a + (pos >> 3), v = pos & 7;
            const float yx = silu_exact<T>(f.x, f.y);
            if (yx != f.z) {
                kout[(size_t)(t0 + tl) * HD + ch + v] = f32_to_bf16(yx);
                const double dlt = (double)yx - (double)f.z;
#pragma unroll
                for (int u = 0; u < NV; ++u)
                    if (u == v) sum[u] += dlt;
            }
        }
    }
    if constexpr (POOL) {
        const double cnt = (double)(b - a);
        float* dst = cent + (size_t)g * HD + ch;
        float r[NV];
#pragma unroll
        for (int v = 0; v < NV; ++v) r[v] = (float)(sum[v] / cnt);
        VecIO<float, NV>::store(dst, r);
    }
}

template <typename T, bool CONV, bool POOL, int MODE, int WK, int NV>
hipError_t launch_t(const Launch& L, const void* k, const float* w, void* kout, float* cent)
{
    const int HD = L.st.H * L.D;
    dim3 grid(L.st.total_blocks, (HD + kThreads * NV - 1) / (kThreads * NV));
    if (grid.x == 0) return hipSuccess;
    hipLaunchKernelGGL((conv_pool_kernel<T, CONV, POOL, MODE, WK, NV>), grid, dim3(kThreads), 0,
                       L.stream, L.st, HD, (const T*)k, w, (T*)kout, cent);
    return hipGetLastError();
}

// 8 channels per thread where a token row has 2048 channels or more (plain
// conv of up to 4 taps and pooling; the SiLU mode and wider filters, whose
// windows would take most of the registers, keep 4)
template <typename T, bool CONV, bool POOL, int MODE, int WK>
hipError_t launch_nv(const Launch& L, const void* k, const float* w, void* kout, float* cent)
{
    if constexpr (MODE == 0 && WK <= 4)
        if (L.st.H * L.D >= 2048) return launch_t<T, CONV, POOL, MODE, WK, 8>(L, k, w, kout, cent);
    return launch_t<T, CONV, POOL, MODE, WK, 4>(L, k, w, kout, cent);
}

template <typename T, bool POOL, int MODE>
hipError_t launch_w(const Launch& L, const void* k, const float* w, int W, void* kout, float* cent)
{
    switch (W) {
        case 1: return launch_nv<T, true, POOL, MODE, 1>(L, k, w, kout, cent);
        case 2: return launch_nv<T, true, POOL, MODE, 2>(L, k, w, kout, cent);
        case 3: return launch_nv<T, true, POOL, MODE, 3>(L, k, w, kout, cent);
        case 4: return launch_nv<T, true, POOL, MODE, 4>(L, k, w, kout, cent);
        case 5: return launch_nv<T, true, POOL, MODE, 5>(L, k, w, kout, cent);
        case 6: return launch_nv<T, true, POOL, MODE, 6>(L, k, w, kout, cent);
        case 7: return launch_nv<T, true, POOL, MODE, 7>(L, k, w, kout, cent);
        case 8: return launch_nv<T, true, POOL, MODE, 8>(L, k, w, kout, cent);
    }
    return hipErrorInvalidValue;
}

template <typename T>
hipError_t dispatch_t(const Launch& L, const void* k, const float* w, int W, int mode,
                      void* kout, float* cent)
{
    const bool conv = kout != nullptr;
    const bool pool = cent != nullptr;
    if (!conv) return launch_nv<T, false, true, 0, 1>(L, k, w, kout, cent);
    if (mode == 0)
        return pool ? launch_w<T, true, 0>(L, k, w, W, kout, cent)
                    : launch_w<T, false, 0>(L, k, w, W, kout, cent);
    return pool ? launch_w<T, true, 1>(L, k, w, W, kout, cent)
                : launch_w<T, false, 1>(L, k, w, W, kout, cent);
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
