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
// Layout: one workgroup = one query block (B threads, one query each) of one
// head; the centroids of the past blocks stream through LDS in tiles of 32
// and are read by all threads as broadcasts.
#include "moba_internal.h"

namespace moba {
namespace {

constexpr int kTile = 32;

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

// ascending sort of the first n entries (others must be INT_MAX)
template <int KMAX>
__device__ __forceinline__ void sort_asc(int (&x)[KMAX])
{
#pragma unroll
    for (int pass = 0; pass < KMAX; ++pass) {
#pragma unroll
        for (int p = (pass & 1); p + 1 < KMAX; p += 2) {
            int lo = min(x[p], x[p + 1]);
            int hi = max(x[p], x[p + 1]);
            x[p] = lo;
            x[p + 1] = hi;
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

hipError_t launch_route(const Launch& L, const void* q, const float* cent, int32_t* idx)
{
    if (L.st.total_blocks == 0) return hipSuccess;
    if (L.dtype == MOBA_BF16)
        return L.D == 64 ? launch_d<uint16_t, 64>(L, q, cent, idx)
                         : launch_d<uint16_t, 128>(L, q, cent, idx);
    return L.D == 64 ? launch_d<float, 64>(L, q, cent, idx)
                     : launch_d<float, 128>(L, q, cent, idx);
}

}  // namespace moba
