// Token-level top-2 pre-gate (AdaFuse digest, section 2-ga: a lightweight
// top-2 router at the first layer fixes each token's expert set, which every
// later layer reuses).
//
// One wave64 per token.  Lane j accumulates the E logits over the columns
// j, j+64, ... in binary64 (the products of fp32 or bf16 operands are exact in
// binary64), a fixed butterfly sums the 64 partials, and lane 0 takes the
// top two (ties -> lower index) and the renormalised pair of weights
// g0 = 1/(1+exp(l1-l0)), g1 = exp(l1-l0)/(1+exp(l1-l0)).
#include "gfx950.hpp"
#include "internal.hpp"

namespace dlm {
namespace {

template <typename T> __device__ __forceinline__ double ldv(const T* p, int64_t i);
template <> __device__ __forceinline__ double ldv<float>(const float* p, int64_t i) {
    return (double)p[i];
}
template <> __device__ __forceinline__ double ldv<uint16_t>(const uint16_t* p, int64_t i) {
    return (double)bf_to_f(p[i]);
}

constexpr int kTokPerBlock = 4;

template <typename T, int EMAX>
__global__ __launch_bounds__(kTokPerBlock* kWave) void pregate_kernel(
    const T* __restrict__ x, const T* __restrict__ Wr, int64_t n_tok, int64_t d, int E,
    int32_t* __restrict__ idx, float* __restrict__ g) {
    const int64_t t = (int64_t)blockIdx.x * kTokPerBlock + wave_id();
    if (t >= n_tok) return;
    const int lane = lane_id();
    double acc[EMAX];
#pragma unroll
    for (int e = 0; e < EMAX; ++e) acc[e] = 0.0;
    const T* xr = x + t * d;
    for (int64_t j = lane; j < d; j += kWave) {
        const double xv = ldv(xr, j);
        const T* w = Wr + j * E;
#pragma unroll
        for (int e = 0; e < EMAX; ++e)
            if (e < E) acc[e] = fma(xv, ldv(w, e), acc[e]);
    }
#pragma unroll
    for (int e = 0; e < EMAX; ++e)
        if (e < E) acc[e] = wave_sum(acc[e]);
    if (lane != 0) return;
    // Top two by strict '>' scans: equal logits keep the lower index.  A NaN
    // logit never compares greater, so the indices stay in range and distinct.
    int i0 = 0;
    double l0 = acc[0];
#pragma unroll
    for (int e = 1; e < EMAX; ++e)
        if (e < E && acc[e] > l0) { l0 = acc[e]; i0 = e; }
    int i1 = (i0 == 0) ? 1 : 0;
    double l1 = (i0 == 0) ? acc[1] : acc[0];
#pragma unroll
    for (int e = 0; e < EMAX; ++e)
        if (e < E && e != i0 && acc[e] > l1) { l1 = acc[e]; i1 = e; }
    const double q = exp(l1 - l0);  // <= 1
    idx[2 * t] = i0;
    idx[2 * t + 1] = i1;
    g[2 * t] = (float)(1.0 / (1.0 + q));
    g[2 * t + 1] = (float)(q / (1.0 + q));
}

template <typename T>
hipError_t launch_t(const void* x, const void* Wr, int64_t T_, int64_t d, int E, int32_t* idx,
                    float* g, hipStream_t s) {
    const dim3 grid((unsigned)((T_ + kTokPerBlock - 1) / kTokPerBlock));
    const dim3 block(kTokPerBlock * kWave);
    const T* xp = (const T*)x;
    const T* wp = (const T*)Wr;
    if (E <= 8)
        hipLaunchKernelGGL((pregate_kernel<T, 8>), grid, block, 0, s, xp, wp, T_, d, E, idx, g);
    else if (E <= 16)
        hipLaunchKernelGGL((pregate_kernel<T, 16>), grid, block, 0, s, xp, wp, T_, d, E, idx, g);
    else
        hipLaunchKernelGGL((pregate_kernel<T, 32>), grid, block, 0, s, xp, wp, T_, d, E, idx, g);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_pregate(const void* x, const void* Wr, int64_t T, int64_t d, int E, int dtype,
                          int32_t* idx, float* g, hipStream_t s) {
    if (dtype == 0) return launch_t<float>(x, Wr, T, d, E, idx, g, s);
    return launch_t<uint16_t>(x, Wr, T, d, E, idx, g, s);
}

}  // namespace dlm
