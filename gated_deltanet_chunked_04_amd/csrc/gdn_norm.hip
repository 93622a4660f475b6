// gdn_norm.hip -- reverse mode of the L2 normalisation of the q and k rows over the key
// dimension, the preprocessing that may precede the path (the FlashQLA pages put
// preprocessing ahead of the fused kernels: edge.aivizor.me community post, its account of
// the chunked-prefill pipeline; their workloads feed unit-norm q and k). The forward,
// x / sqrt(sum x^2 + eps) with eps = 1e-6, happens inside the kernels that stage q and k
// (l2norm_rows); the backward maps dL/dxhat to dL/dx = r (dxhat - xhat (xhat . dxhat)) with
// r = (sum x^2 + eps)^(-1/2), here, after the per-chunk gradients.
//
// Pure streaming: a row is K contiguous values (256 bytes for bf16 at K = 128), held by
// K*esize/16 consecutive lanes with one 16-byte vector each, so a wave reads and writes
// whole contiguous runs and the row's sums take log2(lanes per row) cross-lane adds. Each
// thread keeps two rows' vectors in flight; fp32 arithmetic throughout, outputs rounded to
// nearest even when the input dtype is bf16.
#include "gdn_common.h"
#include "gdn_norm.h"

namespace gdn {

namespace {

constexpr int kNormThreads = 256;
constexpr int kNormUnroll = 2;  // row passes per loop iteration (loads issued before use)

template <typename T> struct Vec16;
template <> struct Vec16<bf16_t> {
    static constexpr int n = 8;
    static __device__ __forceinline__ void load(const bf16_t* p, float* x) {
        const u32x4 w = *reinterpret_cast<const u32x4*>(p);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            x[2 * j] = __uint_as_float(w[j] << 16);
            x[2 * j + 1] = __uint_as_float(w[j] & 0xffff0000u);
        }
    }
    static __device__ __forceinline__ void store(bf16_t* p, const float* x) {
        u32x4 w;
#pragma unroll
        for (int j = 0; j < 4; ++j) w[j] = pack_bf2(x[2 * j], x[2 * j + 1]);
        *reinterpret_cast<u32x4*>(p) = w;
    }
};
template <> struct Vec16<float> {
    static constexpr int n = 4;
    static __device__ __forceinline__ void load(const float* p, float* x) {
        const f32x4 w = *reinterpret_cast<const f32x4*>(p);
#pragma unroll
        for (int j = 0; j < 4; ++j) x[j] = w[j];
    }
    static __device__ __forceinline__ void store(float* p, const float* x) {
        *reinterpret_cast<f32x4*>(p) = f32x4{x[0], x[1], x[2], x[3]};
    }
};

// Sum over the LPR consecutive lanes that hold one row (LPR divides 64; every lane calls it).
template <int LPR>
__device__ __forceinline__ float row_sum(float s) {
#pragma unroll
    for (int o = LPR / 2; o > 0; o >>= 1) s += __shfl_xor(s, o);
    return s;
}

template <typename T, int K>
__global__ __launch_bounds__(kNormThreads) void k_l2norm_bwd(NormArgs a) {
    constexpr int E = Vec16<T>::n;     // values per 16-byte vector
    constexpr int LPR = K / E;         // lanes per row: 8, 16 or 32
    constexpr int RPB = kNormThreads / LPR;
    static_assert(K % E == 0 && 64 % LPR == 0, "row must tile a wave");
    const int lr = threadIdx.x / LPR, c0 = (threadIdx.x % LPR) * E;
    const int64_t total = a.rows0 + a.rows1;
    const int64_t stride = (int64_t)gridDim.x * RPB * kNormUnroll;
    for (int64_t base = (int64_t)blockIdx.x * RPB * kNormUnroll; base < total; base += stride) {
        float x[kNormUnroll][E], y[kNormUnroll][E];
        const T* src[kNormUnroll];
        T* dst[kNormUnroll];
        bool live[kNormUnroll];
#pragma unroll
        for (int u = 0; u < kNormUnroll; ++u) {
            const int64_t r = base + (int64_t)u * RPB + lr;
            live[u] = r < total;
            const bool first = r < a.rows0;
            const int64_t rr = first ? r : r - a.rows0;
            src[u] = reinterpret_cast<const T*>(first ? a.x0 : a.x1) + rr * K + c0;
            dst[u] = reinterpret_cast<T*>(first ? a.y0 : a.y1) + rr * K + c0;
#pragma unroll
            for (int e = 0; e < E; ++e) x[u][e] = y[u][e] = 0.f;
            if (live[u]) {
                Vec16<T>::load(src[u], x[u]);
                Vec16<T>::load(dst[u], y[u]);
            }
        }
#pragma unroll
        for (int u = 0; u < kNormUnroll; ++u) {
            float ss = 0.f;
#pragma unroll
            for (int e = 0; e < E; ++e) ss = fmaf(x[u][e], x[u][e], ss);
            const float r = 1.f / sqrtf(row_sum<LPR>(ss) + kL2Eps);
            float out[E];
            float dot = 0.f;
#pragma unroll
            for (int e = 0; e < E; ++e) dot = fmaf(x[u][e] * r, y[u][e], dot);
            dot = row_sum<LPR>(dot);
#pragma unroll
            for (int e = 0; e < E; ++e) out[e] = r * (y[u][e] - x[u][e] * r * dot);
            if (live[u]) Vec16<T>::store(dst[u], out);
        }
    }
}

template <typename T, int K>
hipError_t launch_t(const NormArgs& a, hipStream_t st) {
    constexpr int RPB = kNormThreads / (K / Vec16<T>::n);
    const int64_t total = a.rows0 + a.rows1;
    if (total <= 0) return hipSuccess;
    const int64_t need = (total + (int64_t)RPB * kNormUnroll - 1) / ((int64_t)RPB * kNormUnroll);
    const int grid = (int)(need < 8192 ? need : 8192);  // grid-stride beyond that
    hipLaunchKernelGGL((k_l2norm_bwd<T, K>), dim3(grid), dim3(kNormThreads), 0, st, a);
    return hipGetLastError();
}

}  // namespace

// dtype 0 = bf16, 1 = fp32 (gdn_dtype); K in {64, 128}
hipError_t launch_l2norm_bwd(const NormArgs& a, int dtype, int K, hipStream_t st) {
    if (dtype == 0) return K == 64 ? launch_t<bf16_t, 64>(a, st) : launch_t<bf16_t, 128>(a, st);
    return K == 64 ? launch_t<float, 64>(a, st) : launch_t<float, 128>(a, st);
}

}  // namespace gdn
