// gdn_norm.h -- the optional L2 normalisation of q and k rows ahead of the path, and its
// reverse mode (declarations; kernels in gdn_norm.hip).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gdn_common.h"

namespace gdn {

constexpr float kL2Eps = 1e-6f;  // added to the row's sum of squares

// Sum of squares of one 16-byte vector's elements.
__device__ __forceinline__ float sumsq_vec(const u32x4& x, bf16_t) {
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const float lo = __uint_as_float(x[i] << 16), hi = __uint_as_float(x[i] & 0xFFFF0000u);
        s = fmaf(hi, hi, fmaf(lo, lo, s));
    }
    return s;
}
__device__ __forceinline__ float sumsq_vec(const u32x4& x, float) {
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) s = fmaf(__uint_as_float(x[i]), __uint_as_float(x[i]), s);
    return s;
}

// Rows of K values held as fetch_tile leaves them (each row's K / VEC vectors in that many
// consecutive lanes of one wave, whatever the thread count) scaled in registers to
// x / sqrt(sum x^2 + eps) and rounded to the element type; zero rows stay zero. Every lane
// of the wave takes part (cross-lane adds).
template <typename T, int K, int N>
__device__ __forceinline__ void l2norm_rows(u32x4 (&x)[N]) {
    constexpr int NVR = K / Elem<T>::kVec;
    static_assert(64 % NVR == 0, "a row inside one wave");
#pragma unroll
    for (int it = 0; it < N; ++it) {
        float ss = sumsq_vec(x[it], T{});
#pragma unroll
        for (int o = NVR / 2; o > 0; o >>= 1) ss += __shfl_xor(ss, o);
        x[it] = scale_vec<T>(x[it], 1.f / sqrtf(ss + kL2Eps));
    }
}

// Reverse mode of the normalisation for two row sets in one launch (q rows, then k rows).
// Rows are the contiguous K-vectors of one token and head, [tokens x heads] of them per set:
//   y <- r (y - xhat (xhat . y)), r = (sum x^2 + eps)^(-1/2), xhat = x r
// (y holds the gradient with respect to the normalised rows on entry, with respect to the
// raw rows x on exit). The forward normalisation happens where q and k are staged.
struct NormArgs {
    const void* x0;
    const void* x1;
    void* y0;
    void* y1;
    int64_t rows0, rows1;
};

hipError_t launch_l2norm_bwd(const NormArgs& a, int dtype, int K, hipStream_t st);

// The recurrent form (gdn_decode.hip) on raw q and k rows, normalised in the kernel.
struct DecodeArgs;
hipError_t launch_decode_qk_l2norm(const DecodeArgs& a, int dtype, int K, int V, hipStream_t st);

}  // namespace gdn
