// gdn_norm.h -- the optional L2 normalisation of q and k rows ahead of the path, and its
// reverse mode (declarations; kernels in gdn_norm.hip).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gdn {

constexpr float kL2Eps = 1e-6f;  // added to the row's sum of squares

// Two row sets in one launch (q rows, then k rows; either count may be 0). Rows are the
// contiguous K-vectors of one token and head, [tokens x heads] of them per set.
//   forward : y = x / sqrt(sum x^2 + eps)                     (x, y distinct buffers)
//   backward: y <- r (y - xhat (xhat . y)), r = (sum x^2 + eps)^(-1/2), xhat = x r
//             (y holds the gradient with respect to the normalised rows on entry, with
//             respect to the raw rows x on exit)
struct NormArgs {
    const void* x0;
    const void* x1;
    void* y0;
    void* y1;
    int64_t rows0, rows1;
};

hipError_t launch_l2norm(const NormArgs& a, int dtype, int K, bool backward, hipStream_t st);

// The recurrent form (gdn_decode.hip) on raw q and k rows, normalised in the kernel.
struct DecodeArgs;
hipError_t launch_decode_qk_l2norm(const DecodeArgs& a, int dtype, int K, int V, hipStream_t st);

}  // namespace gdn
