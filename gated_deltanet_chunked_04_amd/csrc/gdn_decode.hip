// gdn_decode.hip -- the recurrent form of the gated delta rule, token by token from a given
// state: the step after a prefill. The FlashQLA pages' interface takes an initial state so
// that a call continues where the previous one ended (ollai.cn article, "how to use"); a
// decoder continues from the state the chunked forward returned, a few tokens per call.
//   S <- exp(g_t) S (I - beta_t k_t k_t^T) + beta_t v_t k_t^T = a S + beta (v_t - a S k_t) k_t^T,
//   o_t = scale S q_t,   a = exp(g_t)
// One workgroup of 256 threads per (sequence, head) holds the V x K fp32 state in registers for
// all T tokens of the call. Each state row is spread over LPR = K/16 consecutive lanes (8 at
// K = 128), each holding four 4-column vectors of it, interleaved so that for every vector index
// the row's lanes cover one contiguous run of the row (a whole 128-byte line at K = 128): the
// state moves through HBM in fully used lines, and each row's dot products with k and q take
// log2(LPR) cross-lane adds, after which every lane of the row has the sums. Per token the work
// is four fused multiply-adds per state element on the vector ALUs (matrix-vector products:
// nothing for the matrix cores); a call moves the state through HBM twice, so short calls are
// bound by that traffic and by the launch.
// With the q/k L2 normalisation (kL2) the rows k_t, q_t enter as k_t r_k, q_t r_q, r = (sum x^2 +
// eps)^(-1/2): each thread sums the squares over the columns it reads anyway and the row's lanes
// add their parts, so d = r_k (S k_t), the write uses u r_k k_t and o scales by r_q.
#include "gdn_common.h"
#include "gdn_kernels.h"
#include "gdn_norm.h"

namespace gdn {

namespace {

constexpr int kDecThreads = 256;

__device__ __forceinline__ float dot4v(const f32x4& x, const f32x4& y) {
    return x[0] * y[0] + x[1] * y[1] + x[2] * y[2] + x[3] * y[3];
}

// Sum over the LPR consecutive lanes that share a state row (every lane gets the sum).
template <int LPR>
__device__ __forceinline__ float row_sum(float x) {
#pragma unroll
    for (int m = 1; m < LPR; m <<= 1) x += __shfl_xor(x, m);
    return x;
}

template <typename T, int K, int V, bool kL2>
__global__ __launch_bounds__(kDecThreads) void k_decode(DecodeArgs a) {
    constexpr int NCV = 4;               // 4-column vectors of a row per thread
    constexpr int LPR = K / (4 * NCV);   // lanes per state row
    constexpr int RPP = kDecThreads / LPR;  // rows per pass of the workgroup
    constexpr int NR = V / RPP;          // rows per thread
    static_assert(NR * RPP == V && LPR * 4 * NCV == K && LPR <= 64, "state split");
    __shared__ __attribute__((aligned(16))) float sk[K];
    __shared__ __attribute__((aligned(16))) float sq[K];
    const int b = blockIdx.x, h = blockIdx.y;
    const int tid = threadIdx.x;
    const int rl = tid / LPR, cl = tid % LPR;  // row within a pass, lane within the row
    const int64_t H = a.H;
    const size_t VK = (size_t)V * K;
    const size_t sbase = ((size_t)b * H + h) * VK;
    // vector i of row j: columns 4 (i LPR + cl) .. +3 of row rl + j RPP
    auto col = [&](int i) { return 4 * (i * LPR + cl); };
    f32x4 s[NR][NCV];
#pragma unroll
    for (int j = 0; j < NR; ++j)
#pragma unroll
        for (int i = 0; i < NCV; ++i)
            s[j][i] = a.s_in ? *reinterpret_cast<const f32x4*>(a.s_in + sbase + (size_t)(rl + j * RPP) * K + col(i))
                             : zero4();
    const T* q = reinterpret_cast<const T*>(a.q);
    const T* k = reinterpret_cast<const T*>(a.k);
    const T* v = reinterpret_cast<const T*>(a.v);
    T* o = reinterpret_cast<T*>(a.o);
    for (int64_t t = 0; t < a.T; ++t) {
        const size_t tok = ((size_t)b * a.T + t) * H + h;
        lds_sync();  // the previous token's reads of k and q are done
        if (tid < K) {
            sk[tid] = Elem<T>::to_f(k[tok * K + tid]);
            sq[tid] = Elem<T>::to_f(q[tok * K + tid]);
        }
        lds_sync();
        const float al = fast_exp(a.g[tok]);
        const float be = a.beta[tok];
        f32x4 kk[NCV], qq[NCV];
#pragma unroll
        for (int i = 0; i < NCV; ++i) {
            kk[i] = *reinterpret_cast<const f32x4*>(sk + col(i));
            qq[i] = *reinterpret_cast<const f32x4*>(sq + col(i));
        }
        float rk = 1.f, rq = 1.f;
        if constexpr (kL2) {
            float ssk = 0.f, ssq = 0.f;
#pragma unroll
            for (int i = 0; i < NCV; ++i) {
                ssk += dot4v(kk[i], kk[i]);
                ssq += dot4v(qq[i], qq[i]);
            }
            rk = 1.f / sqrtf(row_sum<LPR>(ssk) + kL2Eps);
            rq = 1.f / sqrtf(row_sum<LPR>(ssq) + kL2Eps);
        }
#pragma unroll
        for (int j = 0; j < NR; ++j) {
            const int row = rl + j * RPP;
            // d = (S k)_row, then the write u k^T (k = rk * staged row) and o = scale (S q)_row
            float d = 0.f;
#pragma unroll
            for (int i = 0; i < NCV; ++i) d += dot4v(s[j][i], kk[i]);
            d = row_sum<LPR>(d) * rk;
            const float u = be * (Elem<T>::to_f(v[tok * V + row]) - al * d) * rk;
            float od = 0.f;
#pragma unroll
            for (int i = 0; i < NCV; ++i) {
#pragma unroll
                for (int e = 0; e < 4; ++e) s[j][i][e] = al * s[j][i][e] + u * kk[i][e];
                od += dot4v(s[j][i], qq[i]);
            }
            od = row_sum<LPR>(od) * rq;
            if (cl == 0) o[tok * V + row] = Elem<T>::from_f(a.scale * od);
        }
    }
#pragma unroll
    for (int j = 0; j < NR; ++j)
#pragma unroll
        for (int i = 0; i < NCV; ++i)
            *reinterpret_cast<f32x4*>(a.s_out + sbase + (size_t)(rl + j * RPP) * K + col(i)) = s[j][i];
}

template <bool kL2>
hipError_t launch_decode_t(const DecodeArgs& a, int dtype, int K, int V, hipStream_t st) {
    if (a.B == 0 || a.H == 0) return hipSuccess;
    const dim3 grid((unsigned)a.B, (unsigned)a.H);
#define GDN_DECODE_CASE(TT, KK, VV)                                                           \
    if (K == KK && V == VV) {                                                                 \
        hipLaunchKernelGGL((k_decode<TT, KK, VV, kL2>), grid, dim3(kDecThreads), 0, st, a);  \
        return hipGetLastError();                                                             \
    }
    if (dtype == 0) {
        GDN_DECODE_CASE(bf16_t, 64, 64)
        GDN_DECODE_CASE(bf16_t, 64, 128)
        GDN_DECODE_CASE(bf16_t, 128, 64)
        GDN_DECODE_CASE(bf16_t, 128, 128)
    } else {
        GDN_DECODE_CASE(float, 64, 64)
        GDN_DECODE_CASE(float, 64, 128)
        GDN_DECODE_CASE(float, 128, 64)
        GDN_DECODE_CASE(float, 128, 128)
    }
#undef GDN_DECODE_CASE
    return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_decode(const DecodeArgs& a, int dtype, int K, int V, hipStream_t st) {
    return launch_decode_t<false>(a, dtype, K, V, st);
}

hipError_t launch_decode_qk_l2norm(const DecodeArgs& a, int dtype, int K, int V, hipStream_t st) {
    return launch_decode_t<true>(a, dtype, K, V, st);
}

}  // namespace gdn
