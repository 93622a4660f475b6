// gdn_decode.hip -- the recurrent form of the gated delta rule, token by token from a given
// state: the step after a prefill. The FlashQLA pages' interface takes an initial state so
// that a call continues where the previous one ended (ollai.cn article, "how to use"); a
// decoder continues from the state the chunked forward returned, a few tokens per call.
//   S <- exp(g_t) S (I - beta_t k_t k_t^T) + beta_t v_t k_t^T = a S + beta (v_t - a S k_t) k_t^T,
//   o_t = scale S q_t,   a = exp(g_t)
// One workgroup per (sequence, head) holds the V x K fp32 state in registers for all T tokens
// of the call: thread t owns row t / (K/64) and 64 consecutive columns of it, so the state is
// loaded and stored with contiguous 16-byte vectors and each row's dot products with k and q
// need one cross-lane add when K = 128. Per token the work is four fused multiply-adds per
// state element on the vector ALUs (matrix-vector products: nothing for the matrix cores); a
// call moves the state through HBM twice, so short calls are bound by that traffic and by the
// launch.
// With the q/k L2 normalisation (kL2) the rows k_t, q_t enter as k_t r_k, q_t r_q, r = (sum x^2 +
// eps)^(-1/2): each thread sums the squares over the 64 columns it reads anyway and the row's
// threads add their halves, so d = r_k (S k_t), the write uses u r_k k_t and o scales by r_q.
#include "gdn_common.h"
#include "gdn_kernels.h"
#include "gdn_norm.h"

namespace gdn {

namespace {

template <typename T, int K, int V, bool kL2>
__global__ __launch_bounds__(V * K / 64) void k_decode(DecodeArgs a) {
    constexpr int TPR = K / 64;  // threads per state row
    __shared__ __attribute__((aligned(16))) float sk[K];
    __shared__ __attribute__((aligned(16))) float sq[K];
    const int b = blockIdx.x, h = blockIdx.y;
    const int tid = threadIdx.x;
    const int row = tid / TPR, c0 = (tid % TPR) * 64;
    const int64_t H = a.H;
    const size_t VK = (size_t)V * K;
    const size_t soff = ((size_t)b * H + h) * VK + (size_t)row * K + c0;
    f32x4 s[16];
#pragma unroll
    for (int i = 0; i < 16; ++i)
        s[i] = a.s_in ? *reinterpret_cast<const f32x4*>(a.s_in + soff + 4 * i) : zero4();
    const T* q = reinterpret_cast<const T*>(a.q);
    const T* k = reinterpret_cast<const T*>(a.k);
    const T* v = reinterpret_cast<const T*>(a.v);
    T* o = reinterpret_cast<T*>(a.o);
    for (int64_t t = 0; t < a.T; ++t) {
        const size_t tok = ((size_t)b * a.T + t) * H + h;
        lds_sync();  // the previous token's reads of k and q are done (V >= 64, so NT >= K)
        if (tid < K) {
            sk[tid] = Elem<T>::to_f(k[tok * K + tid]);
            sq[tid] = Elem<T>::to_f(q[tok * K + tid]);
        }
        lds_sync();
        const float al = fast_exp(a.g[tok]);
        const float be = a.beta[tok];
        const float vi = Elem<T>::to_f(v[tok * V + row]);
        // d = (S k)_row over this thread's columns, then across the row's threads
        float d = 0.f, ssk = 0.f;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const f32x4 kk = *reinterpret_cast<const f32x4*>(sk + c0 + 4 * i);
            d += s[i][0] * kk[0] + s[i][1] * kk[1] + s[i][2] * kk[2] + s[i][3] * kk[3];
            if constexpr (kL2) ssk += kk[0] * kk[0] + kk[1] * kk[1] + kk[2] * kk[2] + kk[3] * kk[3];
        }
        if constexpr (TPR == 2) d += __shfl_xor(d, 1);
        float rk = 1.f;
        if constexpr (kL2) {
            if constexpr (TPR == 2) ssk += __shfl_xor(ssk, 1);
            rk = 1.f / sqrtf(ssk + kL2Eps);
            d *= rk;
        }
        const float u = be * (vi - al * d) * rk;  // the write adds u k_t^T, k_t = rk * (staged row)
        float od = 0.f, ssq = 0.f;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const f32x4 kk = *reinterpret_cast<const f32x4*>(sk + c0 + 4 * i);
            const f32x4 qq = *reinterpret_cast<const f32x4*>(sq + c0 + 4 * i);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                s[i][e] = al * s[i][e] + u * kk[e];
                od += s[i][e] * qq[e];
                if constexpr (kL2) ssq += qq[e] * qq[e];
            }
        }
        if constexpr (TPR == 2) od += __shfl_xor(od, 1);
        if constexpr (kL2) {
            if constexpr (TPR == 2) ssq += __shfl_xor(ssq, 1);
            od *= 1.f / sqrtf(ssq + kL2Eps);
        }
        if (tid % TPR == 0) o[tok * V + row] = Elem<T>::from_f(a.scale * od);
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) *reinterpret_cast<f32x4*>(a.s_out + soff + 4 * i) = s[i];
}

template <bool kL2>
hipError_t launch_decode_t(const DecodeArgs& a, int dtype, int K, int V, hipStream_t st) {
    if (a.B == 0 || a.H == 0) return hipSuccess;
    const dim3 grid((unsigned)a.B, (unsigned)a.H);
#define GDN_DECODE_CASE(TT, KK, VV)                                                           \
    if (K == KK && V == VV) {                                                                 \
        hipLaunchKernelGGL((k_decode<TT, KK, VV, kL2>), grid, dim3(VV * KK / 64), 0, st, a); \
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
