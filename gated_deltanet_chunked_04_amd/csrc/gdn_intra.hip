// gdn_intra.hip -- first fused forward kernel: gate cumsum + intra-chunk WY factors.
//
// The FlashQLA pages split the GDN chunked prefill into two fused kernels with a
// context-parallel preprocessing step between them (ollai.cn article, "technical
// principles", last item; "core advantages", first item) and round-trip the
// "intermediate variables" through HBM. This kernel is the first of the two. For one
// chunk of c <= 64 tokens of one head it computes
//   gam_r = sum_{j<=r} g_j                         (gate preprocessing: chunk-local cumsum)
//   A     = strict_lower(diag(beta) (exp(gam_r - gam_j) k_r . k_j))
//   T     = (I + A)^{-1}                          (unit lower triangular, always invertible)
//   w     = T diag(beta exp(gam)) K,    u = T diag(beta) V
// and per-chunk statistics for the CP decision: the chunk's gate total and the largest
// beta_r |k_r|^2. The algebra follows from the gated delta rule
// S_t = exp(g_t) S_{t-1} (I - beta_t k_t k_t^T) + beta_t v_t k_t^T: inside a chunk the
// per-token corrections delta_r = beta_r (v_r - S'_r k_r) solve (I + A) Delta = U - W S^T.
//
// Persistent workgroups of 4 waves, two per CU, each taking one (chunk, head) at a time.
// K is staged in LDS with its rows in fragment order (one 16-byte read per row fragment
// of the Gram tiles), V row-major; T*K and T*V read their columns with LDS transpose loads. The inverse is blocked:
// 16x16 diagonal blocks by forward substitution, then off-diagonal blocks in two levels
// with fp32 matrix-core products. T stays fp32; the products T*K and T*V run on
// the matrix cores in the input precision with fp32 accumulation. For the backward the
// kernel also writes T in the input precision.
#include "gdn_common.h"
#include "gdn_kernels.h"
#include "gdn_norm.h"

#include <algorithm>

namespace gdn {

namespace {

constexpr int kThreads = 256;

template <typename T> struct IntraPad;
// bf16 rows of K + 16 elements (288 bytes): the 16-byte row-fragment reads of K and the
// transposed reads of V meet no bank conflicts (at K + 8, two-way)
template <> struct IntraPad<bf16_t> { static constexpr int row = 16; };
template <> struct IntraPad<float> { static constexpr int row = 4; };


template <typename T, int K, int V>
struct IntraSmem {
    static constexpr int LDK = K + IntraPad<T>::row;   // K in fragment order (Gram rows), then the W output
    static constexpr int LDV = V + IntraPad<T>::row;   // row-major V (then the U output)
    static constexpr int off_k = 0;
    static constexpr int off_v = off_k + 64 * LDK * (int)sizeof(T);
    static constexpr int off_t = off_v + 64 * LDV * (int)sizeof(T);
    static constexpr int off_a = off_t + 64 * kLdA * 4;
    static constexpr int off_gam = off_a + 64 * kLdA * 4;
    static constexpr int off_beta = off_gam + 256;
    static constexpr int off_kk = off_beta + 256;
    static constexpr int off_eg = off_kk + 256;  // e^{gam_j}
    static constexpr int total = off_eg + 256;
};


// One task's inputs in registers (fetched while the previous task computes).
template <typename T, int K, int V>
struct IntraRegs {
    static constexpr int VEC = Elem<T>::kVec;
    static constexpr int NK = 64 * (K / VEC) / 256;
    static constexpr int NV = 64 * (V / VEC) / 256;
    u32x4 k[NK], v[NV];
    float g, beta;  // lanes 0..63 of wave 0
};

template <typename T, int K, int V>
__device__ __forceinline__ void intra_fetch(IntraRegs<T, K, V>& R, const IntraArgs& a, const ChunkTask& x) {
    const int64_t H = a.geo.H;
    fetch_tile<T, K>(R.k, reinterpret_cast<const T*>(a.k) + ((size_t)x.t0 * H + x.h) * K, (size_t)H * K, x.c);
    fetch_tile<T, V>(R.v, reinterpret_cast<const T*>(a.v) + ((size_t)x.t0 * H + x.h) * V, (size_t)H * V, x.c);
    const int tid = threadIdx.x;
    if (tid < 64) {
        const bool in = tid < x.c;
        const int64_t i = (x.t0 + (in ? tid : 0)) * H + x.h;
        R.g = in ? a.g[i] : 0.f;
        R.beta = in ? a.beta[i] : 0.f;
    }
}

// The q/k L2 normalisation of the fetched k rows, in registers: fetch_tile puts each row's
// K / VEC vectors in that many consecutive lanes of one wave, so a row's sum of squares
// takes log2 of that many cross-lane adds; x / sqrt(sum x^2 + eps), rounded to the input
// dtype (rows past the chunk end are zero and stay zero). The rows inside the chunk go to
// kn for the kernels that read k after this one.
template <typename T, int K, int N>
__device__ __forceinline__ void normalise_k(u32x4 (&x)[N], T* kn, size_t ld_g, int rows) {
    constexpr int VEC = Elem<T>::kVec;
    constexpr int NVR = K / VEC;
    constexpr int RPI = kThreads / NVR;
    static_assert(kThreads == 256 && 64 % NVR == 0, "the fetch_tile mapping of this kernel");
    const int r0 = (int)threadIdx.x / NVR, cv = (int)threadIdx.x % NVR;
    l2norm_rows<T, K>(x);
#pragma unroll
    for (int it = 0; it < N; ++it) {
        const int r = r0 + it * RPI;
        if (r < rows) *reinterpret_cast<u32x4*>(kn + (size_t)r * ld_g + cv * VEC) = x[it];
    }
}

// Persistent: each workgroup walks (chunk, head) tasks with a grid stride; the next
// task's k, v, g and beta load into registers while the current task computes. With kL2
// the k rows arrive raw and are normalised before staging (and written out once).
template <typename T, int K, int V, bool kL2>
__global__ __launch_bounds__(kThreads) void k_intra(IntraArgs args) {
    using S = IntraSmem<T, K, V>;
    extern __shared__ __attribute__((aligned(16))) unsigned char smem[];

    T* sK = reinterpret_cast<T*>(smem + S::off_k);
    T* sV = reinterpret_cast<T*>(smem + S::off_v);
    float* sT = reinterpret_cast<float*>(smem + S::off_t);
    float* sA = reinterpret_cast<float*>(smem + S::off_a);
    float* sGam = reinterpret_cast<float*>(smem + S::off_gam);
    float* sBeta = reinterpret_cast<float*>(smem + S::off_beta);
    float* sKK = reinterpret_cast<float*>(smem + S::off_kk);
    float* sEg = reinterpret_cast<float*>(smem + S::off_eg);

    const Geo& geo = args.geo;
    const int64_t H = geo.H;
    const int64_t ntasks = geo.total_chunks * H;
    const int tid = threadIdx.x;
    const int wave = wave_id();
    const int lane = tid & 63;
    const int ln = lane & 15, gq = lane >> 4;

    ChunkTask cur;
    int64_t t = next_chunk_task(geo, blockIdx.x, ntasks, cur);
    if (t >= ntasks) return;
    IntraRegs<T, K, V> R;
    intra_fetch(R, args, cur);
    // the strictly upper blocks of T stay zero for every task (read by the k32 slices of
    // stage 4 and written out with T): zeroed once, before the loop's first barrier
    tri_zero_upper64(sT);
    for (;;) {
        // ---- stage 1: operands into LDS, gate cumsum --------------------------------
        lds_sync();  // the previous task's LDS reads are done
        if constexpr (kL2)
            normalise_k<T, K>(R.k, reinterpret_cast<T*>(args.kn) + ((size_t)cur.t0 * H + cur.h) * K, (size_t)H * K,
                              cur.c);
        put_tile_fo<T, K>(sK, S::LDK, R.k);  // fragment order (read as rows and transposed)
        put_tile<T, V>(sV, S::LDV, R.v);
        const float g_in = R.g, b_in = R.beta;
        // the last task fetches itself again: the fetch stays unconditional
        ChunkTask nxt = cur;
        const int64_t tn = next_chunk_task(geo, t + gridDim.x, ntasks, nxt);
        const bool more = tn < ntasks;
        if (!more) nxt = cur;
        intra_fetch(R, args, nxt);
        const int64_t gc = cur.gc;
        const int h = cur.h;
        const int c = cur.c;
        const int64_t t0 = cur.t0;
        if (wave == 0) {
            const bool in = lane < c;
            const float x = wave_prefix_sum(g_in);
            sGam[lane] = x;   // rows past the chunk end carry the chunk total
            sBeta[lane] = b_in;
            sEg[lane] = fast_exp(x);
            if (in) args.gam[(t0 + lane) * H + h] = x;
        }
        lds_sync();

        // ---- stage 2: A = strict_lower(diag(beta) (D .* K K^T)) -----------------------
        // A K fragment serves as either operand (both use the same slot map), so each wave reads
        // the row blocks it needs once: waves 0 and 1 hold blocks 2w and 2w + 1 and form the three
        // tiles among them, waves 2 and 3 hold blocks 0, 1 and w and form tiles (w, 0) and (w, 1)
        // (40 fragment reads per task instead of two per tile product, 96)
        {
            constexpr int NTT = 3;
            f32x4 acc[NTT];
            int ti[NTT], tj[NTT];
            bool on[NTT];
#pragma unroll
            for (int m = 0; m < NTT; ++m) acc[m] = zero4();
            if (wave < 2) {
                const int b0 = 2 * wave, b1 = 2 * wave + 1;
                ti[0] = b0; tj[0] = b0;
                ti[1] = b1; tj[1] = b0;
                ti[2] = b1; tj[2] = b1;
                on[0] = on[1] = on[2] = true;
#pragma unroll
                for (int kb = 0; kb < K / 32; ++kb) {
                    Frag<T> f0, f1;
                    frag_row_fo(f0, sK, S::LDK, b0 * 16 + ln, kb * 32);
                    frag_row_fo(f1, sK, S::LDK, b1 * 16 + ln, kb * 32);
                    mma(acc[0], f0, f0);
                    mma(acc[1], f0, f1);
                    mma(acc[2], f1, f1);
                }
            } else {
                const int b2 = wave;
                ti[0] = b2; tj[0] = 0;
                ti[1] = b2; tj[1] = 1;
                ti[2] = b2; tj[2] = 1;
                on[0] = on[1] = true;
                on[2] = false;
#pragma unroll
                for (int kb = 0; kb < K / 32; ++kb) {
                    Frag<T> f0, f1, f2;
                    frag_row_fo(f0, sK, S::LDK, ln, kb * 32);
                    frag_row_fo(f1, sK, S::LDK, 16 + ln, kb * 32);
                    frag_row_fo(f2, sK, S::LDK, b2 * 16 + ln, kb * 32);
                    mma(acc[0], f0, f2);
                    mma(acc[1], f1, f2);
                }
            }
            // acc[m][i] = k_j . k_r with j = tj*16 + gq*4 + i, r = ti*16 + ln: four consecutive
            // columns of row r, one vector store
#pragma unroll
            for (int m = 0; m < NTT; ++m) {
                if (on[m]) {
                    const int r = ti[m] * 16 + ln;
                    const float gr = sGam[r], br = sBeta[r];
                    const f32x4 gj = *reinterpret_cast<const f32x4*>(sGam + tj[m] * 16 + gq * 4);
                    f32x4 val;
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int j = tj[m] * 16 + gq * 4 + i;
                        val[i] = (j < r) ? br * fast_exp(gr - gj[i]) * acc[m][i] : 0.f;
                        if (r == j) sKK[r] = br * acc[m][i];
                    }
                    *reinterpret_cast<f32x4*>(sA + r * kLdA + tj[m] * 16 + gq * 4) = val;
                }
            }
        }
        lds_sync();

        // ---- stage 3: T = (I + A)^{-1} --------------------------------------------------
        tri_inverse64(sA, sT);
        if (args.tmat) {
            // T for the backward, in the input precision: the 64 x 64 block is contiguous, so
            // consecutive threads store consecutive 16-byte vectors (whole lines)
            constexpr int VEC = Elem<T>::kVec;
            T* dst = reinterpret_cast<T*>(args.tmat) + ((size_t)gc * H + h) * 4096;
#pragma unroll
            for (int it = 0; it < 4096 / VEC / kThreads; ++it) {
                const int e = (tid + it * kThreads) * VEC;
                const float* src = sT + (e >> 6) * kLdA + (e & 63);
                if constexpr (sizeof(T) == 2) {
                    const f32x4 x0 = *reinterpret_cast<const f32x4*>(src);
                    const f32x4 x1 = *reinterpret_cast<const f32x4*>(src + 4);
                    *reinterpret_cast<u32x4*>(dst + e) = u32x4{pack_bf2(x0.x, x0.y), pack_bf2(x0.z, x0.w),
                                                               pack_bf2(x1.x, x1.y), pack_bf2(x1.z, x1.w)};
                } else {
                    *reinterpret_cast<f32x4*>(dst + e) = *reinterpret_cast<const f32x4*>(src);
                }
            }
        }
        if (wave == 1) {
            // chunk statistics for the CP decision
            const float m = wave_max(lane < c ? sKK[lane] : 0.f);
            if (lane == 0) args.cstat[gc * H + h] = make_float2(sGam[63], m);
        }

        // ---- stage 4: W = T diag(beta e^gam) K, U = T diag(beta) V ------------------------
        const int rt = wave;
        constexpr int NKB = 2;  // k32 slices over the 64 chunk rows
        Frag<T> aw[NKB], au[NKB];
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) {
            Frag<float> tf;
            frag_row(tf, sT, kLdA, rt * 16 + ln, kb * 32);
            float fw[8], fu[8];
            // slots 0..3: columns kb*32 + gq*4 + e; slots 4..7: 16 further
            const f32x4 b0 = *reinterpret_cast<const f32x4*>(sBeta + kb * 32 + gq * 4);
            const f32x4 b1 = *reinterpret_cast<const f32x4*>(sBeta + kb * 32 + 16 + gq * 4);
            const f32x4 g0 = *reinterpret_cast<const f32x4*>(sEg + kb * 32 + gq * 4);  // e^{gam_j}
            const f32x4 g1 = *reinterpret_cast<const f32x4*>(sEg + kb * 32 + 16 + gq * 4);
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float tv = e < 4 ? tf.lo[e] : tf.hi[e - 4];
                const float bj = e < 4 ? b0[e] : b1[e - 4];
                const float gjv = e < 4 ? g0[e] : g1[e - 4];
                fu[e] = tv * bj;
                fw[e] = fu[e] * gjv;
            }
            if constexpr (sizeof(T) == 2) {
                aw[kb].v = u32x4{pack_bf2(fw[0], fw[1]), pack_bf2(fw[2], fw[3]), pack_bf2(fw[4], fw[5]),
                                 pack_bf2(fw[6], fw[7])};
                au[kb].v = u32x4{pack_bf2(fu[0], fu[1]), pack_bf2(fu[2], fu[3]), pack_bf2(fu[4], fu[5]),
                                 pack_bf2(fu[6], fu[7])};
            } else {
                reinterpret_cast<Frag<float>&>(aw[kb]).lo = f32x4{fw[0], fw[1], fw[2], fw[3]};
                reinterpret_cast<Frag<float>&>(aw[kb]).hi = f32x4{fw[4], fw[5], fw[6], fw[7]};
                reinterpret_cast<Frag<float>&>(au[kb]).lo = f32x4{fu[0], fu[1], fu[2], fu[3]};
                reinterpret_cast<Frag<float>&>(au[kb]).hi = f32x4{fu[4], fu[5], fu[6], fu[7]};
            }
        }
        const int nkb = (rt >> 1) + 1;  // T[r][j] = 0 for j > r
        // Transposed tiles: with A = rows of K^T (V^T) and B = the scaled rows of T, accw[ct]
        // holds W^T[ct*16 + gq*4 + i][rt*16 + ln], i.e. four consecutive columns of row
        // rt*16 + ln, which each lane stages with one vector store.
        f32x4 accw[K / 16], accu[V / 16];
#pragma unroll
        for (int ct = 0; ct < K / 16; ++ct) {
            accw[ct] = zero4();
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb) {
                if (kb < nkb) {
                    Frag<T> b;
                    frag_col_fo(b, sK, S::LDK, ct * 16 + ln, kb * 32);  // K^T row ct*16+ln, slots j
                    mma(accw[ct], b, aw[kb]);
                }
            }
        }
#pragma unroll
        for (int ct = 0; ct < V / 16; ++ct) {
            accu[ct] = zero4();
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb) {
                if (kb < nkb) {
                    Frag<T> b;
                    frag_col(b, sV, S::LDV, ct * 16 + ln, kb * 32);  // V^T row ct*16+ln, slots j
                    mma(accu[ct], b, au[kb]);
                }
            }
        }
        lds_sync();
        // outputs staged over K and V, which are no longer read
        T* sWo = sK;
        T* sUo = sV;
        const int orow = rt * 16 + ln;
#pragma unroll
        for (int ct = 0; ct < K / 16; ++ct) store4(sWo + orow * S::LDK + ct * 16 + gq * 4, accw[ct]);
#pragma unroll
        for (int ct = 0; ct < V / 16; ++ct) store4(sUo + orow * S::LDV + ct * 16 + gq * 4, accu[ct]);
        lds_sync();
        store_rows<T, K>(reinterpret_cast<T*>(args.w), t0, H, h, c, sWo, S::LDK);
        store_rows<T, V>(reinterpret_cast<T*>(args.u), t0, H, h, c, sUo, S::LDV);
        if (!more) break;
        cur = nxt;
        t = tn;
    }
}

template <typename T, int K, int V>
hipError_t launch_intra_t(const IntraArgs& a, int cus, hipStream_t st) {
    using S = IntraSmem<T, K, V>;
    static_assert(S::total <= 160 * 1024, "LDS budget");
    auto kern = a.kn ? k_intra<T, K, V, true> : k_intra<T, K, V, false>;
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, S::total);
    if (e != hipSuccess) return e;
    // as many workgroups as fit on the chip at once (LDS-bound), at most one per task
    const int64_t per_cu = std::max(1, (160 * 1024) / S::total);
    const int64_t grid = std::min<int64_t>(a.geo.total_chunks * a.geo.H, per_cu * std::max(cus, 1));
    hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(kThreads), S::total, st, a);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_intra(const IntraArgs& a, int dtype, int cus, hipStream_t st) {
    if (a.geo.total_chunks == 0) return hipSuccess;
    const int K = a.geo.K, V = a.geo.V;
#define GDN_INTRA_CASE(TT, KK, VV) \
    if (K == KK && V == VV) return launch_intra_t<TT, KK, VV>(a, cus, st);
    if (dtype == 0) {
        GDN_INTRA_CASE(bf16_t, 64, 64)
        GDN_INTRA_CASE(bf16_t, 64, 128)
        GDN_INTRA_CASE(bf16_t, 128, 64)
        GDN_INTRA_CASE(bf16_t, 128, 128)
    } else {
        GDN_INTRA_CASE(float, 64, 64)
        GDN_INTRA_CASE(float, 64, 128)
        GDN_INTRA_CASE(float, 128, 64)
        GDN_INTRA_CASE(float, 128, 128)
    }
#undef GDN_INTRA_CASE
    return hipErrorInvalidValue;
}

}  // namespace gdn
