// gdn_recur.hip -- inter-chunk state recurrence (the second fused forward kernel) and
// the intra-card context-parallel (CP) preprocessing around it.
//
// Per chunk of c tokens entering with state S (V x K), with the WY factors w, u of the
// first kernel and gam the chunk-local gate cumsum (Gam its last value):
//   Delta = U - W S^T                       (the chunk's delta-rule corrections)
//   O     = scale (diag(e^gam) Q S^T + (L .* Q K^T) Delta),   L_rj = e^{gam_r-gam_j}, j <= r
//   S'    = e^Gam S + Delta^T diag(e^{Gam-gam}) K
// which is the gated delta rule S_t = exp(g_t) S_{t-1}(I - beta_t k_t k_t^T) + beta_t v_t k_t^T,
// o_t = scale S_t q_t, regrouped by chunk. The chunk map is affine in S:
// S' = S P + R with P = e^Gam I - W^T diag(e^{Gam-gam}) K and R = U^T diag(e^{Gam-gam}) K.
//
// CP (FlashQLA pages: ollai.cn article, "technical principles" items on AutoCP and the
// sliding-window warmup, and "core advantages"): long sequences are cut into
// sub-sequences ("segments") that run in parallel. Each segment needs its entering state:
//   * warmup: rerun the recurrence from a zero state over the W chunks before the
//     segment; exact within tolerance when the gates decay fast over that window;
//   * exact: per segment, run the recurrence from zero to get R~ and, on K extra
//     identity rows with U = 0, the product M of its chunk maps (the pages' "correction
//     M matrix"); then scan S_{s+1} = S_s M_s + R~_s across segments.
// A per sequence-head decision kernel picks between them from the chunk gate totals.
//
// Workgroup layout: 256 threads = 4 waves; a workgroup owns 64 value rows of one
// sequence-head segment, wave w owns 16 of them. The state is kept in registers as
// fp32 accumulator tiles of S^T (K/16 tiles per wave), which feed the matrix cores
// directly as B operands (see gdn_common.h); it is never written to LDS.
#include "gdn_common.h"
#include "gdn_kernels.h"

namespace gdn {

namespace {

constexpr int kThreads = 256;

template <typename T> struct RPad;
template <> struct RPad<bf16_t> { static constexpr int row = 8, tr = 8; };
template <> struct RPad<float> { static constexpr int row = 4, tr = 4; };

template <typename T, int K>
struct RecurSmem {
    static constexpr bool kTrans = sizeof(T) == 2;  // transposed K copy (bf16 only)
    static constexpr int LD = K + RPad<T>::row;
    static constexpr int LDT = 64 + RPad<T>::tr;
    static constexpr int LDU = 64 + RPad<T>::row;
    static constexpr int kMat = 64 * LD * (int)sizeof(T);
    static constexpr int off_q = 0;
    static constexpr int off_k = off_q + kMat;
    static constexpr int off_w = off_k + kMat;
    static constexpr int off_u = off_w + kMat;
    static constexpr int off_pm = off_u + 64 * LDU * (int)sizeof(T);
    static constexpr int off_kt = off_pm + 64 * LDU * (int)sizeof(T);
    static constexpr int off_gam = off_kt + (kTrans ? K * LDT * (int)sizeof(T) : 0);
    static constexpr int total = off_gam + 256;
};

// (row tile, column tile) of the 64x64 P matrix: the 10 lower tiles plus the two upper
// tiles (0,1) and (2,3) that fall inside the k32 slices read by P*Delta (written as zero).
__constant__ int8_t kTriR[12][2] = {{0, 0}, {1, 0}, {1, 1}, {2, 0}, {2, 1}, {2, 2},
                                    {3, 0}, {3, 1}, {3, 2}, {3, 3}, {0, 1}, {2, 3}};

// Stage columns [col0, col0+64) of rows of a [.., H, D] tensor (zero past `rows`).
template <typename T>
__device__ __forceinline__ void stage_cols64(const T* __restrict__ src, int64_t t0, int64_t H, int h,
                                             int D, int col0, int rows, T* dst, int ld) {
    constexpr int VEC = Elem<T>::kVec;
    constexpr int NV = 64 / VEC;
    constexpr int UNITS = 64 * NV;
    const int tid = threadIdx.x;
#pragma unroll
    for (int it = 0; it < UNITS / kThreads; ++it) {
        const int u = tid + it * kThreads;
        const int cv = u % NV, r = u / NV;
        u32x4 x = u32x4{0u, 0u, 0u, 0u};
        if (r < rows) x = *reinterpret_cast<const u32x4*>(src + ((t0 + r) * H + h) * D + col0 + cv * VEC);
        *reinterpret_cast<u32x4*>(dst + r * ld + cv * VEC) = x;
    }
}

template <typename T, int K>
struct ChunkCtx {
    T* sQ;
    T* sK;
    T* sW;
    T* sU;
    T* sPm;
    T* sKt;
    float* sGam;
};

// Load one chunk's operands. kOut needs Q; u columns for value rows [ucol0, ucol0+64)
// (ucol0 < 0: no U rows, zeros).
template <typename T, int K, bool kOut>
__device__ __forceinline__ void load_chunk(const RecurArgs& a, const ChunkCtx<T, K>& cx, int64_t t0, int c,
                                           int h, int ucol0) {
    using S = RecurSmem<T, K>;
    const int64_t H = a.geo.H;
    if (kOut) stage_rows<T, K, true, false>(reinterpret_cast<const T*>(a.q), t0, H, h, c, cx.sQ, S::LD, nullptr, 0);
    if constexpr (S::kTrans)
        stage_rows<T, K, true, true>(reinterpret_cast<const T*>(a.k), t0, H, h, c, cx.sK, S::LD, cx.sKt, S::LDT);
    else
        stage_rows<T, K, true, false>(reinterpret_cast<const T*>(a.k), t0, H, h, c, cx.sK, S::LD, nullptr, 0);
    stage_rows<T, K, true, false>(reinterpret_cast<const T*>(a.w), t0, H, h, c, cx.sW, S::LD, nullptr, 0);
    if (ucol0 >= 0) {
        stage_cols64<T>(reinterpret_cast<const T*>(a.u), t0, H, h, a.geo.V, ucol0, c, cx.sU, S::LDU);
    } else {
        for (int e = threadIdx.x; e < 64 * S::LDU; e += kThreads) cx.sU[e] = T(0);
    }
    const int tid = threadIdx.x;
    if (tid < 64) {
        // chunk-local gate cumsum; rows past the end carry the chunk total
        const int r = tid < c ? tid : c - 1;
        cx.sGam[tid] = a.gam[(t0 + r) * H + h];
    }
}

// One chunk of the recurrence for this wave's 16 value rows.
//   accS[kt] : S^T tiles (rows k = kt*16.., columns = the wave's value rows)
//   kOut     : also produce O rows into o (value columns vcol0 + wave*16 + ln)
template <typename T, int K, bool kOut>
__device__ __forceinline__ void chunk_step(const RecurArgs& a, const ChunkCtx<T, K>& cx, f32x4 (&accS)[K / 16],
                                           int64_t t0, int c, int h, int vcol0) {
    using S = RecurSmem<T, K>;
    const int tid = threadIdx.x;
    const int wave = tid >> 6, lane = tid & 63, ln = lane & 15, gq = lane >> 4;

    Frag<T> sf[K / 32], nsf[K / 32];
#pragma unroll
    for (int kb = 0; kb < K / 32; ++kb) {
        frag_acc(sf[kb], accS[2 * kb], accS[2 * kb + 1]);
        frag_acc(nsf[kb], accS[2 * kb], accS[2 * kb + 1], -1.f);
    }

    if (kOut) {
        // P^T tiles (j-tile, r-tile) of (L .* Q K^T), shared by all waves through LDS.
        for (int idx = wave; idx < 12; idx += 4) {
            const int rt = kTriR[idx][0], jt = kTriR[idx][1];
            f32x4 acc = zero4();
#pragma unroll
            for (int kb = 0; kb < (jt <= rt ? K / 32 : 0); ++kb) {
                Frag<T> fa, fb;
                frag_row(fa, cx.sK, S::LD, jt * 16 + ln, kb * 32);
                frag_row(fb, cx.sQ, S::LD, rt * 16 + ln, kb * 32);
                mma(acc, fa, fb);
            }
            // acc[i] = (Q K^T)[r = rt*16+ln][j = jt*16+gq*4+i]
            const int r = rt * 16 + ln;
            const float gr = cx.sGam[r];
            float v[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int j = jt * 16 + gq * 4 + i;
                v[i] = (j <= r) ? acc[i] * fast_exp(gr - cx.sGam[j]) : 0.f;
            }
            T* dst = cx.sPm + r * S::LDU + jt * 16 + gq * 4;
            if constexpr (sizeof(T) == 2) {
                *reinterpret_cast<u32x2*>(dst) = u32x2{pack_bf2(v[0], v[1]), pack_bf2(v[2], v[3])};
            } else {
                *reinterpret_cast<f32x4*>(dst) = f32x4{v[0], v[1], v[2], v[3]};
            }
        }
    }

    // Delta = U - W S^T   (rows j of the chunk, columns = the wave's value rows)
    f32x4 accD[4];
#pragma unroll
    for (int rt = 0; rt < 4; ++rt) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
            accD[rt][i] = Elem<T>::to_f(cx.sU[(rt * 16 + gq * 4 + i) * S::LDU + wave * 16 + ln]);
#pragma unroll
        for (int kb = 0; kb < K / 32; ++kb) {
            Frag<T> fa;
            frag_row(fa, cx.sW, S::LD, rt * 16 + ln, kb * 32);
            mma(accD[rt], fa, nsf[kb]);
        }
    }

    // O^T tiles: accO[rt][i] = O^T[v = wave*16 + gq*4 + i][r = rt*16 + ln]. The S^T
    // accumulators are an A fragment of S and the Delta accumulators an A fragment of
    // Delta^T, so O^T = S Q^T diag(e^gam) + Delta^T P^T needs no data movement, and each lane
    // ends up with four consecutive value columns of one token row (one vector store).
    if (kOut) {
        f32x4 accO[4];
#pragma unroll
        for (int rt = 0; rt < 4; ++rt) {
            accO[rt] = zero4();
#pragma unroll
            for (int kb = 0; kb < K / 32; ++kb) {
                Frag<T> fb;
                frag_row(fb, cx.sQ, S::LD, rt * 16 + ln, kb * 32);
                mma(accO[rt], sf[kb], fb);
            }
            accO[rt] *= fast_exp(cx.sGam[rt * 16 + ln]);
        }
        __syncthreads();  // P tiles complete
        Frag<T> df[2];
        frag_acc(df[0], accD[0], accD[1]);
        frag_acc(df[1], accD[2], accD[3]);
#pragma unroll
        for (int rt = 0; rt < 4; ++rt) {
#pragma unroll
            for (int kb = 0; kb <= (rt >> 1); ++kb) {
                Frag<T> fb;
                frag_row(fb, cx.sPm, S::LDU, rt * 16 + ln, kb * 32);
                mma(accO[rt], df[kb], fb);
            }
        }
        T* o = reinterpret_cast<T*>(a.o);
        const int64_t H = a.geo.H;
        const int V = a.geo.V;
#pragma unroll
        for (int rt = 0; rt < 4; ++rt) {
            const int r = rt * 16 + ln;
            if (r < c) store4(o + ((t0 + r) * H + h) * V + vcol0 + wave * 16 + gq * 4, accO[rt] * a.scale);
        }
    }

    // S^T <- e^Gam S^T + K^T diag(e^{Gam-gam}) Delta
    const float G = cx.sGam[63];
    const float eG = fast_exp(G);
    Frag<T> dtf[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
        f32x4 r0, r1;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            r0[i] = fast_exp(G - cx.sGam[kb * 32 + gq * 4 + i]);
            r1[i] = fast_exp(G - cx.sGam[kb * 32 + 16 + gq * 4 + i]);
        }
        frag_acc_rows(dtf[kb], accD[2 * kb], accD[2 * kb + 1], r0, r1);
    }
#pragma unroll
    for (int kt = 0; kt < K / 16; ++kt) {
        accS[kt] *= eG;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
            Frag<T> fa;
            if constexpr (S::kTrans)
                frag_row(fa, cx.sKt, S::LDT, kt * 16 + ln, kb * 32);
            else
                frag_col(fa, cx.sK, S::LD, kt * 16 + ln, kb * 32);
            mma(accS[kt], fa, dtf[kb]);
        }
    }
}

// accS <- rows [row0, row0+16) of a [rows][K] fp32 state (S^T tiles)
template <int K>
__device__ __forceinline__ void load_state(f32x4 (&accS)[K / 16], const float* src, int lrow) {
    const int gq = (threadIdx.x & 63) >> 4;
#pragma unroll
    for (int kt = 0; kt < K / 16; ++kt)
        accS[kt] = *reinterpret_cast<const f32x4*>(src + (size_t)lrow * K + kt * 16 + gq * 4);
}
template <int K>
__device__ __forceinline__ void store_state(const f32x4 (&accS)[K / 16], float* dst, int lrow) {
    const int gq = (threadIdx.x & 63) >> 4;
#pragma unroll
    for (int kt = 0; kt < K / 16; ++kt)
        *reinterpret_cast<f32x4*>(dst + (size_t)lrow * K + kt * 16 + gq * 4) = accS[kt];
}

template <typename T, int K, int MODE>
__global__ __launch_bounds__(kThreads) void k_recur(RecurArgs a) {
    using S = RecurSmem<T, K>;
    extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
    ChunkCtx<T, K> cx;
    cx.sQ = reinterpret_cast<T*>(smem + S::off_q);
    cx.sK = reinterpret_cast<T*>(smem + S::off_k);
    cx.sW = reinterpret_cast<T*>(smem + S::off_w);
    cx.sU = reinterpret_cast<T*>(smem + S::off_u);
    cx.sPm = reinterpret_cast<T*>(smem + S::off_pm);
    cx.sKt = reinterpret_cast<T*>(smem + S::off_kt);
    cx.sGam = reinterpret_cast<float*>(smem + S::off_gam);

    const Geo& geo = a.geo;
    const int64_t gs = blockIdx.x;
    const int h = blockIdx.y;
    const int vt = blockIdx.z;
    const int V = geo.V;
    const int64_t H = geo.H;
    SegLoc sg;
    if (!locate_seg(geo, gs, sg)) return;
    const int tid = threadIdx.x;
    const int wave = tid >> 6, lane = tid & 63, ln = lane & 15, gq = lane >> 4;
    const int row = vt * 64 + wave * 16 + ln;  // this lane's state row (value row, or V + M row)
    const size_t VK = (size_t)V * K;

    f32x4 accS[K / 16];
    int cbeg = sg.c0, cend = sg.c1;
    if (MODE == kRecurPrepass) {
        const int mode = a.modes[sg.n * H + h];
        if (mode == 1) {
            if (sg.s == 0 || vt * 64 >= V) return;
            cend = sg.c0;
            cbeg = max(0, sg.c0 - a.warmup);
            if (cbeg == 0 && a.s0)
                load_state<K>(accS, a.s0 + ((size_t)sg.n * H + h) * VK, row);
            else
#pragma unroll
                for (int kt = 0; kt < K / 16; ++kt) accS[kt] = zero4();
        } else if (mode == 2) {
            if (sg.s == sg.nseg - 1) return;
#pragma unroll
            for (int kt = 0; kt < K / 16; ++kt) {
                f32x4 z = zero4();
                if (row >= V) {
#pragma unroll
                    for (int i = 0; i < 4; ++i) z[i] = (kt * 16 + gq * 4 + i == row - V) ? 1.f : 0.f;
                }
                accS[kt] = z;
            }
        } else {
            return;
        }
    } else {
        if (sg.s > 0 && a.use_cp) {
            load_state<K>(accS, a.seginit + ((size_t)gs * H + h) * VK, row);
        } else if (a.s0) {
            load_state<K>(accS, a.s0 + ((size_t)sg.n * H + h) * VK, row);
        } else {
#pragma unroll
            for (int kt = 0; kt < K / 16; ++kt) accS[kt] = zero4();
        }
    }

    const int ucol0 = (vt * 64 < V) ? vt * 64 : -1;
    for (int ci = cbeg; ci < cend; ++ci) {
        const int64_t t0 = sg.bos + (int64_t)ci * 64;
        const int c = min(64, sg.len - ci * 64);
        if (MODE == kRecurStates) {
            // entry state of this chunk, in the input precision
            T* hs = reinterpret_cast<T*>(a.hstates) + ((size_t)(sg.choff + ci) * H + h) * VK + (size_t)row * K;
#pragma unroll
            for (int kt = 0; kt < K / 16; ++kt) {
                if constexpr (sizeof(T) == 2) {
                    *reinterpret_cast<u32x2*>(hs + kt * 16 + gq * 4) =
                        u32x2{pack_bf2(accS[kt][0], accS[kt][1]), pack_bf2(accS[kt][2], accS[kt][3])};
                } else {
                    *reinterpret_cast<f32x4*>(hs + kt * 16 + gq * 4) = accS[kt];
                }
            }
        }
        __syncthreads();
        load_chunk<T, K, MODE == kRecurOut>(a, cx, t0, c, h, ucol0);
        __syncthreads();
        chunk_step<T, K, MODE == kRecurOut>(a, cx, accS, t0, c, h, vt * 64);
    }

    if (MODE == kRecurPrepass) {
        const int mode = a.modes[sg.n * H + h];
        if (mode == 1) {
            store_state<K>(accS, a.seginit_out + ((size_t)gs * H + h) * VK, row);
        } else {
            float* P = a.prep + ((size_t)gs * H + h) * (size_t)(V + K) * K;
            if (row < V) {
                store_state<K>(accS, P, row);
            } else {
                // M^T[k][i] at P + V*K + k*K + i, i = row - V
                const int i = row - V;
#pragma unroll
                for (int kt = 0; kt < K / 16; ++kt)
#pragma unroll
                    for (int e = 0; e < 4; ++e) P[VK + (size_t)(kt * 16 + gq * 4 + e) * K + i] = accS[kt][e];
            }
        }
    } else if (sg.s == sg.nseg - 1 && a.sT) {
        store_state<K>(accS, a.sT + ((size_t)sg.n * H + h) * VK, row);
    }
}

template <typename T, int K, int MODE>
hipError_t launch_recur_t(const RecurArgs& a, int64_t nsegs_grid, int vtiles, hipStream_t st) {
    using S = RecurSmem<T, K>;
    static_assert(S::total <= 160 * 1024, "LDS budget");
    auto kern = k_recur<T, K, MODE>;
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, S::total);
    if (e != hipSuccess) return e;
    dim3 grid((unsigned)nsegs_grid, (unsigned)a.geo.H, (unsigned)vtiles);
    hipLaunchKernelGGL(kern, grid, dim3(kThreads), S::total, st, a);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// CP decision: one wave per sequence-head. Warmup is accepted when, for every segment
// boundary whose window does not reach the sequence start, the gate sum over the W
// chunks before it is <= log(eps) and beta |k|^2 <= 2 on those chunks (then every
// token map exp(g)(I - beta k k^T) has spectral norm <= exp(g), so a wrong state at
// the window start is damped by at least exp(window gate sum)).
__global__ __launch_bounds__(kThreads) void k_decide(DecideArgs a) {
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int64_t p = (int64_t)blockIdx.x * 4 + wave;
    const int H = a.geo.H;
    if (p >= (int64_t)a.geo.N * H) return;
    const int n = (int)(p / H), h = (int)(p % H);
    int32_t nseg, nchunks;
    int64_t segoff, choff;
    seq_segs(a.geo, n, nseg, segoff, nchunks, choff);
    int mode;
    if (nseg <= 1) {
        mode = 0;
    } else if (a.forced) {
        mode = a.forced;
    } else {
        bool ok = true;
        for (int s = 1 + lane; s < nseg; s += 64) {
            const int cb = s * a.geo.seg_len;
            const int w0 = cb - a.warmup;
            if (w0 <= 0) continue;  // window reaches the sequence start: exact
            float sum = 0.f, kk = 0.f;
            for (int m = w0; m < cb; ++m) {
                const float2 st = a.cstat[(choff + m) * H + h];
                sum += st.x;
                kk = fmaxf(kk, st.y);
            }
            ok = ok && (sum <= a.log_eps) && (kk <= 2.f);
        }
        mode = __all(ok) ? 1 : 2;
    }
    if (lane == 0) a.modes[p] = mode;
}

// ---------------------------------------------------------------------------
// Exact CP: S_{s+1} = S_s M_s + R~_s across segments, for sequence-heads in mode 2.
// Grid (N, H, V/64); the state rows live in S^T accumulators as in k_recur.
template <typename T>
__device__ __forceinline__ void frag_row_f32(Frag<T>& f, const float* base, int ld, int row, int k0);
template <>
__device__ __forceinline__ void frag_row_f32(Frag<bf16_t>& f, const float* base, int ld, int row, int k0) {
    const int gq = (threadIdx.x & 63) >> 4;
    const float* p = base + (size_t)row * ld + k0 + gq * 4;
    const f32x4 x = *reinterpret_cast<const f32x4*>(p);
    const f32x4 y = *reinterpret_cast<const f32x4*>(p + 16);
    f.v = u32x4{pack_bf2(x.x, x.y), pack_bf2(x.z, x.w), pack_bf2(y.x, y.y), pack_bf2(y.z, y.w)};
}
template <>
__device__ __forceinline__ void frag_row_f32(Frag<float>& f, const float* base, int ld, int row, int k0) {
    frag_row(f, base, ld, row, k0);
}

template <typename T, int K>
__global__ __launch_bounds__(kThreads) void k_scan(ScanArgs a) {
    const int n = blockIdx.x, h = blockIdx.y, vt = blockIdx.z;
    const int H = a.geo.H, V = a.geo.V;
    if (a.modes[(int64_t)n * H + h] != 2) return;
    int32_t nseg, nchunks;
    int64_t segoff, choff;
    seq_segs(a.geo, n, nseg, segoff, nchunks, choff);
    const int tid = threadIdx.x;
    const int wave = tid >> 6, lane = tid & 63, ln = lane & 15;
    const int row = vt * 64 + wave * 16 + ln;
    const size_t VK = (size_t)V * K;
    f32x4 accS[K / 16];
    if (a.s0)
        load_state<K>(accS, a.s0 + ((size_t)n * H + h) * VK, row);
    else
#pragma unroll
        for (int kt = 0; kt < K / 16; ++kt) accS[kt] = zero4();
    for (int s = 0; s + 1 < nseg; ++s) {
        const float* P = a.prep + ((size_t)(segoff + s) * H + h) * (size_t)(V + K) * K;
        Frag<T> sf[K / 32];
#pragma unroll
        for (int kb = 0; kb < K / 32; ++kb) frag_acc(sf[kb], accS[2 * kb], accS[2 * kb + 1]);
        f32x4 nx[K / 16];
        load_state<K>(nx, P, row);  // R~ rows
#pragma unroll
        for (int kt = 0; kt < K / 16; ++kt) {
#pragma unroll
            for (int kb = 0; kb < K / 32; ++kb) {
                Frag<T> fa;
                frag_row_f32(fa, P + VK, K, kt * 16 + ln, kb * 32);  // M^T rows
                mma(nx[kt], fa, sf[kb]);
            }
        }
#pragma unroll
        for (int kt = 0; kt < K / 16; ++kt) accS[kt] = nx[kt];
        store_state<K>(accS, a.seginit + ((size_t)(segoff + s + 1) * H + h) * VK, row);
    }
}

// ---------------------------------------------------------------------------
// Varlen tables from the device cu_seqlens (one workgroup). Lengths and offsets are
// clamped into [0, Ttot], so a bad cu_seqlens can never send a later kernel out of
// bounds; entries the host sized but the device data does not fill stay marked unused.
__global__ __launch_bounds__(kThreads) void k_tables(TableArgs a) {
    __shared__ int32_t s_ch[kThreads], s_sg[kThreads];
    __shared__ int32_t s_base[2];
    const int tid = threadIdx.x;
    for (int64_t i = tid; i < a.total_chunks; i += kThreads) a.chunk_tab[i] = make_int2(-1, 0);
    for (int64_t i = tid; i < a.total_segs; i += kThreads) a.seg_tab[i] = make_int4(-1, 0, 0, 0);
    if (tid == 0) {
        s_base[0] = 0;
        s_base[1] = 0;
    }
    __syncthreads();
    for (int base = 0; base < a.N; base += kThreads) {
        const int n = base + tid;
        int32_t nch = 0, nsg = 0;
        if (n < a.N) {
            int64_t b = a.cu[n], e = a.cu[n + 1];
            b = b < 0 ? 0 : (b > a.Ttot ? a.Ttot : b);
            e = e < b ? b : (e > a.Ttot ? a.Ttot : e);
            const int32_t len = (int32_t)(e - b);
            a.seq_bos[n] = b;
            a.seq_len[n] = len;
            nch = (len + 63) / 64;
            nsg = nch <= a.seg_len ? 1 : (nch + a.seg_len - 1) / a.seg_len;
        }
        s_ch[tid] = nch;
        s_sg[tid] = nsg;
        __syncthreads();
        // inclusive scan (Hillis-Steele) over the tile
        for (int off = 1; off < kThreads; off <<= 1) {
            const int32_t x = tid >= off ? s_ch[tid - off] : 0;
            const int32_t y = tid >= off ? s_sg[tid - off] : 0;
            __syncthreads();
            s_ch[tid] += x;
            s_sg[tid] += y;
            __syncthreads();
        }
        if (n < a.N) {
            a.seq_choff[n] = s_base[0] + s_ch[tid] - nch;
            a.seq_segoff[n] = s_base[1] + s_sg[tid] - nsg;
        }
        __syncthreads();
        if (tid == kThreads - 1) {
            s_base[0] += s_ch[tid];
            s_base[1] += s_sg[tid];
        }
        __syncthreads();
    }
    if (tid == 0) {
        a.seq_choff[a.N] = s_base[0];
        a.seq_segoff[a.N] = s_base[1];
    }
    __syncthreads();
    // fill: thread per sequence
    for (int n = tid; n < a.N; n += kThreads) {
        const int32_t len = a.seq_len[n];
        const int32_t nch = (len + 63) / 64;
        const int64_t co = a.seq_choff[n];
        for (int j = 0; j < nch; ++j)
            if (co + j < a.total_chunks) a.chunk_tab[co + j] = make_int2(n, j);
        const int64_t so = a.seq_segoff[n];
        const int32_t nsg = a.seq_segoff[n + 1] - a.seq_segoff[n];
        for (int s = 0; s < nsg; ++s) {
            const int c0 = s * a.seg_len;
            const int c1 = min(c0 + a.seg_len, nch);
            if (so + s < a.total_segs) a.seg_tab[so + s] = make_int4(n, s, nsg == 1 ? 0 : c0, nsg == 1 ? nch : c1);
        }
    }
}

}  // namespace

hipError_t launch_recur(const RecurArgs& a, int dtype, int mode, int64_t nsegs_grid, int vtiles,
                        hipStream_t st) {
    if (nsegs_grid == 0) return hipSuccess;
    const int K = a.geo.K;
#define GDN_RECUR_CASE(TT, KK)                                                                       \
    if (K == KK) {                                                                                   \
        if (mode == kRecurOut) return launch_recur_t<TT, KK, kRecurOut>(a, nsegs_grid, vtiles, st);   \
        if (mode == kRecurPrepass) return launch_recur_t<TT, KK, kRecurPrepass>(a, nsegs_grid, vtiles, st); \
        if (mode == kRecurStates) return launch_recur_t<TT, KK, kRecurStates>(a, nsegs_grid, vtiles, st); \
    }
    if (dtype == 0) {
        GDN_RECUR_CASE(bf16_t, 64)
        GDN_RECUR_CASE(bf16_t, 128)
    } else {
        GDN_RECUR_CASE(float, 64)
        GDN_RECUR_CASE(float, 128)
    }
#undef GDN_RECUR_CASE
    return hipErrorInvalidValue;
}

hipError_t launch_decide(const DecideArgs& a, hipStream_t st) {
    const int64_t p = (int64_t)a.geo.N * a.geo.H;
    if (p == 0) return hipSuccess;
    hipLaunchKernelGGL(k_decide, dim3((unsigned)((p + 3) / 4)), dim3(kThreads), 0, st, a);
    return hipGetLastError();
}

hipError_t launch_scan(const ScanArgs& a, int dtype, hipStream_t st) {
    dim3 grid((unsigned)a.geo.N, (unsigned)a.geo.H, (unsigned)(a.geo.V / 64));
    if (a.geo.N == 0) return hipSuccess;
    const int K = a.geo.K;
    if (dtype == 0) {
        if (K == 64) hipLaunchKernelGGL((k_scan<bf16_t, 64>), grid, dim3(kThreads), 0, st, a);
        else hipLaunchKernelGGL((k_scan<bf16_t, 128>), grid, dim3(kThreads), 0, st, a);
    } else {
        if (K == 64) hipLaunchKernelGGL((k_scan<float, 64>), grid, dim3(kThreads), 0, st, a);
        else hipLaunchKernelGGL((k_scan<float, 128>), grid, dim3(kThreads), 0, st, a);
    }
    return hipGetLastError();
}

hipError_t launch_tables(const TableArgs& a, hipStream_t st) {
    hipLaunchKernelGGL(k_tables, dim3(1), dim3(kThreads), 0, st, a);
    return hipGetLastError();
}

}  // namespace gdn
