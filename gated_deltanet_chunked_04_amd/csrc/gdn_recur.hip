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
// Workgroup layout: a workgroup owns RT value rows of one sequence-head segment (128 rows,
// 8 waves, at V = K = 128; 64 rows, 4 waves, otherwise), wave w owns 16 of them. The state is kept in registers as
// fp32 accumulator tiles of S^T (K/16 tiles per wave), which feed the matrix cores
// directly as B operands (see gdn_common.h); it is never written to LDS.
#include "gdn_common.h"
#include "gdn_kernels.h"
#include "gdn_norm.h"

namespace gdn {

namespace {

constexpr int kThreads = 256;  // decision / table kernels

template <typename T> struct RPad;
template <> struct RPad<bf16_t> { static constexpr int row = 8; };
template <> struct RPad<float> { static constexpr int row = 4; };

// RT state rows per workgroup (one wave per 16 rows), chunk operands staged in LDS.
template <typename T, int K, int RT>
struct RCfg {
    static constexpr int NW = RT / 16;
    static constexpr int NT = NW * 64;
    static constexpr int VEC = Elem<T>::kVec;
    // row strides of K + 16 (bf16) elements: the transposed and the row-fragment reads of the
    // staged tiles then meet no bank conflicts (measured: the states pass 180 -> 155 us)
    static constexpr int LD = K + 2 * RPad<T>::row;
    static constexpr int LDU = RT + 2 * RPad<T>::row;
    static constexpr int LDP = 64 + RPad<T>::row;
    static constexpr int kMat = 64 * LD * (int)sizeof(T);
    // the prepass uses k, w, u and the gate cumsum only; the states pass also the q tile (Delta
    // is staged over it); the output passes also q and the P tiles. Each mode allocates only its
    // part, so that prepass workgroups share CUs.
    static constexpr int off_k = 0;
    static constexpr int off_w = off_k + kMat;
    static constexpr int off_u = off_w + kMat;
    static constexpr int off_gam = off_u + 64 * LDU * (int)sizeof(T);
    static constexpr int off_eg = off_gam + 256;  // e^{gam_r}, once per chunk
    static constexpr int off_er = off_eg + 256;   // e^{Gam - gam_r}
    static constexpr int end_prep = off_er + 256;
    static constexpr int off_q = end_prep;
    static constexpr int end_states = off_q + kMat;
    static constexpr int off_pm = end_states;
    static constexpr int total = off_pm + 64 * LDP * (int)sizeof(T);
    // the output passes stage each chunk's O rows here and store them as whole rows (after the
    // next chunk's first barrier, or after the loop for the last chunk)
    static constexpr int off_o = total;
    static constexpr int total_out = off_o + 64 * LDU * (int)sizeof(T);
    static constexpr bool stage_o = total_out <= 160 * 1024;  // (fp32 at K = 128: no room)
    // the passes that record chunk-entry states stage each one past their part ([RT][K],
    // row-major) and store the workgroup's RT contiguous state rows as one linear block
    static constexpr int LDH = K + RPad<T>::row;
    static constexpr int h_bytes = RT * LDH * (int)sizeof(T);
    static constexpr int base_of(bool out, bool rec) {
        return out ? (stage_o ? total_out : total) : (rec ? end_states : end_prep);
    }
    static constexpr int lds_of(bool out, bool rec) {
        return base_of(out, rec) + (rec && base_of(out, rec) + h_bytes <= 160 * 1024 ? h_bytes : 0);
    }
    static_assert(64 * LDU <= 64 * LD, "the q tile holds a [64][RT] Delta tile");
    // register prefetch: 16-byte vectors per thread
    static constexpr int NVK = K / VEC;                        // vectors per row of q/k/w
    static constexpr int NVU = RT / VEC;                       // vectors per row of the u tile
    static constexpr int IQ = 64 * NVK / NT;                   // q, w, k rows
    static constexpr int IU = 64 * NVU / NT;                   // u rows
    static_assert(IQ * NT == 64 * NVK && IU * NT == 64 * NVU, "tile split");
};


// One chunk's operands in registers (loaded ahead of use), fetched in three pieces at
// different points of the step so that the loads drain behind the work.
template <typename T, int K, int RT, bool kQ>
struct ChunkRegs {
    using C = RCfg<T, K, RT>;
    u32x4 q[kQ ? C::IQ : 1];
    u32x4 w[C::IQ];
    u32x4 k[C::IQ];
    u32x4 u[C::IU];
    float gam;
};

template <int kPart, typename T, int K, int RT, bool kQ>
__device__ __forceinline__ void chunk_fetch(ChunkRegs<T, K, RT, kQ>& R, const RecurArgs& a, int64_t t0, int c, int h,
                                            int ucol0) {
    using C = RCfg<T, K, RT>;
    const int64_t H = a.geo.H;
    const size_t ok = ((size_t)t0 * H + h) * K;
    if constexpr (kPart == 0) {
        if constexpr (kQ) fetch_tile<T, K, C::IQ, C::NT>(R.q, reinterpret_cast<const T*>(a.q) + ok, (size_t)H * K, c);
        fetch_tile<T, K, C::IQ, C::NT>(R.w, reinterpret_cast<const T*>(a.w) + ok, (size_t)H * K, c);
    } else if constexpr (kPart == 1) {
        fetch_tile<T, K, C::IQ, C::NT>(R.k, reinterpret_cast<const T*>(a.k) + ok, (size_t)H * K, c);
    } else {
        // the M rows of the exact prepass (ucol0 < 0) have no u columns
        fetch_tile<T, RT, C::IU, C::NT>(R.u, reinterpret_cast<const T*>(a.u) + ((size_t)t0 * H + h) * a.geo.V + max(ucol0, 0),
                                        (size_t)H * a.geo.V, ucol0 >= 0 ? c : 0);
        const int tid = threadIdx.x;
        if (tid < 64) {
            const int r = tid < c ? tid : c - 1;  // rows past the chunk end carry the chunk total
            R.gam = a.gam[(t0 + r) * H + h];
        }
    }
}

template <typename T, int K, int RT>
struct ChunkLds {
    T* sQ;
    T* sK;
    T* sW;
    T* sU;
    T* sPm;
    float* sGam;
    float* sEg = nullptr;  // e^{gam_r} and e^{Gam - gam_r} per chunk row, or null: computed where used
    float* sEr = nullptr;
    T* sO = nullptr;  // output staging [64][RT] (row-major), or null: O goes straight to memory
    T* sH = nullptr;  // chunk-entry state staging [RT][K] (row-major), or null
};

template <typename T, int K, int RT, bool kQ>
__device__ __forceinline__ void chunk_stage(const ChunkRegs<T, K, RT, kQ>& R, const ChunkLds<T, K, RT>& L) {
    using C = RCfg<T, K, RT>;
    // q and w rows in fragment order: every wave reads them as row fragments only (k stays
    // row-major: the prepass and the state pass read it only transposed, and for the output
    // pass's few P-tile rows fragment order did not pay for its split staging writes)
    if constexpr (kQ) put_tile_fo<T, K, C::IQ, C::NT>(L.sQ, C::LD, R.q);
    put_tile_fo<T, K, C::IQ, C::NT>(L.sW, C::LD, R.w);
    put_tile<T, K, C::IQ, C::NT>(L.sK, C::LD, R.k);
    put_tile<T, RT, C::IU, C::NT>(L.sU, C::LDU, R.u);
    if (threadIdx.x < 64) {
        L.sGam[threadIdx.x] = R.gam;
        if (L.sEg) {
            // the chunk total is the last row's cumsum (rows past the chunk end repeat it)
            const float gtot = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(R.gam), 63));
            L.sEg[threadIdx.x] = fast_exp(R.gam);
            L.sEr[threadIdx.x] = fast_exp(gtot - R.gam);
        }
    }
}

// One chunk of the recurrence for this wave's 16 state rows (columns of S^T).
//   accS[kt]: S^T tiles (k rows kt*16.., the wave's 16 state rows)
//   kOut    : also produce O for value columns vcol0 + wave*16 ..
// Part 1 writes this wave's share of the P tiles; the caller's barrier separates it
// from part 2.
// kKfo: the K tile is stored in fragment order (the fused forward's layout) instead of row-major.
template <typename T, int K, int RT, bool kOut, bool kKfo = false>
__device__ __forceinline__ void chunk_part1(const ChunkLds<T, K, RT>& L, const f32x4 (&accS)[K / 16],
                                            Frag<T> (&sf)[K / 32], f32x4 (&accD)[4], f32x4 (&accO)[4]) {
    using C = RCfg<T, K, RT>;
    const int tid = threadIdx.x;
    const int wave = wave_id(), lane = tid & 63, ln = lane & 15, gq = lane >> 4;
    Frag<T> nsf[K / 32];
#pragma unroll
    for (int kb = 0; kb < K / 32; ++kb) {
        frag_acc(sf[kb], accS[2 * kb], accS[2 * kb + 1]);
        frag_acc(nsf[kb], accS[2 * kb], accS[2 * kb + 1], -1.f);
    }
    // bf16 with 128 state rows: one pass over the k32 slices serves the P tiles and O with the
    // same Q fragments; elsewhere (more registers per fragment, or fewer waves) the P tiles
    // take a pass of their own.
    if constexpr (sizeof(T) == 2 && RT == 128) {
        // This wave's P tiles (rows r of Q, columns j of K; at most NPT of them), Delta = U - W S^T
        // (rows j of the chunk, columns = the wave's state rows) and the O^T tiles
        // accO[rt][i] = O^T[v = wave*16 + gq*4 + i][r = rt*16 + ln] in one pass over the k32
        // slices, so each slice's Q fragments serve both the P tiles and O. The S^T accumulators
        // are an A fragment of S and the Delta accumulators an A fragment of Delta^T, so
        // O^T = S Q^T diag(e^gam) + Delta^T P^T needs no data movement, and each lane ends up
        // with four consecutive value columns of one token row.
        constexpr int NPT = (12 + C::NW - 1) / C::NW;
        f32x4 pacc[NPT];
        int prt[NPT], pjt[NPT];
        bool pon[NPT], pmm[NPT];
#pragma unroll
        for (int m = 0; m < NPT; ++m) {
            const int idx = wave + m * C::NW;
            pon[m] = kOut && idx < 12;
            prt[m] = pon[m] ? tri_row(idx) : 0;
            pjt[m] = pon[m] ? tri_col(idx) : 0;
            pmm[m] = pon[m] && pjt[m] <= prt[m];
            pacc[m] = zero4();
        }
#pragma unroll
        for (int rt = 0; rt < 4; ++rt) {
            accD[rt] = col4(L.sU, C::LDU, wave * 16 + ln, rt * 16);
            if (kOut) accO[rt] = zero4();
        }
#pragma unroll
        for (int kb = 0; kb < K / 32; ++kb) {
            Frag<T> fw[4], fq[4], fa[NPT];
#pragma unroll
            for (int rt = 0; rt < 4; ++rt) {
                frag_row_fo(fw[rt], L.sW, C::LD, rt * 16 + ln, kb * 32);
                if (kOut) frag_row_fo(fq[rt], L.sQ, C::LD, rt * 16 + ln, kb * 32);
            }
#pragma unroll
            for (int m = 0; m < NPT; ++m)
                if (pmm[m]) {
                    if constexpr (kKfo) frag_row_fo(fa[m], L.sK, C::LD, pjt[m] * 16 + ln, kb * 32);
                    else frag_row(fa[m], L.sK, C::LD, pjt[m] * 16 + ln, kb * 32);
                }
#pragma unroll
            for (int rt = 0; rt < 4; ++rt) {
                mma(accD[rt], fw[rt], nsf[kb]);
                if (kOut) mma(accO[rt], sf[kb], fq[rt]);
            }
#pragma unroll
            for (int m = 0; m < NPT; ++m) {
                if (pmm[m]) {
                    // the Q rows of this tile: one of the slice's fragments above (wave-uniform pick)
                    Frag<T> fb = fq[0];
                    if (prt[m] == 1) fb = fq[1];
                    if (prt[m] == 2) fb = fq[2];
                    if (prt[m] == 3) fb = fq[3];
                    mma(pacc[m], fa[m], fb);
                }
            }
        }
#pragma unroll
        for (int m = 0; m < NPT; ++m) {
            if (pon[m]) {
                // pacc[i] = (Q K^T)[r = rt*16+ln][j = jt*16+gq*4+i]
                const int r = prt[m] * 16 + ln;
                const float gr = L.sGam[r];
                const f32x4 gj = *reinterpret_cast<const f32x4*>(L.sGam + pjt[m] * 16 + gq * 4);
                f32x4 v;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int j = pjt[m] * 16 + gq * 4 + i;
                    v[i] = (j <= r) ? pacc[m][i] * fast_exp(gr - gj[i]) : 0.f;
                }
                store4(L.sPm + r * C::LDP + frag_pos(pjt[m] * 16 + gq * 4), v);  // fragment order
            }
        }
    } else {
        // Independent accumulators are updated side by side (k32 slice outer, tiles inner) and
        // each slice's fragments are loaded before its products, so neither the matrix-core
        // latency nor the LDS latency sits on a chain of dependent products.
        if (kOut) {
            // this wave's P tiles (rows r of Q, columns j of K), at most NPT of them
            constexpr int NPT = (12 + C::NW - 1) / C::NW;
            f32x4 pacc[NPT];
            int prt[NPT], pjt[NPT];
            bool pon[NPT], pmm[NPT];
#pragma unroll
            for (int m = 0; m < NPT; ++m) {
                const int idx = wave + m * C::NW;
                pon[m] = idx < 12;
                prt[m] = pon[m] ? tri_row(idx) : 0;
                pjt[m] = pon[m] ? tri_col(idx) : 0;
                pmm[m] = pon[m] && pjt[m] <= prt[m];
                pacc[m] = zero4();
            }
#pragma unroll
            for (int kb = 0; kb < K / 32; ++kb) {
                Frag<T> fa[NPT], fb[NPT];
#pragma unroll
                for (int m = 0; m < NPT; ++m) {
                    if (pmm[m]) {
                        if constexpr (kKfo) frag_row_fo(fa[m], L.sK, C::LD, pjt[m] * 16 + ln, kb * 32);
                        else frag_row(fa[m], L.sK, C::LD, pjt[m] * 16 + ln, kb * 32);
                        frag_row_fo(fb[m], L.sQ, C::LD, prt[m] * 16 + ln, kb * 32);
                    }
                }
#pragma unroll
                for (int m = 0; m < NPT; ++m)
                    if (pmm[m]) mma(pacc[m], fa[m], fb[m]);
            }
#pragma unroll
            for (int m = 0; m < NPT; ++m) {
                if (pon[m]) {
                    // pacc[i] = (Q K^T)[r = rt*16+ln][j = jt*16+gq*4+i]
                    const int r = prt[m] * 16 + ln;
                    const float gr = L.sGam[r];
                    const f32x4 gj = *reinterpret_cast<const f32x4*>(L.sGam + pjt[m] * 16 + gq * 4);
                    f32x4 v;
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int j = pjt[m] * 16 + gq * 4 + i;
                        v[i] = (j <= r) ? pacc[m][i] * fast_exp(gr - gj[i]) : 0.f;
                    }
                    store4(L.sPm + r * C::LDP + frag_pos(pjt[m] * 16 + gq * 4), v);  // fragment order
                }
            }
        }
        // Delta = U - W S^T  (rows j of the chunk, columns = the wave's state rows), and
        // O^T tiles: accO[rt][i] = O^T[v = wave*16 + gq*4 + i][r = rt*16 + ln]. The S^T
        // accumulators are an A fragment of S and the Delta accumulators an A fragment of
        // Delta^T, so O^T = S Q^T diag(e^gam) + Delta^T P^T needs no data movement, and each
        // lane ends up with four consecutive value columns of one token row.
#pragma unroll
        for (int rt = 0; rt < 4; ++rt) {
            accD[rt] = col4(L.sU, C::LDU, wave * 16 + ln, rt * 16);
            if (kOut) accO[rt] = zero4();
        }
#pragma unroll
        for (int kb = 0; kb < K / 32; ++kb) {
            Frag<T> fw[4], fq[4];
#pragma unroll
            for (int rt = 0; rt < 4; ++rt) {
                frag_row_fo(fw[rt], L.sW, C::LD, rt * 16 + ln, kb * 32);
                if (kOut) frag_row_fo(fq[rt], L.sQ, C::LD, rt * 16 + ln, kb * 32);
            }
#pragma unroll
            for (int rt = 0; rt < 4; ++rt) {
                mma(accD[rt], fw[rt], nsf[kb]);
                if (kOut) mma(accO[rt], sf[kb], fq[rt]);
            }
        }
    }
    if (kOut) {
#pragma unroll
        for (int rt = 0; rt < 4; ++rt) accO[rt] *= L.sEg ? L.sEg[rt * 16 + ln] : fast_exp(L.sGam[rt * 16 + ln]);
    }
}

template <typename T, int K, int RT, bool kOut, bool kKfo = false>
__device__ __forceinline__ void chunk_part2(const RecurArgs& a, const ChunkLds<T, K, RT>& L, f32x4 (&accS)[K / 16],
                                            f32x4 (&accD)[4], f32x4 (&accO)[4], int64_t t0, int c, int h,
                                            int vcol0, typename Pack4<T>::type (&okeep)[4]) {
    using C = RCfg<T, K, RT>;
    const int tid = threadIdx.x;
    const int wave = wave_id(), lane = tid & 63, ln = lane & 15, gq = lane >> 4;
    if (kOut) {
        Frag<T> df[2];
        frag_acc(df[0], accD[0], accD[1]);
        frag_acc(df[1], accD[2], accD[3]);
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
            Frag<T> fb[4];
#pragma unroll
            for (int rt = 2 * kb; rt < 4; ++rt) frag_row_fo(fb[rt], L.sPm, C::LDP, rt * 16 + ln, kb * 32);
#pragma unroll
            for (int rt = 2 * kb; rt < 4; ++rt) mma(accO[rt], df[kb], fb[rt]);
        }
        T* o = reinterpret_cast<T*>(a.o);
        const int64_t H = a.geo.H;
        const int V = a.geo.V;
#pragma unroll
        for (int rt = 0; rt < 4; ++rt) okeep[rt] = Pack4<T>::make(accO[rt] * a.scale);
        if (L.sO) {
            // staged; stored as whole rows by the caller
#pragma unroll
            for (int rt = 0; rt < 4; ++rt)
                *reinterpret_cast<typename Pack4<T>::type*>(L.sO + (rt * 16 + ln) * C::LDU + wave * 16 + gq * 4) =
                    okeep[rt];
        } else {
            // a full chunk (the wave-uniform common case) stores with no branch per row
#pragma unroll
            for (int rt = 0; rt < 4; ++rt) {
                const int r = rt * 16 + ln;
                if (c == 64 || r < c)
                    *reinterpret_cast<typename Pack4<T>::type*>(o + ((t0 + r) * H + h) * V + vcol0 + wave * 16 +
                                                                gq * 4) = okeep[rt];
            }
        }
    }
    // S^T <- e^Gam S^T + K^T diag(e^{Gam-gam}) Delta
    const float G = L.sGam[63];
    const float eG = fast_exp(G);
    Frag<T> dtf[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
        f32x4 r0, r1;
        if (L.sEr) {
            r0 = *reinterpret_cast<const f32x4*>(L.sEr + kb * 32 + gq * 4);
            r1 = *reinterpret_cast<const f32x4*>(L.sEr + kb * 32 + 16 + gq * 4);
        } else {
            const f32x4 g0 = *reinterpret_cast<const f32x4*>(L.sGam + kb * 32 + gq * 4);
            const f32x4 g1 = *reinterpret_cast<const f32x4*>(L.sGam + kb * 32 + 16 + gq * 4);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                r0[i] = fast_exp(G - g0[i]);
                r1[i] = fast_exp(G - g1[i]);
            }
        }
        frag_acc_rows(dtf[kb], accD[2 * kb], accD[2 * kb + 1], r0, r1);
    }
#pragma unroll
    for (int kt = 0; kt < K / 16; ++kt) accS[kt] *= eG;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
        Frag<T> fa[K / 16];
#pragma unroll
        for (int kt = 0; kt < K / 16; ++kt) {
            if constexpr (kKfo) frag_col_fo(fa[kt], L.sK, C::LD, kt * 16 + ln, kb * 32);  // K^T row k, slots j
            else frag_col(fa[kt], L.sK, C::LD, kt * 16 + ln, kb * 32);
        }
#pragma unroll
        for (int kt = 0; kt < K / 16; ++kt) mma(accS[kt], fa[kt], dtf[kb]);
    }
}

// kL2 (output modes): q arrives raw and its rows are L2-normalised in registers before staging.
template <typename T, int K, int RT, int MODE, bool kL2 = false>
__global__ __launch_bounds__(RT * 4) void k_recur(RecurArgs a) {
    using C = RCfg<T, K, RT>;
    constexpr bool kOut = MODE == kRecurOut || MODE == kRecurOutRec;
    // records each chunk's entry state and Delta for the backward
    constexpr bool kRec = MODE == kRecurStates || MODE == kRecurOutRec;
    extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
    ChunkLds<T, K, RT> L;
    L.sQ = reinterpret_cast<T*>(smem + C::off_q);
    L.sK = reinterpret_cast<T*>(smem + C::off_k);
    L.sW = reinterpret_cast<T*>(smem + C::off_w);
    L.sU = reinterpret_cast<T*>(smem + C::off_u);
    L.sPm = reinterpret_cast<T*>(smem + C::off_pm);
    L.sGam = reinterpret_cast<float*>(smem + C::off_gam);
    if constexpr (MODE == kRecurPrepass) {
        // the prepass, with the least work per chunk step, takes the per-row exponentials from
        // tables made once per chunk (measured: the output pass does better computing its own)
        L.sEg = reinterpret_cast<float*>(smem + C::off_eg);
        L.sEr = reinterpret_cast<float*>(smem + C::off_er);
    }
    constexpr bool kStageO = kOut && C::stage_o;
    if constexpr (kStageO) L.sO = reinterpret_cast<T*>(smem + C::off_o);
    constexpr int kOffH = C::base_of(kOut, kRec);
    constexpr bool kStageH = kRec && C::lds_of(kOut, kRec) > kOffH;
    if constexpr (kStageH) L.sH = reinterpret_cast<T*>(smem + kOffH);

    const Geo& geo = a.geo;
    int64_t gs_ = blockIdx.x;
    int h_ = blockIdx.y, vt_ = blockIdx.z;
    if constexpr (MODE == kRecurPrepass) {
        // the prepass grid may be ranked (sequence-heads with exact maps dispatched first)
        if (!prepass_item(geo, a.modes, a.ranked != 0, (geo.V + K + RT - 1) / RT, gs_, h_, vt_)) return;
    } else if (geo.seg_order) {
        ordered_seg_item(geo, geo.V / RT, gs_, h_, vt_);
    }
    const int64_t gs = gs_;
    const int h = h_;
    const int vt = vt_;
    const int V = geo.V;
    const int64_t H = geo.H;
    SegLoc sg;
    if (!locate_seg(geo, gs, sg)) return;
    const int tid = threadIdx.x;
    const int wave = wave_id(), lane = tid & 63, ln = lane & 15, gq = lane >> 4;
    const int row = vt * RT + wave * 16 + ln;  // this lane's state row (value row, or V + M row)
    const size_t VK = (size_t)V * K;

    f32x4 accS[K / 16];
    int cbeg = sg.c0, cend = sg.c1;
    int mode = 0;
    if (MODE == kRecurPrepass) {
        // Heads whose boundaries all take the warmup (mode 1): this workgroup warms the state
        // entering its segment over the window before it, into seginit. Heads with exact
        // boundaries (mode 2, or 3 when mixed with warmup ones): this workgroup prepares the link
        // to the next segment as a map S -> S M + R~ into prep, the exact map of its segment, or,
        // where that boundary takes the warmup, M = 0 and R~ = the warm state, so that the
        // scan's S M + R~ restarts from it.
        mode = a.modes[sg.n * H + h];
        int win = 0;  // warmup window of the boundary this workgroup prepares (0: exact map)
        if (mode == 1) {
            if (sg.s == 0 || vt * RT >= V) return;
            win = a.bwin[gs * H + h];
        } else if (mode == 2 || mode == 3) {
            if (sg.s == sg.nseg - 1 || vt * RT >= V + K) return;
            win = mode == 3 ? a.bwin[(gs + 1) * H + h] : 0;
        } else {
            return;
        }
        if (win > 0) {
            // the window ends where the boundary's segment starts
            const int cb = mode == 1 ? sg.c0 : sg.c1;
            cend = cb;
            cbeg = max(0, cb - win);
            if (vt * RT >= V) cbeg = cend;  // the M rows of a warm link (whole tiles): M = 0
            if (vt * RT < V && cbeg == 0 && a.s0)
                load_state<K>(accS, a.s0 + ((size_t)sg.n * H + h) * VK, row);
            else
#pragma unroll
                for (int kt = 0; kt < K / 16; ++kt) accS[kt] = zero4();
        } else {
#pragma unroll
            for (int kt = 0; kt < K / 16; ++kt) {
                f32x4 z = zero4();
                if (row >= V) {
#pragma unroll
                    for (int i = 0; i < 4; ++i) z[i] = (kt * 16 + gq * 4 + i == row - V) ? 1.f : 0.f;
                }
                accS[kt] = z;
            }
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

    const int ucol0 = (vt * RT < V) ? vt * RT : -1;
    // Operands are fetched in three pieces issued over each step. Store data is held until
    // the next chunk's staging (see hold()), which waits for the step's loads anyway.
    typedef typename Pack4<T>::type PV;
    constexpr int NFL = 64 * (RT / C::VEC) / C::NT;  // Delta flush vectors per thread
    PV okeep[4], hkeep[K / 16];
    u32x4 okeep_rows[NFL];  // output passes: the previous chunk's O rows as stored
    // the chunk-entry state as stored: 16-byte vectors per lane
    constexpr int NHS = (K / 32 > RT * K / C::VEC / C::NT) ? K / 32 : RT * K / C::VEC / C::NT;
    u32x4 hst[NHS];
    u32x4 fkeep[NFL];
#pragma unroll
    for (int i = 0; i < 4; ++i) okeep[i] = PV{};
#pragma unroll
    for (int i = 0; i < K / 16; ++i) hkeep[i] = PV{};
#pragma unroll
    for (int i = 0; i < NHS; ++i) hst[i] = u32x4{0u, 0u, 0u, 0u};
#pragma unroll
    for (int i = 0; i < NFL; ++i) fkeep[i] = u32x4{0u, 0u, 0u, 0u};
#pragma unroll
    for (int i = 0; i < NFL; ++i) okeep_rows[i] = u32x4{0u, 0u, 0u, 0u};
    // The states and output passes prefetch one chunk ahead; the prepass, which has little
    // work per chunk to cover the loads, two chunks ahead in two alternating buffers.
    constexpr int kDepth = MODE == kRecurPrepass ? 2 : 1;
    ChunkRegs<T, K, RT, kOut> R0, R1;
    auto fetch_all = [&](ChunkRegs<T, K, RT, kOut>& R, int cn) {
        const int64_t tb = sg.bos + (int64_t)cn * 64;
        const int cb = min(64, sg.len - cn * 64);
        chunk_fetch<0>(R, a, tb, cb, h, ucol0);
        chunk_fetch<1>(R, a, tb, cb, h, ucol0);
        chunk_fetch<2>(R, a, tb, cb, h, ucol0);
    };
    auto step = [&](ChunkRegs<T, K, RT, kOut>& R, const int ci) {
        const int64_t t0 = sg.bos + (int64_t)ci * 64;
        const int c = min(64, sg.len - ci * 64);
#pragma unroll
        for (int i = 0; i < 4; ++i) hold(okeep[i]);
#pragma unroll
        for (int i = 0; i < K / 16; ++i) hold(hkeep[i]);
#pragma unroll
        for (int i = 0; i < NHS; ++i) hold(hst[i]);
#pragma unroll
        for (int i = 0; i < NFL; ++i) hold(fkeep[i]);
#pragma unroll
        for (int i = 0; i < NFL; ++i) hold(okeep_rows[i]);
        if (kStageH) {
            // entry state of this chunk, in the input precision, staged (stored after the barrier)
#pragma unroll
            for (int kt = 0; kt < K / 16; ++kt)
                *reinterpret_cast<PV*>(L.sH + (wave * 16 + ln) * C::LDH + kt * 16 + gq * 4) = Pack4<T>::make(accS[kt]);
        } else if (kRec) {
            // entry state of this chunk, in the input precision (no LDS room to stage it: fp32
            // at K = 128)
            T* hs = reinterpret_cast<T*>(a.hstates) + ((size_t)(sg.choff + ci) * H + h) * VK + (size_t)row * K;
#pragma unroll
            for (int kt = 0; kt < K / 16; ++kt) hkeep[kt] = Pack4<T>::make(accS[kt]);
#pragma unroll
            for (int kt = 0; kt < K / 16; ++kt) *reinterpret_cast<PV*>(hs + kt * 16 + gq * 4) = hkeep[kt];
        }
        lds_sync();  // previous chunk's LDS reads are done
        if constexpr (kStageH) {
            // the workgroup's RT rows of this chunk's entry state are one contiguous block
            T* hs = reinterpret_cast<T*>(a.hstates) + ((size_t)(sg.choff + ci) * H + h) * VK + (size_t)vt * RT * K;
            constexpr int NHV = RT * K / C::VEC / C::NT;  // 16-byte vectors per thread
            static_assert(NHV * C::NT * C::VEC == RT * K && NHV <= NHS, "state block split");
#pragma unroll
            for (int it = 0; it < NHV; ++it) {
                const int e = ((int)threadIdx.x + it * C::NT) * C::VEC;
                hst[it] = *reinterpret_cast<const u32x4*>(L.sH + (e / K) * C::LDH + e % K);
            }
#pragma unroll
            for (int it = 0; it < NHV; ++it)
                *reinterpret_cast<u32x4*>(hs + ((int)threadIdx.x + it * C::NT) * C::VEC) = hst[it];
        }
        if (kStageO && ci > cbeg) {
            // the previous chunk's O rows (a full chunk), staged by every wave: whole rows out
            T* dst = reinterpret_cast<T*>(a.o) + ((t0 - 64) * H + h) * V + vt * RT;
            constexpr int NV = RT / C::VEC;
#pragma unroll
            for (int it = 0; it < NFL; ++it) {
                const int u = (int)threadIdx.x + it * C::NT;
                okeep_rows[it] = *reinterpret_cast<const u32x4*>(L.sO + (u / NV) * C::LDU + (u % NV) * C::VEC);
            }
#pragma unroll
            for (int it = 0; it < NFL; ++it) {
                const int u = (int)threadIdx.x + it * C::NT;
                *reinterpret_cast<u32x4*>(dst + (size_t)(u / NV) * H * V + (u % NV) * C::VEC) = okeep_rows[it];
            }
        }
        if (kRec && a.delta && ci > cbeg) {
            // the previous chunk's Delta, staged over the q tile
            T* dst = reinterpret_cast<T*>(a.delta) + ((t0 - 64) * H + h) * V + vt * RT;
            constexpr int NV = RT / C::VEC;
#pragma unroll
            for (int it = 0; it < NFL; ++it) {
                const int u = (int)threadIdx.x + it * C::NT;
                fkeep[it] = *reinterpret_cast<const u32x4*>(L.sQ + (u / NV) * C::LDU + (u % NV) * C::VEC);
            }
#pragma unroll
            for (int it = 0; it < NFL; ++it) {
                const int u = (int)threadIdx.x + it * C::NT;
                *reinterpret_cast<u32x4*>(dst + (size_t)(u / NV) * H * V + (u % NV) * C::VEC) = fkeep[it];
            }
        }
        // (the output pass stages q over the tile just read: every wave's reads first)
        if (MODE == kRecurOutRec && a.delta) lds_sync();
        if constexpr (kL2 && kOut) l2norm_rows<T, K>(R.q);
        chunk_stage<T, K, RT, kOut>(R, L);
        lds_sync();
        // operands kDepth chunks ahead (the last chunk again past the end), in three pieces
        const int cn = min(ci + kDepth, cend - 1);
        const int64_t tn = sg.bos + (int64_t)cn * 64;
        const int cnn = min(64, sg.len - cn * 64);
        chunk_fetch<0>(R, a, tn, cnn, h, ucol0);
        // the states pass has the least work per step to cover the loads: all pieces at once
        if constexpr (MODE == kRecurStates) {
            chunk_fetch<1>(R, a, tn, cnn, h, ucol0);
            chunk_fetch<2>(R, a, tn, cnn, h, ucol0);
        }
        Frag<T> sf[K / 32];
        f32x4 accD[4], accO[4];
        chunk_part1<T, K, RT, kOut>(L, accS, sf, accD, accO);
        if (MODE == kRecurStates && a.delta) {
            // Delta for the backward, staged over the unused q tile ([64][RT], row j) and
            // written out after the next chunk's first barrier
#pragma unroll
            for (int rt = 0; rt < 4; ++rt) put_col4(L.sQ + (rt * 16 + gq * 4) * C::LDU + wave * 16 + ln, C::LDU, accD[rt]);
        }
        if constexpr (MODE != kRecurStates) {
            // u and the gate cumsum too: every chunk's loads land together in one burst across
            // the chip, so the last piece needs most of a step to arrive
            chunk_fetch<1>(R, a, tn, cnn, h, ucol0);
            chunk_fetch<2>(R, a, tn, cnn, h, ucol0);
        }
        if (kOut) lds_sync();  // P tiles complete (and every read of the q tile)
        if (MODE == kRecurOutRec && a.delta) {
            // Delta, staged over the q tile as in the states pass
#pragma unroll
            for (int rt = 0; rt < 4; ++rt) put_col4(L.sQ + (rt * 16 + gq * 4) * C::LDU + wave * 16 + ln, C::LDU, accD[rt]);
        }
        chunk_part2<T, K, RT, kOut>(a, L, accS, accD, accO, t0, c, h, vt * RT, okeep);
    };
    // the entering state may come from a load: wait for it here, before any prefetch, so the
    // loop never sees a load into the state registers in flight
#pragma unroll
    for (int kt = 0; kt < K / 16; ++kt) hold(accS[kt]);
    if constexpr (kDepth == 2) {
        // pairs of chunks without a branch between them (a step skipped inside the loop would
        // leave the compiler unsure how many loads are newer than the next chunk's, and it
        // would wait for all of them), then the last chunk
        if (cbeg < cend) {
            fetch_all(R0, cbeg);
            fetch_all(R1, min(cbeg + 1, cend - 1));
        }
        int ci = cbeg;
        for (; ci + 2 <= cend; ci += 2) {
            step(R0, ci);
            step(R1, ci + 1);
        }
        if (ci < cend) step(R0, ci);
    } else {
        if (cbeg < cend) fetch_all(R0, cbeg);
        for (int ci = cbeg; ci < cend; ++ci) step(R0, ci);
    }

    if ((kStageO || (kRec && a.delta)) && cbeg < cend) {
        lds_sync();
        const int cl = cend - 1;
        const size_t toff = ((sg.bos + (int64_t)cl * 64) * H + h) * V + vt * RT;
        if (kStageO)
            flush_tile<T, RT, C::NT>(reinterpret_cast<T*>(a.o) + toff, (size_t)H * V, min(64, sg.len - cl * 64), L.sO,
                                     C::LDU);
        if (kRec && a.delta)
            flush_tile<T, RT, C::NT>(reinterpret_cast<T*>(a.delta) + toff, (size_t)H * V, min(64, sg.len - cl * 64),
                                     L.sQ, C::LDU);
    }
    if (MODE == kRecurPrepass) {
        if (mode == 1) {
            store_state<K>(accS, a.seginit_out + ((size_t)gs * H + h) * VK, row);
        } else {
            float* P = a.prep + ((size_t)gs * H + h) * (size_t)(V + K) * K;
            if (row < V) {
                store_state<K>(accS, P, row);
            } else if (row < V + K) {
                // M^T[k][i], i = row - V, as a [K][K] matrix in the input precision (the
                // scan's matrix-core operand precision) after the R rows, each row in fragment
                // order (frag_pos) so that the scan loads its A fragments directly
                const int i = frag_pos(row - V);
                T* Mt = reinterpret_cast<T*>(P + VK);
#pragma unroll
                for (int kt = 0; kt < K / 16; ++kt)
#pragma unroll
                    for (int e = 0; e < 4; ++e) Mt[(size_t)(kt * 16 + gq * 4 + e) * K + i] = Elem<T>::from_f(accS[kt][e]);
            }
        }
    } else if (sg.s == sg.nseg - 1 && a.sT) {
        store_state<K>(accS, a.sT + ((size_t)sg.n * H + h) * VK, row);
    }
}

template <typename T, int K, int RT, int MODE, bool kL2 = false>
hipError_t launch_recur_t(const RecurArgs& a, int64_t nsegs_grid, int vtiles, hipStream_t st) {
    using C = RCfg<T, K, RT>;
    constexpr int lds = C::lds_of(MODE == kRecurOut || MODE == kRecurOutRec, MODE == kRecurStates || MODE == kRecurOutRec);
    static_assert(lds <= 160 * 1024, "LDS budget");
    auto kern = k_recur<T, K, RT, MODE, kL2>;
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, lds);
    if (e != hipSuccess) return e;
    // the prepass's ranked one-dimensional grid (see prepass_item), the varlen segment order's
    // (see ordered_seg_item), else (segments, heads, row tiles)
    const dim3 grid = MODE == kRecurPrepass && a.ranked
                          ? dim3((unsigned)((int64_t)vtiles * a.geo.nseg * a.geo.N * a.geo.H), 1u, 1u)
                      : MODE != kRecurPrepass && a.geo.seg_order
                          ? dim3((unsigned)(nsegs_grid * a.geo.H * vtiles), 1u, 1u)
                          : dim3((unsigned)nsegs_grid, (unsigned)a.geo.H, (unsigned)vtiles);
    hipLaunchKernelGGL(kern, grid, dim3(C::NT), lds, st, a);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// CP decision: one wave per sequence-head, one decision per boundary (the start of every
// segment but the first). Warmup over a window of w chunks is accepted at a boundary when the
// window reaches the sequence start (then it runs from the known state: exact), or when the
// gate sum over its w chunks is <= log(eps) and beta |k|^2 <= 2 on them (then every token map
// exp(g)(I - beta k k^T) has spectral norm <= exp(g), so a wrong state at the window start is
// damped by at least exp(window gate sum)). Each boundary takes the shortest w in [W, Wmax]
// that is accepted there, or the exact correction when none is. Each lane walks the chunks
// before (reverse: after) its boundaries once and sets bit w - W of a mask for every accepted
// w. The sequence-head's mode summarises its boundaries: 1 all warmup, 2 all exact, 3 mixed.
__global__ __launch_bounds__(kThreads) void k_decide(DecideArgs a) {
    const int wave = wave_id(), lane = threadIdx.x & 63;
    // one wave per sequence-head and direction (the two directions of one launch side by side)
    const int ndir = a.modes_r ? 2 : 1;
    const int64_t pd = (int64_t)blockIdx.x * 4 + wave;
    const int H = a.geo.H;
    if (pd >= (int64_t)a.geo.N * H * ndir) return;
    const int64_t p = pd / ndir;
    const int n = (int)(p / H), h = (int)(p % H);
    int32_t nseg, nchunks;
    int64_t segoff, choff;
    seq_segs(a.geo, n, nseg, segoff, nchunks, choff);
    const int W = a.warmup, span = a.warmup_max - a.warmup + 1;  // 1 .. 64 candidate windows
    const uint64_t all = span >= 64 ? ~0ull : ((1ull << span) - 1);
    // a.modes gets the decision for a.reverse's direction; a.modes_r, if given, the reverse one
    {
        const int dir = (int)(pd % ndir);
        int32_t* out = dir == 0 ? a.modes : a.modes_r;
        int32_t* wout = dir == 0 ? a.bwin : a.bwin_r;
        const bool rev = dir == 0 ? a.reverse != 0 : true;
        int32_t* bw = wout + segoff * H + h;  // this sequence-head's boundaries, stride H
        if (lane == 0) bw[0] = -1;  // segment 0 has no boundary
        int mode;
        if (nseg <= 1) {
            mode = 0;
        } else if (a.forced) {
            mode = a.forced;
            for (int s = 1 + lane; s < nseg; s += 64) bw[(int64_t)s * H] = a.forced == 1 ? W : 0;
        } else {
            bool any_warm = false, any_exact = false;
            for (int s = 1 + lane; s < nseg; s += 64) {
                const int cb = s * a.geo.seg_len;  // first chunk of segment s
                // forward: the chunks before segment s; reverse: the chunks from segment s on
                // (after segment s-1). A window that reaches the sequence start (end) runs
                // from the known state there: exact.
                const int avail = rev ? nchunks - cb : cb;
                uint64_t m = 0;
                float sum = 0.f, kk = 0.f;
                // the window's statistics in batches of 32 independent loads (one batch up to the
                // default longest window of one 32-chunk sub-sequence)
                for (int w0 = 0; w0 < a.warmup_max; w0 += 32) {
                    float2 st[32];
#pragma unroll
                    for (int j = 0; j < 32; ++j) {
                        const int w = w0 + j + 1;
                        // unconditional loads (no branch between them), clamped into the sequence;
                        // entries past the window are not used
                        const int idx = rev ? min(cb + w - 1, nchunks - 1) : max(cb - w, 0);
                        st[j] = a.cstat[(choff + idx) * H + h];
                    }
                    // (no break inside: the loop unrolls and st stays in registers)
#pragma unroll
                    for (int j = 0; j < 32; ++j) {
                        const int w = w0 + j + 1;
                        if (w <= a.warmup_max && w - 1 < avail) {
                            if (w >= avail) {
                                // this and every longer window start at the sequence start (end)
                                m |= w <= W ? all : (all & (~0ull << (w - W)));
                            } else {
                                sum += st[j].x;
                                kk = fmaxf(kk, st[j].y);
                                if (w >= W && sum <= a.log_eps && kk <= 2.f) m |= 1ull << (w - W);
                            }
                        }
                    }
                    if (w0 + 32 >= avail) break;
                }
                m &= all;
                bw[(int64_t)s * H] = m ? W + __builtin_ctzll(m) : 0;
                any_warm |= m != 0;
                any_exact |= m == 0;
            }
            // over the wave
            const bool warm = __any(any_warm), exact = __any(any_exact);
            mode = exact ? (warm ? 3 : 2) : 1;
        }
        if (lane == 0) out[p] = mode;
    }
}

// ---------------------------------------------------------------------------
// Exact CP: S_{s+1} = S_s M_s + R~_s across segments, for sequence-heads with an exact
// boundary (modes 2 and 3; a warm link of a mixed head carries M = 0 and R~ = its warm state).
// Grid (N, H, V/16): a workgroup carries 16 state rows through the segments of one
// sequence-head. A link is bound by the vector-memory throughput of its CU (every
// workgroup reads the whole M^T), so the rows are spread thin over many CUs: at 16 rows a
// link moves 48 KB per CU (M^T 32 KB, R~ 8 KB, the new state 8 KB) against 96 KB at 64
// rows. Wave w owns the output columns [w K/4, (w+1) K/4) of the 16 rows, as
// accumulator tiles of S^T: (S M)^T = M^T S^T, with the wave's rows of M^T as A fragments
// loaded straight from global memory (the prepasses store M^T in fragment order) and the
// state, staged in LDS once per link in the matrix-core operand precision, as the B
// operand of every wave. Maps and R~ rows travel four links ahead in four register
// buffers; the new state is stored before the next fetch is issued and its registers
// alternate between links, so no link waits for its own stores.
template <typename T, int K>
struct ScanCfg {
    static constexpr int RT = 16;                       // state rows per workgroup
    static constexpr int NRT = RT / 16;                 // row tiles
    static constexpr int NT = 256;
    static constexpr int KW = K / 64;                   // 16-column tiles per wave
    static constexpr int NKB = K / 32;                  // k32 slices
    static constexpr int LDS_ = K + RPad<T>::row;       // staged state row
    static constexpr int total = RT * LDS_ * (int)sizeof(T);
};

template <typename T, int K>
struct ScanMap {
    using SC = ScanCfg<T, K>;
    Frag<T> m[SC::KW][SC::NKB];  // M^T rows (w KW + j) * 16 + ln, k32 slice kb
    f32x4 r[SC::NRT][SC::KW];    // R~[rt*16 + ln][(w KW + j) * 16 + gq*4 ..]
};

template <typename T, int K, int kDepth>
__global__ __launch_bounds__(256) void k_scan(ScanArgs a) {
    using SC = ScanCfg<T, K>;
    constexpr int KW = SC::KW;
    constexpr int NRT = SC::NRT;
    extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
    T* sS = reinterpret_cast<T*>(smem);
    const int n = blockIdx.x, h = blockIdx.y, vt = blockIdx.z;
    const int H = a.geo.H, V = a.geo.V;
    const int mode = a.modes[(int64_t)n * H + h];
    if (mode != 2 && mode != 3) return;  // heads with an exact boundary (warm links carry M = 0)
    int32_t nseg, nchunks;
    int64_t segoff, choff;
    seq_segs(a.geo, n, nseg, segoff, nchunks, choff);
    if (nseg < 2) return;
    const int tid = threadIdx.x;
    const int wave = wave_id(), lane = tid & 63, ln = lane & 15, gq = lane >> 4;
    const int row0 = vt * SC::RT;  // first state row of the workgroup
    const int col0 = wave * KW * 16;
    const size_t VK = (size_t)V * K;
    const size_t PS = (size_t)(V + K) * K;  // floats per (segment, head) map

    // stage a state held as accumulator tiles: row rt*16 + ln, columns col0 + j*16 + gq*4 ..
    auto stage = [&](const f32x4 (&x)[NRT][KW]) {
#pragma unroll
        for (int rt = 0; rt < NRT; ++rt)
#pragma unroll
            for (int j = 0; j < KW; ++j)
                *reinterpret_cast<typename Pack4<T>::type*>(sS + (rt * 16 + ln) * SC::LDS_ + col0 + j * 16 + gq * 4) =
                    Pack4<T>::make(x[rt][j]);
    };
    auto tile_off = [&](int rt, int j) { return (size_t)(row0 + rt * 16 + ln) * K + col0 + j * 16 + gq * 4; };
    {
        f32x4 s0[NRT][KW];
#pragma unroll
        for (int rt = 0; rt < NRT; ++rt)
#pragma unroll
            for (int j = 0; j < KW; ++j)
                s0[rt][j] = a.s0 ? *reinterpret_cast<const f32x4*>(a.s0 + ((size_t)n * H + h) * VK + tile_off(rt, j))
                                 : zero4();
        stage(s0);
    }
    auto fetch = [&](ScanMap<T, K>& M, int s) {
        const float* P = a.prep + ((size_t)(segoff + s) * H + h) * PS;
        const T* Mt = reinterpret_cast<const T*>(P + VK);
#pragma unroll
        for (int j = 0; j < KW; ++j)
#pragma unroll
            for (int kb = 0; kb < SC::NKB; ++kb) frag_row_fo(M.m[j][kb], Mt, K, col0 + j * 16 + ln, kb * 32);
#pragma unroll
        for (int rt = 0; rt < NRT; ++rt)
#pragma unroll
            for (int j = 0; j < KW; ++j) M.r[rt][j] = *reinterpret_cast<const f32x4*>(P + tile_off(rt, j));
    };
    // forward: S_{s+1} = S_s M_s + R_s, s = 0 .. nseg-2
    // reverse: G_{s-1} = G_s M_s + R_s, s = nseg-1 .. 1 (adjoint leaving segment s-1)
    auto src_of = [&](int step) { return a.reverse ? nseg - 1 - step : step; };
    const int nsteps = nseg - 1;
    // maps in flight: four, or two (half the registers: the backward's reverse scan then fits
    // beside a workgroup of the chunk-state pass, which it runs next to)
    static_assert(kDepth == 2 || kDepth == 4, "two or four maps in flight");
    ScanMap<T, K> mb[kDepth];
    f32x4 accA[NRT][KW], accB[NRT][KW];
#pragma unroll
    for (int i = 0; i < kDepth; ++i) fetch(mb[i], src_of(min(i, nsteps - 1)));
    lds_sync();  // initial state staged
    auto one = [&](ScanMap<T, K>& M, f32x4 (&acc)[NRT][KW], const f32x4 (&other)[NRT][KW], int step) {
        const int s = src_of(step);
        const int dst = a.reverse ? s - 1 : s + 1;
#pragma unroll
        for (int rt = 0; rt < NRT; ++rt)
#pragma unroll
            for (int j = 0; j < KW; ++j) acc[rt][j] = M.r[rt][j];
#pragma unroll
        for (int kb = 0; kb < SC::NKB; ++kb) {
            Frag<T> b[NRT];
#pragma unroll
            for (int rt = 0; rt < NRT; ++rt) frag_row(b[rt], sS, SC::LDS_, rt * 16 + ln, kb * 32);  // rows of S
#pragma unroll
            for (int rt = 0; rt < NRT; ++rt)
#pragma unroll
                for (int j = 0; j < KW; ++j) mma(acc[rt][j], M.m[j][kb], b[rt]);
        }
        lds_sync();  // every wave's reads of the staged state are done
        stage(acc);
        float* out = a.seginit + ((size_t)(segoff + dst) * H + h) * VK;
#pragma unroll
        for (int rt = 0; rt < NRT; ++rt)
#pragma unroll
            for (int j = 0; j < KW; ++j) *reinterpret_cast<f32x4*>(out + tile_off(rt, j)) = acc[rt][j];
        // the previous link's stored state stays in its registers until here, so this
        // link's products never waited for those stores
#pragma unroll
        for (int rt = 0; rt < NRT; ++rt)
#pragma unroll
            for (int j = 0; j < KW; ++j) hold(other[rt][j]);
        // this buffer's next map (the last one again past the end), after the stores
        fetch(M, src_of(min(step + kDepth, nsteps - 1)));
        lds_sync();  // the new state is staged
    };
#pragma unroll
    for (int rt = 0; rt < NRT; ++rt)
#pragma unroll
        for (int j = 0; j < KW; ++j) accB[rt][j] = zero4();
    // whole groups of links without branches (a link skipped inside the loop would leave the
    // compiler unsure how many loads are newer than the next map's, and it would wait for
    // all of them), then the rest
    int step = 0;
    for (; step + kDepth <= nsteps; step += kDepth) {
        one(mb[0], accA, accB, step);
        one(mb[1], accB, accA, step + 1);
        if constexpr (kDepth == 4) {
            one(mb[2], accA, accB, step + 2);
            one(mb[3], accB, accA, step + 3);
        }
    }
    if (step < nsteps) one(mb[0], accA, accB, step);
    if constexpr (kDepth == 4) {
        if (step + 1 < nsteps) one(mb[1], accB, accA, step + 1);
        if (step + 2 < nsteps) one(mb[2], accA, accB, step + 2);
    }
}

template <typename T, int K>
hipError_t launch_scan_t(const ScanArgs& a, hipStream_t st) {
    using SC = ScanCfg<T, K>;
    // the reverse scan runs beside the backward's chunk-state pass: two maps in flight
    auto kern = a.reverse ? k_scan<T, K, 2> : k_scan<T, K, 4>;
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, SC::total);
    if (e != hipSuccess) return e;
    dim3 grid((unsigned)a.geo.N, (unsigned)a.geo.H, (unsigned)(a.geo.V / SC::RT));
    hipLaunchKernelGGL(kern, grid, dim3(SC::NT), SC::total, st, a);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Fully fused forward (no CP): the first kernel's intra-chunk step and the recurrence in one
// workgroup per (sequence, head, row tile), chunk after chunk. The gate cumsum, A, T = (I+A)^-1
// and the WY factors W = T diag(beta e^gam) K, U = T diag(beta) V[:, this tile] live in LDS only,
// so the forward moves q, k, v, g, beta in and o out (1,032 B per token-head at K = V = 128 in
// bf16) instead of the split's 2,320 B, at the price of the intra work on the recurrence's serial
// chain. This is the pages' fully fused alternative, which they name as the better design at
// large batch (announcement post, on the two-kernel split's extra memory I/O); the planner picks
// it where the recurrence already runs in several rounds of workgroups.
//
// Layout: the recurrence's tiles (q and w in fragment order, u [64][RT], the P tiles, the gate
// cumsum), k in fragment order (the Gram rows, and the recurrence through its fragment-order
// reads), this tile's value columns of v [64][RT] row-major, A and T in fp32, beta. With eight
// waves (RT = 128) waves 0-3 form W and waves 4-7 U; with four, every wave both.
template <typename T, int K, int RT>
struct FCfg {
    using C = RCfg<T, K, RT>;
    static constexpr int LDV = RT + RPad<T>::row;
    static constexpr int off_v = C::total;
    static constexpr int off_a = off_v + 64 * LDV * (int)sizeof(T);
    static constexpr int off_t = off_a + 64 * kLdA * 4;
    static constexpr int off_beta = off_t + 64 * kLdA * 4;
    static constexpr int total = off_beta + 256;
    static constexpr int IV = 64 * (RT / C::VEC) / C::NT;  // v vectors per thread
    static_assert(IV * C::NT == 64 * (RT / C::VEC), "v tile split");
};

template <typename T, int K, int RT>
struct FusedRegs {
    using C = RCfg<T, K, RT>;
    using F = FCfg<T, K, RT>;
    u32x4 q[C::IQ], k[C::IQ], v[F::IV];
    float g, beta;  // lanes of wave 0
};

template <typename T, int K, int RT>
__device__ __forceinline__ void fused_fetch(FusedRegs<T, K, RT>& R, const RecurArgs& a, int64_t t0, int c, int h,
                                            int vcol0) {
    using C = RCfg<T, K, RT>;
    using F = FCfg<T, K, RT>;
    const int64_t H = a.geo.H;
    const size_t ok = ((size_t)t0 * H + h) * K;
    fetch_tile<T, K, C::IQ, C::NT>(R.q, reinterpret_cast<const T*>(a.q) + ok, (size_t)H * K, c);
    fetch_tile<T, K, C::IQ, C::NT>(R.k, reinterpret_cast<const T*>(a.k) + ok, (size_t)H * K, c);
    fetch_tile<T, RT, F::IV, C::NT>(R.v, reinterpret_cast<const T*>(a.fv) + ((size_t)t0 * H + h) * a.geo.V + vcol0,
                                    (size_t)H * a.geo.V, c);
    const int tid = threadIdx.x;
    if (tid < 64) {
        const bool in = tid < c;
        const int64_t i = (t0 + (in ? tid : 0)) * H + h;
        R.g = in ? a.fg[i] : 0.f;
        R.beta = in ? a.fbeta[i] : 0.f;
    }
}

// kL2: q and k arrive raw and their rows are L2-normalised in registers before staging.
template <typename T, int K, int RT, bool kL2>
__global__ __launch_bounds__(RT * 4) void k_fused(RecurArgs a) {
    using C = RCfg<T, K, RT>;
    using F = FCfg<T, K, RT>;
    constexpr int NW = C::NW;
    extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
    ChunkLds<T, K, RT> L;
    L.sQ = reinterpret_cast<T*>(smem + C::off_q);
    L.sK = reinterpret_cast<T*>(smem + C::off_k);
    L.sW = reinterpret_cast<T*>(smem + C::off_w);
    L.sU = reinterpret_cast<T*>(smem + C::off_u);
    L.sPm = reinterpret_cast<T*>(smem + C::off_pm);
    L.sGam = reinterpret_cast<float*>(smem + C::off_gam);
    T* sV = reinterpret_cast<T*>(smem + F::off_v);
    float* sA = reinterpret_cast<float*>(smem + F::off_a);
    float* sT = reinterpret_cast<float*>(smem + F::off_t);
    float* sBeta = reinterpret_cast<float*>(smem + F::off_beta);

    const Geo& geo = a.geo;
    int64_t gs = blockIdx.x;
    int h = blockIdx.y, vt = blockIdx.z;
    if (geo.seg_order) ordered_seg_item(geo, geo.V / RT, gs, h, vt);  // varlen: longest first
    const int V = geo.V;
    SegLoc sg;
    if (!locate_seg(geo, gs, sg)) return;
    const int tid = threadIdx.x;
    const int wave = wave_id(), lane = tid & 63, ln = lane & 15, gq = lane >> 4;
    const int row = vt * RT + wave * 16 + ln;
    const size_t VK = (size_t)V * K;
    const int vcol0 = vt * RT;

    f32x4 accS[K / 16];
    if (a.s0) {
        load_state<K>(accS, a.s0 + ((size_t)sg.n * geo.H + h) * VK, row);
    } else {
#pragma unroll
        for (int kt = 0; kt < K / 16; ++kt) accS[kt] = zero4();
    }
#pragma unroll
    for (int kt = 0; kt < K / 16; ++kt) hold(accS[kt]);
    const int cbeg = sg.c0, cend = sg.c1;
    if (cbeg < cend) {
        typedef typename Pack4<T>::type PV;
        PV okeep[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) okeep[i] = PV{};
        FusedRegs<T, K, RT> R;
        fused_fetch(R, a, sg.bos + (int64_t)cbeg * 64, min(64, sg.len - cbeg * 64), h, vcol0);
        // the strictly upper blocks of T stay zero for every chunk
        tri_zero_upper64(sT);
        for (int ci = cbeg; ci < cend; ++ci) {
            const int64_t t0 = sg.bos + (int64_t)ci * 64;
            const int c = min(64, sg.len - ci * 64);
#pragma unroll
            for (int i = 0; i < 4; ++i) hold(okeep[i]);
            lds_sync();  // the previous chunk's LDS reads are done
            // ---- stage: q, k (fragment order), this tile's v columns, gate cumsum, beta ----
            if constexpr (kL2) {
                l2norm_rows<T, K>(R.q);
                l2norm_rows<T, K>(R.k);
            }
            put_tile_fo<T, K, C::IQ, C::NT>(L.sQ, C::LD, R.q);
            put_tile_fo<T, K, C::IQ, C::NT>(L.sK, C::LD, R.k);
            put_tile<T, RT, F::IV, C::NT>(sV, F::LDV, R.v);
            if (wave == 0) {
                const float x = wave_prefix_sum(R.g);  // rows past the chunk end carry the total
                L.sGam[lane] = x;
                sBeta[lane] = R.beta;
            }
            // the next chunk's operands (the last chunk again past the end)
            {
                const int cn = min(ci + 1, cend - 1);
                fused_fetch(R, a, sg.bos + (int64_t)cn * 64, min(64, sg.len - cn * 64), h, vcol0);
            }
            lds_sync();
            // ---- A = strict_lower(diag(beta) (e^{gam_r - gam_j} K K^T)): lower 16x16 tiles ----
            {
                constexpr int NTT = (10 + NW - 1) / NW;
                f32x4 acc[NTT];
                int ti[NTT], tj[NTT];
                bool on[NTT];
#pragma unroll
                for (int m = 0; m < NTT; ++m) {
                    const int idx = wave + NW * m;
                    on[m] = idx < 10;
                    ti[m] = tri_row(min(idx, 9));
                    tj[m] = tri_col(min(idx, 9));
                    acc[m] = zero4();
                }
#pragma unroll
                for (int kb = 0; kb < K / 32; ++kb) {
                    Frag<T> fa[NTT], fb[NTT];
#pragma unroll
                    for (int m = 0; m < NTT; ++m) {
                        frag_row_fo(fa[m], L.sK, C::LD, tj[m] * 16 + ln, kb * 32);
                        frag_row_fo(fb[m], L.sK, C::LD, ti[m] * 16 + ln, kb * 32);
                    }
#pragma unroll
                    for (int m = 0; m < NTT; ++m) mma(acc[m], fa[m], fb[m]);
                }
                // acc[m][i] = k_j . k_r, j = tj*16 + gq*4 + i, r = ti*16 + ln
#pragma unroll
                for (int m = 0; m < NTT; ++m) {
                    if (on[m]) {
                        const int r = ti[m] * 16 + ln;
                        const float gr = L.sGam[r], br = sBeta[r];
                        const f32x4 gj = *reinterpret_cast<const f32x4*>(L.sGam + tj[m] * 16 + gq * 4);
                        f32x4 val;
#pragma unroll
                        for (int i = 0; i < 4; ++i) {
                            const int j = tj[m] * 16 + gq * 4 + i;
                            val[i] = (j < r) ? br * fast_exp(gr - gj[i]) * acc[m][i] : 0.f;
                        }
                        *reinterpret_cast<f32x4*>(sA + r * kLdA + tj[m] * 16 + gq * 4) = val;
                    }
                }
            }
            lds_sync();
            // ---- T = (I + A)^-1 (waves 0-3) ----
            tri_inverse64(sA, sT);
            // ---- W = T diag(beta e^gam) K (row tile rw), U = T diag(beta) V (row tile ru) --------
            {
                const bool doW = NW == 4 || wave < 4;
                const bool doU = NW == 4 || wave >= 4;
                const int rt = wave & 3;
                Frag<T> aw[2], au[2];
#pragma unroll
                for (int kb = 0; kb < 2; ++kb) {
                    Frag<float> tf;
                    frag_row(tf, sT, kLdA, rt * 16 + ln, kb * 32);
                    const f32x4 b0 = *reinterpret_cast<const f32x4*>(sBeta + kb * 32 + gq * 4);
                    const f32x4 b1 = *reinterpret_cast<const f32x4*>(sBeta + kb * 32 + 16 + gq * 4);
                    const f32x4 g0 = *reinterpret_cast<const f32x4*>(L.sGam + kb * 32 + gq * 4);
                    const f32x4 g1 = *reinterpret_cast<const f32x4*>(L.sGam + kb * 32 + 16 + gq * 4);
                    float fw[8], fu[8];
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        const float tv = e < 4 ? tf.lo[e] : tf.hi[e - 4];
                        const float bj = e < 4 ? b0[e] : b1[e - 4];
                        const float gjv = e < 4 ? g0[e] : g1[e - 4];
                        fu[e] = tv * bj;
                        fw[e] = fu[e] * fast_exp(gjv);
                    }
                    aw[kb].v = u32x4{pack_bf2(fw[0], fw[1]), pack_bf2(fw[2], fw[3]), pack_bf2(fw[4], fw[5]),
                                     pack_bf2(fw[6], fw[7])};
                    au[kb].v = u32x4{pack_bf2(fu[0], fu[1]), pack_bf2(fu[2], fu[3]), pack_bf2(fu[4], fu[5]),
                                     pack_bf2(fu[6], fu[7])};
                }
                const int nkb = (rt >> 1) + 1;  // T[r][j] = 0 for j > r
                const int orow = rt * 16 + ln;
                if (doW) {
                    // transposed tiles: accw[ct][i] = W[orow][ct*16 + gq*4 + i]
                    f32x4 accw[K / 16];
#pragma unroll
                    for (int ct = 0; ct < K / 16; ++ct) {
                        accw[ct] = zero4();
#pragma unroll
                        for (int kb = 0; kb < 2; ++kb) {
                            if (kb < nkb) {
                                Frag<T> b;
                                frag_col_fo(b, L.sK, C::LD, ct * 16 + ln, kb * 32);  // K^T row ct*16+ln, slots j
                                mma(accw[ct], b, aw[kb]);
                            }
                        }
                    }
#pragma unroll
                    for (int ct = 0; ct < K / 16; ++ct) store4(L.sW + orow * C::LD + frag_pos(ct * 16 + gq * 4), accw[ct]);
                }
                if (doU) {
                    f32x4 accu[RT / 16];
#pragma unroll
                    for (int ct = 0; ct < RT / 16; ++ct) {
                        accu[ct] = zero4();
#pragma unroll
                        for (int kb = 0; kb < 2; ++kb) {
                            if (kb < nkb) {
                                Frag<T> b;
                                frag_col(b, sV, F::LDV, ct * 16 + ln, kb * 32);  // V^T row ct*16+ln, slots j
                                mma(accu[ct], b, au[kb]);
                            }
                        }
                    }
#pragma unroll
                    for (int ct = 0; ct < RT / 16; ++ct) store4(L.sU + orow * C::LDU + ct * 16 + gq * 4, accu[ct]);
                }
            }
            lds_sync();
            // ---- the recurrence step on the staged tiles ----
            Frag<T> sf[K / 32];
            f32x4 accD[4], accO[4];
            chunk_part1<T, K, RT, true, true>(L, accS, sf, accD, accO);
            lds_sync();  // P tiles complete
            chunk_part2<T, K, RT, true, true>(a, L, accS, accD, accO, t0, c, h, vcol0, okeep);
        }
    }
    if (a.sT) store_state<K>(accS, a.sT + ((size_t)sg.n * geo.H + h) * VK, row);
}

template <typename T, int K, int RT>
hipError_t launch_fused_t(const RecurArgs& a, int64_t nseqs, int vtiles, hipStream_t st) {
    using F = FCfg<T, K, RT>;
    static_assert(F::total <= 160 * 1024, "LDS budget");
    auto kern = a.q_l2 ? k_fused<T, K, RT, true> : k_fused<T, K, RT, false>;
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, F::total);
    if (e != hipSuccess) return e;
    const dim3 grid = a.geo.seg_order ? dim3((unsigned)(nseqs * a.geo.H * vtiles), 1u, 1u)
                                      : dim3((unsigned)nseqs, (unsigned)a.geo.H, (unsigned)vtiles);
    hipLaunchKernelGGL(kern, grid, dim3(RT * 4), F::total, st, a);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Varlen tables from the device cu_seqlens (one workgroup). Lengths and offsets are
// clamped into [0, Ttot], so a bad cu_seqlens can never send a later kernel out of
// bounds; entries the host sized but the device data does not fill stay marked unused.
__global__ __launch_bounds__(kThreads) void k_tables(TableArgs a) {
    __shared__ int32_t s_ch[kThreads], s_sg[kThreads];
    __shared__ int32_t s_base[2];
    __shared__ int32_t s_bin[kOrderBins];  // the segment order's counting sort
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
    // fill: a wave per 64 sequences; each sequence's chunk entries are written by all 64 lanes
    // (its count and first chunk shuffled from the lane that holds it), its segment entries by
    // its own lane
    const int lane = tid & 63;
    for (int nb = tid - lane; nb < a.N; nb += kThreads) {
        const int n = nb + lane;
        const int32_t nch = n < a.N ? (a.seq_len[n] + 63) / 64 : 0;
        const int32_t co = n < a.N ? a.seq_choff[n] : 0;
        for (int src = 0; src < 64; ++src) {
            const int32_t m = __shfl(nch, src), cs = __shfl(co, src);
            for (int j = lane; j < m; j += 64)
                if (cs + j < a.total_chunks) a.chunk_tab[cs + j] = make_int2(nb + src, j);
        }
        if (n < a.N) {
            const int64_t so = a.seq_segoff[n];
            const int32_t nsg = a.seq_segoff[n + 1] - a.seq_segoff[n];
            for (int s = 0; s < nsg; ++s) {
                const int c0 = s * a.seg_len;
                const int c1 = min(c0 + a.seg_len, nch);
                if (so + s < a.total_segs) a.seg_tab[so + s] = make_int4(n, s, nsg == 1 ? 0 : c0, nsg == 1 ? nch : c1);
            }
        }
    }
    if (a.seg_order == nullptr) return;
    // The segment order, most chunks first: a counting sort on the chunk count (clamped to the
    // last bin). Segments with equal counts land in any order, which changes no result (every
    // workgroup's work is the same wherever the grid puts it); unused entries count as empty.
    auto bin_of = [&](int64_t i) {
        const int4 e = a.seg_tab[i];
        return e.x < 0 ? 0 : min(e.w - e.z, kOrderBins - 1);
    };
    for (int i = tid; i < kOrderBins; i += kThreads) s_bin[i] = 0;
    __syncthreads();  // also makes this workgroup's segment entries visible to all its threads
    for (int64_t i = tid; i < a.total_segs; i += kThreads) atomicAdd(&s_bin[bin_of(i)], 1);
    __syncthreads();
    // first slot of each bin: the segments in the bins above it (thread t sums the bins of
    // ranks [t P, t P + P) counted from the top, then a scan over the threads)
    constexpr int P = kOrderBins / kThreads;
    int32_t cnt[P], sum = 0;
#pragma unroll
    for (int j = 0; j < P; ++j) {
        cnt[j] = s_bin[kOrderBins - 1 - (tid * P + j)];
        sum += cnt[j];
    }
    s_ch[tid] = sum;
    __syncthreads();
    for (int off = 1; off < kThreads; off <<= 1) {
        const int32_t x = tid >= off ? s_ch[tid - off] : 0;
        __syncthreads();
        s_ch[tid] += x;
        __syncthreads();
    }
    int32_t at = s_ch[tid] - sum;
#pragma unroll
    for (int j = 0; j < P; ++j) {
        s_bin[kOrderBins - 1 - (tid * P + j)] = at;
        at += cnt[j];
    }
    __syncthreads();
    for (int64_t i = tid; i < a.total_segs; i += kThreads) a.seg_order[atomicAdd(&s_bin[bin_of(i)], 1)] = (int32_t)i;
}

}  // namespace

hipError_t launch_recur(const RecurArgs& a, int dtype, int mode, int64_t nsegs_grid, int vtiles,
                        hipStream_t st) {
    if (nsegs_grid == 0) return hipSuccess;
    const int K = a.geo.K;
    const int RT = recur_rows(a.geo.V, K);
#define GDN_RECUR_CASE(TT, KK, RR)                                                                         \
    if (K == KK && RT == RR) {                                                                             \
        if (mode == kRecurOut)                                                                             \
            return a.q_l2 ? launch_recur_t<TT, KK, RR, kRecurOut, true>(a, nsegs_grid, vtiles, st)          \
                          : launch_recur_t<TT, KK, RR, kRecurOut>(a, nsegs_grid, vtiles, st);               \
        if (mode == kRecurOutRec)                                                                          \
            return a.q_l2 ? launch_recur_t<TT, KK, RR, kRecurOutRec, true>(a, nsegs_grid, vtiles, st)       \
                          : launch_recur_t<TT, KK, RR, kRecurOutRec>(a, nsegs_grid, vtiles, st);            \
        if (mode == kRecurPrepass) return launch_recur_t<TT, KK, RR, kRecurPrepass>(a, nsegs_grid, vtiles, st); \
        if (mode == kRecurStates) return launch_recur_t<TT, KK, RR, kRecurStates>(a, nsegs_grid, vtiles, st); \
    }
    if (dtype == 0) {
        GDN_RECUR_CASE(bf16_t, 64, 64)
        GDN_RECUR_CASE(bf16_t, 128, 64)
        GDN_RECUR_CASE(bf16_t, 128, 128)
    } else {
        GDN_RECUR_CASE(float, 64, 64)
        GDN_RECUR_CASE(float, 128, 64)
        GDN_RECUR_CASE(float, 128, 128)
    }
#undef GDN_RECUR_CASE
    return hipErrorInvalidValue;
}

hipError_t launch_fused(const RecurArgs& a, int dtype, int64_t nseqs, int vtiles, hipStream_t st) {
    if (nseqs == 0) return hipSuccess;
    if (dtype != 0) return hipErrorInvalidValue;  // bf16 only (fp32 tiles exceed the LDS)
    const int K = a.geo.K;
    const int RT = recur_rows(a.geo.V, K);
    if (K == 64 && RT == 64) return launch_fused_t<bf16_t, 64, 64>(a, nseqs, vtiles, st);
    if (K == 128 && RT == 64) return launch_fused_t<bf16_t, 128, 64>(a, nseqs, vtiles, st);
    if (K == 128 && RT == 128) return launch_fused_t<bf16_t, 128, 128>(a, nseqs, vtiles, st);
    return hipErrorInvalidValue;
}

hipError_t launch_decide(const DecideArgs& a, hipStream_t st) {
    const int64_t p = (int64_t)a.geo.N * a.geo.H * (a.modes_r ? 2 : 1);
    if (p == 0) return hipSuccess;
    hipLaunchKernelGGL(k_decide, dim3((unsigned)((p + 3) / 4)), dim3(kThreads), 0, st, a);
    return hipGetLastError();
}

hipError_t launch_scan(const ScanArgs& a, int dtype, hipStream_t st) {
    if (a.geo.N == 0) return hipSuccess;
    const int K = a.geo.K;
    // 16 state rows per workgroup whatever the recurrence uses: the scan is a serial chain
    // per sequence-head, and more workgroups per head shorten each link
    if (dtype == 0) {
        if (K == 64) return launch_scan_t<bf16_t, 64>(a, st);
        if (K == 128) return launch_scan_t<bf16_t, 128>(a, st);
    } else {
        if (K == 64) return launch_scan_t<float, 64>(a, st);
        if (K == 128) return launch_scan_t<float, 128>(a, st);
    }
    return hipErrorInvalidValue;
}

hipError_t launch_tables(const TableArgs& a, hipStream_t st) {
    hipLaunchKernelGGL(k_tables, dim3(1), dim3(kThreads), 0, st, a);
    return hipGetLastError();
}

}  // namespace gdn
