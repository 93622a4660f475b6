// gdn_bwd.hip -- backward of the GDN chunked prefill (the pages ask for fwd and bwd entry
// points; ollai.cn article, "main features", and say the backward "was the hardest part").
//
// Reverse mode of the chunk map, derived from the gated delta rule. For a chunk entering
// with state S, with G = dL/dS' the adjoint of the state leaving it and dO the output
// gradient (P = L .* Q K^T with the chunk's decay mask, Kt = diag(e^{Gam-gam}) K):
//   dDelta = P^T dO + Kt G^T
//   G_in   = e^Gam G + dO^T diag(e^gam) Q - dDelta^T W      (adjoint entering the chunk)
// G_in is affine in G with the transposed chunk map, so the same CP scheme as the forward
// splits the serial chain: warmup windows after each sub-sequence, or exact maps composed
// from the end. The per-chunk gradients then run in parallel over all chunks (k_bwd_chunk):
//   state side: Delta = U - W S^T, dQt = dO S, dP = dO U^T - dQt W^T, dKt = Delta G,
//     dW = -dDelta S  ->  dq, the P and Kt terms of dk and d(gam), dW, dU
//   WY side: with T = (I + A)^{-1} (written by the intra-chunk kernel); dT = dW Bk^T + dU Bv^T,
//     dA = strict_lower(-T^T dT T^T), dBk = T^T dW, dBv = T^T dU  ->  dk, dv, dbeta, and
//     dg as the in-chunk reverse cumulative sum of d(gam).
#include <type_traits>

#include "gdn_common.h"
#include "gdn_kernels.h"
#include "gdn_norm.h"

namespace gdn {

namespace {

template <typename T> struct BPad;
template <> struct BPad<bf16_t> { static constexpr int row = 8; };
template <> struct BPad<float> { static constexpr int row = 4; };
// The [64][K] tiles that k_bwd_chunk reads transposed most (K, Q, dW) and its 64x64 matrices:
// in bf16 at K = V = 128 a row stride of K + 16 elements (144; 80 for 64 columns) halves the cost
// of the transpose reads of fragment-order tiles against K + 8, whose rows collide in the LDS banks
// on every such read (measured with the LDS bank-conflict counters: k_bwd_chunk 531 -> 485 us at
// the 32K workload). The LDS budget leaves the other tiles at K + 8.
template <typename T> struct BPadK;
template <> struct BPadK<bf16_t> { static constexpr int row = 16; };
template <> struct BPadK<float> { static constexpr int row = 4; };

// ---------------------------------------------------------------------------
// Reverse adjoint recurrence. RT adjoint rows (value rows, or V + M-hat rows in the
// exact prepass) per workgroup, one wave per 16 rows; the adjoint lives in registers as
// fp32 accumulator tiles of G^T, which are a B fragment of G^T.
template <typename T, int K, int RT>
struct VCfg {
    static constexpr int NW = RT / 16;
    static constexpr int NT = NW * 64;
    static constexpr int VEC = Elem<T>::kVec;
    static constexpr int LD = K + 2 * BPad<T>::row;    // row-major q, scaled q, k, w  [64][K]
    static constexpr int LDD = RT + 2 * BPad<T>::row;  // row-major dO tile            [64][RT]
    static constexpr int LDP = 64 + BPad<T>::row;   // P^T                          [64][64]
    static constexpr int kMat = 64 * LD * (int)sizeof(T);
    static constexpr int off_q = 0;                 // Q
    static constexpr int off_qs = off_q + kMat;     // scale * e^gam_r * Q
    static constexpr int off_k = off_qs + kMat;     // K
    static constexpr int off_w = off_k + kMat;      // W
    static constexpr int off_do = off_w + kMat;     // dO
    static constexpr int off_pm = off_do + 64 * LDD * (int)sizeof(T);
    static constexpr int off_dd = off_pm + 64 * LDP * (int)sizeof(T);   // dDelta tile [64][RT]
    static constexpr int off_gam = off_dd + 64 * LDD * (int)sizeof(T);
    static constexpr int off_er = off_gam + 256;  // e^{Gam - gam_j}, once per chunk
    static constexpr int total = off_er + 256;
    static constexpr int NVK = K / VEC;
    static constexpr int NVD = RT / VEC;
    static constexpr int IK = 64 * NVK / NT;   // q, k, w rows
    static constexpr int ID = 64 * NVD / NT;   // dO rows
    static_assert(IK * NT == 64 * NVK && ID * NT == 64 * NVD, "tile split");
};


template <typename T, int K, int RT>
struct RevRegs {
    using C = VCfg<T, K, RT>;
    u32x4 q[C::IK], k[C::IK], w[C::IK];
    float gq[C::IK];  // gate cumsum of the q row (scales its copy)
    u32x4 d[C::ID];
    float gam;
};

// One chunk's operands in three pieces, issued at different points of a step.
template <int kPart, typename T, int K, int RT>
__device__ __forceinline__ void rev_fetch(RevRegs<T, K, RT>& R, const RevArgs& a, int64_t t0, int c, int h,
                                          int dcol0) {
    using C = VCfg<T, K, RT>;
    const int64_t H = a.geo.H;
    const size_t ok = ((size_t)t0 * H + h) * K;
    if constexpr (kPart == 0) {
        fetch_tile<T, K, C::IK, C::NT>(R.q, reinterpret_cast<const T*>(a.q) + ok, (size_t)H * K, c);
        fetch_tile<T, K, C::IK, C::NT>(R.k, reinterpret_cast<const T*>(a.k) + ok, (size_t)H * K, c);
        // gate cumsum of each q row this thread holds (rows r0 + it * NT / NVK)
        const int r0 = (int)threadIdx.x / C::NVK;
#pragma unroll
        for (int it = 0; it < C::IK; ++it) {
            const int r = r0 + it * (C::NT / C::NVK);
            R.gq[it] = a.gam[(t0 + min(r, c - 1)) * H + h];
        }
    } else if constexpr (kPart == 1) {
        fetch_tile<T, K, C::IK, C::NT>(R.w, reinterpret_cast<const T*>(a.w) + ok, (size_t)H * K, c);
    } else {
        // the M-hat rows of the exact prepass (dcol0 < 0) have no output gradient
        fetch_tile<T, RT, C::ID, C::NT>(R.d, reinterpret_cast<const T*>(a.d_o) + ((size_t)t0 * H + h) * a.geo.V +
                                                 max(dcol0, 0),
                                        (size_t)H * a.geo.V, dcol0 >= 0 ? c : 0);
        const int tid = threadIdx.x;
        if (tid < 64) {
            const int r = tid < c ? tid : c - 1;
            R.gam = a.gam[(t0 + r) * H + h];
        }
    }
}

template <typename T, int K, int RT>
struct RevLds {
    T* sQ;
    T* sQs;  // scale * e^gam_r * Q
    T* sK;
    T* sW;
    T* sD;   // dO
    T* sPm;  // P^T [j][r]
    float* sGam;
    float* sEr;  // e^{Gam - gam_j}
};

template <typename T, int K, int RT>
__device__ __forceinline__ void rev_stage(const RevRegs<T, K, RT>& R, const RevLds<T, K, RT>& L, float scale) {
    using C = VCfg<T, K, RT>;
    // q and k rows in fragment order (read as row fragments only); w row-major (read transposed)
    put_tile_fo<T, K, C::IK, C::NT>(L.sQ, C::LD, R.q);
    put_tile_fo<T, K, C::IK, C::NT>(L.sK, C::LD, R.k);
    put_tile<T, K, C::IK, C::NT>(L.sW, C::LD, R.w);
#pragma unroll
    for (int it = 0; it < C::IK; ++it) {
        const int e = (int)threadIdx.x + it * C::NT;
        const int r = e / C::NVK, cv = e % C::NVK;
        *reinterpret_cast<u32x4*>(L.sQs + r * C::LD + cv * C::VEC) = scale_vec<T>(R.q[it], scale * fast_exp(R.gq[it]));
    }
    put_tile<T, RT, C::ID, C::NT>(L.sD, C::LDD, R.d);
    if (threadIdx.x < 64) {
        // the chunk total is the last row's cumsum (rows past the chunk end repeat it)
        const float gtot = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(R.gam), 63));
        L.sGam[threadIdx.x] = R.gam;
        L.sEr[threadIdx.x] = fast_exp(gtot - R.gam);
    }
}

// kL2: q arrives raw and its rows are L2-normalised in registers before staging.
template <typename T, int K, int RT, int MODE, bool kL2 = false>
__global__ __launch_bounds__(RT * 4) void k_reverse(RevArgs a) {
    using C = VCfg<T, K, RT>;
    extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
    RevLds<T, K, RT> L;
    L.sQ = reinterpret_cast<T*>(smem + C::off_q);
    L.sQs = reinterpret_cast<T*>(smem + C::off_qs);
    L.sK = reinterpret_cast<T*>(smem + C::off_k);
    L.sW = reinterpret_cast<T*>(smem + C::off_w);
    L.sD = reinterpret_cast<T*>(smem + C::off_do);
    L.sPm = reinterpret_cast<T*>(smem + C::off_pm);
    L.sGam = reinterpret_cast<float*>(smem + C::off_gam);
    L.sEr = reinterpret_cast<float*>(smem + C::off_er);
    T* sDd = reinterpret_cast<T*>(smem + C::off_dd);

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
    const int row = vt * RT + wave * 16 + ln;
    const size_t VK = (size_t)V * K;

    f32x4 accG[K / 16];
    int cbeg = sg.c0, cend = sg.c1;  // processed from cend-1 down to cbeg
    int mode = 0;
    const bool last = sg.s == sg.nseg - 1;
    if (MODE == kRecurPrepass) {
        // As the forward's prepass, mirrored: heads whose boundaries all take the warmup (mode 1)
        // warm the adjoint leaving this segment over the window after it, into seginit; heads with
        // exact boundaries (mode 2, or 3 mixed) prepare the link from this segment to the one before
        // as a map G -> G M + R~ into prep: the exact map of this segment, or, where the boundary
        // at its start takes the warmup, M = 0 and R~ = the warm adjoint over the window after it.
        mode = a.modes[sg.n * H + h];
        int win = 0;
        if (mode == 1) {
            if (last || vt * RT >= V) return;
            win = a.bwin[(gs + 1) * H + h];  // the boundary at the start of the next segment
        } else if (mode == 2 || mode == 3) {
            if (sg.s == 0 || vt * RT >= V + K) return;
            win = mode == 3 ? a.bwin[gs * H + h] : 0;
        } else {
            return;
        }
        if (win > 0) {
            // the window starts where the boundary's segment starts; from a zero adjoint, or from
            // d(final state) when it reaches the sequence end
            const int cb = mode == 1 ? sg.c1 : sg.c0;
            cbeg = cb;
            cend = min(cb + win, sg.nchunks);
            if (vt * RT >= V) cend = cbeg;  // the M rows of a warm link (whole tiles): M = 0
            if (vt * RT < V && cend == sg.nchunks && a.dsT)
                load_state<K>(accG, a.dsT + ((size_t)sg.n * H + h) * VK, row);
            else
#pragma unroll
                for (int kt = 0; kt < K / 16; ++kt) accG[kt] = zero4();
        } else {
#pragma unroll
            for (int kt = 0; kt < K / 16; ++kt) {
                f32x4 z = zero4();
                if (row >= V) {
#pragma unroll
                    for (int i = 0; i < 4; ++i) z[i] = (kt * 16 + gq * 4 + i == row - V) ? 1.f : 0.f;
                }
                accG[kt] = z;
            }
        }
    } else {
        if (!last && a.use_cp) {
            load_state<K>(accG, a.seginit + ((size_t)gs * H + h) * VK, row);
        } else if (a.dsT) {
            load_state<K>(accG, a.dsT + ((size_t)sg.n * H + h) * VK, row);
        } else {
#pragma unroll
            for (int kt = 0; kt < K / 16; ++kt) accG[kt] = zero4();
        }
    }

    const bool has_do = vt * RT < V;  // M-hat rows of the exact prepass carry no output gradient
    const int dcol0 = has_do ? vt * RT : -1;
    // Operands are fetched in three pieces over each step: one chunk ahead in the output
    // pass, two (alternating buffers) in the prepass, which has little work per chunk.
    // Store data is held until the next chunk's staging (see hold()).
    constexpr int kDepth = MODE == kRecurPrepass ? 2 : 1;
    typedef typename Pack4<T>::type PV;
    constexpr int NFL = 64 * (RT / C::VEC) / C::NT;  // dDelta flush vectors per thread
    PV gkeep[K / 16];
    u32x4 fkeep[NFL];
#pragma unroll
    for (int i = 0; i < K / 16; ++i) gkeep[i] = PV{};
#pragma unroll
    for (int i = 0; i < NFL; ++i) fkeep[i] = u32x4{0u, 0u, 0u, 0u};
    RevRegs<T, K, RT> R0, R1;
    auto fetch_all = [&](RevRegs<T, K, RT>& R, int cn) {
        const int64_t tb = sg.bos + (int64_t)cn * 64;
        const int cb = min(64, sg.len - cn * 64);
        rev_fetch<0>(R, a, tb, cb, h, dcol0);
        rev_fetch<1>(R, a, tb, cb, h, dcol0);
        rev_fetch<2>(R, a, tb, cb, h, dcol0);
    };
    constexpr int NPT = (12 + C::NW - 1) / C::NW;  // P^T tiles per wave
    auto step = [&](RevRegs<T, K, RT>& R, const int ci) {
        const int64_t t0 = sg.bos + (int64_t)ci * 64;
#pragma unroll
        for (int i = 0; i < K / 16; ++i) hold(gkeep[i]);
#pragma unroll
        for (int i = 0; i < NFL; ++i) hold(fkeep[i]);
        if (MODE == kRecurOut) {
            // adjoint of the state leaving this chunk
            T* gs_out = reinterpret_cast<T*>(a.gstates) + ((size_t)(sg.choff + ci) * H + h) * VK + (size_t)row * K;
#pragma unroll
            for (int kt = 0; kt < K / 16; ++kt) gkeep[kt] = Pack4<T>::make(accG[kt]);
#pragma unroll
            for (int kt = 0; kt < K / 16; ++kt) *reinterpret_cast<PV*>(gs_out + kt * 16 + gq * 4) = gkeep[kt];
        }
        lds_sync();
        if (MODE == kRecurOut && a.ddelta && ci < cend - 1) {
            // the previous (later) chunk's dDelta
            T* dst = reinterpret_cast<T*>(a.ddelta) + ((t0 + 64) * H + h) * V + vt * RT;
            const int cp = min(64, sg.len - (ci + 1) * 64);
            constexpr int NV = RT / C::VEC;
#pragma unroll
            for (int it = 0; it < NFL; ++it) {
                const int u = (int)threadIdx.x + it * C::NT;
                fkeep[it] = *reinterpret_cast<const u32x4*>(sDd + (u / NV) * C::LDD + (u % NV) * C::VEC);
            }
#pragma unroll
            for (int it = 0; it < NFL; ++it) {
                const int u = (int)threadIdx.x + it * C::NT;
                if (u / NV < cp) *reinterpret_cast<u32x4*>(dst + (size_t)(u / NV) * H * V + (u % NV) * C::VEC) = fkeep[it];
            }
        }
        if constexpr (kL2) l2norm_rows<T, K>(R.q);
        rev_stage<T, K, RT>(R, L, a.scale);
        lds_sync();
        const int cn = max(ci - kDepth, cbeg);
        const int64_t tn = sg.bos + (int64_t)cn * 64;
        const int cnn = min(64, sg.len - cn * 64);
        rev_fetch<0>(R, a, tn, cnn, h, dcol0);

        Frag<T> gf[K / 32];
#pragma unroll
        for (int kb = 0; kb < K / 32; ++kb) frag_acc(gf[kb], accG[2 * kb], accG[2 * kb + 1]);
        const float Gm = L.sGam[63];
        f32x4 accD[4];
#pragma unroll
        for (int jt = 0; jt < 4; ++jt) accD[jt] = zero4();
        if constexpr (sizeof(T) == 2 && RT == 128) {
            // P^T[j][r] = e^{gam_r - gam_j} (Q K^T)[r][j] for r >= j (this wave's tiles, staged
            // row-major by j; none for the M rows of the exact prepass) and the Kt G^T part of the
            // dDelta tiles (rows j, columns = the wave's adjoint rows). Independent accumulators are
            // updated side by side (k32 slice outer, tiles inner) and each slice's fragments are
            // loaded before its products.
            f32x4 pacc[NPT];
            int prt[NPT], pjt[NPT];
            bool pon[NPT], pmm[NPT];
#pragma unroll
            for (int m = 0; m < NPT; ++m) {
                const int idx = wave + m * C::NW;
                pon[m] = has_do && idx < 12;
                prt[m] = pon[m] ? tri_row(idx) : 0;
                pjt[m] = pon[m] ? tri_col(idx) : 0;
                pmm[m] = pon[m] && pjt[m] <= prt[m];
                pacc[m] = zero4();
            }
            // bf16 with 128 adjoint rows: the P^T tiles take their K rows from the same k32
            // fragments as dDelta, in one pass
#pragma unroll
            for (int kb = 0; kb < K / 32; ++kb) {
                Frag<T> fk[4], fq[NPT];
#pragma unroll
                for (int jt = 0; jt < 4; ++jt) frag_row_fo(fk[jt], L.sK, C::LD, jt * 16 + ln, kb * 32);
#pragma unroll
                for (int m = 0; m < NPT; ++m)
                    if (pmm[m]) frag_row_fo(fq[m], L.sQ, C::LD, prt[m] * 16 + ln, kb * 32);
#pragma unroll
                for (int jt = 0; jt < 4; ++jt) mma(accD[jt], fk[jt], gf[kb]);
#pragma unroll
                for (int m = 0; m < NPT; ++m) {
                    if (pmm[m]) {
                        Frag<T> fb = fk[0];  // wave-uniform pick of the tile's K rows
                        if (pjt[m] == 1) fb = fk[1];
                        if (pjt[m] == 2) fb = fk[2];
                        if (pjt[m] == 3) fb = fk[3];
                        mma(pacc[m], fq[m], fb);  // lane holds [r = rt*16+gq*4+i][j = jt*16+ln]
                    }
                }
            }
#pragma unroll
            for (int m = 0; m < NPT; ++m) {
                if (pon[m]) {
                    const int j = pjt[m] * 16 + ln;
                    const float gj = L.sGam[j];
                    const f32x4 gr = *reinterpret_cast<const f32x4*>(L.sGam + prt[m] * 16 + gq * 4);
                    f32x4 v;
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int r = prt[m] * 16 + gq * 4 + i;
                        v[i] = (r >= j) ? a.scale * pacc[m][i] * fast_exp(gr[i] - gj) : 0.f;
                    }
                    store4(L.sPm + j * C::LDP + frag_pos(prt[m] * 16 + gq * 4), v);  // fragment order
                }
            }
        } else {
            // Independent accumulators are updated side by side (k32 slice outer, tiles inner)
            // and each slice's fragments are loaded before its products.
            if (has_do) {
                // P^T[j][r] = e^{gam_r - gam_j} (Q K^T)[r][j] for r >= j, staged row-major by j
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
                            frag_row_fo(fa[m], L.sQ, C::LD, prt[m] * 16 + ln, kb * 32);
                            frag_row_fo(fb[m], L.sK, C::LD, pjt[m] * 16 + ln, kb * 32);
                        }
                    }
#pragma unroll
                    for (int m = 0; m < NPT; ++m)
                        if (pmm[m]) mma(pacc[m], fa[m], fb[m]);  // lane holds [r = rt*16+gq*4+i][j = jt*16+ln]
                }
#pragma unroll
                for (int m = 0; m < NPT; ++m) {
                    if (pon[m]) {
                        const int j = pjt[m] * 16 + ln;
                        const float gj = L.sGam[j];
                        const f32x4 gr = *reinterpret_cast<const f32x4*>(L.sGam + prt[m] * 16 + gq * 4);
                        f32x4 v;
#pragma unroll
                        for (int i = 0; i < 4; ++i) {
                            const int r = prt[m] * 16 + gq * 4 + i;
                            v[i] = (r >= j) ? a.scale * pacc[m][i] * fast_exp(gr[i] - gj) : 0.f;
                        }
                        store4(L.sPm + j * C::LDP + frag_pos(prt[m] * 16 + gq * 4), v);  // fragment order
                    }
                }
            }
            // dDelta tiles (rows j, columns = the wave's adjoint rows): Kt G^T part
#pragma unroll
            for (int kb = 0; kb < K / 32; ++kb) {
                Frag<T> fa[4];
#pragma unroll
                for (int jt = 0; jt < 4; ++jt) frag_row_fo(fa[jt], L.sK, C::LD, jt * 16 + ln, kb * 32);
#pragma unroll
                for (int jt = 0; jt < 4; ++jt) mma(accD[jt], fa[jt], gf[kb]);
            }
        }
#pragma unroll
        for (int jt = 0; jt < 4; ++jt) accD[jt] *= *reinterpret_cast<const f32x4*>(L.sEr + jt * 16 + gq * 4);
        rev_fetch<1>(R, a, tn, cnn, h, dcol0);
        // bf16: dO and the gate cumsum too (every chunk's loads land together in one burst
        // across the chip, so the last piece needs most of a step to arrive); fp32, whose
        // operands take twice the registers, at the end of the step
        if constexpr (sizeof(T) == 2) rev_fetch<2>(R, a, tn, cnn, h, dcol0);
        lds_sync();  // P^T complete
        if (has_do) {
#pragma unroll
            for (int rb = 0; rb < 2; ++rb) {
                Frag<T> fb, fa[4];
                frag_col(fb, L.sD, C::LDD, wave * 16 + ln, rb * 32);  // dO column v, slots r
#pragma unroll
                for (int jt = 0; jt <= 2 * rb + 1; ++jt) frag_row_fo(fa[jt], L.sPm, C::LDP, jt * 16 + ln, rb * 32);
#pragma unroll
                for (int jt = 0; jt <= 2 * rb + 1; ++jt) mma(accD[jt], fa[jt], fb);
            }
        }
        if (MODE == kRecurOut && a.ddelta) {
            // dDelta (= dU) for the per-chunk gradients, staged [64][RT] by row j and
            // written out after the next chunk's first barrier
#pragma unroll
            for (int jt = 0; jt < 4; ++jt) put_col4(sDd + (jt * 16 + gq * 4) * C::LDD + wave * 16 + ln, C::LDD, accD[jt]);
        }
        // G^T <- e^Gam G^T + (e^gam Q)^T dO - W^T dDelta
        const float eG = fast_exp(Gm);
        Frag<T> ddf[2];
        frag_acc(ddf[0], accD[0], accD[1], -1.f);
        frag_acc(ddf[1], accD[2], accD[3], -1.f);
        Frag<T> dof[2];
        if (has_do) {
#pragma unroll
            for (int rb = 0; rb < 2; ++rb) frag_col(dof[rb], L.sD, C::LDD, wave * 16 + ln, rb * 32);
        }
#pragma unroll
        for (int kt = 0; kt < K / 16; ++kt) accG[kt] *= eG;
#pragma unroll
        for (int jb = 0; jb < 2; ++jb) {
            Frag<T> fw[K / 16];
#pragma unroll
            for (int kt = 0; kt < K / 16; ++kt) frag_col(fw[kt], L.sW, C::LD, kt * 16 + ln, jb * 32);  // W^T row k, slots j
#pragma unroll
            for (int kt = 0; kt < K / 16; ++kt) mma(accG[kt], fw[kt], ddf[jb]);
            if (has_do) {
                Frag<T> fq[K / 16];
#pragma unroll
                for (int kt = 0; kt < K / 16; ++kt)
                    frag_col(fq[kt], L.sQs, C::LD, kt * 16 + ln, jb * 32);  // (scale e^gam Q)^T row k, slots r
#pragma unroll
                for (int kt = 0; kt < K / 16; ++kt) mma(accG[kt], fq[kt], dof[jb]);
            }
        }
        if constexpr (sizeof(T) != 2) rev_fetch<2>(R, a, tn, cnn, h, dcol0);
    };
    // the entering adjoint may come from a load: wait for it before any prefetch
#pragma unroll
    for (int kt = 0; kt < K / 16; ++kt) hold(accG[kt]);
    if constexpr (kDepth == 2) {
        // pairs of chunks without a branch between them (see the forward recurrence), then
        // the first chunk
        if (cbeg < cend) {
            fetch_all(R0, cend - 1);
            fetch_all(R1, max(cend - 2, cbeg));
        }
        int ci = cend - 1;
        for (; ci - 1 >= cbeg; ci -= 2) {
            step(R0, ci);
            step(R1, ci - 1);
        }
        if (ci >= cbeg) step(R0, ci);
    } else {
        if (cbeg < cend) fetch_all(R0, cend - 1);
        for (int ci = cend - 1; ci >= cbeg; --ci) step(R0, ci);
    }

    if (MODE == kRecurOut && a.ddelta && cbeg < cend) {
        lds_sync();
        flush_tile<T, RT, C::NT>(reinterpret_cast<T*>(a.ddelta) + ((sg.bos + (int64_t)cbeg * 64) * H + h) * V + vt * RT,
                                 (size_t)H * V, min(64, sg.len - cbeg * 64), sDd, C::LDD);
    }
    if (MODE == kRecurPrepass) {
        if (mode == 1) {
            store_state<K>(accG, a.seginit_out + ((size_t)(gs - 0) * H + h) * VK, row);
        } else {
            float* P = a.prep + ((size_t)gs * H + h) * (size_t)(V + K) * K;
            if (row < V) {
                store_state<K>(accG, P, row);
            } else if (row < V + K) {
                // M^T in the input precision after the R rows, rows in fragment order, as the
                // forward's prepass
                const int i = frag_pos(row - V);
                T* Mt = reinterpret_cast<T*>(P + VK);
#pragma unroll
                for (int kt = 0; kt < K / 16; ++kt)
#pragma unroll
                    for (int e = 0; e < 4; ++e) Mt[(size_t)(kt * 16 + gq * 4 + e) * K + i] = Elem<T>::from_f(accG[kt][e]);
            }
        }
    } else if (sg.s == 0 && a.ds0) {
        store_state<K>(accG, a.ds0 + ((size_t)sg.n * H + h) * VK, row);
    }
}

template <typename T, int K, int RT, int MODE>
hipError_t launch_reverse_t(const RevArgs& a, int64_t nsegs_grid, int vtiles, hipStream_t st) {
    using C = VCfg<T, K, RT>;
    static_assert(C::total <= 160 * 1024, "LDS budget");
    auto kern = a.q_l2 ? k_reverse<T, K, RT, MODE, true> : k_reverse<T, K, RT, MODE, false>;
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, C::total);
    if (e != hipSuccess) return e;
    // the prepass's ranked one-dimensional grid (see prepass_item), the varlen segment order's
    // (see ordered_seg_item), else (segments, heads, row tiles)
    const dim3 grid = MODE == kRecurPrepass && a.ranked
                          ? dim3((unsigned)((int64_t)vtiles * a.geo.nseg * a.geo.N * a.geo.H), 1u, 1u)
                      : MODE != kRecurPrepass && a.geo.seg_order
                          ? dim3((unsigned)(nsegs_grid * a.geo.H * vtiles), 1u, 1u)
                          : dim3((unsigned)nsegs_grid, (unsigned)a.geo.H, (unsigned)vtiles);
    hipLaunchKernelGGL(kern, grid, dim3(C::NT), C::total, st, a);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Per-chunk gradients: the state side, then the WY side, in one kernel. A persistent
// workgroup (8 waves, one per CU) walks the (chunk, head) tasks; the next task's operands
// travel into registers while the current task computes, so HBM traffic overlaps the
// work instead of alternating with it.
//
// Delta = U - W S^T comes from the state pass and dDelta (= dU) from the reverse pass,
// both of which form them anyway; with them, every state-side product contracts over
// the value dimension:
//   dQt = dO S, dW = -dDelta S     (S read as column slices: waves w, w+4 own k in
//                                   [K/4 w, K/4 (w+1)) and split the chunk-row tiles)
//   dKt = Delta G, dP = dO Delta^T (waves w, w+4 own chunk rows of one 16-row tile each and split
//                                   the tiles along the other dimension)
// so no partial sums over k cross waves. Most tiles are
// held transposed (rows over k or chunk rows, columns over r), which makes them A
// fragments of their transposes and lets every lane write four consecutive columns of
// its row with one vector store.
//
// LDS: every tile that is read as row fragments (all but S, G and Y) is stored with its
// rows in fragment order (frag_pos): one 16-byte read per bf16 row fragment, and the
// transposed reads of the same tiles go through frag_col_fo. K stays for both sides. The
// state side holds S, G, Q, scale * dO, Delta and dDelta
// (the L .* dP exchange later goes over Delta). dDelta is the WY side's dU as it stands;
// dW goes over S once the state side ends, and V, T and two 64x64 scratch matrices of
// the WY side go into the rest of that space (the hole between dW and dDelta first, then
// past dDelta).
struct WyPlace {
    int off[5];  // V, T, Y, Mx, dT
    int end;
};
constexpr WyPlace place_wy(int h0, int h1, int tail, int vmat, int xmat) {
    WyPlace p{};
    int cur = h0, tl = tail;
    for (int i = 0; i < 5; ++i) {
        const int s = i == 0 ? vmat : xmat;
        if (cur + s <= h1) {
            p.off[i] = cur;
            cur += s;
        } else {
            p.off[i] = tl;
            tl += s;
        }
    }
    p.end = tl;
    return p;
}

template <typename T, int K, int V>
struct BCfg {
    static constexpr int VEC = Elem<T>::kVec;
    static constexpr int LDK = (K == 128 && V == 128) ? K + BPadK<T>::row : K + BPad<T>::row;
    static constexpr int LDS = K + BPad<T>::row;
    static constexpr int LDV = V + BPad<T>::row;
    static constexpr int LDX = (K == 128 && V == 128) ? 64 + BPadK<T>::row : 64 + BPad<T>::row;
    static constexpr int kMK = 64 * LDK * (int)sizeof(T);  // one [64][K] matrix
    static constexpr int LDU = LDV;  // dDelta
    static constexpr int kMV = 64 * LDV * (int)sizeof(T);  // one [64][V] matrix
    static constexpr int kMU = 64 * LDU * (int)sizeof(T);  // the dDelta tile
    static constexpr int kMX = 64 * LDX * (int)sizeof(T);  // one [64][64] matrix
    static constexpr int kSt = V * LDS * (int)sizeof(T);   // one [V][K] state
    static constexpr int off_k = 0;
    // state side
    static constexpr int off_s = kMK;
    static constexpr int off_g = off_s + kSt;
    static constexpr int off_q = off_g + kSt;
    static constexpr int off_d = off_q + kMK;    // scale * dO
    static constexpr int off_dl = off_d + kMV;   // Delta, then the L .* dP exchange
    static constexpr int off_x = off_dl;
    static constexpr int off_dd = off_dl + kMV;  // dDelta (the WY side's dU)
    static constexpr int end_state = off_dd + kMU;
    // WY side
    static constexpr int off_dw = off_s;
    static constexpr WyPlace wy = place_wy(off_dw + kMK, off_dd, end_state, kMV, kMX);
    static constexpr int off_v = wy.off[0];
    static constexpr int off_tm = wy.off[1];  // T = (I + A)^{-1}
    static constexpr int off_y = wy.off[2];   // Y = dT T^T
    static constexpr int off_mx = wy.off[3];  // Mx = dA .* (beta_a e^{gam_a - gam_c})
    static constexpr int off_dt = wy.off[4];  // dT, exchanged between the two wave halves
    // small arrays after both
    static constexpr int off_gam = end_state > wy.end ? end_state : wy.end;
    static constexpr int off_beta = off_gam + 256;
    static constexpr int off_red = off_beta + 256;  // [4][64] fp32 column partials
    static constexpr int off_row = off_red + 1024;  // [2][64] fp32 row parts (one per wave half)
    static constexpr int off_qd = off_row + 512;    // [4][64] e^gam dQt . Q partials over k slices
    static constexpr int off_dgs = off_qd + 1024;   // [64] state-side d(gam)
    static constexpr int off_sc = off_dgs + 256;    // [16] fp32 scalars (two per wave)
    static constexpr int off_db = off_sc + 64;      // [2][64] fp32 dbeta parts (one per wave half)
    static constexpr int off_eg = off_db + 512;     // [64] e^{gam_r}
    static constexpr int off_er = off_eg + 256;     // [64] e^{Gam - gam_r}
    static constexpr int total = off_er + 256;
    // Where the WY side leaves a hole between its last matrix (dT) and dDelta large enough (bf16 at
    // K = V = 128: the state side's Q, dO and Delta tiles, dead once the state side ends), dq
    // and then dk and dv are staged there ([64][K + 8], row-major) and stored as whole rows.
    static constexpr int LDG = K + BPad<T>::row;
    static constexpr int kMG = 64 * LDG * (int)sizeof(T);
    static constexpr int off_gst = wy.off[4] + kMX;  // past dT
    static constexpr bool stage_grads = sizeof(T) == 2 && K == V && wy.end == end_state &&
                                        off_gst >= off_q && off_gst + 2 * kMG <= off_dd;
    static_assert(LDX <= LDV, "the exchange fits over Delta");
    static_assert(kMK <= kSt, "dW fits over S");
    // eight waves; 16-byte vectors per thread of one task's operands
    static constexpr int NT = 512;
    static constexpr int NS = V * (K / VEC) / NT;    // S or G
    static constexpr int NK = 64 * (K / VEC) / NT;   // q, k
    static constexpr int NV = 64 * (V / VEC) / NT;   // dO, Delta, dDelta, v
    static constexpr int NX = 64 * (64 / VEC) / NT;  // T
    static_assert(NS * NT == V * (K / VEC) && NK * NT == 64 * (K / VEC) && NV * NT == 64 * (V / VEC) &&
                      NX * NT == 64 * (64 / VEC),
                  "vector split");
};

// One task's operands in registers, in the two groups that are fetched at different
// points of the previous task: the chunk rows (q, k, dO, Delta, dDelta, T, gate cumsum,
// beta), then S, G and v.
template <typename T, int K, int V, bool kCarry>
struct BRegs {
    using C = BCfg<T, K, V>;
    // with the adjoint carried in the kernel, G and dDelta are formed here instead of loaded
    u32x4 q[C::NK], k[C::NK], d[C::NV], dl[C::NV], dd[kCarry ? 1 : C::NV];
    u32x4 s[C::NS], g[kCarry ? 1 : C::NS];
    float gam, beta;
};

// The next task's operands travel in small groups issued at different points of the
// current task's WY side: a burst of all of them would stall the issuing waves on the
// CU's load queue instead of draining behind the matrix work.
template <int kGroup, typename T, int K, int V, bool kCarry>
__device__ __forceinline__ void bwd_fetch(BRegs<T, K, V, kCarry>& R, const BwdChunkArgs& a, const ChunkTask& x) {
    using C = BCfg<T, K, V>;
    const int64_t H = a.geo.H;
    const size_t ok = ((size_t)x.t0 * H + x.h) * K, ov = ((size_t)x.t0 * H + x.h) * V;
    const size_t st = ((size_t)x.gc * H + x.h) * (size_t)V * K;
    if constexpr (kGroup == 0) {
        fetch_tile<T, K, C::NK, C::NT>(R.q, reinterpret_cast<const T*>(a.q) + ok, (size_t)H * K, x.c);
        fetch_tile<T, K, C::NK, C::NT>(R.k, reinterpret_cast<const T*>(a.k) + ok, (size_t)H * K, x.c);
        const int tid = threadIdx.x;
        if (tid < 64) {
            const bool in = tid < x.c;
            R.gam = a.gam[(x.t0 + (in ? tid : x.c - 1)) * H + x.h];
            R.beta = in ? a.beta[(x.t0 + tid) * H + x.h] : 0.f;
        }
    } else if constexpr (kGroup == 1) {
        fetch_tile<T, V, C::NV, C::NT>(R.d, reinterpret_cast<const T*>(a.d_o) + ov, (size_t)H * V, x.c);
    } else if constexpr (kGroup == 2) {
        fetch_tile<T, V, C::NV, C::NT>(R.dl, reinterpret_cast<const T*>(a.delta) + ov, (size_t)H * V, x.c);
        if constexpr (!kCarry)
            fetch_tile<T, V, C::NV, C::NT>(R.dd, reinterpret_cast<const T*>(a.ddelta) + ov, (size_t)H * V, x.c);
    } else if constexpr (kGroup == 3) {
        fetch_tile<T, K, C::NS, C::NT>(R.s, reinterpret_cast<const T*>(a.hstates) + st, K, V);
    } else {
        if constexpr (!kCarry)
            fetch_tile<T, K, C::NS, C::NT>(R.g, reinterpret_cast<const T*>(a.gstates) + st, K, V);
    }
}

// v and T of the task being processed, loaded during its state side for its WY side.
template <typename T, int K, int V>
struct VTRegs {
    using C = BCfg<T, K, V>;
    u32x4 v[C::NV], t[C::NX];
};
template <typename T, int K, int V>
__device__ __forceinline__ void bwd_fetch_vt(VTRegs<T, K, V>& R, const BwdChunkArgs& a, const ChunkTask& x) {
    using C = BCfg<T, K, V>;
    const int64_t H = a.geo.H;
    fetch_tile<T, V, C::NV, C::NT>(R.v, reinterpret_cast<const T*>(a.v) + ((size_t)x.t0 * H + x.h) * V,
                                   (size_t)H * V, x.c);
    fetch_tile<T, 64, C::NX, C::NT>(R.t, reinterpret_cast<const T*>(a.tmat) + ((size_t)x.gc * H + x.h) * 4096, 64,
                                    64);
}

// Four consecutive LDS elements as fp32.
__device__ __forceinline__ f32x4 ld4(const bf16_t* p) {
    const u32x2 x = *reinterpret_cast<const u32x2*>(p);
    return f32x4{__uint_as_float(x.x << 16), __uint_as_float(x.x & 0xFFFF0000u), __uint_as_float(x.y << 16),
                 __uint_as_float(x.y & 0xFFFF0000u)};
}
__device__ __forceinline__ f32x4 ld4(const float* p) { return *reinterpret_cast<const f32x4*>(p); }

// x.lo * y.lo + x.hi * y.hi + acc for two packed bf16 pairs (one v_dot2 instruction)
__device__ __forceinline__ float dot2_bf16(uint32_t x, uint32_t y, float acc) {
    typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, x), __builtin_bit_cast(bf16x2_t, y), acc,
                                           false);
}

__device__ __forceinline__ float dot4(const f32x4& a, const f32x4& b) {
    return a[0] * b[0] + a[1] * b[1] + a[2] * b[2] + a[3] * b[3];
}

// Sum over the four lanes that share ln (lane groups gq = 0..3).
__device__ __forceinline__ float sum_gq(float x) { return sum_rows(x); }

// Per-slot scaling of a bf16 fragment by a per-row factor f (in LDS): slot e of lane group gq is
// row k0 + kappa(gq, e) of the contraction and gets f[k0 + kappa(gq, e)].
__device__ __forceinline__ Frag<bf16_t> scale_slots(const Frag<bf16_t>& x, const float* f, int k0) {
    const int gq = threadIdx.x >> 4 & 3;
    const f32x4 a = *reinterpret_cast<const f32x4*>(f + k0 + gq * 4);
    const f32x4 b = *reinterpret_cast<const f32x4*>(f + k0 + 16 + gq * 4);
    Frag<bf16_t> o;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const f32x4& y = i < 2 ? a : b;  // u32 i holds slots 2i, 2i+1
        const int e = (i & 1) * 2;
        o.v[i] = pack_bf2(__uint_as_float(x.v[i] << 16) * y[e], __uint_as_float(x.v[i] & 0xFFFF0000u) * y[e + 1]);
    }
    return o;
}


// kL2: q arrives raw and its rows are L2-normalised in registers before staging (dq is then
// the gradient with respect to the normalised rows).
//
// kCarry: the reverse adjoint recurrence runs inside this kernel. One workgroup per
// (sub-sequence, head) walks its chunks from the last to the first and keeps G, the adjoint of
// the state leaving the chunk, as fp32 accumulator tiles of G^T (wave w: value rows 16w ..
// 16w+15, every k; V = 128), from the sub-sequence's entering adjoint (d(final state), or the
// reverse CP's). Each task then forms what the adjoint pass would have stored:
//   dDelta = P^T (scale dO) + diag(e^{Gam-gam}) K G^T          (P = L .* Q K^T)
// and afterwards the adjoint entering the chunk, which the next task (the chunk before) uses:
//   G <- e^Gam G + (e^gam Q)^T (scale dO) - W^T dDelta,   W^T dDelta = K^T diag(beta e^gam) dBv
// with dBv = T^T dDelta from the WY side (W = T diag(beta e^gam) K), so W itself is never needed.
// No adjoint pass, no per-chunk adjoint or dDelta round trip through memory.
template <typename T, int K, int V, bool kL2 = false, bool kCarry = false>
__global__ __launch_bounds__(512) void k_bwd_chunk(BwdChunkArgs a) {
    using C = BCfg<T, K, V>;
    constexpr int NT = C::NT;
    static_assert(!kCarry || (V == 128 && sizeof(T) == 2), "the carried adjoint: one 16-row value tile per wave");
    extern __shared__ __attribute__((aligned(16))) unsigned char smem[];

    const Geo& geo = a.geo;
    const int64_t H = geo.H;
    const int64_t ntasks = geo.total_chunks * H;
    const int tid = threadIdx.x;
    const int wave = wave_id(), lane = tid & 63, ln = lane & 15, gq = lane >> 4;
    // Wave w + 4 hf (half hf) takes, in the row-split products, the chunk rows of row tile rt
    // (w for the first half, 3 - w for the second) and splits the tiles along the other
    // dimension with the other half: half hf takes the j, c, b tiles 2hf, 2hf+1, the k tiles
    // hf*K/32 .., the v tiles hf*V/32 .. and, in the column-split products, the row tiles 2hf,
    // 2hf+1 of its k slice. The mirrored row tiles of the second half make the two waves on one
    // SIMD share the causal triangle's tiles evenly: nlive of a wave's two j (b) tiles lie on
    // or below the diagonal, and the P / dP and dT products compute only those (a branch on the
    // count, wave-uniform).
    const int w = wave & 3, hf = wave >> 2;
    const int rt = hf ? 3 - w : w;
    const int nlive = (2 * hf <= rt) + (2 * hf + 1 <= rt);
    const int r = rt * 16 + ln;    // this lane's chunk row in "column" roles
    constexpr int KW = K / 64;     // k tiles (of 16) per k slice in the column-split products
    constexpr int KH = K / 32;     // k tiles per half
    constexpr int VH = V / 32;     // v tiles per half

    ChunkTask cur;
    int64_t t = 0;
    // kCarry: this workgroup's sub-sequence and head, walked from chunk sg.c1 - 1 down to sg.c0
    SegLoc sg;
    int64_t gseg = 0;
    int hc = 0;
    f32x4 accG[kCarry ? K / 16 : 1];  // G^T: rows k (tile kt), columns v = wave * 16 + ln
    const int vrow = wave * 16 + ln;
    const size_t VK = (size_t)V * K;
    auto seg_task = [&](int ci, ChunkTask& x) {
        x.gc = sg.choff + ci;
        x.t0 = sg.bos + (int64_t)ci * 64;
        x.h = hc;
        x.c = min(64, sg.len - ci * 64);
    };
    if constexpr (kCarry) {
        gseg = blockIdx.x / H;
        hc = (int)(blockIdx.x - gseg * H);
        if (!locate_seg(geo, gseg, sg)) return;
        if (sg.s < sg.nseg - 1 && a.use_cp)
            load_state<K>(accG, a.seginit_r + ((size_t)gseg * H + hc) * VK, vrow);
        else if (a.dsT)
            load_state<K>(accG, a.dsT + ((size_t)sg.n * H + hc) * VK, vrow);
        else
#pragma unroll
            for (int kt = 0; kt < K / 16; ++kt) accG[kt] = zero4();
        // the entering adjoint may come from a load: wait for it before any prefetch
#pragma unroll
        for (int kt = 0; kt < K / 16; ++kt) hold(accG[kt]);
        if (sg.c1 <= sg.c0) {  // no chunks: the adjoint passes through
            if (sg.s == 0 && a.ds0) store_state<K>(accG, a.ds0 + ((size_t)sg.n * H + hc) * VK, vrow);
            return;
        }
        t = sg.c1 - 1;
        seg_task((int)t, cur);
    } else {
        t = next_chunk_task(geo, blockIdx.x, ntasks, cur);
        if (t >= ntasks) return;
    }
    BRegs<T, K, V, kCarry> R;  // the next task's operands
    VTRegs<T, K, V> RV;  // v and T of this task
    bwd_fetch<0>(R, a, cur);
    bwd_fetch<1>(R, a, cur);
    bwd_fetch<2>(R, a, cur);
    bwd_fetch<3>(R, a, cur);
    bwd_fetch<4>(R, a, cur);

    for (;;) {
        // The LDS pointers are formed anew each task from an offset the compiler cannot see
        // through (it is zero): otherwise it hoists every per-lane LDS address out of the
        // loop and keeps dozens of them live (and spilled) across the whole task.
        int zero_off = 0;
        asm volatile("" : "+s"(zero_off));
        unsigned char* sm = smem + zero_off;
        T* sK = reinterpret_cast<T*>(sm + C::off_k);
        T* sS = reinterpret_cast<T*>(sm + C::off_s);
        T* sG = reinterpret_cast<T*>(sm + C::off_g);
        T* sQ = reinterpret_cast<T*>(sm + C::off_q);
        T* sD = reinterpret_cast<T*>(sm + C::off_d);
        T* sDl = reinterpret_cast<T*>(sm + C::off_dl);
        T* sX = reinterpret_cast<T*>(sm + C::off_x);
        T* sdU = reinterpret_cast<T*>(sm + C::off_dd);
        T* sdW = reinterpret_cast<T*>(sm + C::off_dw);
        T* sV = reinterpret_cast<T*>(sm + C::off_v);
        T* sTm = reinterpret_cast<T*>(sm + C::off_tm);
        T* sY = reinterpret_cast<T*>(sm + C::off_y);
        T* sMx = reinterpret_cast<T*>(sm + C::off_mx);
        T* sDT = reinterpret_cast<T*>(sm + C::off_dt);
        float* sGam = reinterpret_cast<float*>(sm + C::off_gam);
        float* sBeta = reinterpret_cast<float*>(sm + C::off_beta);
        float* sRed = reinterpret_cast<float*>(sm + C::off_red);
        float* sRow = reinterpret_cast<float*>(sm + C::off_row);
        float* sQd = reinterpret_cast<float*>(sm + C::off_qd);
        float* sDgs = reinterpret_cast<float*>(sm + C::off_dgs);
        float* sSc = reinterpret_cast<float*>(sm + C::off_sc);
        float* sDb = reinterpret_cast<float*>(sm + C::off_db);
        float* sEg = reinterpret_cast<float*>(sm + C::off_eg);
        float* sEr = reinterpret_cast<float*>(sm + C::off_er);
        // ---- stage this task (the previous task's LDS reads are done) ---------------------
        lds_sync();
        if constexpr (kL2) l2norm_rows<T, K>(R.q);
        put_tile_fo<T, K, C::NK, NT>(sQ, C::LDK, R.q);
        put_tile_fo<T, K, C::NK, NT>(sK, C::LDK, R.k);
        // dO enters every product together with the query scale (o = scale S q)
        // scale * dO and Delta are read as row fragments only: rows in fragment order
        put_tile_fo<T, V, C::NV, NT>(sD, C::LDV, R.d, a.scale);
        put_tile_fo<T, V, C::NV, NT>(sDl, C::LDV, R.dl);
        if constexpr (!kCarry) put_tile_fo<T, V, C::NV, NT>(sdU, C::LDU, R.dd);
        if (tid < 64) {
            // the decay factors that depend on one row only, once per chunk (the chunk total
            // Gam is the last row's cumsum)
            const float gtot = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(R.gam), 63));
            sGam[tid] = R.gam;
            sBeta[tid] = R.beta;
            sEg[tid] = fast_exp(R.gam);
            sEr[tid] = fast_exp(gtot - R.gam);
        }
        lds_sync();
        // The last task fetches itself again: unconditional fetches end the previous
        // operands' live range at the staging above.
        ChunkTask nxt = cur;
        int64_t tn;
        bool more;
        if constexpr (kCarry) {
            tn = t - 1;  // the chunk before
            more = tn >= sg.c0;
            if (more) seg_task((int)tn, nxt);
        } else {
            tn = next_chunk_task(geo, t + gridDim.x, ntasks, nxt);
            more = tn < ntasks;
            if (!more) nxt = cur;
        }

        const int c = cur.c;
        const int64_t t0 = cur.t0;
        const int h = cur.h;
        const float Gm = sGam[63];
        const float gr = sGam[r];
        const float ekt = sEr[r];

        // ======================= state side, rows r of this wave =======================
        // ---- P (rows j, cols r) and dP^T[j][r] = sum_v Delta[j][v] dO[r][v], this half's j tiles
        f32x4 dPT[2], PmQ[2];
        {
            Frag<T> qr[K / 32], dor[V / 32];
#pragma unroll
            for (int kb = 0; kb < K / 32; ++kb) frag_row_fo(qr[kb], sQ, C::LDK, r, kb * 32);
#pragma unroll
            for (int vb = 0; vb < V / 32; ++vb) frag_row_fo(dor[vb], sD, C::LDV, r, vb * 32);
            // the live j tiles (the mask below zeroes j > r within them): one straight block of
            // independent products per tile count
#pragma unroll
            for (int m = 0; m < 2; ++m) {
                dPT[m] = zero4();
                PmQ[m] = zero4();
            }
            auto products = [&](auto nm_) {
                constexpr int NM = decltype(nm_)::value;
#pragma unroll
                for (int vb = 0; vb < V / 32; ++vb) {
                    Frag<T> fd[NM];
#pragma unroll
                    for (int m = 0; m < NM; ++m) frag_row_fo(fd[m], sDl, C::LDV, (2 * hf + m) * 16 + ln, vb * 32);
#pragma unroll
                    for (int m = 0; m < NM; ++m) mma(dPT[m], fd[m], dor[vb]);
                }
#pragma unroll
                for (int kb = 0; kb < K / 32; ++kb) {
                    Frag<T> fk[NM];
#pragma unroll
                    for (int m = 0; m < NM; ++m) frag_row_fo(fk[m], sK, C::LDK, (2 * hf + m) * 16 + ln, kb * 32);
#pragma unroll
                    for (int m = 0; m < NM; ++m) mma(PmQ[m], fk[m], qr[kb]);
                }
            };
            if (nlive == 2)
                products(std::integral_constant<int, 2>{});
            else if (nlive == 1)
                products(std::integral_constant<int, 1>{});
        }
        // kCarry: P[r][j] = e^{gam_r - gam_j} (Q K^T)[r][j] (j <= r) for dDelta, staged over the
        // dDelta tile (rows r, fragment order) until dDelta replaces it
        T* sPr = sdU;
        // the causal decay e^{gam_r - gam_j} (0 for j > r) of this lane's P entries, used here and
        // for L .* dP below
        f32x4 dec[2];
#pragma unroll
        for (int m = 0; m < 2; ++m) {
            const int jt = 2 * hf + m;
            const f32x4 gj = ld4(sGam + jt * 16 + gq * 4);
#pragma unroll
            for (int i = 0; i < 4; ++i) dec[m][i] = (jt <= rt && jt * 16 + gq * 4 + i <= r) ? fast_exp(gr - gj[i]) : 0.f;
        }
        if constexpr (kCarry) {
#pragma unroll
            for (int m = 0; m < 2; ++m) {
                const int jt = 2 * hf + m;
                store4(sPr + r * C::LDX + frag_pos(jt * 16 + gq * 4), PmQ[m] * dec[m]);
            }
        }
        // S and G are fetched last in the previous task and staged only here, so that their
        // registers are free over that task's WY side and their loads land behind the products above
        // (kCarry: G from its accumulators, rows v = this wave's 16 value rows)
        put_tile<T, K, C::NS, NT>(sS, C::LDS, R.s);
        if constexpr (kCarry) {
#pragma unroll
            for (int kt = 0; kt < K / 16; ++kt) store4(sG + vrow * C::LDS + kt * 16 + gq * 4, accG[kt]);
        } else {
            put_tile<T, K, C::NS, NT>(sG, C::LDS, R.g);
        }
        lds_sync();
        // kCarry: dDelta^T tiles [v = this wave's rows][j] (stored after the next barrier, once
        // every wave has read P), then the first part of the adjoint update
        f32x4 ddT[kCarry ? 4 : 1];
        if constexpr (kCarry) {
            Frag<T> gfr[K / 32];
#pragma unroll
            for (int kb = 0; kb < K / 32; ++kb) frag_acc(gfr[kb], accG[2 * kb], accG[2 * kb + 1]);  // G rows v, slots k
            // diag(e^{Gam-gam_j}) K G^T, column j of each tile
#pragma unroll
            for (int jt = 0; jt < 4; ++jt) {
                ddT[jt] = zero4();
                Frag<T> fk[K / 32];
#pragma unroll
                for (int kb = 0; kb < K / 32; ++kb) frag_row_fo(fk[kb], sK, C::LDK, jt * 16 + ln, kb * 32);  // K row j
#pragma unroll
                for (int kb = 0; kb < K / 32; ++kb) mma(ddT[jt], gfr[kb], fk[kb]);
                ddT[jt] *= sEr[jt * 16 + ln];
            }
            // + (scale dO)^T P: contraction over the chunk rows r >= j
            Frag<T> dof[2];
#pragma unroll
            for (int rb = 0; rb < 2; ++rb) frag_col_fo(dof[rb], sD, C::LDV, vrow, rb * 32);  // scale dO column v, slots r
#pragma unroll
            for (int jt = 0; jt < 4; ++jt) {
#pragma unroll
                for (int rb = jt >> 1; rb < 2; ++rb) {
                    Frag<T> fp;
                    frag_col_fo(fp, sPr, C::LDX, jt * 16 + ln, rb * 32);  // P column j, slots r
                    mma(ddT[jt], dof[rb], fp);
                }
            }
            // G^T <- e^Gam G^T + Q^T diag(e^gam) (scale dO)  (the rest after the WY side)
            const float eG = fast_exp(Gm);
            Frag<T> dos[2];
#pragma unroll
            for (int rb = 0; rb < 2; ++rb) dos[rb] = scale_slots(dof[rb], sEg, rb * 32);
#pragma unroll
            for (int kt = 0; kt < K / 16; ++kt) {
                accG[kt] *= eG;
#pragma unroll
                for (int rb = 0; rb < 2; ++rb) {
                    Frag<T> fq;
                    frag_col_fo(fq, sQ, C::LDK, kt * 16 + ln, rb * 32);  // Q column k, slots r
                    mma(accG[kt], fq, dos[rb]);
                }
            }
        }
        // e^Gam <G, S> over the whole state (each thread a slice; in bf16 two products per
        // instruction, exact in fp32, with fp32 accumulation)
        float gs = 0.f;
        {
            constexpr int VEC = Elem<T>::kVec;
#pragma unroll 4
            for (int e = tid; e < V * K / VEC; e += NT) {
                const int vv = e / (K / VEC), kk = (e % (K / VEC)) * VEC;
                if constexpr (sizeof(T) == 2) {
                    const u32x4 gv = *reinterpret_cast<const u32x4*>(sG + vv * C::LDS + kk);
                    const u32x4 sv = *reinterpret_cast<const u32x4*>(sS + vv * C::LDS + kk);
#pragma unroll
                    for (int i = 0; i < 4; ++i) gs = dot2_bf16(gv[i], sv[i], gs);
                } else {
#pragma unroll
                    for (int i = 0; i < VEC; i += 4)
                        gs += dot4(ld4(sG + vv * C::LDS + kk + i), ld4(sS + vv * C::LDS + kk + i));
                }
            }
        }
        // ---- dKt^T[k][r] = sum_v G[v][k] Delta[r][v]  (rows k of this half, cols r) ------------
        f32x4 dKT[KH];
        {
            Frag<T> dtr[V / 32];
#pragma unroll
            for (int vb = 0; vb < V / 32; ++vb) frag_row_fo(dtr[vb], sDl, C::LDV, r, vb * 32);
#pragma unroll
            for (int i = 0; i < KH; ++i) dKT[i] = zero4();
#pragma unroll
            for (int vb = 0; vb < V / 32; ++vb) {
                Frag<T> fg[KH];
#pragma unroll
                for (int i = 0; i < KH; ++i)
                    frag_col(fg[i], sG, C::LDS, (hf * KH + i) * 16 + ln, vb * 32);  // G^T row k, slots v
#pragma unroll
                for (int i = 0; i < KH; ++i) mma(dKT[i], fg[i], dtr[vb]);
            }
        }
        // mask, decay, the P terms of d(gam), and L .* dP
        float drow = 0.f;  // d(gam_r) terms accumulated in this lane (summed over gq below)
        f32x4 LdP[2];
#pragma unroll
        for (int m = 0; m < 2; ++m) {
            const int jt = 2 * hf + m;
            f32x4 colpart;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float e = dec[m][i];
                const float x = dPT[m][i] * PmQ[m][i] * e;  // dP .* P at (query r, key j)
                drow += x;
                colpart[i] = x;
                LdP[m][i] = dPT[m][i] * e;
            }
            // column sums over the wave's 16 query rows -> key j (each key belongs to one half)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float s = sum_ln(colpart[i]);
                if (ln == 0) sRed[w * 64 + jt * 16 + gq * 4 + i] = -s;
            }
        }
        // d(gam) from Kt: -e^{Gam-gam_r} sum_k dKt[r][k] K[r][k]; the chunk total gets the sum
        float ktk = 0.f;
#pragma unroll
        for (int i = 0; i < KH; ++i) ktk += dot4(dKT[i], ld4(sK + r * C::LDK + frag_pos((hf * KH + i) * 16 + gq * 4)));
        ktk *= ekt;
        drow -= ktk;
        {
            const float t1 = sum_ln(sum_gq(ktk));  // one value per (r, gq); summed over all lanes it is sum_r
            const float g1 = sum_gq(sum_ln(gs));
            if (lane == 0) {
                sSc[wave] = t1;
                sSc[8 + wave] = g1;
            }
        }
        drow = sum_gq(drow);
        if (gq == 0) sRow[hf * 64 + r] = drow;
        lds_sync();  // every read of Delta is done: the exchange overwrites it
        if constexpr (kCarry) {
            // dDelta over P (every wave's reads of P are done): rows j, this wave's value columns
#pragma unroll
            for (int jt = 0; jt < 4; ++jt) store4(sdU + (jt * 16 + ln) * C::LDU + frag_pos(vrow - ln + gq * 4), ddT[jt]);
        }
        // exchange L .* dP: sX[query r][key j]
#pragma unroll
        for (int m = 0; m < 2; ++m) store4(sX + r * C::LDX + frag_pos((2 * hf + m) * 16 + gq * 4), LdP[m]);
        lds_sync();
        // dk terms of the state side for the wave's rows as keys y = r, this half's k tiles:
        // e^{Gam-gam_y} dKt^T + Q^T (L .* dP)[:, y]
        f32x4 dkpart[KH];
        {
            Frag<T> xc[2];
            frag_col_fo(xc[0], sX, C::LDX, r, 0);  // (L .* dP) column y, slots r'
            frag_col_fo(xc[1], sX, C::LDX, r, 32);
#pragma unroll
            for (int i = 0; i < KH; ++i) {
                dkpart[i] = dKT[i] * ekt;
#pragma unroll
                for (int yb = 0; yb < 2; ++yb) {
                    Frag<T> fq;
                    frag_col_fo(fq, sQ, C::LDK, (hf * KH + i) * 16 + ln, yb * 32);  // Q^T row k, slots r'
                    mma(dkpart[i], fq, xc[yb]);
                }
            }
        }
        // ======= state side, k slice w (KW tiles), row tiles 2hf, 2hf+1 of the chunk =======
        // dQt^T[k][r] = sum_v S[v][k] dO[r][v],  dW^T[k][r] = -sum_v S[v][k] dDelta[r][v] (the
        // products accumulate the sum; its sign is applied where dW is staged)
        {
            const int k0 = w * (K / 4);
            f32x4 dQT[KW][2], dWT[KW][2];
            Frag<T> sfc[KW][V / 32];
#pragma unroll
            for (int j = 0; j < KW; ++j)
#pragma unroll
                for (int vb = 0; vb < V / 32; ++vb)
                    frag_col(sfc[j][vb], sS, C::LDS, k0 + j * 16 + ln, vb * 32);  // S^T row k, slots v
#pragma unroll
            for (int m = 0; m < 2; ++m) {
                const int rr = 2 * hf + m;
                Frag<T> fdo[V / 32], fdd[V / 32];
#pragma unroll
                for (int vb = 0; vb < V / 32; ++vb) {
                    frag_row_fo(fdo[vb], sD, C::LDV, rr * 16 + ln, vb * 32);
                    frag_row_fo(fdd[vb], sdU, C::LDU, rr * 16 + ln, vb * 32);
                }
#pragma unroll
                for (int j = 0; j < KW; ++j) {
                    dQT[j][m] = zero4();
                    dWT[j][m] = zero4();
#pragma unroll
                    for (int vb = 0; vb < V / 32; ++vb) {
                        mma(dQT[j][m], sfc[j][vb], fdo[vb]);
                        mma(dWT[j][m], sfc[j][vb], fdd[vb]);
                    }
                }
            }
            // v and T of this task for the WY side: late enough to add no registers to the
            // products above, early enough for the loads to land before the WY staging
            bwd_fetch_vt(RV, a, cur);
            // dq^T = e^{gam_r} dQt^T + K^T (L .* dP)^T, and e^{gam_r} sum_k dQt[r][k] Q[r][k]
            // over this wave's k slice
            Frag<T> kc[KW][2];
#pragma unroll
            for (int j = 0; j < KW; ++j) {
                frag_col_fo(kc[j][0], sK, C::LDK, k0 + j * 16 + ln, 0);  // K^T row k, slots j'
                frag_col_fo(kc[j][1], sK, C::LDK, k0 + j * 16 + ln, 32);
            }
            f32x4 dqs[C::stage_grads ? KW : 1][2];  // staging: dq tiles of rows (2hf+m)*16+ln
#pragma unroll
            for (int m = 0; m < 2; ++m) {
                const int row = (2 * hf + m) * 16 + ln;
                const float eg = sEg[row];
                Frag<T> xr[2];
                frag_row_fo(xr[0], sX, C::LDX, row, 0);  // (L .* dP) row r, slots j'
                frag_row_fo(xr[1], sX, C::LDX, row, 32);
                T* dq = reinterpret_cast<T*>(a.dq) + ((t0 + row) * H + h) * K + k0;
                float qd = 0.f;
                f32x4 accq[KW];
#pragma unroll
                for (int j = 0; j < KW; ++j) {
                    qd += dot4(dQT[j][m], ld4(sQ + row * C::LDK + frag_pos(k0 + j * 16 + gq * 4)));
                    accq[j] = dQT[j][m] * eg;
                    mma(accq[j], kc[j][0], xr[0]);
                    mma(accq[j], kc[j][1], xr[1]);
                }
                if constexpr (C::stage_grads) {
#pragma unroll
                    for (int j = 0; j < KW; ++j) dqs[j][m] = accq[j];  // staged after the barrier below
                } else if constexpr (KW == 2) {
                    store_pair<T>(dq, accq[0], accq[1], row < c);  // k0 = 32w: whole 32-column runs
                } else {
#pragma unroll
                    for (int j = 0; j < KW; ++j)
                        if (row < c) store4(dq + j * 16 + gq * 4, accq[j]);
                }
                qd = sum_gq(qd) * eg;
                if (gq == 0) sQd[w * 64 + row] = qd;
            }
            lds_sync();  // the state side's LDS reads are done: the WY side reuses the space
            if constexpr (C::stage_grads) {
                T* sGq = reinterpret_cast<T*>(sm + C::off_gst);
#pragma unroll
                for (int j = 0; j < KW; ++j)
#pragma unroll
                    for (int m = 0; m < 2; ++m)
                        store4(sGq + ((2 * hf + m) * 16 + ln) * C::LDG + k0 + j * 16 + gq * 4, dqs[j][m]);
            }
            // dW (rows r) in the operand type, over S
#pragma unroll
            for (int j = 0; j < KW; ++j)
#pragma unroll
                for (int m = 0; m < 2; ++m) {
                    const int row = (2 * hf + m) * 16 + ln;
                    store4(sdW + row * C::LDK + frag_pos(k0 + j * 16 + gq * 4), row < c ? -dWT[j][m] : zero4());
                }
        }

        // ================================= WY side =====================================
        if (tid < 64) {
            float d = sRow[tid] + sRow[64 + tid] + sRed[tid] + sRed[64 + tid] + sRed[128 + tid] + sRed[192 + tid] +
                      sQd[tid] + sQd[64 + tid] + sQd[128 + tid] + sQd[192 + tid];
            if (tid == c - 1) {
                float kt_all = 0.f, gs_all = 0.f;
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    kt_all += sSc[i];
                    gs_all += sSc[8 + i];
                }
                d += kt_all + fast_exp(Gm) * gs_all;
            }
            sDgs[tid] = d;
        }
        put_tile_fo<T, V, C::NV, NT>(sV, C::LDV, RV.v);  // fragment order
        put_tile_fo<T, 64, C::NX, NT>(sTm, C::LDX, RV.t);
        lds_sync();
        if constexpr (C::stage_grads) {
            // dq as whole rows (no loads are in flight here: the next task's start after this)
            flush_tile<T, K, NT>(reinterpret_cast<T*>(a.dq) + (t0 * H + h) * K, (size_t)H * K, c,
                                 reinterpret_cast<const T*>(sm + C::off_gst), C::LDG);
        }
        // The next task's operands load over the rest of this one, issued late (where few
        // registers are live, so that nothing spills or waits on them) and in groups.
        bwd_fetch<0>(R, a, nxt);
        const int ra = r;
        f32x4 kkk[2];  // K K^T, rows c of this half's tiles, cols a = ra (from the dT step)
        // ---- dT[a][b] = beta_b e^{gam_b} (dW K^T)[a][b] + beta_b (dU V^T)[a][b], b < a, this
        // half's b tiles (rows b, cols a), exchanged through LDS as dT[a][b]
        {
            f32x4 x[2], y[2];
            if constexpr (kL2) {
                // both b tiles, masked: with the raw-q normalisation the count branch below
                // needs one register more than the kernel has
                Frag<T> wf[K / 32], uf[V / 32], kra[K / 32];
#pragma unroll
                for (int kb = 0; kb < K / 32; ++kb) frag_row_fo(wf[kb], sdW, C::LDK, ra, kb * 32);
#pragma unroll
                for (int kb = 0; kb < K / 32; ++kb) frag_row_fo(kra[kb], sK, C::LDK, ra, kb * 32);
#pragma unroll
                for (int vb = 0; vb < V / 32; ++vb) frag_row_fo(uf[vb], sdU, C::LDU, ra, vb * 32);
                // both b tiles (the mask below zeroes b >= a)
#pragma unroll
                for (int m = 0; m < 2; ++m) {
                    x[m] = zero4();
                    y[m] = zero4();
                    kkk[m] = zero4();
                }
                // the same K row fragments give K K^T (rows c = b, cols a) for the dA step below
#pragma unroll
                for (int kb = 0; kb < K / 32; ++kb) {
                    Frag<T> fk[2];
#pragma unroll
                    for (int m = 0; m < 2; ++m) frag_row_fo(fk[m], sK, C::LDK, (2 * hf + m) * 16 + ln, kb * 32);
#pragma unroll
                    for (int m = 0; m < 2; ++m) {
                        mma(x[m], fk[m], wf[kb]);      // rows b, cols a: (K dW^T)[b][a]
                        mma(kkk[m], fk[m], kra[kb]);   // rows c, cols a: k_c . k_a
                    }
                }
#pragma unroll
                for (int vb = 0; vb < V / 32; ++vb) {
                    Frag<T> fv[2];
#pragma unroll
                    for (int m = 0; m < 2; ++m) frag_row_fo(fv[m], sV, C::LDV, (2 * hf + m) * 16 + ln, vb * 32);
#pragma unroll
                    for (int m = 0; m < 2; ++m) mma(y[m], fv[m], uf[vb]);
                }
            } else {
                // the live b tiles (the mask below zeroes b >= a within them)
#pragma unroll
                for (int m = 0; m < 2; ++m) {
                    x[m] = zero4();
                    y[m] = zero4();
                    kkk[m] = zero4();
                }
                auto products = [&](auto nm_) {
                    constexpr int NM = decltype(nm_)::value;
                    Frag<T> wf[K / 32], uf[V / 32], kra[K / 32];
#pragma unroll
                    for (int kb = 0; kb < K / 32; ++kb) frag_row_fo(wf[kb], sdW, C::LDK, ra, kb * 32);
#pragma unroll
                    for (int kb = 0; kb < K / 32; ++kb) frag_row_fo(kra[kb], sK, C::LDK, ra, kb * 32);
#pragma unroll
                    for (int vb = 0; vb < V / 32; ++vb) frag_row_fo(uf[vb], sdU, C::LDU, ra, vb * 32);
                    // the same K row fragments give K K^T (rows c = b, cols a) for the dA step below
#pragma unroll
                    for (int kb = 0; kb < K / 32; ++kb) {
                        Frag<T> fk[NM];
#pragma unroll
                        for (int m = 0; m < NM; ++m) frag_row_fo(fk[m], sK, C::LDK, (2 * hf + m) * 16 + ln, kb * 32);
#pragma unroll
                        for (int m = 0; m < NM; ++m) {
                            mma(x[m], fk[m], wf[kb]);      // rows b, cols a: (K dW^T)[b][a]
                            mma(kkk[m], fk[m], kra[kb]);   // rows c, cols a: k_c . k_a
                        }
                    }
#pragma unroll
                    for (int vb = 0; vb < V / 32; ++vb) {
                        Frag<T> fv[NM];
#pragma unroll
                        for (int m = 0; m < NM; ++m) frag_row_fo(fv[m], sV, C::LDV, (2 * hf + m) * 16 + ln, vb * 32);
#pragma unroll
                        for (int m = 0; m < NM; ++m) mma(y[m], fv[m], uf[vb]);
                    }
                };
                if (nlive == 2)
                    products(std::integral_constant<int, 2>{});
                else if (nlive == 1)
                    products(std::integral_constant<int, 1>{});
            }
#pragma unroll
            for (int m = 0; m < 2; ++m) {
                const int bt = 2 * hf + m;
                const f32x4 gb = ld4(sEg + bt * 16 + gq * 4);  // e^{gam_b}
                const f32x4 bb = ld4(sBeta + bt * 16 + gq * 4);
                f32x4 dT;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int b = bt * 16 + gq * 4 + e;
                    dT[e] = (b < ra) ? bb[e] * (gb[e] * x[m][e] + y[m][e]) : 0.f;
                }
                store4(sDT + ra * C::LDX + frag_pos(bt * 16 + gq * 4), dT);  // dT[a][b], fragment order
            }
        }
        lds_sync();
        bwd_fetch<1>(R, a, nxt);
        // ---- Y = dT T^T: tiles Y^T[c][a] = sum_b T[c][b] dT[a][b] (T[c][b] = 0 for b > c),
        // this half's c tiles -------------------------------------------------------------------
        {
            Frag<T> dtf[2];
            frag_row_fo(dtf[0], sDT, C::LDX, ra, 0);  // dT row a, slots b
            frag_row_fo(dtf[1], sDT, C::LDX, ra, 32);
            f32x4 y[2];
#pragma unroll
            for (int m = 0; m < 2; ++m) y[m] = zero4();
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
                Frag<T> ft[2];
#pragma unroll
                for (int m = 0; m < 2; ++m) frag_row_fo(ft[m], sTm, C::LDX, (2 * hf + m) * 16 + ln, kb * 32);
#pragma unroll
                for (int m = 0; m < 2; ++m) mma(y[m], ft[m], dtf[kb]);
            }
#pragma unroll
            for (int m = 0; m < 2; ++m) store4(sY + ra * C::LDX + (2 * hf + m) * 16 + gq * 4, y[m]);  // Y[a][c]
        }
        lds_sync();
        bwd_fetch<2>(R, a, nxt);
        // ---- dA[a][c] = -sum_x T[x][a] Y[x][c] for c < a (T[x][a] = 0 for x < a); with the
        // raw A[a][c] = e^{gam_a - gam_c} k_a.k_c: dbeta, d(gam), and Mx = dA beta_a e^{..},
        // this half's c tiles
        float dbeta_row = 0.f, dgam_row = 0.f;
        Frag<T> ta[2];
        frag_col_fo(ta[0], sTm, C::LDX, ra, 0);  // T column a, slots x
        frag_col_fo(ta[1], sTm, C::LDX, ra, 32);
        {
            const float ba = sBeta[ra];
            f32x4 dd[2];
#pragma unroll
            for (int m = 0; m < 2; ++m) dd[m] = zero4();
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
                Frag<T> fy[2];
#pragma unroll
                for (int m = 0; m < 2; ++m)
                    frag_col(fy[m], sY, C::LDX, (2 * hf + m) * 16 + ln, kb * 32);  // Y^T row c, slots x
#pragma unroll
                for (int m = 0; m < 2; ++m) mma(dd[m], fy[m], ta[kb]);  // rows c, cols a: (T^T Y)^T
            }
#pragma unroll
            for (int m = 0; m < 2; ++m) {
                const int ct = 2 * hf + m;
                const f32x4 d = dd[m], kk = kkk[m];
                f32x4 colpart, mx;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int cc = ct * 16 + gq * 4 + e;
                    const bool lower = cc < ra;
                    const float dcy = lower ? dec[m][e] : 0.f;  // the causal decay of P, without its diagonal
                    const float ar = dcy * kk[e];  // raw A[a][c]
                    const float dA = lower ? -d[e] : 0.f;
                    dbeta_row += dA * ar;
                    dgam_row += dA * ar * ba;
                    colpart[e] = dA * ar * ba;
                    mx[e] = dA * ba * dcy;
                }
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const float s = sum_ln(colpart[e]);
                    if (ln == 0) sRed[w * 64 + ct * 16 + gq * 4 + e] = -s;
                }
                store4(sMx + ra * C::LDX + frag_pos(ct * 16 + gq * 4), mx);  // Mx[a][c]
            }
        }
        lds_sync();
        // ---- dBk^T = dW^T T, dBv^T = dU^T T (rows k / v, cols a);  dK, dV, this half's tiles ---
        Frag<T> mrow[2], mcol[2];
        frag_row_fo(mrow[0], sMx, C::LDX, ra, 0);  // Mx row a, slots c
        frag_row_fo(mrow[1], sMx, C::LDX, ra, 32);
        frag_col_fo(mcol[0], sMx, C::LDX, ra, 0);  // Mx column a, slots c
        frag_col_fo(mcol[1], sMx, C::LDX, ra, 32);
        const float ba = sBeta[ra], ega = sEg[ra];
        {
            T* dkp = reinterpret_cast<T*>(a.dk) + ((t0 + ra) * H + h) * K;
            f32x4 dkv[KH];
#pragma unroll
            for (int i = 0; i < KH; ++i) {
                const int kt = hf * KH + i;
                f32x4 bk = zero4(), mk = zero4();
#pragma unroll
                for (int xb = 0; xb < 2; ++xb) {
                    Frag<T> fw, fk;
                    frag_col_fo(fw, sdW, C::LDK, kt * 16 + ln, xb * 32);  // dW^T row k, slots x
                    mma(bk, fw, ta[xb]);
                    frag_col_fo(fk, sK, C::LDK, kt * 16 + ln, xb * 32);   // K^T row k, slots c
                    mma(mk, fk, mrow[xb]);
                    mma(mk, fk, mcol[xb]);
                }
                // dbeta, dgam from Bk = diag(beta e^gam) K
                const float s = dot4(bk, ld4(sK + ra * C::LDK + frag_pos(kt * 16 + gq * 4)));
                dbeta_row += ega * s;
                dgam_row += ba * ega * s;
                dkv[i] = dkpart[i] + mk + bk * (ba * ega);
            }
            if constexpr (C::stage_grads) {
                T* sGk = reinterpret_cast<T*>(sm + C::off_gst);
#pragma unroll
                for (int i = 0; i < KH; ++i) store4(sGk + ra * C::LDG + (hf * KH + i) * 16 + gq * 4, dkv[i]);
            } else {
                // this half's k tiles in pairs: whole 32-column runs of the row
#pragma unroll
                for (int i = 0; i < KH; i += 2) store_pair<T>(dkp + (hf * KH + i) * 16, dkv[i], dkv[i + 1], ra < c);
            }
        }
        f32x4 bvk[kCarry ? VH : 1];  // kCarry: dBv[a = ra][this half's v tiles], for the adjoint update
        {
            T* dvp = reinterpret_cast<T*>(a.dv) + ((t0 + ra) * H + h) * V;
            f32x4 dvv[VH];
#pragma unroll
            for (int i = 0; i < VH; ++i) {
                const int vt = hf * VH + i;
                f32x4 bv = zero4();
#pragma unroll
                for (int xb = 0; xb < 2; ++xb) {
                    Frag<T> fu;
                    frag_col_fo(fu, sdU, C::LDU, vt * 16 + ln, xb * 32);  // dU^T row v, slots x
                    mma(bv, fu, ta[xb]);
                }
                dbeta_row += dot4(bv, ld4(sV + ra * C::LDV + frag_pos(vt * 16 + gq * 4)));
                dvv[i] = bv * ba;
                if constexpr (kCarry) bvk[i] = bv;
            }
            if constexpr (C::stage_grads) {
                T* sGv = reinterpret_cast<T*>(sm + C::off_gst + C::kMG);
#pragma unroll
                for (int i = 0; i < VH; ++i) store4(sGv + ra * C::LDG + (hf * VH + i) * 16 + gq * 4, dvv[i]);
            } else {
#pragma unroll
                for (int i = 0; i < VH; i += 2) store_pair<T>(dvp + (hf * VH + i) * 16, dvv[i], dvv[i + 1], ra < c);
            }
        }
        if constexpr (!C::stage_grads) {
            bwd_fetch<3>(R, a, nxt);
            bwd_fetch<4>(R, a, nxt);
        }
        dbeta_row = sum_gq(dbeta_row);
        dgam_row = sum_gq(dgam_row);
        if (gq == 0) {
            sRow[hf * 64 + ra] = dgam_row;
            sDb[hf * 64 + ra] = dbeta_row;
        }
        lds_sync();
        if constexpr (C::stage_grads) {
            // dk and dv as whole rows
            flush_tile<T, K, NT>(reinterpret_cast<T*>(a.dk) + (t0 * H + h) * K, (size_t)H * K, c,
                                 reinterpret_cast<const T*>(sm + C::off_gst), C::LDG);
            flush_tile<T, V, NT>(reinterpret_cast<T*>(a.dv) + (t0 * H + h) * V, (size_t)H * V, c,
                                 reinterpret_cast<const T*>(sm + C::off_gst + C::kMG), C::LDG);
            // the next task's S (and G) after these stores, so that no wait for their data
            // registers lands on those loads
            bwd_fetch<3>(R, a, nxt);
            bwd_fetch<4>(R, a, nxt);
        }
        // ---- dbeta, and d(gam) total with dg = reverse cumulative sum within the chunk ---------
        if (wave == 0) {
            // suffix sum over the chunk's rows: a prefix scan over the lanes in reversed order
            const int i = 63 - lane;
            float d = 0.f;
            if (i < c)
                d = sDgs[i] + sRow[i] + sRow[64 + i] + sRed[i] + sRed[64 + i] + sRed[128 + i] + sRed[192 + i];
            d = wave_prefix_sum(d);
            if (i < c) a.dg[(t0 + i) * H + h] = d;
        } else if (wave == 1) {
            if (lane < c) a.dbeta[(t0 + lane) * H + h] = sDb[lane] + sDb[64 + lane];
        }
        if constexpr (kCarry) {
            // G^T -= K^T X, X = diag(beta e^gam) dBv (= W^T dDelta): this lane's row a = ra of X over
            // the state's space (every read of dW, V and the rest of the WY side is done), then
            // every wave its value columns
            T* sXb = reinterpret_cast<T*>(sm + C::off_s);
            const float bea = -ba * ega;  // negated: G^T -= K^T X
#pragma unroll
            for (int i = 0; i < VH; ++i) store4(sXb + ra * C::LDV + frag_pos((hf * VH + i) * 16 + gq * 4), bvk[i] * bea);
            lds_sync();
            Frag<T> nx[2];  // -X
#pragma unroll
            for (int ab = 0; ab < 2; ++ab) frag_col_fo(nx[ab], sXb, C::LDV, vrow, ab * 32);  // -X column v, slots a
#pragma unroll
            for (int kt = 0; kt < K / 16; ++kt) {
#pragma unroll
                for (int ab = 0; ab < 2; ++ab) {
                    Frag<T> fk;
                    frag_col_fo(fk, sK, C::LDK, kt * 16 + ln, ab * 32);  // K column k, slots a
                    mma(accG[kt], fk, nx[ab]);
                }
            }
        }
        if (!more) break;
        cur = nxt;
        t = tn;
    }
    // the adjoint entering the sub-sequence's first chunk: d(initial state) at a sequence start
    if constexpr (kCarry) {
        if (sg.s == 0 && a.ds0) store_state<K>(accG, a.ds0 + ((size_t)sg.n * H + hc) * VK, vrow);
    }
}

template <typename T, int K, int V>
hipError_t launch_bwd_chunk_t(const BwdChunkArgs& a, int grid, hipStream_t st) {
    using C = BCfg<T, K, V>;
    static_assert(C::total <= 160 * 1024, "LDS budget");
    auto kern = a.q_l2 ? k_bwd_chunk<T, K, V, true> : k_bwd_chunk<T, K, V, false>;
    if constexpr (V == 128 && sizeof(T) == 2) {
        // one workgroup per (sub-sequence, head), each carrying its adjoint
        if (a.carry) {
            kern = a.q_l2 ? k_bwd_chunk<T, K, V, true, true> : k_bwd_chunk<T, K, V, false, true>;
            grid = (int)(a.geo.total_segs * a.geo.H);
        }
    }
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, C::total);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(C::NT), C::total, st, a);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_reverse(const RevArgs& a, int dtype, int mode, int64_t nsegs_grid, int vtiles, hipStream_t st) {
    if (nsegs_grid == 0) return hipSuccess;
    const int K = a.geo.K;
    const int RT = recur_rows(a.geo.V, K);
#define GDN_REV_CASE(TT, KK, RR)                                                                          \
    if (K == KK && RT == RR) {                                                                            \
        if (mode == kRecurOut) return launch_reverse_t<TT, KK, RR, kRecurOut>(a, nsegs_grid, vtiles, st);  \
        if (mode == kRecurPrepass) return launch_reverse_t<TT, KK, RR, kRecurPrepass>(a, nsegs_grid, vtiles, st); \
    }
    if (dtype == 0) {
        GDN_REV_CASE(bf16_t, 64, 64)
        GDN_REV_CASE(bf16_t, 128, 64)
        GDN_REV_CASE(bf16_t, 128, 128)
    } else {
        GDN_REV_CASE(float, 64, 64)  // the fp32 backward supports K = V = 64 only
    }
#undef GDN_REV_CASE
    return hipErrorInvalidValue;
}


#define GDN_BWD_CASES(FN)                                              \
    if (dtype == 0) {                                                  \
        if (K == 64 && V == 64) return FN<bf16_t, 64, 64>(a, grid, st);    \
        if (K == 64 && V == 128) return FN<bf16_t, 64, 128>(a, grid, st);  \
        if (K == 128 && V == 64) return FN<bf16_t, 128, 64>(a, grid, st);  \
        if (K == 128 && V == 128) return FN<bf16_t, 128, 128>(a, grid, st); \
    } else {                                                           \
        if (K == 64 && V == 64) return FN<float, 64, 64>(a, grid, st);     \
    }

hipError_t launch_bwd_chunk(const BwdChunkArgs& a, int dtype, int grid, hipStream_t st) {
    // (carrying the adjoint, sub-sequences without chunks still pass d(final state) through)
    if ((a.carry ? a.geo.total_segs : a.geo.total_chunks) == 0 || grid < 1) return hipSuccess;
    if (a.carry && (a.geo.V != 128 || dtype != 0)) return hipErrorInvalidValue;
    const int K = a.geo.K, V = a.geo.V;
    GDN_BWD_CASES(launch_bwd_chunk_t)
    return hipErrorInvalidValue;
}
#undef GDN_BWD_CASES

}  // namespace gdn
