// gdn_kernels.h -- argument blocks and launchers of the libgdn kernels.
// Host and device code both include this file; nothing here is part of the C ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gdn {

// Where sequences, chunks and sub-sequences ("segments") live.
// Uniform batches (varlen == 0) compute everything from T; packed batches
// read the tables built on the device from cu_seqlens.
struct Geo {
    int32_t N, H, K, V;
    int64_t T;            // tokens per batch row (uniform) / packed total (varlen)
    int32_t varlen;
    int32_t nt;           // chunks per sequence (uniform)
    int32_t seg_len;      // chunks per segment
    int32_t nseg;         // segments per sequence (uniform)
    int64_t total_chunks;
    int64_t total_segs;
    const int64_t* seq_bos;     // [N]   (varlen)
    const int32_t* seq_len;     // [N]
    const int32_t* seq_choff;   // [N+1] first global chunk of each sequence
    const int32_t* seq_segoff;  // [N+1] first global segment of each sequence
    const int2* chunk_tab;      // [total_chunks] (n, chunk index in sequence); n < 0: unused
    const int4* seg_tab;        // [total_segs]   (n, s, c0, c1); n < 0: unused
    const int32_t* seg_order;   // [total_segs]   (varlen) segments, most chunks first; null: none
};

struct ChunkLoc {
    int32_t n;        // sequence
    int32_t j;        // chunk index in the sequence
    int64_t t0;       // first token (flattened)
    int32_t c;        // tokens in this chunk (1..64)
};

__device__ __forceinline__ bool locate_chunk(const Geo& g, int64_t gc, ChunkLoc& L) {
    if (g.varlen) {
        const int2 e = g.chunk_tab[gc];
        if (e.x < 0) return false;
        L.n = e.x;
        L.j = e.y;
        const int32_t len = g.seq_len[e.x];
        L.t0 = g.seq_bos[e.x] + (int64_t)e.y * 64;
        L.c = min(64, len - e.y * 64);
    } else {
        L.n = (int32_t)(gc / g.nt);
        L.j = (int32_t)(gc % g.nt);
        L.t0 = (int64_t)L.n * g.T + (int64_t)L.j * 64;
        L.c = (int32_t)min((int64_t)64, g.T - (int64_t)L.j * 64);
    }
    return L.c > 0;
}

// (chunk, head) tasks of the persistent per-chunk kernels: task t is chunk t / H, head t % H.
struct ChunkTask {
    int64_t gc;  // global chunk
    int64_t t0;  // first token (flattened)
    int h;
    int c;       // tokens in the chunk
};

// First valid task at or after t, stepping by the grid; ntasks when there is none.
__device__ __forceinline__ int64_t next_chunk_task(const Geo& geo, int64_t t, int64_t ntasks, ChunkTask& x) {
    for (; t < ntasks; t += gridDim.x) {
        ChunkLoc L;
        const int64_t gc = t / geo.H;
        if (locate_chunk(geo, gc, L)) {
            x.gc = gc;
            x.t0 = L.t0;
            x.h = (int)(t - gc * geo.H);
            x.c = L.c;
            return t;
        }
    }
    return ntasks;
}

struct SegLoc {
    int32_t n, s, c0, c1;  // sequence, segment index, chunk range [c0, c1) in the sequence
    int32_t nseg;          // segments of this sequence
    int32_t nchunks;       // chunks of this sequence
    int64_t bos;
    int32_t len;
    int64_t choff;         // global index of the sequence's first chunk
};

__device__ __forceinline__ bool locate_seg(const Geo& g, int64_t gs, SegLoc& S) {
    if (g.varlen) {
        const int4 e = g.seg_tab[gs];
        if (e.x < 0) return false;
        S.n = e.x;
        S.s = e.y;
        S.c0 = e.z;
        S.c1 = e.w;
        S.nseg = g.seq_segoff[e.x + 1] - g.seq_segoff[e.x];
        S.bos = g.seq_bos[e.x];
        S.len = g.seq_len[e.x];
        S.nchunks = (S.len + 63) / 64;
        S.choff = g.seq_choff[e.x];
    } else {
        S.n = (int32_t)(gs / g.nseg);
        S.s = (int32_t)(gs % g.nseg);
        S.c0 = S.s * g.seg_len;
        S.c1 = min(S.c0 + g.seg_len, g.nt);
        S.nseg = g.nseg;
        S.bos = (int64_t)S.n * g.T;
        S.len = (int32_t)g.T;
        S.nchunks = g.nt;
        S.choff = (int64_t)S.n * g.nt;
    }
    return true;
}

// Per sequence: segments count and the global index of segment 0.
__device__ __forceinline__ void seq_segs(const Geo& g, int32_t n, int32_t& nseg, int64_t& segoff,
                                         int32_t& nchunks, int64_t& choff) {
    if (g.varlen) {
        segoff = g.seq_segoff[n];
        nseg = g.seq_segoff[n + 1] - g.seq_segoff[n];
        nchunks = (g.seq_len[n] + 63) / 64;
        choff = g.seq_choff[n];
    } else {
        segoff = (int64_t)n * g.nseg;
        nseg = g.nseg;
        nchunks = g.nt;
        choff = (int64_t)n * g.nt;
    }
}

// The CP prepasses of uniform-length batches run on a one-dimensional grid in which the
// workgroups of the sequence-heads with exact maps (modes 2 and 3), which walk whole
// sub-sequences, come first in dispatch order, the row tiles of each segment (the map rows
// too) side by side; the other sequence-heads (warm windows only) follow in the order of the
// plain grid (row tile slowest, then head, then sequence, then segment). With the plain grid
// the long workgroups of a late head wait for free CUs behind the short ones. Sequence-heads
// are counted in the key order h * N + n (head major), the plain grid's.
// The sequence-head (n * H + h) of rank q among those with (long) or without exact maps.
__device__ __forceinline__ int32_t head_of_rank(const int32_t* modes, int32_t N, int32_t H, bool long_, int32_t q) {
    const int lane = threadIdx.x & 63;
    const int32_t nh = N * H;
    for (int32_t b = 0; b < nh; b += 64) {
        const int32_t k = b + lane;
        const int32_t p = k < nh ? (k % N) * H + k / N : 0;
        const bool ok = k < nh && (modes[p] >= 2) == long_;
        const uint64_t m = __ballot(ok);
        const int32_t c = __popcll(m);
        if (q < c) {
            // the q-th lane of m
            const uint32_t below = __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
            const int32_t kk = b + (int32_t)__builtin_ctzll(__ballot(ok && (int32_t)below == q));
            return (kk % N) * H + kk / N;
        }
        q -= c;
    }
    return -1;
}

// The (global segment, head, row tile) of a CP prepass workgroup: the ranked one-dimensional
// grid above when `ranked`, else (segment, head, row tile) = (blockIdx.x, blockIdx.y, blockIdx.z).
__device__ __forceinline__ bool prepass_item(const Geo& geo, const int32_t* modes, bool ranked, int vtiles,
                                             int64_t& gs, int& h, int& vt) {
    if (!ranked) {
        gs = blockIdx.x;
        h = blockIdx.y;
        vt = blockIdx.z;
        return true;
    }
    const int lane = threadIdx.x & 63;
    const int32_t nh = geo.N * geo.H, nseg = geo.nseg;
    int32_t nlong = 0;
    for (int32_t b = 0; b < nh; b += 64) nlong += __popcll(__ballot(b + lane < nh && modes[b + lane] >= 2));
    const int64_t L = blockIdx.x, per_head = (int64_t)nseg * vtiles, A = (int64_t)nlong * per_head;
    int32_t p, s;
    if (L < A) {  // heads with exact maps: row tiles fastest (both are whole walks), then segments
        const int64_t w = L % per_head;
        p = head_of_rank(modes, geo.N, geo.H, true, (int32_t)(L / per_head));
        vt = (int)(w % vtiles);
        s = (int32_t)(w / vtiles);
    } else {  // the others: row tile, then head rank, then segment
        const int64_t Lr = L - A, per_vt = (int64_t)(nh - nlong) * nseg;
        vt = (int)(Lr / per_vt);
        const int64_t r = Lr % per_vt;
        p = head_of_rank(modes, geo.N, geo.H, false, (int32_t)(r / nseg));
        s = (int32_t)(r % nseg);
    }
    if (p < 0) return false;
    const int32_t n = p / geo.H;
    h = p - n * geo.H;
    gs = (int64_t)n * nseg + s;
    return true;
}

// The (global segment, head, row tile) of a varlen recurrence workgroup when the varlen tables
// hold a segment order: a one-dimensional grid, segment rank slowest, then head, then row tile,
// so that the longest sequences' workgroups are dispatched first (when the workgroups outnumber
// the CUs, or share the chip with another pass, the rest fill in behind them).
__device__ __forceinline__ void ordered_seg_item(const Geo& geo, int vtiles, int64_t& gs, int& h, int& vt) {
    const int64_t L = blockIdx.x, per_seg = (int64_t)geo.H * vtiles;
    const int64_t r = L / per_seg;
    const int w = (int)(L - r * per_seg);
    gs = geo.seg_order[r];
    h = w / vtiles;
    vt = w - h * vtiles;
}

// ---------------------------------------------------------------------------
struct IntraArgs {
    Geo geo;
    const void* k;
    const void* v;
    const float* g;
    const float* beta;
    float* gam;      // [Ttot, H]
    void* w;         // [Ttot, H, K]
    void* u;         // [Ttot, H, V]
    float2* cstat;   // [total_chunks, H]: (chunk gate total, max beta*|k|^2)
    void* tmat;      // [total_chunks, H, 64, 64] T = (I + A)^{-1} row-major, or null (not written)
    void* kn;        // [Ttot, H, K]: k is raw, its rows are normalised in the kernel and written
                     // here for the later kernels (the q/k L2 normalisation), or null
};

enum RecurMode : int {
    kRecurOut = 0,      // outputs O (and the final state) for each segment
    kRecurPrepass = 1,  // CP preprocessing: warmup windows and exact (R, M) segment maps
    kRecurStates = 2,   // chunk-entry states for the backward (h), no output
    kRecurOutRec = 3    // the output pass recording h and Delta too (a forward that keeps them)
};

struct RecurArgs {
    Geo geo;
    const void* q;
    const void* k;
    const float* gam;
    const void* w;
    const void* u;
    const float* s0;          // [N,H,V,K] or null
    void* o;                  // [Ttot,H,V]
    float* sT;                // [N,H,V,K] or null
    const float* seginit;     // [total_segs,H,V,K] initial state of every segment (s >= 1)
    float* seginit_out;       // prepass: warmup states written here
    float* prep;              // prepass: exact maps per [total_segs,H]: R rows [V][K] fp32, then M^T
                              // [K][K] in the input precision, in a (V+K) x K fp32 slot
    const int32_t* modes;     // [N,H] 0 no split, 1 every boundary warmup, 2 every one exact, 3 mixed
    const int32_t* bwin;      // [total_segs,H] per boundary (the start of segment gs, s >= 1): the
                              // warmup window in chunks, 0 = exact, -1 = no boundary (s = 0)
    void* hstates;            // kRecurStates, kRecurOutRec: [total_chunks,H,V,K] entry state of every chunk
    void* delta;              // same modes: [Ttot,H,V] Delta = U - W S^T of every chunk, or null
    float scale;
    int32_t use_cp;           // segments >= 1 read seginit
    int32_t q_l2;             // output modes: q is raw, its rows are L2-normalised as staged
    int32_t ranked;           // prepass: the ranked grid (see head_by_rank)
    // the fully fused forward (launch_fused) reads the raw inputs instead of w, u and the gate cumsum
    const void* fv;           // [Ttot,H,V]
    const float* fg;          // [Ttot,H]
    const float* fbeta;       // [Ttot,H]
};

struct DecideArgs {
    Geo geo;
    const float2* cstat;
    int32_t* modes;    // [N,H] per sequence-head summary (see RecurArgs)
    int32_t* bwin;     // [total_segs,H] per boundary window (see RecurArgs)
    int32_t warmup;    // shortest window W
    int32_t warmup_max;  // longest window (W .. W + 63)
    float log_eps;
    int32_t forced;  // 0 gate test, 1 warmup, 2 exact
    int32_t reverse; // 1: windows after each segment end (backward adjoint pass)
    int32_t* modes_r;  // optional second output: the reverse decision, from the same launch
    int32_t* bwin_r;
};

struct ScanArgs {
    Geo geo;
    const float* s0;       // forward: initial state; reverse: d(final state) (either may be null)
    const float* prep;
    float* seginit;
    const int32_t* modes;
    int32_t reverse;       // 1: G_{s-1} = G_s M_s + R_s from the last segment down
};

struct RevArgs {
    Geo geo;
    const void* q;
    const void* k;
    const float* gam;
    const void* w;
    const void* d_o;
    const float* dsT;         // [N,H,V,K] or null
    float* ds0;               // [N,H,V,K] or null: gradient of the initial state
    const float* seginit;     // [total_segs,H,V,K] adjoint at the end of every segment but the last
    float* seginit_out;       // prepass: warmup adjoints written here
    float* prep;              // prepass: reverse maps, laid out as the forward's
    const int32_t* modes;
    const int32_t* bwin;      // [total_segs,H] per boundary (the start of segment gs): the window after
                              // it in chunks, 0 = exact, -1 = no boundary
    void* gstates;            // [total_chunks,H,V,K] adjoint of the state leaving every chunk
    void* ddelta;             // kRecurOut: [Ttot,H,V] dL/dDelta of every chunk, or null
    float scale;
    int32_t use_cp;
    int32_t q_l2;             // q is raw, its rows are L2-normalised as staged
    int32_t ranked;           // prepass: the ranked grid (see head_by_rank)
};

struct BwdChunkArgs {
    Geo geo;
    const void* q;
    const void* k;
    const void* v;
    const float* g;
    const float* beta;
    const float* gam;
    const void* d_o;
    const void* delta;        // [Ttot,H,V] Delta = U - W S^T (from the state pass)
    const void* ddelta;       // [Ttot,H,V] dL/dDelta = dU (from the reverse pass)
    const void* hstates;      // [total_chunks,H,V,K] state entering every chunk
    const void* gstates;      // [total_chunks,H,V,K] adjoint of the state leaving every chunk
    const void* tmat;         // [total_chunks,H,64,64] T = (I + A)^{-1} of every chunk
    void* dq;
    void* dk;
    void* dv;
    float* dg;
    float* dbeta;
    float scale;
    int32_t q_l2;             // q is raw, its rows are L2-normalised as staged (dq is then with
                              // respect to the normalised rows)
    // carry: one workgroup per (sub-sequence, head) carries the adjoint through its chunks in
    // reverse (no adjoint pass: gstates and ddelta unused); V = 128, bf16 only
    int32_t carry;
    int32_t use_cp;           // carry: sub-sequences but a sequence's last start from seginit_r
    const float* seginit_r;   // carry: [total_segs,H,V,K] adjoint leaving each sub-sequence (reverse CP)
    const float* dsT;         // carry: [N,H,V,K] d(final state), or null
    float* ds0;               // carry: [N,H,V,K] d(initial state) out, or null
};

struct TableArgs {
    const int32_t* cu;
    int32_t N;
    int64_t Ttot;
    int32_t seg_len;
    int64_t total_chunks;
    int64_t total_segs;
    int64_t* seq_bos;
    int32_t* seq_len;
    int32_t* seq_choff;
    int32_t* seq_segoff;
    int2* chunk_tab;
    int4* seg_tab;
    int32_t* seg_order;  // null: no order built
};

// Bins of the varlen segment order's counting sort (chunk counts; longer segments share the last).
constexpr int kOrderBins = 4096;

// State rows per workgroup of the recurrence kernels: all 128 value rows when
// V = K = 128 (8 waves), else 64 (4 waves). V and K are multiples of it.
__host__ __device__ constexpr int recur_rows(int V, int K) { return (V == 128 && K == 128) ? 128 : 64; }

// Launchers (return hipGetLastError of the launch).
hipError_t launch_tables(const TableArgs& a, hipStream_t st);
hipError_t launch_intra(const IntraArgs& a, int dtype, int cus, hipStream_t st);  // persistent grid
hipError_t launch_decide(const DecideArgs& a, hipStream_t st);
hipError_t launch_recur(const RecurArgs& a, int dtype, int mode, int64_t nsegs_grid, int vtiles,
                        hipStream_t st);
hipError_t launch_scan(const ScanArgs& a, int dtype, hipStream_t st);
// the fully fused forward without CP: grid (sequences, H, value-row tiles); bf16 only
hipError_t launch_fused(const RecurArgs& a, int dtype, int64_t nseqs, int vtiles, hipStream_t st);
hipError_t launch_reverse(const RevArgs& a, int dtype, int mode, int64_t nsegs_grid, int vtiles, hipStream_t st);
// grid: persistent workgroups (one per CU; each walks tasks gc * H + h with a grid stride)
hipError_t launch_bwd_chunk(const BwdChunkArgs& a, int dtype, int grid, hipStream_t st);

// Recurrent form (decode): T tokens of B sequences from a given state.
struct DecodeArgs {
    const void* q;            // [B,T,H,K]
    const void* k;            // [B,T,H,K]
    const void* v;            // [B,T,H,V]
    const float* g;           // [B,T,H]
    const float* beta;        // [B,T,H]
    const float* s_in;        // [B,H,V,K] or null (zeros)
    float* s_out;             // [B,H,V,K] (may be s_in)
    void* o;                  // [B,T,H,V]
    int64_t B, T, H;
    float scale;
};
hipError_t launch_decode(const DecodeArgs& a, int dtype, int K, int V, hipStream_t st);

}  // namespace gdn
