// gdn_api.hip -- the C ABI of libgdn: argument checks, the AutoCP planner, workspace
// layout and the launch sequence. Host code only; kernels live in the other files.
//
// AutoCP rule (FlashQLA pages, ollai.cn article, "core advantages", AutoCP item): split
// sequences inside the card only when batch x heads <= 40, or batch x heads <= 56 and the
// sequence is at least 8192 tokens long ("batch" read as the number of sequences, "seq_len"
// as the longest one). Those thresholds were tuned on a 132-SM GPU and are kept as
// GDN_CP_PAGES; the default decides what they stand for on this device: whether the serial
// recurrence would leave compute units idle (make_plan). The sub-sequence length is chosen
// from the CU count either way.
#include <math.h>
#include <stdlib.h>
#include <string.h>

#include <algorithm>
#include <mutex>
#include <vector>

#include "../../include/gdn.h"
#include "gdn_kernels.h"
#include "gdn_norm.h"

namespace gdn {
namespace {

constexpr size_t kAlign = 256;
constexpr int kDefaultWarmup = 8;
constexpr int kMaxWindowSpan = 64;  // candidate warmup windows W .. W + 63 (one 64-bit mask)

size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

struct Plan {
    int32_t N = 0;
    int64_t H = 0;
    int32_t varlen = 0;
    int64_t Ttot = 0;
    int64_t max_len = 0;
    int64_t total_chunks = 0;
    int32_t nt = 0;        // uniform: chunks per sequence
    int32_t cp_on = 0;
    int32_t seg_len = 1;
    int32_t nseg = 1;      // uniform: segments per sequence
    int64_t total_segs = 0;
    int32_t W = kDefaultWarmup;
    int32_t Wmax = kDefaultWarmup;
    float eps = 1e-4f;
    int32_t forced = 0;
    int32_t esize = 2;
    // forward workspace
    size_t o_kn = 0, o_gam = 0, o_w = 0, o_u = 0, o_cstat = 0, o_bos = 0, o_len = 0, o_choff = 0, o_segoff = 0,
           o_ctab = 0, o_stab = 0, o_sord = 0, o_modes = 0, o_bwin = 0, o_seginit = 0, o_prep = 0, fwd_bytes = 0;
    // backward workspace: the forward's layout, then these
    size_t o_modes_r = 0, o_bwin_r = 0, o_seginit_r = 0, o_prep_r = 0, o_h = 0, o_gst = 0, o_tm = 0, o_dl = 0, o_ddl = 0,
           bwd_bytes = 0;
    // desc->cp_states: the forward-direction CP decisions, windows and sub-sequence entry states
    size_t c_bwin = 0, c_seginit = 0, cp_bytes = 0;
    int32_t cus = 256;   // compute units (desc->num_cus, else the device's)
    int32_t bwd_ok = 1;  // fp32 backward supports K = V = 64 only (LDS)
    int32_t fused = 0;   // the forward runs fully fused (no CP, bf16, no kept intermediates)
    int32_t carry = 0;   // the backward's per-chunk kernel carries the adjoint (no adjoint pass)
    int32_t seg_order = 0;  // varlen: the recurrence grids take the segments most chunks first
};

int query_cus() {
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 256;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
        return 256;
    return cus;
}

gdn_status make_plan(const gdn_desc* d, Plan& p) {
    if (!d) return GDN_ERR_INVALID_ARG;
    for (int i = 0; i < 5; ++i)
        if (d->reserved[i] != 0) return GDN_ERR_INVALID_ARG;
    if (d->flags & ~(GDN_FLAG_KEEP_FORWARD | GDN_FLAG_REUSE_FORWARD | GDN_FLAG_QK_L2NORM | GDN_FLAG_BWD_ADJOINT_PASS |
                     GDN_FLAG_FWD_FUSED | GDN_FLAG_FWD_SPLIT | GDN_FLAG_REUSE_CP))
        return GDN_ERR_INVALID_ARG;
    if (reinterpret_cast<uintptr_t>(d->cp_states) % kAlign) return GDN_ERR_INVALID_ARG;
    if ((d->flags & GDN_FLAG_FWD_FUSED) && (d->flags & GDN_FLAG_FWD_SPLIT)) return GDN_ERR_INVALID_ARG;
    if (d->B < 1 || d->T < 0 || d->H < 1 || d->K < 1 || d->V < 1) return GDN_ERR_INVALID_ARG;
    if (!(d->chunk == 0 || d->chunk == 64)) return GDN_ERR_UNSUPPORTED;
    if (!(d->K == 64 || d->K == 128) || !(d->V == 64 || d->V == 128)) return GDN_ERR_UNSUPPORTED;
    if (d->dtype != GDN_DTYPE_BF16 && d->dtype != GDN_DTYPE_FP32) return GDN_ERR_INVALID_ARG;
    if (!isfinite(d->scale)) return GDN_ERR_INVALID_ARG;
    if (d->cp_mode < GDN_CP_AUTO || d->cp_mode > GDN_CP_PAGES) return GDN_ERR_INVALID_ARG;
    if (d->warmup_chunks < 0 || d->warmup_chunks > 16) return GDN_ERR_INVALID_ARG;
    if (d->warmup_max_chunks < 0) return GDN_ERR_INVALID_ARG;
    if (d->seg_chunks < 0 || d->num_cus < 0) return GDN_ERR_INVALID_ARG;
    if (!(d->warmup_eps >= 0.f && d->warmup_eps < 1.f)) return GDN_ERR_INVALID_ARG;
    if (d->H > 65535) return GDN_ERR_UNSUPPORTED;
    p.esize = d->dtype == GDN_DTYPE_BF16 ? 2 : 4;
    p.H = d->H;
    p.W = d->warmup_chunks ? d->warmup_chunks : kDefaultWarmup;
    if (d->warmup_max_chunks && (d->warmup_max_chunks < p.W || d->warmup_max_chunks > p.W + kMaxWindowSpan - 1))
        return GDN_ERR_INVALID_ARG;
    p.eps = d->warmup_eps > 0.f ? d->warmup_eps : (d->dtype == GDN_DTYPE_BF16 ? 1e-4f : 1e-6f);
    p.Ttot = d->B * d->T;
    int64_t max_nt = 0;
    if (d->cu_seqlens || d->cu_seqlens_host) {
        if (!d->cu_seqlens || !d->cu_seqlens_host || d->B != 1 || d->num_seqs < 1) return GDN_ERR_INVALID_ARG;
        const int32_t* cu = d->cu_seqlens_host;
        if (cu[0] != 0 || cu[d->num_seqs] != d->T) return GDN_ERR_INVALID_ARG;
        p.varlen = 1;
        p.N = d->num_seqs;
        for (int32_t n = 0; n < p.N; ++n) {
            const int64_t len = (int64_t)cu[n + 1] - cu[n];
            if (len < 0) return GDN_ERR_INVALID_ARG;
            p.max_len = std::max(p.max_len, len);
            p.total_chunks += (len + 63) / 64;
        }
        max_nt = (p.max_len + 63) / 64;
    } else {
        if (d->B > INT32_MAX) return GDN_ERR_INVALID_ARG;
        p.N = (int32_t)d->B;
        p.max_len = d->T;
        p.nt = (int32_t)((d->T + 63) / 64);
        p.total_chunks = (int64_t)p.N * p.nt;
        max_nt = p.nt;
    }
    if (p.total_chunks > INT32_MAX || max_nt > INT32_MAX / 2) return GDN_ERR_UNSUPPORTED;
    // the per-chunk kernels address a 64-row tile of [T, H, D] with 32-bit byte offsets
    if (d->H * std::max(d->K, d->V) * 64 * 4 >= ((int64_t)1 << 31)) return GDN_ERR_UNSUPPORTED;

    p.cus = d->num_cus > 0 ? d->num_cus : query_cus();
    // AutoCP. The recurrence runs one workgroup per (sequence-head, row tile, sub-sequence):
    // one per CU at V = K = 128 (8 waves, ~95 KB of LDS), two otherwise.
    const int64_t NH = (int64_t)p.N * d->H;
    const int vtiles = (int)(d->V / recur_rows((int)d->V, (int)d->K));
    const int per_cu = recur_rows((int)d->V, (int)d->K) == 128 ? 1 : 2;
    const int64_t target = (int64_t)per_cu * p.cus;  // workgroups to aim for
    const int64_t units = NH * vtiles;                // workgroups per sub-sequence layer
    bool cp = false;
    // chunk steps per recurrence slot that the whole batch needs, were it spread evenly
    const int64_t balance = (p.total_chunks * d->H * vtiles + target - 1) / std::max<int64_t>(target, 1);
    bool imbalance = false;
    switch (d->cp_mode) {
        case GDN_CP_AUTO:
            // split when the grid would fill at most half of the slots without it and the longest
            // sequence spans two sub-sequences of the minimum length (measured on this part:
            // N*H = 64 at 8K tokens, forward 0.67 -> 0.34 ms; the pages' rule keeps it off there)
            cp = 2 * units <= target && max_nt >= 32;
            // packed sequences of unequal length that fill the slots: split when the longest one
            // takes 1.5x the chunk steps per slot the batch needs, into sub-sequences of half
            // that (measured on this part: 8 sequences of 1K-16K tokens x 32 heads, longest 225
            // chunks against 129, forward + backward 5.03 -> 4.40 ms at 64-chunk sub-sequences)
            if (!cp && p.varlen && 2 * max_nt >= 3 * balance && max_nt >= 64) cp = imbalance = true;
            break;
        case GDN_CP_PAGES: cp = (NH <= 40) || (NH <= 56 && p.max_len >= 8192); break;
        case GDN_CP_OFF: cp = false; break;
        default: cp = true; break;
    }
    p.forced = d->cp_mode == GDN_CP_WARMUP ? 1 : (d->cp_mode == GDN_CP_EXACT ? 2 : 0);
    int64_t seg_len = std::max<int64_t>(max_nt, 1);
    if (cp) {
        if (d->seg_chunks > 0) {
            seg_len = d->seg_chunks;
        } else if (imbalance) {
            seg_len = std::max<int64_t>(32, (balance + 1) / 2);
        } else {
            const int64_t want = std::max<int64_t>(1, target / std::max<int64_t>(units, 1));
            seg_len = std::max<int64_t>(16, (max_nt + want - 1) / want);
            // CP asked for on a batch that already fills the slots: sub-sequences of half the
            // chunk steps per slot it needs, as AUTO takes for unequal packed sequences
            if (seg_len >= max_nt && d->cp_mode != GDN_CP_AUTO && d->cp_mode != GDN_CP_PAGES)
                seg_len = std::max<int64_t>(16, (balance + 1) / 2);
        }
        if (seg_len >= max_nt) {
            cp = false;
            seg_len = std::max<int64_t>(max_nt, 1);
        }
    }
    p.cp_on = cp ? 1 : 0;
    p.seg_len = (int32_t)seg_len;
    // A sequence-head whose gates do not meet the warmup bound over W chunks may take a longer
    // window, by default up to one sub-sequence: the warmup then still costs less than the
    // exact correction (a (V+K)-row pass over the whole sub-sequence plus the segment scan).
    p.Wmax = d->warmup_max_chunks
                 ? d->warmup_max_chunks
                 : (int32_t)std::min<int64_t>(std::max<int64_t>(seg_len, p.W), p.W + kMaxWindowSpan - 1);
    if (p.varlen) {
        p.total_segs = 0;
        const int32_t* cu = d->cu_seqlens_host;
        for (int32_t n = 0; n < p.N; ++n) {
            const int64_t nch = ((int64_t)cu[n + 1] - cu[n] + 63) / 64;
            p.total_segs += nch <= seg_len ? 1 : (nch + seg_len - 1) / seg_len;
        }
    } else {
        p.nseg = p.nt <= seg_len ? 1 : (int32_t)((p.nt + seg_len - 1) / seg_len);
        p.total_segs = (int64_t)p.N * p.nseg;
    }
    if (p.total_segs > INT32_MAX) return GDN_ERR_UNSUPPORTED;

    // forward workspace
    const size_t H = (size_t)d->H, K = (size_t)d->K, V = (size_t)d->V, T = (size_t)p.Ttot;
    size_t off = 0;
    auto take = [&](size_t bytes) {
        const size_t o = off;
        off = align_up(off + bytes);
        return o;
    };
    if (d->flags & GDN_FLAG_QK_L2NORM)  // normalised k rows, first: the same offset in both layouts
        p.o_kn = take(T * H * K * p.esize);
    p.o_gam = take(T * H * 4);
    p.o_w = take(T * H * K * p.esize);
    p.o_u = take(T * H * V * p.esize);
    p.o_cstat = take((size_t)p.total_chunks * H * 8);
    p.o_modes = take((size_t)p.N * H * 4);  // CP mode per sequence-head [N,H]
    p.o_bwin = take((size_t)p.total_segs * H * 4);  // warmup window per boundary [total_segs,H]
    if (p.varlen) {
        p.o_bos = take((size_t)p.N * 8);
        p.o_len = take((size_t)p.N * 4);
        p.o_choff = take((size_t)(p.N + 1) * 4);
        p.o_segoff = take((size_t)(p.N + 1) * 4);
        p.o_ctab = take((size_t)p.total_chunks * 8);
        p.o_stab = take((size_t)p.total_segs * 16);
        // Longest sequences first in the recurrence grids (the one-dimensional grid's work-items,
        // at most 4 * H * V per segment, must fit 32 bits).
        p.seg_order = (int64_t)p.total_segs * H * V * 4 < ((int64_t)1 << 32);
        if (p.seg_order) p.o_sord = take((size_t)p.total_segs * 4);
    }
    if (p.cp_on) {
        p.o_seginit = take((size_t)p.total_segs * H * V * K * 4);
        p.o_prep = take((size_t)p.total_segs * H * (V + K) * K * 4);
        // the same three regions in the caller's desc->cp_states
        p.c_bwin = align_up((size_t)p.N * H * 4);
        p.c_seginit = p.c_bwin + align_up((size_t)p.total_segs * H * 4);
        p.cp_bytes = p.c_seginit + align_up((size_t)p.total_segs * H * V * K * 4);
    }
    if ((d->flags & GDN_FLAG_REUSE_CP) && p.cp_on && !d->cp_states) return GDN_ERR_INVALID_ARG;
    // T = (I + A)^{-1} per chunk, the chunk-entry states h and Delta = U - W S^T: written by
    // the forward when it keeps its intermediates, always by the backward (which reads them);
    // the same offsets in both layouts
    p.o_tm = take((size_t)p.total_chunks * H * 64 * 64 * p.esize);
    p.o_h = take((size_t)p.total_chunks * H * V * K * p.esize);
    p.o_dl = take(T * H * V * p.esize);
    p.fwd_bytes = std::max<size_t>((d->flags & GDN_FLAG_KEEP_FORWARD) ? off : p.o_tm, kAlign);
    // backward workspace continues after the forward's
    if (p.cp_on) {
        p.o_modes_r = take((size_t)p.N * H * 4);
        p.o_bwin_r = take((size_t)p.total_segs * H * 4);
        p.o_seginit_r = take((size_t)p.total_segs * H * V * K * 4);
        p.o_prep_r = take((size_t)p.total_segs * H * (V + K) * K * 4);
    }
    // The per-chunk backward kernel carries the adjoint itself (one workgroup per sub-sequence and
    // head, walking its chunks in reverse) where the sub-sequences are balanced: with CP, or uniform
    // batches. Then no adjoint pass runs, and the chunk-exit adjoints and dDelta take no space.
    p.carry = d->V == 128 && d->dtype == GDN_DTYPE_BF16 && (p.cp_on || !p.varlen) &&
              !(d->flags & GDN_FLAG_BWD_ADJOINT_PASS) && p.total_segs * d->H <= INT32_MAX;
    if (!p.carry) {
        p.o_gst = take((size_t)p.total_chunks * H * V * K * p.esize);
        p.o_ddl = take(T * H * V * p.esize);
    }
    p.bwd_bytes = std::max<size_t>(off, kAlign);
    p.bwd_ok = (d->dtype == GDN_DTYPE_BF16) || (d->K == 64 && d->V == 64);
    // The fully fused forward: possible without CP, in bf16, when nothing is kept for the backward;
    // chosen when the recurrence already needs at least two rounds of workgroups on the chip (then
    // the split's intra kernel no longer runs beside an idle recurrence, and the bytes decide).
    const bool fusable = !p.cp_on && d->dtype == GDN_DTYPE_BF16 && !(d->flags & GDN_FLAG_KEEP_FORWARD);
    if (d->flags & GDN_FLAG_FWD_FUSED) p.fused = fusable;
    else if (d->flags & GDN_FLAG_FWD_SPLIT) p.fused = 0;
    else p.fused = fusable && units >= 2 * target;
    return GDN_OK;
}

Geo make_geo(const gdn_desc* d, const Plan& p, unsigned char* ws) {
    Geo g;
    memset(&g, 0, sizeof(g));
    g.N = p.N;
    g.H = (int32_t)d->H;
    g.K = (int32_t)d->K;
    g.V = (int32_t)d->V;
    g.T = p.varlen ? p.Ttot : d->T;
    g.varlen = p.varlen;
    g.nt = p.nt;
    g.seg_len = p.seg_len;
    g.nseg = p.nseg;
    g.total_chunks = p.total_chunks;
    g.total_segs = p.total_segs;
    if (p.varlen) {
        g.seq_bos = reinterpret_cast<const int64_t*>(ws + p.o_bos);
        g.seq_len = reinterpret_cast<const int32_t*>(ws + p.o_len);
        g.seq_choff = reinterpret_cast<const int32_t*>(ws + p.o_choff);
        g.seq_segoff = reinterpret_cast<const int32_t*>(ws + p.o_segoff);
        g.chunk_tab = reinterpret_cast<const int2*>(ws + p.o_ctab);
        g.seg_tab = reinterpret_cast<const int4*>(ws + p.o_stab);
        if (p.seg_order) g.seg_order = reinterpret_cast<const int32_t*>(ws + p.o_sord);
    }
    return g;
}


#define GDN_TRY_HIP(x)                           \
    do {                                         \
        hipError_t e_ = (x);                     \
        if (e_ != hipSuccess) return GDN_ERR_HIP; \
    } while (0)

// ---------------------------------------------------------------------------
// Kernel timing (gdn_profile_enable / gdn_profile_read).
enum KernelId { kKTables = 0, kKIntra, kKDecide, kKPrepass, kKScan, kKRecurOut, kKRecurStates,
                kKBwdPrepass, kKBwdScan, kKBwdReverse, kKBwdChunk, kKDecode, kKL2NormBwd, kKFused, kKCount };
const char* const kKernelNames[kKCount] = {"tables", "intra", "cp_decide", "cp_prepass", "cp_scan",
                                           "recur_out", "recur_states", "bwd_cp_prepass", "bwd_cp_scan",
                                           "bwd_reverse", "bwd_chunk", "recurrent", "qk_l2norm_bwd", "fused_fwd"};
struct Pending {
    int kid;
    hipEvent_t start, stop;
};
struct Profiler {
    std::mutex mu;
    bool on = false;
    std::vector<hipEvent_t> pool;
    std::vector<Pending> pending;
    int64_t launches[kKCount] = {};
    double total_ms[kKCount] = {};
    hipEvent_t get() {
        if (!pool.empty()) {
            hipEvent_t e = pool.back();
            pool.pop_back();
            return e;
        }
        hipEvent_t e = nullptr;
        if (hipEventCreate(&e) != hipSuccess) return nullptr;
        return e;
    }
};
Profiler& profiler() {
    static Profiler p;
    return p;
}

// Brackets one launch with events when profiling is on.
struct ProfScope {
    int kid;
    hipStream_t st;
    hipEvent_t a = nullptr, b = nullptr;
    ProfScope(int k, hipStream_t s) : kid(k), st(s) {
        Profiler& p = profiler();
        std::lock_guard<std::mutex> g(p.mu);
        if (!p.on) return;
        a = p.get();
        b = p.get();
        if (a && b) (void)hipEventRecord(a, st);
    }
    ~ProfScope() {
        if (!a || !b) return;
        (void)hipEventRecord(b, st);
        Profiler& p = profiler();
        std::lock_guard<std::mutex> g(p.mu);
        p.pending.push_back(Pending{kid, a, b});
    }
};

#define GDN_LAUNCH(kid, st, call)         \
    do {                                  \
        ProfScope ps_(kid, st);           \
        hipError_t e_ = (call);           \
        if (e_ != hipSuccess) return GDN_ERR_HIP; \
    } while (0)

// A second stream per device, for the backward's two independent recurrences, with the
// two events that fork it from and join it to the caller's stream. Created on first use
// with the default priority and kept until the process ends. The caller holds side_mutex()
// from the fork to the join, so that concurrent callers do not interleave event records.
struct SideStream {
    hipStream_t s = nullptr;
    hipEvent_t fork = nullptr, join = nullptr;
};
constexpr int kMaxDevices = 64;
std::mutex& side_mutex() {
    static std::mutex m;
    return m;
}
gdn_status side_stream(hipStream_t st, SideStream& out) {
    static SideStream per_dev[kMaxDevices];
    int dev = -1, cur = -1;
    if (hipStreamGetDevice(st, &dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return GDN_ERR_HIP;
    SideStream& x = per_dev[dev];
    if (!x.s) {
        if (hipGetDevice(&cur) != hipSuccess) return GDN_ERR_HIP;
        if (cur != dev && hipSetDevice(dev) != hipSuccess) return GDN_ERR_HIP;
        SideStream y;
        bool ok = hipStreamCreateWithFlags(&y.s, hipStreamNonBlocking) == hipSuccess &&
                  hipEventCreateWithFlags(&y.fork, hipEventDisableTiming) == hipSuccess &&
                  hipEventCreateWithFlags(&y.join, hipEventDisableTiming) == hipSuccess;
        if (cur != dev && hipSetDevice(cur) != hipSuccess) ok = false;
        if (!ok) return GDN_ERR_HIP;  // (a partial set is not kept)
        x = y;
    }
    out = x;
    return GDN_OK;
}

gdn_status check_ws(const Plan& p, size_t need, void* ws, size_t bytes) {
    if (!ws || bytes < need) return GDN_ERR_WORKSPACE;
    if (reinterpret_cast<uintptr_t>(ws) % kAlign) return GDN_ERR_WORKSPACE;
    (void)p;
    return GDN_OK;
}

// GDN_FLAG_QK_L2NORM: the intra-chunk kernel normalises the k rows as it stages them and
// writes them here for the later kernels (null without the flag); the kernels that read q
// normalise its rows as they stage them (q_l2 in their arguments).
void* kn_of(const gdn_desc* d, const Plan& p, unsigned char* ws) {
    return (d->flags & GDN_FLAG_QK_L2NORM) ? ws + p.o_kn : nullptr;
}

// Where the forward-direction CP decisions (per sequence-head mode, per boundary window) and
// sub-sequence entry states live: the caller's desc->cp_states when set and `caller` (the
// forward always writes them there; a backward reads them there when it reuses the forward's
// results), else the workspace.
struct CpRegion {
    int32_t* modes;
    int32_t* bwin;
    float* seginit;  // null without CP
};
CpRegion cp_region(const gdn_desc* d, const Plan& p, unsigned char* ws, bool caller) {
    if (caller && d->cp_states && p.cp_on) {
        unsigned char* c = static_cast<unsigned char*>(d->cp_states);
        return {reinterpret_cast<int32_t*>(c), reinterpret_cast<int32_t*>(c + p.c_bwin),
                reinterpret_cast<float*>(c + p.c_seginit)};
    }
    return {reinterpret_cast<int32_t*>(ws + p.o_modes), reinterpret_cast<int32_t*>(ws + p.o_bwin),
            p.cp_on ? reinterpret_cast<float*>(ws + p.o_seginit) : nullptr};
}

// Tables (varlen) + intra-chunk kernel into the given output buffers.
// The varlen tables' arguments (built on the device from cu_seqlens into the workspace).
TableArgs table_args(const gdn_desc* d, const Plan& p, unsigned char* ws) {
    TableArgs t{};
    t.cu = d->cu_seqlens;
    t.N = p.N;
    t.Ttot = p.Ttot;
    t.seg_len = p.seg_len;
    t.total_chunks = p.total_chunks;
    t.total_segs = p.total_segs;
    t.seq_bos = reinterpret_cast<int64_t*>(ws + p.o_bos);
    t.seq_len = reinterpret_cast<int32_t*>(ws + p.o_len);
    t.seq_choff = reinterpret_cast<int32_t*>(ws + p.o_choff);
    t.seq_segoff = reinterpret_cast<int32_t*>(ws + p.o_segoff);
    t.chunk_tab = reinterpret_cast<int2*>(ws + p.o_ctab);
    t.seg_tab = reinterpret_cast<int4*>(ws + p.o_stab);
    t.seg_order = p.seg_order ? reinterpret_cast<int32_t*>(ws + p.o_sord) : nullptr;
    return t;
}

gdn_status run_intra(const gdn_desc* d, const Plan& p, unsigned char* ws, const void* k, const void* v,
                     const float* g, const float* beta, float* gam, void* w, void* u, hipStream_t st,
                     void* tmat = nullptr, void* kn = nullptr) {
    if (p.varlen) GDN_LAUNCH(kKTables, st, launch_tables(table_args(d, p, ws), st));
    IntraArgs ia{};
    ia.geo = make_geo(d, p, ws);
    ia.k = k;
    ia.v = v;
    ia.g = g;
    ia.beta = beta;
    ia.gam = gam;
    ia.w = w;
    ia.u = u;
    ia.cstat = reinterpret_cast<float2*>(ws + p.o_cstat);
    ia.tmat = tmat;
    ia.kn = kn;
    GDN_LAUNCH(kKIntra, st, launch_intra(ia, d->dtype, p.cus, st));
    return GDN_OK;
}

// The CP decision: per sequence-head modes [N,H] and per boundary windows [total_segs,H] in one
// direction, and optionally the other direction's (the backward's adjoint pass) in the same launch.
// The CP prepasses run on the ranked grid (sequence-heads with exact maps dispatched first)
// for uniform-length batches (its one dimension holds every workgroup).
int32_t prepass_ranked(const Plan& p) {
    return !p.varlen && (int64_t)p.N * p.H * p.nseg * 4 < ((int64_t)1 << 31) ? 1 : 0;
}

gdn_status run_decide(const gdn_desc* d, const Plan& p, unsigned char* ws, int32_t* modes, int32_t* bwin,
                      hipStream_t st, int reverse = 0, int32_t* modes_r = nullptr, int32_t* bwin_r = nullptr) {
    DecideArgs da{};
    da.reverse = reverse;
    da.modes_r = modes_r;
    da.bwin_r = bwin_r;
    da.geo = make_geo(d, p, ws);
    da.cstat = reinterpret_cast<const float2*>(ws + p.o_cstat);
    da.modes = modes;
    da.bwin = bwin;
    da.warmup = p.W;
    da.warmup_max = p.Wmax;
    da.log_eps = logf(p.eps);
    da.forced = p.forced;
    GDN_LAUNCH(kKDecide, st, launch_decide(da, st));
    return GDN_OK;
}

gdn_status run_fwd(const gdn_desc* desc, const Plan& p, const void* q, const void* k, const void* v,
                   const float* g, const float* beta, const float* initial_state, void* o, float* final_state,
                   unsigned char* ws, hipStream_t st);

// ---------------------------------------------------------------------------
// The forward's workspace for callers that cannot allocate (gdn_chunk_fwd_noalloc): a fixed
// device array, one copy per GPU, resolved once per device with that device current. In host
// code the array's name stands for a host-side shadow, not a device address: only the address
// hipGetSymbolAddress returns for the device is ever handed to a kernel.
constexpr size_t kNoAllocScratchBytes = GDN_NOALLOC_SCRATCH_BYTES;

}  // namespace

static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

namespace {

gdn_status noalloc_scratch(hipStream_t st, unsigned char** out) {
    static std::mutex mu;
    static unsigned char* per_dev[kMaxDevices] = {};
    int dev = -1;
    if (hipStreamGetDevice(st, &dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return GDN_ERR_HIP;
    std::lock_guard<std::mutex> lock(mu);
    if (!per_dev[dev]) {
        int cur = -1;
        if (hipGetDevice(&cur) != hipSuccess) return GDN_ERR_HIP;
        if (cur != dev && hipSetDevice(dev) != hipSuccess) return GDN_ERR_HIP;
        void* ptr = nullptr;
        const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (cur != dev && hipSetDevice(cur) != hipSuccess) return GDN_ERR_HIP;
        if (e != hipSuccess || !ptr || reinterpret_cast<uintptr_t>(ptr) % kAlign) return GDN_ERR_HIP;
        per_dev[dev] = static_cast<unsigned char*>(ptr);
    }
    *out = per_dev[dev];
    return GDN_OK;
}

}  // namespace
}  // namespace gdn

using namespace gdn;

extern "C" {

int gdn_abi_version(void) { return GDN_ABI_VERSION; }

const char* gdn_status_string(gdn_status s) {
    switch (s) {
        case GDN_OK: return "ok";
        case GDN_ERR_INVALID_ARG: return "invalid argument";
        case GDN_ERR_UNSUPPORTED: return "unsupported configuration";
        case GDN_ERR_WORKSPACE: return "workspace missing, misaligned or too small";
        case GDN_ERR_HIP: return "HIP runtime or kernel launch error";
    }
    return "unknown status";
}

gdn_status gdn_plan(const gdn_desc* desc, gdn_plan_info* out) {
    if (!out) return GDN_ERR_INVALID_ARG;
    Plan p;
    const gdn_status s = make_plan(desc, p);
    if (s != GDN_OK) return s;
    memset(out, 0, sizeof(*out));
    out->num_seqs = p.N;
    out->cp_on = p.cp_on;
    out->seg_chunks = p.seg_len;
    out->warmup_chunks = p.W;
    out->warmup_max_chunks = p.Wmax;
    out->warmup_eps = p.eps;
    out->v_tiles = (int32_t)(desc->V / recur_rows((int)desc->V, (int)desc->K));
    out->max_len = p.max_len;
    out->total_chunks = p.total_chunks;
    out->total_segments = p.total_segs;
    out->fwd_workspace_bytes = p.fwd_bytes;
    out->bwd_workspace_bytes = p.bwd_bytes;
    out->cp_states_bytes = p.cp_bytes;
    out->fused_fwd = p.fused;
    out->bwd_carried = p.carry;
    return GDN_OK;
}

gdn_status gdn_chunk_fwd_workspace_size(const gdn_desc* desc, size_t* bytes) {
    if (!bytes) return GDN_ERR_INVALID_ARG;
    Plan p;
    const gdn_status s = make_plan(desc, p);
    if (s != GDN_OK) return s;
    *bytes = p.fwd_bytes;
    return GDN_OK;
}

gdn_status gdn_chunk_fwd(const gdn_desc* desc, const void* q, const void* k, const void* v, const float* g,
                         const float* beta, const float* initial_state, void* o, float* final_state,
                         void* workspace, size_t workspace_bytes, void* stream) {
    Plan p;
    gdn_status s = make_plan(desc, p);
    if (s != GDN_OK) return s;
    if (p.Ttot > 0 && (!q || !k || !v || !g || !beta || !o)) return GDN_ERR_INVALID_ARG;
    if ((s = check_ws(p, p.fwd_bytes, workspace, workspace_bytes)) != GDN_OK) return s;
    return run_fwd(desc, p, q, k, v, g, beta, initial_state, o, final_state,
                   static_cast<unsigned char*>(workspace), reinterpret_cast<hipStream_t>(stream));
}

gdn_status gdn_chunk_fwd_noalloc(const gdn_desc* desc, const void* q, const void* k, const void* v, const float* g,
                                 const float* beta, const float* initial_state, void* o, float* final_state,
                                 void* stream) {
    Plan p;
    gdn_status s = make_plan(desc, p);
    if (s != GDN_OK) return s;
    // kept intermediates would be overwritten by the next call on the same GPU
    if (desc->flags & (GDN_FLAG_KEEP_FORWARD | GDN_FLAG_REUSE_FORWARD)) return GDN_ERR_INVALID_ARG;
    if (p.Ttot > 0 && (!q || !k || !v || !g || !beta || !o)) return GDN_ERR_INVALID_ARG;
    if (p.fwd_bytes > kNoAllocScratchBytes) return GDN_ERR_WORKSPACE;
    hipStream_t st = reinterpret_cast<hipStream_t>(stream);
    unsigned char* ws = nullptr;
    if ((s = noalloc_scratch(st, &ws)) != GDN_OK) return s;
    return run_fwd(desc, p, q, k, v, g, beta, initial_state, o, final_state, ws, st);
}

}  // extern "C"

namespace gdn {
namespace {

gdn_status run_fwd(const gdn_desc* desc, const Plan& p, const void* q, const void* k, const void* v,
                   const float* g, const float* beta, const float* initial_state, void* o, float* final_state,
                   unsigned char* ws, hipStream_t st) {
    gdn_status s = GDN_OK;
    if (p.fused) {
        if (p.varlen) GDN_LAUNCH(kKTables, st, launch_tables(table_args(desc, p, ws), st));
        RecurArgs fa{};
        memset(&fa, 0, sizeof(fa));
        fa.geo = make_geo(desc, p, ws);
        fa.q = q;
        fa.k = k;
        fa.fv = v;
        fa.fg = g;
        fa.fbeta = beta;
        fa.s0 = initial_state;
        fa.o = o;
        fa.sT = final_state;
        fa.scale = desc->scale;
        fa.q_l2 = (desc->flags & GDN_FLAG_QK_L2NORM) != 0;
        GDN_LAUNCH(kKFused, st, launch_fused(fa, desc->dtype, p.total_segs,
                                             (int)(desc->V / recur_rows((int)desc->V, (int)desc->K)), st));
        return GDN_OK;
    }
    float* gam = reinterpret_cast<float*>(ws + p.o_gam);
    void* w = ws + p.o_w;
    void* u = ws + p.o_u;
    // with GDN_FLAG_KEEP_FORWARD the intra pass also leaves T for the backward; with
    // GDN_FLAG_QK_L2NORM it normalises k and the later kernels read its copy
    void* kn = kn_of(desc, p, ws);
    if ((s = run_intra(desc, p, ws, k, v, g, beta, gam, w, u, st,
                       (desc->flags & GDN_FLAG_KEEP_FORWARD) ? ws + p.o_tm : nullptr, kn)) != GDN_OK)
        return s;
    if (kn) k = kn;

    RecurArgs ra{};
    memset(&ra, 0, sizeof(ra));
    ra.geo = make_geo(desc, p, ws);
    ra.q = q;
    ra.k = k;
    ra.gam = gam;
    ra.w = w;
    ra.u = u;
    ra.s0 = initial_state;
    ra.o = o;
    ra.sT = final_state;
    ra.scale = desc->scale;
    ra.use_cp = p.cp_on;
    ra.q_l2 = kn != nullptr;
    const CpRegion cpr = cp_region(desc, p, ws, true);
    int32_t* modes = cpr.modes;
    int32_t* bwin = cpr.bwin;
    ra.modes = modes;
    ra.bwin = bwin;
    if (p.cp_on) {
        float* seginit = cpr.seginit;
        float* prep = reinterpret_cast<float*>(ws + p.o_prep);
        if ((s = run_decide(desc, p, ws, modes, bwin, st)) != GDN_OK) return s;
        ra.seginit_out = seginit;
        ra.prep = prep;
        ra.ranked = prepass_ranked(p);
        const int rt = recur_rows((int)desc->V, (int)desc->K);
        GDN_LAUNCH(kKPrepass, st, launch_recur(ra, desc->dtype, kRecurPrepass, p.total_segs,
                                               (int)((desc->V + desc->K + rt - 1) / rt), st));
        ScanArgs sa{};
        sa.geo = ra.geo;
        sa.s0 = initial_state;
        sa.prep = prep;
        sa.seginit = seginit;
        sa.modes = modes;
        GDN_LAUNCH(kKScan, st, launch_scan(sa, desc->dtype, st));
        ra.seginit = seginit;
    }
    // a forward that keeps its intermediates also records h and Delta (where a backward exists)
    const bool rec = (desc->flags & GDN_FLAG_KEEP_FORWARD) && p.bwd_ok;
    if (rec) {
        ra.hstates = ws + p.o_h;
        ra.delta = ws + p.o_dl;
    }
    GDN_LAUNCH(kKRecurOut, st, launch_recur(ra, desc->dtype, rec ? kRecurOutRec : kRecurOut, p.total_segs,
                                            (int)(desc->V / recur_rows((int)desc->V, (int)desc->K)), st));
    return GDN_OK;
}

}  // namespace
}  // namespace gdn

extern "C" {

gdn_status gdn_chunk_bwd_workspace_size(const gdn_desc* desc, size_t* bytes) {
    if (!bytes) return GDN_ERR_INVALID_ARG;
    Plan p;
    const gdn_status s = make_plan(desc, p);
    if (s != GDN_OK) return s;
    if (!p.bwd_ok) return GDN_ERR_UNSUPPORTED;
    *bytes = p.bwd_bytes;
    return GDN_OK;
}

gdn_status gdn_chunk_bwd(const gdn_desc* desc, const void* q, const void* k, const void* v, const float* g,
                         const float* beta, const float* initial_state, const void* d_o,
                         const float* d_final_state, void* dq, void* dk, void* dv, float* dg, float* dbeta,
                         float* d_initial_state, void* workspace, size_t workspace_bytes, void* stream) {
    Plan p;
    gdn_status s = make_plan(desc, p);
    if (s != GDN_OK) return s;
    if (!p.bwd_ok) return GDN_ERR_UNSUPPORTED;
    if (p.Ttot > 0 && (!q || !k || !v || !g || !beta || !d_o || !dq || !dk || !dv || !dg || !dbeta))
        return GDN_ERR_INVALID_ARG;
    if ((s = check_ws(p, p.bwd_bytes, workspace, workspace_bytes)) != GDN_OK) return s;
    hipStream_t st = reinterpret_cast<hipStream_t>(stream);
    unsigned char* ws = static_cast<unsigned char*>(workspace);
    float* gam = reinterpret_cast<float*>(ws + p.o_gam);
    void* w = ws + p.o_w;
    void* u = ws + p.o_u;
    // 1. the forward's intra-chunk pass (kept by a GDN_FLAG_KEEP_FORWARD forward, or recomputed),
    // on the normalised q and k with GDN_FLAG_QK_L2NORM (kept too, at the same offsets)
    const bool reuse = (desc->flags & GDN_FLAG_REUSE_FORWARD) != 0;
    const void* k_raw = k;
    void* kn = kn_of(desc, p, ws);
    if (!reuse && (s = run_intra(desc, p, ws, k, v, g, beta, gam, w, u, st, ws + p.o_tm, kn)) != GDN_OK) return s;
    if (kn) k = kn;
    const int rt = recur_rows((int)desc->V, (int)desc->K);
    const int vtiles = (int)(desc->V / rt);
    const int vktiles = (int)((desc->V + desc->K + rt - 1) / rt);
    // The forward states pass (2) and the reverse adjoint pass (3) read only what the intra
    // pass wrote and write disjoint workspace regions: (3) runs on a second stream, forked
    // from the caller's after (1) and joined to it before (4).
    // both CP decisions (forward windows for the state pass, windows after each segment for
    // the adjoint pass) in one launch ahead of the fork
    // the forward-direction CP results come from the forward (kept workspace or desc->cp_states)
    // or are recomputed into the workspace
    const bool reuse_cp = reuse || (desc->flags & GDN_FLAG_REUSE_CP);
    const CpRegion cpr = cp_region(desc, p, ws, reuse_cp);
    int32_t* modes = cpr.modes;
    int32_t* bwin = cpr.bwin;
    int32_t* modes_r = p.cp_on ? reinterpret_cast<int32_t*>(ws + p.o_modes_r) : nullptr;
    int32_t* bwin_r = p.cp_on ? reinterpret_cast<int32_t*>(ws + p.o_bwin_r) : nullptr;
    if (p.cp_on) {
        if (reuse_cp) s = run_decide(desc, p, ws, modes_r, bwin_r, st, 1);
        else s = run_decide(desc, p, ws, modes, bwin, st, 0, modes_r, bwin_r);
        if (s != GDN_OK) return s;
    }
    // With the carried adjoint only the reverse CP (if any) goes to the side stream.
    const bool carry = p.carry != 0;
    const bool fork = p.cp_on || !carry;
    std::unique_lock<std::mutex> side_lock(side_mutex(), std::defer_lock);
    SideStream side;
    hipStream_t st2 = st;
    if (fork) {
        side_lock.lock();
        if ((s = side_stream(st, side)) != GDN_OK) return s;
        st2 = side.s;
        if (hipEventRecord(side.fork, st) != hipSuccess || hipStreamWaitEvent(st2, side.fork, 0) != hipSuccess)
            return GDN_ERR_HIP;
    }
    // Without CP the reverse adjoint pass walks whole sequences and is the longer chain: it goes
    // on the caller's stream, which the hardware reaches first after the fork, so that all its
    // workgroups (the longest sequences' too) take the chip at once and the states pass fills
    // in behind them; otherwise the forward-direction chain stays on the caller's stream.
    const bool swap = fork && !carry && !p.cp_on;
    const hipStream_t sm = swap ? st2 : st;  // the forward-direction chain (2)
    const hipStream_t sr2 = swap ? st : st2;  // the reverse chain (3)
    // 2. chunk-entry states and Delta, with the forward's CP (kept by the forward when reused)
    RecurArgs ra{};
    memset(&ra, 0, sizeof(ra));
    ra.geo = make_geo(desc, p, ws);
    ra.k = k;
    ra.gam = gam;
    ra.w = w;
    ra.u = u;
    ra.s0 = initial_state;
    ra.scale = desc->scale;
    ra.use_cp = p.cp_on;
    ra.modes = modes;
    ra.bwin = bwin;
    ra.hstates = ws + p.o_h;
    ra.delta = ws + p.o_dl;
    if (!reuse_cp && p.cp_on) {
        float* seginit = cpr.seginit;
        float* prep = reinterpret_cast<float*>(ws + p.o_prep);
        ra.seginit_out = seginit;
        ra.prep = prep;
        ra.ranked = prepass_ranked(p);
        GDN_LAUNCH(kKPrepass, sm, launch_recur(ra, desc->dtype, kRecurPrepass, p.total_segs, vktiles, sm));
        ScanArgs sa{};
        memset(&sa, 0, sizeof(sa));
        sa.geo = ra.geo;
        sa.s0 = initial_state;
        sa.prep = prep;
        sa.seginit = seginit;
        sa.modes = modes;
        GDN_LAUNCH(kKScan, sm, launch_scan(sa, desc->dtype, sm));
        ra.seginit = seginit;
    } else if (p.cp_on) {
        ra.seginit = cpr.seginit;
    }
    if (!reuse) GDN_LAUNCH(kKRecurStates, sm, launch_recur(ra, desc->dtype, kRecurStates, p.total_segs, vtiles, sm));
    // 3. reverse adjoint pass, with CP mirrored (windows and scan from the sequence end)
    const gdn_status sr = [&]() -> gdn_status {
    hipStream_t st = sr2;
    RevArgs va;
    memset(&va, 0, sizeof(va));
    va.geo = ra.geo;
    va.q = q;
    va.k = k;
    va.gam = gam;
    va.w = w;
    va.d_o = d_o;
    va.dsT = d_final_state;
    va.ds0 = d_initial_state;
    va.gstates = carry ? nullptr : ws + p.o_gst;
    va.ddelta = carry ? nullptr : ws + p.o_ddl;
    va.scale = desc->scale;
    va.use_cp = p.cp_on;
    va.q_l2 = kn != nullptr;
    if (p.cp_on) {
        float* seginit_r = reinterpret_cast<float*>(ws + p.o_seginit_r);
        float* prep_r = reinterpret_cast<float*>(ws + p.o_prep_r);
        va.modes = modes_r;
        va.bwin = bwin_r;
        va.seginit_out = seginit_r;
        va.prep = prep_r;
        va.ranked = prepass_ranked(p);
        GDN_LAUNCH(kKBwdPrepass, st, launch_reverse(va, desc->dtype, kRecurPrepass, p.total_segs, vktiles, st));
        ScanArgs sa{};
        memset(&sa, 0, sizeof(sa));
        sa.geo = ra.geo;
        sa.s0 = d_final_state;
        sa.prep = prep_r;
        sa.seginit = seginit_r;
        sa.modes = modes_r;
        sa.reverse = 1;
        GDN_LAUNCH(kKBwdScan, st, launch_scan(sa, desc->dtype, st));
        va.seginit = seginit_r;
    }
    if (!carry) GDN_LAUNCH(kKBwdReverse, st, launch_reverse(va, desc->dtype, kRecurOut, p.total_segs, vtiles, st));
    return GDN_OK;
    }();
    // join, also after a failed launch on the side stream
    if (fork && (hipEventRecord(side.join, st2) != hipSuccess || hipStreamWaitEvent(st, side.join, 0) != hipSuccess))
        return GDN_ERR_HIP;
    if (sr != GDN_OK) return sr;
    // 4. per-chunk gradients
    BwdChunkArgs ba;
    memset(&ba, 0, sizeof(ba));
    ba.geo = ra.geo;
    ba.q = q;
    ba.k = k;
    ba.v = v;
    ba.g = g;
    ba.beta = beta;
    ba.gam = gam;
    ba.d_o = d_o;
    ba.delta = ws + p.o_dl;
    ba.ddelta = carry ? nullptr : ws + p.o_ddl;
    ba.hstates = ws + p.o_h;
    ba.gstates = carry ? nullptr : ws + p.o_gst;
    ba.tmat = ws + p.o_tm;
    ba.dq = dq;
    ba.dk = dk;
    ba.dv = dv;
    ba.dg = dg;
    ba.dbeta = dbeta;
    ba.scale = desc->scale;
    ba.q_l2 = kn != nullptr;
    ba.carry = carry;
    ba.use_cp = p.cp_on;
    ba.seginit_r = p.cp_on ? reinterpret_cast<const float*>(ws + p.o_seginit_r) : nullptr;
    ba.dsT = d_final_state;
    ba.ds0 = d_initial_state;
    const int64_t tasks = p.total_chunks * (int64_t)desc->H;
    GDN_LAUNCH(kKBwdChunk, st, launch_bwd_chunk(ba, desc->dtype, (int)std::min<int64_t>(tasks, p.cus), st));
    // 5. dq and dk back through the normalisation to the raw rows, in place
    if ((desc->flags & GDN_FLAG_QK_L2NORM) && p.Ttot > 0) {
        NormArgs na{};
        na.x0 = q;
        na.y0 = dq;
        na.x1 = k_raw;
        na.y1 = dk;
        na.rows0 = na.rows1 = p.Ttot * (int64_t)desc->H;
        GDN_LAUNCH(kKL2NormBwd, st, launch_l2norm_bwd(na, desc->dtype, (int)desc->K, st));
    }
    return GDN_OK;
}

gdn_status gdn_recurrent_fwd(const gdn_desc* desc, const void* q, const void* k, const void* v, const float* g,
                             const float* beta, const float* state_in, float* state_out, void* o, void* stream) {
    if (!desc) return GDN_ERR_INVALID_ARG;
    for (int i = 0; i < 5; ++i)
        if (desc->reserved[i] != 0) return GDN_ERR_INVALID_ARG;
    if (desc->cu_seqlens || desc->cu_seqlens_host || desc->cp_states || (desc->flags & ~GDN_FLAG_QK_L2NORM))
        return GDN_ERR_INVALID_ARG;
    if (desc->B < 1 || desc->T < 0 || desc->H < 1 || desc->K < 1 || desc->V < 1) return GDN_ERR_INVALID_ARG;
    if (!(desc->K == 64 || desc->K == 128) || !(desc->V == 64 || desc->V == 128)) return GDN_ERR_UNSUPPORTED;
    if (desc->dtype != GDN_DTYPE_BF16 && desc->dtype != GDN_DTYPE_FP32) return GDN_ERR_INVALID_ARG;
    if (!isfinite(desc->scale)) return GDN_ERR_INVALID_ARG;
    if (desc->B > INT32_MAX || desc->H > 65535) return GDN_ERR_UNSUPPORTED;
    if (!state_out || (desc->T > 0 && (!q || !k || !v || !g || !beta || !o))) return GDN_ERR_INVALID_ARG;
    DecodeArgs da{};
    da.q = q;
    da.k = k;
    da.v = v;
    da.g = g;
    da.beta = beta;
    da.s_in = state_in;
    da.s_out = state_out;
    da.o = o;
    da.B = desc->B;
    da.T = desc->T;
    da.H = desc->H;
    da.scale = desc->scale;
    hipStream_t st = reinterpret_cast<hipStream_t>(stream);
    if (desc->flags & GDN_FLAG_QK_L2NORM)
        GDN_LAUNCH(kKDecode, st, launch_decode_qk_l2norm(da, desc->dtype, (int)desc->K, (int)desc->V, st));
    else
        GDN_LAUNCH(kKDecode, st, launch_decode(da, desc->dtype, (int)desc->K, (int)desc->V, st));
    return GDN_OK;
}

gdn_status gdn_intra_chunk(const gdn_desc* desc, const void* k, const void* v, const float* g,
                           const float* beta, float* gam_out, void* w_out, void* u_out, void* workspace,
                           size_t workspace_bytes, void* stream) {
    Plan p;
    gdn_status s = make_plan(desc, p);
    if (s != GDN_OK) return s;
    if (p.Ttot > 0 && (!k || !v || !g || !beta || !gam_out || !w_out || !u_out)) return GDN_ERR_INVALID_ARG;
    if ((s = check_ws(p, p.fwd_bytes, workspace, workspace_bytes)) != GDN_OK) return s;
    unsigned char* ws = static_cast<unsigned char*>(workspace);
    hipStream_t st = reinterpret_cast<hipStream_t>(stream);
    return run_intra(desc, p, ws, k, v, g, beta, gam_out, w_out, u_out, st, nullptr, kn_of(desc, p, ws));
}

gdn_status gdn_cp_modes(const gdn_desc* desc, const void* k, const void* v, const float* g, const float* beta,
                        int32_t* modes_out, void* workspace, size_t workspace_bytes, void* stream) {
    Plan p;
    gdn_status s = make_plan(desc, p);
    if (s != GDN_OK) return s;
    if (!modes_out || (p.Ttot > 0 && (!k || !v || !g || !beta))) return GDN_ERR_INVALID_ARG;
    if ((s = check_ws(p, p.fwd_bytes, workspace, workspace_bytes)) != GDN_OK) return s;
    hipStream_t st = reinterpret_cast<hipStream_t>(stream);
    unsigned char* ws = static_cast<unsigned char*>(workspace);
    if ((s = run_intra(desc, p, ws, k, v, g, beta, reinterpret_cast<float*>(ws + p.o_gam), ws + p.o_w,
                       ws + p.o_u, st, nullptr, kn_of(desc, p, ws))) != GDN_OK)
        return s;
    return run_decide(desc, p, ws, modes_out, reinterpret_cast<int32_t*>(ws + p.o_bwin), st);
}

gdn_status gdn_cp_windows(const gdn_desc* desc, const void* k, const void* v, const float* g, const float* beta,
                          int32_t* fwd_windows, int32_t* rev_windows, void* workspace, size_t workspace_bytes,
                          void* stream) {
    Plan p;
    gdn_status s = make_plan(desc, p);
    if (s != GDN_OK) return s;
    if (!fwd_windows || (p.Ttot > 0 && (!k || !v || !g || !beta))) return GDN_ERR_INVALID_ARG;
    if ((s = check_ws(p, p.fwd_bytes, workspace, workspace_bytes)) != GDN_OK) return s;
    hipStream_t st = reinterpret_cast<hipStream_t>(stream);
    unsigned char* ws = static_cast<unsigned char*>(workspace);
    if ((s = run_intra(desc, p, ws, k, v, g, beta, reinterpret_cast<float*>(ws + p.o_gam), ws + p.o_w,
                       ws + p.o_u, st, nullptr, kn_of(desc, p, ws))) != GDN_OK)
        return s;
    // the per sequence-head summaries of both directions land in the forward workspace's modes
    // array (the reverse one last, from the same thread)
    int32_t* modes = reinterpret_cast<int32_t*>(ws + p.o_modes);
    return run_decide(desc, p, ws, modes, fwd_windows, st, 0, rev_windows ? modes : nullptr, rev_windows);
}

gdn_status gdn_profile_enable(int enable) {
    Profiler& p = profiler();
    std::lock_guard<std::mutex> g(p.mu);
    p.on = enable != 0;
    return GDN_OK;
}

int gdn_profile_read(gdn_kernel_time* out, int max_entries) {
    Profiler& p = profiler();
    std::lock_guard<std::mutex> g(p.mu);
    int rc = 0;
    for (const Pending& e : p.pending) {
        float ms = 0.f;
        if (hipEventSynchronize(e.stop) != hipSuccess || hipEventElapsedTime(&ms, e.start, e.stop) != hipSuccess)
            rc = -1;
        p.launches[e.kid] += 1;
        p.total_ms[e.kid] += ms;
        p.pool.push_back(e.start);
        p.pool.push_back(e.stop);
    }
    p.pending.clear();
    if (rc < 0) return -1;
    int n = 0;
    for (int k = 0; k < kKCount; ++k) {
        if (p.launches[k] == 0) continue;
        if (out && n < max_entries) {
            memset(&out[n], 0, sizeof(out[n]));
            strncpy(out[n].name, kKernelNames[k], sizeof(out[n].name) - 1);
            out[n].launches = p.launches[k];
            out[n].total_ms = p.total_ms[k];
            ++n;
        }
        p.launches[k] = 0;
        p.total_ms[k] = 0.0;
    }
    return n;
}

}  // extern "C"
