/*
 * gdn.h -- C ABI of libgdn: Gated DeltaNet (GDN) chunked prefill, forward and
 * backward, on one AMD Instinct MI355X (gfx950).
 *
 * The operation. The FlashQLA pages describe a linear-attention kernel library
 * for the Gated Delta Network's chunked prefill (ollai.cn article, sections
 * "what it is" and "main features"): it takes q, k, v, a gate g and a write
 * strength beta, returns O and the final state, and accepts an optional
 * initial state and packed variable-length sequences via cu_seqlens
 * ("how to use"). It offers low-level forward / backward entry points
 * ("main features", two-level API). The pages print no formula; this library
 * computes the standard gated delta rule, per sequence and head,
 *
 *     S_t = exp(g_t) S_{t-1} (I - beta_t k_t k_t^T) + beta_t v_t k_t^T
 *     o_t = scale * S_t q_t
 *
 * S is V x K (row i over the value dimension, column j over the key
 * dimension). The state enters as initial_state (zeros when NULL) and leaves
 * as final_state. g is a natural-log decay (exp(g_t) multiplies the state).
 * q and k are used as given (no normalisation inside).
 *
 * Layouts (all row-major, contiguous, device memory unless stated):
 *   q, k, dq, dk        [B, T, H, K]   element type desc->dtype
 *   v, o, d_o, dv       [B, T, H, V]   element type desc->dtype
 *   g, beta, dg, dbeta  [B, T, H]      fp32
 *   initial_state, final_state, d_final_state, d_initial_state
 *                       [N, H, V, K]   fp32, N = number of sequences
 *   With varlen (cu_seqlens != NULL) B must be 1, T is the packed token count
 *   and sequence n owns tokens [cu_seqlens[n], cu_seqlens[n+1]).
 *
 * How it runs (the split the pages describe in "technical principles" and
 * "core advantages"): a gate-cumsum + intra-chunk kernel writes the WY factors
 * w and u, an optional intra-card context-parallel (CP) preprocessing step
 * gives every sub-sequence its initial state, and an inter-chunk recurrence
 * kernel produces O and the final state. CP turns on by itself for small
 * batch x heads ("AutoCP"; the pages' thresholds, B*H <= 40 or B*H <= 56 with
 * seq_len >= 8192, were tuned for a 132-SM part: here the default turns CP on when
 * the recurrence would otherwise leave compute units idle, GDN_CP_PAGES keeps the
 * pages' rule) and picks per sub-sequence boundary either the exact correction or a
 * sliding-window warmup of a few chunks where the gate decay makes the warmup exact within
 * tolerance ("gate-driven" warmup, "core advantages").
 *
 * Ownership and errors: the caller allocates every buffer, including the
 * workspace, whose size the *_workspace_size calls return. The library
 * allocates no memory (gdn_chunk_fwd_noalloc's fixed scratch array is part of
 * the library's image, see there), keeps no pointer after a call returns, never
 * synchronises the host with the device and never aborts. All work is
 * enqueued on `stream` (a hipStream_t; NULL = the default stream). Outputs
 * are overwritten, never accumulated, and must not alias inputs. Argument
 * checks run on the host before any launch; a failed launch reports
 * GDN_ERR_HIP. Results are deterministic (no atomics).
 */
#ifndef GDN_H_
#define GDN_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define GDN_ABI_VERSION 10

typedef enum gdn_status {
    GDN_OK = 0,
    GDN_ERR_INVALID_ARG = 1, /* null pointer, bad size, inconsistent cu_seqlens */
    GDN_ERR_UNSUPPORTED = 2, /* K or V not in {64,128}, chunk != 64, sizes beyond 32-bit grids */
    GDN_ERR_WORKSPACE = 3,   /* workspace NULL or smaller than required */
    GDN_ERR_HIP = 4          /* a HIP call or kernel launch failed */
} gdn_status;

typedef enum gdn_dtype {
    GDN_DTYPE_BF16 = 0, /* q,k,v,o and their gradients in bf16; fp32 accumulation and state */
    GDN_DTYPE_FP32 = 1  /* everything fp32 */
} gdn_dtype;

typedef enum gdn_cp_mode {
    GDN_CP_AUTO = 0,   /* CP when the recurrence would leave compute units idle without it: the
                          sequence-heads' row tiles fill at most half of its workgroup slots
                          and the longest sequence spans two sub-sequences of 16 chunks or
                          more; or, for packed sequences, when the longest one takes 1.5x
                          (and at least 64) the chunk steps per slot the batch needs, in
                          sub-sequences of half that (at least 32); a gate test at every
                          sub-sequence boundary picks warmup or exact there */
    GDN_CP_OFF = 1,    /* one serial pass per sequence-head */
    GDN_CP_ON = 2,     /* CP regardless of the shape rule; per-boundary gate test. Without
                          seg_chunks, a batch that already fills the slots takes sub-sequences
                          of half the chunk steps per slot it needs (at least 16) */
    GDN_CP_EXACT = 3,  /* CP, exact correction for every sequence-head */
    GDN_CP_WARMUP = 4, /* CP, warmup for every sequence-head (caller asserts fast decay) */
    GDN_CP_PAGES = 5   /* the pages' AutoCP thresholds, tuned for a 132-SM part: CP iff
                          N*H <= 40, or N*H <= 56 and the longest sequence >= 8192 tokens */
} gdn_cp_mode;

/* desc->flags: keeping the forward's intermediates for the backward of a training step.
 * GDN_FLAG_KEEP_FORWARD    gdn_chunk_fwd leaves in its workspace what the backward
 *                          recomputes otherwise: the chunk gate cumsums, w, u, T = (I+A)^-1,
 *                          the CP decisions, the sub-sequence entry states, every chunk's
 *                          entry state and Delta = U - W S^T (the forward workspace then
 *                          includes room for T, the states and Delta).
 * GDN_FLAG_REUSE_FORWARD   gdn_chunk_bwd starts from them instead of recomputing the
 *                          intra-chunk pass, the forward CP preprocessing and the chunk-state
 *                          pass. The caller
 *                          guarantees that the same workspace last held a KEEP_FORWARD
 *                          forward of the same inputs and descriptor (flags aside), with
 *                          no other call on it since except REUSE_FORWARD backwards. */
#define GDN_FLAG_KEEP_FORWARD 1
#define GDN_FLAG_REUSE_FORWARD 2

/* GDN_FLAG_QK_L2NORM: q and k are raw; the path scales every row of K values (one token,
 * one head) to x / sqrt(sum x^2 + 1e-6) and runs on those rows, the preprocessing the pages place
 * ahead of the fused kernels (edge.aivizor.me community post, its account of the chunked-prefill
 * pipeline) with the unit-norm q and k their workloads use. The kernels normalise the rows as
 * they stage them; the intra-chunk kernel writes the normalised k rows once for the later ones,
 * at the start of the workspace (T x H x K values in the input dtype more, in both layouts).
 * gdn_chunk_bwd then returns dq and dk with respect to the raw q and k:
 * dx = r (dxhat - xhat (xhat . dxhat)), r = (sum x^2 + 1e-6)^(-1/2). With
 * GDN_FLAG_REUSE_FORWARD the normalised k rows come from the kept forward, which must have had
 * this flag too. gdn_intra_chunk and gdn_cp_modes normalise k; gdn_recurrent_fwd normalises q
 * and k inside its kernel (fp32 rows, not rounded to the input dtype). */
#define GDN_FLAG_QK_L2NORM 4

/* GDN_FLAG_BWD_ADJOINT_PASS: gdn_chunk_bwd runs the reverse adjoint recurrence as a pass of its
 * own that stores every chunk's adjoint and dDelta for the per-chunk gradient kernel. By default,
 * at V = 128 in bf16 with CP on or a uniform batch, the per-chunk gradient kernel carries the
 * adjoint itself (one workgroup per sub-sequence and head walking its chunks in reverse), which
 * moves fewer bytes; the flag keeps the other path selectable, for comparison. Same results within
 * rounding. */
#define GDN_FLAG_BWD_ADJOINT_PASS 8

/* The fully fused forward: with CP off, bf16 inputs and no kept intermediates, gdn_chunk_fwd can run
 * the intra-chunk step and the recurrence in one kernel (one workgroup per sequence, head and row
 * tile, walking the chunks in order), so w, u and the gate cumsum never go to memory: 1,032 instead
 * of 2,320 bytes per token-head at K = V = 128. The pages name the fully fused design as the one
 * with less memory I/O at large batch (announcement post, on the two-kernel split). The plan picks it
 * where it measures faster (gdn_plan_info.fused_fwd); GDN_FLAG_FWD_FUSED asks for it wherever it is
 * supported, GDN_FLAG_FWD_SPLIT never. Same results within rounding. */
#define GDN_FLAG_FWD_FUSED 16
#define GDN_FLAG_FWD_SPLIT 32

/* Carrying the forward's CP results to the backward (a checkpoint of a few MB instead of the
 * intra-chunk intermediates): with CP on, the backward's chunk-state pass needs the same
 * sub-sequence entry states that the forward's CP preprocessing (decision, prepass, segment scan;
 * ollai.cn article, "technical principles") already produced. gdn_chunk_fwd writes its CP
 * decisions and those states to desc->cp_states when that pointer is set; gdn_chunk_bwd with
 * GDN_FLAG_REUSE_CP reads them from there instead of running the forward-direction
 * preprocessing again (it still recomputes the intra-chunk pass and decides the reverse
 * direction itself). The caller guarantees that a gdn_chunk_fwd of the same inputs and
 * descriptor (flags aside) last wrote the buffer. A GDN_FLAG_REUSE_FORWARD backward reads them
 * there too when the pointer is set (its forward wrote them there); any other backward leaves
 * the buffer alone. Without CP the flag does nothing and the buffer is not touched.
 * GDN_FLAG_REUSE_CP with CP on and desc->cp_states NULL returns GDN_ERR_INVALID_ARG. */
#define GDN_FLAG_REUSE_CP 64

/* Problem descriptor. Zero-initialise, then fill. */
typedef struct gdn_desc {
    int64_t B, T, H, K, V;          /* batch, tokens per row (packed total if varlen), heads, key dim, value dim */
    int32_t chunk;                  /* chunk length; must be 64 (0 = 64) */
    int32_t dtype;                  /* gdn_dtype */
    float scale;                    /* query scale applied to o (the rule above has none: pass 1.0) */
    int32_t num_seqs;               /* varlen: N (>= 1); ignored otherwise */
    const int32_t* cu_seqlens;      /* device [N+1] token offsets, or NULL (then N = B) */
    const int32_t* cu_seqlens_host; /* host copy of cu_seqlens; required with it (planning needs no sync) */
    int32_t cp_mode;                /* gdn_cp_mode */
    int32_t warmup_chunks;          /* warmup window in chunks, 1..16 (0 = 8) */
    int32_t seg_chunks;             /* CP sub-sequence length in chunks (0 = chosen from the CU count) */
    float warmup_eps;               /* warmup acceptance: exp(window gate sum) <= eps (0 = 1e-4 bf16, 1e-6 fp32) */
    int32_t num_cus;                /* compute units to plan for (0 = query the current device) */
    int32_t flags;                  /* GDN_FLAG_* (0 = none) */
    int32_t warmup_max_chunks;      /* longest warmup window a sequence-head may take when
                                       warmup_chunks do not meet the acceptance bound (AUTO, ON):
                                       warmup_chunks..warmup_chunks+63, or 0 = the sub-sequence
                                       length (at least warmup_chunks, at most warmup_chunks+63);
                                       equal to warmup_chunks keeps one fixed window */
    int32_t reserved[5];            /* must be zero */
    void* cp_states;                /* device buffer of gdn_plan_info.cp_states_bytes bytes, 256-byte
                                       aligned, or NULL: see GDN_FLAG_REUSE_CP (owned by the caller;
                                       gdn_recurrent_fwd requires NULL) */
} gdn_desc;

/* Host-side plan of a call (filled by gdn_plan; no device work). */
typedef struct gdn_plan_info {
    int32_t num_seqs;               /* N */
    int32_t cp_on;                  /* 1 if the call splits sequences into sub-sequences */
    int32_t seg_chunks;             /* chunks per sub-sequence (the last one may be shorter) */
    int32_t warmup_chunks;          /* warmup window W in chunks (the shortest one taken) */
    int32_t warmup_max_chunks;      /* longest warmup window a sequence-head may take */
    float warmup_eps;               /* warmup acceptance threshold */
    int32_t v_tiles;                /* value-row tiles per sequence-head in the recurrence kernel */
    int64_t max_len;                /* longest sequence, tokens */
    int64_t total_chunks;           /* sum over sequences of ceil(len / 64) */
    int64_t total_segments;         /* sum over sequences of sub-sequence counts */
    size_t fwd_workspace_bytes;
    size_t bwd_workspace_bytes;
    size_t cp_states_bytes;         /* size of desc->cp_states (CP decisions and sub-sequence entry
                                       states, fp32 [total_segments, H, V, K]); 0 when CP is off */
    int32_t fused_fwd;              /* 1 if gdn_chunk_fwd runs the fully fused forward */
    int32_t bwd_carried;            /* 1 if gdn_chunk_bwd's per-chunk kernel carries the adjoint
                                       (no separate adjoint pass) */
    int32_t reserved_out[2];
} gdn_plan_info;

/* ABI version (GDN_ABI_VERSION of the built library). */
int gdn_abi_version(void);

/* Static English text for a status code; never NULL. */
const char* gdn_status_string(gdn_status status);

/* Validate `desc` and fill `out` with the plan the calls below would use:
 * whether CP is on (AutoCP, "core advantages"; see gdn_cp_mode), sub-sequence
 * length, warmup window and workspace sizes. Host only: reads
 * cu_seqlens_host, never cu_seqlens; queries the device CU count only when
 * desc->num_cus == 0. */
gdn_status gdn_plan(const gdn_desc* desc, gdn_plan_info* out);

/* Workspace bytes that gdn_chunk_fwd needs for `desc`. */
gdn_status gdn_chunk_fwd_workspace_size(const gdn_desc* desc, size_t* bytes);

/* Forward (the pages' low-level fwd entry, "main features"): O and the final
 * state of the gated delta rule above.
 *   q, k, v, g, beta : inputs (layouts above)
 *   initial_state    : [N,H,V,K] fp32 or NULL (zeros)
 *   o                : output [B,T,H,V]
 *   final_state      : output [N,H,V,K] fp32, or NULL (not written)
 *   workspace        : device scratch of at least gdn_chunk_fwd_workspace_size bytes, 256-byte aligned
 *                      (with GDN_FLAG_KEEP_FORWARD, the one the backward will receive)
 *   stream           : hipStream_t (NULL = default stream)
 * Returns GDN_OK once all work is enqueued. */
gdn_status gdn_chunk_fwd(const gdn_desc* desc, const void* q, const void* k, const void* v,
                         const float* g, const float* beta, const float* initial_state,
                         void* o, float* final_state,
                         void* workspace, size_t workspace_bytes, void* stream);

/* For callers that cannot allocate device memory (code under HIP graph capture, serving loops
 * or harnesses that forbid hipMalloc): gdn_chunk_fwd with its workspace taken from a fixed
 * array inside the library, GDN_NOALLOC_SCRATCH_BYTES per GPU, which each GPU the call runs
 * on holds from the first call there until the process ends (that first call resolves the
 * array's address: make it once before capturing a graph). Same arguments, layouts and
 * results as gdn_chunk_fwd without the workspace; the caller still owns every input and
 * output. It allocates nothing.
 * Errors: a descriptor whose forward workspace (gdn_chunk_fwd_workspace_size) exceeds
 * GDN_NOALLOC_SCRATCH_BYTES returns GDN_ERR_WORKSPACE, and GDN_FLAG_KEEP_FORWARD or
 * GDN_FLAG_REUSE_FORWARD returns GDN_ERR_INVALID_ARG (kept intermediates would not outlive
 * the next call), both before any launch; otherwise as gdn_chunk_fwd.
 * Every call on one GPU shares that GPU's array, and the array keeps the last call's contents
 * (nothing in it needs to start at zero: every kernel writes what it reads in the same call).
 * Calls that overlap on one GPU (on different streams, or from several host threads) race on
 * the array: the caller serialises them. */
#define GDN_NOALLOC_SCRATCH_BYTES ((size_t)128 << 20)
gdn_status gdn_chunk_fwd_noalloc(const gdn_desc* desc, const void* q, const void* k, const void* v,
                                 const float* g, const float* beta, const float* initial_state,
                                 void* o, float* final_state, void* stream);

/* Workspace bytes that gdn_chunk_bwd needs for `desc`. */
gdn_status gdn_chunk_bwd_workspace_size(const gdn_desc* desc, size_t* bytes);

/* Backward (the pages' low-level bwd entry): gradients of
 * L = <d_o, O> + <d_final_state, final_state> with respect to every input.
 *   q, k, v, g, beta, initial_state : the forward's inputs (initial_state may be NULL)
 *   d_o             : [B,T,H,V] upstream gradient of O
 *   d_final_state   : [N,H,V,K] fp32 upstream gradient of the final state, or NULL (zeros)
 *   dq, dk, dv      : outputs, same layouts and dtype as q, k, v
 *   dg, dbeta       : outputs [B,T,H] fp32 (dg is with respect to the raw per-token g)
 *   d_initial_state : output [N,H,V,K] fp32, or NULL (not written)
 * The forward is recomputed inside, unless desc->flags has GDN_FLAG_REUSE_FORWARD (then the
 * intra-chunk pass and the forward CP preprocessing come from the workspace; see above) or
 * GDN_FLAG_REUSE_CP (then the forward CP preprocessing comes from desc->cp_states).
 * The reverse adjoint pass runs on a second stream of the library's (one per device, made on
 * the first call with the default priority), forked from `stream` and joined back to it
 * before the per-chunk gradients: work enqueued on `stream` afterwards sees every output.
 * Concurrent calls from several host threads are serialised while they enqueue. */
gdn_status gdn_chunk_bwd(const gdn_desc* desc, const void* q, const void* k, const void* v,
                         const float* g, const float* beta, const float* initial_state,
                         const void* d_o, const float* d_final_state,
                         void* dq, void* dk, void* dv, float* dg, float* dbeta,
                         float* d_initial_state,
                         void* workspace, size_t workspace_bytes, void* stream);

/* Recurrent form: the gated delta rule token by token from a given state, for decoding
 * after a prefill (the pages' interface continues a call from the previous one's state,
 * ollai.cn article, "how to use"). Every sequence b has desc->T tokens (T >= 0; a decoder
 * passes 1 or a few); no cu_seqlens, no CP, no workspace; desc->flags 0 or GDN_FLAG_QK_L2NORM
 * (raw q and k, normalised per token as in gdn_chunk_fwd).
 *   q, k [B,T,H,K]; v, o [B,T,H,V] (desc->dtype); g, beta [B,T,H] fp32 (layouts above)
 *   state_in  : [B,H,V,K] fp32 state entering the first token, or NULL (zeros); typically
 *               the final_state of gdn_chunk_fwd or of the previous call
 *   state_out : [B,H,V,K] fp32 state after the last token (required); may be state_in
 *               itself (updated in place)
 * One workgroup per (sequence, head) keeps its state in registers across the T tokens; the
 * state is read and written once per call. Same status codes as the calls above (K, V not
 * in {64,128}: GDN_ERR_UNSUPPORTED). */
gdn_status gdn_recurrent_fwd(const gdn_desc* desc, const void* q, const void* k, const void* v,
                             const float* g, const float* beta, const float* state_in,
                             float* state_out, void* o, void* stream);

/* Intra-chunk step alone (the first fused kernel): chunk-local cumulative gate
 * sum and the WY factors, for kernel-level checks. With gam the chunk-local
 * cumsum of g, A = strict_lower(diag(beta) (exp(gam_r - gam_j) k_r.k_j)) and
 * T = (I + A)^-1 per chunk:
 *   gam_out [B,T,H] fp32; w_out = T diag(beta exp(gam)) K  [B,T,H,K];
 *   u_out   = T diag(beta) V  [B,T,H,V]  (dtype desc->dtype).
 * Uses the forward workspace. */
gdn_status gdn_intra_chunk(const gdn_desc* desc, const void* k, const void* v,
                           const float* g, const float* beta,
                           float* gam_out, void* w_out, void* u_out,
                           void* workspace, size_t workspace_bytes, void* stream);

/* CP decision per sequence-head, as the forward would take it. The decision is made per
 * boundary (the start of every sub-sequence but a sequence's first): the warmup over the
 * shortest window from warmup_chunks to warmup_max_chunks chunks that meets the acceptance
 * bound there, else the exact correction ("gate-driven" warmup, ollai.cn article, "core
 * advantages"); the exact maps and the scan then run only across the exact boundaries.
 * modes_out [N, H] int32 (device): 0 = no split needed, 1 = every boundary takes the warmup,
 * 2 = every boundary takes the exact correction, 3 = both kinds (mixed).
 * Uses the forward workspace; runs the intra-chunk kernel to get the gates. */
gdn_status gdn_cp_modes(const gdn_desc* desc, const void* k, const void* v,
                        const float* g, const float* beta, int32_t* modes_out,
                        void* workspace, size_t workspace_bytes, void* stream);

/* The per-boundary CP decision itself (see gdn_cp_modes): fwd_windows [S, H] int32 (device),
 * S = gdn_plan_info.total_segments, row gs for the boundary at the start of global sub-sequence
 * gs (a sequence's sub-sequences are consecutive): the warmup window in chunks before it, 0 =
 * exact correction, -1 = no boundary (a sequence's first sub-sequence). rev_windows, if not
 * NULL, the same for the backward's adjoint pass (windows after each boundary). Uses the
 * forward workspace; runs the intra-chunk kernel to get the gates. */
gdn_status gdn_cp_windows(const gdn_desc* desc, const void* k, const void* v,
                          const float* g, const float* beta, int32_t* fwd_windows,
                          int32_t* rev_windows, void* workspace, size_t workspace_bytes,
                          void* stream);

/* Per-kernel timing, for measurement tools (off by default). While enabled, each kernel
 * launch of the calls above is bracketed by two HIP events recorded on the call's stream
 * (this adds a few microseconds per launch). gdn_profile_read waits for the recorded
 * events, writes up to max_entries per-kernel totals (kernel name, launches, total
 * milliseconds) and clears them; it returns the number of entries written, or -1 on a
 * HIP error. The state is process-wide and guarded by a mutex. */
typedef struct gdn_kernel_time {
    char name[32];
    int64_t launches;
    double total_ms;
} gdn_kernel_time;

gdn_status gdn_profile_enable(int enable);
int gdn_profile_read(gdn_kernel_time* out, int max_entries);

#ifdef __cplusplus
}
#endif

#endif /* GDN_H_ */
