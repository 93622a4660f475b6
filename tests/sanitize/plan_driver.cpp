// Host-side sweep of libgdn's C ABI under AddressSanitizer and UndefinedBehaviorSanitizer: the
// planner over many shapes, every documented argument error, and the forward's launch sequence
// with the kernel launchers stubbed out (tests/sanitize/stubs.cpp). No device memory is touched:
// the pointers handed over are never dereferenced on the host. Prints "ok ..." on success;
// any sanitizer report aborts the process.
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <vector>

#include "gdn.h"

extern int g_launches;

static int failures = 0;
#define EXPECT(cond)                                                    \
    do {                                                                \
        if (!(cond)) {                                                  \
            fprintf(stderr, "FAILED %s:%d: %s\n", __FILE__, __LINE__, #cond); \
            ++failures;                                                 \
        }                                                               \
    } while (0)

static gdn_desc base(int64_t B, int64_t T, int64_t H, int64_t K, int64_t V, int dtype) {
    gdn_desc d;
    memset(&d, 0, sizeof(d));
    d.B = B;
    d.T = T;
    d.H = H;
    d.K = K;
    d.V = V;
    d.dtype = dtype;
    d.scale = 1.f;
    d.num_cus = 256;  // no device query
    return d;
}

// fake, 256-byte aligned device addresses: only compared and offset on the host
static void* fake(uintptr_t i) { return reinterpret_cast<void*>((uintptr_t)0x7f0000000000ull + i * 0x100000000ull); }

int main() {
    int plans = 0;
    const int64_t Ts[] = {0, 1, 63, 64, 65, 1000, 4096, 32768, 262144};
    const int64_t Hs[] = {1, 2, 16, 40, 41, 56, 57, 256};
    const int64_t Bs[] = {1, 2, 8};
    const int KVs[] = {64, 128};
    for (int64_t B : Bs)
        for (int64_t T : Ts)
            for (int64_t H : Hs)
                for (int K : KVs)
                    for (int V : KVs)
                        for (int dt = 0; dt < 2; ++dt)
                            for (int cp = 0; cp <= 5; ++cp) {
                                gdn_desc d = base(B, T, H, K, V, dt);
                                d.cp_mode = cp;
                                d.warmup_chunks = (int)(T % 17);
                                gdn_plan_info p;
                                const gdn_status s = gdn_plan(&d, &p);
                                EXPECT(s == GDN_OK);
                                if (s != GDN_OK) continue;
                                ++plans;
                                EXPECT(p.num_seqs == B);
                                EXPECT(p.seg_chunks >= 1);
                                EXPECT(p.total_chunks == B * ((T + 63) / 64));
                                EXPECT(p.fwd_workspace_bytes >= 256 && p.fwd_workspace_bytes % 256 == 0);
                                EXPECT(p.bwd_workspace_bytes >= p.fwd_workspace_bytes);
                                if (p.cp_on) EXPECT(p.seg_chunks < (T + 63) / 64);
                                size_t f = 0, b = 0;
                                EXPECT(gdn_chunk_fwd_workspace_size(&d, &f) == GDN_OK && f == p.fwd_workspace_bytes);
                                const gdn_status sb = gdn_chunk_bwd_workspace_size(&d, &b);
                                EXPECT(sb == GDN_OK || (dt == 1 && (K != 64 || V != 64)));
                            }
    // packed sequences, including empty ones, under every CP mode
    srand(7);
    for (int trial = 0; trial < 200; ++trial) {
        const int N = 1 + rand() % 40;
        std::vector<int32_t> cu(N + 1, 0);
        for (int n = 0; n < N; ++n) cu[n + 1] = cu[n] + (rand() % 5 == 0 ? 0 : rand() % 20000);
        gdn_desc d = base(1, cu[N], 1 + rand() % 64, 128, 128, rand() % 2);
        d.num_seqs = N;
        d.cu_seqlens = reinterpret_cast<const int32_t*>(fake(1));
        d.cu_seqlens_host = cu.data();
        d.cp_mode = trial % 6;
        d.seg_chunks = trial % 3 == 0 ? 16 + trial % 40 : 0;
        d.flags = (trial % 8 == 0 ? GDN_FLAG_QK_L2NORM : 0) | (trial % 5 == 0 ? GDN_FLAG_FWD_FUSED : 0);
        gdn_plan_info p;
        EXPECT(gdn_plan(&d, &p) == GDN_OK);
        ++plans;
        int64_t chunks = 0;
        for (int n = 0; n < N; ++n) chunks += (cu[n + 1] - cu[n] + 63) / 64;
        EXPECT(p.total_chunks == chunks);
        EXPECT(p.total_segments >= N);
        // the forward's launch sequence with stubbed kernels
        const int before = g_launches;
        EXPECT(gdn_chunk_fwd(&d, fake(2), fake(3), fake(4), (const float*)fake(5), (const float*)fake(6), nullptr,
                             fake(7), (float*)fake(8), fake(9), p.fwd_workspace_bytes, nullptr) == GDN_OK);
        EXPECT(g_launches > before || cu[N] == 0);
        EXPECT((p.cp_states_bytes > 0) == (p.cp_on != 0));
        if (p.cp_on) {
            // the same forward leaving its CP results in a caller buffer: the same launches
            const int nf = g_launches - before;
            gdn_desc c = d;
            c.cp_states = fake(14);
            const int l1 = g_launches;
            EXPECT(gdn_chunk_fwd(&c, fake(2), fake(3), fake(4), (const float*)fake(5), (const float*)fake(6), nullptr,
                                 fake(7), (float*)fake(8), fake(9), p.fwd_workspace_bytes, nullptr) == GDN_OK);
            EXPECT(g_launches - l1 == nf);
            c.cp_states = nullptr;
            c.flags |= GDN_FLAG_REUSE_CP;  // a backward told to reuse it needs it
            EXPECT(gdn_plan(&c, &p) == GDN_ERR_INVALID_ARG);
            EXPECT(gdn_plan(&d, &p) == GDN_OK);
        }
        EXPECT(gdn_intra_chunk(&d, fake(3), fake(4), (const float*)fake(5), (const float*)fake(6), (float*)fake(10),
                               fake(11), fake(12), fake(9), p.fwd_workspace_bytes, nullptr) == GDN_OK);
        EXPECT(gdn_cp_modes(&d, fake(3), fake(4), (const float*)fake(5), (const float*)fake(6), (int32_t*)fake(13),
                            fake(9), p.fwd_workspace_bytes, nullptr) == GDN_OK);
        // a workspace one byte short, or misaligned, is refused before any launch
        const int l0 = g_launches;
        EXPECT(gdn_chunk_fwd(&d, fake(2), fake(3), fake(4), (const float*)fake(5), (const float*)fake(6), nullptr,
                             fake(7), nullptr, fake(9), p.fwd_workspace_bytes - 1, nullptr) == GDN_ERR_WORKSPACE);
        EXPECT(gdn_chunk_fwd(&d, fake(2), fake(3), fake(4), (const float*)fake(5), (const float*)fake(6), nullptr,
                             fake(7), nullptr, (char*)fake(9) + 16, p.fwd_workspace_bytes, nullptr) == GDN_ERR_WORKSPACE);
        EXPECT(g_launches == l0);
    }
    // argument errors, each refused before any launch
    {
        const int l0 = g_launches;
        gdn_plan_info p;
        size_t bytes = 0;
        EXPECT(gdn_plan(nullptr, &p) == GDN_ERR_INVALID_ARG);
        gdn_desc d = base(1, 100, 2, 128, 128, 0);
        EXPECT(gdn_plan(&d, nullptr) == GDN_ERR_INVALID_ARG);
        EXPECT(gdn_chunk_fwd_workspace_size(&d, nullptr) == GDN_ERR_INVALID_ARG);
        gdn_desc e = d;
        e.reserved[4] = 1;
        EXPECT(gdn_plan(&e, &p) == GDN_ERR_INVALID_ARG);
        e = d; e.flags = 128;
        EXPECT(gdn_plan(&e, &p) == GDN_ERR_INVALID_ARG);
        e = d; e.cp_states = reinterpret_cast<void*>(0x10010);  // misaligned
        EXPECT(gdn_plan(&e, &p) == GDN_ERR_INVALID_ARG);
        e = d; e.chunk = 32;
        EXPECT(gdn_plan(&e, &p) == GDN_ERR_UNSUPPORTED);
        e = d; e.K = 96;
        EXPECT(gdn_plan(&e, &p) == GDN_ERR_UNSUPPORTED);
        e = d; e.dtype = 7;
        EXPECT(gdn_plan(&e, &p) == GDN_ERR_INVALID_ARG);
        e = d; e.cp_mode = 6;
        EXPECT(gdn_plan(&e, &p) == GDN_ERR_INVALID_ARG);
        e = d; e.warmup_chunks = 17;
        EXPECT(gdn_plan(&e, &p) == GDN_ERR_INVALID_ARG);
        e = d; e.warmup_chunks = 8; e.warmup_max_chunks = 7;
        EXPECT(gdn_plan(&e, &p) == GDN_ERR_INVALID_ARG);
        e = d; e.warmup_max_chunks = 8 + 64;
        EXPECT(gdn_plan(&e, &p) == GDN_ERR_INVALID_ARG);
        e = d; e.warmup_eps = 1.f;
        EXPECT(gdn_plan(&e, &p) == GDN_ERR_INVALID_ARG);
        e = d; e.B = 0;
        EXPECT(gdn_plan(&e, &p) == GDN_ERR_INVALID_ARG);
        e = d; e.T = -1;
        EXPECT(gdn_plan(&e, &p) == GDN_ERR_INVALID_ARG);
        e = d; e.H = 70000;
        EXPECT(gdn_plan(&e, &p) == GDN_ERR_UNSUPPORTED);
        // cu_seqlens: host copy missing, wrong end, decreasing, B > 1
        int32_t cu[4] = {0, 40, 30, 100};
        e = d; e.num_seqs = 3; e.cu_seqlens = reinterpret_cast<const int32_t*>(fake(1));
        EXPECT(gdn_plan(&e, &p) == GDN_ERR_INVALID_ARG);
        e.cu_seqlens_host = cu;
        EXPECT(gdn_plan(&e, &p) == GDN_ERR_INVALID_ARG);
        cu[2] = 60; cu[3] = 99;
        EXPECT(gdn_plan(&e, &p) == GDN_ERR_INVALID_ARG);
        cu[3] = 100;
        EXPECT(gdn_plan(&e, &p) == GDN_OK);
        e.B = 2;
        EXPECT(gdn_plan(&e, &p) == GDN_ERR_INVALID_ARG);
        // fp32 backward beyond K = V = 64
        e = base(1, 100, 2, 128, 128, GDN_DTYPE_FP32);
        EXPECT(gdn_chunk_bwd_workspace_size(&e, &bytes) == GDN_ERR_UNSUPPORTED);
        // null tensors
        EXPECT(gdn_plan(&d, &p) == GDN_OK);
        EXPECT(gdn_chunk_fwd(&d, nullptr, fake(3), fake(4), (const float*)fake(5), (const float*)fake(6), nullptr,
                             fake(7), nullptr, fake(9), p.fwd_workspace_bytes, nullptr) == GDN_ERR_INVALID_ARG);
        EXPECT(gdn_chunk_fwd(&d, fake(2), fake(3), fake(4), (const float*)fake(5), (const float*)fake(6), nullptr,
                             fake(7), nullptr, nullptr, p.fwd_workspace_bytes, nullptr) == GDN_ERR_WORKSPACE);
        EXPECT(gdn_chunk_bwd(&d, fake(2), fake(3), fake(4), (const float*)fake(5), (const float*)fake(6), nullptr,
                             nullptr, nullptr, fake(7), fake(8), fake(9), (float*)fake(10), (float*)fake(11), nullptr,
                             fake(12), p.bwd_workspace_bytes, nullptr) == GDN_ERR_INVALID_ARG);
        EXPECT(gdn_chunk_bwd(&d, fake(2), fake(3), fake(4), (const float*)fake(5), (const float*)fake(6), nullptr,
                             fake(13), nullptr, fake(7), fake(8), fake(9), (float*)fake(10), (float*)fake(11), nullptr,
                             fake(12), p.bwd_workspace_bytes - 256, nullptr) == GDN_ERR_WORKSPACE);
        gdn_desc r = base(4, 1, 16, 128, 128, 0);
        EXPECT(gdn_recurrent_fwd(&r, fake(1), fake(2), fake(3), (const float*)fake(4), (const float*)fake(5), nullptr,
                                 nullptr, fake(6), nullptr) == GDN_ERR_INVALID_ARG);
        r.flags = GDN_FLAG_KEEP_FORWARD;
        EXPECT(gdn_recurrent_fwd(&r, fake(1), fake(2), fake(3), (const float*)fake(4), (const float*)fake(5), nullptr,
                                 (float*)fake(7), fake(6), nullptr) == GDN_ERR_INVALID_ARG);
        EXPECT(g_launches == l0);
        r.flags = GDN_FLAG_QK_L2NORM;
        EXPECT(gdn_recurrent_fwd(&r, fake(1), fake(2), fake(3), (const float*)fake(4), (const float*)fake(5), nullptr,
                                 (float*)fake(7), fake(6), nullptr) == GDN_OK);
        EXPECT(g_launches == l0 + 1);
        for (int s = 0; s < 8; ++s) EXPECT(gdn_status_string((gdn_status)s) != nullptr);
        // the no-allocation forward refuses, before any launch or HIP call, a problem beyond its
        // fixed array, kept intermediates and missing tensors
        const int l1 = g_launches;
        gdn_desc big = base(1, 262144, 16, 128, 128, 0);
        EXPECT(gdn_chunk_fwd_noalloc(&big, fake(2), fake(3), fake(4), (const float*)fake(5), (const float*)fake(6),
                                     nullptr, fake(7), nullptr, nullptr) == GDN_ERR_WORKSPACE);
        gdn_desc keep = base(1, 1000, 2, 128, 128, 0);
        keep.flags = GDN_FLAG_KEEP_FORWARD;
        EXPECT(gdn_chunk_fwd_noalloc(&keep, fake(2), fake(3), fake(4), (const float*)fake(5), (const float*)fake(6),
                                     nullptr, fake(7), nullptr, nullptr) == GDN_ERR_INVALID_ARG);
        keep.flags = GDN_FLAG_REUSE_FORWARD;
        EXPECT(gdn_chunk_fwd_noalloc(&keep, fake(2), fake(3), fake(4), (const float*)fake(5), (const float*)fake(6),
                                     nullptr, fake(7), nullptr, nullptr) == GDN_ERR_INVALID_ARG);
        keep.flags = 0;
        EXPECT(gdn_chunk_fwd_noalloc(&keep, fake(2), nullptr, fake(4), (const float*)fake(5), (const float*)fake(6),
                                     nullptr, fake(7), nullptr, nullptr) == GDN_ERR_INVALID_ARG);
        EXPECT(g_launches == l1);
    }
    if (failures) {
        fprintf(stderr, "%d expectation(s) failed\n", failures);
        return 1;
    }
    printf("ok plans=%d launches=%d\n", plans, g_launches);
    return 0;
}
