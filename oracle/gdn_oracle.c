/*
 * gdn_oracle.c -- CPU oracle for Gated DeltaNet (GDN) chunked prefill.
 *
 * TEST INFRASTRUCTURE ONLY. Nothing on the GPU product path may include,
 * link or call this file; only the tests, the smoke check and the CPU
 * baseline of the benchmark use it. It shares no code with the HIP library.
 *
 * What it computes: the gated delta rule written token by token, in fp64,
 * exactly as it is defined, with no chunking, blocking or reordering.
 * The rule is named by the FlashQLA pages ("Gated Delta Network (GDN)",
 * ollai.cn FlashQLA article, section "main features"), which give no formula;
 * the recurrence used is the standard gated delta rule
 *
 *     S_t = exp(g_t) * S_{t-1} * (I - beta_t k_t k_t^T) + beta_t v_t k_t^T
 *     o_t = scale * S_t q_t
 *
 * with S a V x K matrix (rows over the value dimension, columns over the key
 * dimension). Per row i of S this is, with s = row i and a = exp(g_t):
 *     s <- a*s;  u = s.k_t;  s <- s + beta_t (v_t[i] - u) k_t;  o_t[i] = scale s.q_t
 * which is the same product regrouped (S (I - b k k^T) = S - b (S k) k^T).
 *
 * The call returns O and the final state and accepts an optional initial
 * state and packed variable-length sequences (cu_seqlens), as the pages'
 * "how to use" section describes (ollai.cn FlashQLA article).
 *
 * The backward is the hand-derived reverse mode of that token loop:
 * per token t, walking backwards with G = dL/dS_t (starting from dL/dS_T):
 *   1. G += scale do_t q_t^T;  dq_t = scale S_t^T do_t
 *   2. S' = a S_{t-1};  u = S' k_t;  d = beta_t (v_t - u);  dd = G k_t
 *   3. dk_t = G^T d - beta_t S'^T dd;  dv_t = beta_t dd;  dbeta_t = dd.(v_t - u)
 *   4. dS' = G - beta_t dd k_t^T;  dg_t = <dS', S'>_F;  G <- a dS'
 * and d(initial state) = G after the first token. S_{t-1} is recomputed from
 * checkpoints taken every ORACLE_CKPT tokens in a forward sweep.
 *
 * Layouts (all row-major, fp64): q, k: [Ttot][H][K]; v, o, do: [Ttot][H][V];
 * g, beta, dg, dbeta: [Ttot][H]; states: [nseq][H][V][K]; cu: [nseq+1]
 * token offsets (cu[0] = 0, cu[nseq] = Ttot, non-decreasing).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORACLE_CKPT 64
#define ORACLE_ROWBLOCK 32

static int check_cu(int64_t nseq, const int64_t* cu) {
    if (nseq < 0 || !cu || cu[0] != 0) return -1;
    for (int64_t n = 0; n < nseq; ++n)
        if (cu[n + 1] < cu[n]) return -1;
    return 0;
}

/* One forward token step on rows [r0, r1) of S; writes o rows if o != NULL. */
static void step_rows(double* S, int64_t K, int64_t r0, int64_t r1,
                      const double* kt, const double* vt, const double* qt,
                      double a, double b, double scale, double* ot) {
    for (int64_t i = r0; i < r1; ++i) {
        double* s = S + i * K;
        double u = 0.0;
        for (int64_t j = 0; j < K; ++j) {
            s[j] *= a;
            u += s[j] * kt[j];
        }
        const double c = b * (vt[i] - u);
        double oi = 0.0;
        for (int64_t j = 0; j < K; ++j) {
            s[j] += c * kt[j];
            if (ot) oi += s[j] * qt[j];
        }
        if (ot) ot[i] = scale * oi;
    }
}

int gdn_oracle_fwd(int64_t nseq, const int64_t* cu, int64_t H, int64_t K, int64_t V,
                   const double* q, const double* k, const double* v,
                   const double* g, const double* beta, double scale,
                   const double* s0, double* o, double* sT, int nthreads) {
    if (check_cu(nseq, cu) || H <= 0 || K <= 0 || V <= 0) return -1;
    const int64_t nrb = (V + ORACLE_ROWBLOCK - 1) / ORACLE_ROWBLOCK;
    const int64_t ntask = nseq * H * nrb;
    int bad = 0;
#ifdef _OPENMP
#pragma omp parallel for schedule(dynamic, 1) num_threads(nthreads > 0 ? nthreads : 1)
#endif
    for (int64_t task = 0; task < ntask; ++task) {
        const int64_t n = task / (H * nrb);
        const int64_t h = (task / nrb) % H;
        const int64_t rb = task % nrb;
        const int64_t r0 = rb * ORACLE_ROWBLOCK;
        const int64_t r1 = r0 + ORACLE_ROWBLOCK < V ? r0 + ORACLE_ROWBLOCK : V;
        double* S = (double*)malloc((size_t)(V * K) * sizeof(double));
        if (!S) { bad = 1; continue; }
        const int64_t soff = (n * H + h) * V * K;
        if (s0) memcpy(S + r0 * K, s0 + soff + r0 * K, (size_t)((r1 - r0) * K) * sizeof(double));
        else memset(S + r0 * K, 0, (size_t)((r1 - r0) * K) * sizeof(double));
        for (int64_t t = cu[n]; t < cu[n + 1]; ++t) {
            const int64_t th = t * H + h;
            step_rows(S, K, r0, r1, k + th * K, v + th * V, q + th * K,
                      exp(g[th]), beta[th], scale, o ? o + th * V : NULL);
        }
        if (sT) memcpy(sT + soff + r0 * K, S + r0 * K, (size_t)((r1 - r0) * K) * sizeof(double));
        free(S);
    }
    return bad ? -2 : 0;
}

int gdn_oracle_bwd(int64_t nseq, const int64_t* cu, int64_t H, int64_t K, int64_t V,
                   const double* q, const double* k, const double* v,
                   const double* g, const double* beta, double scale,
                   const double* s0, const double* d_o, const double* dsT,
                   double* dq, double* dk, double* dv, double* dg, double* dbeta,
                   double* ds0, int nthreads) {
    if (check_cu(nseq, cu) || H <= 0 || K <= 0 || V <= 0) return -1;
    const int64_t VK = V * K;
    const int64_t ntask = nseq * H;
    int bad = 0;
#ifdef _OPENMP
#pragma omp parallel for schedule(dynamic, 1) num_threads(nthreads > 0 ? nthreads : 1)
#endif
    for (int64_t task = 0; task < ntask; ++task) {
        const int64_t n = task / H, h = task % H;
        const int64_t bos = cu[n], eos = cu[n + 1], len = eos - bos;
        const int64_t nck = (len + ORACLE_CKPT - 1) / ORACLE_CKPT;
        const int64_t soff = (n * H + h) * VK;
        double* ck = (double*)malloc((size_t)((nck > 0 ? nck : 1) * VK) * sizeof(double));
        double* buf = (double*)malloc((size_t)((ORACLE_CKPT + 1) * VK) * sizeof(double));
        double* G = (double*)malloc((size_t)VK * sizeof(double));
        double* del = (double*)malloc((size_t)V * sizeof(double));
        double* dd = (double*)malloc((size_t)V * sizeof(double));
        double* um = (double*)malloc((size_t)V * sizeof(double));
        if (!ck || !buf || !G || !del || !dd || !um) {
            bad = 1;
            free(ck); free(buf); free(G); free(del); free(dd); free(um);
            continue;
        }
        /* forward sweep: checkpoint the state entering every ORACLE_CKPT tokens */
        double* S = buf;
        if (s0) memcpy(S, s0 + soff, (size_t)VK * sizeof(double));
        else memset(S, 0, (size_t)VK * sizeof(double));
        for (int64_t t = bos; t < eos; ++t) {
            if ((t - bos) % ORACLE_CKPT == 0)
                memcpy(ck + ((t - bos) / ORACLE_CKPT) * VK, S, (size_t)VK * sizeof(double));
            const int64_t th = t * H + h;
            step_rows(S, K, 0, V, k + th * K, v + th * V, NULL, exp(g[th]), beta[th], scale, NULL);
        }
        if (dsT) memcpy(G, dsT + soff, (size_t)VK * sizeof(double));
        else memset(G, 0, (size_t)VK * sizeof(double));
        for (int64_t c = nck - 1; c >= 0; --c) {
            const int64_t t0 = bos + c * ORACLE_CKPT;
            const int64_t t1 = t0 + ORACLE_CKPT < eos ? t0 + ORACLE_CKPT : eos;
            /* buf[0] = S_{t0-1}; buf[m] = S_{t0+m-1} */
            memcpy(buf, ck + c * VK, (size_t)VK * sizeof(double));
            for (int64_t t = t0; t < t1; ++t) {
                double* dst = buf + (t - t0 + 1) * VK;
                memcpy(dst, buf + (t - t0) * VK, (size_t)VK * sizeof(double));
                const int64_t th = t * H + h;
                step_rows(dst, K, 0, V, k + th * K, v + th * V, NULL, exp(g[th]), beta[th], scale, NULL);
            }
            for (int64_t t = t1 - 1; t >= t0; --t) {
                const int64_t th = t * H + h;
                const double* St = buf + (t - t0 + 1) * VK;
                const double* Sp = buf + (t - t0) * VK; /* S_{t-1}; S' = a * Sp */
                const double* qt = q + th * K;
                const double* kt = k + th * K;
                const double* vt = v + th * V;
                const double* dot = d_o + th * V;
                const double a = exp(g[th]), b = beta[th];
                double* dqt = dq + th * K;
                double* dkt = dk + th * K;
                double* dvt = dv + th * V;
                /* 1. output adjoint */
                for (int64_t j = 0; j < K; ++j) dqt[j] = 0.0;
                for (int64_t i = 0; i < V; ++i) {
                    const double di = scale * dot[i];
                    double* Gi = G + i * K;
                    const double* Si = St + i * K;
                    for (int64_t j = 0; j < K; ++j) {
                        Gi[j] += di * qt[j];
                        dqt[j] += di * Si[j];
                    }
                }
                /* 2. u = S'k, delta, d(delta) = G k */
                for (int64_t i = 0; i < V; ++i) {
                    const double* Gi = G + i * K;
                    const double* Pi = Sp + i * K;
                    double ui = 0.0, gi = 0.0;
                    for (int64_t j = 0; j < K; ++j) {
                        ui += a * Pi[j] * kt[j];
                        gi += Gi[j] * kt[j];
                    }
                    um[i] = ui;
                    del[i] = b * (vt[i] - ui);
                    dd[i] = gi;
                }
                /* 3. dk, dv, dbeta */
                double dbt = 0.0;
                for (int64_t j = 0; j < K; ++j) dkt[j] = 0.0;
                for (int64_t i = 0; i < V; ++i) {
                    const double* Gi = G + i * K;
                    const double* Pi = Sp + i * K;
                    for (int64_t j = 0; j < K; ++j)
                        dkt[j] += Gi[j] * del[i] - b * a * Pi[j] * dd[i];
                    dvt[i] = b * dd[i];
                    dbt += dd[i] * (vt[i] - um[i]);
                }
                dbeta[th] = dbt;
                /* 4. dS' = G - b dd k^T, dg = <dS', S'>, G <- a dS' */
                double dgt = 0.0;
                for (int64_t i = 0; i < V; ++i) {
                    double* Gi = G + i * K;
                    const double* Pi = Sp + i * K;
                    for (int64_t j = 0; j < K; ++j) {
                        const double dsp = Gi[j] - b * dd[i] * kt[j];
                        dgt += dsp * a * Pi[j];
                        Gi[j] = a * dsp;
                    }
                }
                dg[th] = dgt;
            }
        }
        if (ds0) memcpy(ds0 + soff, G, (size_t)VK * sizeof(double));
        free(ck); free(buf); free(G); free(del); free(dd); free(um);
    }
    return bad ? -2 : 0;
}

int gdn_oracle_num_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
