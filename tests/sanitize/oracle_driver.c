/* The CPU oracle (oracle/gdn_oracle.c) under AddressSanitizer and UndefinedBehaviorSanitizer:
 * forward and reverse mode on small packed batches (empty, one-token and ragged sequences, with
 * and without states), checking only that every output is finite and that a sequence's final
 * state equals its initial state when it has no tokens. Test infrastructure only. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

int gdn_oracle_fwd(int64_t nseq, const int64_t* cu, int64_t H, int64_t K, int64_t V, const double* q,
                   const double* k, const double* v, const double* g, const double* beta, double scale,
                   const double* s0, double* o, double* sT, int nthreads);
int gdn_oracle_bwd(int64_t nseq, const int64_t* cu, int64_t H, int64_t K, int64_t V, const double* q,
                   const double* k, const double* v, const double* g, const double* beta, double scale,
                   const double* s0, const double* d_o, const double* dsT, double* dq, double* dk, double* dv,
                   double* dg, double* dbeta, double* ds0, int nthreads);

static double urand(void) { return (double)rand() / RAND_MAX - 0.5; }

static double* fill(size_t n, double lo, double hi) {
    double* x = malloc((n ? n : 1) * sizeof(double));
    for (size_t i = 0; i < n; ++i) x[i] = lo + (hi - lo) * (urand() + 0.5);
    return x;
}

static int finite_all(const double* x, size_t n) {
    for (size_t i = 0; i < n; ++i)
        if (!isfinite(x[i])) return 0;
    return 1;
}

int main(void) {
    srand(3);
    const int64_t lens[][6] = {{0, 1, 63, 64, 65, 130}, {200, 0, 0, 7, 64, 1}};
    int bad = 0;
    for (int c = 0; c < 2; ++c) {
        const int64_t N = 6, H = 2, K = 8 + 4 * c, V = 12 - 4 * c;
        int64_t cu[7] = {0};
        for (int n = 0; n < N; ++n) cu[n + 1] = cu[n] + lens[c][n];
        const int64_t T = cu[N];
        double *q = fill(T * H * K, -1, 1), *k = fill(T * H * K, -0.3, 0.3), *v = fill(T * H * V, -1, 1);
        double *g = fill(T * H, -0.2, 0.0), *b = fill(T * H, 0.0, 1.0), *dO = fill(T * H * V, -1, 1);
        double *s0 = c ? fill(N * H * V * K, -0.1, 0.1) : NULL, *dsT = fill(N * H * V * K, -0.1, 0.1);
        double *o = fill(T * H * V, 0, 0), *sT = fill(N * H * V * K, 0, 0);
        double *dq = fill(T * H * K, 0, 0), *dk = fill(T * H * K, 0, 0), *dv = fill(T * H * V, 0, 0);
        double *dg = fill(T * H, 0, 0), *db = fill(T * H, 0, 0), *ds0 = fill(N * H * V * K, 0, 0);
        if (gdn_oracle_fwd(N, cu, H, K, V, q, k, v, g, b, 0.7, s0, o, sT, 2) != 0) bad |= 1;
        if (gdn_oracle_bwd(N, cu, H, K, V, q, k, v, g, b, 0.7, s0, dO, dsT, dq, dk, dv, dg, db, ds0, 2) != 0) bad |= 2;
        if (!finite_all(o, T * H * V) || !finite_all(sT, N * H * V * K) || !finite_all(dq, T * H * K) ||
            !finite_all(dk, T * H * K) || !finite_all(dv, T * H * V) || !finite_all(dg, T * H) ||
            !finite_all(db, T * H) || !finite_all(ds0, N * H * V * K))
            bad |= 4;
        for (int n = 0; n < N; ++n) {
            if (lens[c][n]) continue;
            for (int64_t i = 0; i < H * V * K; ++i) {
                const double want = s0 ? s0[n * H * V * K + i] : 0.0;
                if (sT[n * H * V * K + i] != want || ds0[n * H * V * K + i] != dsT[n * H * V * K + i]) bad |= 8;
            }
        }
        free(q); free(k); free(v); free(g); free(b); free(dO); free(s0); free(dsT); free(o); free(sT);
        free(dq); free(dk); free(dv); free(dg); free(db); free(ds0);
    }
    if (bad) {
        fprintf(stderr, "oracle driver: failure mask %d\n", bad);
        return 1;
    }
    printf("ok\n");
    return 0;
}
