/* Runs every function of the fp64 oracle (oracle/gdr_oracle.c) on small seeded
 * inputs under the address and undefined-behaviour sanitizers: all gate kinds,
 * with and without initial state, several thread counts, lengths around the
 * checkpoint spacing, and the bad-argument paths.  It checks that the outputs
 * are finite, that T decode steps reproduce the forward, and that the thread
 * count does not change any result.  Exits non-zero on the first failure. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "../../oracle/gdr_oracle.h"

static uint64_t g_state = 0x9E3779B97F4A7C15ull;
static double urand(void) { /* xorshift64*, uniform in [0, 1) */
    g_state ^= g_state >> 12;
    g_state ^= g_state << 25;
    g_state ^= g_state >> 27;
    return (double)((g_state * 0x2545F4914F6CDD1Dull) >> 11) / 9007199254740992.0;
}
static double* arr(size_t n, double lo, double hi) {
    double* a = (double*)malloc((n ? n : 1) * sizeof(double));
    for (size_t i = 0; i < n; ++i) a[i] = lo + (hi - lo) * urand();
    return a;
}
static int finite_all(const double* a, size_t n) {
    for (size_t i = 0; i < n; ++i)
        if (!isfinite(a[i])) return 0;
    return 1;
}
static int fails = 0;
#define CHECK(c, msg)                                            \
    do {                                                         \
        if (!(c)) {                                              \
            fprintf(stderr, "FAIL line %d: %s\n", __LINE__, msg); \
            ++fails;                                             \
        }                                                        \
    } while (0)

static void one(int64_t B, int64_t T, int64_t H, int64_t d, int gate, int s0) {
    const size_t n = (size_t)(B * T * H * d), nt = (size_t)(B * T * H), ns = (size_t)(B * H * d * d);
    const size_t na = gate == ORACLE_GATE_CHANNEL ? n : nt;
    double *q = arr(n, -0.3, 0.3), *k = arr(n, -0.3, 0.3), *v = arr(n, -1, 1), *beta = arr(nt, 0, 1),
           *alpha = arr(na, 0.5, 1), *S0 = s0 ? arr(ns, -0.05, 0.05) : NULL, *dO = arr(n, -1, 1),
           *dST = arr(ns, -0.1, 0.1), *dE = arr(n, -1, 1);
    double *o = arr(n, 0, 0), *ST = arr(ns, 0, 0), *E = arr(n, 0, 0), *o4 = arr(n, 0, 0), *ST4 = arr(ns, 0, 0);
    double *dq = arr(n, 0, 0), *dk = arr(n, 0, 0), *dv = arr(n, 0, 0), *db = arr(nt, 0, 0), *da = arr(na, 0, 0),
           *dS0 = arr(ns, 0, 0);
    const double* al = gate == ORACLE_GATE_NONE ? NULL : alpha;
    double* dal = gate == ORACLE_GATE_NONE ? NULL : da;
    CHECK(oracle_forward(B, T, H, d, d, gate, 0.7, q, k, v, beta, al, S0, o, ST, 1) == 0, "forward");
    CHECK(oracle_forward(B, T, H, d, d, gate, 0.7, q, k, v, beta, al, S0, o4, ST4, 4) == 0, "forward x4");
    CHECK(memcmp(o, o4, n * sizeof(double)) == 0 && memcmp(ST, ST4, ns * sizeof(double)) == 0,
          "thread count changed the forward");
    CHECK(finite_all(o, n) && finite_all(ST, ns), "forward not finite");
    CHECK(oracle_forward_errors(B, T, H, d, d, gate, 0.7, q, k, v, beta, al, S0, o4, ST4, E, 3) == 0, "errors");
    CHECK(memcmp(o, o4, n * sizeof(double)) == 0, "forward_errors changed o");
    CHECK(oracle_backward(B, T, H, d, d, gate, 0.7, q, k, v, beta, al, S0, dO, dST, dq, dk, dv, db, dal, dS0, 2) == 0,
          "backward");
    CHECK(finite_all(dq, n) && finite_all(dk, n) && finite_all(dv, n) && finite_all(db, nt) && finite_all(dS0, ns),
          "backward not finite");
    CHECK(oracle_backward_errors(B, T, H, d, d, gate, 0.7, q, k, v, beta, al, S0, dO, NULL, dE, dq, dk, dv, db, dal,
                                 NULL, 5) == 0, "backward_errors");
    /* T decode steps reproduce the forward's outputs and final state */
    if (T > 0) {
        double* S = arr(ns, 0, 0);
        if (S0) memcpy(S, S0, ns * sizeof(double));
        const size_t row = (size_t)(H * d);
        double *qt = arr((size_t)B * row, 0, 0), *kt = arr((size_t)B * row, 0, 0), *vt = arr((size_t)B * row, 0, 0),
               *bt = arr((size_t)(B * H), 0, 0), *at = arr((size_t)B * row, 0, 0), *ot = arr((size_t)B * row, 0, 0);
        double maxdiff = 0;
        for (int64_t t = 0; t < T; ++t) {
            for (int64_t b = 0; b < B; ++b) {
                const size_t src = (size_t)((b * T + t) * H);
                memcpy(qt + b * row, q + src * d, row * sizeof(double));
                memcpy(kt + b * row, k + src * d, row * sizeof(double));
                memcpy(vt + b * row, v + src * d, row * sizeof(double));
                memcpy(bt + b * H, beta + src, (size_t)H * sizeof(double));
                if (gate == ORACLE_GATE_CHANNEL) memcpy(at + b * row, alpha + src * d, row * sizeof(double));
                if (gate == ORACLE_GATE_SCALAR) memcpy(at + b * H, alpha + src, (size_t)H * sizeof(double));
            }
            CHECK(oracle_decode(B, H, d, d, gate, 0.7, qt, kt, vt, bt, gate ? at : NULL, S, ot, 2) == 0, "decode");
            for (int64_t b = 0; b < B; ++b)
                for (size_t i = 0; i < row; ++i) {
                    const double x = fabs(ot[b * row + i] - o[(size_t)((b * T + t) * H) * d + i]);
                    if (x > maxdiff) maxdiff = x;
                }
        }
        for (size_t i = 0; i < ns; ++i)
            if (fabs(S[i] - ST[i]) > maxdiff) maxdiff = fabs(S[i] - ST[i]);
        CHECK(maxdiff < 1e-12, "decode steps differ from the forward");
        free(S); free(qt); free(kt); free(vt); free(bt); free(at); free(ot);
    }
    /* Gated DeltaNet-2 with equal gates reproduces the forward above */
    {
        double *g = arr(n, 0, 0), *og = arr(n, 0, 0), *STg = arr(ns, 0, 0);
        for (size_t i = 0; i < n; ++i) g[i] = beta[i / (size_t)d];
        CHECK(oracle_gdn2_forward(B, T, H, d, d, gate, 0.7, q, k, v, g, g, al, S0, og, STg, 3) == 0, "gdn2 forward");
        double md = 0;
        for (size_t i = 0; i < n; ++i) md = fmax(md, fabs(og[i] - o[i]));
        for (size_t i = 0; i < ns; ++i) md = fmax(md, fabs(STg[i] - ST[i]));
        CHECK(md < 1e-12, "gdn2 with equal gates differs from the forward");
        if (T > 0) {
            double* S = arr(ns, 0, 0);
            CHECK(oracle_gdn2_decode(B, H, d, d, gate, 0.7, q, k, v, g, g, al, S, og, 2) == 0, "gdn2 decode");
            free(S);
        }
        free(g); free(og); free(STg);
    }
    double* hin = arr(n, -1, 1), *hout = arr(n, 0, 0), *lam = arr((size_t)(H * d), -1, 1), *dlam = arr((size_t)(H * d), 0, 0);
    CHECK(oracle_clvr_forward(B, T, H, d, hin, v, lam, hout) == 0, "clvr forward");
    CHECK(oracle_clvr_forward(B, T, H, d, hin, v, NULL, hin) == 0, "clvr in place");
    CHECK(oracle_clvr_backward(B, T, H, d, dO, v, lam, dv, dlam) == 0, "clvr backward");
    free(hin); free(hout); free(lam); free(dlam);
    free(q); free(k); free(v); free(beta); free(alpha); free(S0); free(dO); free(dST); free(dE);
    free(o); free(ST); free(E); free(o4); free(ST4); free(dq); free(dk); free(dv); free(db); free(da); free(dS0);
}

int main(void) {
    const int64_t Ts[] = {0, 1, 2, 3, 15, 16, 17, 50};
    for (int g = 0; g < 3; ++g)
        for (size_t i = 0; i < sizeof Ts / sizeof Ts[0]; ++i)
            for (int s0 = 0; s0 < 2; ++s0) one(2, Ts[i], 3, 5, g, s0);
    one(1, 37, 2, 16, ORACLE_GATE_CHANNEL, 1);
    /* bad arguments are refused, never dereferenced */
    double x[4] = {0};
    CHECK(oracle_forward(-1, 4, 1, 1, 1, 0, 1.0, x, x, x, x, NULL, NULL, x, NULL, 1) == -1, "negative B");
    CHECK(oracle_forward(1, 1, 1, 1, 1, 9, 1.0, x, x, x, x, x, NULL, x, NULL, 1) == -1, "unknown gate");
    CHECK(oracle_forward(1, 1, 1, 1, 1, 0, 1.0, NULL, x, x, x, NULL, NULL, x, NULL, 1) == -1, "NULL q");
    printf("oracle driver: %d failures\n", fails);
    return fails ? 1 : 0;
}
