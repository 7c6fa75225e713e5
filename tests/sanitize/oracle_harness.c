/*
 * Drives every entry point of oracle/oracle.c through valid calls, calls
 * with invalid blocks (the per-block early returns) and calls with invalid
 * arguments (the early -1 returns), so that a build with address,
 * undefined-behaviour and leak sanitizers sees every allocation and free
 * path.  Exits 0 when every return code is the one expected; the sanitizers
 * abort or report on any memory error, undefined behaviour or leak.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

int oracle_chain(const void *, const void *, int, const int32_t *, const float *, int, int, int,
                 double, int32_t *, int32_t *, double *, double *, double *, int32_t *, int);
int oracle_chain_pointmass(const void *, int, const int32_t *, const float *, int, int, int,
                           double, int32_t *, int32_t *, double *, double *, double *, int32_t *,
                           int);
int oracle_chain_alpha(const void *, const void *, int, int, int, int, double, double *, int);
int oracle_outcome_topk(const void *, int, const int32_t *, int, int, int, double, int,
                        int32_t *, int32_t *, double *, double *, double *);
int oracle_tree_greedy(const void *, int, const int32_t *, const int32_t *, int, int, int,
                       int32_t *, int32_t *, int32_t *, int32_t *, int);
int oracle_tree_build(const void *, int, int, int, int, double, int, int, int, const int32_t *,
                      int32_t *, int32_t *, int32_t *, double *, int32_t *, double *);
int oracle_tree_score(const void *, int, int, int, int, double, int, const int32_t *,
                      const int32_t *, const int32_t *, const int32_t *, double *);
int oracle_tree_stochastic(const void *, const void *, int, const int32_t *, const int32_t *,
                           const float *, int, int, int, double, int32_t *, int32_t *, int32_t *,
                           double *, double *, double *);

static int fails = 0;
#define EXPECT(call, want)                                                              \
    do {                                                                                \
        int rc_ = (call);                                                               \
        if (rc_ != (want)) {                                                            \
            fprintf(stderr, "line %d: %s returned %d, want %d\n", __LINE__, #call, rc_, \
                    (want));                                                            \
            ++fails;                                                                    \
        }                                                                               \
    } while (0)

static float frand(unsigned *s)
{
    *s = *s * 1664525u + 1013904223u;
    return (float)((*s >> 8) & 0xffff) / 65536.0f * 4.0f - 2.0f;
}

int main(void)
{
    enum { B = 3, G = 4, V = 50, N = 9, M = 13, W = 3, BUD = 12 };
    unsigned seed = 7;
    float tgt[B * (G + 1) * V], drf[B * G * V], u[B * (G + 1)];
    float tt[B * N * V], td[B * N * V], ut[B * N], zb[B * M * V];
    int32_t tok[B * G], par[B * N], ntok[B * N];
    for (int i = 0; i < B * (G + 1) * V; ++i) tgt[i] = frand(&seed);
    for (int i = 0; i < B * G * V; ++i) drf[i] = frand(&seed);
    for (int i = 0; i < B * N * V; ++i) { tt[i] = frand(&seed); td[i] = frand(&seed); }
    for (int i = 0; i < B * M * V; ++i) zb[i] = frand(&seed);
    for (int i = 0; i < B * (G + 1); ++i) u[i] = (frand(&seed) + 2.0f) / 4.0f;
    for (int i = 0; i < B * N; ++i) ut[i] = (frand(&seed) + 2.0f) / 4.0f;
    for (int i = 0; i < B * G; ++i) tok[i] = (int32_t)(seed = seed * 69069u + 1u) % V;
    for (int b = 0; b < B; ++b)
        for (int j = 0; j < N; ++j) {
            par[b * N + j] = j == 0 ? -1 : (j - 1) / 2;
            ntok[b * N + j] = (j * 7 + b) % V;
        }
    /* block 1 invalid in several ways: a NaN, a token out of range */
    drf[1 * G * V + 2 * V + 3] = NAN;
    tok[2 * G + 1] = V;
    tt[1 * N * V + 4 * V] = INFINITY;
    par[2 * N + 5] = 7;
    zb[1 * M * V + 2 * V + 1] = NAN;

    int32_t acc[B], out[B * (G + 1)], fb[B], node[B], outt[B * N], amax[B * N];
    double dist[B * V], mar[B], rat[B * G], alpha[B * G], allp[B * (G + 1) * V];
    int32_t ck[B * 4], ca[B * 4], bpar[B * BUD], btok[B * BUD], brow[B * BUD], bn[B];
    double cp[B * 4], hit[B], bsc[B * BUD], gap[B], sc2[B * BUD], talpha[B * N];

    for (int nt = 1; nt <= 4; nt += 3) {
        EXPECT(oracle_chain(tgt, drf, 0, tok, u, B, G, V, 0.8, acc, out, dist, mar, rat, fb, nt), 0);
        EXPECT(oracle_chain(tgt, drf, 0, tok, u, B, G, V, 0.8, acc, out, NULL, NULL, NULL, NULL, nt),
               0);
        EXPECT(oracle_chain_pointmass(tgt, 0, tok, u, B, G, V, 0.8, acc, out, dist, mar, rat, fb, nt),
               0);
        EXPECT(oracle_tree_greedy(tt, 0, par, ntok, B, N, V, acc, node, outt, amax, nt), 0);
    }
    EXPECT(oracle_chain_alpha(tgt, drf, 0, B, G, V, 1.0, alpha, 2), 0);
    EXPECT(oracle_outcome_topk(tgt, 0, tok, B, G, V, 0.9, 4, ck, ca, cp, hit, allp), 0);
    EXPECT(oracle_tree_build(zb, 0, B, M, V, 1.0, W, 3, BUD, NULL, bpar, btok, brow, bsc, bn, gap),
           0);
    EXPECT(oracle_tree_score(zb, 0, B, M, V, 1.0, BUD, bpar, btok, brow, bn, sc2), 0);
    EXPECT(oracle_tree_stochastic(tt, td, 0, par, ntok, ut, B, N, V, 1.0, acc, node, outt, dist,
                                  mar, talpha),
           0);
    /* invalid arguments: every entry point returns -1 before allocating */
    EXPECT(oracle_chain(NULL, drf, 0, tok, u, B, G, V, 1.0, acc, out, NULL, NULL, NULL, NULL, 1), -1);
    EXPECT(oracle_chain(tgt, drf, 0, tok, u, B, G, V, -1.0, acc, out, NULL, NULL, NULL, NULL, 1), -1);
    EXPECT(oracle_chain_pointmass(tgt, 7, tok, u, B, G, V, 1.0, acc, out, NULL, NULL, NULL, NULL, 1),
           -1);
    EXPECT(oracle_chain_alpha(tgt, drf, 0, 0, G, V, 1.0, alpha, 1), -1);
    EXPECT(oracle_outcome_topk(tgt, 0, tok, B, G, V, 1.0, 0, ck, ca, cp, hit, NULL), -1);
    EXPECT(oracle_tree_greedy(tt, 0, par, ntok, B, 0, V, acc, node, outt, NULL, 1), -1);
    EXPECT(oracle_tree_build(zb, 0, B, M, V, 1.0, 0, 3, BUD, NULL, bpar, btok, brow, bsc, bn, gap),
           -1);
    EXPECT(oracle_tree_score(zb, 0, B, M, V, NAN, BUD, bpar, btok, brow, bn, sc2), -1);
    EXPECT(oracle_tree_stochastic(tt, td, 0, par, ntok, NULL, B, N, V, 1.0, acc, node, outt, NULL,
                                  NULL, NULL),
           -1);
    if (fails) {
        fprintf(stderr, "%d unexpected return code(s)\n", fails);
        return 1;
    }
    printf("oracle harness: every entry point, valid and invalid calls, returned as expected\n");
    return 0;
}
