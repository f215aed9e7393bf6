/*
 * Runs every function of the CPU reference (oracle/bastion_oracle.c) on
 * small inputs, for a build with AddressSanitizer and UndefinedBehavior-
 * Sanitizer (test infrastructure; tests/test_sanitizers_cpu.py builds and
 * runs it).  Exit status 0 when every call returned and nothing was
 * reported.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

void oracle_softmax_topk(const void *, int, int64_t, int, int64_t, int, double *, double *,
                         int32_t *, double *, int32_t *);
void oracle_best_first(const int32_t *, const float *, const int32_t *, int, int, int, int, int,
                       const double *, int64_t, double, int32_t *, int32_t *, int32_t *, float *,
                       double *, int32_t *, int32_t *);
void oracle_budget_select(const double *, const int32_t *, int, int, int, const double *, int64_t,
                          double, int32_t *, double *);
void oracle_tree_mask(const int32_t *, const int32_t *, int, int, const int32_t *, uint32_t *,
                      int32_t *);
void oracle_accept(const int32_t *, const int32_t *, const int32_t *, int, int, int,
                   const int32_t *, int32_t *, int32_t *, int32_t *);
void oracle_mixture(const void *, int, const float *, int, int, int, int, int64_t, int, double *,
                    int32_t *, double *, int32_t *, int32_t *, double *, int32_t *);
void oracle_mixture_tree(const float *, const int32_t *, const int32_t *, const float *,
                         const int32_t *, int, int, int, int, int, int32_t *, int32_t *,
                         int32_t *, float *, double *, int32_t *, int32_t *);
void oracle_mixture_marginal(const void *, int, const float *, int, int, int, int, int64_t, int,
                             double *, int32_t *, double *, double *, int32_t *);
void oracle_qdep_sequences(const void *, int, const float *, int, int, int, int, int64_t,
                           const int32_t *, int, double *);
void oracle_sample_nodes(const void *, int, int, int, int, int64_t, const int32_t *, double,
                         uint32_t, int32_t *, double *);
void oracle_mixture_sample(const float *, int, int, double, const double *, const int32_t *, int,
                           int32_t *, int32_t *);

static float frand(unsigned *s) {
    *s = *s * 1664525u + 1013904223u;
    return (float)((*s >> 8) & 0xFFFF) / 4096.0f - 8.0f;
}

int main(void) {
    enum { B = 3, b = 4, V = 97, k = 5, NMAX = 40, K = 3 };
    unsigned seed = 1;
    float *x = malloc(sizeof(float) * B * b * V);
    for (int i = 0; i < B * b * V; ++i) x[i] = frand(&seed);
    x[5] = -INFINITY;
    x[2 * V + 3] = NAN;                       /* a bad row */
    double rm[B * b], rs[B * b], p[B * b * k];
    int32_t ids[B * b * k], st[B * b];
    oracle_softmax_topk(x, 0, B * b, V, V, k, rm, rs, ids, p, st);
    float q[B * b * k];
    for (int i = 0; i < B * b * k; ++i) q[i] = (float)p[i];
    int W1 = NMAX + 1, W = (W1 + 31) / 32;
    int32_t par[B * 41], dep[B * 41], tok[B * 41], nn[B], qs[B];
    float rho[B * 41];
    double ah[B * 41], cost[41];
    for (int n = 0; n <= NMAX; ++n) cost[n] = 1.0 + 0.02 * n * n;
    oracle_best_first(ids, q, st, B, b, k, NMAX, 1, NULL, 0, 1.0, par, dep, tok, rho, ah, nn, qs);
    oracle_best_first(ids, q, st, B, b, k, NMAX, 1, cost, 0, 1.0, par, dep, tok, rho, ah, nn, qs);
    int32_t nst[B];
    double sc[B * 41];
    oracle_budget_select(ah, nn, B, NMAX, 1, cost, 0, 1.0, nst, sc);
    uint32_t *mask = malloc(sizeof(uint32_t) * B * W1 * W);
    int32_t pos[B * 41], pb[B] = {3, 0, 9};
    par[5] = 7;                               /* a malformed link */
    oracle_tree_mask(par, nn, B, NMAX, pb, mask, pos);
    int32_t tgt[B * 41], al[B], an[B * (b + 1)], bo[B];
    for (int i = 0; i < B * 41; ++i) tgt[i] = ids[(i % (b * k))];
    oracle_accept(par, tok, nn, B, NMAX, b, tgt, al, an, bo);

    float *xm = malloc(sizeof(float) * B * K * b * V);
    for (int i = 0; i < B * K * b * V; ++i) xm[i] = frand(&seed);
    float prior[B * K];
    for (int i = 0; i < B * K; ++i) prior[i] = frand(&seed) / 8.0f;
    int C = K * k;
    double pw[B * K], qd[B * K], cp[B * b * 15 * K];
    int32_t ch[B * K * b], cc[B * b], ct[B * b * 15], rst[B * K * b];
    oracle_mixture(xm, 0, prior, B, K, b, V, V, k, pw, ch, qd, cc, ct, cp, rst);
    float wq[B * K], cq[B * b * 15 * K];
    for (int i = 0; i < B * K; ++i) wq[i] = (float)pw[i];
    for (int i = 0; i < B * b * C * K; ++i) cq[i] = (float)cp[i];
    oracle_mixture_tree(wq, cc, ct, cq, rst, B, K, b, C, NMAX, par, dep, tok, rho, ah, nn, qs);
    int32_t mi[B * b * k];
    double mp[B * b * k], mcp[B * b * k * K];
    oracle_mixture_marginal(xm, 0, prior, B, K, b, V, V, k, pw, mi, mp, mcp, rst);
    double qseq[B * 2];
    int32_t seqs[B * 2 * b];
    for (int i = 0; i < B * 2 * b; ++i) seqs[i] = i % V;
    oracle_qdep_sequences(xm, 0, prior, B, K, b, V, V, seqs, 2, qseq);
    int32_t smp[B * 41];
    double ssc[B * 41];
    float *tl = malloc(sizeof(float) * B * 41 * V);
    for (int i = 0; i < B * 41 * V; ++i) tl[i] = frand(&seed);
    oracle_sample_nodes(tl, 0, B, NMAX, V, V, nn, 0.9, 77u, smp, ssc);
    oracle_sample_nodes(tl, 0, B, NMAX, V, V, nn, 0.0, 77u, smp, ssc);
    double u[B] = {0.1, 0.5, 0.99};
    int32_t zz[B], dr[B * b];
    oracle_mixture_sample(prior, B, K, 0.7, u, ch, b, zz, dr);
    oracle_mixture_sample(prior, B, K, 0.0, u, ch, b, zz, dr);
    free(x);
    free(mask);
    free(xm);
    free(tl);
    printf("oracle driver ok\n");
    return 0;
}
