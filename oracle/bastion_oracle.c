/*
 * bastion_oracle.c -- plain, slow CPU reference for the tree-drafting hot path.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the CPU
 * baseline leg of the benchmark load this file's library.  It shares no code,
 * header, table or constant with the HIP library, and nothing in the product
 * path calls it.  It is written for a reader to check against the pages by
 * eye: every step is the plain definition, in double precision where the
 * pages leave the precision open, with no blocking, fusion or reordering.
 *
 * Sources (AI-written summaries of two papers, as web pages):
 *  [B-M1]  "Bastion: Budget-Aware Speculative Decoding with Tree-structured
 *          Block Diffusion Drafting" (gist.science, Dutch and French pages),
 *          technical summary, Methodology 1 "tree-based block-diffusion
 *          drafting": one drafter pass gives position-wise marginals q_k(.);
 *          candidates at different positions combine freely into a prefix
 *          tree; node i at depth d(i) scores rho(i) = prod_{k<=d(i)} q_k(x_ik).
 *  [B-M2]  same page, Methodology 2 "acceptance surrogate and best-first
 *          expansion": A_hat(T) = sum_{i in T} rho(i); best-first repeatedly
 *          adds the valid node with the highest rho; optimal for A_hat under
 *          a fixed budget, with a concave A_hat(N).
 *  [B-M3]  same page, Methodology 3 "hardware-aware online budget
 *          controller": roofline verify latency; grow the tree until
 *          S(N) = A_hat(T_N) * L_AR / C(N) starts to decrease.
 *  [B-Res] same page, Experimental results: greedy decoding (temperature 0)
 *          with tree-structured verification by the target.
 *  [D-M1]  "DBLAST: Dependent Block Drafting for Stochastic Speculative
 *          Decoding" (gist.science, Dutch page), Methodology 1 "dependent
 *          block sampling via a latent mixture": factorised proposal
 *          q(x_1:b|y) = prod_i q_i(x_i|y) and the CP mixture
 *          q_dep(x_1:b|y) = sum_z q(z|y) prod_i q_i(x_i|y,z); at inference a
 *          branch is decoded greedily in one pass.
 *
 * Readings where the pages are silent (stated once here, used below):
 *  - rho of the root is the empty product 1 and the root is part of T, so
 *    A_hat(T_0) = 1 and A_hat counts committed tokens.
 *  - N counts non-root nodes.
 *  - candidates of a depth-d node are the k most likely tokens of position
 *    d+1, ranked by (logit desc, token id asc).
 *  - softmax is over the full vocabulary at temperature 1.
 *  - rho is a float32 product, one rounding per factor, rho(child) =
 *    fl32(rho(parent) * q); A_hat and S(N) are float64.
 *  - best-first ties: (rho desc, depth asc, token asc, parent index asc).
 *  - "until S starts to decrease": the first n >= nmin with S(n+1) < S(n).
 *  - mask row i holds node i and all its ancestors (root included).
 *  - position id of node i = pos_base + depth(i).
 *  - greedy acceptance walks from the root while the target's argmax at the
 *    current node equals the token of one of its children.
 *  - mixture tree: candidates of position i are the union over branches of
 *    their top-k; a node scores sum_z w_z prod_{i<=d} q_i(x_i|z), with the
 *    per-branch products float32 and the sum a float32 fma chain over z.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORACLE_OK 0
#define ORACLE_BAD_LOGITS 1
#define ORACLE_EXHAUSTED 2

int oracle_abi_version(void) { return 1; }

#ifdef _OPENMP
#include <omp.h>
int oracle_num_threads(void) { return omp_get_max_threads(); }
void oracle_set_num_threads(int n) { omp_set_num_threads(n > 0 ? n : 1); }
#else
int oracle_num_threads(void) { return 1; }
void oracle_set_num_threads(int n) { (void)n; }
#endif

/* bf16 is the upper half of an IEEE binary32. */
static double logit_at(const void *base, int dtype, int64_t idx)
{
    float f;
    if (dtype == 0) {
        f = ((const float *)base)[idx];
    } else {
        uint32_t bits = (uint32_t)((const uint16_t *)base)[idx] << 16;
        memcpy(&f, &bits, sizeof f);
    }
    return (double)f;
}

/* ------------------------------------------------------------------------
 * Position-wise marginals and their top-k  [B-M1].
 * For each row: M = max_v l_v, S = sum_v exp(l_v - M),
 * p(v) = exp(l_v - M) / S, and the k tokens ranked first by
 * (logit desc, id asc), each with its p.
 * A row is bad when it holds a NaN or +inf, or when every entry is -inf;
 * any other row (however large its logits) gets its softmax.
 * ------------------------------------------------------------------------ */
void oracle_softmax_topk(const void *logits, int dtype, int64_t nrows, int V,
                         int64_t row_stride, int k, double *row_max,
                         double *row_sum, int32_t *topk_ids, double *topk_p,
                         int32_t *row_status)
{
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t r = 0; r < nrows; ++r) {
        double *x = (double *)malloc(sizeof(double) * (size_t)V);
        unsigned char *taken = (unsigned char *)calloc((size_t)V, 1);
        int bad = 0;
        double M = -INFINITY;
        for (int v = 0; v < V; ++v) {
            x[v] = logit_at(logits, dtype, r * row_stride + v);
            if (isnan(x[v]) || x[v] == INFINITY)
                bad = 1;
            else if (x[v] > M)
                M = x[v];
        }
        if (M == -INFINITY)
            bad = 1;
        row_status[r] = bad ? ORACLE_BAD_LOGITS : ORACLE_OK;
        if (bad) {
            row_max[r] = 0.0;
            row_sum[r] = 0.0;
            for (int j = 0; j < k; ++j) {
                topk_ids[r * k + j] = -1;
                topk_p[r * k + j] = 0.0;
            }
            free(x);
            free(taken);
            continue;
        }
        double S = 0.0;
        for (int v = 0; v < V; ++v)
            S += exp(x[v] - M);
        row_max[r] = M;
        row_sum[r] = S;
        /* k rounds of "take the best remaining token". */
        for (int j = 0; j < k; ++j) {
            int best = -1;
            for (int v = 0; v < V; ++v) {
                if (taken[v])
                    continue;
                if (best < 0 || x[v] > x[best])  /* ties keep the smaller id */
                    best = v;
            }
            taken[best] = 1;
            topk_ids[r * k + j] = best;
            topk_p[r * k + j] = exp(x[best] - M) / S;
        }
        free(x);
        free(taken);
    }
}

/* ------------------------------------------------------------------------
 * Budget rule  [B-M3]:  S(n) = A_hat[n] * L_AR / C[n];
 * N* = the first n in [nmin, count-1] with S(n+1) < S(n), else count.
 * ------------------------------------------------------------------------ */
static int budget_rule(const double *ahat, int count, int nmin,
                       const double *cost_q, double l_ar, double *s_curve)
{
    if (s_curve)
        for (int n = 0; n <= count; ++n)
            s_curve[n] = ahat[n] * l_ar / cost_q[n];
    for (int n = nmin; n < count; ++n) {
        double s_n = ahat[n] * l_ar / cost_q[n];
        double s_next = ahat[n + 1] * l_ar / cost_q[n + 1];
        if (s_next < s_n)
            return n;
    }
    return count;
}

/* ------------------------------------------------------------------------
 * Best-first expansion  [B-M1] [B-M2] [B-M3].
 * A candidate is (rho, depth, token, parent).  "Better" is the order
 * (rho desc, depth asc, token asc, parent asc).
 * ------------------------------------------------------------------------ */
typedef struct {
    float rho;
    int depth;
    int token;
    int parent;
} cand_t;

static int better(const cand_t *a, const cand_t *b)
{
    if (a->rho != b->rho)
        return a->rho > b->rho;
    if (a->depth != b->depth)
        return a->depth < b->depth;
    if (a->token != b->token)
        return a->token < b->token;
    return a->parent < b->parent;
}

static void pad_tree(int q, int from, int nmax, int32_t *parent, int32_t *depth,
                     int32_t *token, float *rho, double *ahat)
{
    for (int i = from; i <= nmax; ++i) {
        int64_t o = (int64_t)q * (nmax + 1) + i;
        parent[o] = -1;
        depth[o] = -1;
        token[o] = -1;
        rho[o] = 0.0f;
        ahat[o] = 0.0;
    }
}

/*
 * topk_ids/topk_q: [B, b, k] (the candidates of each position and their
 * probabilities, float32); row_status: [B, b] or NULL.
 * cost: NULL for a fixed budget N = nmax, else [.., nmax+1] per query at
 * cost + q * cost_qstride (stride 0 shares one table).
 * Outputs [B, nmax+1]: nodes in pop order, node 0 the root (parent -1,
 * depth 0, token -1, rho 1); entries after n_nodes[q] are padding
 * (parent -1, depth -1, token -1, rho 0, ahat 0).
 */
void oracle_best_first(const int32_t *topk_ids, const float *topk_q,
                       const int32_t *row_status, int B, int b, int k, int nmax,
                       int nmin, const double *cost, int64_t cost_qstride,
                       double l_ar, int32_t *parent, int32_t *depth,
                       int32_t *token, float *rho, double *ahat,
                       int32_t *n_nodes, int32_t *qstatus)
{
#pragma omp parallel for schedule(dynamic, 1)
    for (int q = 0; q < B; ++q) {
        int64_t o = (int64_t)q * (nmax + 1);
        int bad = 0;
        if (row_status)
            for (int p = 0; p < b; ++p)
                if (row_status[q * b + p] != ORACLE_OK)
                    bad = 1;
        if (bad) {
            /* the tree is the root alone */
            parent[o] = -1;
            depth[o] = 0;
            token[o] = -1;
            rho[o] = 1.0f;
            ahat[o] = 1.0;
            pad_tree(q, 1, nmax, parent, depth, token, rho, ahat);
            n_nodes[q] = 0;
            qstatus[q] = ORACLE_BAD_LOGITS;
            continue;
        }
        cand_t *front = (cand_t *)malloc(sizeof(cand_t) * (size_t)(nmax + 1) * k);
        int nfront = 0;
        /* the root */
        parent[o] = -1;
        depth[o] = 0;
        token[o] = -1;
        rho[o] = 1.0f;
        ahat[o] = 1.0;
        for (int j = 0; j < k; ++j) {
            cand_t c;
            c.rho = 1.0f * topk_q[((int64_t)q * b + 0) * k + j];
            c.depth = 1;
            c.token = topk_ids[((int64_t)q * b + 0) * k + j];
            c.parent = 0;
            front[nfront++] = c;
        }
        int count = 0;
        while (count < nmax && nfront > 0) {
            int best = 0;
            for (int f = 1; f < nfront; ++f)
                if (better(&front[f], &front[best]))
                    best = f;
            cand_t c = front[best];
            front[best] = front[--nfront];
            int n = ++count;
            parent[o + n] = c.parent;
            depth[o + n] = c.depth;
            token[o + n] = c.token;
            rho[o + n] = c.rho;
            ahat[o + n] = ahat[o + n - 1] + (double)c.rho;
            if (c.depth < b) {
                for (int j = 0; j < k; ++j) {
                    cand_t ch;
                    float qv = topk_q[((int64_t)q * b + c.depth) * k + j];
                    ch.rho = c.rho * qv;
                    ch.depth = c.depth + 1;
                    ch.token = topk_ids[((int64_t)q * b + c.depth) * k + j];
                    ch.parent = n;
                    front[nfront++] = ch;
                }
            }
        }
        int nstar = count;
        if (cost)
            nstar = budget_rule(ahat + o, count, nmin, cost + q * cost_qstride,
                                l_ar, NULL);
        pad_tree(q, nstar + 1, nmax, parent, depth, token, rho, ahat);
        n_nodes[q] = nstar;
        qstatus[q] = (nstar == count && count < nmax) ? ORACLE_EXHAUSTED : ORACLE_OK;
        free(front);
    }
}

/* ------------------------------------------------------------------------
 * The budget rule on a recorded A_hat curve  [B-M3].
 * ahat: [B, nmax+1] with entries 0..n_avail[q] valid.
 * nstar[B]; s_curve [B, nmax+1] (optional): S(n) for n <= n_avail[q], 0 after.
 * ------------------------------------------------------------------------ */
void oracle_budget_select(const double *ahat, const int32_t *n_avail, int B,
                          int nmax, int nmin, const double *cost,
                          int64_t cost_qstride, double l_ar, int32_t *nstar,
                          double *s_curve)
{
    for (int q = 0; q < B; ++q) {
        int count = n_avail[q];
        double *sc = s_curve ? s_curve + (int64_t)q * (nmax + 1) : NULL;
        if (sc)
            for (int n = 0; n <= nmax; ++n)
                sc[n] = 0.0;
        nstar[q] = budget_rule(ahat + (int64_t)q * (nmax + 1), count, nmin,
                               cost + q * cost_qstride, l_ar, sc);
    }
}

/* ------------------------------------------------------------------------
 * Ancestor mask and position ids for a tree-structured verifier ([B-Res]:
 * the target checks the whole tree in one pass; the pages give no format).
 * Row i of mask[q] (W = ceil((nmax+1)/32) words, LSB first) has bit j set iff
 * j == i or j is an ancestor of i.  position_ids = pos_base[q] + depth(i),
 * depth counted by walking parents.  Rows after n_nodes[q] are zero and their
 * position id is -1.  The walk stops at the first link that is not a valid
 * parent (0 <= parent < child).
 * ------------------------------------------------------------------------ */
void oracle_tree_mask(const int32_t *parent, const int32_t *n_nodes, int B,
                      int nmax, const int32_t *pos_base, uint32_t *mask,
                      int32_t *position_ids)
{
    int W = (nmax + 1 + 31) / 32;
    for (int q = 0; q < B; ++q) {
        int n = n_nodes[q];
        if (n < 0)
            n = -1;
        if (n > nmax)
            n = nmax;
        for (int i = 0; i <= nmax; ++i) {
            uint32_t *row = mask + ((int64_t)q * (nmax + 1) + i) * W;
            for (int w = 0; w < W; ++w)
                row[w] = 0u;
            int64_t po = (int64_t)q * (nmax + 1) + i;
            if (i > n) {
                position_ids[po] = -1;
                continue;
            }
            int j = i, steps = 0;
            row[j / 32] |= 1u << (j % 32);
            while (j > 0) {
                int p = parent[(int64_t)q * (nmax + 1) + j];
                if (p < 0 || p >= j)
                    break;
                row[p / 32] |= 1u << (p % 32);
                j = p;
                ++steps;
            }
            position_ids[po] = (pos_base ? pos_base[q] : 0) + steps;
        }
    }
}

/* ------------------------------------------------------------------------
 * Greedy acceptance  [B-Res] (temperature 0).
 * target[q, i] is the target model's argmax token after node i's path.
 * From the root: while some child c of the current node (c > current,
 * parent[c] == current, c <= n_nodes) has token[c] == target[current], move
 * to it (the lowest such c).  At most b moves.
 * accept_len = number of moves; accept_nodes[q, 0..len] the path (root
 * first), -1 after; bonus = target at the last accepted node.
 * ------------------------------------------------------------------------ */
void oracle_accept(const int32_t *parent, const int32_t *token,
                   const int32_t *n_nodes, int B, int nmax, int b,
                   const int32_t *target, int32_t *accept_len,
                   int32_t *accept_nodes, int32_t *bonus)
{
    for (int q = 0; q < B; ++q) {
        int64_t o = (int64_t)q * (nmax + 1);
        int n = n_nodes[q] > nmax ? nmax : n_nodes[q];
        int cur = 0, len = 0;
        int32_t *path = accept_nodes + (int64_t)q * (b + 1);
        for (int m = 0; m <= b; ++m)
            path[m] = -1;
        path[0] = 0;
        while (len < b) {
            int t = target[o + cur];
            int found = -1;
            for (int c = cur + 1; c <= n; ++c)
                if (parent[o + c] == cur && token[o + c] == t) {
                    found = c;
                    break;
                }
            if (found < 0)
                break;
            cur = found;
            path[++len] = cur;
        }
        accept_len[q] = len;
        bonus[q] = target[o + cur];
    }
}

/* ------------------------------------------------------------------------
 * Latent mixture  [D-M1].
 * branch rows are [B, K, b, V]; prior logits [B, K].
 *  w = softmax(prior logits) (float64);
 *  chain z: x^(z)_i = top-1 token of branch z at position i (greedy branch);
 *  q_dep(x^(z)) = sum_z' w_z' prod_i p_{z',i}(x^(z)_i), with
 *  p_{z',i}(x) = exp(l - M) / S of row (z', i) at token x;
 *  candidates of position i: the sorted union over z of the k best tokens
 *  of row (z, i); cand_p[q, i, c, z] = p_{z,i}(cand c).
 * Uses oracle_softmax_topk for the rows.
 * Outputs: prior_w [B,K], chain_tokens [B,K,b], qdep_chain [B,K],
 * cand_count [B,b], cand_tokens [B,b,K*k] (-1 padded),
 * cand_p [B,b,K*k,K] (0 padded), row_status [B,K,b].
 * ------------------------------------------------------------------------ */
static double row_prob(const void *logits, int dtype, int64_t row, int64_t stride,
                       int token, double M, double S)
{
    return exp(logit_at(logits, dtype, row * stride + token) - M) / S;
}

void oracle_mixture(const void *branch_logits, int dtype, const float *prior_logits,
                    int B, int K, int b, int V, int64_t row_stride, int k,
                    double *prior_w, int32_t *chain_tokens, double *qdep_chain,
                    int32_t *cand_count, int32_t *cand_tokens, double *cand_p,
                    int32_t *row_status)
{
    int64_t nrows = (int64_t)B * K * b;
    double *row_max = (double *)malloc(sizeof(double) * (size_t)nrows);
    double *row_sum = (double *)malloc(sizeof(double) * (size_t)nrows);
    int32_t *ids = (int32_t *)malloc(sizeof(int32_t) * (size_t)nrows * k);
    double *p = (double *)malloc(sizeof(double) * (size_t)nrows * k);
    oracle_softmax_topk(branch_logits, dtype, nrows, V, row_stride, k, row_max,
                        row_sum, ids, p, row_status);
    int C = K * k;
#pragma omp parallel for schedule(dynamic, 1)
    for (int q = 0; q < B; ++q) {
        /* prior */
        double pm = -INFINITY, ps = 0.0;
        for (int z = 0; z < K; ++z)
            if ((double)prior_logits[q * K + z] > pm)
                pm = (double)prior_logits[q * K + z];
        for (int z = 0; z < K; ++z)
            ps += exp((double)prior_logits[q * K + z] - pm);
        for (int z = 0; z < K; ++z)
            prior_w[q * K + z] = exp((double)prior_logits[q * K + z] - pm) / ps;
        int bad = 0;
        for (int z = 0; z < K; ++z)
            for (int i = 0; i < b; ++i)
                if (row_status[((int64_t)q * K + z) * b + i] != ORACLE_OK)
                    bad = 1;
        /* chains */
        for (int z = 0; z < K; ++z)
            for (int i = 0; i < b; ++i)
                chain_tokens[((int64_t)q * K + z) * b + i] =
                    bad ? -1 : ids[(((int64_t)q * K + z) * b + i) * k + 0];
        for (int z = 0; z < K; ++z) {
            double qd = 0.0;
            if (!bad) {
                for (int zp = 0; zp < K; ++zp) {
                    double prod = 1.0;
                    for (int i = 0; i < b; ++i) {
                        int64_t row = ((int64_t)q * K + zp) * b + i;
                        int x = chain_tokens[((int64_t)q * K + z) * b + i];
                        prod *= row_prob(branch_logits, dtype, row, row_stride, x,
                                         row_max[row], row_sum[row]);
                    }
                    qd += prior_w[q * K + zp] * prod;
                }
            }
            qdep_chain[q * K + z] = qd;
        }
        /* candidate union per position, ascending token order */
        for (int i = 0; i < b; ++i) {
            int32_t *ct = cand_tokens + ((int64_t)q * b + i) * C;
            double *cp = cand_p + ((int64_t)q * b + i) * C * K;
            int cnt = 0;
            for (int c = 0; c < C; ++c) {
                ct[c] = -1;
                for (int z = 0; z < K; ++z)
                    cp[c * K + z] = 0.0;
            }
            if (!bad) {
                for (int z = 0; z < K; ++z)
                    for (int j = 0; j < k; ++j) {
                        int t = ids[(((int64_t)q * K + z) * b + i) * k + j];
                        int seen = 0;
                        for (int c = 0; c < cnt; ++c)
                            if (ct[c] == t)
                                seen = 1;
                        if (!seen)
                            ct[cnt++] = t;
                    }
                /* insertion sort, ascending */
                for (int a = 1; a < cnt; ++a) {
                    int t = ct[a], m = a;
                    while (m > 0 && ct[m - 1] > t) {
                        ct[m] = ct[m - 1];
                        --m;
                    }
                    ct[m] = t;
                }
                for (int c = 0; c < cnt; ++c)
                    for (int z = 0; z < K; ++z) {
                        int64_t row = ((int64_t)q * K + z) * b + i;
                        cp[c * K + z] = row_prob(branch_logits, dtype, row, row_stride,
                                                 ct[c], row_max[row], row_sum[row]);
                    }
            }
            cand_count[q * b + i] = cnt;
        }
    }
    free(row_max);
    free(row_sum);
    free(ids);
    free(p);
}

/* ------------------------------------------------------------------------
 * Candidates from the mixture marginal  [D-M1] with [B-M1].
 * The latent mixture's position-i marginal is
 *   m_i(x) = sum_z w_z p_{z,i}(x),   w = softmax(prior logits),
 * p_{z,i} the full-vocabulary softmax of branch row (z, i).  The candidates
 * of position i are the k tokens ranked first by (m desc, token asc); each
 * comes with m and with p_{z,i}(x) for every branch z (the mixture tree's
 * per-branch factors).  float64 throughout.
 * Outputs: prior_w [B,K], marg_ids [B,b,k], marg_p [B,b,k],
 * cand_p [B,b,k,K], row_status [B,K,b].
 * ------------------------------------------------------------------------ */
void oracle_mixture_marginal(const void *branch_logits, int dtype,
                             const float *prior_logits, int B, int K, int b, int V,
                             int64_t row_stride, int k, double *prior_w,
                             int32_t *marg_ids, double *marg_p, double *cand_p,
                             int32_t *row_status)
{
    int64_t nrows = (int64_t)B * K * b;
    double *row_max = (double *)malloc(sizeof(double) * (size_t)nrows);
    double *row_sum = (double *)malloc(sizeof(double) * (size_t)nrows);
    int32_t *ids = (int32_t *)malloc(sizeof(int32_t) * (size_t)nrows);
    double *p1 = (double *)malloc(sizeof(double) * (size_t)nrows);
    oracle_softmax_topk(branch_logits, dtype, nrows, V, row_stride, 1, row_max,
                        row_sum, ids, p1, row_status);
#pragma omp parallel for schedule(dynamic, 1)
    for (int qi = 0; qi < B * b; ++qi) {
        int q = qi / b, i = qi - q * b;
        double pm = -INFINITY, ps = 0.0;
        for (int z = 0; z < K; ++z)
            if ((double)prior_logits[q * K + z] > pm)
                pm = (double)prior_logits[q * K + z];
        for (int z = 0; z < K; ++z)
            ps += exp((double)prior_logits[q * K + z] - pm);
        if (i == 0)
            for (int z = 0; z < K; ++z)
                prior_w[q * K + z] = exp((double)prior_logits[q * K + z] - pm) / ps;
        int bad = 0;
        for (int z = 0; z < K; ++z)
            for (int j = 0; j < b; ++j)
                if (row_status[((int64_t)q * K + z) * b + j] != ORACLE_OK)
                    bad = 1;
        int32_t *oid = marg_ids + (int64_t)qi * k;
        double *op = marg_p + (int64_t)qi * k;
        double *oc = cand_p + (int64_t)qi * k * K;
        if (bad) {
            for (int j = 0; j < k; ++j) {
                oid[j] = -1;
                op[j] = 0.0;
                for (int z = 0; z < K; ++z)
                    oc[j * K + z] = 0.0;
            }
            continue;
        }
        /* the marginal of every token */
        double *m = (double *)malloc(sizeof(double) * (size_t)V);
        unsigned char *taken = (unsigned char *)calloc((size_t)V, 1);
        for (int x = 0; x < V; ++x) {
            double acc = 0.0;
            for (int z = 0; z < K; ++z) {
                int64_t row = ((int64_t)q * K + z) * b + i;
                double w = exp((double)prior_logits[q * K + z] - pm) / ps;
                acc += w * exp(logit_at(branch_logits, dtype, row * row_stride + x) - row_max[row]) /
                       row_sum[row];
            }
            m[x] = acc;
        }
        /* k rounds of "take the best remaining token" */
        for (int j = 0; j < k; ++j) {
            int best = -1;
            for (int x = 0; x < V; ++x) {
                if (taken[x])
                    continue;
                if (best < 0 || m[x] > m[best])   /* ties keep the smaller id */
                    best = x;
            }
            taken[best] = 1;
            oid[j] = best;
            op[j] = m[best];
            for (int z = 0; z < K; ++z) {
                int64_t row = ((int64_t)q * K + z) * b + i;
                oc[j * K + z] = exp(logit_at(branch_logits, dtype, row * row_stride + best) -
                                    row_max[row]) / row_sum[row];
            }
        }
        free(m);
        free(taken);
    }
    free(row_max);
    free(row_sum);
    free(ids);
    free(p1);
}

/*
 * q_dep of arbitrary token sequences  [D-M1]:
 * seqs [B, n, b] -> out [B, n] = sum_z w_z prod_i p_{z,i}(seq_i).
 */
void oracle_qdep_sequences(const void *branch_logits, int dtype,
                           const float *prior_logits, int B, int K, int b, int V,
                           int64_t row_stride, const int32_t *seqs, int n,
                           double *out)
{
    (void)V;
    int64_t nrows = (int64_t)B * K * b;
    double *row_max = (double *)malloc(sizeof(double) * (size_t)nrows);
    double *row_sum = (double *)malloc(sizeof(double) * (size_t)nrows);
    int32_t *ids = (int32_t *)malloc(sizeof(int32_t) * (size_t)nrows);
    double *p = (double *)malloc(sizeof(double) * (size_t)nrows);
    int32_t *st = (int32_t *)malloc(sizeof(int32_t) * (size_t)nrows);
    oracle_softmax_topk(branch_logits, dtype, nrows, V, row_stride, 1, row_max,
                        row_sum, ids, p, st);
    for (int q = 0; q < B; ++q) {
        double pm = -INFINITY, ps = 0.0;
        for (int z = 0; z < K; ++z)
            if ((double)prior_logits[q * K + z] > pm)
                pm = (double)prior_logits[q * K + z];
        for (int z = 0; z < K; ++z)
            ps += exp((double)prior_logits[q * K + z] - pm);
        for (int s = 0; s < n; ++s) {
            double total = 0.0;
            for (int z = 0; z < K; ++z) {
                double prod = 1.0;
                for (int i = 0; i < b; ++i) {
                    int64_t row = ((int64_t)q * K + z) * b + i;
                    int x = seqs[((int64_t)q * n + s) * b + i];
                    prod *= row_prob(branch_logits, dtype, row, row_stride, x,
                                     row_max[row], row_sum[row]);
                }
                total += exp((double)prior_logits[q * K + z] - pm) / ps * prod;
            }
            out[(int64_t)q * n + s] = total;
        }
    }
    free(row_max);
    free(row_sum);
    free(ids);
    free(p);
    free(st);
}

/* ------------------------------------------------------------------------
 * Mixture tree  [D-M1] with [B-M1]/[B-M2] best-first.
 * Inputs: w [B,K] float32 (branch weights), cand_count [B,b],
 * cand_tokens [B,b,C], cand_q [B,b,C,K] float32 (q_i(cand|z)), C = slots,
 * row_status [B,K,b] or NULL (a bad row makes the whole query bad).
 * A node keeps r_z = fl32 product of q_i(x_i|z) along its path (root: 1).
 * Its score is the float32 fma chain acc = fma(w_z, r_z, acc), z = 0..K-1,
 * from acc = 0.  Best-first on (score desc, depth asc, token asc, parent asc)
 * with a fixed budget nmax.  A_hat[0] = 1.  Outputs as oracle_best_first.
 * ------------------------------------------------------------------------ */
typedef struct {
    cand_t c;
    int slot;   /* which r-vector block holds this candidate's r_z */
} mcand_t;

void oracle_mixture_tree(const float *w, const int32_t *cand_count,
                         const int32_t *cand_tokens, const float *cand_q,
                         const int32_t *row_status, int B, int K, int b, int C,
                         int nmax, int32_t *parent, int32_t *depth, int32_t *token,
                         float *rho, double *ahat, int32_t *n_nodes,
                         int32_t *qstatus)
{
#pragma omp parallel for schedule(dynamic, 1)
    for (int q = 0; q < B; ++q) {
        int64_t o = (int64_t)q * (nmax + 1);
        int bad = 0;
        if (row_status)
            for (int r = 0; r < K * b; ++r)
                if (row_status[(int64_t)q * K * b + r] != ORACLE_OK)
                    bad = 1;
        if (bad) {
            /* the tree is the root alone */
            parent[o] = -1;
            depth[o] = 0;
            token[o] = -1;
            rho[o] = 1.0f;
            ahat[o] = 1.0;
            pad_tree(q, 1, nmax, parent, depth, token, rho, ahat);
            n_nodes[q] = 0;
            qstatus[q] = ORACLE_BAD_LOGITS;
            continue;
        }
        int64_t cap = (int64_t)(nmax + 1) * C + 1;
        mcand_t *front = (mcand_t *)malloc(sizeof(mcand_t) * (size_t)cap);
        float *rfront = (float *)malloc(sizeof(float) * (size_t)cap * K);
        float *rnode = (float *)malloc(sizeof(float) * (size_t)(nmax + 1) * K);
        int nfront = 0, nslots = 0;
        parent[o] = -1;
        depth[o] = 0;
        token[o] = -1;
        rho[o] = 1.0f;
        ahat[o] = 1.0;
        for (int z = 0; z < K; ++z)
            rnode[z] = 1.0f;
        /* children of a popped node n (its r in rnode[n]) */
#define PUSH_CHILDREN(nodeidx, d)                                                  \
    do {                                                                           \
        int pos_ = (d);                                                            \
        int cnt_ = cand_count[q * b + pos_];                                       \
        for (int c_ = 0; c_ < cnt_; ++c_) {                                        \
            float *r_ = rfront + (int64_t)nslots * K;                             \
            const float *qz_ = cand_q + (((int64_t)q * b + pos_) * C + c_) * K;    \
            float acc_ = 0.0f;                                                     \
            for (int z_ = 0; z_ < K; ++z_) {                                       \
                r_[z_] = rnode[(int64_t)(nodeidx) * K + z_] * qz_[z_];             \
                acc_ = fmaf(w[q * K + z_], r_[z_], acc_);                          \
            }                                                                      \
            mcand_t m_;                                                            \
            m_.c.rho = acc_;                                                       \
            m_.c.depth = pos_ + 1;                                                 \
            m_.c.token = cand_tokens[((int64_t)q * b + pos_) * C + c_];            \
            m_.c.parent = (nodeidx);                                               \
            m_.slot = nslots++;                                                    \
            front[nfront++] = m_;                                                  \
        }                                                                          \
    } while (0)
        PUSH_CHILDREN(0, 0);
        int count = 0;
        while (count < nmax && nfront > 0) {
            int best = 0;
            for (int f = 1; f < nfront; ++f)
                if (better(&front[f].c, &front[best].c))
                    best = f;
            mcand_t m = front[best];
            front[best] = front[--nfront];
            int n = ++count;
            parent[o + n] = m.c.parent;
            depth[o + n] = m.c.depth;
            token[o + n] = m.c.token;
            rho[o + n] = m.c.rho;
            ahat[o + n] = ahat[o + n - 1] + (double)m.c.rho;
            for (int z = 0; z < K; ++z)
                rnode[(int64_t)n * K + z] = rfront[(int64_t)m.slot * K + z];
            if (m.c.depth < b)
                PUSH_CHILDREN(n, m.c.depth);
        }
#undef PUSH_CHILDREN
        pad_tree(q, count + 1, nmax, parent, depth, token, rho, ahat);
        n_nodes[q] = count;
        qstatus[q] = count < nmax ? ORACLE_EXHAUSTED : ORACLE_OK;
        free(front);
        free(rfront);
        free(rnode);
    }
}

/* ------------------------------------------------------------------------
 * Stochastic variants.
 *
 * Counter-based uniforms: the MurmurHash3 32-bit finalizer (fmix32, Austin
 * Appleby, public domain) applied to a key built from (seed, query, node,
 * token); u = ((h >> 8) + 1/2) / 2^24, in (0, 1).  The key:
 *   a = fmix32(seed + 0x9E3779B9 (q + 1)),
 *   c = fmix32(a ^ 0x85EBCA6B (node + 1)),
 *   h = fmix32(c ^ token),   all arithmetic mod 2^32.
 * ------------------------------------------------------------------------ */
static uint32_t fmix32(uint32_t h)
{
    h ^= h >> 16;
    h *= 0x85EBCA6Bu;
    h ^= h >> 13;
    h *= 0xC2B2AE35u;
    h ^= h >> 16;
    return h;
}

static double uniform_at(uint32_t seed, uint32_t q, uint32_t node, uint32_t token)
{
    uint32_t a = fmix32(seed + 0x9E3779B9u * (q + 1u));
    uint32_t c = fmix32(a ^ (0x85EBCA6Bu * (node + 1u)));
    uint32_t h = fmix32(c ^ token);
    return ((double)(h >> 8) + 0.5) / 16777216.0;
}

/*
 * A draw from the target's distribution at every tree node  [B-Res] with a
 * target temperature (the DBlast page evaluates targets at temperatures
 * 0.7-1.5, Problem statement and Experimental results): node i of query q
 * draws x from softmax(l / T) of its logits row, by the Gumbel-max rule
 * x = argmax_v (l_v / T + g_v), g_v = -log(-log(u_v)) (ties: smaller token);
 * T = 0 is the argmax of l (greedy).  float64.  Rows after n_nodes[q] get
 * -1.  logits [B, nmax+1, V] (row_stride between nodes); sampled and score
 * [B, nmax+1] (score: the winning l/T + g, or l for T = 0).
 */
void oracle_sample_nodes(const void *logits, int dtype, int B, int nmax, int V,
                         int64_t row_stride, const int32_t *n_nodes, double temperature,
                         uint32_t seed, int32_t *sampled, double *score)
{
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t r = 0; r < (int64_t)B * (nmax + 1); ++r) {
        int q = (int)(r / (nmax + 1)), node = (int)(r - (int64_t)q * (nmax + 1));
        if (node > n_nodes[q]) {
            sampled[r] = -1;
            score[r] = 0.0;
            continue;
        }
        int best = -1;
        double bs = -INFINITY;
        for (int v = 0; v < V; ++v) {
            double l = logit_at(logits, dtype, r * row_stride + v);
            double sc = l;
            if (temperature > 0.0) {
                double u = uniform_at(seed, (uint32_t)q, (uint32_t)node, (uint32_t)v);
                sc = l / temperature - log(-log(u));
            }
            if (best < 0 || sc > bs) {
                best = v;
                bs = sc;
            }
        }
        sampled[r] = best;
        score[r] = bs;
    }
}

/*
 * The uniform of (seed, q, node, token) as defined above (exposed so that
 * tests can check draws against it).
 */
double oracle_uniform_at(uint32_t seed, uint32_t q, uint32_t node, uint32_t token)
{
    return uniform_at(seed, q, node, token);
}

/*
 * DBlast branch sampling  [D-M1] (at inference one branch is decoded
 * greedily; the latent category is drawn with a temperature Z_T):
 * z = the smallest index with u < sum_{z' <= z} w_z', w = softmax(prior / Z_T)
 * in float64 (Z_T = 0: the argmax of the prior, ties to the smaller index).
 * draft[q] = chain_tokens[q, z].  u [B] in [0, 1).
 */
void oracle_mixture_sample(const float *prior_logits, int B, int K, double temperature,
                           const double *u, const int32_t *chain_tokens, int b,
                           int32_t *z_out, int32_t *draft)
{
    for (int q = 0; q < B; ++q) {
        int z = 0;
        if (temperature <= 0.0) {
            for (int j = 1; j < K; ++j)
                if (prior_logits[q * K + j] > prior_logits[q * K + z])
                    z = j;
        } else {
            double pm = -INFINITY, ps = 0.0;
            for (int j = 0; j < K; ++j)
                if ((double)prior_logits[q * K + j] / temperature > pm)
                    pm = (double)prior_logits[q * K + j] / temperature;
            for (int j = 0; j < K; ++j)
                ps += exp((double)prior_logits[q * K + j] / temperature - pm);
            double cdf = 0.0;
            z = K - 1;
            for (int j = 0; j < K; ++j) {
                cdf += exp((double)prior_logits[q * K + j] / temperature - pm) / ps;
                if (u[q] < cdf) {
                    z = j;
                    break;
                }
            }
        }
        z_out[q] = z;
        for (int i = 0; i < b; ++i)
            draft[(int64_t)q * b + i] = chain_tokens[((int64_t)q * K + z) * b + i];
    }
}
