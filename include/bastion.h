/*
 * bastion.h -- C ABI of the MI355X (gfx950) tree-drafting hot path.
 *
 * The library turns block-diffusion drafter logits [B, b, V] into
 * budget-optimal, prefix-closed candidate trees, ready for a tree-structured
 * verifier, and scores the greedy chains of a latent-mixture drafter.
 *
 * Sources (AI-written summaries of two papers, published as web pages):
 *   [BASTION] "Bastion: Budget-Aware Speculative Decoding with
 *             Tree-structured Block Diffusion Drafting", gist.science
 *             (Dutch and French pages), technical summary:
 *             Methodology 1 (position-wise marginals q_k, prefix tree, path
 *             score rho(i) = prod_{k<=d(i)} q_k(x_ik)), Methodology 2
 *             (A_hat(T) = sum_{i in T} rho(i), best-first expansion),
 *             Methodology 3 (roofline verify latency, stop when
 *             S(N) = A_hat(T_N) * L_AR / C(N) starts to decrease),
 *             Experimental results (greedy decoding, tree verification).
 *   [DBLAST]  "DBLAST: Dependent Block Drafting for Stochastic Speculative
 *             Decoding", gist.science (Dutch page), Methodology 1
 *             (q_dep(x_1:b|y) = sum_z q(z|y) prod_i q_i(x_i|y,z), greedy
 *             decoding of a branch).
 *
 * Conventions shared by every call:
 *  - All array pointers are DEVICE pointers owned by the caller.  The library
 *    allocates nothing and keeps no state between calls; scratch memory is a
 *    caller-provided workspace.
 *  - `stream` is a hipStream_t passed as void* (NULL = the default stream).
 *    Every call only enqueues work on it and returns; results are visible
 *    after the stream is synchronised.
 *  - The return value reports argument problems synchronously.  On
 *    BASTION_EINVAL / BASTION_EUNSUPPORTED / BASTION_EWORKSPACE nothing has
 *    been launched and nothing has been written.
 *  - Per-query data problems are reported in `qstatus` (BASTION_Q_*).
 *  - N counts non-root nodes; a tree has N+1 nodes.  Node 0 is the root (the
 *    last verified token): parent -1, depth 0, token -1, rho 1.  Nodes are
 *    stored in the order best-first added them, so parent[i] < i and the
 *    first n+1 entries of a tree built with budget N form the tree built
 *    with budget n.  The root counts in A_hat with rho = 1, so A_hat is the
 *    expected number of committed tokens (accepted drafts plus the bonus).
 *  - Ties: top-k ranks by (logit desc, token id asc); best-first pops by
 *    (rho desc, depth asc, token asc, parent index asc).
 *  - rho is a float32 product with one rounding per factor,
 *    rho(child) = fl32(rho(parent) * q); A_hat and S(N) are float64.
 *  - Limits: 1 <= b <= 32, 1 <= k <= 32, k <= V <= 524288, 1 <= nmax <= 1023,
 *    0 <= nmin <= nmax, 1 <= K <= 16, B <= 16384.  V is bounded by the
 *    19-bit token field of the pop-order keys and B by the launch grid.
 *
 * Where the calls differ from the plain statement of the problem (logits
 * in, a budgeted prefix-closed tree out, accepted length after
 * verification), and why:
 *  - bastion_build_trees takes pos_base and fills the verifier's mask and
 *    position ids inside the same launch when out->mask is set: the tree is
 *    still in LDS there, so the mask costs no second pass over the tree.
 *  - bastion_budget_select takes n_avail: a recorded A_hat curve may end
 *    before nmax (a candidate tree smaller than the budget).
 *  - bastion_tree_mask takes no depth array: depth is recounted along the
 *    parent links, so a malformed link cannot desynchronise the two.
 *  - bastion_mixture_score takes row_stride (as bastion_build_trees does)
 *    and returns its per-branch outputs in a struct, since they are many.
 *  - bastion_build_trees and bastion_mixture_score take a caller-owned
 *    workspace (the library allocates nothing).
 */
#ifndef BASTION_H
#define BASTION_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define BASTION_ABI_VERSION 1

/* return codes */
#define BASTION_OK 0
#define BASTION_EINVAL 1        /* bad argument (null pointer, size, limit) */
#define BASTION_EUNSUPPORTED 2  /* valid request the library cannot serve */
#define BASTION_EHIP 3          /* the HIP runtime reported an error */
#define BASTION_EWORKSPACE 4    /* workspace missing or too small */

/* per-query status */
#define BASTION_Q_OK 0
#define BASTION_Q_BAD_LOGITS 1  /* a row holds NaN or +inf, or is all -inf:
                                   the tree is the root alone */
#define BASTION_Q_EXHAUSTED 2   /* informational: the candidate tree had
                                   fewer nodes than the budget asked for */
#define BASTION_Q_RANGE 3       /* library limit, not a property of the
                                   method: a row's maximum logit has magnitude
                                   above 2^20, where the float32 softmax is
                                   not guaranteed to 1e-5; the row is refused
                                   like a bad one (the tree is the root alone)
                                   and BASTION_Q_BAD_LOGITS takes precedence */

/* logits storage types */
#define BASTION_F32 0
#define BASTION_BF16 1

int32_t bastion_abi_version(void);
const char *bastion_status_string(int32_t status);

/*
 * Workspace.  bastion_build_trees and bastion_mixture_score need a caller
 * allocated device workspace of at least bastion_workspace_bytes(...) bytes
 * (K = 1 for bastion_build_trees).  Its first bytes hold arrival counters
 * that must be zero before the first call: bastion_workspace_init() clears
 * them (enqueued on `stream`), and every completed call leaves them zero
 * again, so a workspace is initialised once and reused.  Calls that use the
 * same workspace must not overlap in time (use one stream per workspace).
 */
size_t bastion_workspace_bytes(int32_t B, int32_t K, int32_t b, int32_t V,
                               int32_t k, int32_t nmax, int32_t dtype);
int32_t bastion_workspace_init(void *ws, size_t ws_bytes, void *stream);

/* Outputs of a tree build.  Array shapes use W1 = nmax + 1 and
 * W = ceil((nmax + 1) / 32). */
typedef struct bastion_tree_out {
    int32_t *topk_ids;     /* [B, b, k]  candidate tokens of each position   */
    float *topk_q;         /* [B, b, k]  their softmax probability q          */
    float *row_max;        /* [B, b]     max logit of the row                 */
    float *row_sum;        /* [B, b]     sum_v exp(l_v - row_max)             */
    int32_t *parent;       /* [B, W1]    pop-order tree; -1 padding           */
    int32_t *depth;        /* [B, W1]    -1 padding                           */
    int32_t *token;        /* [B, W1]    -1 padding                           */
    float *rho;            /* [B, W1]    path score; 0 padding                */
    double *ahat;          /* [B, W1]    A_hat(T_n) for n <= n_nodes; 0 after */
    int32_t *n_nodes;      /* [B]        N of the emitted tree                */
    int32_t *qstatus;      /* [B]        BASTION_Q_*                          */
    uint32_t *mask;        /* [B, W1, W] ancestor bit rows, or NULL (below)   */
    int32_t *position_ids; /* [B, W1]    pos_base + depth, or NULL            */
} bastion_tree_out;

/*
 * bastion_build_trees -- [BASTION] Methodology 1-3 in one launch.
 *
 * logits: row r = q*b + p (query q, position p) starts at element
 *   r * row_stride of a dense array of `dtype` (BASTION_F32 or BASTION_BF16);
 *   row_stride >= V; the pointer must be aligned to the element size.  Any V
 *   and stride work; rows that start on a 16-byte boundary stream fastest.
 * For every row: the full-vocabulary softmax at temperature 1
 *   (row_max, row_sum) and its k most likely tokens with their q.
 * For every query: best-first expansion of the prefix tree whose depth-d
 *   nodes have the k candidates of position d+1 as children, scoring nodes
 *   by rho and recording A_hat after every addition.
 * Budget: cost == NULL gives a fixed budget N = nmax (fewer if the candidate
 *   tree is smaller: BASTION_Q_EXHAUSTED).  Otherwise cost points to the
 *   verify-latency table C(n), n = 0..nmax, of query q at
 *   cost + q * cost_qstride (stride 0 shares one table), and the tree stops
 *   at N* = the first n >= nmin with S(n+1) < S(n), where
 *   S(n) = A_hat(T_n) * l_ar / C(n); if S never decreases, N* is the
 *   largest size reachable within nmax.  C(n) must be > 0.
 * Tree outputs: see bastion_tree_out.  If out->mask is not NULL the call
 *   also emits the verifier mask and position ids exactly as
 *   bastion_tree_mask would (pos_base may be NULL for 0); out->position_ids
 *   must then be non-NULL too.
 * A query with a bad row (BASTION_Q_BAD_LOGITS) gets the root alone:
 *   n_nodes = 0, entry 0 the root, padding after it.
 * Errors: EINVAL for null required pointers, sizes outside the limits,
 *   row_stride < V, a logits pointer not aligned to its element, nmin > nmax,
 *   or (with cost) cost_qstride < 0 or l_ar not a positive finite number;
 *   EWORKSPACE when ws is NULL, not 16-byte aligned, or ws_bytes is too
 *   small.
 */
int32_t bastion_build_trees(const void *logits, int32_t dtype, int32_t B, int32_t b,
                            int32_t V, int64_t row_stride, int32_t k, int32_t nmax,
                            int32_t nmin, const double *cost, int64_t cost_qstride,
                            double l_ar, const int32_t *pos_base,
                            const bastion_tree_out *out, void *ws, size_t ws_bytes,
                            void *stream);

/*
 * bastion_build_trees_noalloc -- bastion_build_trees for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc.  Same arguments and outputs
 * without the workspace: the call's scratch is a 4 MiB device array inside
 * the library, one copy per GPU, held until the process ends.  The call
 * allocates nothing; it clears the array's arrival counters with a kernel
 * on `stream` before its own launch.  Every call on a GPU shares that GPU's
 * array, so calls that overlap in time on one GPU (other streams, other
 * host threads) race and must be serialised by the caller.
 * Errors: as bastion_build_trees, plus EUNSUPPORTED when the call's launch
 * plan needs more than bastion_noalloc_scratch_bytes() of scratch (it needs
 * 256 KiB + 4 bytes per row, plus per-segment records when rows are split,
 * about 0.5 MiB at B = 256, b = 16); EHIP if the array's device address
 * cannot be obtained.
 */
int32_t bastion_build_trees_noalloc(const void *logits, int32_t dtype, int32_t B, int32_t b,
                                    int32_t V, int64_t row_stride, int32_t k, int32_t nmax,
                                    int32_t nmin, const double *cost, int64_t cost_qstride,
                                    double l_ar, const int32_t *pos_base,
                                    const bastion_tree_out *out, void *stream);
size_t bastion_noalloc_scratch_bytes(void);

/*
 * bastion_budget_select -- [BASTION] Methodology 3 on a recorded A_hat curve.
 * ahat [B, nmax+1] (entries 0..n_avail[q] valid, e.g. from a fixed-budget
 * build); cost as in bastion_build_trees.  nstar[q] = the first
 * n in [nmin, n_avail[q]-1] with S(n+1) < S(n), else n_avail[q].
 * s_curve [B, nmax+1] (may be NULL) receives S(n) for n <= n_avail[q] and 0
 * after.  Errors: EINVAL for null required pointers, B < 1, nmax outside
 * the limits, nmin < 0 or nmin > nmax.  n_avail[q] is clamped to [0, nmax].
 */
int32_t bastion_budget_select(const double *ahat, const int32_t *n_avail, int32_t B,
                              int32_t nmax, int32_t nmin, const double *cost,
                              int64_t cost_qstride, double l_ar, int32_t *nstar,
                              double *s_curve, void *stream);

/*
 * bastion_tree_mask -- verifier inputs for [BASTION] tree-structured
 * verification (Experimental results); the pages fix no format.
 * For query q and node i <= n_nodes[q]: row i of mask (W = ceil((nmax+1)/32)
 * uint32 words, bit j of word j/32 at position j%32) has bit j set iff j == i
 * or j is an ancestor of i (the root included); position_ids[q, i] =
 * pos_base[q] (0 if pos_base is NULL) + depth(i), depth counted along parent
 * links.  Rows after n_nodes[q] are zero with position id -1.  A parent link
 * that is not 0 <= parent[i] < i ends the walk (the bits found so far stay).
 * Errors: EINVAL for null required pointers, B < 1, nmax outside the limits.
 */
int32_t bastion_tree_mask(const int32_t *parent, const int32_t *n_nodes, int32_t B,
                          int32_t nmax, const int32_t *pos_base, uint32_t *mask,
                          int32_t *position_ids, void *stream);

/*
 * bastion_accept -- [BASTION] greedy (temperature 0) acceptance.
 * target [B, nmax+1]: the target model's argmax token after each node's
 * path.  From the root, while a child c of the current node (parent[c] ==
 * current, current < c <= n_nodes[q]) has token[c] == target[current], move
 * to the lowest such c; at most b moves.  accept_len[q] = number of moves,
 * accept_nodes[q, 0..b] the visited nodes (root first, -1 after),
 * bonus[q] = target at the last visited node (the token the target commits
 * after the accepted drafts).
 * Errors: EINVAL for null pointers, B < 1, b or nmax outside the limits.
 */
int32_t bastion_accept(const int32_t *parent, const int32_t *token, const int32_t *n_nodes,
                       int32_t B, int32_t b, int32_t nmax, const int32_t *target,
                       int32_t *accept_len, int32_t *accept_nodes, int32_t *bonus,
                       void *stream);

/*
 * bastion_set_tuning -- launch-plan overrides for tuning and tests, not
 * part of the method: segments > 0 splits every row over that many blocks,
 * split_trees 0 / 1 forces the trees into the streaming launch / a launch
 * of their own; 0 and -1 restore the library's own plan.  Process-wide; the
 * environment variables BASTION_SEGMENTS and BASTION_SPLIT_TREES set the
 * initial values when the library loads.  Outputs do not depend on it.
 */
void bastion_set_tuning(int32_t segments, int32_t split_trees);

/*
 * Outputs of the latent-mixture call.  C = K * k candidate slots per
 * position.
 */
typedef struct bastion_mixture_out {
    float *prior_q;         /* [B, K]       q(z|y) = softmax of the prior logits   */
    int32_t *chain_tokens;  /* [B, K, b]    greedy chain of branch z (top-1 ids)   */
    double *qdep_chain;     /* [B, K]       q_dep of chain z                       */
    int32_t *cand_count;    /* [B, b]       |union over z of the branch top-k|     */
    int32_t *cand_tokens;   /* [B, b, C]    that union, ascending; -1 padding      */
    float *cand_q;          /* [B, b, C, K] q_i(token | z); 0 padding              */
    float *row_max;         /* [B, K, b]    per-branch row statistics              */
    float *row_sum;         /* [B, K, b]                                            */
} bastion_mixture_out;

/*
 * bastion_mixture_score -- [DBLAST] Methodology 1.
 * branch_logits: row ((q*K + z)*b + i) at element row * row_stride, as in
 *   bastion_build_trees; prior_logits [B, K] float32.
 * prior_q = softmax(prior logits).  Chain z is the greedy decode of branch z
 *   (the top-1 token of every position); its score is
 *   q_dep = sum_z' q(z'|y) prod_i q_i(x_i | y, z'), float64.
 * Tree (optional, when tree != NULL): best-first over the prefix tree whose
 *   depth-d nodes have the candidate union of position d+1 as children; a
 *   node keeps r_z = fl32 product of q_i(x_i|z) along its path (root 1) and
 *   scores rho = the float32 fma chain acc = fma(prior_q[z], r_z, acc),
 *   z = 0..K-1 from acc = 0, i.e. its q_dep with later positions
 *   marginalised out.  Fixed budget nmax; only parent, depth, token, rho,
 *   ahat, n_nodes, qstatus (and mask / position_ids when non-NULL) of
 *   `tree` are used.  The candidate slots (cand_*) are always written.
 * Errors: as bastion_build_trees, plus K outside [1, 16].
 */
int32_t bastion_mixture_score(const void *branch_logits, int32_t dtype,
                              const float *prior_logits, int32_t B, int32_t K, int32_t b,
                              int32_t V, int64_t row_stride, int32_t k, int32_t nmax,
                              const bastion_mixture_out *mix, const bastion_tree_out *tree,
                              void *ws, size_t ws_bytes, void *stream);

/* Outputs of the mixture-marginal call. */
typedef struct bastion_marginal_out {
    float *prior_q;        /* [B, K]        q(z|y) = softmax of the prior logits  */
    float *row_max;        /* [B, K, b]     per-branch row statistics             */
    float *row_sum;        /* [B, K, b]                                           */
    int32_t *marg_ids;     /* [B, b, k]     tokens ranked by the marginal         */
    float *marg_q;         /* [B, b, k]     their marginal sum_z q(z|y) q_i(x|z)  */
    float *cand_q;         /* [B, b, k, K]  q_i(token | z) of every branch        */
} bastion_marginal_out;

/*
 * bastion_mixture_marginal -- [DBLAST] Methodology 1: the latent mixture
 * mixes its branches with weights q(z|y), so position i's marginal is
 * m_i(x) = sum_z q(z|y) q_i(x|y,z).  Candidates of position i: the k tokens
 * ranked first by (m_i desc, token asc), with m_i and every branch's
 * q_i(x|z) (an alternative to bastion_mixture_score's union of the branches'
 * top-k).  m is formed in float32 as sum_z (q(z|y) / S_z) 2^(l log2 e - c_z)
 * from each branch row's max and sum (a first streaming pass), so two
 * tokens whose marginals agree to float32 rounding may rank either way.
 * Tree (when tree != NULL): best-first over these candidates with the
 * mixture score of bastion_mixture_score.  Three launches: the branch rows'
 * statistics, the marginal pass (one block per query and position, reading
 * the K rows of its position once more), the tree stage.
 * Arguments, workspace and errors as bastion_mixture_score.
 */
int32_t bastion_mixture_marginal(const void *branch_logits, int32_t dtype,
                                 const float *prior_logits, int32_t B, int32_t K, int32_t b,
                                 int32_t V, int64_t row_stride, int32_t k, int32_t nmax,
                                 const bastion_marginal_out *marg, const bastion_tree_out *tree,
                                 void *ws, size_t ws_bytes, void *stream);

/*
 * bastion_sample_nodes -- sampled (non-greedy) verification: one draw per
 * tree node from the target's distribution at temperature T.  [BASTION]
 * Experimental results evaluate greedy decoding; [DBLAST] Problem statement
 * and Experimental results evaluate targets at temperatures 0.7-1.5.  The
 * pages give no acceptance rule for sampled tree verification; this is the
 * target-sampling walk (SpecInfer's naive sampling, Miao et al. 2024):
 * bastion_accept with these draws as `target` moves from the root to the
 * child whose token equals the current node's draw until none does, and
 * commits that draw as the bonus -- lossless for any fixed tree.
 * logits [B, nmax+1, V] (row (q, i) at element (q*(nmax+1) + i)*row_stride):
 *   the target's logits after node i's path, finite or -inf.
 * sampled [B, nmax+1]: for i <= n_nodes[q] the draw
 *   x = argmax_v (l_v / T + g_v) (ties: smaller token), g_v = -log(-log(u_v)),
 *   computed in float32; T = 0 draws the argmax of l.  Entries after
 *   n_nodes[q] are -1.  The uniforms are counter-based (MurmurHash3's 32-bit
 *   finalizer fmix32): with a = fmix32(seed + 0x9E3779B9 (q+1)),
 *   c = fmix32(a ^ 0x85EBCA6B (i+1)), h = fmix32(c ^ v) (mod 2^32),
 *   u_v = ((h >> 8) + 1/2) / 2^24; the same seed gives the same draws.
 * Errors: EINVAL for null pointers, sizes outside the limits (0 <= nmax <=
 *   1023, V <= 524288), row_stride < V, a misaligned pointer, T < 0 or not
 *   finite.
 */
int32_t bastion_sample_nodes(const void *logits, int32_t dtype, int32_t B, int32_t nmax, int32_t V,
                             int64_t row_stride, const int32_t *n_nodes, float temperature,
                             uint32_t seed, int32_t *sampled, void *stream);

/*
 * bastion_mixture_sample -- [DBLAST] Methodology 1, inference: the latent
 * category is drawn with a temperature Z_T and its branch decoded greedily.
 * z[q] = the smallest index with u[q] < sum_{z' <= z} w_z',
 * w = softmax(prior_logits[q] / Z_T) in float64 (Z_T = 0: the argmax, ties
 * to the smaller index); draft[q, :] = chain_tokens[q, z, :] (the greedy
 * chains of bastion_mixture_score).  u [B] float64 in [0, 1), supplied by
 * the caller.  Errors: EINVAL for null pointers, K or b outside the limits,
 * Z_T < 0 or not finite.
 */
int32_t bastion_mixture_sample(const float *prior_logits, int32_t B, int32_t K, double temperature,
                               const double *u, const int32_t *chain_tokens, int32_t b,
                               int32_t *z_out, int32_t *draft, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* BASTION_H */
