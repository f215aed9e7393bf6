// build_params.hpp -- kernel arguments of the fused build kernel, shared by
// the kernel (build_trees.hip) and the entry points (api.hip).
#pragma once

#include <stdint.h>

namespace bastion {

struct BuildParams {
    const char *logits;
    int64_t row_stride_bytes;
    int B, b, V, k, nmax, nmin, S;
    const double *cost;
    int64_t cost_qstride;
    double l_ar;
    const int32_t *pos_base;
    int32_t *topk_ids;
    float *topk_q, *row_max, *row_sum;
    int32_t *parent, *depth, *token;
    float *rho;
    double *ahat;
    int32_t *n_nodes, *qstatus;
    uint32_t *mask;
    int32_t *position_ids;
    uint32_t *row_ticket, *query_ticket;
    int32_t *row_status;
    char *partials;       // [rows, S] records of kPartialBytes(k)
    int partial_bytes;
    // latent mixture (mode 1): rows are ((q*K + z)*b + i)
    int mode;             // 0: trees over [B, b, V]; 1: mixture over [B, K, b, V]
    int K;
    int rows_per_query;   // b, or K * b
    int is_bf16;
    float *row_ms;        // [rows, 2] row max and internal sum, or NULL
    const float *prior;   // [B, K]
    float *prior_q;       // [B, K]
    int32_t *chain_tokens;
    double *qdep;
    int32_t *cand_count, *cand_tokens;
    float *cand_q;
    int mix_tree;         // 1: build the mixture tree into parent/depth/...
    int mix_marginal;     // 1: candidates from the mixture marginal (marg_*)
    int32_t *marg_ids;    // [B, b, k] tokens ranked by the mixture marginal
    float *marg_q;        // [B, b, k] their marginal sum_z w_z q_i(x|z)
    float *marg_cq;       // [B, b, k, K] q_i(x|z) of every branch
    int split_trees;      // 1: the trees run in a launch of their own (mode 0)
    int resident_blocks;  // stream blocks the machine holds at once
    uint64_t *stamps;     // stamped build only: per-block timestamps of the
                          // stream launch, then of the second launch's blocks
    int64_t stamp_second; // slot-block index where the second launch's start
};

}  // namespace bastion
