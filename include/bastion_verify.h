/*
 * bastion_verify.h -- C ABI of the tree's consumer on gfx950: one attention
 * layer of a tree-structured verifier.
 *
 * Source: "Bastion: Budget-Aware Speculative Decoding with Tree-structured
 * Block Diffusion Drafting", gist.science (Dutch and French pages):
 *   Experimental results -- the target verifies the drafted tree in one
 *     forward pass (tree-structured verification);
 *   Methodology 3 -- the verify latency T_verify(N) of that pass enters the
 *     budget controller through a roofline model calibrated on observed
 *     runtimes.
 * The pages fix no attention formulation.  This one is the common one for
 * the pages' target models (Qwen3, Llama-3.1): grouped-query attention
 * (Hq query heads share Hkv key/value heads), rotary position embedding
 * (rotate-half pairs (d, d + D/2)), softmax scaled by 1/sqrt(D).
 *
 * Conventions as in bastion.h: device pointers owned by the caller, work
 * enqueued on `stream`, synchronous status (nothing launched on an error).
 */
#ifndef BASTION_VERIFY_H
#define BASTION_VERIFY_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Workspace bytes of bastion_tree_attention for these sizes (0 if invalid). */
size_t bastion_tree_attention_workspace_bytes(int32_t S, int32_t T, int32_t Hq, int32_t Hkv,
                                              int32_t Lmax);

/*
 * bastion_tree_attention -- S sequences, each verifying a tree of T = N + 1
 * tokens (node 0 the root, the last committed token) behind ctx_len[s]
 * cached tokens.
 *
 * qkv: bf16 rows of the q/k/v projection, row s*T + t for tree token t of
 *   sequence s, qkv_row_stride elements apart (>= (Hq + 2 Hkv) D, a multiple
 *   of 8); q head h at columns [h D, (h+1) D), k head h at
 *   [(Hq + h) D, ...), v head h at [(Hq + Hkv + h) D, ...).
 * k_cache: bf16 [S][Hkv][Lmax][D]; v_cache: bf16 [S][Hkv][Lmax/32][D][32]
 *   (tiles of 32 slots, a dim's 32 slots contiguous: value dim d of slot j
 *   at [s][h][j/32][d][j%32]).  Slots
 *   0 .. ctx-1 hold the cached tokens (k already rotated at its position);
 *   the call writes the tree tokens' rotated k and their v into slots
 *   ctx .. ctx+T-1, where ctx = ctx_len[s] clamped to [0, cap] with
 *   cap = max_ctx if 0 <= max_ctx < Lmax - T, else Lmax - T.  max_ctx is the
 *   caller's host-side bound of the contexts: it sizes the launch (chunks of
 *   keys up to cap + T), so a tight bound saves blocks.
 * position_ids [S][T] int32 (bastion_build_trees' pos_base + depth with
 *   pos_base = ctx): each tree token's q and k are rotated at its position:
 *   the pair (x_d, x_{d+D/2}), d < D/2, by the float32 angle
 *   fl(pos * inv_freq[d]) to (x_d cos - x_{d+D/2} sin,
 *   x_{d+D/2} cos + x_d sin), computed in float32 and rounded to bf16.
 * mask [S][T][W] uint32, W = ceil(T/32): bastion_build_trees' ancestor
 *   mask; tree token i attends to every cached token and to tree token j
 *   iff bit j of its row is set.
 * out: bf16 [S*T][Hq*D], token-major like qkv: the attention output of
 *   q head h = kv_head * (Hq/Hkv) + g.  Scores and softmax in float32; the
 *   probabilities enter the value product rounded to bf16.
 * Limits: D = 128, Hq % Hkv == 0, 1 <= T <= 1024, S * Hq * T < 2^31,
 *   T <= Lmax <= 16384, Lmax % 32 == 0; qkv, caches and out 16-byte aligned; ws
 *   256-byte aligned with at least bastion_tree_attention_workspace_bytes.
 * Errors: EINVAL (pointers, sizes, strides, alignment), EUNSUPPORTED (D,
 *   S * Hq * T, or Lmax above 16384), EWORKSPACE.
 * The workspace holds the rotated q rows and, for sequences whose keys span
 *   more than one chunk, the chunks' partial outputs; the chunk length
 *   follows from (S, Hkv, cap + T) so that the launch has about 1024 blocks
 *   (at least 128 keys per chunk; BASTION_ATTN_BLOCKS, read once, changes
 *   that target).
 */
int32_t bastion_tree_attention(const void *qkv, int64_t qkv_row_stride, int32_t S, int32_t T,
                               int32_t Hq, int32_t Hkv, int32_t D, void *k_cache, void *v_cache,
                               int32_t Lmax, const int32_t *ctx_len, int32_t max_ctx,
                               const int32_t *position_ids, const uint32_t *mask, int32_t W,
                               const float *inv_freq, void *out, void *ws, size_t ws_bytes,
                               void *stream);

#ifdef __cplusplus
}
#endif

#endif /* BASTION_VERIFY_H */
