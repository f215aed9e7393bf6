// api.hip -- the extern "C" entry points of libbastion.so: argument
// validation, workspace layout, launch planning and launches.  No call
// allocates memory; every check happens before the first HIP call, so an
// EINVAL / EUNSUPPORTED / EWORKSPACE return means nothing was enqueued.
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#include <atomic>

#include "device_common.hpp"

#include "api_internal.hpp"
#include "build_params.hpp"
#include "mixture.hpp"

// launchers, defined next to their kernels

hipError_t bastion_launch_build(const bastion::BuildParams &P, int dtype, hipStream_t s,
                                int *smem_out);
hipError_t bastion_launch_budget_select(const double *ahat, const int32_t *n_avail, int B, int nmax,
                                        int nmin, const double *cost, int64_t cost_qstride,
                                        double l_ar, int32_t *nstar, double *s_curve,
                                        hipStream_t s);
hipError_t bastion_launch_tree_mask(const int32_t *parent, const int32_t *n_nodes, int B,
                                    int nmax, const int32_t *pos_base, uint32_t *mask,
                                    int32_t *position_ids, hipStream_t s);
hipError_t bastion_launch_accept(const int32_t *parent, const int32_t *token,
                                 const int32_t *n_nodes, int B, int b, int nmax,
                                 const int32_t *target, int32_t *accept_len,
                                 int32_t *accept_nodes, int32_t *bonus, hipStream_t s);
hipError_t bastion_launch_fill_u32(uint32_t *p, size_t n, uint32_t v, hipStream_t s);

namespace {

using namespace bastion;

// Workspace layout.  The arrival counters sit at fixed offsets at the head
// so that a workspace can be reused across shapes.
constexpr size_t kTicketWords = 65536;
constexpr size_t kRowTicketWords = 49152;            // per-row counters
constexpr size_t kQueryTicketBase = kRowTicketWords;  // per-query counters
constexpr size_t kTicketBytes = kTicketWords * 4;
constexpr int kMaxSegments = 64;
constexpr int kBlocksPerCu = 4;   // stream blocks of 256 threads resident per CU
constexpr int kMaxDevices = 64;

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

int esize(int dtype) { return dtype == BASTION_BF16 ? 2 : 4; }

// Compute units of the current device, read once per device.
std::atomic<int> g_cus[kMaxDevices];

int device_cus() {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return 256;
    int v = g_cus[dev].load(std::memory_order_relaxed);
    if (v <= 0) {
        if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
            v <= 0)
            v = 256;
        g_cus[dev].store(v, std::memory_order_relaxed);
    }
    return v;
}

// Launch-plan overrides for tuning and tests (bastion_set_tuning), first
// taken from BASTION_SEGMENTS / BASTION_SPLIT_TREES when the library loads.
std::atomic<int> g_force_segments{0};     // > 0: segments per row
std::atomic<int> g_force_split{-1};       // 0 / 1: trees in the stream launch / their own

struct TuningFromEnv {
    TuningFromEnv() {
        const char *e = getenv("BASTION_SEGMENTS");
        if (e && atoi(e) > 0) g_force_segments.store(atoi(e));
        e = getenv("BASTION_SPLIT_TREES");
        if (e) g_force_split.store(atoi(e) != 0 ? 1 : 0);
    }
} g_tuning_from_env;

#ifdef BASTION_STAMPS
// stamped build: the timestamp buffer of the following calls (device)
uint64_t *g_stamps = nullptr;
#endif

// timestamps of a call whose stream launch has `grid` blocks
void set_stamps(BuildParams &P, int64_t grid) {
#ifdef BASTION_STAMPS
    P.stamps = g_stamps;
    P.stamp_second = grid;
#else
    (void)P;
    (void)grid;
#endif
}

struct Layout {
    size_t row_status, partials, row_ms, mtopk_ids, mtopk_q, total;
    int S;
};

// Segments per row.  Enough blocks to cover the machine: kBlocksPerCu
// resident blocks on each CU, or one per CU when the whole input is small
// (at most 16 MiB), where every block's fixed latency (start, merge,
// hand-off) outweighs its streaming.  No segment shorter than 16 KiB (four
// 16-byte loads per thread).
int plan_segments(int64_t rows, int V, int dtype) {
    const int64_t row_bytes = int64_t(V) * esize(dtype);
    const int64_t cus = device_cus();
    const int64_t target = rows * row_bytes <= (int64_t(16) << 20) ? cus : kBlocksPerCu * cus;
    int S = int((target + rows - 1) / rows);
    const int forced = g_force_segments.load(std::memory_order_relaxed);
    if (forced > 0) S = forced;
    const int64_t by_size = row_bytes / (forced > 0 ? 4096 : 16384);
    if (S > by_size) S = int(by_size);
    if (S > kMaxSegments) S = kMaxSegments;
    if (S < 1) S = 1;
    if (S > 1 && rows > int64_t(kRowTicketWords)) S = 1;
    return S;
}

// with_mixture: also the row statistics and branch top-k that the
// latent-mixture call keeps between its two launches
Layout layout(int64_t rows, int k, int S, bool with_mixture = true) {
    Layout L;
    L.S = S;
    L.row_status = kTicketBytes;
    L.partials = align256(L.row_status + size_t(rows) * 4);
    L.row_ms = align256(L.partials + (S > 1 ? size_t(rows) * S * size_t(16 + 8 * k) : 0));
    const size_t mix = with_mixture ? 1 : 0;
    L.mtopk_ids = align256(L.row_ms + mix * size_t(rows) * 8);
    L.mtopk_q = align256(L.mtopk_ids + mix * size_t(rows) * k * 4);
    L.total = align256(L.mtopk_q + mix * size_t(rows) * k * 4);
    return L;
}

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

int32_t to_status(hipError_t e) { return e == hipSuccess ? BASTION_OK : BASTION_EHIP; }

bool sizes_ok(int32_t B, int32_t b, int32_t V, int32_t k, int32_t nmax) {
    return B >= 1 && B <= 16384 && b >= 1 && b <= kMaxB && k >= 1 && k <= kMaxK && V >= k &&
           V <= kMaxV && nmax >= 1 && nmax <= kMaxNmax;
}

bool tree_out_ok(const bastion_tree_out *o, bool need_rows) {
    if (!o) return false;
    if (need_rows && (!o->topk_ids || !o->topk_q || !o->row_max || !o->row_sum)) return false;
    if (!o->parent || !o->depth || !o->token || !o->rho || !o->ahat || !o->n_nodes || !o->qstatus)
        return false;
    if (o->mask && !o->position_ids) return false;
    return true;
}

}  // namespace

extern "C" {

int32_t bastion_abi_version(void) { return BASTION_ABI_VERSION; }

const char *bastion_status_string(int32_t status) {
    switch (status) {
        case BASTION_OK: return "ok";
        case BASTION_EINVAL: return "invalid argument";
        case BASTION_EUNSUPPORTED: return "unsupported request";
        case BASTION_EHIP: return "HIP runtime error";
        case BASTION_EWORKSPACE: return "workspace missing or too small";
        default: return "unknown status";
    }
}

size_t bastion_workspace_bytes(int32_t B, int32_t K, int32_t b, int32_t V, int32_t k,
                               int32_t nmax, int32_t dtype) {
    (void)nmax;
    if (B < 1 || K < 1 || b < 1 || V < 1 || k < 1 || (dtype != BASTION_F32 && dtype != BASTION_BF16))
        return 0;
    const int64_t rows = int64_t(B) * K * b;
    return layout(rows, k, plan_segments(rows, V, dtype)).total;
}

int32_t bastion_workspace_init(void *ws, size_t ws_bytes, void *stream) {
    if (!ws || !aligned16(ws)) return BASTION_EINVAL;
    if (ws_bytes < kTicketBytes) return BASTION_EWORKSPACE;
    return to_status(bastion_launch_fill_u32(static_cast<uint32_t *>(ws), kTicketWords, 0u,
                                             static_cast<hipStream_t>(stream)));
}

}  // extern "C"

// bastion_build_trees on a given scratch area (api_internal.hpp).
int32_t bastion::build_trees_on(const void *logits, int32_t dtype, int32_t B, int32_t b,
                                int32_t V, int64_t row_stride, int32_t k, int32_t nmax,
                                int32_t nmin, const double *cost, int64_t cost_qstride,
                                double l_ar, const int32_t *pos_base,
                                const bastion_tree_out *out, void *ws, size_t ws_bytes,
                                void *stream, ScratchSource scratch) {
    if (!logits || (dtype != BASTION_F32 && dtype != BASTION_BF16)) return BASTION_EINVAL;
    if (!sizes_ok(B, b, V, k, nmax) || nmin < 0 || nmin > nmax) return BASTION_EINVAL;
    if (row_stride < V || (reinterpret_cast<uintptr_t>(logits) % esize(dtype)) != 0)
        return BASTION_EINVAL;
    if (!tree_out_ok(out, true)) return BASTION_EINVAL;
    if (cost && (cost_qstride < 0 || !(l_ar > 0.0) || l_ar > 1e300)) return BASTION_EINVAL;
    const int64_t rows = int64_t(B) * b;
    const int S = plan_segments(rows, V, dtype);
    // a library-owned scratch holds only what this call uses
    const Layout L = layout(rows, k, S, scratch == nullptr);
    if (scratch) {
        const int32_t st = scratch(L.total, &ws, &ws_bytes);
        if (st != BASTION_OK) return st;
    }
    if (!ws || !aligned16(ws) || ws_bytes < L.total) return BASTION_EWORKSPACE;

    BuildParams P;
    memset(&P, 0, sizeof P);
    char *w = static_cast<char *>(ws);
    P.logits = static_cast<const char *>(logits);
    P.row_stride_bytes = row_stride * esize(dtype);
    P.B = B; P.b = b; P.V = V; P.k = k; P.nmax = nmax; P.nmin = nmin; P.S = S;
    P.cost = cost; P.cost_qstride = cost_qstride; P.l_ar = l_ar; P.pos_base = pos_base;
    P.topk_ids = out->topk_ids; P.topk_q = out->topk_q; P.row_max = out->row_max;
    P.row_sum = out->row_sum; P.parent = out->parent; P.depth = out->depth;
    P.token = out->token; P.rho = out->rho; P.ahat = out->ahat; P.n_nodes = out->n_nodes;
    P.qstatus = out->qstatus; P.mask = out->mask; P.position_ids = out->position_ids;
    P.row_ticket = reinterpret_cast<uint32_t *>(w);
    P.query_ticket = reinterpret_cast<uint32_t *>(w) + kQueryTicketBase;
    P.row_status = reinterpret_cast<int32_t *>(w + L.row_status);
    P.partials = w + L.partials;
    P.partial_bytes = 16 + 8 * k;
    P.mode = 0;
    P.K = 1;
    P.rows_per_query = b;
    P.is_bf16 = dtype == BASTION_BF16;
    P.row_ms = nullptr;
    P.resident_blocks = kBlocksPerCu * device_cus();
    set_stamps(P, rows * S);
    // trees in a launch of their own (one block of 16 waves per query) when
    // the stream grid fills the machine more than once, where a tree would
    // hold a slot that later rows wait for; otherwise the whole call is one
    // kernel
    P.split_trees = rows * S > P.resident_blocks ? 1 : 0;
    const int forced = g_force_split.load(std::memory_order_relaxed);
    if (forced >= 0) P.split_trees = forced;
    const hipStream_t s = static_cast<hipStream_t>(stream);
    if (scratch) {
        // a library-owned scratch keeps the last call's contents: clear the
        // arrival counters first (with a kernel, so that a caller may
        // capture the call in a graph)
        const hipError_t e = bastion_launch_fill_u32(reinterpret_cast<uint32_t *>(w), kTicketWords,
                                                     0u, s);
        if (e != hipSuccess) return BASTION_EHIP;
    }
    return to_status(bastion_launch_build(P, dtype, s, nullptr));
}

extern "C" {

int32_t bastion_build_trees(const void *logits, int32_t dtype, int32_t B, int32_t b, int32_t V,
                            int64_t row_stride, int32_t k, int32_t nmax, int32_t nmin,
                            const double *cost, int64_t cost_qstride, double l_ar,
                            const int32_t *pos_base, const bastion_tree_out *out, void *ws,
                            size_t ws_bytes, void *stream) {
    return bastion::build_trees_on(logits, dtype, B, b, V, row_stride, k, nmax, nmin, cost,
                                   cost_qstride, l_ar, pos_base, out, ws, ws_bytes, stream,
                                   nullptr);
}

#ifdef BASTION_STAMPS
// Stamped build only: per-block timestamps of the following calls go to
// `buf` (device, kStampSlots words per block of the stream launch, then per
// block of the second launch), or nowhere when buf is NULL.
void bastion_debug_set_stamps(uint64_t *buf) { g_stamps = buf; }
#endif

void bastion_set_tuning(int32_t segments, int32_t split_trees) {
    g_force_segments.store(segments > 0 ? segments : 0);
    g_force_split.store(split_trees < 0 ? -1 : (split_trees != 0 ? 1 : 0));
}

int32_t bastion_budget_select(const double *ahat, const int32_t *n_avail, int32_t B, int32_t nmax,
                              int32_t nmin, const double *cost, int64_t cost_qstride, double l_ar,
                              int32_t *nstar, double *s_curve, void *stream) {
    if (!ahat || !n_avail || !cost || !nstar) return BASTION_EINVAL;
    if (B < 1 || nmax < 1 || nmax > kMaxNmax || nmin < 0 || nmin > nmax) return BASTION_EINVAL;
    if (cost_qstride < 0 || !(l_ar > 0.0) || l_ar > 1e300) return BASTION_EINVAL;
    return to_status(bastion_launch_budget_select(ahat, n_avail, B, nmax, nmin, cost, cost_qstride,
                                                  l_ar, nstar, s_curve,
                                                  static_cast<hipStream_t>(stream)));
}

int32_t bastion_tree_mask(const int32_t *parent, const int32_t *n_nodes, int32_t B, int32_t nmax,
                          const int32_t *pos_base, uint32_t *mask, int32_t *position_ids,
                          void *stream) {
    if (!parent || !n_nodes || !mask || !position_ids) return BASTION_EINVAL;
    if (B < 1 || nmax < 1 || nmax > kMaxNmax) return BASTION_EINVAL;
    return to_status(bastion_launch_tree_mask(parent, n_nodes, B, nmax, pos_base, mask,
                                              position_ids, static_cast<hipStream_t>(stream)));
}

int32_t bastion_accept(const int32_t *parent, const int32_t *token, const int32_t *n_nodes,
                       int32_t B, int32_t b, int32_t nmax, const int32_t *target,
                       int32_t *accept_len, int32_t *accept_nodes, int32_t *bonus, void *stream) {
    if (!parent || !token || !n_nodes || !target || !accept_len || !accept_nodes || !bonus)
        return BASTION_EINVAL;
    if (B < 1 || b < 1 || b > kMaxB || nmax < 1 || nmax > kMaxNmax) return BASTION_EINVAL;
    return to_status(bastion_launch_accept(parent, token, n_nodes, B, b, nmax, target, accept_len,
                                           accept_nodes, bonus, static_cast<hipStream_t>(stream)));
}

}  // extern "C"

namespace {

// bastion_mixture_score (mix) or bastion_mixture_marginal (marg), on the
// caller's workspace
int32_t mixture_call(const void *branch_logits, int32_t dtype, const float *prior_logits, int32_t B,
                     int32_t K, int32_t b, int32_t V, int64_t row_stride, int32_t k, int32_t nmax,
                     const bastion_mixture_out *mix, const bastion_marginal_out *marg,
                     const bastion_tree_out *tree, void *ws, size_t ws_bytes, void *stream) {
    if (!branch_logits || !prior_logits || (dtype != BASTION_F32 && dtype != BASTION_BF16))
        return BASTION_EINVAL;
    if (K < 1 || K > kMaxBranches || !sizes_ok(B, b, V, k, nmax)) return BASTION_EINVAL;
    if (row_stride < V || (reinterpret_cast<uintptr_t>(branch_logits) % esize(dtype)) != 0)
        return BASTION_EINVAL;
    if (mix && (!mix->prior_q || !mix->chain_tokens || !mix->qdep_chain || !mix->cand_count ||
                !mix->cand_tokens || !mix->cand_q || !mix->row_max || !mix->row_sum))
        return BASTION_EINVAL;
    if (marg && (!marg->prior_q || !marg->row_max || !marg->row_sum || !marg->marg_ids ||
                 !marg->marg_q || !marg->cand_q))
        return BASTION_EINVAL;
    if (!mix == !marg) return BASTION_EINVAL;
    if (tree && !tree_out_ok(tree, false)) return BASTION_EINVAL;
    // the query stage keeps every position's candidates and q tables and the
    // running list in the LDS of one CU
    if (mix_layout(K, b, k, nmax, marg ? k : 0).total > kMixMaxLds) return BASTION_EUNSUPPORTED;
    const int64_t rows = int64_t(B) * K * b;
    const int S = plan_segments(rows, V, dtype);
    const Layout L = layout(rows, k, S);
    if (!ws || !aligned16(ws) || ws_bytes < L.total) return BASTION_EWORKSPACE;

    BuildParams P;
    memset(&P, 0, sizeof P);
    char *w = static_cast<char *>(ws);
    P.logits = static_cast<const char *>(branch_logits);
    P.row_stride_bytes = row_stride * esize(dtype);
    P.B = B; P.b = b; P.V = V; P.k = k; P.nmax = nmax; P.nmin = 0; P.S = S;
    P.cost = nullptr; P.cost_qstride = 0; P.l_ar = 1.0; P.pos_base = nullptr;
    P.topk_ids = reinterpret_cast<int32_t *>(w + L.mtopk_ids);
    P.topk_q = reinterpret_cast<float *>(w + L.mtopk_q);
    P.row_max = mix ? mix->row_max : marg->row_max;
    P.row_sum = mix ? mix->row_sum : marg->row_sum;
    if (tree) {
        P.parent = tree->parent; P.depth = tree->depth; P.token = tree->token;
        P.rho = tree->rho; P.ahat = tree->ahat; P.n_nodes = tree->n_nodes;
        P.qstatus = tree->qstatus; P.mask = tree->mask; P.position_ids = tree->position_ids;
    }
    P.row_ticket = reinterpret_cast<uint32_t *>(w);
    P.query_ticket = reinterpret_cast<uint32_t *>(w) + kQueryTicketBase;
    P.row_status = reinterpret_cast<int32_t *>(w + L.row_status);
    P.partials = w + L.partials;
    P.partial_bytes = 16 + 8 * k;
    P.mode = 1;
    P.K = K;
    P.rows_per_query = K * b;
    P.is_bf16 = dtype == BASTION_BF16;
    P.row_ms = reinterpret_cast<float *>(w + L.row_ms);
    P.resident_blocks = kBlocksPerCu * device_cus();
    set_stamps(P, rows * S);
    P.prior = prior_logits;
    P.prior_q = mix ? mix->prior_q : marg->prior_q;
    if (mix) {
        P.chain_tokens = mix->chain_tokens;
        P.qdep = mix->qdep_chain;
        P.cand_count = mix->cand_count;
        P.cand_tokens = mix->cand_tokens;
        P.cand_q = mix->cand_q;
    } else {
        P.mix_marginal = 1;
        P.marg_ids = marg->marg_ids;
        P.marg_q = marg->marg_q;
        P.marg_cq = marg->cand_q;
    }
    P.mix_tree = tree ? 1 : 0;
    return to_status(bastion_launch_build(P, dtype, static_cast<hipStream_t>(stream), nullptr));
}


}  // namespace

extern "C" {

int32_t bastion_mixture_score(const void *branch_logits, int32_t dtype, const float *prior_logits,
                              int32_t B, int32_t K, int32_t b, int32_t V, int64_t row_stride,
                              int32_t k, int32_t nmax, const bastion_mixture_out *mix,
                              const bastion_tree_out *tree, void *ws, size_t ws_bytes,
                              void *stream) {
    if (!mix) return BASTION_EINVAL;
    return mixture_call(branch_logits, dtype, prior_logits, B, K, b, V, row_stride, k, nmax, mix,
                        nullptr, tree, ws, ws_bytes, stream);
}

int32_t bastion_mixture_marginal(const void *branch_logits, int32_t dtype,
                                 const float *prior_logits, int32_t B, int32_t K, int32_t b,
                                 int32_t V, int64_t row_stride, int32_t k, int32_t nmax,
                                 const bastion_marginal_out *marg, const bastion_tree_out *tree,
                                 void *ws, size_t ws_bytes, void *stream) {
    if (!marg) return BASTION_EINVAL;
    return mixture_call(branch_logits, dtype, prior_logits, B, K, b, V, row_stride, k, nmax,
                        nullptr, marg, tree, ws, ws_bytes, stream);
}

}  // extern "C"
