// tree_ops.hip -- small per-query gfx950 kernels on finished trees:
//   budget_select (Bastion, Methodology 3, on a recorded A_hat curve),
//   tree_mask     (ancestor bit rows and position ids for the verifier),
//   accept        (greedy acceptance against the target's argmax tokens).
// One block per query; all of them are far from any bandwidth limit.
#include "device_common.hpp"

namespace bastion {

// One thread per query walks its S(n) curve in order.
__global__ void budget_select_kernel(const double *ahat, const int32_t *n_avail, int B, int nmax,
                                     int nmin, const double *cost, int64_t cost_qstride,
                                     double l_ar, int32_t *nstar, double *s_curve) {
    const int q = blockIdx.x * blockDim.x + threadIdx.x;
    if (q >= B) return;
    int count = n_avail[q];
    count = count < 0 ? 0 : (count > nmax ? nmax : count);
    const double *a = ahat + int64_t(q) * (nmax + 1);
    const double *c = cost + int64_t(q) * cost_qstride;
    double *sc = s_curve ? s_curve + int64_t(q) * (nmax + 1) : nullptr;
    int found = count;
    double prev = (a[0] * l_ar) / c[0];
    if (sc) sc[0] = prev;
    for (int n = 1; n <= nmax; ++n) {
        if (n > count) {
            if (sc) sc[n] = 0.0;
            continue;
        }
        const double s = (a[n] * l_ar) / c[n];
        if (sc) sc[n] = s;
        if (found == count && n - 1 >= nmin && s < prev) found = n - 1;
        prev = s;
    }
    nstar[q] = found;
}

// Block per query: parents staged in LDS, then every (row, word) pair walks
// its ancestors.
__global__ void tree_mask_kernel(const int32_t *parent, const int32_t *n_nodes, int nmax,
                                 const int32_t *pos_base, uint32_t *mask, int32_t *position_ids) {
    extern __shared__ int32_t par[];
    const int q = blockIdx.x;
    const int W1 = nmax + 1, W = (W1 + 31) / 32;
    const int64_t o = int64_t(q) * W1;
    for (int i = threadIdx.x; i < W1; i += blockDim.x) par[i] = parent[o + i];
    __syncthreads();
    int n = n_nodes[q];
    n = n < -1 ? -1 : (n > nmax ? nmax : n);
    const int32_t pb = pos_base ? pos_base[q] : 0;
    for (int e = threadIdx.x; e < W1 * W; e += blockDim.x) {
        const int i = e / W, w = e - i * W;
        uint32_t bits = 0;
        int steps = 0;
        if (i <= n) {
            int j = i;
            if (j / 32 == w) bits |= 1u << (j & 31);
            while (j > 0) {
                const int p = par[j];
                if (p < 0 || p >= j) break;
                if (p / 32 == w) bits |= 1u << (p & 31);
                j = p;
                ++steps;
            }
        }
        mask[(o + i) * W + w] = bits;
        if (w == 0) position_ids[o + i] = i <= n ? pb + steps : -1;
    }
}

// One wave per query; candidate children of the current node are searched
// 64 at a time, the lowest matching index wins.
__global__ void accept_kernel(const int32_t *parent, const int32_t *token, const int32_t *n_nodes,
                              int b, int nmax, const int32_t *target, int32_t *accept_len,
                              int32_t *accept_nodes, int32_t *bonus) {
    extern __shared__ int32_t sh[];
    int32_t *par = sh;
    int32_t *tok = sh + (nmax + 1);
    const int q = blockIdx.x, lane = threadIdx.x;
    const int W1 = nmax + 1;
    const int64_t o = int64_t(q) * W1;
    for (int i = lane; i < W1; i += kWave) {
        par[i] = parent[o + i];
        tok[i] = token[o + i];
    }
    int n = n_nodes[q];
    n = n > nmax ? nmax : n;
    wave_sync();
    int cur = 0, len = 0;
    int mine = lane == 0 ? 0 : -1;   // lane m holds path[m]
    while (len < b) {
        const int t = target[o + cur];
        int found = -1;
        for (int c0 = cur + 1; c0 <= n && found < 0; c0 += kWave) {
            const int c = c0 + lane;
            const bool hit = c <= n && par[c] == cur && tok[c] == t;
            const uint64_t m = __ballot(hit);
            if (m) found = c0 + __ffsll((unsigned long long)m) - 1;
        }
        if (found < 0) break;
        cur = found;
        ++len;
        if (lane == len) mine = cur;
    }
    if (lane <= b) accept_nodes[int64_t(q) * (b + 1) + lane] = mine;
    if (lane == 0) {
        accept_len[q] = len;
        bonus[q] = target[o + cur];
    }
}

__global__ void fill_u32_kernel(uint32_t *p, size_t n, uint32_t v) {
    for (size_t i = size_t(blockIdx.x) * blockDim.x + threadIdx.x; i < n;
         i += size_t(gridDim.x) * blockDim.x)
        p[i] = v;
}

}  // namespace bastion

hipError_t bastion_launch_fill_u32(uint32_t *p, size_t n, uint32_t v, hipStream_t s) {
    hipLaunchKernelGGL(bastion::fill_u32_kernel, dim3(64), dim3(256), 0, s, p, n, v);
    return hipGetLastError();
}

hipError_t bastion_launch_budget_select(const double *ahat, const int32_t *n_avail, int B, int nmax,
                                        int nmin, const double *cost, int64_t cost_qstride,
                                        double l_ar, int32_t *nstar, double *s_curve,
                                        hipStream_t s) {
    const int threads = 64;
    hipLaunchKernelGGL(bastion::budget_select_kernel, dim3((B + threads - 1) / threads),
                       dim3(threads), 0, s, ahat, n_avail, B, nmax, nmin, cost, cost_qstride,
                       l_ar, nstar, s_curve);
    return hipGetLastError();
}

hipError_t bastion_launch_tree_mask(const int32_t *parent, const int32_t *n_nodes, int B,
                                    int nmax, const int32_t *pos_base, uint32_t *mask,
                                    int32_t *position_ids, hipStream_t s) {
    hipLaunchKernelGGL(bastion::tree_mask_kernel, dim3(B), dim3(256), (nmax + 1) * 4, s, parent,
                       n_nodes, nmax, pos_base, mask, position_ids);
    return hipGetLastError();
}

hipError_t bastion_launch_accept(const int32_t *parent, const int32_t *token,
                                 const int32_t *n_nodes, int B, int b, int nmax,
                                 const int32_t *target, int32_t *accept_len,
                                 int32_t *accept_nodes, int32_t *bonus, hipStream_t s) {
    hipLaunchKernelGGL(bastion::accept_kernel, dim3(B), dim3(64), 2 * (nmax + 1) * 4, s, parent,
                       token, n_nodes, b, nmax, target, accept_len, accept_nodes, bonus);
    return hipGetLastError();
}
