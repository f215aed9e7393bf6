// stochastic.hip -- the sampled (non-greedy) variants on gfx950.
//
//  * sample_nodes_kernel: one draw per tree node from the target's
//    distribution at temperature T, softmax(l / T) of the node's logits row
//    (the DBlast page evaluates targets at temperatures 0.7-1.5, Problem
//    statement and Experimental results), by the Gumbel-max rule
//    x = argmax_v (l_v / T + g_v), g_v = -log(-log(u_v)), one streaming pass
//    over the row with no normaliser.  The uniforms are counter-based: the
//    MurmurHash3 32-bit finalizer (fmix32, Austin Appleby) of a key built
//    from (seed, query, node, token), so any element's draw is reproducible
//    without storing noise.  With these draws as the targets, bastion_accept
//    performs the target-sampling walk: at the current node draw x from the
//    target; move to the child whose token is x, else stop and commit x --
//    lossless for any fixed tree (the committed tokens are distributed as
//    the target's own sampling).
//  * mixture_sample_kernel: the DBlast branch draw (Methodology 1: at
//    inference the latent category is drawn, with temperature Z_T, and its
//    branch decoded greedily): z from softmax(prior / Z_T) by inverse CDF
//    at a caller-supplied uniform, float64; the draft is branch z's chain.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "device_common.hpp"

namespace bastion {

namespace {

typedef uint32_t su32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 sbf16x8 __attribute__((ext_vector_type(8)));

__device__ __forceinline__ uint32_t fmix32(uint32_t h) {
    h ^= h >> 16;
    h *= 0x85EBCA6Bu;
    h ^= h >> 13;
    h *= 0xC2B2AE35u;
    h ^= h >> 16;
    return h;
}

// u in (0, 1) of element `token` of a row whose key is c
__device__ __forceinline__ float uniform_of(uint32_t c, uint32_t token) {
    const uint32_t h = fmix32(c ^ token);
    return (float(h >> 8) + 0.5f) * (1.0f / 16777216.0f);
}

// Draw key of one element: (score, smaller token first); T = 0 keeps l.
__device__ __forceinline__ uint64_t draw_key(float l, uint32_t c, uint32_t token, float inv_t,
                                             bool tempered) {
    float sc = l;
    if (tempered) {
        const float u = uniform_of(c, token);
        sc = __builtin_fmaf(l, inv_t, -__logf(-__logf(u)));
    }
    return topk_key(sc, token);
}

template <typename T> struct SElem;
template <> struct SElem<float> {
    static constexpr int kPer = 4;
    __device__ static float at(const char *row, int64_t i) {
        return reinterpret_cast<const float *>(row)[i];
    }
    __device__ static void decode(su32x4 r, float *f) {
#pragma unroll
        for (int j = 0; j < 4; ++j) f[j] = __uint_as_float(r[j]);
    }
};
template <> struct SElem<__bf16> {
    static constexpr int kPer = 8;
    __device__ static float at(const char *row, int64_t i) {
        return float(reinterpret_cast<const __bf16 *>(row)[i]);
    }
    __device__ static void decode(su32x4 r, float *f) {
        const sbf16x8 h = __builtin_bit_cast(sbf16x8, r);
#pragma unroll
        for (int j = 0; j < 8; ++j) f[j] = float(h[j]);
    }
};

constexpr int kSThreads = 256;

// Block per (query, node) row; rows after the query's n_nodes get -1.
template <typename T>
__global__ __launch_bounds__(kSThreads) void sample_nodes_kernel(
    const char *logits, int64_t row_stride_bytes, int nmax, int V, const int32_t *n_nodes,
    float inv_t, int tempered, uint32_t seed, int32_t *sampled) {
    constexpr int E = SElem<T>::kPer;
    const int64_t r = blockIdx.x;
    const int q = int(r / (nmax + 1)), node = int(r - int64_t(q) * (nmax + 1));
    if (node > n_nodes[q]) {
        if (threadIdx.x == 0) sampled[r] = -1;
        return;
    }
    const char *row = logits + r * row_stride_bytes;
    const uint32_t a = fmix32(seed + 0x9E3779B9u * uint32_t(q + 1));
    const uint32_t c = fmix32(a ^ (0x85EBCA6Bu * uint32_t(node + 1)));
    const bool tmp = tempered != 0;
    // elements before the first 16-byte boundary, aligned vectors, the rest
    int head = int(((16u - (uint32_t(reinterpret_cast<uintptr_t>(row)) & 15u)) & 15u) /
                   sizeof(T));
    head = head > V ? V : head;
    const int nvec = (V - head) / E;
    uint64_t best = 0;
    const su32x4 *vr = reinterpret_cast<const su32x4 *>(row + head * int(sizeof(T)));
    constexpr int U = 4;
    for (int v0 = threadIdx.x; v0 < nvec; v0 += kSThreads * U) {
        su32x4 raw[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int v = v0 + u * kSThreads;
            raw[u] = __builtin_nontemporal_load(vr + (v < nvec ? v : nvec - 1));
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int v = v0 + u * kSThreads;
            if (v < nvec) {
                float f[E];
                SElem<T>::decode(raw[u], f);
#pragma unroll
                for (int j = 0; j < E; ++j) {
                    const uint32_t tok = uint32_t(head + v * E + j);
                    const uint64_t k = draw_key(f[j], c, tok, inv_t, tmp);
                    best = k > best ? k : best;
                }
            }
        }
    }
    for (int e = threadIdx.x; e < head + (V - head - nvec * E); e += kSThreads) {
        const int tok = e < head ? e : head + nvec * E + (e - head);
        const uint64_t k = draw_key(SElem<T>::at(row, tok), c, uint32_t(tok), inv_t, tmp);
        best = k > best ? k : best;
    }
    best = wave_max_u64(best);
    __shared__ uint64_t s_best[kSThreads / kWave];
    if ((threadIdx.x & 63) == 0) s_best[threadIdx.x >> 6] = best;
    __syncthreads();
    if (threadIdx.x == 0) {
        uint64_t m = s_best[0];
        for (int w = 1; w < kSThreads / kWave; ++w) m = s_best[w] > m ? s_best[w] : m;
        sampled[r] = topk_key_token(m);
    }
}

// Thread per query.
__global__ void mixture_sample_kernel(const float *prior, int B, int K, double temperature,
                                      const double *u, const int32_t *chains, int b, int32_t *z_out,
                                      int32_t *draft) {
    const int q = blockIdx.x * blockDim.x + threadIdx.x;
    if (q >= B) return;
    const float *p = prior + int64_t(q) * K;
    int z = 0;
    if (!(temperature > 0.0)) {
        for (int j = 1; j < K; ++j) z = p[j] > p[z] ? j : z;
    } else {
        double pm = -INFINITY, ps = 0.0;
        for (int j = 0; j < K; ++j) pm = fmax(pm, double(p[j]) / temperature);
        for (int j = 0; j < K; ++j) ps += exp(double(p[j]) / temperature - pm);
        double cdf = 0.0;
        z = K - 1;
        for (int j = 0; j < K; ++j) {
            cdf += exp(double(p[j]) / temperature - pm) / ps;
            if (u[q] < cdf) {
                z = j;
                break;
            }
        }
    }
    z_out[q] = z;
    for (int i = 0; i < b; ++i) draft[int64_t(q) * b + i] = chains[(int64_t(q) * K + z) * b + i];
}

}  // namespace

}  // namespace bastion

extern "C" {

int32_t bastion_sample_nodes(const void *logits, int32_t dtype, int32_t B, int32_t nmax, int32_t V,
                             int64_t row_stride, const int32_t *n_nodes, float temperature,
                             uint32_t seed, int32_t *sampled, void *stream) {
    using namespace bastion;
    if (!logits || !n_nodes || !sampled) return BASTION_EINVAL;
    if (dtype != BASTION_F32 && dtype != BASTION_BF16) return BASTION_EINVAL;
    if (B < 1 || nmax < 0 || nmax > kMaxNmax || V < 1 || V > kMaxV || row_stride < V)
        return BASTION_EINVAL;
    if (!(temperature >= 0.0f) || temperature > 1e30f) return BASTION_EINVAL;
    const int es = dtype == BASTION_BF16 ? 2 : 4;
    if (reinterpret_cast<uintptr_t>(logits) % es != 0) return BASTION_EINVAL;
    const hipStream_t s = static_cast<hipStream_t>(stream);
    const int64_t rows = int64_t(B) * (nmax + 1);
    const bool tmp = temperature > 0.0f;
    const float inv_t = tmp ? 1.0f / temperature : 0.0f;
    const char *lg = static_cast<const char *>(logits);
    if (dtype == BASTION_BF16)
        hipLaunchKernelGGL(sample_nodes_kernel<__bf16>, dim3(unsigned(rows)), dim3(kSThreads), 0, s,
                           lg, row_stride * es, nmax, V, n_nodes, inv_t, int(tmp), seed, sampled);
    else
        hipLaunchKernelGGL(sample_nodes_kernel<float>, dim3(unsigned(rows)), dim3(kSThreads), 0, s,
                           lg, row_stride * es, nmax, V, n_nodes, inv_t, int(tmp), seed, sampled);
    return hipGetLastError() == hipSuccess ? BASTION_OK : BASTION_EHIP;
}

int32_t bastion_mixture_sample(const float *prior_logits, int32_t B, int32_t K, double temperature,
                               const double *u, const int32_t *chain_tokens, int32_t b,
                               int32_t *z_out, int32_t *draft, void *stream) {
    using namespace bastion;
    if (!prior_logits || !u || !chain_tokens || !z_out || !draft) return BASTION_EINVAL;
    if (B < 1 || K < 1 || K > kMaxBranches || b < 1 || b > kMaxB) return BASTION_EINVAL;
    if (!(temperature >= 0.0) || temperature > 1e300) return BASTION_EINVAL;
    hipLaunchKernelGGL(mixture_sample_kernel, dim3(unsigned((B + 63) / 64)), dim3(64), 0,
                       static_cast<hipStream_t>(stream), prior_logits, B, K, temperature, u,
                       chain_tokens, b, z_out, draft);
    return hipGetLastError() == hipSuccess ? BASTION_OK : BASTION_EHIP;
}

}  // extern "C"
