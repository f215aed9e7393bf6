// verify.hip -- the tree's consumer on gfx950: one attention layer of a
// tree-structured verifier (Bastion page, Experimental results: the target
// checks the whole drafted tree in one forward pass; Methodology 3: the
// verify latency T_verify(N) is calibrated on observed runtimes of that
// pass).
//
// For every sequence s the N+1 tree tokens (node 0, the root, first) are
// appended to the sequence's KV cache behind its ctx cached tokens, and each
// tree token attends to every cached token and to the tree tokens its
// ancestor-mask row marks (its ancestors and itself).  Three launches:
//   1. append: rotary position embedding of the tree tokens' q and k at
//      their position ids (pos_base + depth), rounded to bf16; k and v go
//      into the cache, q into a scratch laid out for the attention kernel;
//   2. attention: per (128 query rows, KV head, key split of 128 keys),
//      eight waves of 16 query rows each; each 32-key step's K and V tiles
//      are loaded once into LDS for the block (double-buffered: the next
//      step's loads are in flight during this step).  S^T = K Q^T and O^T += V^T P^T on MFMA
//      (v_mfma_f32_16x16x32_bf16): the S^T tile leaves each lane holding
//      eight scores of one query row, which is exactly the B operand P^T of
//      the second product, so the probabilities never leave registers.
//      Online softmax (running max and sum per row) in float32;
//   3. combine: the key splits' partial results, merged by their maxima.
// Layouts: K cache [S][Hkv][Lmax][D] (a key's dims contiguous, the A operand
// of S^T); V cache [S][Hkv][Lmax/32][D][32], tiles of 32 keys with a dim's
// keys contiguous (the A operand of O^T), so that one 32-key step reads one
// contiguous 8 KiB tile.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "bastion.h"
#include "bastion_verify.h"

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kD = 128;           // head dim
constexpr int kHalf = kD / 2;     // rotary pairs (d, d + 64)
constexpr int kRowsPerWave = 16;  // one MFMA tile of query rows
constexpr int kWaves = 8;
constexpr int kRowsPerBlock = kRowsPerWave * kWaves;
constexpr int kKeyStep = 32;      // keys per O^T MFMA step (two S^T tiles)
constexpr int kSplitKeys = 128;   // keys per split

struct AttnArgs {
    const __bf16 *qkv;        // [S*T][*] rows of the q/k/v projection
    int64_t qkv_stride;       // elements per row
    int S, T, Hq, Hkv, G, Lmax, W, rows, rows_pad, splits;
    int ctx_cap;              // contexts are clamped to [0, ctx_cap]
    __bf16 *kc, *vc;          // caches (vc in 32-key tiles)
    const int32_t *ctx;       // [S]
    const int32_t *pos;       // [S][T]
    const uint32_t *mask;     // [S][T][W]
    const float *inv_freq;    // [kHalf]
    __bf16 *qs;               // [S][Hkv][rows_pad][kD] rotated q (rows past rows unused)
    float *opart;             // [splits][S][Hkv][rows_pad][kD]
    float *ml;                // [splits][S][Hkv][rows_pad][2]
    __bf16 *out;              // [S*T][Hq * kD]
    float scale_log2;         // log2(e) / sqrt(kD)
};

// cached tokens of sequence s, clamped to the launch's bound (at most
// Lmax - T, so that the tree fits the cache)
__device__ __forceinline__ int ctx_of(const AttnArgs &A, int s) {
    return min(max(A.ctx[s], 0), A.ctx_cap);
}

// element offset of the V-cache tile holding `key` of (s, h)
__device__ __forceinline__ int64_t vtile(const AttnArgs &A, int s, int h, int key) {
    return ((int64_t(s) * A.Hkv + h) * (A.Lmax / 32) + (key >> 5)) * (kD * 32);
}

// ---- 1. append ------------------------------------------------------------
// Block per tree token (s, t); threads over (head, pair) for q and k and over
// (head, dim) for v.  Rotation of the pair (x1, x2) = (x[d], x[d + 64]) by the
// angle fl32(pos * inv_freq[d]): (x1 cos - x2 sin, x2 cos + x1 sin), float32,
// rounded to bf16.
__global__ __launch_bounds__(256) void append_kernel(AttnArgs A) {
    const int st = blockIdx.x;
    const int s = st / A.T, t = st - s * A.T;
    const int ctx = ctx_of(A, s);
    const float pos = float(A.pos[int64_t(s) * A.T + t]);
    const __bf16 *row = A.qkv + int64_t(st) * A.qkv_stride;
    const int nq = A.Hq * kHalf, nk = A.Hkv * kHalf;
    for (int e = threadIdx.x; e < nq + nk; e += blockDim.x) {
        const bool isq = e < nq;
        const int e2 = isq ? e : e - nq;
        const int h = e2 / kHalf, d = e2 - h * kHalf;
        const __bf16 *src = row + (isq ? 0 : A.Hq * kD) + h * kD;
        const float x1 = float(src[d]), x2 = float(src[d + kHalf]);
        const float ang = pos * A.inv_freq[d];
        float sn, cs;
        sincosf(ang, &sn, &cs);
        const float y1 = x1 * cs - x2 * sn;
        const float y2 = x2 * cs + x1 * sn;
        __bf16 *dst;
        if (isq) {
            const int hk = h / A.G, g = h - hk * A.G;
            dst = A.qs + ((int64_t(s) * A.Hkv + hk) * A.rows_pad + (t * A.G + g)) * kD;
        } else {
            dst = A.kc + ((int64_t(s) * A.Hkv + h) * A.Lmax + (ctx + t)) * kD;
        }
        dst[d] = __bf16(y1);
        dst[d + kHalf] = __bf16(y2);
    }
    const __bf16 *vsrc = row + (A.Hq + A.Hkv) * kD;
    for (int e = threadIdx.x; e < A.Hkv * kD; e += blockDim.x) {
        const int h = e / kD, d = e - h * kD;
        const int key = ctx + t;
        A.vc[vtile(A, s, h, key) + d * 32 + (key & 31)] = vsrc[h * kD + d];
    }
}

// ---- 2. attention ---------------------------------------------------------
__device__ __forceinline__ float xor16_max(float v) {
    return fmaxf(v, __shfl_xor(v, 16));
}

// One 32-key step's tiles in LDS, shared by the block's waves: K as
// [key][dim] (rows padded by 16 bytes), V as [dim][key] (rows padded by 16
// bytes); double-buffered.
constexpr int kKPad = kD + 8, kVPad = kKeyStep + 8;

struct StepRegs {
    bf16x8 k, v;   // this thread's share of a step's tiles (16 bytes of each)
};

constexpr int kSteps = kSplitKeys / kKeyStep;   // steps of one split

// Thread x of the block loads 16 bytes of the K tile (key x / 16, dims
// 8 (x % 16) ..) and 16 bytes of the V tile (dim x / 4, keys 8 (x % 4) ..)
// of the step at kb.  Rows and tiles past the cache are clamped into it; the
// contents of slots past the sequence do not matter (their scores are
// masked, their v zeroed when stored).  The addresses do not depend on the
// sequence's context, so these loads go out with the block's first ones.
__device__ __forceinline__ StepRegs load_step(const __bf16 *kbase, const __bf16 *vbase, int kb,
                                              int Lmax) {
    const int x = threadIdx.x;
    StepRegs R;
    const int key = min(kb + (x >> 4), Lmax - 1);
    R.k = *reinterpret_cast<const bf16x8 *>(kbase + int64_t(key) * kD + 8 * (x & 15));
    const int tile = min(kb, Lmax - 32) >> 5;
    R.v = *reinterpret_cast<const bf16x8 *>(vbase + int64_t(tile) * (kD * 32) + (x >> 2) * 32 +
                                            8 * (x & 3));
    return R;
}

// The step's tiles into LDS; v of keys at or past k1 set to zero (a slot
// past the sequence may hold anything, NaN included).
__device__ __forceinline__ void store_step(__bf16 (*ks)[kKPad], __bf16 (*vs)[kVPad], StepRegs R,
                                           int kb, int k1) {
    const int x = threadIdx.x;
    const int k8 = 8 * (x & 3);
#pragma unroll
    for (int e = 0; e < 8; ++e) R.v[e] = kb + k8 + e < k1 ? R.v[e] : __bf16(0.0f);
    *reinterpret_cast<bf16x8 *>(&ks[x >> 4][8 * (x & 15)]) = R.k;
    *reinterpret_cast<bf16x8 *>(&vs[x >> 2][k8]) = R.v;
}

__global__ __launch_bounds__(kWaves * 64) void attention_kernel(AttnArgs A) {
    static_assert(kWaves * 64 == 32 * (kD / 8) && kWaves * 64 == kD * 4, "one load per thread");
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int h = blockIdx.y;
    const int s = blockIdx.z / A.splits, c = blockIdx.z - s * A.splits;
    const int k0 = c * kSplitKeys;
    const int64_t hs = int64_t(s) * A.Hkv + h;
    const __bf16 *kbase = A.kc + hs * A.Lmax * kD;
    const __bf16 *vbase = A.vc + hs * int64_t(A.Lmax) * kD;   // the head's first tile
    // every step's tiles of the split, issued first (one round trip for all)
    StepRegs R[kSteps];
#pragma unroll
    for (int i = 0; i < kSteps; ++i) R[i] = load_step(kbase, vbase, k0 + i * kKeyStep, A.Lmax);
    const int ctx = ctx_of(A, s);
    const int L = ctx + A.T;
    if (k0 >= L) return;          // a split past this sequence's keys (whole block)
    const int k1 = min(L, k0 + kSplitKeys);
    const int row0 = blockIdx.x * kRowsPerBlock + w * kRowsPerWave;
    const bool active = row0 < A.rows;   // idle waves still load and synchronise
    const int r16 = lane & 15, g4 = lane >> 4;
    const int myrow = row0 + r16;
    const int qr = min(myrow, A.rows - 1);   // rows past the last read a real one
    const int tok = qr / A.G;

    __shared__ __align__(16) __bf16 ks[2][kKeyStep][kKPad];
    __shared__ __align__(16) __bf16 vs[2][kD][kVPad];
    // the ancestor-mask rows of the wave's 16 query rows: the per-step bit
    // lookups wait on LDS only, never on the next step's global loads
    __shared__ uint32_t smask[kWaves][kRowsPerWave][32];
    {
        const uint32_t *mrow = A.mask + (int64_t(s) * A.T + tok) * A.W;
        for (int x = g4; x < A.W; x += 4) smask[w][r16][x] = mrow[x];
    }
    // Q^T, the B operand of S^T = K Q^T: lane (r16, g4) holds dims
    // 32 st + 8 g4 .. + 7 of its row
    bf16x8 qv[4];
    const __bf16 *qrow = A.qs + (hs * A.rows_pad + qr) * kD;
#pragma unroll
    for (int st = 0; st < 4; ++st) qv[st] = *reinterpret_cast<const bf16x8 *>(qrow + 32 * st + 8 * g4);

    store_step(ks[0], vs[0], R[0], k0, k1);
    __syncthreads();
    const uint32_t *mrow = smask[w][r16];
    float m = -INFINITY, lsum = 0.0f;
    f32x4 o[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) o[j] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};

#pragma unroll
    for (int i = 0; i < kSteps; ++i) {
        const int kb = k0 + i * kKeyStep;
        if (kb >= k1) break;      // block-uniform
        const int buf = i & 1;
        if (active) {
            f32x4 s0 = {0.0f, 0.0f, 0.0f, 0.0f}, s1 = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
            for (int st = 0; st < 4; ++st) {
                const bf16x8 a0 = *reinterpret_cast<const bf16x8 *>(&ks[buf][r16][32 * st + 8 * g4]);
                const bf16x8 a1 = *reinterpret_cast<const bf16x8 *>(&ks[buf][16 + r16][32 * st + 8 * g4]);
                s0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a0, qv[st], s0, 0, 0, 0);
                s1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a1, qv[st], s1, 0, 0, 0);
            }
            // lane (r16, g4) now holds row r16's scores of keys kb + 4 g4 + r
            // (s0) and kb + 16 + 4 g4 + r (s1), r = 0..3
            float v[8];
            const int kq = kb + 4 * g4;
#pragma unroll
            for (int r = 0; r < 8; ++r) {
                const int kk = kq + (r < 4 ? r : 12 + r);
                const float sc = (r < 4 ? s0[r] : s1[r - 4]) * A.scale_log2;
                const int j = min(max(kk - ctx, 0), A.T - 1);
                const bool bit = (mrow[j >> 5] >> (j & 31)) & 1u;
                const bool vis = kk < k1 && (kk < ctx || bit);
                v[r] = vis ? sc : -INFINITY;
            }
            float tmax = v[0];
#pragma unroll
            for (int r = 1; r < 8; ++r) tmax = fmaxf(tmax, v[r]);
            tmax = xor16_max(tmax);
            tmax = fmaxf(tmax, __shfl_xor(tmax, 32));
            const float mn = fmaxf(m, tmax);
            const bool live = mn > -INFINITY;
            const float alpha = live ? __builtin_amdgcn_exp2f(m - mn) : 1.0f;
            bf16x8 pb;
            float ps = 0.0f;
#pragma unroll
            for (int r = 0; r < 8; ++r) {
                const float p = live ? __builtin_amdgcn_exp2f(v[r] - mn) : 0.0f;
                ps += p;
                pb[r] = __bf16(p);
            }
            lsum = lsum * alpha + ps;
            m = mn;
            // V^T, the A operand of O^T += V^T P^T: dim 16 j + r16, keys in
            // the order of the lane's scores (4 of each S^T tile)
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const __bf16 *vr = &vs[buf][16 * j + r16][4 * g4];
                const bf16x4 lo = *reinterpret_cast<const bf16x4 *>(vr);
                const bf16x4 hi = *reinterpret_cast<const bf16x4 *>(vr + 16);
                bf16x8 av;
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    av[r] = lo[r];
                    av[4 + r] = hi[r];
                }
#pragma unroll
                for (int r = 0; r < 4; ++r) o[j][r] *= alpha;
                o[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, pb, o[j], 0, 0, 0);
            }
        }
        // every wave is done with the other buffer since the last barrier
        if (i + 1 < kSteps) store_step(ks[buf ^ 1], vs[buf ^ 1], R[i + 1], kb + kKeyStep, k1);
        __syncthreads();
    }
    if (!active) return;
    // the row's sum over its four lanes
    lsum += __shfl_xor(lsum, 16);
    lsum += __shfl_xor(lsum, 32);
    if (myrow >= A.rows) return;
    // O^T tile j, register r: dim 16 j + 4 g4 + r of row r16
    if (A.splits == 1) {
        const int t = myrow / A.G, g = myrow - t * A.G;
        __bf16 *dst = A.out + (int64_t(s) * A.T + t) * (int64_t(A.Hq) * kD) + (h * A.G + g) * kD;
        const float inv = lsum > 0.0f ? 1.0f / lsum : 0.0f;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            bf16x4 ov;
#pragma unroll
            for (int r = 0; r < 4; ++r) ov[r] = __bf16(o[j][r] * inv);
            *reinterpret_cast<bf16x4 *>(dst + 16 * j + 4 * g4) = ov;
        }
        return;
    }
    const int64_t prow = ((int64_t(c) * A.S + s) * A.Hkv + h) * A.rows_pad + myrow;
    float *op = A.opart + prow * kD;
#pragma unroll
    for (int j = 0; j < 8; ++j) *reinterpret_cast<f32x4 *>(op + 16 * j + 4 * g4) = o[j];
    if (g4 == 0) {
        A.ml[2 * prow] = m;
        A.ml[2 * prow + 1] = lsum;
    }
}

// ---- 3. combine -----------------------------------------------------------
// One wave per (s, h, row): lane l holds the partial maxima and sums of
// splits l, l + 64, ..; the row's maximum and normaliser are wave
// reductions; then lane l accumulates dims 2 l, 2 l + 1 over the splits,
// eight partial rows in flight at a time.
__global__ __launch_bounds__(256) void combine_kernel(AttnArgs A) {
    const int lane = threadIdx.x & 63;
    const int wid = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (wid >= A.S * A.Hkv * A.rows) return;
    const int sh = wid / A.rows, row = wid - sh * A.rows;   // sh = s * Hkv + h
    const int s = sh / A.Hkv, h = sh - s * A.Hkv;
    const int live = (ctx_of(A, s) + A.T + kSplitKeys - 1) / kSplitKeys;
    const int64_t stride = int64_t(A.S) * A.Hkv * A.rows_pad;   // one split's rows
    const int64_t base = int64_t(sh) * A.rows_pad + row;
    float mc[2], lc[2];
    float M = -INFINITY;
#pragma unroll
    for (int u = 0; u < 2; ++u) {   // live <= 128 splits (Lmax <= 16384)
        const int c = lane + 64 * u;
        mc[u] = c < live ? A.ml[2 * (c * stride + base)] : -INFINITY;
        lc[u] = c < live ? A.ml[2 * (c * stride + base) + 1] : 0.0f;
        M = fmaxf(M, mc[u]);
    }
    for (int o = 32; o >= 1; o >>= 1) M = fmaxf(M, __shfl_xor(M, o));
    float f[2], den = 0.0f;
#pragma unroll
    for (int u = 0; u < 2; ++u) {
        f[u] = mc[u] > -INFINITY ? __builtin_amdgcn_exp2f(mc[u] - M) : 0.0f;
        den += f[u] * lc[u];
    }
    for (int o = 32; o >= 1; o >>= 1) den += __shfl_xor(den, o);
    float a0 = 0.0f, a1 = 0.0f;
    for (int c0 = 0; c0 < live; c0 += 8) {
        float2 v[8];
        float fw[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const int c = min(c0 + u, live - 1);
            v[u] = *reinterpret_cast<const float2 *>(A.opart + (c * stride + base) * kD + 2 * lane);
            const float fc = __shfl(f[(c >> 6) & 1], c & 63);
            fw[u] = c0 + u < live ? fc : 0.0f;
        }
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            a0 += fw[u] * v[u].x;
            a1 += fw[u] * v[u].y;
        }
    }
    const float inv = den > 0.0f ? 1.0f / den : 0.0f;
    const int t = row / A.G, g = row - t * A.G;
    __bf16 *dst = A.out + (int64_t(s) * A.T + t) * (int64_t(A.Hq) * kD) + (h * A.G + g) * kD;
    dst[2 * lane] = __bf16(a0 * inv);
    dst[2 * lane + 1] = __bf16(a1 * inv);
}

int splits_for(int keys) { return (keys + kSplitKeys - 1) / kSplitKeys; }

int pad_rows(int rows) { return (rows + kRowsPerBlock - 1) / kRowsPerBlock * kRowsPerBlock; }

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

// workspace: rotated q, partial outputs, partial (max, sum); sized for the
// largest launch (contexts up to Lmax - T)
void ws_layout(int S, int T, int Hq, int Hkv, int Lmax, size_t &oq, size_t &oo, size_t &om,
               size_t &total) {
    const int G = Hq / Hkv;
    const int rows_pad = pad_rows(T * G);
    const int splits = splits_for(Lmax);
    oq = 0;
    oo = align256(oq + size_t(S) * Hkv * rows_pad * kD * 2);
    om = align256(oo + (splits > 1 ? size_t(splits) * S * Hkv * rows_pad * kD * 4 : 0));
    total = align256(om + (splits > 1 ? size_t(splits) * S * Hkv * rows_pad * 2 * 4 : 0));
}

bool aligned(const void *p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

}  // namespace

extern "C" {

size_t bastion_tree_attention_workspace_bytes(int32_t S, int32_t T, int32_t Hq, int32_t Hkv,
                                              int32_t Lmax) {
    if (S < 1 || T < 1 || Hkv < 1 || Hq < Hkv || Hq % Hkv != 0 || Lmax < T) return 0;
    size_t a, b, c, total;
    ws_layout(S, T, Hq, Hkv, Lmax, a, b, c, total);
    return total;
}

int32_t bastion_tree_attention(const void *qkv, int64_t qkv_row_stride, int32_t S, int32_t T,
                               int32_t Hq, int32_t Hkv, int32_t D, void *k_cache, void *v_cache,
                               int32_t Lmax, const int32_t *ctx_len, int32_t max_ctx,
                               const int32_t *position_ids, const uint32_t *mask, int32_t W,
                               const float *inv_freq, void *out, void *ws, size_t ws_bytes,
                               void *stream) {
    if (!qkv || !k_cache || !v_cache || !ctx_len || !position_ids || !mask || !inv_freq || !out)
        return BASTION_EINVAL;
    if (S < 1 || T < 1 || T > 1024 || Hkv < 1 || Hq < Hkv || Hq % Hkv != 0) return BASTION_EINVAL;
    if (int64_t(S) * Hq * T >= (int64_t(1) << 31) || Lmax > 16384) return BASTION_EUNSUPPORTED;
    const int G = Hq / Hkv;
    if (G > 16 || 16 % G != 0) return BASTION_EUNSUPPORTED;
    if (D != kD) return BASTION_EUNSUPPORTED;
    if (W != (T + 31) / 32 || Lmax < T || Lmax % 32 != 0) return BASTION_EINVAL;
    if (qkv_row_stride < int64_t(Hq + 2 * Hkv) * kD || qkv_row_stride % 8 != 0)
        return BASTION_EINVAL;
    if (!aligned(qkv, 16) || !aligned(k_cache, 16) || !aligned(v_cache, 16) || !aligned(out, 16))
        return BASTION_EINVAL;
    size_t oq, oo, om, total;
    ws_layout(S, T, Hq, Hkv, Lmax, oq, oo, om, total);
    if (!ws || !aligned(ws, 256) || ws_bytes < total) return BASTION_EWORKSPACE;
    AttnArgs A;
    A.qkv = static_cast<const __bf16 *>(qkv);
    A.qkv_stride = qkv_row_stride;
    A.S = S; A.T = T; A.Hq = Hq; A.Hkv = Hkv; A.G = G; A.Lmax = Lmax; A.W = W;
    A.rows = T * G;
    A.rows_pad = pad_rows(A.rows);
    A.ctx_cap = (max_ctx >= 0 && max_ctx < Lmax - T) ? max_ctx : Lmax - T;
    A.splits = splits_for(A.ctx_cap + T);
    A.kc = static_cast<__bf16 *>(k_cache);
    A.vc = static_cast<__bf16 *>(v_cache);
    A.ctx = ctx_len;
    A.pos = position_ids;
    A.mask = mask;
    A.inv_freq = inv_freq;
    char *w = static_cast<char *>(ws);
    A.qs = reinterpret_cast<__bf16 *>(w + oq);
    A.opart = reinterpret_cast<float *>(w + oo);
    A.ml = reinterpret_cast<float *>(w + om);
    A.out = static_cast<__bf16 *>(out);
    A.scale_log2 = 1.44269504088896340736f / sqrtf(float(kD));
    const hipStream_t st = static_cast<hipStream_t>(stream);
    hipLaunchKernelGGL(append_kernel, dim3(unsigned(S * T)), dim3(256), 0, st, A);
    hipLaunchKernelGGL(attention_kernel, dim3(unsigned(A.rows_pad / kRowsPerBlock), unsigned(Hkv),
                                              unsigned(S * A.splits)),
                       dim3(kWaves * 64), 0, st, A);
    if (A.splits > 1) {
        const int64_t waves = int64_t(S) * Hkv * A.rows;
        hipLaunchKernelGGL(combine_kernel, dim3(unsigned((waves + 3) / 4)), dim3(256), 0, st, A);
    }
    return hipGetLastError() == hipSuccess ? BASTION_OK : BASTION_EHIP;
}

}  // extern "C"
