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
//   1. append: per (sequence, 32-slot cache tile, group of heads): the
//      rotary embedding of the tree tokens' q and k at their position ids
//      (each (token, pair) angle's sine and cosine computed once, in LDS,
//      for all heads of the group), rounded to bf16; k and v go into the
//      cache (v as whole 64-byte tile rows), q into a scratch laid out for
//      the attention kernel;
//   2. attention: per (sequence, KV head, chunk of keys) one block of eight
//      waves holds up to 384 query rows of the KV head (the
//      tree's T tokens times the Hq/Hkv query heads that share it: 260 at
//      N = 64 and 4 heads per KV head), so each key's k and v are read from
//      HBM once.  The chunk streams through LDS in 32-key steps (K as
//      [key][dim], V as [dim][key]); four steps of loads are in flight in
//      registers while the waves compute on the LDS copy of the current
//      step.  S^T = K Q^T and O^T += V^T P^T on MFMA
//      (v_mfma_f32_16x16x32_bf16): the S^T tile leaves each lane holding
//      eight scores of one query row, which is exactly the B operand P^T of
//      the second product, so the probabilities never leave registers.
//      Online softmax (running max and sum per row) in float32.  A
//      sequence whose keys fit one chunk writes its output directly;
//   3. combine: the chunks' partial results of the other sequences, merged
//      by their maxima.
// Chunk length: as long as the launch still has enough blocks to fill the
// machine (about 1024 for the grid), at least 128 keys, so that partial
// results stay a small fraction of the key/value bytes when many sequences
// are verified at once.
// Layouts: K cache [S][Hkv][Lmax][D] (a key's dims contiguous, the A operand
// of S^T); V cache [S][Hkv][Lmax/32][D][32], tiles of 32 keys with a dim's
// keys contiguous (the A operand of O^T), so that one 32-key step reads one
// contiguous 8 KiB tile of each.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stdlib.h>

#include <atomic>


#include "bastion.h"
#include "bastion_verify.h"

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kD = 128;           // head dim
constexpr int kHalf = kD / 2;     // rotary pairs (d, d + 64)
constexpr int kTile = 16;         // query rows per MFMA tile
constexpr int kKeyStep = 32;      // keys per O^T MFMA step (two S^T tiles)
constexpr int kWaves = 8;         // attention block: two waves per SIMD
constexpr int kTpw = 3;           // row tiles per wave
constexpr int kTilesPerBlock = kWaves * kTpw;   // 384 query rows per block
constexpr int kPrefetch = 4;      // steps of loads in flight in registers
constexpr float kLazy = 8.0f;     // log2 headroom before a row's reference max is raised
constexpr int kMinChunk = 128;    // shortest key chunk
constexpr int kRotHeads = 8;      // heads per rotation block of the append
constexpr int kValHeads = 2;      // KV heads per value block of the append

int target_blocks() {
    // the grid size the chunk length aims for; BASTION_ATTN_BLOCKS overrides
    // it (tuning), read once
    static const int v = [] {
        const char *e = getenv("BASTION_ATTN_BLOCKS");
        const int x = e ? atoi(e) : 0;
        return x >= 64 && x <= (1 << 20) ? x : 1024;
    }();
    return v;
}

struct AttnArgs {
    const __bf16 *qkv;        // [S*T][*] rows of the q/k/v projection
    int64_t qkv_stride;       // elements per row
    int S, T, Hq, Hkv, G, Lmax, W, rows;
    int ctx_cap;              // contexts are clamped to [0, ctx_cap]
    int chunk, chunks;        // keys per chunk (multiple of 32), chunks in the grid
    int tiles;                // row tiles, ceil(rows / 16)
    __bf16 *kc, *vc;          // caches (vc in 32-key tiles)
    const int32_t *ctx;       // [S]
    const int32_t *pos;       // [S][T]
    const uint32_t *mask;     // [S][T][W]
    const float *inv_freq;    // [kHalf]
    __bf16 *qs;               // [S][Hkv][rows][kD] rotated q
    float *opart;             // [chunks][S][Hkv][rows][kD]
    float *ml;                // [chunks][S][Hkv][rows][2]
    __bf16 *out;              // [S*T][Hq * kD]
    float scale_log2;         // log2(e) / sqrt(kD)
    int rot_groups, val_groups, key_tiles;   // append grid
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
// Block (group, tile, s): the tree tokens whose slots ctx + t fall in the
// group's 32-slot tile jt of the cache (counted from the tile of slot ctx).
// Rotation groups take kRotHeads heads of [0, Hq + Hkv) (q heads, then k
// heads); value groups take kValHeads KV heads.  Rotation of the pair
// (x1, x2) = (x[d], x[d + 64]) by the angle fl32(pos * inv_freq[d]):
// (x1 cos - x2 sin, x2 cos + x1 sin), float32, rounded to bf16.
__global__ __launch_bounds__(256) void append_kernel(AttnArgs A) {
    const int grp = blockIdx.x, jt = blockIdx.y, s = blockIdx.z, tid = threadIdx.x;
    const int ctx = ctx_of(A, s);
    const int tile = (ctx >> 5) + jt;
    const int lo = max(ctx, tile * 32), hi = min(ctx + A.T, tile * 32 + 32);
    if (lo >= hi) return;
    const int ta = lo - ctx, ntok = hi - lo;
    const __bf16 *rows = A.qkv + int64_t(s) * A.T * A.qkv_stride;
    if (grp < A.rot_groups) {
        __shared__ float s_cos[32][kHalf], s_sin[32][kHalf];
        for (int e = tid; e < ntok * kHalf; e += 256) {
            const int tl = e / kHalf, d = e - tl * kHalf;
            const float ang = float(A.pos[int64_t(s) * A.T + ta + tl]) * A.inv_freq[d];
            float sn, cs;
            sincosf(ang, &sn, &cs);
            s_cos[tl][d] = cs;
            s_sin[tl][d] = sn;
        }
        __syncthreads();
        const int h0 = grp * kRotHeads;
        const int nh = min(kRotHeads, A.Hq + A.Hkv - h0);
        // item: (token, head, 8 pairs); the 8 items of a head are adjacent
        for (int e = tid; e < ntok * nh * 8; e += 256) {
            const int dv = e & 7, th = e >> 3;
            const int tl = th / nh, hh = h0 + (th - tl * nh);
            const int t = ta + tl, d0 = 8 * dv;
            const __bf16 *src = rows + int64_t(t) * A.qkv_stride + hh * kD + d0;
            const bf16x8 x1 = *reinterpret_cast<const bf16x8 *>(src);
            const bf16x8 x2 = *reinterpret_cast<const bf16x8 *>(src + kHalf);
            bf16x8 y1, y2;
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const float cs = s_cos[tl][d0 + i], sn = s_sin[tl][d0 + i];
                const float a = float(x1[i]), b = float(x2[i]);
                y1[i] = __bf16(a * cs - b * sn);
                y2[i] = __bf16(b * cs + a * sn);
            }
            __bf16 *dst;
            if (hh < A.Hq) {
                const int hk = hh / A.G, g = hh - hk * A.G;
                dst = A.qs + ((int64_t(s) * A.Hkv + hk) * A.rows + (int64_t(t) * A.G + g)) * kD;
            } else {
                dst = A.kc + ((int64_t(s) * A.Hkv + (hh - A.Hq)) * A.Lmax + (ctx + t)) * kD;
            }
            *reinterpret_cast<bf16x8 *>(dst + d0) = y1;
            *reinterpret_cast<bf16x8 *>(dst + d0 + kHalf) = y2;
        }
        return;
    }
    // value group: item (head, dim, 8 slots of the tile), the 4 items of a
    // dim adjacent so that a 64-byte tile row is written by 4 lanes
    const int hv0 = (grp - A.rot_groups) * kValHeads;
    const int nh = min(kValHeads, A.Hkv - hv0);
    const __bf16 *vcol = rows + (A.Hq + A.Hkv) * kD;
    for (int e = tid; e < nh * kD * 4; e += 256) {
        const int q4 = e & 3, hd = e >> 2;
        const int hl = hd / kD, d = hd - hl * kD, h = hv0 + hl;
        const int k8 = tile * 32 + 8 * q4;
        if (k8 + 8 <= lo || k8 >= hi) continue;
        bf16x8 *dst = reinterpret_cast<bf16x8 *>(A.vc + vtile(A, s, h, k8) + d * 32 + 8 * q4);
        bf16x8 v;
        const bool whole = k8 >= lo && k8 + 8 <= hi;
        if (!whole) v = *dst;   // slots outside the tree keep what they hold
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int key = k8 + i;
            if (key >= lo && key < hi)
                v[i] = vcol[int64_t(key - ctx) * A.qkv_stride + h * kD + d];
        }
        *dst = v;
    }
}

// ---- 2. attention ---------------------------------------------------------
// max over the four lanes r16 + 16 g4 of a row (lanes 16 and 32 apart),
// with the cross-row swaps (VALU, no LDS round trip)
__device__ __forceinline__ float row4_max(float v) {
    const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false,
                                                    false);
    v = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
    const auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false,
                                                    false);
    return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

// One 32-key step's tiles in LDS, shared by the block's waves: K as
// [key][dim] (rows padded by 16 bytes; keys 8a + 4h + r of the step in row
// 16h + 4a + r), V as [dim][key] (rows padded by 16
// bytes); double-buffered.
constexpr int kKPad = kD + 8, kVPad = kKeyStep + 8;

// A step's K tile (32 keys x 128 dims) and V tile (128 dims x 32 keys) are
// each one contiguous 8 KiB range of their cache: 16 wave-sized pieces of
// 1 KiB, pieces 0-7 the K tile and 8-15 the V tile.  Wave w loads pieces
// w and w + 8; each lane loads 16 bytes at a constant offset from the
// step's (block-uniform) base, so no per-lane address arithmetic is
// repeated per step.
struct Steps {
    static constexpr int kVpt = 16 / kWaves;
    bf16x8 r[kPrefetch][kVpt];

    // the loads of the step whose tiles start at kst / vst into slot j
    __device__ __forceinline__ void load(int j, int wv, const char *kst, const char *vst) {
        const int lane = threadIdx.x & 63;
#pragma unroll
        for (int v = 0; v < kVpt; ++v) {
            const int q = wv + kWaves * v;
            const char *p = (q < 8 ? kst : vst) + 16 * (64 * (q & 7) + lane);
            r[j][v] = __builtin_nontemporal_load(reinterpret_cast<const bf16x8 *>(p));
        }
    }

    // slot j into the LDS buffers; v of keys at or past k1 set to zero (a
    // slot past the chunk's keys may hold anything, NaN included) unless
    // the whole step is inside the chunk
    __device__ __forceinline__ void store(int j, int wv, __bf16 (*ks)[kKPad], __bf16 (*vs)[kVPad],
                                          int kb, int k1) {
        const int lane = threadIdx.x & 63;
        const bool full = kb + kKeyStep <= k1;
#pragma unroll
        for (int v = 0; v < kVpt; ++v) {
            const int q = wv + kWaves * v;
            bf16x8 val = r[j][v];
            const int x = 64 * (q & 7) + lane;
            if (q < 8) {
                // key 8a + 4h + r of the step goes to row 16h + 4a + r, so that
                // S^T's two 16-row blocks give lane g4 the keys 8 g4 .. 8 g4 + 7
                const int kp = q & 7;   // the piece's keys are 4 kp .. 4 kp + 3
                const int row = 16 * (kp & 1) + 4 * (kp >> 1) + (lane >> 4);
                *reinterpret_cast<bf16x8 *>(&ks[row][8 * (x & 15)]) = val;
            } else {
                const int k8 = 8 * (x & 3);
                if (!full) {
#pragma unroll
                    for (int e = 0; e < 8; ++e) val[e] = kb + k8 + e < k1 ? val[e] : __bf16(0.0f);
                }
                *reinterpret_cast<bf16x8 *>(&vs[x >> 2][k8]) = val;
            }
        }
    }
};

// Block (s * Hkv + h, row block, chunk): eight waves, wave w holding row
// tiles w, w + 8, w + 16 of the row block (16 rows each) with their Q^T in
// registers (wave w runs on SIMD w % 4: 17 tiles, 65 tokens times 4 heads,
// put 5, 4, 4, 4 tiles on the four SIMDs).  The block streams the chunk's
// keys in 32-key steps through double-buffered LDS tiles, four steps of
// loads in flight in registers.  Softmax reference per row: raised to the
// row's running maximum only when a score passes it by more than 2^kLazy
// (then the row's sum and output are rescaled), so probabilities stay below
// 2^kLazy and the rescale is rare.
__global__ __launch_bounds__(kWaves * 64) void attention_kernel(AttnArgs A) {
    const int lane = threadIdx.x & 63;
    const int w = __builtin_amdgcn_readfirstlane(int(threadIdx.x) >> 6);
    const int sh = blockIdx.x, rb = blockIdx.y, c = blockIdx.z;
    const int s = sh / A.Hkv, h = sh - s * A.Hkv;
    // block-uniform: keeps every step bound and tile base in scalar registers
    const int ctx = __builtin_amdgcn_readfirstlane(ctx_of(A, s));
    const int L = ctx + A.T;
    const int k0 = c * A.chunk;
    if (k0 >= L) return;          // a chunk past this sequence's keys (whole block)
    const int k1 = min(L, k0 + A.chunk);
    const int last = (k1 - k0 + kKeyStep - 1) / kKeyStep - 1;   // the chunk's last step
    const bool single = L <= A.chunk;                          // one chunk: write the output
    const int64_t hs = int64_t(s) * A.Hkv + h;
    const char *kbase = reinterpret_cast<const char *>(A.kc + hs * A.Lmax * kD);
    const char *vbase = reinterpret_cast<const char *>(A.vc + hs * int64_t(A.Lmax) * kD);
    // the tiles of step st of the chunk (clamped to its last step)
    auto ktile = [&](int st) { return kbase + int64_t(k0 + kKeyStep * min(st, last)) * (kD * 2); };
    auto vtile_of = [&](int st) {
        return vbase + int64_t((k0 >> 5) + min(st, last)) * (kD * 32 * 2);
    };

    Steps R;
#pragma unroll
    for (int j = 0; j < kPrefetch; ++j) R.load(j, w, ktile(j), vtile_of(j));

    const int r16 = lane & 15, g4 = lane >> 4;
    __shared__ __align__(16) __bf16 ks[2][kKeyStep][kKPad];
    __shared__ __align__(16) __bf16 vs[2][kD][kVPad];
    // the ancestor-mask rows of the block's query rows [kTilesPerBlock * 16][W]
    extern __shared__ uint32_t smask[];
    int row0[kTpw];
    bool active[kTpw];
    bf16x8 qv[kTpw][4];
    const bool tree_keys = k1 > ctx;   // the chunk reaches the tree's own keys
#pragma unroll
    for (int u = 0; u < kTpw; ++u) {
        const int lt = w + kWaves * u;                 // tile inside the block
        const int tile = rb * kTilesPerBlock + lt;
        row0[u] = tile * kTile;
        active[u] = tile < A.tiles;                    // wave-uniform
        const int qr = min(row0[u] + r16, A.rows - 1);   // rows past the last read a real one
        if (tree_keys) {
            const uint32_t *mrow = A.mask + (int64_t(s) * A.T + qr / A.G) * A.W;
            for (int x = g4; x < A.W; x += 4) smask[(lt * kTile + r16) * A.W + x] = mrow[x];
        }
        // Q^T, the B operand of S^T = K Q^T: lane (r16, g4) holds dims
        // 32 st + 8 g4 .. + 7 of its row
        const __bf16 *qrow = A.qs + (hs * A.rows + qr) * kD;
#pragma unroll
        for (int st = 0; st < 4; ++st)
            qv[u][st] = *reinterpret_cast<const bf16x8 *>(qrow + 32 * st + 8 * g4);
    }

    R.store(0, w, ks[0], vs[0], k0, k1);
    R.load(0, w, ktile(kPrefetch), vtile_of(kPrefetch));
    __syncthreads();

    float m[kTpw], lsum[kTpw];
    f32x4 o[kTpw][8];
#pragma unroll
    for (int u = 0; u < kTpw; ++u) {
        m[u] = -INFINITY;
        lsum[u] = 0.0f;
#pragma unroll
        for (int j = 0; j < 8; ++j) o[u][j] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    }

    // one 32-key step: compute on LDS buffer i & 1, then move step i + 1
    // from its register slot into the other buffer and refill the slot with
    // step i + 1 + kPrefetch (past the chunk's last step these are repeats
    // of it, stored into a buffer nobody reads)
    auto step = [&](const int i, const int uu) {
        const int kb = k0 + i * kKeyStep;
        const int buf = i & 1;
        // every key of the step is a cached token inside the chunk
        const bool plain = kb + kKeyStep <= ctx;
        // S^T of every tile of the wave; each K fragment is read from LDS
        // once and used for all of them
        f32x4 s0[kTpw], s1[kTpw];
#pragma unroll
        for (int u = 0; u < kTpw; ++u) {
            s0[u] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
            s1[u] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
        }
#pragma unroll
        for (int st = 0; st < 4; ++st) {
            const bf16x8 a0 = *reinterpret_cast<const bf16x8 *>(&ks[buf][r16][32 * st + 8 * g4]);
            const bf16x8 a1 = *reinterpret_cast<const bf16x8 *>(&ks[buf][16 + r16][32 * st + 8 * g4]);
#pragma unroll
            for (int u = 0; u < kTpw; ++u) {
                if (!active[u]) continue;
                s0[u] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a0, qv[u][st], s0[u], 0, 0, 0);
                s1[u] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a1, qv[u][st], s1[u], 0, 0, 0);
            }
        }
        // lane (r16, g4) now holds row r16's scores of keys kb + 8 g4 + r
        // (s0) and kb + 8 g4 + 4 + r (s1), r = 0..3
        bf16x8 pb[kTpw];
#pragma unroll
        for (int u = 0; u < kTpw; ++u) {
            if (!active[u]) continue;
            float v[8];
            const int kq = kb + 8 * g4;
            const uint32_t *mrow = smask + ((w + kWaves * u) * kTile + r16) * A.W;
#pragma unroll
            for (int r = 0; r < 8; ++r) {
                // raw score: the scale enters the max (monotone) and the exp2's fma
                const float sc = r < 4 ? s0[u][r] : s1[u][r - 4];
                if (plain) {
                    v[r] = sc;
                } else {
                    const int kk = kq + r;
                    const int j = min(max(kk - ctx, 0), A.T - 1);
                    const bool bit = (mrow[j >> 5] >> (j & 31)) & 1u;
                    const bool vis = kk < k1 && (kk < ctx || bit);
                    v[r] = vis ? sc : -INFINITY;
                }
            }
            float tmax = v[0];
#pragma unroll
            for (int r = 1; r < 8; ++r) tmax = fmaxf(tmax, v[r]);
            tmax = row4_max(tmax) * A.scale_log2;
            // raise the reference of rows whose scores pass it by 2^kLazy
            const bool raise = tmax > m[u] + kLazy;
            if (__ballot(raise)) {   // wave-uniform, rare after the first steps
                const float mn = raise ? tmax : m[u];
                const float alpha = raise ? __builtin_amdgcn_exp2f(m[u] - mn) : 1.0f;   // 0 from -inf
                lsum[u] *= alpha;
#pragma unroll
                for (int j = 0; j < 8; ++j)
#pragma unroll
                    for (int r = 0; r < 4; ++r) o[u][j][r] *= alpha;
                m[u] = mn;
            }
            const bool live = m[u] > -INFINITY;
            float ps = 0.0f;
#pragma unroll
            for (int r = 0; r < 8; ++r) {
                const float p =
                    live ? __builtin_amdgcn_exp2f(__builtin_fmaf(v[r], A.scale_log2, -m[u])) : 0.0f;
                ps += p;
                pb[u][r] = __bf16(p);
            }
            lsum[u] += ps;
        }
        // O^T += V^T P^T: V^T fragment j (dim 16 j + r16, the lane's keys
        // 8 g4 .. 8 g4 + 7) read once for all tiles
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const bf16x8 av = *reinterpret_cast<const bf16x8 *>(&vs[buf][16 * j + r16][8 * g4]);
#pragma unroll
            for (int u = 0; u < kTpw; ++u) {
                if (!active[u]) continue;
                o[u][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, pb[u], o[u][j], 0, 0, 0);
            }
        }
        const int nx = (uu + 1) % kPrefetch;
        R.store(nx, w, ks[buf ^ 1], vs[buf ^ 1], kb + kKeyStep, k1);
        R.load(nx, w, ktile(i + 1 + kPrefetch), vtile_of(i + 1 + kPrefetch));
        __syncthreads();
    };
    // whole groups of kPrefetch steps with no exit inside, then the rest
    const int nsteps = last + 1;
    int i0 = 0;
    for (; i0 + kPrefetch <= nsteps; i0 += kPrefetch) {
#pragma unroll
        for (int uu = 0; uu < kPrefetch; ++uu) step(i0 + uu, uu);
    }
#pragma unroll
    for (int uu = 0; uu < kPrefetch - 1; ++uu)
        if (i0 + uu < nsteps) step(i0 + uu, uu);

#pragma unroll
    for (int u = 0; u < kTpw; ++u) {
        if (!active[u]) continue;
        // the row's sum over its four lanes
        float ls = lsum[u];
        ls += __shfl_xor(ls, 16);
        ls += __shfl_xor(ls, 32);
        const int myrow = row0[u] + r16;
        if (myrow >= A.rows) continue;
        // O^T tile j, register r: dim 16 j + 4 g4 + r of row r16
        if (single) {
            const int t = myrow / A.G, g = myrow - t * A.G;
            __bf16 *dst = A.out + (int64_t(s) * A.T + t) * (int64_t(A.Hq) * kD) + (h * A.G + g) * kD;
            const float inv = ls > 0.0f ? 1.0f / ls : 0.0f;
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                bf16x4 ov;
#pragma unroll
                for (int r = 0; r < 4; ++r) ov[r] = __bf16(o[u][j][r] * inv);
                *reinterpret_cast<bf16x4 *>(dst + 16 * j + 4 * g4) = ov;
            }
            continue;
        }
        const int64_t prow = ((int64_t(c) * A.S + s) * A.Hkv + h) * A.rows + myrow;
        float *op = A.opart + prow * kD;
#pragma unroll
        for (int j = 0; j < 8; ++j) *reinterpret_cast<f32x4 *>(op + 16 * j + 4 * g4) = o[u][j];
        if (g4 == 0) {
            A.ml[2 * prow] = m[u];
            A.ml[2 * prow + 1] = ls;
        }
    }
}

// ---- 3. combine -----------------------------------------------------------
// One wave per (s, h, row) of a sequence with more than one chunk: lane l
// holds the partial maxima and sums of chunks l, l + 64; the row's maximum
// and normaliser are wave reductions; then lane l accumulates dims 2 l,
// 2 l + 1 over the chunks, eight partial rows in flight at a time.
__global__ __launch_bounds__(256) void combine_kernel(AttnArgs A) {
    const int lane = threadIdx.x & 63;
    const int wid = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (wid >= A.S * A.Hkv * A.rows) return;
    const int sh = wid / A.rows, row = wid - sh * A.rows;   // sh = s * Hkv + h
    const int s = sh / A.Hkv, h = sh - s * A.Hkv;
    const int live = (ctx_of(A, s) + A.T + A.chunk - 1) / A.chunk;
    if (live <= 1) return;   // written by the attention kernel
    const int64_t stride = int64_t(A.S) * A.Hkv * A.rows;   // one chunk's rows
    const int64_t base = int64_t(sh) * A.rows + row;
    float mc[2], lc[2];
    float M = -INFINITY;
#pragma unroll
    for (int u = 0; u < 2; ++u) {   // live <= 128 chunks (Lmax <= 16384, chunks >= 128 keys)
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

// ---- launch geometry -------------------------------------------------------
int tiles_of(int rows) { return (rows + kTile - 1) / kTile; }
int row_blocks_of(int rows) { return (tiles_of(rows) + kTilesPerBlock - 1) / kTilesPerBlock; }

int round32(int64_t x) { return int((x + 31) / 32 * 32); }

// keys per chunk for keys = cap + T slots per sequence
int chunk_for(int keys, int S, int Hkv, int row_blocks) {
    const int64_t units = int64_t(S) * Hkv * row_blocks;
    int c = round32((int64_t(keys) * units + target_blocks() - 1) / target_blocks());
    c = c < kMinChunk ? kMinChunk : c;
    const int whole = round32(keys);
    return c < whole ? c : whole;
}

// the most chunks any launch of these sizes uses (every cap <= Lmax - T)
int max_chunks(int S, int Hkv, int row_blocks, int Lmax) {
    const int64_t units = int64_t(S) * Hkv * row_blocks;
    const int64_t a = (Lmax + kMinChunk - 1) / kMinChunk;
    const int64_t b = target_blocks() / units + 2;
    return int(a < b ? a : b);
}

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

// workspace: rotated q, partial outputs, partial (max, sum)
void ws_layout(int S, int T, int Hq, int Hkv, int Lmax, size_t &oq, size_t &oo, size_t &om,
               size_t &total) {
    const int G = Hq / Hkv;
    const int rows = T * G;
    const int chunks = max_chunks(S, Hkv, row_blocks_of(rows), Lmax);
    oq = 0;
    oo = align256(oq + size_t(S) * Hkv * rows * kD * 2);
    om = align256(oo + (chunks > 1 ? size_t(chunks) * S * Hkv * rows * kD * 4 : 0));
    total = align256(om + (chunks > 1 ? size_t(chunks) * S * Hkv * rows * 2 * 4 : 0));
}

bool aligned(const void *p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

size_t attention_lds(int W) { return size_t(kTilesPerBlock) * kTile * W * 4; }

hipError_t launch_attention(const AttnArgs &A, int row_blocks, hipStream_t st) {
    // the dynamic LDS bound, raised once per device to the most any launch
    // uses (W <= 32): with the static tiles that passes 64 KiB
    static std::atomic<uint32_t> raised{0};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return hipErrorInvalidDevice;
    const uint32_t bit = 1u << (dev & 31);
    if (!(raised.load() & bit)) {
        const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(attention_kernel),
                                                 hipFuncAttributeMaxDynamicSharedMemorySize,
                                                 int(attention_lds(32)));
        if (e != hipSuccess) return e;
        raised.fetch_or(bit);
    }
    hipLaunchKernelGGL(attention_kernel,
                       dim3(unsigned(A.S * A.Hkv), unsigned(row_blocks), unsigned(A.chunks)),
                       dim3(kWaves * 64), attention_lds(A.W), st, A);
    return hipGetLastError();
}

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
    A.tiles = tiles_of(A.rows);
    const int row_blocks = row_blocks_of(A.rows);
    A.ctx_cap = (max_ctx >= 0 && max_ctx < Lmax - T) ? max_ctx : Lmax - T;
    A.chunk = chunk_for(A.ctx_cap + T, S, Hkv, row_blocks);
    A.chunks = (A.ctx_cap + T + A.chunk - 1) / A.chunk;
    if (A.chunks > max_chunks(S, Hkv, row_blocks, Lmax)) return BASTION_EHIP;   // cannot happen
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
    A.rot_groups = (Hq + Hkv + kRotHeads - 1) / kRotHeads;
    A.val_groups = (Hkv + kValHeads - 1) / kValHeads;
    A.key_tiles = (T + 31) / 32 + 1;
    const hipStream_t st = static_cast<hipStream_t>(stream);
    hipLaunchKernelGGL(append_kernel,
                       dim3(unsigned(A.rot_groups + A.val_groups), unsigned(A.key_tiles), unsigned(S)),
                       dim3(256), 0, st, A);
    const hipError_t e = launch_attention(A, row_blocks, st);
    if (e != hipSuccess) return BASTION_EHIP;
    if (A.chunks > 1) {
        const int64_t waves = int64_t(S) * Hkv * A.rows;
        hipLaunchKernelGGL(combine_kernel, dim3(unsigned((waves + 3) / 4)), dim3(256), 0, st, A);
    }
    return hipGetLastError() == hipSuccess ? BASTION_OK : BASTION_EHIP;
}

}  // extern "C"
