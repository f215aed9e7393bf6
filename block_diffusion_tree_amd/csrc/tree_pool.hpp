// tree_pool.hpp -- the fast path of the best-first tree for one query
// (Bastion, Methodology 1-2 on the gist.science page: path score rho, pop
// order by rho; Methodology 3: the stop acts on the pop order).
//
// Best-first pops the N largest keys of the candidate tree, and the N-th
// largest key has rho >= t for any t with at least N nodes at or above it.
// So:
//   1. a lower bound t comes from a small family of real nodes whose rho is
//      cheap to form in parallel: every node of the first D complete levels
//      (D as large as fits 1024 nodes) plus, deeper, the top-1 path and every
//      node one deviation away from it.  The family's rho values go into a
//      1024-bin histogram of their float bits; t is the lower edge of the
//      first bin (from the top) where the count reaches N.
//   2. one wave enumerates, level by level, every node with rho >= t.  A
//      parent's children come in rank order with non-increasing rho (q is
//      sorted and float products are monotone), so each parent contributes
//      a prefix of its ranks.  Right after a level is generated its nodes
//      are ranked among themselves by (rho, token, parent's rank in its own
//      level); that is best-first's order inside one depth, since the pop
//      order of same-depth parents is their in-level order.  The key of a
//      node carries its parent's in-level rank, so keys are unique and
//      compare exactly as best-first does.  The caller falls back to the
//      exact round-by-round build if the pool outgrows its capacity.
//   3. every pool entry counts the keys larger than its own (all 256
//      threads, the comparisons split over the waves); the count is its pop
//      index minus one, and the first min(pool, N) entries are the tree.
#pragma once

#include "device_common.hpp"
#include "tree_rounds.hpp"

namespace bastion {

constexpr int kHistBins = 1024;     // float bits >> 20, rho in [0, 2)
constexpr int kFamilyLevels = 1024; // nodes of the complete top levels
constexpr int kMaxDigits = 10;      // levels of at most 1024 nodes (k >= 2)

// pool slots for a tree of tree_regs(nmax) = G registers of 64 nodes: twice
// the tree; none beyond G = 8 (the slot must fit the 10-bit key field)
__host__ __device__ constexpr int pool_cap(int G) { return G <= 8 ? 128 * G : 0; }
constexpr int kLvlFloats = kFamilyLevels;   // family scratch

typedef uint32_t pool_u32x4 __attribute__((ext_vector_type(4)));

struct PoolLds {
    uint64_t *key;     // [cap] by slot
    int32_t *par;      // [cap] parent slot, -1 for the root
    float *rho;        // [cap]
    int32_t *lrank;    // [cap] rank inside its level
    int32_t *pop;      // [cap] slot -> pop index (minus one while counting)
    uint32_t *hist;    // [kHistBins]
};


__device__ __forceinline__ void hist_add(uint32_t *hist, float rho) {
    uint32_t bin = __float_as_uint(rho) >> 20;
    bin = bin < kHistBins ? bin : kHistBins - 1;
    atomicAdd(hist + bin, 1u);
}

// inclusive prefix sum over the 64 lanes: DPP row shifts (zero fill) inside
// each 16-lane row, then the totals of the rows below
__device__ __forceinline__ uint32_t wave_incl_scan_u32(uint32_t v) {
    v += dpp32<0x111>(v);   // row_shr:1
    v += dpp32<0x112>(v);   // row_shr:2
    v += dpp32<0x114>(v);   // row_shr:4
    v += dpp32<0x118>(v);   // row_shr:8
    const uint32_t r0 = uint32_t(__builtin_amdgcn_readlane(int(v), 15));
    const uint32_t r1 = uint32_t(__builtin_amdgcn_readlane(int(v), 31));
    const uint32_t r2 = uint32_t(__builtin_amdgcn_readlane(int(v), 47));
    const int row = lane_id() >> 4;
    return v + (row > 0 ? r0 : 0u) + (row > 1 ? r1 : 0u) + (row > 2 ? r2 : 0u);
}

// Step 1, by the whole block.  qtab[(d-1)*kp + j] is q of rank j at depth d
// (rows padded with zeros to kp, a multiple of 8); q0col[d-1] is q of rank 0
// at depth d (kMaxB entries, zero past b).  lvl holds kFamilyLevels floats
// of scratch.  Returns (block-uniform) the lower bound t,
// 0 when the family holds fewer than n nodes.
template <int THREADS>
__device__ __forceinline__ float family_bound(const float *qtab, const float *q0col, int b, int k,
                                              int kp, int n, uint32_t *hist, float *lvl,
                                              float *s_out) {
    const int tid = threadIdx.x;
    for (int i = tid; i < kHistBins; i += THREADS) hist[i] = 0u;
    // complete levels 1..D (D as large as fits kFamilyLevels nodes)
    int D = 0, tot = 0, szD = 1;
    while (D < b && tot + szD * k <= kFamilyLevels) {
        szD *= k;
        tot += szD;
        ++D;
    }
    // parent index i / k of node i of a level (i < 1024, k <= 32:
    // (i * ceil(65536 / k)) >> 16 is exact)
    const uint32_t inv_k = (65536u + uint32_t(k) - 1u) / uint32_t(k);
    int off = 0, prev = 0, sz = 1;
    for (int d = 1; d <= D; ++d) {
        sz *= k;
        __syncthreads();   // level d-1 (and the zeroed histogram) complete
        for (int i = tid; i < sz; i += THREADS) {
            const int p = int((uint32_t(i) * inv_k) >> 16), j = i - p * k;
            const float rp = d == 1 ? 1.0f : lvl[prev + p];
            const float v = __fmul_rn(rp, qtab[(d - 1) * kp + j]);
            lvl[off + i] = v;
            hist_add(hist, v);
        }
        prev = off;
        off += sz;
    }
    // deeper than D: the top-1 path (pair index npair) and the paths leaving
    // it once, at depth e with rank j >= 1, then following rank 0.  Each
    // thread forms its path's rho from depth 1 in registers.
    if (D < b) {
        const int npair = b * (k - 1);
        float q0[kMaxB];
#pragma unroll
        for (int d = 0; d < kMaxB; ++d) q0[d] = q0col[d];
        for (int pi = tid; pi <= npair; pi += THREADS) {
            const int e = pi < npair ? pi / (k - 1) + 1 : b + 1;
            const int j = pi < npair ? pi - (e - 1) * (k - 1) + 1 : 0;
            const float qe = qtab[(e <= b ? e - 1 : 0) * kp + j];
            float r = 1.0f;
#pragma unroll
            for (int d = 1; d <= kMaxB; ++d) {
                if (d <= b) {
                    r = __fmul_rn(r, d == e ? qe : q0[d - 1]);
                    if (d > D && d >= (e <= b ? e : 1)) hist_add(hist, r);
                }
            }
        }
    }
    __syncthreads();
    if (tid < kWave) {
        // lane l owns bins 1008-16l .. 1023-16l; c[15] is its highest
        const int lane = tid;
        const pool_u32x4 *h4 =
            reinterpret_cast<const pool_u32x4 *>(hist + (kHistBins - 16 - 16 * lane));
        uint32_t c[16], own = 0;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const pool_u32x4 v = h4[i];
            c[4 * i + 0] = v[0];
            c[4 * i + 1] = v[1];
            c[4 * i + 2] = v[2];
            c[4 * i + 3] = v[3];
        }
#pragma unroll
        for (int i = 0; i < 16; ++i) own += c[i];
        const uint32_t incl = wave_incl_scan_u32(own);
        const uint64_t reach = __ballot(incl >= uint32_t(n));
        if (reach) {
            const int l = __ffsll((unsigned long long)reach) - 1;
            if (lane == l) {
                uint32_t acc = incl - own;
                int bin = kHistBins - 16 - 16 * lane;
                for (int i = 15; i >= 0; --i) {
                    acc += c[i];
                    if (acc >= uint32_t(n)) {
                        bin = kHistBins - 16 - 16 * lane + i;
                        break;
                    }
                }
                *s_out = __uint_as_float(uint32_t(bin) << 20);
            }
        } else if (lane == 0) {
            *s_out = 0.0f;
        }
    }
    __syncthreads();
    return *s_out;
}

// number of keys[f0..f1) greater than x; eight loads in flight at a time
__device__ __forceinline__ int count_greater(const uint64_t *keys, int f0, int f1, uint64_t x) {
    int r = 0;
    for (int f = f0; f < f1; f += 8) {
        uint64_t y[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) y[i] = keys[f + i < f1 ? f + i : f1 - 1];
#pragma unroll
        for (int i = 0; i < 8; ++i) r += (f + i < f1 && y[i] > x) ? 1 : 0;
    }
    return r;
}

// Step 2, by one wave: every node with rho >= t, parents before children.
// Lane l handles rank l % kk of parent l / kk of a chunk (kk: k rounded up
// to a power of two).  L.key has kPoolPad spare slots past cap, so a level
// can be ranked with unconditional loads of zero-padded keys.  Returns the
// node count, or -1 past cap.
constexpr int kPoolPad = 16;

__device__ int pool_enumerate(const PoolLds &L, const float *qtab, const int32_t *ttab, int b,
                              int k, int kp, float t, int cap) {
    const int lane = lane_id();
    const uint64_t lt = lanemask_lt();
    int sh = 0;
    while ((1 << sh) < k) ++sh;
    const int pl = lane >> sh, j = lane & ((1 << sh) - 1), ppc = kWave >> sh;
    const int jc = j < k ? j : k - 1;
    // counts are wave-uniform; readfirstlane keeps them in scalar registers
    int lo = 0, hi = 0, n = 0;
    bool over = false;
    float qj = qtab[jc];
    int tj = ttab[jc];
    for (int d = 1; d <= b; ++d) {
        const int np = __builtin_amdgcn_readfirstlane(d == 1 ? 1 : hi - lo);
        if (np == 0) break;
        // the next level's q and token, loaded one level ahead
        const int dn = d < b ? d : 0;
        const float qn = qtab[dn * kp + jc];
        const int tn = ttab[dn * kp + jc];
        const int n0 = n;
        if (lane < kPoolPad) L.key[n0 + lane] = 0;   // padding for the ranking below
        for (int p0 = 0; p0 < np; p0 += ppc) {
            const int p = p0 + pl;
            const bool valid = p < np && j < k;
            const int pc = lo + (p < np ? p : np - 1);
            const float rp = d == 1 ? 1.0f : L.rho[pc];
            const int pr = d == 1 ? 0 : L.lrank[pc];
            const float v = __fmul_rn(rp, qj);
            const bool ok = valid && v >= t;
            const uint64_t m = __ballot(ok);
            const int c = __builtin_amdgcn_readfirstlane(popc64(m));
            if (n + c > cap) {
                over = true;
                break;
            }
            if (ok) {
                const int s = n + popc64(m & lt);
                L.key[s] = tree_key(v, d, tj, pr);
                L.par[s] = d == 1 ? -1 : lo + p;
                L.rho[s] = v;
            }
            n = __builtin_amdgcn_readfirstlane(n + c);
        }
        if (over) break;
        wave_sync();
        // rank the level's nodes among themselves (keys are unique)
        const int m = n - n0;
        if (m == 1) {
            if (lane == 0) L.lrank[n0] = 0;
        } else if (m <= kPoolPad) {
            const uint64_t x = L.key[n0 + (lane < m ? lane : 0)];
            uint64_t y[kPoolPad];
#pragma unroll
            for (int i = 0; i < kPoolPad; ++i) y[i] = L.key[n0 + i];
            int r = 0;
#pragma unroll
            for (int i = 0; i < kPoolPad; ++i) r += y[i] > x ? 1 : 0;
            if (lane < m) L.lrank[n0 + lane] = r;
        } else {
            for (int s0 = n0; s0 < n; s0 += kWave) {
                const int s = s0 + lane;
                const uint64_t x = s < n ? L.key[s] : ~uint64_t(0);
                const int r = count_greater(L.key, n0, n, x);
                if (s < n) L.lrank[s] = r;
            }
        }
        wave_sync();
        lo = hi;
        hi = n;
        qj = qn;
        tj = tn;
    }
    return over ? -1 : n;
}

// Step 3, by the whole block (n >= 1).  L.pop[s] receives the pop index of
// slot s; the pop-order records 1..cnt (cnt =
// min(n, nmax)) go to par/dep/tok/rho.  Elements are taken 64 per wave; when
// there are fewer than four such groups the waves of a group split the
// comparisons and add their counts.  Returns cnt.
template <int THREADS>
__device__ __forceinline__ int pool_rank(const PoolLds &L, int n, int nmax, int32_t *par,
                                         int32_t *dep, int32_t *tok, float *rho) {
    constexpr int W = THREADS / kWave;
    const int tid = threadIdx.x, lane = tid & (kWave - 1), wv = tid / kWave;
    const int groups = (n + kWave - 1) / kWave;
    const int split = groups >= W ? 1 : W / groups;   // waves per group
    const int chunk = (n + split - 1) / split;
    if (split > 1) {
        for (int e = tid; e < n; e += THREADS) L.pop[e] = 0;
        __syncthreads();
    }
    for (int g0 = wv / split; g0 < groups; g0 += W / split) {
        const int e = g0 * kWave + lane;
        const int part = wv % split;
        const int f0 = part * chunk, f1 = f0 + chunk < n ? f0 + chunk : n;
        if (e < n) {
            const int r = count_greater(L.key, f0, f1, L.key[e]);
            if (split == 1) L.pop[e] = r + 1;
            else if (r) atomicAdd(L.pop + e, r);
        }
    }
    __syncthreads();
    const int cnt = n < nmax ? n : nmax;
    for (int e = tid; e < n; e += THREADS) {
        const int pe = L.pop[e] + (split == 1 ? 0 : 1);
        if (pe <= cnt) {
            const int ps = L.par[e];
            const uint64_t x = L.key[e];
            par[pe] = ps < 0 ? 0 : L.pop[ps] + (split == 1 ? 0 : 1);
            dep[pe] = tree_key_depth(x);
            tok[pe] = tree_key_token(x);
            rho[pe] = tree_key_rho(x);
        }
    }
    return cnt;
}

}  // namespace bastion
