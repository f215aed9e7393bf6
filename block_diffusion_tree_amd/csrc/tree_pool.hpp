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
//   2. every node with rho >= t, level by level.  A parent's children come
//      in rank order with non-increasing rho (q is sorted and float products
//      are monotone), so each parent contributes a prefix of its ranks.
//      Such pools are a few parallel chains that branch at uncertain
//      positions: one wave follows them, a chain per lane in registers,
//      while none branches; from the first level where one branches the
//      whole block expands the levels from LDS.  The caller falls back to
//      the exact round-by-round build if the pool outgrows its capacity.
//   3. every pool node's pop index is one plus the number of keys that pop
//      before it, counted by rho bins (bucket_rank); nodes that agree on
//      (rho, depth, token) pop in their parents' order, found by walking up
//      both parent chains to the first ancestors that differ.  The first
//      min(pool, N) are the tree.
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
// the trees' own launch, with LDS to spare: four slots per tree node up to
// G = 4 (1024 slots, what the field holds), so that loose bounds of deep
// trees stay on the pool path
__host__ __device__ constexpr int pool_cap_wide(int G) { return G <= 4 ? 256 * G : pool_cap(G); }
constexpr int kLvlFloats = kFamilyLevels;   // family scratch

typedef uint32_t pool_u32x4 __attribute__((ext_vector_type(4)));
typedef float pool_f32x4 __attribute__((ext_vector_type(4)));
typedef int32_t pool_i32x4 __attribute__((ext_vector_type(4)));

struct PoolLds {
    uint64_t *key;     // [cap] tree_key (the pool's parent field is 0; the
                       // family's holds the node's family identity)
    int32_t *par;      // [cap] parent slot, -1 for the root (pool path)
    float *rho;        // [cap] (pool path)
    int32_t *lrank;    // [cap] adjacent to rho: with it, bucket_rank's
                       // placement of up to cap 64-bit keys
    int32_t *pop;      // [cap] pop index
    uint32_t *hist;    // [kHistBins]
};


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

// Where the one-wave enumeration stops: the first level where a chain
// branches (its parents [lo, hi), d its depth); the block continues there
// (pool_wide).
struct PoolWide {
    int lo, hi, d;
    bool wide;
};

// Step 2, by one wave: every node with rho >= t, parents before children,
// up to the first level where a chain branches (then w.wide is set and the
// block goes on with pool_wide).  Returns the node count so far, or -1 past
// cap.
__device__ int pool_enumerate(const PoolLds &L, const float *qtab, const int32_t *ttab, int b,
                              int k, int kp, float t, int cap, PoolWide &w) {
    const int lane = lane_id();
    const uint64_t lt = lanemask_lt();
    // lane l < 32 holds q of rank 0 at depth l+1, lane 32 + l that of rank 1;
    // tok0: token of rank 0 at depth l+1
    const int dl = lane & 31;
    const int dr = dl < b ? dl : 0;
    const float colq = qtab[dr * kp + (lane >= 32 && k > 1 ? 1 : 0)];
    const int tok0 = ttab[dr * kp];
    // level 1: the root's children are the ranks with q >= t, a prefix, and
    // their in-level order is the rank order
    const float q1v = lane < k ? qtab[lane] : 0.0f;
    const bool ok1 = lane < k && q1v >= t;
    int n = __builtin_amdgcn_readfirstlane(popc64(__ballot(ok1)));
    if (n > cap) return -1;
    if (ok1) {
        L.key[lane] = tree_key(q1v, 1, ttab[lane], 0);
        L.par[lane] = -1;
        L.rho[lane] = q1v;
    }
    bool alive = ok1;
    float rho = q1v;
    int slot = lane;
    int lo = 0, hi = n, d = 2;
    bool wide = false, over = false;
    // chains in lanes
    for (; d <= b && hi > lo; ++d) {
        const float q0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(colq), d - 1));
        const float q1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(colq), 32 + d - 1));
        const float v0 = __fmul_rn(rho, q0);
        const bool ok0 = alive && v0 >= t;
        const bool br = alive && k > 1 && __fmul_rn(rho, q1) >= t;
        if (__ballot(br) == 0) {
            // no chain branches: each continues with its rank-0 child
            const uint64_t m = __ballot(ok0);
            const int c = __builtin_amdgcn_readfirstlane(popc64(m));
            if (n + c > cap) {
                over = true;
                break;
            }
            const int s = n + popc64(m & lt);
            const int t0 = __builtin_amdgcn_readlane(tok0, d - 1);
            if (ok0) {
                L.key[s] = tree_key(v0, d, t0, 0);
                L.par[s] = slot;
                L.rho[s] = v0;
            }
            alive = ok0;
            rho = v0;
            slot = s;
            lo = n;
            n = __builtin_amdgcn_readfirstlane(n + c);
            hi = n;
        } else {
            // a chain branches: the block takes over at this level
            wide = true;
            break;
        }
    }
    w.lo = lo;
    w.hi = hi;
    w.d = d;
    w.wide = wide;
    return over ? -1 : n;
}

// Step 2 continued, by the whole block, from the first branching level: each
// thread takes rank j (of k rounded up to a power of two) of one parent;
// the level's qualifying children get slots through a block-wide prefix of
// the waves' ballots (slot order within a level is free: step 3 orders the
// keys).  Returns the node count, or -1 past cap (block-uniform).  Ends
// with a barrier.
template <int THREADS>
__device__ int pool_wide(const PoolLds &L, const float *qtab, const int32_t *ttab, int b, int k,
                         int kp, float t, int cap, int lo, int hi, int d, int n) {
    constexpr int W = THREADS / kWave;
    __shared__ int s_cnt[W];
    const int tid = threadIdx.x, lane = tid & (kWave - 1);
    const int wv = __builtin_amdgcn_readfirstlane(tid / kWave);
    const uint64_t lt = lanemask_lt();
    int sh = 0;
    while ((1 << sh) < k) ++sh;
    const int pl = tid >> sh, j = tid & ((1 << sh) - 1), ppc = THREADS >> sh;
    const int jc = j < k ? j : k - 1;
    for (; d <= b && hi > lo; ++d) {
        const int np = hi - lo;
        const float qj = qtab[(d - 1) * kp + jc];
        const int tj = ttab[(d - 1) * kp + jc];
        const int n0 = n;
        for (int p0 = 0; p0 < np; p0 += ppc) {
            const int p = p0 + pl;
            const bool valid = p < np && j < k;
            const int pc = lo + (p < np ? p : np - 1);
            const float v = __fmul_rn(L.rho[pc], qj);
            const bool ok = valid && v >= t;
            const uint64_t m = __ballot(ok);
            if (lane == 0) s_cnt[wv] = popc64(m);
            __syncthreads();
            int before = 0, tot = 0;
#pragma unroll
            for (int x = 0; x < W; ++x) {
                const int c = s_cnt[x];
                before += x < wv ? c : 0;
                tot += c;
            }
            if (n + tot > cap) return -1;
            if (ok) {
                const int s = n + before + popc64(m & lt);
                L.key[s] = tree_key(v, d, tj, 0);
                L.par[s] = pc;
                L.rho[s] = v;
            }
            n += tot;
            __syncthreads();   // the counts are read; the level's keys are written
        }
        lo = n0;
        hi = n;
    }
    return n;
}

// Pop counts of n keys by rho bins, whole block (1 <= n <= 1024; every
// key's rho >= t; pop zero on entry): pop[e] = the number of keys that pop
// before key e.  The
// bins (bc: kHistBins counters, zero on entry, left non-zero) split [t, 1]
// as finely as 1024 bins allow (rho bits >> (20 - ex), less t's bin); every
// key of a higher bin pops first, and a key is compared only with the keys
// of its own bin, which are first placed together in sb (n entries) with
// their indices: in sx, or, when sx is null, in the keys' low 10 bits (which
// the comparisons then ignore).  Keys equal but for their low 10 bits pop
// in the order before(x, e, y, f) gives (does key y, index f, pop before
// key x, index e?).
// Up to kPairMax keys are instead compared all with all, each key's count
// split over THREADS / n threads (pop zero on entry; bc untouched).
constexpr int kPairMax = 64;

template <int THREADS, typename Tie>
__device__ __forceinline__ void bucket_rank(const uint64_t *key, int n, float t, uint32_t *bc,
                                            uint64_t *sb, int32_t *sx, int32_t *pop, Tie before) {
    const int tid = threadIdx.x, lane = tid & (kWave - 1);
    if (n <= kPairMax) {
        const int P = THREADS / n;   // parts per key
        const int chunk = (n + P - 1) / P;
        const int e = tid % n, part = tid / n;
        if (part < P) {
            const uint64_t x = key[e], xm = x | 1023u;
            const int f0 = part * chunk, f1 = f0 + chunk < n ? f0 + chunk : n;
            int gt = 0;
            uint64_t ties = 0;   // chunk <= n <= 64
            for (int f = f0; f < f1; ++f) {
                const uint64_t ym = key[f] | 1023u;
                gt += ym > xm ? 1 : 0;
                ties |= uint64_t(ym == xm && f != e) << (f - f0);
            }
            // equal keys after the scan, one partner per lane at a time: the
            // wave walks parents as often as its lane with the most ties
            while (ties) {
                const int f = f0 + __builtin_ctzll(ties);
                ties &= ties - 1;
                if (before(x, e, key[f], f)) ++gt;
            }
            if (gt) atomicAdd(pop + e, gt);
        }
        __syncthreads();
        return;
    }
    constexpr int kPer = 1024 / THREADS > 0 ? 1024 / THREADS : 1;
    const int tbin = int(__float_as_uint(t) >> 20);
    const int R = 1017 - tbin;   // bins up to rho = 1 (bin 1016)
    int ex = 0;
    while (ex < 20 && (R << (ex + 1)) <= kHistBins) ++ex;
    int arr[kPer], fb[kPer];
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
        const int e = tid + i * THREADS;
        fb[i] = 0;
        arr[i] = 0;
        if (e < n) {
            const uint32_t rb = uint32_t(key[e] >> 34) - 1u;   // rho's bits
            fb[i] = min(max(int(rb >> (20 - ex)) - (tbin << ex), 0), kHistBins - 1);
            arr[i] = int(atomicAdd(bc + fb[i], 1u));
        }
    }
    __syncthreads();
    if (tid < kWave) {
        // bins 16 lane .. 16 lane + 15: counts -> keys in higher bins
        pool_u32x4 *b4 = reinterpret_cast<pool_u32x4 *>(bc + 16 * lane);
        uint32_t c[16], own = 0;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const pool_u32x4 v = b4[i];
#pragma unroll
            for (int j = 0; j < 4; ++j) c[4 * i + j] = v[j];
        }
#pragma unroll
        for (int i = 0; i < 16; ++i) own += c[i];
        const uint32_t incl = wave_incl_scan_u32(own);
        uint32_t run = uint32_t(__builtin_amdgcn_readlane(int(incl), kWave - 1)) - incl;
#pragma unroll
        for (int i = 15; i >= 0; --i) {
            const uint32_t ci = c[i];
            c[i] = run;
            run += ci;
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            pool_u32x4 v;
#pragma unroll
            for (int j = 0; j < 4; ++j) v[j] = c[4 * i + j];
            b4[i] = v;
        }
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
        const int e = tid + i * THREADS;
        if (e < n) {
            const int slot = int(bc[fb[i]]) + arr[i];
            if (sx) {
                sb[slot] = key[e];
                sx[slot] = e;
            } else {
                sb[slot] = (key[e] & ~uint64_t(1023)) | uint64_t(e);
            }
        }
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
        const int e = tid + i * THREADS;
        if (e < n) {
            const uint64_t x = key[e], xm = x | 1023u;
            const int f0 = int(bc[fb[i]]);
            const int f1 = fb[i] > 0 ? int(bc[fb[i] - 1]) : n;
            const int self = f0 + arr[i];   // where the placement put key e
            int gt = f0;
            // 64 places of the bin at a time: count the larger keys, mark the
            // equal ones (same rho, depth and token), then order those by
            // their parents, one partner per lane at a time
            for (int w0 = f0; w0 < f1; w0 += kWave) {
                const int w1 = w0 + kWave < f1 ? w0 + kWave : f1;
                uint64_t ties = 0;
                for (int f = w0; f < w1; ++f) {
                    const uint64_t ym = sb[f] | 1023u;
                    gt += ym > xm ? 1 : 0;
                    ties |= uint64_t(ym == xm && f != self) << (f - w0);
                }
                while (ties) {
                    const int f = w0 + __builtin_ctzll(ties);
                    ties &= ties - 1;
                    const uint64_t y = sb[f];
                    if (before(x, e, y, sx ? sx[f] : int(y & 1023u))) ++gt;
                }
            }
            pop[e] = gt;
        }
    }
    __syncthreads();
}

// Step 3, by the whole block (1 <= n <= 1024; L.hist zero on entry): the pop
// index of every pool node (L.pop holds the number of nodes before it) and
// the pop-order records 1..cnt (cnt = min(n, nmax)) in par/dep/tok/rho, the
// ranks by rho bins (bucket_rank).  Returns cnt.
template <int THREADS>
__device__ __forceinline__ int pool_rank(const PoolLds &L, int n, int nmax, float t,
                                         int32_t *par, int32_t *dep, int32_t *tok, float *rho) {
    const int tid = threadIdx.x;
    // equal (rho, depth, token): the parents' order, from the first
    // ancestors (same depth) whose keys differ; L.rho and L.lrank (adjacent,
    // free once the pool is enumerated) hold the binned keys
    bucket_rank<THREADS>(L.key, n, t, L.hist, reinterpret_cast<uint64_t *>(L.rho), nullptr, L.pop,
                         [&](uint64_t, int e, uint64_t, int f) {
                             int a = L.par[e], c = L.par[f];
                             while (a != c && a >= 0 && c >= 0) {
                                 const uint64_t ka = L.key[a] | 1023u, kc = L.key[c] | 1023u;
                                 if (ka != kc) return kc > ka;
                                 a = L.par[a];
                                 c = L.par[c];
                             }
                             return false;
                         });
    const int cnt = n < nmax ? n : nmax;
    for (int e = tid; e < n; e += THREADS) {
        const int pe = L.pop[e] + 1;
        if (pe <= cnt) {
            const int ps = L.par[e];
            const uint64_t x = L.key[e];
            par[pe] = ps < 0 ? 0 : L.pop[ps] + 1;
            dep[pe] = tree_key_depth(x);
            tok[pe] = tree_key_token(x);
            rho[pe] = tree_key_rho(x);
        }
    }
    return cnt;
}

}  // namespace bastion
