// tree_family.hpp -- the pool of the best-first tree for one query taken from
// a family of real nodes (Bastion, Methodology 1-2 on the gist.science page:
// path score rho = product of the position marginals along the path, pop
// order by rho).
//
// Best-first pops the N largest keys of the candidate tree.  The family is
// every node of the first D complete levels (D as large as fits 1024 nodes)
// plus, deeper, the top-1 path and every path that leaves it once (rank
// j >= 1 at depth e, rank 0 elsewhere).  Its rho values are formed in
// parallel, in the same float order as best-first (depth 1 first, one
// rounding per factor).
//   family_bound:  a 1024-bin histogram of the family's float bits gives t,
//                  the lower edge of the first bin (from the top) where the
//                  count reaches N; at least N real nodes have rho >= t, so
//                  the tree is among the nodes with rho >= t (the pool).
//   family_select: every family node with rho >= t gets a slot.  A node
//                  outside the family descends from a child of a family node
//                  that is not in the family, and rho never grows along a
//                  path, so if none of those children reaches t the family
//                  holds the whole pool.  Otherwise the caller enumerates the
//                  pool level by level (tree_pool.hpp).
//   family_rank:   a node's pop index is one plus the number of pool keys
//                  that pop before it: every key of a higher rho bin, and
//                  those of its own bin that compare above it; equal (rho,
//                  depth, token) keys are ordered as best-first orders them,
//                  by their parents, which the nodes' family identities
//                  resolve directly.
//
// All three run branch-light on every wave of the block: one wave's
// dependent LDS round trips and VALU-to-scalar transitions dominate here,
// so walks keep their state in VALU registers, read per-depth columns with
// 16-byte broadcast loads, and lanes without a node store to a sink slot.
#pragma once

#include "device_common.hpp"
#include "tree_pool.hpp"

namespace bastion {

constexpr int kColLen = kMaxB + 4;                   // FamilyCols entries
constexpr int kFamGroups = kFamilyLevels / kWave;    // ballot groups of complete nodes
constexpr int kFamRounds = 4;                        // path rounds of 256 (b * (k - 1) < 1024)
constexpr int kPoolPad = 8;                          // zero keys after the pool's last slot

// Per-depth columns of the q / token tables (kColLen entries each, zero past
// the last valid depth, 16-byte aligned):
//   q0[x]  q of rank 0 at depth x + 1
//   q1n[x] q of rank 1 at depth x + 2
//   t0[x]  token of rank 0 at depth x + 1
struct FamilyCols {
    const float *q0, *q1n;
    const int32_t *t0;
};

// LDS scratch of family_select
struct FamilyWork {
    uint64_t *cmask;   // [kFamGroups] qualifying complete-level nodes, 64 per group
    int32_t *gpre;     // [kFamGroups] complete nodes before each group
    int32_t *wtot;     // [kFamRounds * waves] path-node counts per (round, wave)
    int32_t *flag;     // [4] escape flag (zero on entry); the top-1 path's
                       // offset inside its (round, wave), that entry, its
                       // first slot
};

// Complete top levels of the family: D levels (as many as fit kFamilyLevels
// nodes), tot nodes.  Level d holds k^d nodes from index k + ... + k^(d-1).
__host__ __device__ inline int family_depth(int b, int k, int &tot) {
    int D = 0, szD = 1;
    tot = 0;
    while (D < b && tot + szD * k <= kFamilyLevels) {
        szD *= k;
        tot += szD;
        ++D;
    }
    return D;
}

__device__ __forceinline__ int hist_bin(float rho) {
    const uint32_t bin = __float_as_uint(rho) >> 20;
    return int(bin < kHistBins ? bin : kHistBins - 1);
}

// x / k for 0 <= x < 1024 and 1 <= k <= 32 (inv = ceil(65536 / k))
__device__ __forceinline__ int div_small(int x, uint32_t inv) {
    return int((uint32_t(x) * inv) >> 16);
}

// Pool keys of the family path: tree_key's fields with the low field holding
// the node's family identity instead of a parent: its index inside its level
// for a node of the complete levels (depth <= D); for a path node 0 (the
// top-1 path) or (e - 1) * 32 + j (rank j >= 1 at depth e).
__device__ __forceinline__ uint64_t fam_key(float rho, int d, int tok, int id) {
    return tree_key(rho, d, tok, 1023) | uint64_t(id);
}
__device__ __forceinline__ int fam_id(uint64_t key) { return int(key & 1023u); }

// A path leaving the top-1 path once: pi = (e - 1)(k - 1) + j - 1 for rank
// j >= 1 at depth e; pi == npair is the top-1 path itself.  Family nodes of
// a path are its nodes at depths >= dstart = max(D + 1, e).
struct Chain {
    bool valid, top;
    int e, j, dstart;
    float qe;
    int te;
};
__device__ __forceinline__ Chain make_chain(int pi, int npair, int b, int k, int kp, int D,
                                            uint32_t inv_km1, const float *qtab,
                                            const int32_t *ttab) {
    Chain c;
    c.valid = pi <= npair;
    c.top = pi == npair;
    const bool dev = c.valid && !c.top;
    c.e = dev ? div_small(pi, inv_km1) + 1 : b + 1;
    c.j = dev ? pi - (c.e - 1) * (k - 1) + 1 : 0;
    c.dstart = (!c.top && c.e > D) ? c.e : D + 1;
    const int row = dev ? c.e - 1 : 0;
    c.qe = qtab[row * kp + c.j];
    c.te = ttab[row * kp + c.j];
    return c;
}

// What family_bound's path walk leaves in registers for family_select when
// one thread holds one path (b * (k - 1) < THREADS): the path's rho at every
// depth, rho one depth above its first family node, and the largest rho of a
// child off the path (rank 1 one depth down) below a family node.
struct FamRegs {
    float rv[kMaxB];
    float rp, escm;
};

// Step 1, by the whole block.  hist (kHistBins + kWave bins) must be zero
// and visible to the block.  Writes the complete levels' rho to lvl[0, tot).
// Returns the lower bound t (every wave reads the histogram itself), 0 when
// the family holds fewer than n nodes; with bound2, also the bound of n2
// nodes.
// TWO: also count the nodes of the paths that take rank 1 at two depths
// (real nodes outside the family: they only tighten the bound)
template <int THREADS, bool TWO = false>
__device__ __forceinline__ float family_bound(const float *qtab, const int32_t *ttab,
                                              const FamilyCols &F, int b, int k, int kp, int n,
                                              uint32_t *hist, float *lvl, FamRegs &R,
                                              uint64_t *st = nullptr, int n2 = 0,
                                              float *bound2 = nullptr) {
    (void)st;
    constexpr int W = THREADS / kWave;
    const int tid = threadIdx.x, lane = lane_id();
    const int wv = __builtin_amdgcn_readfirstlane(tid / kWave);
    b = __builtin_amdgcn_readfirstlane(b);
    int tot;
    const int D = family_depth(b, k, tot);
    const uint32_t inv_k = (65536u + uint32_t(k) - 1u) / uint32_t(k);
    // complete levels, level by level inside each wave: the levels above D in
    // every wave (identical values), level D split over the waves; the
    // histogram takes levels above D from wave 0 only
    int off = 0, prev = 0, sz = 1;
    for (int d = 1; d <= D; ++d) {
        sz *= k;
        const bool last = d == D;
        const int i0 = last ? wv * kWave : 0, step = last ? W * kWave : kWave;
        const bool counts = last || wv == 0;
        for (int i = i0 + lane; i < sz; i += step) {
            const int p = div_small(i, inv_k), j = i - p * k;
            const float rp = d == 1 ? 1.0f : lvl[prev + p];
            const float v = __fmul_rn(rp, qtab[(d - 1) * kp + j]);
            lvl[off + i] = v;
            if (counts) atomicAdd(hist + hist_bin(v), 1u);
        }
        wave_sync();
        prev = off;
        off += sz;
    }
    BASTION_STAMP(st, 10);
    // deeper than D: the top-1 path and the paths leaving it once
    if (D < b) {
        const int npair = b * (k - 1);
        const uint32_t inv_km1 = (65536u + uint32_t(k - 1) - 1u) / uint32_t(k - 1);
        if (npair < THREADS) {
            // one path per thread, kept in registers for family_select
            const Chain c = make_chain(tid, npair, b, k, kp, D, inv_km1, qtab, ttab);
            const int lo = c.valid ? c.dstart : kMaxB + 1;
            float r = 1.0f, rp = 1.0f, em = 0.0f;
#pragma unroll
            for (int i = 0; i < kMaxB; ++i) R.rv[i] = 0.0f;   // depths past b: below any t > 0
#pragma unroll
            for (int g4 = 0; g4 < kMaxB / 4; ++g4) {
                const int d0 = 1 + 4 * g4;
                if (d0 <= b) {
                    const pool_f32x4 q4 = *reinterpret_cast<const pool_f32x4 *>(F.q0 + d0 - 1);
                    const pool_f32x4 n4 = *reinterpret_cast<const pool_f32x4 *>(F.q1n + d0 - 1);
#pragma unroll
                    for (int u = 0; u < 4; ++u) {
                        const int d = d0 + u;
                        if (d <= b) {
                            rp = d == c.dstart ? r : rp;
                            r = __fmul_rn(r, d == c.e ? c.qe : q4[u]);
                            R.rv[4 * g4 + u] = r;
                            em = d >= lo ? fmaxf(em, __fmul_rn(r, n4[u])) : em;
                            if (d > D) atomicAdd(hist + (d >= lo ? hist_bin(r) : kHistBins + lane), 1u);
                        }
                    }
                }
            }
            R.rp = rp;
            R.escm = em;
        }
        for (int p0 = 0; npair >= THREADS && p0 <= npair; p0 += THREADS) {
            const Chain c = make_chain(p0 + tid, npair, b, k, kp, D, inv_km1, qtab, ttab);
            const int lo = c.valid ? c.dstart : kMaxB + 1;
            float r = 1.0f;
            for (int d0 = 1; d0 <= b; d0 += 4) {
                const pool_f32x4 q4 = *reinterpret_cast<const pool_f32x4 *>(F.q0 + d0 - 1);
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    const int d = d0 + u;
                    if (d <= b) {
                        r = __fmul_rn(r, d == c.e ? c.qe : q4[u]);
                        if (d > D) atomicAdd(hist + (d >= lo ? hist_bin(r) : kHistBins + lane), 1u);
                    }
                }
            }
        }
    }
    if (TWO && D < b && k > 1) {
        // rank 1 at depths e1 < e2, rank 0 elsewhere: the nodes at depths
        // >= e2 below the complete levels, with rho in best-first's order
        for (int pi = tid; pi < b * b; pi += THREADS) {
            const int e1 = pi / b + 1, e2 = pi - (e1 - 1) * b + 1;
            if (e1 < e2) {
                float r = 1.0f;
                for (int d = 1; d <= b; ++d) {
                    const float q = (d == e1 || d == e2) ? qtab[(d - 1) * kp + 1] : F.q0[d - 1];
                    r = __fmul_rn(r, q);
                    if (d >= e2 && d > D) atomicAdd(hist + hist_bin(r), 1u);
                }
            }
        }
    }
    __syncthreads();
    BASTION_STAMP(st, 11);
    // lane l owns bins 1008-16l .. 1023-16l; cb[15] is its highest
    const pool_u32x4 *h4 = reinterpret_cast<const pool_u32x4 *>(hist + (kHistBins - 16 - 16 * lane));
    uint32_t cb[16], own = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const pool_u32x4 v = h4[i];
        cb[4 * i + 0] = v[0];
        cb[4 * i + 1] = v[1];
        cb[4 * i + 2] = v[2];
        cb[4 * i + 3] = v[3];
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) own += cb[i];
    const uint32_t incl = wave_incl_scan_u32(own);
    // The lower edge of the first bin (from the top) where the count reaches
    // m; 0 when the family holds fewer than m nodes.  The count from the top
    // grows toward a lane's lower bins, so on the first lane whose inclusive
    // count reaches m the bin is 15 - (its bins still below m) in its block.
    const uint32_t m1 = uint32_t(n), m2 = uint32_t(n2 >= 1 ? n2 : n);
    uint32_t acc = incl - own;
    int below1 = 0, below2 = 0;
#pragma unroll
    for (int i = 15; i >= 0; --i) {
        acc += cb[i];
        below1 += acc < m1 ? 1 : 0;
        below2 += acc < m2 ? 1 : 0;
    }
    const int base = kHistBins - 1 - 16 * lane;
    auto edge = [&](uint32_t m, int below) -> float {
        const uint64_t reach = __ballot(incl >= m);
        if (reach == 0) return 0.0f;
        const int l = __builtin_amdgcn_readfirstlane(__ffsll((unsigned long long)reach) - 1);
        const int bin = __builtin_amdgcn_readlane(base - below, l);
        return __uint_as_float(uint32_t(bin) << 20);
    };
    if (bound2) *bound2 = n2 >= 1 ? edge(m2, below2) : 0.0f;
    return edge(m1, below1);
}

// Step 2, by the whole block, after family_bound (lvl holds the complete
// levels' rho).  Slots: the complete-level nodes in index order, then the
// paths' nodes (path order, depth order; the top-1 path is path npair).
// Each slot's key is fam_key(rho, depth, token, identity); Wk.gpre and
// Wk.flag[3] keep what family_rank needs to link parents (FamGeom).
// Returns the pool size n, block-uniform; -1 if the family does not hold the
// pool.  Slots past cap are not written (the caller falls back when
// n > cap); lanes without a node store to slot cap + kPoolPad + lane, and
// slots n .. n + kPoolPad - 1 get zero keys.  Ends with a barrier.
template <int THREADS>
__device__ int family_select(const PoolLds &L, const float *qtab, const int32_t *ttab,
                             const FamilyCols &F, const FamilyWork &Wk, const FamRegs &R, int b,
                             int k, int kp, float t, int cap, const float *lvl,
                             uint64_t *st = nullptr) {
    (void)st;
    constexpr int W = THREADS / kWave, MC = kFamilyLevels / THREADS;
    static_assert(kFamilyLevels % THREADS == 0 && MC * W == kFamGroups, "family groups");
    const int tid = threadIdx.x, lane = lane_id();
    const int wv = __builtin_amdgcn_readfirstlane(tid / kWave);
    const uint64_t lt = lanemask_lt();
    b = __builtin_amdgcn_readfirstlane(b);
    int tot;
    const int D = family_depth(b, k, tot);
    const uint32_t inv_k = (65536u + uint32_t(k) - 1u) / uint32_t(k);
    int kD = 1;
    for (int x = 0; x < D; ++x) kD *= k;
    const int firstD = tot - kD;   // index of node (D, 0)
    const int rowD = D < b ? D : 0;
    // t = 0 (a family smaller than n): every node qualifies, so the family
    // holds the pool only if it is the whole tree
    if (!(t > 0.0f) && D < b) return -1;
    bool esc = false;

    // complete levels: one ballot mask per 64 nodes (group m * W + wave)
    float cv[MC];
    uint64_t cm[MC];
#pragma unroll
    for (int m = 0; m < MC; ++m) {
        const int g = tid + m * THREADS;
        cv[m] = lvl[g];
        const bool ok = m * THREADS < tot && g < tot && cv[m] >= t;
        cm[m] = __ballot(ok);
        if (lane == 0) Wk.cmask[m * W + wv] = cm[m];
        if (ok && D < b && g >= firstD) {
            // level D: children outside the family are every rank past one
            // deviation from the top-1 path, rank 0 too past two
            int nz = 0, x = g - firstD;
            for (int y = 0; y < D; ++y) {
                const int xq = div_small(x, inv_k);
                nz += x != xq * k ? 1 : 0;
                x = xq;
            }
            if (nz >= 1 && __fmul_rn(cv[m], qtab[rowD * kp + (nz >= 2 ? 0 : 1)]) >= t) esc = true;
        }
    }

    // one path per lane (the top-1 path too): rho never grows with depth, so
    // a path's qualifying nodes are the depths dstart .. last
    const int npair = D < b ? b * (k - 1) : -1;
    const int rounds = npair >= 0 ? npair / THREADS + 1 : 0;
    const uint32_t inv_km1 = k > 1 ? (65536u + uint32_t(k - 1) - 1u) / uint32_t(k - 1) : 1u;
    const int bfull = b & ~3;
    int cn[kFamRounds], cbase[kFamRounds];
    float crp[kFamRounds];
#pragma unroll
    for (int rd = 0; rd < kFamRounds; ++rd) {
        cn[rd] = 0;
        cbase[rd] = 0;
        crp[rd] = 1.0f;
        if (rd < rounds) {
            const Chain c = make_chain(rd * THREADS + tid, npair, b, k, kp, D, inv_km1, qtab, ttab);
            // every per-depth test is one compare against a lane value: the
            // deepest qualifying depth (last), the deepest node whose rank-1
            // child qualifies (escd; q1n is zero past the last depth and
            // t > 0), rho at dstart - 1 (rp)
            float rp = 1.0f;
            int last = 0;
            bool escp = false;
            if (rounds == 1) {
                // the path's values from family_bound's walk (zero past b,
                // and t > 0 here); rho never grows along the path
                if (b <= 16) {
#pragma unroll
                    for (int i = 0; i < 16; ++i) last += R.rv[i] >= t ? 1 : 0;
                } else {
#pragma unroll
                    for (int i = 0; i < kMaxB; ++i) last += R.rv[i] >= t ? 1 : 0;
                }
                rp = R.rp;
                escp = R.escm >= t;
            } else {
                float r = 1.0f;
                int escd = 0;
                auto step = [&](int d, float q, float qn) {
                    rp = d == c.dstart ? r : rp;
                    r = __fmul_rn(r, d == c.e ? c.qe : q);
                    last = r >= t ? d : last;
                    escd = __fmul_rn(r, qn) >= t ? d : escd;
                };
                for (int d0 = 1; d0 <= bfull; d0 += 4) {
                    const pool_f32x4 q4 = *reinterpret_cast<const pool_f32x4 *>(F.q0 + d0 - 1);
                    const pool_f32x4 n4 = *reinterpret_cast<const pool_f32x4 *>(F.q1n + d0 - 1);
#pragma unroll
                    for (int u = 0; u < 4; ++u) step(d0 + u, q4[u], n4[u]);
                }
                for (int d = bfull + 1; d <= b; ++d) step(d, F.q0[d - 1], F.q1n[d - 1]);
                escp = escd >= c.dstart;
            }
            // the top-1 path's children off it are one-deviation paths
            const bool dev = c.valid && !c.top;
            cn[rd] = (c.valid && last >= c.dstart) ? last - c.dstart + 1 : 0;
            crp[rd] = rp;
            esc = esc || (dev && escp);
            const uint32_t incl = wave_incl_scan_u32(uint32_t(cn[rd]));
            cbase[rd] = int(incl) - cn[rd];
            if (lane == kWave - 1) Wk.wtot[rd * W + wv] = int(incl);
            if (c.top) {
                Wk.flag[1] = cbase[rd];
                Wk.flag[2] = rd * W + wv;
            }
        }
    }
    if (esc) Wk.flag[0] = 1;
    __syncthreads();
    BASTION_STAMP(st, 12);
    if (Wk.flag[0] != 0) return -1;

    // slot bases: complete nodes by group prefix, paths by (round, wave)
    // one scan for both: complete nodes per group (low 16 bits), path nodes
    // per (round, wave) (high 16 bits; at most 992 * 32 in all)
    const int gq = lane < kFamGroups ? lane : 0;
    const uint64_t gm = lane < kFamGroups ? Wk.cmask[gq] : 0ull;
    const int nwt = rounds * W;
    const int wtv = lane < nwt ? Wk.wtot[lane] : 0;
    const uint32_t both = uint32_t(popc64(gm)) | (uint32_t(wtv) << 16);
    const uint32_t incl2 = wave_incl_scan_u32(both);
    const int gpre = int(incl2 & 0xFFFFu) - popc64(gm);   // lane g: complete nodes before group g
    const int nA = __builtin_amdgcn_readlane(int(incl2 & 0xFFFFu), kFamGroups - 1);
    const int wpre = int(incl2 >> 16) - wtv;                // lane q: path nodes before entry q
    const int nB = __builtin_amdgcn_readlane(int(incl2 >> 16), kWave - 1);
    if (wv == 0 && lane < kFamGroups) Wk.gpre[lane] = gpre;
    const int n = nA + nB;
    if (n > cap) {
        __syncthreads();   // every wave has read the masks and counts
        return n;
    }
    const int dummy = cap + kPoolPad + lane;
    if (tid < kPoolPad) L.key[n + tid] = 0;
    // family_rank's bins (every wave has read the bound's histogram)
    for (int i = tid; i < kHistBins; i += THREADS) L.hist[i] = 0u;
    const int baseB = nA;
    // the top-1 path's first family node (depth D + 1), for the parent links
    const int topbase = npair >= 0 ? baseB + Wk.flag[1] +
                                         __builtin_amdgcn_readlane(wpre, __builtin_amdgcn_readfirstlane(Wk.flag[2]))
                                   : 0;
    if (tid == 0) Wk.flag[3] = topbase;
    // complete-level nodes, by their owners
#pragma unroll
    for (int m = 0; m < MC; ++m) {
        const int g = tid + m * THREADS;
        const int grp = m * W + wv;
        if ((cm[m] >> lane) & 1u) {
            const int s = __builtin_amdgcn_readlane(gpre, grp) + popc64(cm[m] & lt);
            int d = 1, loff = 0, lsz = k;
            while (g >= loff + lsz) {
                loff += lsz;
                lsz *= k;
                ++d;
            }
            const int i = g - loff, jj = i - div_small(i, inv_k) * k;
            if (s < cap) L.key[s] = fam_key(cv[m], d, ttab[(d - 1) * kp + jj], i);
        }
    }
    // the paths, by their owners: nodes dstart .. dstart + cn - 1
    // (blocks of up to 256 threads: the wider blocks of the trees' own
    // launch have no registers to spare for it and walk the path again)
    constexpr bool kRegWrites = THREADS <= 256;
    if (kRegWrites && rounds == 1 && b <= 16) {
        // the path's rho at every depth is still in registers from
        // family_bound's walk: every node's key at once, tokens by 16-byte
        // column loads
        const Chain c = make_chain(tid, npair, b, k, kp, D, inv_km1, qtab, ttab);
        const int s0 = baseB + __builtin_amdgcn_readlane(wpre, wv) + cbase[0];
        const int code = c.top ? 0 : (c.e - 1) * 32 + c.j;
        const int cnc = cn[0] < cap - s0 ? cn[0] : cap - s0;
        pool_i32x4 t4[4];
#pragma unroll
        for (int g = 0; g < 4; ++g) t4[g] = *reinterpret_cast<const pool_i32x4 *>(F.t0 + 4 * g);
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int d = i + 1, off = d - c.dstart;
            const int tk = d == c.e ? c.te : t4[i >> 2][i & 3];
            L.key[off >= 0 && off < cnc ? s0 + off : dummy] = fam_key(R.rv[i], d, tk, code);
        }
    }
#pragma unroll
    for (int rd = 0; rd < kFamRounds; ++rd) {
        if (rd < rounds && !(kRegWrites && rounds == 1 && b <= 16)) {
            const Chain c = make_chain(rd * THREADS + tid, npair, b, k, kp, D, inv_km1, qtab, ttab);
            const int s0 = baseB + __builtin_amdgcn_readlane(wpre, rd * W + wv) + cbase[rd];
            const int code = c.top ? 0 : (c.e - 1) * 32 + c.j;
            const int cmax = int(wave_max_u32(uint32_t(cn[rd])));
            const int cnc = cn[rd] < cap - s0 ? cn[rd] : cap - s0;   // slots below cap
            float r = crp[rd];
            // depth dstart + i; the next depth's column entries load ahead
            int dn = c.dstart <= b ? c.dstart : b;
            float qn = F.q0[dn - 1];
            int tn = F.t0[dn - 1];
            for (int i = 0; i < cmax; ++i) {
                const int d = c.dstart + i;
                const float q = d == c.e ? c.qe : qn;
                const int tk = d == c.e ? c.te : tn;
                dn = d + 1 <= b ? d + 1 : b;
                qn = F.q0[dn - 1];
                tn = F.t0[dn - 1];
                r = __fmul_rn(r, q);
                const int w = i < cnc ? s0 + i : dummy;
                L.key[w] = fam_key(r, d, tk, code);
            }
        }
    }
    __syncthreads();
    return n;
}

// What family_rank needs of family_select's layout.
struct FamGeom {
    int D, k, kp, firstD, topbase;
    uint32_t inv_k;
    const float *lvl;       // complete levels' rho
    const int32_t *ttab;    // token table
    const uint64_t *cmask;  // qualifying complete nodes per group
    const int32_t *gpre;    // complete nodes before each group
};

__device__ __forceinline__ int level_off(const FamGeom &G, int x) {   // first index of level x
    int off = 0, sz = G.k;
    for (int l = 1; l < x; ++l) {
        off += sz;
        sz *= G.k;
    }
    return off;
}

// slot of complete-level node g (it must be in the pool)
__device__ __forceinline__ int fam_cslot(const FamGeom &G, int g) {
    const int grp = g >> 6;
    return G.gpre[grp] + popc64(G.cmask[grp] & ((uint64_t(1) << (g & 63)) - 1));
}

// pop order of two complete-level ancestors at depth x (level indices a, c):
// does c pop first?
__device__ __forceinline__ bool fam_level_before(const FamGeom &G, int x, int a, int c) {
    const int off = level_off(G, x);
    const float ra = G.lvl[off + a], rc = G.lvl[off + c];
    if (ra != rc) return rc > ra;
    const int da = a - div_small(a, G.inv_k) * G.k, dc = c - div_small(c, G.inv_k) * G.k;
    return G.ttab[(x - 1) * G.kp + dc] < G.ttab[(x - 1) * G.kp + da];
}

// Does pool node f (key xf, slot sf) pop before node e (xe, se), for equal
// rho, depth and token?  Best-first orders them as their parents, walked up
// until the keys differ.  Below the deepest depth x where their rank digits
// differ both take the same factors, so their rho keep the order (float
// products are monotone) and the walk decides as the ancestors at depth x
// compare: larger rho first, then smaller token.  x and those ancestors
// follow from the nodes' family identities.
__device__ __forceinline__ bool fam_tie_before(const FamGeom &G, const uint64_t *key, uint64_t xe,
                                               int se, uint64_t xf, int sf) {
    const int d = tree_key_depth(xe);
    const int ie = fam_id(xe), jf = fam_id(xf);
    if (d <= G.D) {
        // complete levels: ancestor indices one level up at a time until
        // their last digits differ
        int a = ie, c = jf;
        for (int y = d - 1; y >= 1; --y) {
            a = div_small(a, G.inv_k);
            c = div_small(c, G.inv_k);
            if (a - div_small(a, G.inv_k) * G.k != c - div_small(c, G.inv_k) * G.k)
                return fam_level_before(G, y, a, c);
        }
        return false;
    }
    // paths: identity 0 is the top-1 path, else rank j at depth e
    const int ee = ie ? (ie >> 5) + 1 : 0, fe = jf ? (jf >> 5) + 1 : 0;
    if (ee == fe) return (jf & 31) < (ie & 31);   // same split point: rank order
    const int x = ee > fe ? ee : fe;
    if (x > G.D) {
        // both ancestors at depth x are path nodes, d - x slots up
        const uint64_t ka = key[se - (d - x)] | 1023u, kc = key[sf - (d - x)] | 1023u;
        return kc > ka;
    }
    // both split inside the complete levels: their ancestors at depth x
    auto anc = [&](int ev, int id) -> int {
        if (ev == x) return id & 31;
        int idx = ev ? (id & 31) : 0;
        for (int y = ev; y < x; ++y) idx *= G.k;
        return ev ? idx : 0;
    };
    return fam_level_before(G, x, anc(ee, ie), anc(fe, jf));
}

// parent slot of pool node s (key x), -1 for the root
__device__ __forceinline__ int fam_parent(const FamGeom &G, uint64_t x, int s) {
    const int d = tree_key_depth(x), id = fam_id(x);
    if (d == 1) return -1;
    if (d <= G.D) return fam_cslot(G, level_off(G, d - 1) + div_small(id, G.inv_k));
    const int e = id ? (id >> 5) + 1 : 0, j = id & 31;
    const int dstart = (id && e > G.D) ? e : G.D + 1;
    if (d > dstart) return s - 1;
    if (id && e <= G.D) {
        int pw = 1;
        for (int y = e; y < G.D; ++y) pw *= G.k;
        return fam_cslot(G, G.firstD + j * pw);
    }
    if (id && e - 1 > G.D) return G.topbase + (e - 1) - (G.D + 1);
    return G.D >= 1 ? fam_cslot(G, G.firstD) : -1;
}

// Step 3 after family_select, by the whole block (1 <= n <= cap <= 1024;
// L.hist zero on entry; every key has rho >= t): pop index = 1 + the number
// of pool keys that pop first.  The keys are binned by rho (L.hist: fine
// bins over [t, 1], as many mantissa bits as 1024 bins hold), every key of a
// higher bin pops first, and a key is compared only with the keys of its own
// bin, placed together in L.rho / L.par (free on the family path).  Writes
// the pop-order records 1..cnt (cnt = min(n, nmax)) into par/dep/tok/rho
// (nmax + 2 entries; index nmax + 1 takes the stores of nodes past cnt) and
// returns cnt.
template <int THREADS>
__device__ int family_rank(const PoolLds &L, const FamGeom &G, int n, int nmax, float t,
                           int32_t *par, int32_t *dep, int32_t *tok, float *rho,
                           uint64_t *st = nullptr) {
    (void)st;
    const int tid = threadIdx.x;
    n = __builtin_amdgcn_readfirstlane(n);
    bucket_rank<THREADS>(L.key, n, t, L.hist, reinterpret_cast<uint64_t *>(L.rho), L.par, L.pop,
                         [&](uint64_t x, int e, uint64_t y, int f) {
                             return fam_tie_before(G, L.key, x, e, y, f);
                         });
    BASTION_STAMP(st, 13);
    const int cnt = n < nmax ? n : nmax;
    for (int e = tid; e < n; e += THREADS) {
        const int pe = L.pop[e] + 1;
        const uint64_t x = L.key[e];
        const int ps = fam_parent(G, x, e);
        const int pp = L.pop[ps >= 0 ? ps : 0] + 1;
        const int w = pe <= cnt ? pe : nmax + 1;
        par[w] = ps >= 0 ? pp : 0;
        dep[w] = tree_key_depth(x);
        tok[w] = tree_key_token(x);
        rho[w] = tree_key_rho(x);
    }
    return cnt;
}

}  // namespace bastion
