// tree_rounds.hpp -- level-synchronous best-first tree for one query, run by
// one wave (Bastion, Methodology 1-2 on the gist.science page: path score
// rho, surrogate A_hat, best-first expansion; Methodology 3: stop where S(N)
// starts to decrease).
//
// Best-first with a total order on keys pops the N largest keys of the
// whole candidate tree (keys strictly decrease from a node to its children),
// in key order.  The N largest keys among nodes of depth <= d can only have
// parents among the N largest of depth <= d-1 (a parent outranks its child
// and adding nodes only raises the N-th key), so
//     R_d = top-N( R_{d-1}  U  children of the depth-(d-1) nodes of R_{d-1} )
// and R_b is the tree, already sorted in pop order.  A child's tie-break
// field holds its parent's rank among the depth-(d-1) entries of R_{d-1};
// ranks among one depth never change later (evictions remove the smallest
// keys first), so the same field resolves the parent's pop index at the end.
//
// R lives in G registers per lane (element i = lane i % 64 of register
// i / 64), sorted in descending key order; a round merges each rank's
// children (a sorted column) with a reverse + elementwise max + bitonic
// merge, or by sorted insertion when only one or two of them qualify.
#pragma once

#include "device_common.hpp"

namespace bastion {

// ---- xor-partner exchange inside one register (all 64 lanes active) ----
constexpr int kDppRowShl4 = 0x104;   // lane i <- lane i+4 (same row)
constexpr int kDppRowShr4 = 0x114;   // lane i <- lane i-4 (same row)
constexpr int kDppRowRor8 = 0x128;   // lane i <- lane (i+8) mod 16 = i ^ 8
constexpr int kDppWaveShr1 = 0x138;  // lane i <- lane i-1 (lane 0 <- old)

template <int S>
__device__ __forceinline__ uint32_t xpartner(uint32_t x) {
    if constexpr (S == 1) {
        return dpp32<kDppXor1>(x);
    } else if constexpr (S == 2) {
        return dpp32<kDppXor2>(x);
    } else if constexpr (S == 4) {
        const uint32_t up = dpp32<kDppRowShl4>(x), dn = dpp32<kDppRowShr4>(x);
        return (lane_id() & 4) ? dn : up;
    } else if constexpr (S == 8) {
        return dpp32<kDppRowRor8>(x);
    } else if constexpr (S == 16) {
        uint32_t a, b;
        swap16(x, a, b);
        return (lane_id() & 16) ? a : b;
    } else {
        uint32_t a, b;
        swap32(x, a, b);
        return (lane_id() & 32) ? a : b;
    }
}

// lane i <- lane 63 - i
__device__ __forceinline__ uint32_t reverse64(uint32_t x) {
    return xpartner<16>(xpartner<32>(dpp32<kDppMirror>(x)));
}

__device__ __forceinline__ bool key_gt(uint32_t ah, uint32_t al, uint32_t bh, uint32_t bl) {
    return ah > bh || (ah == bh && al > bl);
}

// compare-exchange with the xor-S partner: the lower lane keeps the larger
// key when `desc`, the smaller otherwise
template <int S>
__device__ __forceinline__ void cmpx(uint32_t &h, uint32_t &l, bool desc) {
    const uint32_t oh = xpartner<S>(h), ol = xpartner<S>(l);
    const bool ogt = key_gt(oh, ol, h, l);
    const bool lower = (lane_id() & S) == 0;
    const bool take = (desc == lower) ? ogt : !ogt;
    h = take ? oh : h;
    l = take ? ol : l;
}

// bitonic sort of one register into descending order
__device__ __forceinline__ void sort64_desc(uint32_t &h, uint32_t &l) {
    const int lane = lane_id();
    cmpx<1>(h, l, (lane & 2) == 0);
    cmpx<2>(h, l, (lane & 4) == 0);
    cmpx<1>(h, l, (lane & 4) == 0);
    cmpx<4>(h, l, (lane & 8) == 0);
    cmpx<2>(h, l, (lane & 8) == 0);
    cmpx<1>(h, l, (lane & 8) == 0);
    cmpx<8>(h, l, (lane & 16) == 0);
    cmpx<4>(h, l, (lane & 16) == 0);
    cmpx<2>(h, l, (lane & 16) == 0);
    cmpx<1>(h, l, (lane & 16) == 0);
    cmpx<16>(h, l, (lane & 32) == 0);
    cmpx<8>(h, l, (lane & 32) == 0);
    cmpx<4>(h, l, (lane & 32) == 0);
    cmpx<2>(h, l, (lane & 32) == 0);
    cmpx<1>(h, l, (lane & 32) == 0);
    cmpx<32>(h, l, true);
    cmpx<16>(h, l, true);
    cmpx<8>(h, l, true);
    cmpx<4>(h, l, true);
    cmpx<2>(h, l, true);
    cmpx<1>(h, l, true);
}

// bitonic sort of one 32-bit value per lane into ascending lane order
template <int S>
__device__ __forceinline__ uint32_t cmpx_u32(uint32_t v, bool asc) {
    const uint32_t o = xpartner<S>(v);
    const bool lower = (lane_id() & S) == 0;
    return (lower == asc) ? min(v, o) : max(v, o);
}

__device__ __forceinline__ uint32_t sort64_asc_u32(uint32_t v) {
    const int lane = lane_id();
    v = cmpx_u32<1>(v, (lane & 2) == 0);
    v = cmpx_u32<2>(v, (lane & 4) == 0);
    v = cmpx_u32<1>(v, (lane & 4) == 0);
    v = cmpx_u32<4>(v, (lane & 8) == 0);
    v = cmpx_u32<2>(v, (lane & 8) == 0);
    v = cmpx_u32<1>(v, (lane & 8) == 0);
    v = cmpx_u32<8>(v, (lane & 16) == 0);
    v = cmpx_u32<4>(v, (lane & 16) == 0);
    v = cmpx_u32<2>(v, (lane & 16) == 0);
    v = cmpx_u32<1>(v, (lane & 16) == 0);
    v = cmpx_u32<16>(v, (lane & 32) == 0);
    v = cmpx_u32<8>(v, (lane & 32) == 0);
    v = cmpx_u32<4>(v, (lane & 32) == 0);
    v = cmpx_u32<2>(v, (lane & 32) == 0);
    v = cmpx_u32<1>(v, (lane & 32) == 0);
    v = cmpx_u32<32>(v, true);
    v = cmpx_u32<16>(v, true);
    v = cmpx_u32<8>(v, true);
    v = cmpx_u32<4>(v, true);
    v = cmpx_u32<2>(v, true);
    v = cmpx_u32<1>(v, true);
    return v;
}

// bitonic sequence in one register -> descending
__device__ __forceinline__ void merge64_desc(uint32_t &h, uint32_t &l) {
    cmpx<32>(h, l, true);
    cmpx<16>(h, l, true);
    cmpx<8>(h, l, true);
    cmpx<4>(h, l, true);
    cmpx<2>(h, l, true);
    cmpx<1>(h, l, true);
}

// the running top-N list
template <int G>
struct TopList {
    uint32_t h[G], l[G];

    __device__ __forceinline__ void clear() {
#pragma unroll
        for (int g = 0; g < G; ++g) h[g] = l[g] = 0;
    }
    // element s (wave-uniform index) as a 64-bit key
    __device__ __forceinline__ uint64_t at(int s) const {
        const int gs = s >> 6, ls = s & 63;
        uint32_t vh = 0, vl = 0;
#pragma unroll
        for (int g = 0; g < G; ++g) {
            const uint32_t th = uint32_t(__builtin_amdgcn_readlane(int(h[g]), ls));
            const uint32_t tl = uint32_t(__builtin_amdgcn_readlane(int(l[g]), ls));
            vh = (gs == g) ? th : vh;
            vl = (gs == g) ? tl : vl;
        }
        return (uint64_t(vh) << 32) | vl;
    }
    // drop everything at index >= n
    __device__ __forceinline__ void truncate(int n) {
        const int lane = lane_id();
#pragma unroll
        for (int g = 0; g < G; ++g) {
            const bool keep = g * kWave + lane < n;
            h[g] = keep ? h[g] : 0u;
            l[g] = keep ? l[g] : 0u;
        }
    }
    // sorted insertion (the last element falls off)
    __device__ __forceinline__ void insert(uint64_t key) {
        const uint32_t kh = uint32_t(key >> 32), kl = uint32_t(key);
        int pos = 0;
#pragma unroll
        for (int g = 0; g < G; ++g) pos += popc64(__ballot(key_gt(h[g], l[g], kh, kl)));
        const int lane = lane_id();
        int ch = 0, cl = 0;   // lane 63 of the previous register
#pragma unroll
        for (int g = 0; g < G; ++g) {
            const int lh = __builtin_amdgcn_readlane(int(h[g]), 63);
            const int ll = __builtin_amdgcn_readlane(int(l[g]), 63);
            const uint32_t sh = uint32_t(__builtin_amdgcn_update_dpp(ch, int(h[g]), kDppWaveShr1, 0xF, 0xF, false));
            const uint32_t sl = uint32_t(__builtin_amdgcn_update_dpp(cl, int(l[g]), kDppWaveShr1, 0xF, 0xF, false));
            const int idx = g * kWave + lane;
            h[g] = idx > pos ? sh : (idx == pos ? kh : h[g]);
            l[g] = idx > pos ? sl : (idx == pos ? kl : l[g]);
            ch = lh;
            cl = ll;
        }
    }
    // merge a descending column (one register, zeros after its end)
    __device__ __forceinline__ void merge(uint32_t ch, uint32_t cl) {
        const uint32_t rh = reverse64(ch), rl = reverse64(cl);
        const bool gt = key_gt(rh, rl, h[G - 1], l[G - 1]);
        h[G - 1] = gt ? rh : h[G - 1];
        l[G - 1] = gt ? rl : l[G - 1];
        // bitonic merge over G registers: cross-register strides first
#pragma unroll
        for (int s = G / 2; s >= 1; s >>= 1) {
#pragma unroll
            for (int g = 0; g < G; ++g) {
                if (g & s) continue;
                const int u = g + s;
                const bool ugt = key_gt(h[u], l[u], h[g], l[g]);
                const uint32_t th = h[g], tl = l[g];
                h[g] = ugt ? h[u] : h[g];
                l[g] = ugt ? l[u] : l[g];
                h[u] = ugt ? th : h[u];
                l[u] = ugt ? tl : l[u];
            }
        }
#pragma unroll
        for (int g = 0; g < G; ++g) merge64_desc(h[g], l[g]);
    }
};

struct RoundsLds {
    float *qtab;       // [b * kp] candidate q of each position, rank order
    int32_t *ttab;     // [b * kp] candidate tokens (rows padded to kp)
    int kp;            // row stride: k rounded up to a multiple of 8
    uint64_t *col;     // [64 * G] compaction buffer for one column
    int32_t *par, *dep, *tok;   // [nmax + 2] node records (pop order)
    float *rho;
    double *ahat, *cost;
    int32_t *map;      // [nmax + 2] (depth base + rank) -> pop index
    int32_t *base;     // [34] first map slot of each depth
};

// Builds R (the top-nmax keys, pop order); returns the number of nodes.
template <int G>
__device__ int rounds_build(TopList<G> &R, const RoundsLds &S, int b, int k, int nmax) {
    const int lane = lane_id();
    const uint64_t lt = lanemask_lt();
    R.clear();
    // depth 1: the root's children, rank order is almost sorted; sort them
    {
        uint32_t h = 0, l = 0;
        if (lane < k) {
            const uint64_t key = tree_key(S.qtab[lane], 1, S.ttab[lane], 0);
            h = uint32_t(key >> 32);
            l = uint32_t(key);
        }
        sort64_desc(h, l);
        R.h[0] = h;
        R.l[0] = l;
    }
    int cnt = k < nmax ? k : nmax;
    R.truncate(cnt);
    for (int d = 2; d <= b; ++d) {
        // the depth-(d-1) entries of R are the parents; p = rank among them
        // snapshot the parents (merges below reorder R's lanes)
        bool isp[G];
        int pr[G];
        float prho[G];
        int m = 0;
#pragma unroll
        for (int g = 0; g < G; ++g) {
            const uint64_t key = (uint64_t(R.h[g]) << 32) | R.l[g];
            isp[g] = key != 0 && tree_key_depth(key) == d - 1;
            prho[g] = tree_key_rho(key);
            const uint64_t msk = __ballot(isp[g]);
            pr[g] = m + popc64(msk & lt);
            m += popc64(msk);
        }
        if (m == 0) break;
        uint64_t tau = cnt == nmax ? R.at(nmax - 1) : 0;
        for (int j = 0; j < k; ++j) {
            const float qj = S.qtab[(d - 1) * S.kp + j];
            const int tj = S.ttab[(d - 1) * S.kp + j];
            uint64_t ck[G];
            int L = 0;
            int off[G];
#pragma unroll
            for (int g = 0; g < G; ++g) {
                ck[g] = 0;
                if (isp[g]) ck[g] = tree_key(__fmul_rn(prho[g], qj), d, tj, pr[g]);
                const bool sv = ck[g] > tau;
                ck[g] = sv ? ck[g] : 0;
                off[g] = L;
                L += popc64(__ballot(sv));
            }
            if (L == 0) continue;
            if (L <= 2) {
                // one or two qualify: sorted insertion
#pragma unroll
                for (int g = 0; g < G; ++g) {
                    uint64_t msk = __ballot(ck[g] != 0);
                    while (msk) {
                        const int src = __ffsll((unsigned long long)msk) - 1;
                        msk &= msk - 1;
                        const uint64_t key =
                            (uint64_t(uint32_t(__builtin_amdgcn_readlane(int(uint32_t(ck[g] >> 32)), src))) << 32) |
                            uint32_t(__builtin_amdgcn_readlane(int(uint32_t(ck[g])), src));
                        R.insert(key);
                    }
                }
            } else {
                // compact the qualifying prefix of the column (already in
                // descending order), then merge it 64 at a time
#pragma unroll
                for (int g = 0; g < G; ++g) {
                    const uint64_t msk = __ballot(ck[g] != 0);
                    if (ck[g] != 0) S.col[off[g] + popc64(msk & lt)] = ck[g];
                }
                wave_sync();
                for (int c0 = 0; c0 < L; c0 += kWave) {
                    const uint64_t key = c0 + lane < L ? S.col[c0 + lane] : 0;
                    R.merge(uint32_t(key >> 32), uint32_t(key));
                }
                wave_sync();
            }
            cnt = cnt + L < nmax ? cnt + L : nmax;
            R.truncate(cnt);
            tau = cnt == nmax ? R.at(nmax - 1) : 0;
        }
    }
    return cnt;
}

}  // namespace bastion
