// mixture.hpp -- the latent-mixture stage for one query (DBlast, Methodology
// 1 on the gist.science page: q_dep(x_1:b | y) = sum_z q(z|y) prod_i
// q_i(x_i | y, z); a branch is decoded greedily), run by the block that
// finishes the query's last branch row.
//
//   1. prior weights w = softmax(prior logits), float64 (stored as float32);
//   2. chain z = the top-1 token of every position of branch z;
//      q_dep(chain z) = sum_z' w_z' prod_i q_i(x_i | z'), float64, each q
//      from the branch row's max and sum at the chain token (logit gather);
//   3. per position, the union of the branches' top-k tokens in ascending
//      order and q_i(token | z) for every branch (float32, the same formula
//      as the row's own top-k q).  All positions are handled at once: one
//      round trip loads every branch row's top-k ids, the unions are formed
//      in LDS, and every logit the stage needs (chains and candidates) is
//      gathered in a few batches of independent loads;
//   4. when asked, the best-first tree over those candidates.  A node keeps
//      r_z = fl32 product of q_i(x_i | z) along its path and is scored by the
//      float32 fma chain sum_z w_z r_z; children score no higher than their
//      parent, so the level-synchronous argument of the plain tree holds:
//      after round d the running list holds the N best nodes of depth <= d,
//      round d merging the children of its depth-(d-1) nodes.  A child's key
//      carries its parent's rank among the depth-(d-1) entries, which is
//      best-first's parent-order tie-break.  Candidates that beat the list's
//      N-th key are buffered and merged kMixSurv at a time.  The rounds read
//      their positions' q tables from LDS, where the gathers left them.
#pragma once

#include "device_common.hpp"
#include "build_params.hpp"

namespace bastion {

constexpr int kMixSurv = 512;   // survivors buffered between merges
constexpr int kMixMaxLds = 160 * 1024;   // LDS of one CU

struct MixLayout {
    int w, wq, prod, rowm, rows, chain, ids, first, ctok, cnt, qc, cq, rkey, rr, nkey, nr, ptab, ptab2,
        skey, sinfo, rankb, lob, map, base, par, dep, tok, rho, ahat, total;
};

__host__ __device__ inline int mix_align16(int x) { return (x + 15) & ~15; }

// Three regions: arrays live through the whole stage (among them every
// position's q table, written by the gathers and read by the rounds); arrays
// used only before the tree rounds (every position's ids, first-occurrence
// flags, the chains' q); arrays used only by the rounds.  The last two share
// space.  The stage has a launch of its own, one block per CU, so the
// layout may use up to kMixMaxLds bytes.
// C: candidate slots per position (K * k for the unions of the branches'
// top-k, k for the marginal's top-k)
__host__ __device__ inline MixLayout mix_layout(int K, int b, int k, int nmax, int C = 0) {
    MixLayout L;
    C = C > 0 ? C : K * k;
    const int nn = nmax + 2;
    int o = 0;
    L.w = o;     o = mix_align16(o + 8 * K);
    L.wq = o;    o = mix_align16(o + 4 * K);
    L.prod = o;  o = mix_align16(o + 8 * K * K);
    L.rowm = o;  o = mix_align16(o + 4 * K * b);
    L.rows = o;  o = mix_align16(o + 4 * K * b);
    L.chain = o; o = mix_align16(o + 4 * K * b);
    L.ctok = o;  o = mix_align16(o + 4 * b * C);   // unions, ascending, per position
    L.cnt = o;   o = mix_align16(o + 4 * b);
    L.map = o;   o = mix_align16(o + 4 * nn);
    L.base = o;  o = mix_align16(o + 4 * 40);
    L.par = o;   o = mix_align16(o + 4 * nn);
    L.dep = o;   o = mix_align16(o + 4 * nn);
    L.tok = o;   o = mix_align16(o + 4 * nn);
    L.rho = o;   o = mix_align16(o + 4 * nn);
    L.ahat = o;  o = mix_align16(o + 8 * nn);
    // every position's q table, written by the gathers, read by the rounds
    L.cq = o;    o = mix_align16(o + 4 * b * C * K);   // [pos][z][c]
    // before the rounds
    int a = o;
    L.ids = a;   a = mix_align16(a + 4 * b * C);   // every position's top-k ids
    L.first = a; a = mix_align16(a + 4 * b * C);
    L.qc = a;    a = mix_align16(a + 4 * K * K * b); // q_i(chain z | z')
    // the rounds
    int r = o;
    L.rkey = r;  r = mix_align16(r + 8 * nmax);
    L.rr = r;    r = mix_align16(r + 4 * nmax * K);
    L.nkey = r;  r = mix_align16(r + 8 * nmax);
    L.nr = r;    r = mix_align16(r + 4 * nmax * K);
    L.ptab = r;  r = mix_align16(r + 4 * nmax * K);
    L.ptab2 = r; r = mix_align16(r + 4 * nmax * K);
    L.skey = r;  r = mix_align16(r + 8 * kMixSurv);
    L.sinfo = r; r = mix_align16(r + 4 * kMixSurv);
    L.rankb = r; r = mix_align16(r + 4 * (nmax + kMixSurv));
    L.lob = r;   r = mix_align16(r + 4 * (nmax + kMixSurv));
    L.total = a > r ? a : r;
    return L;
}

struct MixLds {
    double *w, *prod;
    float *wq, *rowm, *rows, *cq, *rr, *nr, *ptab, *ptab2;
    int32_t *chain, *ids, *first, *ctok, *cnt, *sinfo, *rankb, *lob, *map, *base, *par, *dep, *tok;
    float *qc;
    uint64_t *rkey, *nkey, *skey;
    float *rho;
    double *ahat;
    int C;   // candidates per position: the stride of a cq row
};

__device__ __forceinline__ MixLds mix_lds(char *smem, const MixLayout &L, int C) {
    MixLds M;
    M.w = reinterpret_cast<double *>(smem + L.w);
    M.wq = reinterpret_cast<float *>(smem + L.wq);
    M.prod = reinterpret_cast<double *>(smem + L.prod);
    M.rowm = reinterpret_cast<float *>(smem + L.rowm);
    M.rows = reinterpret_cast<float *>(smem + L.rows);
    M.chain = reinterpret_cast<int32_t *>(smem + L.chain);
    M.ids = reinterpret_cast<int32_t *>(smem + L.ids);
    M.first = reinterpret_cast<int32_t *>(smem + L.first);
    M.ctok = reinterpret_cast<int32_t *>(smem + L.ctok);
    M.cnt = reinterpret_cast<int32_t *>(smem + L.cnt);
    M.qc = reinterpret_cast<float *>(smem + L.qc);
    M.cq = reinterpret_cast<float *>(smem + L.cq);
    M.rkey = reinterpret_cast<uint64_t *>(smem + L.rkey);
    M.rr = reinterpret_cast<float *>(smem + L.rr);
    M.nkey = reinterpret_cast<uint64_t *>(smem + L.nkey);
    M.nr = reinterpret_cast<float *>(smem + L.nr);
    M.ptab = reinterpret_cast<float *>(smem + L.ptab);
    M.ptab2 = reinterpret_cast<float *>(smem + L.ptab2);
    M.rankb = reinterpret_cast<int32_t *>(smem + L.rankb);
    M.lob = reinterpret_cast<int32_t *>(smem + L.lob);
    M.skey = reinterpret_cast<uint64_t *>(smem + L.skey);
    M.sinfo = reinterpret_cast<int32_t *>(smem + L.sinfo);
    M.map = reinterpret_cast<int32_t *>(smem + L.map);
    M.base = reinterpret_cast<int32_t *>(smem + L.base);
    M.par = reinterpret_cast<int32_t *>(smem + L.par);
    M.dep = reinterpret_cast<int32_t *>(smem + L.dep);
    M.tok = reinterpret_cast<int32_t *>(smem + L.tok);
    M.rho = reinterpret_cast<float *>(smem + L.rho);
    M.ahat = reinterpret_cast<double *>(smem + L.ahat);
    M.C = C;
    return M;
}

// fma-chain score of the child of parent p with candidate c: its r_z are
// fl32(r_z(parent) * q(c | z))
__device__ __forceinline__ float mix_child(const MixLds &M, int K, int p, int c) {
    float acc = 0.0f;
#pragma unroll 8
    for (int z = 0; z < K; ++z)
        acc = __builtin_fmaf(M.wq[z], __fmul_rn(M.ptab[p * K + z], M.cq[z * M.C + c]), acc);
    return acc;
}

// Merge the ns buffered survivors (all of the round's depth) into the
// running list (nR sorted keys in M.rkey / M.rr, at most nmax).  An
// element's new place is the number of larger keys: the list entries above
// a survivor by binary search, the survivors above any element counted in
// parts by several threads (M.rankb, zero on entry, is left zero).  The
// merged list goes to M.nkey / M.nr; the caller swaps the buffers.  With
// `parents`, the survivors that land also write their r values to M.ptab2
// in list order (the parents of the next round: the landed survivors are
// the largest ones, and a survivor's index among them is its place minus
// the list entries above it) and their number to *np_next (zero on entry).
// Whole block.  Returns the new list length.
template <int THREADS>
__device__ int mix_merge(const MixLds &M, int K, int nmax, int nR, int ns, bool parents, int *np_next) {
    const int tid = threadIdx.x;
    const int nE = nR + ns;
    const int P = nE < THREADS ? THREADS / nE : 1;   // parts per element
    const int per = (ns + P - 1) / P;
    for (int t = tid; t < nE * P; t += THREADS) {
        const int part = t / nE, e = t - part * nE;
        const uint64_t x = e < nR ? M.rkey[e] : M.skey[e - nR];
        int cnt = 0;
        if (part == 0) {
            if (e < nR) {
                cnt = e;
            } else {
                // larger keys of the sorted list: binary search
                int lo = 0, hi = nR;
                while (lo < hi) {
                    const int mid = (lo + hi) >> 1;
                    if (M.rkey[mid] > x) lo = mid + 1;
                    else hi = mid;
                }
                cnt = lo;
                M.lob[e] = lo;
            }
        }
        // survivors above x in this part: eight independent counts keep
        // eight LDS reads in flight
        const int s0 = part * per, s1 = s0 + per < ns ? s0 + per : ns;
        int cnt8[8] = {0, 0, 0, 0, 0, 0, 0, 0};
        int s = s0;
        for (; s + 8 <= s1; s += 8) {
#pragma unroll
            for (int u = 0; u < 8; ++u) cnt8[u] += M.skey[s + u] > x ? 1 : 0;
        }
        for (; s < s1; ++s) cnt8[0] += M.skey[s] > x ? 1 : 0;
#pragma unroll
        for (int u = 0; u < 8; ++u) cnt += cnt8[u];
        atomicAdd(M.rankb + e, cnt);
    }
    __syncthreads();
    for (int e = tid; e < nE; e += THREADS) {
        const int rank = M.rankb[e];
        M.rankb[e] = 0;
        if (rank < nmax) {
            if (e < nR) {
                M.nkey[rank] = M.rkey[e];
#pragma unroll 8
                for (int z = 0; z < K; ++z) M.nr[rank * K + z] = M.rr[e * K + z];
            } else {
                M.nkey[rank] = M.skey[e - nR];
                const int info = M.sinfo[e - nR];
                const int p = info >> 16, c = info & 0xFFFF;
                const int pi = rank - M.lob[e];
#pragma unroll 8
                for (int z = 0; z < K; ++z) {
                    const float v = __fmul_rn(M.ptab[p * K + z], M.cq[z * M.C + c]);
                    M.nr[rank * K + z] = v;
                    if (parents) M.ptab2[pi * K + z] = v;
                }
                if (parents) atomicMax(np_next, pi + 1);
            }
        }
    }
    __syncthreads();
    return nE < nmax ? nE : nmax;
}

// The merged list becomes the running one.
__device__ __forceinline__ void swap_list(MixLds &L) {
    uint64_t *tk = L.rkey;
    L.rkey = L.nkey;
    L.nkey = tk;
    float *tr = L.rr;
    L.rr = L.nr;
    L.nr = tr;
}

__device__ __forceinline__ float mix_logit(const BuildParams &P, int64_t row, int token,
                                           int is_bf16) {
    const char *p = P.logits + row * P.row_stride_bytes;
    if (is_bf16) return float(reinterpret_cast<const __bf16 *>(p)[token]);
    return reinterpret_cast<const float *>(p)[token];
}

// Pop-order tree records 1..cnt from the sorted running list (one wave).
__device__ inline void mix_resolve(const MixLds &M, int b, int nmax, int cnt) {
    const int lane = lane_id();
    const uint64_t lt = lanemask_lt();
    int basev = 0;
    for (int d = 1; d <= b; ++d) {
        if (lane == 0) M.base[d] = basev;
        for (int e0 = 0; e0 < cnt; e0 += kWave) {
            const int e = e0 + lane;
            const bool v = e < cnt && tree_key_depth(M.rkey[e]) == d;
            const uint64_t m = __ballot(v);
            if (v) M.map[basev + popc64(m & lt)] = e + 1;
            basev += popc64(m);
        }
    }
    wave_sync();
    for (int e = lane; e < cnt; e += kWave) {
        const uint64_t key = M.rkey[e];
        const int d = tree_key_depth(key);
        int mi = M.base[d - 1] + tree_key_parent(key);
        mi = mi < nmax ? mi : nmax;
        M.par[e + 1] = d == 1 ? 0 : M.map[mi];
        M.dep[e + 1] = d;
        M.tok[e + 1] = tree_key_token(key);
        M.rho[e + 1] = tree_key_rho(key);
    }
    if (lane == 0) {
        M.par[0] = -1;
        M.dep[0] = 0;
        M.tok[0] = -1;
        M.rho[0] = 1.0f;
        M.ahat[0] = 1.0;
    }
    wave_sync();
}

}  // namespace bastion
