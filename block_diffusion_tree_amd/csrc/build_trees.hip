// build_trees.hip -- the fused gfx950 kernel behind bastion_build_trees.
//
// One launch does, for logits [B, b, V]:
//   1. stream every row once from HBM (16-byte loads, 4 waves per block,
//      each row split into S segments), keeping an online softmax
//      (max / rescaled sum, one exp per element) and a filtered top-k
//      (per-wave threshold; the few elements that beat it go through LDS);
//   2. merge the S segment results of a row in the block that finishes the
//      row last (arrival ticket), writing q = exp(l - M) / S for its top-k;
//   3. in the block that finishes a query's last row (second ticket), build
//      the best-first tree (Bastion, Methodology 1-2: rho products, A_hat),
//      apply the online stop of Methodology 3, and emit the pop-order tree,
//      the ancestor mask and the position ids.
// Nothing waits on another block, so the grid needs no co-residency.
#include "device_common.hpp"
#include "build_params.hpp"

namespace bastion {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

constexpr int kThreads = 256;               // 4 waves
constexpr int kWavesPerBlock = kThreads / kWave;
constexpr int kCap = 256;                   // per-wave candidate buffer (keys)



// storage-type traits ------------------------------------------------------
template <typename T> struct Elem;
template <> struct Elem<float> {
    static constexpr int kPerVec = 4;
    static constexpr uint32_t kNegInfWord = 0xFF800000u;
    __device__ static __forceinline__ void decode(u32x4 r, float *f) {
#pragma unroll
        for (int j = 0; j < 4; ++j) f[j] = __uint_as_float(r[j]);
    }
    __device__ static __forceinline__ float at(const char *p, int64_t elem) {
        return reinterpret_cast<const float *>(p)[elem];
    }
};
template <> struct Elem<__bf16> {
    static constexpr int kPerVec = 8;
    static constexpr uint32_t kNegInfWord = 0xFF80FF80u;
    __device__ static __forceinline__ void decode(u32x4 r, float *f) {
        bf16x8 h = __builtin_bit_cast(bf16x8, r);
#pragma unroll
        for (int j = 0; j < 8; ++j) f[j] = (float)h[j];
    }
    __device__ static __forceinline__ float at(const char *p, int64_t elem) {
        return (float)reinterpret_cast<const __bf16 *>(p)[elem];
    }
};

template <int U>
struct WaveScratch {
    u32x4 stage_raw[kWave * U];
    int32_t stage_vec[kWave * U];
    uint64_t cand[kCap];
};

// ---------------------------------------------------------------------------
// Per-wave state of the streaming stage.
// ---------------------------------------------------------------------------
struct LaneSoftmax {
    float m;   // running max of this lane's elements
    float c;   // scale_ref(m)
    float s;   // sum of 2^(l*log2e - c)
};

template <typename T, int U>
struct Streamer {
    WaveScratch<U> *ws;
    int k;
    float thv;     // float form of the wave threshold (-inf: none yet)
    uint64_t thk;  // the wave's current k-th best key (0: fewer than k so far)
    int cnt;       // keys in ws->cand
    int nstage;
    int head;      // elements of the row before its first 16-byte aligned vector
    bool booted;   // the first tile has set a threshold

    __device__ void compact() {
        uint64_t kth;
        cnt = wave_select_topk<kCap / kWave>(ws->cand, cnt, k, kth);
        thk = kth;
        thv = kth ? topk_key_value(kth) : -INFINITY;
    }

    // Append the keys of the staged vectors that beat the threshold.
    __device__ void drain_stage() {
        constexpr int E = Elem<T>::kPerVec;
        const int lane = lane_id();
        const int total = nstage * E;
        for (int base = 0; base < total; base += kWave) {
            if (cnt + kWave > kCap) compact();
            const int e = base + lane;
            const bool ok = e < total;
            uint64_t key = 0;
            if (ok) {
                const int sv = e / E, sj = e - sv * E;
                float f[E];
                Elem<T>::decode(ws->stage_raw[sv], f);
                float v = f[0];
#pragma unroll
                for (int j = 1; j < E; ++j) v = (sj == j) ? f[j] : v;
                key = topk_key(v, uint32_t(head + ws->stage_vec[sv] * E + sj));
            }
            const bool p = ok && key > thk;
            const uint64_t msk = __ballot(p);
            if (p) ws->cand[cnt + popc64(msk & lanemask_lt())] = key;
            cnt += popc64(msk);
            wave_sync();
        }
        nstage = 0;
        // keep the threshold close to the true k-th key seen so far
        if (cnt >= 2 * k + 8) compact();
    }

    // Candidates that are single elements (the scalar tail of a row).
    __device__ void offer_scalar(bool ok, float v, uint32_t token) {
        if (cnt + kWave > kCap) compact();
        uint64_t key = ok ? topk_key(v, token) : 0;
        const bool p = ok && key > thk;
        const uint64_t msk = __ballot(p);
        if (p) ws->cand[cnt + popc64(msk & lanemask_lt())] = key;
        cnt += popc64(msk);
        wave_sync();
    }

    // One tile: U vectors per lane.  raw[u] is row vector vbase + u * 256 +
    // threadIdx.x; valid[u] false marks padding (filled with -inf).
    __device__ __forceinline__ void tile(const u32x4 *raw, int vbase, const bool *valid,
                                         LaneSoftmax &sm) {
        constexpr int E = Elem<T>::kPerVec;
        float f[U][E];
        float vmax[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            Elem<T>::decode(raw[u], f[u]);
            float a = f[u][0];
#pragma unroll
            for (int j = 1; j < E; ++j) a = fmaxf(a, f[u][j]);
            vmax[u] = a;
        }
        float tmax = vmax[0];
#pragma unroll
        for (int u = 1; u < U; ++u) tmax = fmaxf(tmax, vmax[u]);
        const float m_new = fmaxf(sm.m, tmax);
        const float c_new = scale_ref(m_new);
        float acc = sm.s * __builtin_amdgcn_exp2f(sm.c - c_new);
        float part[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            float e[E];
#pragma unroll
            for (int j = 0; j < E; ++j)
                e[j] = __builtin_amdgcn_exp2f(__builtin_fmaf(f[u][j], kLog2e, -c_new));
            // pairwise sum of the vector
#pragma unroll
            for (int w = E / 2; w >= 1; w >>= 1)
#pragma unroll
                for (int j = 0; j < w; ++j) e[j] += e[j + w];
            part[u] = e[0];
        }
#pragma unroll
        for (int w = U / 2; w >= 1; w >>= 1)
#pragma unroll
            for (int u = 0; u < w; ++u) part[u] += part[u + w];
        sm.s = acc + part[0];
        sm.m = m_new;
        sm.c = c_new;

        if (!booted) {
            // first tile: the k-th largest lane maximum is a lower bound of
            // the k-th largest element (k distinct elements reach it)
            booted = true;
            const float t0 = wave_kth_largest(tmax, k);
            if (thk == 0 && t0 > thv) {
                thv = t0;
                thk = uint64_t(ord_f32(t0)) << 32;   // below every key of value t0
            }
        }
        bool pass[U];
        bool any = false;
#pragma unroll
        for (int u = 0; u < U; ++u) {
            pass[u] = valid[u] && vmax[u] >= thv;
            any |= pass[u];
        }
        if (__ballot(any)) {
            const uint64_t lt = lanemask_lt();
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const uint64_t msk = __ballot(pass[u]);
                if (msk) {
                    if (pass[u]) {
                        const int slot = nstage + popc64(msk & lt);
                        ws->stage_raw[slot] = raw[u];
                        ws->stage_vec[slot] = vbase + u * kThreads + int(threadIdx.x);
                    }
                    nstage += popc64(msk);
                }
            }
            wave_sync();
            drain_stage();
        }
    }
};

template <typename T>
__device__ __forceinline__ u32x4 load_vec(const char *row, int v) {
    return __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(row) + v);
}

// ---------------------------------------------------------------------------
// Segment of a row -> (m, s relative to scale_ref(m)) and the top-k keys,
// left in wave 0's candidate buffer (cand[0..nsel)) of the block.
// ---------------------------------------------------------------------------
struct SegmentResult {
    float m, s;
    int nsel;
};

template <typename T, int U>
__device__ SegmentResult stream_segment(const BuildParams &P, const char *row, int seg, char *smem) {
    constexpr int E = Elem<T>::kPerVec;
    constexpr int ES = int(sizeof(T));
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    WaveScratch<U> *scr = reinterpret_cast<WaveScratch<U> *>(smem);

    // The row is split into: `head` elements up to the first 16-byte
    // boundary, `nvec` aligned vectors, and `tail` elements after them.
    const int V = P.V;
    int head = int(((16u - (uint32_t(reinterpret_cast<uintptr_t>(row)) & 15u)) & 15u) / ES);
    head = head > V ? V : head;
    const int nvec = (V - head) / E;
    const int tail = V - head - nvec * E;
    const char *rowv = row + head * ES;

    // vectors [v_lo, v_hi) of this segment
    const int per = nvec / P.S, rem = nvec % P.S;
    const int v_lo = seg * per + (seg < rem ? seg : rem);
    const int v_hi = v_lo + per + (seg < rem ? 1 : 0);

    Streamer<T, U> st;
    st.ws = &scr[wv];
    st.k = P.k;
    st.thv = -INFINITY;
    st.thk = 0;
    st.cnt = 0;
    st.nstage = 0;
    st.head = head;
    st.booted = false;
    LaneSoftmax sm{-INFINITY, scale_ref(-INFINITY), 0.0f};

    const int span = kThreads * U;
    const int n = v_hi - v_lo;
    const int ntiles = n / span;
    bool all[U];
#pragma unroll
    for (int u = 0; u < U; ++u) all[u] = true;
    const int vlo = v_lo;
    u32x4 A[U], Bv[U];
    auto fill = [&](u32x4 *dst, int t) {
#pragma unroll
        for (int u = 0; u < U; ++u) dst[u] = load_vec<T>(rowv, vlo + t * span + u * kThreads + tid);
    };
    if (ntiles > 0) fill(A, 0);
    int t = 0;
    for (; t + 1 < ntiles; t += 2) {
        fill(Bv, t + 1);
        st.tile(A, vlo + t * span, all, sm);
        if (t + 2 < ntiles) fill(A, t + 2);
        st.tile(Bv, vlo + (t + 1) * span, all, sm);
    }
    if (t < ntiles) st.tile(A, vlo + t * span, all, sm);
    // ragged tile
    {
        bool ok[U];
        bool anyv = false;
        const int vb = vlo + ntiles * span;
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int vi = vb + u * kThreads + tid;
            ok[u] = vi < v_hi;
            anyv |= ok[u];
            const u32x4 ninf = {Elem<T>::kNegInfWord, Elem<T>::kNegInfWord,
                                Elem<T>::kNegInfWord, Elem<T>::kNegInfWord};
            A[u] = ok[u] ? load_vec<T>(rowv, vi) : ninf;
        }
        if (__ballot(anyv)) st.tile(A, vb, ok, sm);
    }
    // unaligned head and tail of the row (fewer than 2E elements), handled
    // by wave 0 of the last segment
    if (seg == P.S - 1 && (head + tail) > 0 && wv == 0) {
        const bool ok = lane < head + tail;
        const int elem = lane < head ? lane : head + nvec * E + (lane - head);
        const float v = ok ? Elem<T>::at(row, elem) : -INFINITY;
        const float m_new = fmaxf(sm.m, v);
        const float c_new = scale_ref(m_new);
        sm.s = sm.s * __builtin_amdgcn_exp2f(sm.c - c_new) +
               (ok ? __builtin_amdgcn_exp2f(__builtin_fmaf(v, kLog2e, -c_new)) : 0.0f);
        sm.m = m_new;
        sm.c = c_new;
        st.offer_scalar(ok, v, uint32_t(elem));
    }
    // at most 64 keys per wave go to the block merge
    if (st.cnt > kWave) st.compact();

    // ---- block merge: softmax state ----
    __shared__ float red_m[kWavesPerBlock], red_s[kWavesPerBlock];
    __shared__ int red_n[kWavesPerBlock];
    const float wm = wave_max_f32(sm.m);
    const float wc = scale_ref(wm);
    const float ws_ = wave_sum_f32(sm.s * __builtin_amdgcn_exp2f(sm.c - wc));
    if (lane == 0) {
        red_m[wv] = wm;
        red_s[wv] = ws_;
        red_n[wv] = st.cnt;
    }
    __syncthreads();
    SegmentResult res;
    float M = red_m[0];
#pragma unroll
    for (int i = 1; i < kWavesPerBlock; ++i) M = fmaxf(M, red_m[i]);
    const float C = scale_ref(M);
    float Ssum = 0.0f;
#pragma unroll
    for (int i = 0; i < kWavesPerBlock; ++i)
        Ssum += red_s[i] * __builtin_amdgcn_exp2f(scale_ref(red_m[i]) - C);
    res.m = M;
    res.s = Ssum;
    // ---- block merge: top-k (wave 0 gathers the other waves' keys) ----
    if (wv == 0) {
        int total = red_n[0];
        for (int w = 1; w < kWavesPerBlock; ++w) {
            const int nw = red_n[w];
            if (lane < nw) scr[0].cand[total + lane] = scr[w].cand[lane];
            total += nw;
        }
        wave_sync();
        uint64_t kth;
        res.nsel = wave_select_topk<kCap / kWave>(scr[0].cand, total, P.k, kth);
    }
    return res;  // res.nsel valid in wave 0 only
}

// ---------------------------------------------------------------------------
// Cross-block hand-off.  Data that another block reads (segment records,
// the rows' top-k, row status) is written and read with agent-scope atomic
// accesses, which gfx950 performs coherently across XCDs (sc1), so no L2
// write-back or invalidate is needed.  arrive_last: every thread waits for
// its stores to complete, then one thread counts the block in; the last of
// `total` blocks gets true.  The counter is reset to 0 for the next call.
// ---------------------------------------------------------------------------
template <typename V>
__device__ __forceinline__ void st_agent(V *p, V v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
template <typename V>
__device__ __forceinline__ V ld_agent(const V *p) {
    return __hip_atomic_load(const_cast<V *>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ bool arrive_last(uint32_t *ticket, uint32_t total) {
    __shared__ int flag;
    __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0): this thread's stores are done
    __syncthreads();
    if (threadIdx.x == 0) {
        const uint32_t old = atomicAdd(ticket, 1u);
        const bool last = (old == total - 1);
        if (last) atomicExch(ticket, 0u);
        flag = last;
    }
    __syncthreads();
    return flag != 0;
}

// ---------------------------------------------------------------------------
// Tree stage: one wave builds the best-first tree of one query.
//
// The frontier holds one key per popped node p (slot p): p's best child not
// popped yet.  Children of a node are offered in rank order (rank j = j-th
// candidate of the position), which is their pop order unless a rounding tie
// of rho puts a larger token first; positions where that can happen, or
// products that leave the normal float range, switch the node to an exact
// path (argmax over its remaining children).  Everything a pop touches lives
// in registers: slot arrays and candidate tables are spread over lanes and
// accessed with v_readlane / v_writelane, so a pop has no LDS round trip.
// LDS keeps the node records for the output and the tables for the exact
// path.
// ---------------------------------------------------------------------------
struct TreeLayout {
    int qtab, ttab, par, dep, tok, rho, popm, ahat, cost, total;
};

__host__ __device__ inline int align16(int x) { return (x + 15) & ~15; }

__host__ __device__ inline TreeLayout tree_layout(int b, int k, int nmax) {
    TreeLayout L;
    const int nn = nmax + 2;
    int o = 0;
    L.qtab = o; o = align16(o + 4 * b * k);
    L.ttab = o; o = align16(o + 4 * b * k);
    L.par = o;  o = align16(o + 4 * nn);
    L.dep = o;  o = align16(o + 4 * nn);
    L.tok = o;  o = align16(o + 4 * nn);
    L.rho = o;  o = align16(o + 4 * nn);
    L.popm = o; o = align16(o + 4 * nn);
    L.ahat = o; o = align16(o + 8 * nn);
    L.cost = o; o = align16(o + 8 * nn);
    L.total = o;
    return L;
}

// Element s of a wave-distributed array lives in lane s % 64 of register
// s / 64; s must be wave-uniform.
template <int G>
struct LaneArray {
    uint32_t r[G];
    __device__ __forceinline__ void fill(uint32_t v) {
#pragma unroll
        for (int i = 0; i < G; ++i) r[i] = v;
    }
    // every register is touched so that the array never becomes a
    // dynamically indexed (scratch) object
    __device__ __forceinline__ uint32_t get(int s) const {
        const int g = s >> 6, l = s & 63;
        uint32_t v = 0;
#pragma unroll
        for (int i = 0; i < G; ++i) {
            const uint32_t t = uint32_t(__builtin_amdgcn_readlane(int(r[i]), l));
            v = (g == i) ? t : v;
        }
        return v;
    }
    __device__ __forceinline__ void set(int s, uint32_t v) {
        const int g = s >> 6;
        const bool mine = lane_id() == (s & 63);
#pragma unroll
        for (int i = 0; i < G; ++i) r[i] = (mine && g == i) ? v : r[i];
    }
};

constexpr uint32_t kSlowNode = 256u;   // cursor flag: exact sibling order path
constexpr int kDppWaveShl1 = 0x130;     // lane i <- lane i+1 (lane 63 <- old)
constexpr int kDppWaveShr1 = 0x138;     // lane i <- lane i-1 (lane 0 <- old)

// Frontier kept sorted in descending key order: element i (lane i % 64 of
// register i / 64) is the i-th best key, unused elements are 0.  The best
// key is lane 0 of register 0; removing it is one wave shift per register,
// inserting is a compare + ballot + popcount for the position and one
// wave shift per register.
template <int G>
struct SortedFrontier {
    uint32_t h[G], l[G];
    __device__ __forceinline__ void clear() {
#pragma unroll
        for (int g = 0; g < G; ++g) h[g] = l[g] = 0;
    }
    __device__ __forceinline__ uint64_t front() const {
        return (uint64_t(uint32_t(__builtin_amdgcn_readfirstlane(int(h[0])))) << 32) |
               uint32_t(__builtin_amdgcn_readfirstlane(int(l[0])));
    }
    __device__ __forceinline__ void pop_front() {
        int ch = 0, cl = 0;   // lane 0 of the next register
#pragma unroll
        for (int g = G - 1; g >= 0; --g) {
            const int nh = __builtin_amdgcn_readlane(int(h[g]), 0);
            const int nl = __builtin_amdgcn_readlane(int(l[g]), 0);
            h[g] = uint32_t(__builtin_amdgcn_update_dpp(ch, int(h[g]), kDppWaveShl1, 0xF, 0xF, false));
            l[g] = uint32_t(__builtin_amdgcn_update_dpp(cl, int(l[g]), kDppWaveShl1, 0xF, 0xF, false));
            ch = nh;
            cl = nl;
        }
    }
    __device__ __forceinline__ void insert(uint64_t key) {
        const uint32_t kh = uint32_t(key >> 32), kl = uint32_t(key);
        int pos = 0;
#pragma unroll
        for (int g = 0; g < G; ++g) {
            const bool gt = h[g] > kh || (h[g] == kh && l[g] > kl);
            pos += popc64(__ballot(gt));
        }
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
};

template <int G>
struct PopState {
    SortedFrontier<G> F;     // every offered key but `pending`
    uint64_t pending;        // one more offered key (0: none)
    LaneArray<G> nrho;       // float bits of each popped node's rho
    LaneArray<G> ncur;       // rank of the child on offer (| kSlowNode)
    LaneArray<G> qt, tt;     // candidate tables: entry pos * k + j
    uint32_t qf, tf, ql, sf; // lane = position: q / token of rank 0, q of
                             // rank k-1, rank order is safe at this position
    const float *qtab;       // LDS copies of the tables (exact path)
    const int32_t *ttab;
    uint32_t *popm;          // LDS: popped-rank mask of exact-path nodes
    int k;

    // exact path: best child of node n (rho rn, depth dn + 1 children at
    // position dn) among ranks not in `popped`; returns key, sets rank
    __device__ __forceinline__ uint64_t exact_child(int n, float rn, int dn, uint32_t popped,
                                                    int &rank) {
        const int lane = lane_id();
        const bool in = lane < k && !((popped >> lane) & 1u);
        uint64_t key = 0;
        if (in) key = tree_key(__fmul_rn(rn, qtab[dn * k + lane]), dn + 1, ttab[dn * k + lane], n);
        const uint64_t best = wave_max_u64(key);
        rank = best ? __ffsll((unsigned long long)__ballot(in && key == best)) - 1 : 0;
        return best;
    }

    // node n (rho rn, depth dn < b) joins the tree: key of its first child
    __device__ __forceinline__ uint64_t first_child(int n, float rn, int dn) {
        const float q0 = __uint_as_float(uint32_t(__builtin_amdgcn_readlane(int(qf), dn)));
        const float qk = __uint_as_float(uint32_t(__builtin_amdgcn_readlane(int(ql), dn)));
        const uint32_t safe = uint32_t(__builtin_amdgcn_readlane(int(sf), dn));
        uint64_t key;
        uint32_t cur;
        if (safe && __fmul_rn(rn, qk) >= 0x1p-125f) {
            key = tree_key(__fmul_rn(rn, q0), dn + 1, __builtin_amdgcn_readlane(int(tf), dn), n);
            cur = 0;
        } else {
            int rank;
            key = exact_child(n, rn, dn, 0u, rank);
            if (lane_id() == 0) popm[n] = 0u;
            cur = uint32_t(rank) | kSlowNode;
        }
        nrho.set(n, __float_as_uint(rn));
        ncur.set(n, cur);
        return key;
    }

    // the child on offer at node p (at depth d) was popped: key of the next
    __device__ __forceinline__ uint64_t next_child(int p, int d) {
        const uint32_t cur = ncur.get(p);
        const float rp = __uint_as_float(nrho.get(p));
        uint64_t key = 0;
        if (!(cur & kSlowNode)) {
            const int c = int(cur) + 1;
            if (c < k) {
                const int e = (d - 1) * k + c;
                key = tree_key(__fmul_rn(rp, __uint_as_float(qt.get(e))), d, int(tt.get(e)), p);
            }
            ncur.set(p, uint32_t(c));
        } else {
            const uint32_t popped = popm[p] | (1u << (cur & 255u));
            int rank;
            key = exact_child(p, rp, d - 1, popped, rank);
            if (lane_id() == 0) popm[p] = popped;
            ncur.set(p, uint32_t(rank) | kSlowNode);
        }
        return key;
    }

    // take the best offered key (0 when none is left)
    __device__ __forceinline__ uint64_t pop() {
        const uint64_t fr = F.front();
        if (pending > fr) {
            const uint64_t t = pending;
            pending = 0;
            return t;
        }
        if (fr) F.pop_front();
        return fr;
    }

    // new offers: the best of (pending, a, c) stays pending, the rest go to
    // the sorted array
    __device__ __forceinline__ void offer(uint64_t a, uint64_t c) {
        uint64_t x = pending, y = a, z = c;
        if (y > x) { const uint64_t t = x; x = y; y = t; }
        if (z > x) { const uint64_t t = x; x = z; z = t; }
        pending = x;
        if (y) F.insert(y);
        if (z) F.insert(z);
    }
};

template <int G>
__device__ void tree_stage(const BuildParams &P, int q, char *smem) {
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const TreeLayout L = tree_layout(P.b, P.k, P.nmax);
    float *qtab = reinterpret_cast<float *>(smem + L.qtab);
    int32_t *ttab = reinterpret_cast<int32_t *>(smem + L.ttab);
    int32_t *par = reinterpret_cast<int32_t *>(smem + L.par);
    int32_t *dep = reinterpret_cast<int32_t *>(smem + L.dep);
    int32_t *tok = reinterpret_cast<int32_t *>(smem + L.tok);
    float *rho = reinterpret_cast<float *>(smem + L.rho);
    uint32_t *popm = reinterpret_cast<uint32_t *>(smem + L.popm);
    double *ahat = reinterpret_cast<double *>(smem + L.ahat);
    double *cost = reinterpret_cast<double *>(smem + L.cost);
    __shared__ int s_bad, s_nstar, s_status;
    const int b = P.b, k = P.k, bk = b * k;

    const int64_t tk0 = int64_t(q) * bk;
    for (int e = tid; e < bk; e += kThreads) {
        qtab[e] = ld_agent(P.topk_q + tk0 + e);
        ttab[e] = ld_agent(P.topk_ids + tk0 + e);
    }
    const bool online = P.cost != nullptr;
    if (online)
        for (int e = tid; e <= P.nmax; e += kThreads)
            cost[e] = P.cost[int64_t(q) * P.cost_qstride + e];
    if (tid == 0) s_bad = 0;
    __syncthreads();
    if (tid < b && ld_agent(P.row_status + int64_t(q) * b + tid) != BASTION_Q_OK)
        atomicOr(&s_bad, 1);
    __syncthreads();
    const bool bad = s_bad != 0;

    if (!bad && wv == 0) {
        PopState<G> S;
        S.qtab = qtab;
        S.ttab = ttab;
        S.popm = popm;
        S.k = k;
#pragma unroll
        for (int g = 0; g < G; ++g) {
            const int e = lane + kWave * g;
            S.qt.r[g] = e < bk ? __float_as_uint(qtab[e]) : 0u;
            S.tt.r[g] = e < bk ? uint32_t(ttab[e]) : 0u;
        }
        S.qf = S.tf = S.ql = S.sf = 0;
        if (lane < b) {
            const int o = lane * k;
            S.qf = __float_as_uint(qtab[o]);
            S.tf = uint32_t(ttab[o]);
            S.ql = __float_as_uint(qtab[o + k - 1]);
            // rank order is the pop order at this position for every parent
            // whose products stay normal, unless two neighbours are within
            // 2^-22 of each other with the larger token first
            uint32_t safe = 1;
            for (int j = 0; j + 1 < k; ++j) {
                const double a = qtab[o + j], c = qtab[o + j + 1];
                if (ttab[o + j] > ttab[o + j + 1] && a < c * (1.0 + 0x1p-22)) safe = 0;
            }
            S.sf = safe;
        }
        S.F.clear();
        S.pending = 0;
        S.nrho.fill(0);
        S.ncur.fill(0);
        if (lane == 0) {
            par[0] = -1;
            dep[0] = 0;
            tok[0] = -1;
            rho[0] = 1.0f;
            ahat[0] = 1.0;
        }
        S.offer(S.first_child(0, 1.0f, 0), 0);
        int count = 0, nstar = -1, status = BASTION_Q_OK;
        double ah = 1.0;
        double s_prev = online ? (1.0 * P.l_ar) / cost[0] : 0.0;
        while (true) {
            const uint64_t top = S.pop();
            if (top == 0) {
                nstar = count;
                status = count < P.nmax ? BASTION_Q_EXHAUSTED : BASTION_Q_OK;
                break;
            }
            const int p = tree_key_parent(top);
            const int d = tree_key_depth(top);
            const int tkn = tree_key_token(top);
            const float r = tree_key_rho(top);
            const int n = count + 1;
            const double ah_n = ah + double(r);
            if (online) {
                const double s_n = (ah_n * P.l_ar) / cost[n];
                if (n - 1 >= P.nmin && s_n < s_prev) {
                    nstar = n - 1;
                    break;
                }
                s_prev = s_n;
            }
            count = n;
            ah = ah_n;
            if (lane == 0) {
                par[n] = p;
                dep[n] = d;
                tok[n] = tkn;
                rho[n] = r;
                ahat[n] = ah_n;
            }
            if (count == P.nmax) {
                nstar = count;
                break;
            }
            const uint64_t sib = S.next_child(p, d);
            const uint64_t kid = d < b ? S.first_child(n, r, d) : 0;
            S.offer(sib, kid);
        }
        if (lane == 0) {
            s_nstar = nstar;
            s_status = status;
        }
    }
    __syncthreads();
    const int nstar = bad ? 0 : s_nstar;
    const int status = bad ? BASTION_Q_BAD_LOGITS : s_status;
    const int W1 = P.nmax + 1;
    const int64_t o = int64_t(q) * W1;
    for (int i = tid; i < W1; i += kThreads) {
        const bool v = i <= nstar && !bad;
        P.parent[o + i] = v ? (i == 0 ? -1 : par[i]) : -1;
        P.depth[o + i] = v ? (i == 0 ? 0 : dep[i]) : -1;
        P.token[o + i] = v ? (i == 0 ? -1 : tok[i]) : -1;
        P.rho[o + i] = v ? (i == 0 ? 1.0f : rho[i]) : 0.0f;
        P.ahat[o + i] = v ? (i == 0 ? 1.0 : ahat[i]) : 0.0;
    }
    if (bad && tid == 0) {
        P.parent[o] = -1;
        P.depth[o] = 0;
        P.token[o] = -1;
        P.rho[o] = 1.0f;
        P.ahat[o] = 1.0;
    }
    if (tid == 0) {
        P.n_nodes[q] = nstar;
        P.qstatus[q] = status;
    }
    if (P.mask) {
        const int W = (W1 + 31) / 32;
        const int32_t pb = P.pos_base ? P.pos_base[q] : 0;
        for (int e = tid; e < W1 * W; e += kThreads) {
            const int i = e / W, w = e - i * W;
            uint32_t bits = 0;
            int steps = 0;
            if (i <= nstar) {
                int j = i;
                if (j / 32 == w) bits |= 1u << (j & 31);
                while (j > 0 && steps < b) {
                    j = par[j];
                    ++steps;
                    if (j / 32 == w) bits |= 1u << (j & 31);
                }
            }
            P.mask[(o + i) * W + w] = bits;
            if (w == 0) P.position_ids[o + i] = i <= nstar ? pb + steps : -1;
        }
    }
}

// ---------------------------------------------------------------------------
// The kernel.  Block x handles segment x % S of row x / S.
// ---------------------------------------------------------------------------
constexpr int partial_bytes(int k) { return 16 + 8 * k; }

template <typename T, int U, int R>
__global__ __launch_bounds__(kThreads, (R >= 16 ? 2 : 4)) void build_trees_kernel(BuildParams P) {
    extern __shared__ __align__(16) char smem[];
    const int row = blockIdx.x / P.S;
    const int seg = blockIdx.x - row * P.S;
    const int q = row / P.b;
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const char *rowp = P.logits + int64_t(row) * P.row_stride_bytes;

    SegmentResult sr = stream_segment<T, U>(P, rowp, seg, smem);
    WaveScratch<U> *scr = reinterpret_cast<WaveScratch<U> *>(smem);
    uint64_t *cand = scr[0].cand;

    float M = sr.m, Ssum = sr.s;
    int nsel = sr.nsel;
    if (P.S > 1) {
        char *rec = P.partials + (int64_t(row) * P.S + seg) * P.partial_bytes;
        if (wv == 0) {
            if (lane == 0) {
                st_agent(reinterpret_cast<float *>(rec), M);
                st_agent(reinterpret_cast<float *>(rec) + 1, Ssum);
                st_agent(reinterpret_cast<int32_t *>(rec) + 2, nsel);
            }
            if (lane < P.k)
                st_agent(reinterpret_cast<uint64_t *>(rec + 16) + lane,
                         lane < nsel ? cand[lane] : uint64_t(0));
        }
        if (!arrive_last(P.row_ticket + row, uint32_t(P.S))) return;
        // merge the S segment records of this row (wave 0)
        if (wv == 0) {
            const char *base = P.partials + int64_t(row) * P.S * P.partial_bytes;
            float lm = -INFINITY;
            for (int s = lane; s < P.S; s += kWave)
                lm = fmaxf(lm, ld_agent(reinterpret_cast<const float *>(base + int64_t(s) * P.partial_bytes)));
            M = wave_max_f32(lm);
            const float C = scale_ref(M);
            float ls = 0.0f;
            for (int s = lane; s < P.S; s += kWave) {
                const float *r = reinterpret_cast<const float *>(base + int64_t(s) * P.partial_bytes);
                ls += ld_agent(r + 1) * __builtin_amdgcn_exp2f(scale_ref(ld_agent(r)) - C);
            }
            Ssum = wave_sum_f32(ls);
            // keys: append with the same capacity/compaction rule as the stream
            int cnt = 0;
            uint64_t thk = 0, kth;
            const int tot = P.S * P.k;
            for (int e0 = 0; e0 < tot; e0 += kWave) {
                if (cnt + kWave > kCap) {
                    cnt = wave_select_topk<kCap / kWave>(cand, cnt, P.k, kth);
                    thk = kth;
                }
                const int e = e0 + lane;
                uint64_t key = 0;
                if (e < tot) {
                    const int s = e / P.k, j = e - s * P.k;
                    key = ld_agent(reinterpret_cast<const uint64_t *>(base + int64_t(s) * P.partial_bytes + 16) + j);
                }
                const bool p = key != 0 && key > thk;
                const uint64_t msk = __ballot(p);
                if (p) cand[cnt + popc64(msk & lanemask_lt())] = key;
                cnt += popc64(msk);
                wave_sync();
            }
            nsel = wave_select_topk<kCap / kWave>(cand, cnt, P.k, kth);
        }
    }
    // ---- finish the row (wave 0) ----
    if (wv == 0) {
        const bool badrow = (nsel < P.k) || !(Ssum == Ssum) || !(fabsf(M) <= kMaxAbsRowMax);
        const int64_t o = int64_t(row) * P.k;
        if (lane < P.k) {
            if (badrow) {
                st_agent(P.topk_ids + o + lane, int32_t(-1));
                st_agent(P.topk_q + o + lane, 0.0f);
            } else {
                const uint64_t key = cand[lane];
                const float C = scale_ref(M);
                const float e = __builtin_amdgcn_exp2f(__builtin_fmaf(topk_key_value(key), kLog2e, -C));
                st_agent(P.topk_ids + o + lane, topk_key_token(key));
                st_agent(P.topk_q + o + lane, e / Ssum);
            }
        }
        if (lane == 0) {
            const float C = scale_ref(M);
            const float d = __builtin_fmaf(M, kLog2e, -C);   // rounding residual of C
            P.row_max[row] = badrow ? 0.0f : M;
            P.row_sum[row] = badrow ? 0.0f : Ssum * __builtin_amdgcn_exp2f(-d);
            st_agent(P.row_status + row, int32_t(badrow ? BASTION_Q_BAD_LOGITS : BASTION_Q_OK));
        }
    }
    if (!arrive_last(P.query_ticket + q, uint32_t(P.b))) return;
    tree_stage<R>(P, q, smem);
}

// ---------------------------------------------------------------------------
// Host-side launch helpers (called from api.hip).
// ---------------------------------------------------------------------------
template <typename T, int U, int R>
static hipError_t launch_one(const BuildParams &P, int smem, hipStream_t s) {
    auto kern = build_trees_kernel<T, U, R>;
    const int64_t grid = int64_t(P.B) * P.b * P.S;
    hipLaunchKernelGGL(kern, dim3(unsigned(grid)), dim3(kThreads), smem, s, P);
    return hipGetLastError();
}

template <typename T, int U>
static hipError_t launch_r(const BuildParams &P, int smem, hipStream_t s) {
    // lane arrays must hold nmax + 1 slots and b * k table entries
    const int slots = (P.nmax + 1) > (P.b * P.k) ? (P.nmax + 1) : (P.b * P.k);
    if (slots <= 64) return launch_one<T, U, 1>(P, smem, s);
    if (slots <= 128) return launch_one<T, U, 2>(P, smem, s);
    if (slots <= 256) return launch_one<T, U, 4>(P, smem, s);
    if (slots <= 512) return launch_one<T, U, 8>(P, smem, s);
    return launch_one<T, U, 16>(P, smem, s);
}

}  // namespace bastion

// entry used by api.hip
hipError_t bastion_launch_build(const bastion::BuildParams &P, int dtype, hipStream_t s,
                                int *smem_out) {
    using namespace bastion;
    constexpr int U = 4;
    const int stream_smem = int(sizeof(WaveScratch<U>)) * kWavesPerBlock;
    const int tree_smem = tree_layout(P.b, P.k, P.nmax).total;
    const int smem = stream_smem > tree_smem ? stream_smem : tree_smem;
    if (smem_out) *smem_out = smem;
    if (dtype == BASTION_BF16) return launch_r<__bf16, U>(P, smem, s);
    return launch_r<float, U>(P, smem, s);
}
