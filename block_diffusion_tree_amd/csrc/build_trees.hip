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
// Nothing waits on another block, so the grid needs no co-residency.  The
// latent-mixture call streams its branch rows the same way and then runs its
// per-query stage in a second launch (mixture_kernel).
#include "device_common.hpp"
#include "build_params.hpp"
#include "tree_rounds.hpp"
#include "tree_pool.hpp"
#include "tree_family.hpp"
#include "mixture.hpp"

namespace bastion {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

constexpr int kThreads = 256;               // 4 waves
constexpr int kWavesPerBlock = kThreads / kWave;
constexpr int kCap = 256;                   // per-wave candidate buffer (keys)
#ifndef BASTION_FUSED_STAGED
#define BASTION_FUSED_STAGED 0
#endif
// the staged online build (tree_stage) in the trees of the stream launch too
constexpr bool kFusedStaged = BASTION_FUSED_STAGED != 0;

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

// Block merge of the waves' candidate keys (each wave's list in its own
// scratch, at most 64 keys, counts in n[]), by wave 0: the k best in
// descending order into scr[0].cand; returns their number.  lb: a key that
// at least min(k, all keys) of them reach.
template <int U>
__device__ __forceinline__ int block_topk(WaveScratch<U> *scr, const int *n, int k, uint64_t lb,
                                          uint64_t &kth) {
    const int lane = __lane_id();
    uint64_t kv[kThreads / kWave];
#pragma unroll
    for (int w = 0; w < kThreads / kWave; ++w) kv[w] = lane < n[w] ? scr[w].cand[lane] : 0;
    return wave_topk_keys<kThreads / kWave>(kv, k, lb, scr[0].cand, kth);
}

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
    uint64_t *bth; // the block's best such key (LDS): any wave's k-th best key
                   // bounds the segment's k-th best from below, so every wave
                   // filters with the largest one published
    int cnt;       // keys in ws->cand
    int nstage;
    int head;      // elements of the row before its first 16-byte aligned vector
    bool booted;   // the first tile has set a threshold

    __device__ void compact() {
        uint64_t kth;
        cnt = wave_select_topk<kCap / kWave, true>(ws->cand, cnt, k, kth);
        if (kth > thk) {
            thk = kth;
            thv = topk_key_value(kth);
            if (lane_id() == 0) atomicMax(reinterpret_cast<unsigned long long *>(bth), kth);
        }
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
        // keep the threshold close to the true k-th key seen so far: a
        // compaction costs k rounds of a wave argmax, a looser threshold lets
        // more vectors through to the stage; every 4k + 8 keys measured best
        // (2k + 8: 2 us slower on the main workload, 8k + 8: 3 us)
        if (cnt >= 4 * k + 8) compact();
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
        const uint64_t bk = *bth;   // read early: its latency hides under the tile's work
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
                if (lane_id() == 0) atomicMax(reinterpret_cast<unsigned long long *>(bth), thk);
            }
        }
        if (bk > thk) {
            thk = bk;
            thv = topk_key_value(bk);
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
        }
    }

    // Keys of the vectors a tile staged.  Called after the next tile's loads
    // are out, so that two tiles stay in flight while it runs, and before the
    // next tile stages (the stage holds one tile).
    __device__ __forceinline__ void flush() {
        if (nstage > 0) drain_stage();
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
__device__ __forceinline__ SegmentResult stream_segment(const BuildParams &P, const char *row, int seg, char *smem) {
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

    __shared__ uint64_t s_bth;
    if (tid == 0) s_bth = 0;
    __syncthreads();
    Streamer<T, U> st;
    st.bth = &s_bth;
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
    const int ntot = (n + span - 1) / span;   // tiles, the last one possibly partial
    const int vlo = v_lo;
    // Every tile load is issued unconditionally: a lane past the segment's
    // end reads the segment's last vector instead (the whole wave then reads
    // one line) and its slot is masked to -inf before use.  A load under a
    // condition would make the compiler's wait for a tile also wait for the
    // loads issued after it, and the pair's second tile would then be
    // processed with nothing in flight.
    u32x4 A[U], Bv[U];
    bool okA[U], okB[U];
    auto fill = [&](u32x4 *dst, bool *ok, int t) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int vi = vlo + t * span + u * kThreads + tid;
            ok[u] = vi < v_hi;
            dst[u] = load_vec<T>(rowv, ok[u] ? vi : v_hi - 1);
        }
    };
    auto mask = [&](u32x4 *tl, const bool *ok, int t) {
        if ((t + 1) * span <= n) return;   // full tile
        const u32x4 ninf = {Elem<T>::kNegInfWord, Elem<T>::kNegInfWord, Elem<T>::kNegInfWord,
                            Elem<T>::kNegInfWord};
#pragma unroll
        for (int u = 0; u < U; ++u) tl[u] = ok[u] ? tl[u] : ninf;
    };
    if (ntot > 0) {
        fill(A, okA, 0);
        // The instruction arbiter favours older waves, so the blocks sharing
        // a CU would otherwise finish one after another and leave the CU
        // with a single streaming block at the end.  When the grid fits the
        // machine at once and the segments are long (8 tiles or more: the
        // short ones are latency-bound), each block keeps to a schedule: its
        // share of 6.4 TB/s among the blocks, timed from its start on the
        // 100 MHz real-time counter; a block behind it raises its priority,
        // one ahead of it lowers it (four tiers), which keeps the
        // co-resident blocks level.  Otherwise (larger grids run in rounds
        // of blocks that start at different times) a wave's priority falls
        // as its segment progresses.  (Progress tiers: 0.8 us slower on the
        // 64 x 16 x 151936 bf16 workload; the schedule: 5 us slower on the
        // 256 x 16 x 128256 fp32 sweep, 10 us on the 8-branch mixture; a
        // later start for blocks dispatched later: 1.2 us slower.)
        int tier = -1;
        const bool sched = int(gridDim.x) <= P.resident_blocks && ntot >= 8;
        const uint64_t clk0 = __builtin_amdgcn_s_memrealtime();
        const int64_t tick_pair = int64_t(2) * span * 16 * int(gridDim.x) / 64000;   // 10 ns ticks
        for (int t = 0; t < ntot; t += 2) {
            int nt;
            if (sched) {
                const int64_t lag =
                    int64_t(__builtin_amdgcn_s_memrealtime() - clk0) - int64_t(t / 2) * tick_pair;
                nt = lag > tick_pair ? 0 : lag > 0 ? 1 : lag > -tick_pair ? 2 : 3;
            } else {
                nt = (4 * t) / ntot;
            }
            if (nt != tier) {
                tier = nt;
                if (nt == 0) __builtin_amdgcn_s_setprio(3);
                else if (nt == 1) __builtin_amdgcn_s_setprio(2);
                else if (nt == 2) __builtin_amdgcn_s_setprio(1);
                else __builtin_amdgcn_s_setprio(0);
            }
            fill(Bv, okB, t + 1);
            st.flush();   // the previous pair's second tile
            mask(A, okA, t);
            st.tile(A, vlo + t * span, okA, sm);
            fill(A, okA, t + 2);
            st.flush();
            if (t + 1 < ntot) {
                mask(Bv, okB, t + 1);
                st.tile(Bv, vlo + (t + 1) * span, okB, sm);
            }
        }
        st.flush();
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
    // ---- block merge: top-k (wave 0), bounded below by the block threshold ----
    if (wv == 0) {
        uint64_t kth;
        res.nsel = block_topk<U>(scr, red_n, P.k, s_bth, kth);
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

__device__ __forceinline__ bool arrive_last(uint32_t *ticket, uint32_t total) {
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
// Tree stage (one block per query, the last one to finish a row of it): the
// level-synchronous best-first build of tree_rounds.hpp, parent resolution,
// A_hat, the online stop and the outputs.
// ---------------------------------------------------------------------------
__host__ __device__ inline int align16(int x) { return (x + 15) & ~15; }

// LDS row stride of the q / token tables: k padded to a multiple of 8
__host__ __device__ inline int qrow_stride(int k) { return (k + 7) & ~7; }

__host__ __device__ inline int tree_regs(int nmax) {
    const int need = (nmax + kWave - 1) / kWave;
    return need <= 1 ? 1 : need <= 2 ? 2 : need <= 4 ? 4 : need <= 8 ? 8 : 16;
}

struct TreeLayout {
    int qtab, ttab, col, par, dep, tok, rho, ahat, cost, map, base;
    int pkey, ppar, prho, plrank, ppop, hist, plvl, q0col, fwork, total;
};

// wide: the pool capacity of the trees' own launch (pool_cap_wide)
__host__ __device__ inline TreeLayout tree_layout(int b, int k, int nmax, int threads = kThreads,
                                                  bool wide = false) {
    TreeLayout L;
    const int nn = nmax + 2;
    const int cap = wide ? pool_cap_wide(tree_regs(nmax)) : pool_cap(tree_regs(nmax));
    int o = 0;
    L.qtab = o; o = align16(o + 4 * b * qrow_stride(k));
    L.ttab = o; o = align16(o + 4 * b * qrow_stride(k));
    L.col = o;  o = align16(o + 8 * kWave * tree_regs(nmax));
    L.par = o;  o = align16(o + 4 * nn);
    L.dep = o;  o = align16(o + 4 * nn);
    L.tok = o;  o = align16(o + 4 * nn);
    L.rho = o;  o = align16(o + 4 * nn);
    L.ahat = o; o = align16(o + 8 * nn);
    L.cost = o; o = align16(o + 8 * nn);
    L.map = o;  o = align16(o + 4 * nn);
    L.base = o; o = align16(o + 4 * 40);
    // pool arrays: cap slots, kPoolPad zero keys, one store-sink slot per lane
    const int pslots = cap > 0 ? cap + kPoolPad + kWave : 0;
    L.pkey = o; o = align16(o + 8 * pslots);
    L.ppar = o; o = align16(o + 4 * pslots);
    L.prho = o; o = align16(o + 4 * pslots);
    L.plrank = o; o = align16(o + 4 * pslots);
    L.ppop = o; o = align16(o + 4 * pslots);
    L.hist = o; o = align16(o + (cap > 0 ? 4 * (kHistBins + kWave) : 0));
    L.plvl = o; o = align16(o + (cap > 0 ? 4 * kLvlFloats : 0));
    L.q0col = o; o = align16(o + 3 * 4 * kColLen);   // FamilyCols q0, q1n, t0
    // FamilyWork: cmask, gpre, wtot, flag
    L.fwork = o; o = align16(o + 8 * kFamGroups + 4 * kFamGroups + 4 * kFamRounds * (threads / kWave) + 16);
    L.total = o;
    return L;
}

__device__ __forceinline__ uint32_t *TL_hist(char *smem, const TreeLayout &TL) {
    return reinterpret_cast<uint32_t *>(smem + TL.hist);
}

// The exact round-by-round build of tree_rounds.hpp plus parent resolution:
// pop-order records 1..cnt into S.par/dep/tok/rho; returns cnt (one wave).
template <int G>
__device__ int exact_build(const RoundsLds &S, int b, int k, int nmax) {
    const int lane = lane_id();
    const uint64_t lt = lanemask_lt();
    TopList<G> R;
    const int cnt = rounds_build<G>(R, S, b, k, nmax);
    // rank of every node among the nodes of its depth -> pop index
    int basev = 0;
    for (int d = 1; d <= b; ++d) {
        if (lane == 0) S.base[d] = basev;
#pragma unroll
        for (int g = 0; g < G; ++g) {
            const uint64_t key = (uint64_t(R.h[g]) << 32) | R.l[g];
            const bool v = key != 0 && tree_key_depth(key) == d;
            const uint64_t msk = __ballot(v);
            if (v) S.map[basev + popc64(msk & lt)] = g * kWave + lane + 1;
            basev += popc64(msk);
        }
    }
    wave_sync();
#pragma unroll
    for (int g = 0; g < G; ++g) {
        const int e = g * kWave + lane;
        if (e < cnt) {
            const uint64_t key = (uint64_t(R.h[g]) << 32) | R.l[g];
            const int d = tree_key_depth(key);
            const int pf = tree_key_parent(key);
            int mi = S.base[d - 1] + pf;
            mi = mi < nmax ? mi : nmax;   // a valid tree never needs the clamp
            S.par[e + 1] = d == 1 ? 0 : S.map[mi];
            S.dep[e + 1] = d;
            S.tok[e + 1] = tree_key_token(key);
            S.rho[e + 1] = tree_key_rho(key);
        }
    }
    return cnt;
}

// A_hat[n] = 1 + rho[1] + ... + rho[n], float64, n = 1..cnt (one wave; rho
// and ahat in LDS, pop order).
__device__ void ahat_fill(const float *rho, double *ahat, int cnt) {
    const int lane = lane_id();
    // A_hat: float64 running sum in pop order (the order best-first adds).
    // When the smallest rho is at least 2^(L-30), with 2^L > cnt + 1,
    // every rho is a multiple of ulp(smallest) and every partial sum is
    // below 2^L, so all sums are exact in float64 and a parallel scan
    // gives the same bits as the running sum.
    const uint32_t rb = cnt >= 1 ? __float_as_uint(rho[cnt]) : 0u;
    const int Lb = 32 - __clz(cnt + 1);
    const bool exact = cnt >= 1 && (rb >> 23) != 0u && int(rb >> 23) - 127 >= Lb - 30;
    if (exact) {
        double carry = 1.0;
        for (int c0 = 0; c0 < cnt; c0 += kWave) {
            const int n = c0 + 1 + lane;
            double v = n <= cnt ? double(rho[n]) : 0.0;
#pragma unroll
            for (int sft = 1; sft < kWave; sft <<= 1) {
                const double o = __shfl_up(v, sft);
                v += lane >= sft ? o : 0.0;
            }
            if (n <= cnt) ahat[n] = carry + v;
            carry += __shfl(v, kWave - 1);
        }
    } else if (lane == 0) {
        double ah = 1.0;
        int n = 1;
        for (; n + 8 <= cnt + 1; n += 8) {
            float r[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) r[i] = rho[n + i];
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                ah += double(r[i]);
                ahat[n + i] = ah;
            }
        }
        for (; n <= cnt; ++n) {
            ah += double(rho[n]);
            ahat[n] = ah;
        }
    }
    wave_sync();
}

// Pop-order outputs of one query (records 1..nstar in par/dep/tok/rho/ahat,
// LDS), padding, n_nodes, qstatus and, when requested, the ancestor mask and
// position ids (whole block).
template <int NT = kThreads>
__device__ void emit_tree(const BuildParams &P, int q, const int32_t *par, const int32_t *dep,
                          const int32_t *tok, const float *rho, const double *ahat, int nstar,
                          bool bad, int status) {
    const int tid = threadIdx.x, nmax = P.nmax, b = P.b;
    const int W1 = nmax + 1;
    const int64_t o = int64_t(q) * W1;
    for (int i = tid; i < W1; i += NT) {
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
        constexpr int kRegWords = 8;   // trees of up to 255 nodes
        if (W <= kRegWords && W1 * W > NT) {
            // more (node, word) pairs than threads: one thread per node, a
            // single walk up from the node setting the bits of every word,
            // held in registers
            for (int i = tid; i < W1; i += NT) {
                uint32_t bits[kRegWords];
#pragma unroll
                for (int w = 0; w < kRegWords; ++w) bits[w] = 0u;
                int steps = 0;
                if (i <= nstar) {
                    int j = i;
#pragma unroll
                    for (int w = 0; w < kRegWords; ++w) bits[w] |= (j >> 5) == w ? 1u << (j & 31) : 0u;
                    while (j > 0 && steps < b) {
                        j = par[j];
                        ++steps;
#pragma unroll
                        for (int w = 0; w < kRegWords; ++w)
                            bits[w] |= (j >> 5) == w ? 1u << (j & 31) : 0u;
                    }
                }
#pragma unroll
                for (int w = 0; w < kRegWords; ++w)
                    if (w < W) P.mask[(o + i) * W + w] = bits[w];
                P.position_ids[o + i] = i <= nstar ? pb + steps : -1;
            }
            return;
        }
        // one thread per (node, mask word), each walking up from the node
        for (int e = tid; e < W1 * W; e += NT) {
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

// st: this block's timestamps (stamped build), or null
// STAGED: the staged online build; WIDE: the larger pool (both in the trees'
// own launch)
template <int G, int NT = kThreads, bool STAGED = false, bool WIDE = false>
__device__ __forceinline__ void tree_stage(const BuildParams &P, int q, char *smem, uint64_t *st) {
    (void)st;
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const TreeLayout TL = tree_layout(P.b, P.k, P.nmax, NT, WIDE);
    RoundsLds S;
    S.qtab = reinterpret_cast<float *>(smem + TL.qtab);
    S.ttab = reinterpret_cast<int32_t *>(smem + TL.ttab);
    S.col = reinterpret_cast<uint64_t *>(smem + TL.col);
    S.par = reinterpret_cast<int32_t *>(smem + TL.par);
    S.dep = reinterpret_cast<int32_t *>(smem + TL.dep);
    S.tok = reinterpret_cast<int32_t *>(smem + TL.tok);
    S.rho = reinterpret_cast<float *>(smem + TL.rho);
    S.ahat = reinterpret_cast<double *>(smem + TL.ahat);
    S.cost = reinterpret_cast<double *>(smem + TL.cost);
    S.map = reinterpret_cast<int32_t *>(smem + TL.map);
    S.base = reinterpret_cast<int32_t *>(smem + TL.base);
    __shared__ int s_bad, s_nstar, s_status;
    const int b = P.b, k = P.k, bk = b * k, nmax = P.nmax;

    const int64_t tk0 = int64_t(q) * bk;
    const int kp = qrow_stride(k);
    S.kp = kp;
    constexpr int kPoolCap = WIDE ? pool_cap_wide(G) : pool_cap(G);
    // per-depth columns for the family walks (FamilyCols)
    float *fq0 = reinterpret_cast<float *>(smem + TL.q0col);
    float *fq1n = fq0 + kColLen;
    int32_t *ft0 = reinterpret_cast<int32_t *>(fq1n + kColLen);
    // the row status loads go out with the table loads: one round trip
    const int32_t rst = tid < b ? ld_agent(P.row_status + int64_t(q) * b + tid) : int32_t(BASTION_Q_OK);
    for (int e = tid; e < b * kp; e += NT) {
        const int d = e / kp, j = e - d * kp;
        const float qv = j < k ? ld_agent(P.topk_q + tk0 + d * k + j) : 0.0f;
        const int32_t tv = j < k ? ld_agent(P.topk_ids + tk0 + d * k + j) : 0;
        S.qtab[e] = qv;
        S.ttab[e] = tv;
        if (j == 0) {
            fq0[d] = qv;
            ft0[d] = tv;
        }
        if (j == 1 && d >= 1) fq1n[d - 1] = qv;
    }
    for (int d = tid; d < kColLen; d += NT) {
        if (d >= b) {
            fq0[d] = 0.0f;
            ft0[d] = 0;
        }
        if (d >= b - 1 || k < 2) fq1n[d] = 0.0f;
    }
    FamilyWork FW;
    FW.cmask = reinterpret_cast<uint64_t *>(smem + TL.fwork);
    FW.gpre = reinterpret_cast<int32_t *>(FW.cmask + kFamGroups);
    FW.wtot = FW.gpre + kFamGroups;
    FW.flag = FW.wtot + kFamRounds * (NT / kWave);
    if (kPoolCap > 0) {
        uint32_t *hist = reinterpret_cast<uint32_t *>(smem + TL.hist);
        int32_t *pop = reinterpret_cast<int32_t *>(smem + TL.ppop);
        for (int i = tid; i < kHistBins + kWave; i += NT) hist[i] = 0u;
        for (int i = tid; i < kPoolCap + kPoolPad + kWave; i += NT) pop[i] = 0;
        if (tid == 0) FW.flag[0] = 0;
    }
    const bool online = P.cost != nullptr;
    if (online)
        for (int e = tid; e <= nmax; e += NT)
            S.cost[e] = P.cost[int64_t(q) * P.cost_qstride + e];
    if (tid == 0) s_bad = 0;
    __syncthreads();
    if (rst != BASTION_Q_OK) atomicOr(&s_bad, rst == BASTION_Q_RANGE ? 2 : 1);
    __syncthreads();
    BASTION_STAMP(st, 4);
    const bool bad = s_bad != 0;
    // a bad row outranks a row outside the float32 range
    const int bad_status = (s_bad & 1) ? BASTION_Q_BAD_LOGITS : BASTION_Q_RANGE;

    __shared__ int s_pool, s_pass, s_more;
    // Online stop, staged: best-first trees of budgets n1 < nmax are
    // prefixes of one another (same pop order, same A_hat sums), so if the
    // stop falls inside the first n1 = kStageNodes nodes, the tree of budget
    // n1 is the answer and the full budget is never ranked.  The first stage
    // is skipped when no stop can fall inside it: with at least n1 real
    // nodes at rho >= t1 (the family's bound for n1 nodes), rho(n+1) >= t1
    // and A_hat(n) <= 1 + n rho_1 for n < n1, so S cannot fall while
    // t1 C(n) >= (1 + n rho_1) (C(n+1) - C(n)).
    constexpr int kStageNodes = 32;
    const bool staged = STAGED && online && nmax > kStageNodes;
    PoolLds PL;
    FamilyCols F;
    FamRegs FR;
    float *lvl = nullptr;
    float bound = 0.0f, bound1 = 0.0f;
    if (kPoolCap > 0 && !bad) {
        PL.key = reinterpret_cast<uint64_t *>(smem + TL.pkey);
        PL.par = reinterpret_cast<int32_t *>(smem + TL.ppar);
        PL.rho = reinterpret_cast<float *>(smem + TL.prho);
        PL.lrank = reinterpret_cast<int32_t *>(smem + TL.plrank);
        PL.pop = reinterpret_cast<int32_t *>(smem + TL.ppop);
        PL.hist = reinterpret_cast<uint32_t *>(smem + TL.hist);
        lvl = reinterpret_cast<float *>(smem + TL.plvl);
        F.q0 = fq0;
        F.q1n = fq1n;
        F.t0 = ft0;
        // the trees' own launch also counts two-deviation paths: a tighter bound
        // for deep trees (in the stream launch it measured 1.5-2 us slower)
        bound = family_bound<NT, WIDE>(S.qtab, S.ttab, F, b, k, kp, nmax, PL.hist, lvl, FR, st,
                                 staged ? kStageNodes : 0, &bound1);
        BASTION_STAMP(st, 5);
    }
    // pass 0 is the first stage, pass 1 the whole budget
    int pass0 = 1;
    if (staged) {
        if (tid == 0) s_pass = 1;
        if (!bad && wv == 0) {
            // stage one unless the certificate holds for every n in [nmin, n1)
            const float rho1 = S.qtab[0];
            bool may_stop = !(bound1 > 0.0f);
            for (int n = P.nmin + lane; n < kStageNodes && !may_stop; n += kWave) {
                const double dc = S.cost[n + 1] - S.cost[n];
                may_stop = double(bound1) * S.cost[n] < (1.0 + double(n) * rho1) * (dc > 0.0 ? dc : 0.0);
            }
            const bool any = __ballot(may_stop) != 0;
            if (lane == 0) s_pass = any ? 0 : 1;
        }
        __syncthreads();
        pass0 = s_pass;
    }

    for (int pass = pass0; pass < 2; ++pass) {
        // the best-first tree of budget N from the pool of nodes at or above
        // t (the exact build when there is no pool), its A_hat and the stop
        const int N = pass == 0 ? kStageNodes : nmax;
        int cnt = -1;
        if (kPoolCap > 0 && !bad) {
            const float t = pass == 0 ? bound1 : bound;
            if (pass > pass0) {
                // the second stage starts from the pool state of the first
                int32_t *pop = reinterpret_cast<int32_t *>(smem + TL.ppop);
                for (int i = tid; i < kPoolCap + kPoolPad + kWave; i += NT) pop[i] = 0;
                if (tid == 0) FW.flag[0] = 0;
                __syncthreads();
            }
            // the family usually holds every node at or above the bound; if
            // not, one wave enumerates them level by level
            const int nf = family_select<NT>(PL, S.qtab, S.ttab, F, FW, FR, b, k, kp, t,
                                             kPoolCap, lvl, st);
            BASTION_STAMP(st, 6);
            if (nf >= 1 && nf <= kPoolCap) {
                FamGeom FG;
                int tot;
                FG.D = family_depth(b, k, tot);
                int kD = 1;
                for (int x = 0; x < FG.D; ++x) kD *= k;
                FG.k = k;
                FG.kp = kp;
                FG.firstD = tot - kD;
                FG.topbase = FW.flag[3];
                FG.inv_k = (65536u + uint32_t(k) - 1u) / uint32_t(k);
                FG.lvl = lvl;
                FG.ttab = S.ttab;
                FG.cmask = FW.cmask;
                FG.gpre = FW.gpre;
                cnt = family_rank<NT>(PL, FG, nf, N, t, S.par, S.dep, S.tok, S.rho, st);
            } else if (nf == -1) {
                // one wave while the levels fit it, then the whole block
                __shared__ int s_pw[3];
                if (wv == 0) {
                    PoolWide pw;
                    const int n = pool_enumerate(PL, S.qtab, S.ttab, b, k, kp, t, kPoolCap, pw);
                    if (lane == 0) {
                        s_pool = n;
                        s_pw[0] = pw.lo;
                        s_pw[1] = pw.hi;
                        s_pw[2] = pw.wide ? pw.d : 0;
                    }
                    if (NT == kWave)
                        for (int i = lane; i < kHistBins; i += kWave) PL.hist[i] = 0u;
                } else {
                    // meanwhile the other waves clear pool_rank's bins
                    for (int i = tid - kWave; i < kHistBins; i += NT - kWave) PL.hist[i] = 0u;
                }
                __syncthreads();
                int n = s_pool;
                if (n >= 1 && s_pw[2] > 0)
                    n = pool_wide<NT>(PL, S.qtab, S.ttab, b, k, kp, t, kPoolCap, s_pw[0], s_pw[1],
                                      s_pw[2], n);
                if (n >= 1) cnt = pool_rank<NT>(PL, n, N, t, S.par, S.dep, S.tok, S.rho);
            }
            __syncthreads();
        }

        BASTION_STAMP(st, 7);
        if (!bad && wv == 0) {
            if (cnt < 0) cnt = exact_build<G>(S, b, k, N);
            if (lane == 0) {
                S.par[0] = -1;
                S.dep[0] = 0;
                S.tok[0] = -1;
                S.rho[0] = 1.0f;
                S.ahat[0] = 1.0;
            }
            wave_sync();
            ahat_fill(S.rho, S.ahat, cnt);
            int nstar = cnt;
            bool found = false;
            if (online) {
                // the first n >= nmin with S(n+1) < S(n)
                for (int c0 = 0; c0 < cnt; c0 += kWave) {
                    const int n = c0 + lane;
                    bool dec = false;
                    if (n < cnt && n >= P.nmin) {
                        const double s0 = (S.ahat[n] * P.l_ar) / S.cost[n];
                        const double s1 = (S.ahat[n + 1] * P.l_ar) / S.cost[n + 1];
                        dec = s1 < s0;
                    }
                    const uint64_t msk = __ballot(dec);
                    if (msk) {
                        nstar = c0 + __ffsll((unsigned long long)msk) - 1;
                        found = true;
                        break;
                    }
                }
            }
            if (lane == 0) {
                s_nstar = nstar;
                s_status = (nstar == cnt && cnt < nmax) ? BASTION_Q_EXHAUSTED : BASTION_Q_OK;
                // the first stage decides only a stop inside it or a tree
                // that ended before its budget
                s_more = (pass == 0 && !found && cnt == N) ? 1 : 0;
            }
        }
        __syncthreads();
        if (!staged || bad || s_more == 0) break;
    }
    __syncthreads();
    BASTION_STAMP(st, 8);
    const int nstar = bad ? 0 : s_nstar;
    const int status = bad ? bad_status : s_status;
    emit_tree<NT>(P, q, S.par, S.dep, S.tok, S.rho, S.ahat, nstar, bad, status);
    BASTION_STAMP(st, 9);
}

// Latent-mixture stage of one query (mixture.hpp): prior weights, chains and
// their q_dep, candidate unions with q per branch, and the mixture tree.
template <int NT>
__device__ void mixture_stage(const BuildParams &P, int q, char *smem) {
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int K = P.K, b = P.b, k = P.k, nmax = P.nmax;
    const int C = P.mix_marginal ? k : K * k;
    MixLds M = mix_lds(smem, mix_layout(K, b, k, nmax, C), C);
    const int64_t r0 = int64_t(q) * K * b;
    __shared__ int s_bad, s_ns, s_np;
    __shared__ uint64_t s_tau;
    if (tid == 0) s_bad = 0;
    for (int i = tid; i < b; i += NT) M.cnt[i] = 0;
    __syncthreads();
    // one round trip: row statistics, row status and every position's top-k
    // ids (ids[pos * C + z * k + j] = candidate j of branch z)
    for (int e = tid; e < K * b; e += NT) {
        M.rowm[e] = ld_agent(P.row_ms + 2 * (r0 + e));
        M.rows[e] = ld_agent(P.row_ms + 2 * (r0 + e) + 1);
        const int32_t rst = ld_agent(P.row_status + r0 + e);
        if (rst != BASTION_Q_OK) atomicOr(&s_bad, rst == BASTION_Q_RANGE ? 2 : 1);
    }
    for (int e = tid; e < b * C && !P.mix_marginal; e += NT) {
        const int pos = e / C, c = e - pos * C;
        const int z = c / k, j = c - z * k;
        M.ids[e] = ld_agent(P.topk_ids + (r0 + z * b + pos) * k + j);
    }
    if (wv == 0) {
        // prior weights, float64 softmax: lane z forms exp(prior_z - max);
        // the sum runs in branch order on every lane
        const double pz = lane < K ? double(P.prior[q * K + lane]) : -INFINITY;
        double pm = pz;
#pragma unroll
        for (int o = 32; o >= 1; o >>= 1) pm = fmax(pm, __shfl_xor(pm, o));
        const double ez = lane < K ? exp(pz - pm) : 0.0;
        double ps = 0.0;
        for (int z = 0; z < K; ++z) ps += __shfl(ez, z);
        if (lane < K) {
            const double w = ez / ps;
            M.w[lane] = w;
            M.wq[lane] = float(w);
            P.prior_q[q * K + lane] = float(w);
        }
    }
    __syncthreads();
    const int64_t cbase = int64_t(q) * b * C;
    if (s_bad && P.mix_marginal) {
        // the marginal pass wrote the (empty) candidates; the root alone
        emit_tree<NT>(P, q, M.par, M.dep, M.tok, M.rho, M.ahat, 0, true,
                      (s_bad & 1) ? BASTION_Q_BAD_LOGITS : BASTION_Q_RANGE);
        return;
    }
    if (s_bad) {
        // a bad branch row: no chains, no candidates, the root alone
        for (int e = tid; e < K * b; e += NT) P.chain_tokens[r0 + e] = -1;
        for (int z = tid; z < K; z += NT) P.qdep[q * K + z] = 0.0;
        for (int e = tid; e < b * C; e += NT) P.cand_tokens[cbase + e] = -1;
        for (int e = tid; e < b * C * K; e += NT) P.cand_q[cbase * K + e] = 0.0f;
        for (int i = tid; i < b; i += NT) P.cand_count[int64_t(q) * b + i] = 0;
        if (P.mix_tree)
            emit_tree<NT>(P, q, M.par, M.dep, M.tok, M.rho, M.ahat, 0, true,
                          (s_bad & 1) ? BASTION_Q_BAD_LOGITS : BASTION_Q_RANGE);
        return;
    }
    if (P.mix_marginal) {
        // candidates of the marginal pass: k per position, with every
        // branch's q, into the tables the rounds read
        for (int e = tid; e < b * C; e += NT) {
            const int pos = e / C, c = e - pos * C;
            const int64_t o = (int64_t(q) * b + pos) * C + c;
            M.ctok[e] = P.marg_ids[o];
            for (int z = 0; z < K; ++z) M.cq[(pos * K + z) * C + c] = P.marg_cq[o * K + z];
        }
        for (int i = tid; i < b; i += NT) M.cnt[i] = C;
        __syncthreads();
    } else {
    // chains: the top-1 token of every branch row (chain[z * b + i])
    for (int e = tid; e < K * b; e += NT) {
        const int z = e / b, i = e - z * b;
        const int t = M.ids[i * C + z * k];
        M.chain[e] = t;
        P.chain_tokens[r0 + e] = t;
    }
    if (C <= kWave) {
        // unions, one position per wave at a time: sort the C tokens across
        // the lanes (ascending; padding lanes hold INT_MAX), keep the first of
        // every run of equal tokens
        for (int pos = wv; pos < b; pos += NT / kWave) {
            int t = lane < C ? M.ids[pos * C + lane] : 0x7FFFFFFF;
            t = int(sort64_asc_u32(uint32_t(t)));
            const int prev = __shfl_up(t, 1);
            const bool keep = lane < C && (lane == 0 || prev != t);
            const uint64_t m = __ballot(keep);
            if (keep) M.ctok[pos * C + popc64(m & lanemask_lt())] = t;
            if (lane == 0) M.cnt[pos] = popc64(m);
        }
    } else {
        // unions, every position at once: first occurrences ...
        for (int e = tid; e < b * C; e += NT) {
            const int pos = e / C, c = e - pos * C;
            const int32_t *ids = M.ids + pos * C;
            const int t = ids[c];
            int f = 1;
            for (int c2 = 0; c2 < c; ++c2) f = (ids[c2] == t) ? 0 : f;
            M.first[e] = f;
        }
        __syncthreads();
        // ... then their ascending ranks
        for (int e = tid; e < b * C; e += NT) {
            const int pos = e / C, c = e - pos * C;
            if (M.first[e]) {
                const int32_t *ids = M.ids + pos * C;
                const int32_t *fst = M.first + pos * C;
                const int t = ids[c];
                int r = 0;
                for (int c2 = 0; c2 < C; ++c2) r += (fst[c2] && ids[c2] < t) ? 1 : 0;
                M.ctok[pos * C + r] = t;
                atomicAdd(M.cnt + pos, 1);
            }
        }
    }
    __syncthreads();
    for (int e = tid; e < b * C; e += NT) {
        const int pos = e / C, c = e - pos * C;
        P.cand_tokens[cbase + e] = c < M.cnt[pos] ? M.ctok[e] : -1;
    }
    for (int i = tid; i < b; i += NT) P.cand_count[int64_t(q) * b + i] = M.cnt[i];
    // every logit the stage needs, in batches of independent loads:
    //   chain entries  x < K*K*b: (z, z', i) -> q_i(chain z | z') into qc;
    //   candidate entries: (pos, c, z) -> q_pos(ctok | z) into cand_q
    // (the row's own top-k formula: exp2(l log2e - C) / S)
    {
        constexpr int NB = 16;
        const int nch = K * K * b, tot = nch + b * C * K;
        for (int x0 = 0; x0 < tot; x0 += NB * NT) {
            float lv[NB];
            int lr[NB];
#pragma unroll
            for (int u = 0; u < NB; ++u) {
                // the entry's branch row and token, without branches; an
                // entry past the end or past its position's union re-reads
                // token 0 of the query's first row and is discarded
                const int x = x0 + u * NT + tid;
                const bool ch = x < nch;
                const int zz = x / b, i = x - zz * b;                 // chain entry
                const int y = x - nch;
                const int pc = y / K, zc = y - pc * K;                // candidate entry
                const int pos = pc / C, c = pc - pos * C;
                // (y < 0 for chain entries: clamp what it indexes)
                const int posc = (y >= 0 && pos < b) ? pos : 0;
                const int cc = (y >= 0 && c < C) ? c : 0;
                const int zcc = y >= 0 ? zc : 0;
                const bool cv = !ch && x < tot && cc < M.cnt[posc];
                const int zch = ch ? zz : 0;
                const int row = ch ? (zch - (zch / K) * K) * b + i : zcc * b + posc;
                const int tok = ch ? M.chain[(zch / K) * b + i] : M.ctok[posc * C + cc];
                lr[u] = (ch || cv) ? row : -1;
                lv[u] = mix_logit(P, r0 + (lr[u] >= 0 ? row : 0), lr[u] >= 0 ? tok : 0, P.is_bf16);
            }
#pragma unroll
            for (int u = 0; u < NB; ++u) {
                const int x = x0 + u * NT + tid;
                const float v = lr[u] >= 0
                    ? __builtin_amdgcn_exp2f(__builtin_fmaf(lv[u], kLog2e, -scale_ref(M.rowm[lr[u]]))) /
                          M.rows[lr[u]]
                    : 0.0f;
                if (x < nch) {
                    M.qc[x] = v;
                } else if (x < tot) {
                    // LDS: candidate fastest, so that a wave's lanes (one
                    // candidate each) read consecutive words in the rounds
                    const int y = x - nch;
                    const int pc = y / K, zc = y - pc * K;
                    const int pos = pc / C, c = pc - pos * C;
                    M.cq[(pos * K + zc) * C + c] = v;
                    P.cand_q[cbase * K + y] = v;
                }
            }
        }
    }
    __syncthreads();
    // q_dep: thread (z, z') forms prod_i q_i(chain z | z') in float64
    for (int t = tid; t < K * K; t += NT) {
        double pr = 1.0;
        for (int i = 0; i < b; ++i) pr *= double(M.qc[t * b + i]);
        M.prod[t] = pr;
    }
    __syncthreads();
    for (int z = tid; z < K; z += NT) {
        double qd = 0.0;
        for (int zp = 0; zp < K; ++zp) qd += M.w[zp] * M.prod[z * K + zp];
        P.qdep[q * K + z] = qd;
    }
    }   // unions, gathers and q_dep of the branch chains
    if (!P.mix_tree) return;
    // the tree, round by round (each position's q table is in LDS).  The
    // running list and the parent table are double-buffered: a merge writes
    // the other buffers, which then become the current ones.
    MixLds L = M;
    int nR = 0;
    int np = 1;               // the first tree round has one parent: the root
    bool scan = false;        // parents to be found by a scan of the list
    __shared__ int s_npn;
    for (int i = tid; i < nmax + kMixSurv; i += NT) L.rankb[i] = 0;
    if (tid < K) L.ptab[tid] = 1.0f;
    for (int d = 1; d <= b; ++d) {
        const int pos = d - 1;
        L.cq = M.cq + pos * C * K;
        L.ctok = M.ctok + pos * C;
        const int cnt = M.cnt[pos];
        if (scan && wv == 0) {
            // after a round merged in several parts: the parents are the
            // depth-(d-1) entries, in list order
            const uint64_t lt = lanemask_lt();
            int n = 0;
            for (int e0 = 0; e0 < nR; e0 += kWave) {
                const int e = e0 + lane;
                const bool v = e < nR && tree_key_depth(L.rkey[e]) == d - 1;
                const uint64_t m = __ballot(v);
                if (v) {
                    const int pp = n + popc64(m & lt);
#pragma unroll 8
                    for (int z = 0; z < K; ++z) L.ptab[pp * K + z] = L.rr[e * K + z];
                }
                n += popc64(m);
            }
            if (lane == 0) s_np = n;
        }
        if (tid == 0) {
            s_ns = 0;
            s_npn = 0;
            s_tau = nR == nmax ? L.rkey[nmax - 1] : 0;
        }
        __syncthreads();
        if (scan) np = s_np;
        if (np == 0) break;
        const int total = np * cnt;
        // one pass over all children without barriers: the survivors (keys
        // above the running list's N-th) go to the buffer while it has room,
        // one buffer reservation per wave
        {
            const uint64_t tau = s_tau;
            const uint64_t lt = lanemask_lt();
            // survivors of one wave step: one buffer reservation per wave
            auto keep = [&](bool sv, uint64_t key, int info) {
                const uint64_t m = __ballot(sv);
                if (m) {
                    int slot0 = 0;
                    if (lane == 0) slot0 = atomicAdd(&s_ns, popc64(m));
                    slot0 = __shfl(slot0, 0);
                    const int slot = slot0 + popc64(m & lt);
                    if (sv && slot < kMixSurv) {
                        L.skey[slot] = key;
                        L.sinfo[slot] = info;
                    }
                }
            };
            for (int base = 0; base < total; base += NT) {
                const int idx = base + tid;
                bool sv = false;
                uint64_t key = 0;
                int info = 0;
                if (idx < total) {
                    const int p = idx / cnt, c = idx - p * cnt;
                    const float score = mix_child(L, K, p, c);
                    key = tree_key(score, d, L.ctok[c], p);
                    sv = key > tau;
                    info = (p << 16) | c;
                }
                keep(sv, key, info);
            }
        }
        __syncthreads();
        const int ns = s_ns;
        if (ns <= kMixSurv) {
            scan = false;
            np = 0;
            if (ns > 0) {
                nR = mix_merge<NT>(L, K, nmax, nR, ns, true, &s_npn);
                np = s_npn;
                swap_list(L);
                float *t = L.ptab;
                L.ptab = L.ptab2;
                L.ptab2 = t;
            }
        } else {
            // too many survivors (the list is still filling): chunk by chunk,
            // merging as the buffer fills, which raises the N-th key
            scan = true;
            __syncthreads();
            if (tid == 0) s_ns = 0;
            __syncthreads();
            constexpr int CH = NT < kMixSurv / 2 ? NT : kMixSurv / 2;   // children per chunk
            for (int base = 0; base < total; base += CH) {
                const int idx = base + tid;
                if (tid < CH && idx < total) {
                    const int p = idx / cnt, c = idx - p * cnt;
                    const float score = mix_child(L, K, p, c);
                    const uint64_t key = tree_key(score, d, L.ctok[c], p);
                    if (key > s_tau) {
                        const int slot = atomicAdd(&s_ns, 1);
                        L.skey[slot] = key;
                        L.sinfo[slot] = (p << 16) | c;
                    }
                }
                __syncthreads();
                const int nsc = s_ns;
                // every thread has read the count before the next chunk adds
                // to it, so that all threads take the same branch below
                __syncthreads();
                // merge when the buffer could not take another chunk, at the
                // end of the round, and while the list is not full
                if (nsc > 0 && (nsc > kMixSurv - CH || base + CH >= total || nR < nmax)) {
                    nR = mix_merge<NT>(L, K, nmax, nR, nsc, false, nullptr);
                    swap_list(L);
                    if (tid == 0) {
                        s_ns = 0;
                        s_tau = nR == nmax ? L.rkey[nmax - 1] : 0;
                    }
                    __syncthreads();
                }
            }
        }
        __syncthreads();
    }
    M.rkey = L.rkey;
    if (wv == 0) {
        mix_resolve(M, b, nmax, nR);
        ahat_fill(M.rho, M.ahat, nR);
    }
    __syncthreads();
    emit_tree<NT>(P, q, M.par, M.dep, M.tok, M.rho, M.ahat, nR, false,
              nR < nmax ? BASTION_Q_EXHAUSTED : BASTION_Q_OK);
}

// ---------------------------------------------------------------------------
// The kernel.  Block x handles segment x % S of row x / S.
// ---------------------------------------------------------------------------
constexpr int partial_bytes(int k) { return 16 + 8 * k; }

// MODE 0: trees (tree_stage with R registers); MODE 1: latent mixture.
template <typename T, int U, int R, int MODE>
__global__ __launch_bounds__(kThreads, (R >= 16 ? 2 : 4)) void build_trees_kernel(BuildParams P) {
    extern __shared__ __align__(16) char smem[];
    const int row = blockIdx.x / P.S;
    const int seg = blockIdx.x - row * P.S;
    const int q = row / P.rows_per_query;
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const char *rowp = P.logits + int64_t(row) * P.row_stride_bytes;
    BASTION_STAMP(P.stamps, 0);
    BASTION_STAMP_WHERE(P.stamps);

    SegmentResult sr = stream_segment<T, U>(P, rowp, seg, smem);
    BASTION_STAMP(P.stamps, 1);
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
        // merge the S segment records of this row (wave 0); every load is
        // issued before the first result is used (one round trip)
        if (wv == 0) {
            const char *base = P.partials + int64_t(row) * P.S * P.partial_bytes;
            const int tot = P.S * P.k;
            constexpr int kRegKeys = kCap / kWave;
            const bool in_regs = tot <= kRegKeys * kWave;
            uint64_t kv[kRegKeys];
#pragma unroll
            for (int i = 0; i < kRegKeys; ++i) {
                const int e = i * kWave + lane;
                const int sg = e / P.k, j = e - sg * P.k;
                kv[i] = in_regs && e < tot
                            ? ld_agent(reinterpret_cast<const uint64_t *>(
                                           base + int64_t(sg) * P.partial_bytes + 16) + j)
                            : uint64_t(0);
            }
            // (m, s) of segment `lane` (S <= 64)
            const uint64_t ms = lane < P.S ? ld_agent(reinterpret_cast<const uint64_t *>(
                                                 base + int64_t(lane) * P.partial_bytes))
                                           : uint64_t(0);
            const float lm = lane < P.S ? __uint_as_float(uint32_t(ms)) : -INFINITY;
            M = wave_max_f32(lm);
            const float C = scale_ref(M);
            const float ls = lane < P.S ? __uint_as_float(uint32_t(ms >> 32)) *
                                              __builtin_amdgcn_exp2f(scale_ref(lm) - C)
                                        : 0.0f;
            Ssum = wave_sum_f32(ls);
            uint64_t kth;
            if (in_regs) {
                // a record with k keys bounds the row's k-th best by its last one
                uint64_t last = 0;
#pragma unroll
                for (int i = 0; i < kRegKeys; ++i) {
                    const int e = i * kWave + lane;
                    if (e < tot && e % P.k == P.k - 1 && kv[i] > last) last = kv[i];
                }
                nsel = wave_topk_keys<kRegKeys>(kv, P.k, wave_max_u64(last), cand, kth);
            } else {
                // keys: append with the same capacity/compaction rule as the stream
                int cnt = 0;
                uint64_t thk = 0;
                for (int e0 = 0; e0 < tot; e0 += kWave) {
                    if (cnt + kWave > kCap) {
                        cnt = wave_select_topk<kCap / kWave>(cand, cnt, P.k, kth);
                        thk = kth;
                    }
                    const int e = e0 + lane;
                    uint64_t key = 0;
                    if (e < tot) {
                        const int s = e / P.k, j = e - s * P.k;
                        key = ld_agent(reinterpret_cast<const uint64_t *>(
                                           base + int64_t(s) * P.partial_bytes + 16) + j);
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
    }
    // ---- finish the row (wave 0) ----
    if (wv == 0) {
        // a NaN or +inf entry, or a row of -inf only, is bad input; a finite
        // row max beyond 2^20 is outside the library's float32 range
        const bool invalid = (nsel < P.k) || !(Ssum == Ssum) || !(fabsf(M) <= 3.402823466e38f);
        const bool badrow = invalid || !(fabsf(M) <= kMaxAbsRowMax);
        const int32_t rowst = invalid ? BASTION_Q_BAD_LOGITS : BASTION_Q_RANGE;
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
            st_agent(P.row_status + row, badrow ? rowst : int32_t(BASTION_Q_OK));
            if (P.row_ms) {
                st_agent(P.row_ms + 2 * row, M);
                st_agent(P.row_ms + 2 * row + 1, Ssum);
            }
        }
    }
    BASTION_STAMP(P.stamps, 2);
    // latent mixture: the query stage runs in its own launch (mixture_kernel)
    if constexpr (MODE == 1) return;
    // more blocks than fit the machine at once: trees in their own launch
    if (P.split_trees) return;
    if (!arrive_last(P.query_ticket + q, uint32_t(P.rows_per_query))) return;
    // The query stage is latency-bound and other queries' streams on this CU
    // wait for its results no more than it waits for them: issue ahead of
    // them (a finished stream leaves this block's waves at priority 0).
    __builtin_amdgcn_s_setprio(3);
    BASTION_STAMP(P.stamps, 3);
    tree_stage<R, kThreads, kFusedStaged>(P, q, smem, P.stamps);
}

// ---------------------------------------------------------------------------
// Candidates from the latent mixture's marginal (DBlast page, Methodology 1:
// q_dep mixes the branches with weights q(z|y), so position i's marginal is
// m_i(x) = sum_z q(z|y) q_i(x|y,z)): one block per (query, position), after
// the stream launch left every branch row's max and sum.  The block streams
// the K branch rows of its position together, forms
// m(x) = sum_z (w_z / S_z) 2^(l_z(x) log2 e - c_z) in float32 (w_z / S_z
// rounded once from float64) and keeps the k largest (m desc, token asc)
// with the stream's threshold-filtered candidate buffers.
// ---------------------------------------------------------------------------
template <typename T>
__global__ __launch_bounds__(kThreads) void marginal_kernel(BuildParams P) {
    extern __shared__ __align__(16) char smem[];
    constexpr int U = 4;
    constexpr int E = Elem<T>::kPerVec;
    const int b = P.b, K = P.K, k = P.k, V = P.V;
    const int q = blockIdx.x / b, i = blockIdx.x - q * b;
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int64_t r0 = int64_t(q) * K * b;   // the query's first branch row
    const int64_t ob = (int64_t(q) * b + i) * k;
    __shared__ float s_a[kMaxBranches], s_c[kMaxBranches], s_s[kMaxBranches];
    __shared__ int s_bad;
    __shared__ uint64_t s_bth;
    if (tid == 0) {
        s_bad = 0;
        s_bth = 0;
    }
    __syncthreads();
    for (int e = tid; e < K * b; e += kThreads)
        if (ld_agent(P.row_status + r0 + e) != BASTION_Q_OK) atomicOr(&s_bad, 1);
    if (wv == 0) {
        // prior weights in float64, as the mixture stage forms them
        const double pz = lane < K ? double(P.prior[q * K + lane]) : -INFINITY;
        double pm = pz;
#pragma unroll
        for (int o = 32; o >= 1; o >>= 1) pm = fmax(pm, __shfl_xor(pm, o));
        const double ez = lane < K ? exp(pz - pm) : 0.0;
        double ps = 0.0;
        for (int z = 0; z < K; ++z) ps += __shfl(ez, z);
        if (lane < K) {
            const int64_t row = r0 + int64_t(lane) * b + i;
            const float M = ld_agent(P.row_ms + 2 * row), S = ld_agent(P.row_ms + 2 * row + 1);
            s_c[lane] = scale_ref(M);
            s_s[lane] = S;
            s_a[lane] = float((ez / ps) / double(S));
            if (i == 0) P.prior_q[q * K + lane] = float(ez / ps);
        }
    }
    __syncthreads();
    if (s_bad) {
        for (int j = tid; j < k; j += kThreads) {
            P.marg_ids[ob + j] = -1;
            P.marg_q[ob + j] = 0.0f;
            for (int z = 0; z < K; ++z) P.marg_cq[(ob + j) * K + z] = 0.0f;
        }
        return;
    }
    WaveScratch<U> *scr = reinterpret_cast<WaveScratch<U> *>(smem);
    Streamer<T, U> st;
    st.ws = &scr[wv];
    st.k = k;
    st.thv = -INFINITY;
    st.thk = 0;
    st.cnt = 0;
    st.nstage = 0;
    st.head = 0;
    st.booted = true;
    st.bth = &s_bth;
    const char *base = P.logits + (r0 + i) * P.row_stride_bytes;   // branch z: + z * b rows
    const int64_t zstride = int64_t(b) * P.row_stride_bytes;
    // 16-byte vectors when every row of the position starts on 16 bytes
    const bool vec = ((reinterpret_cast<uintptr_t>(base) | uintptr_t(zstride)) & 15u) == 0;
    const int nvec = vec ? V / E : 0;
    for (int v0 = 0; v0 < nvec; v0 += kThreads) {
        const int v = v0 + tid;
        const bool ok = v < nvec;
        float m[E];
#pragma unroll
        for (int j = 0; j < E; ++j) m[j] = 0.0f;
#pragma unroll 4
        for (int z = 0; z < K; ++z) {
            const u32x4 raw = load_vec<T>(base + z * zstride, ok ? v : nvec - 1);
            float f[E];
            Elem<T>::decode(raw, f);
            const float a = s_a[z], c = s_c[z];
#pragma unroll
            for (int j = 0; j < E; ++j)
                m[j] += a * __builtin_amdgcn_exp2f(__builtin_fmaf(f[j], kLog2e, -c));
        }
        float vmax = m[0];
#pragma unroll
        for (int j = 1; j < E; ++j) vmax = fmaxf(vmax, m[j]);
        const uint64_t bk = s_bth;
        if (bk > st.thk) {
            st.thk = bk;
            st.thv = topk_key_value(bk);
        }
        if (__ballot(ok && vmax >= st.thv)) {
#pragma unroll
            for (int j = 0; j < E; ++j)
                st.offer_scalar(ok && m[j] >= st.thv, m[j], uint32_t(v * E + j));
        }
    }
    // elements after the last vector (or every element of unaligned rows)
    for (int e0 = nvec * E; e0 < V; e0 += kThreads) {
        const int e = e0 + tid;
        const bool ok = e < V;
        float m = 0.0f;
        for (int z = 0; z < K && ok; ++z)
            m += s_a[z] * __builtin_amdgcn_exp2f(
                              __builtin_fmaf(Elem<T>::at(base + z * zstride, e), kLog2e, -s_c[z]));
        st.offer_scalar(ok, m, uint32_t(e));
    }
    if (st.cnt > kWave) st.compact();
    // block merge: wave 0 gathers every wave's keys and selects the k best
    __shared__ int red_n[kWavesPerBlock];
    if (lane == 0) red_n[wv] = st.cnt;
    __syncthreads();
    if (wv == 0) {
        uint64_t kth;
        const int nsel = block_topk<U>(scr, red_n, k, *st.bth, kth);
        if (lane < k) {
            const uint64_t key = lane < nsel ? scr[0].cand[lane] : 0;
            const int tok = lane < nsel ? topk_key_token(key) : -1;
            P.marg_ids[ob + lane] = tok;
            P.marg_q[ob + lane] = lane < nsel ? topk_key_value(key) : 0.0f;
            for (int z = 0; z < K; ++z) {
                // the branch row's own q formula at the token
                const float l = tok >= 0 ? Elem<T>::at(base + z * zstride, tok) : 0.0f;
                P.marg_cq[(ob + lane) * K + z] =
                    tok >= 0 ? __builtin_amdgcn_exp2f(__builtin_fmaf(l, kLog2e, -s_c[z])) / s_s[z]
                             : 0.0f;
            }
        }
    }
}

// The latent-mixture stage, one block per query, launched after the stream
// kernel on the same stream.  A mixture stage is long (every position's
// unions, gathers and a tree round per position); run inside the stream
// kernel it held CU slots and issue cycles that the remaining rows needed.
constexpr int kMixThreads = 1024;   // the stage has a CU to itself: 16 waves per query

__global__ __launch_bounds__(kMixThreads) void mixture_kernel(BuildParams P) {
    extern __shared__ __align__(16) char smem[];
    uint64_t *st = P.stamps ? P.stamps + P.stamp_second * kStampSlots : nullptr;
    (void)st;
    BASTION_STAMP(st, 3);
    mixture_stage<kMixThreads>(P, int(blockIdx.x), smem);
    BASTION_STAMP(st, 9);
}

// The trees of a call whose stream grid does not fit the machine at once,
// one block per query, launched after the stream kernel on the same stream.
// Run by the last row block of a query inside the stream grid, a tree would
// hold a block slot while rows of later queries wait to be dispatched.
// The block has a CU to itself, so it takes 16 waves (8 with the two largest
// running lists, whose registers would not fit 16): the stage's comparison
// and walk loops are latency-bound at one wave per SIMD.
template <int R>
constexpr int tree_threads() { return R >= 8 ? 512 : 1024; }

template <int R>
__global__ __launch_bounds__(tree_threads<R>()) void tree_kernel(BuildParams P) {
    extern __shared__ __align__(16) char smem[];
    uint64_t *st = P.stamps ? P.stamps + P.stamp_second * kStampSlots : nullptr;
    BASTION_STAMP(st, 3);
    tree_stage<R, tree_threads<R>(), true, true>(P, int(blockIdx.x), smem, st);
}

// ---------------------------------------------------------------------------
// Host-side launch helpers (called from api.hip).
// ---------------------------------------------------------------------------
template <typename T, int U, int R, int MODE = 0>
static hipError_t launch_one(const BuildParams &P, int smem, hipStream_t s) {
    auto kern = build_trees_kernel<T, U, R, MODE>;
    const int64_t grid = int64_t(P.B) * P.rows_per_query * P.S;
    hipLaunchKernelGGL(kern, dim3(unsigned(grid)), dim3(kThreads), smem, s, P);
    if (MODE == 0 && P.split_trees) {
        const int tsm = tree_layout(P.b, P.k, P.nmax, tree_threads<R>(), true).total;
        if (tsm > 65536) {
            const hipError_t ea = hipFuncSetAttribute(reinterpret_cast<const void *>(tree_kernel<R>),
                                                      hipFuncAttributeMaxDynamicSharedMemorySize, tsm);
            if (ea != hipSuccess) return ea;
        }
        hipLaunchKernelGGL(tree_kernel<R>, dim3(unsigned(P.B)), dim3(tree_threads<R>()), tsm, s, P);
    }
    return hipGetLastError();
}

template <typename T, int U>
static hipError_t launch_r(const BuildParams &P, int smem, hipStream_t s) {
    // the running top-N list holds nmax keys in tree_regs(nmax) registers
    if (P.mode == 1) {
        const hipError_t e = launch_one<T, U, 1, 1>(P, smem, s);
        if (e != hipSuccess) return e;
        if (P.mix_marginal) {
            hipLaunchKernelGGL(marginal_kernel<T>, dim3(unsigned(P.B * P.b)), dim3(kThreads),
                               int(sizeof(WaveScratch<U>)) * kWavesPerBlock, s, P);
            if (!P.mix_tree) return hipGetLastError();
        }
        const int msmem = mix_layout(P.K, P.b, P.k, P.nmax, P.mix_marginal ? P.k : 0).total;
        if (msmem > 65536) {
            const hipError_t ea = hipFuncSetAttribute(reinterpret_cast<const void *>(mixture_kernel),
                                                      hipFuncAttributeMaxDynamicSharedMemorySize, msmem);
            if (ea != hipSuccess) return ea;
        }
        hipLaunchKernelGGL(mixture_kernel, dim3(unsigned(P.B)), dim3(kMixThreads), msmem, s, P);
        return hipGetLastError();
    }
    switch (tree_regs(P.nmax)) {
        case 1: return launch_one<T, U, 1>(P, smem, s);
        case 2: return launch_one<T, U, 2>(P, smem, s);
        case 4: return launch_one<T, U, 4>(P, smem, s);
        case 8: return launch_one<T, U, 8>(P, smem, s);
        default: return launch_one<T, U, 16>(P, smem, s);
    }
}

}  // namespace bastion

// entry used by api.hip
hipError_t bastion_launch_build(const bastion::BuildParams &P, int dtype, hipStream_t s,
                                int *smem_out) {
    using namespace bastion;
    constexpr int U = 4;
    const int stream_smem = int(sizeof(WaveScratch<U>)) * kWavesPerBlock;
    BuildParams Q = P;
    // trees whose LDS exceeds what a stream block may hold without an
    // attribute (64 KiB; only b = 32, k = 32 with 257 <= nmax <= 512) run in
    // the trees' own launch, which requests its LDS explicitly
    if (Q.mode == 0 && !Q.split_trees && tree_layout(Q.b, Q.k, Q.nmax).total > 65536)
        Q.split_trees = 1;
    // the mixture stage has a launch of its own
    const int tree_smem = (Q.mode == 1 || Q.split_trees) ? 0 : tree_layout(Q.b, Q.k, Q.nmax).total;
    const int smem = stream_smem > tree_smem ? stream_smem : tree_smem;
    if (smem_out) *smem_out = smem;
    if (dtype == BASTION_BF16) return launch_r<__bf16, U>(Q, smem, s);
    return launch_r<float, U>(Q, smem, s);
}
