// device_common.hpp -- small device helpers shared by the gfx950 kernels:
// order-preserving keys, 64-lane wave reductions and compaction.
//
// Everything here assumes wave64 (gfx950) and blocks whose size is a multiple
// of 64.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "bastion.h"

namespace bastion {

constexpr int kWave = 64;
constexpr float kLog2e = 1.44269504088896340736f;
constexpr float kMaxAbsRowMax = 1048576.0f;  // 2^20

// Kernel-side limits (the host validates against the same numbers).
constexpr int kMaxB = 32;      // positions per block
constexpr int kMaxK = 32;      // candidates per position
constexpr int kMaxNmax = 1023; // non-root nodes
constexpr int kMaxV = 524288;  // tokens (19-bit field in the tree key)
constexpr int kMaxBranches = 16;

// Block timestamps behind the phase table of the stamped build (compiled
// with -DBASTION_STAMPS; absent from the product library).  Thread 0 of the
// block records the 100 MHz real-time counter into its block's slots.
constexpr int kStampSlots = 16;
#ifdef BASTION_STAMPS
#define BASTION_STAMP(stamps, slot)                                                        \
    do {                                                                                   \
        if ((stamps) && threadIdx.x == 0)                                                  \
            (stamps)[size_t(blockIdx.x) * kStampSlots + (slot)] =                          \
                __builtin_amdgcn_s_memrealtime();                                          \
    } while (0)
#define BASTION_STAMP_WHERE(stamps)                                                        \
    do {                                                                                   \
        if ((stamps) && threadIdx.x == 0) {                                                \
            (stamps)[size_t(blockIdx.x) * kStampSlots + 14] =                              \
                uint64_t(__builtin_amdgcn_s_getreg((3 << 11) | 20));  /* XCC_ID */        \
            (stamps)[size_t(blockIdx.x) * kStampSlots + 15] =                              \
                uint64_t(__builtin_amdgcn_s_getreg((31 << 11) | 4));  /* HW_ID */         \
        }                                                                                  \
    } while (0)
#else
#define BASTION_STAMP(stamps, slot) do { } while (0)
#define BASTION_STAMP_WHERE(stamps) do { } while (0)
#endif

__device__ __forceinline__ int lane_id() { return __lane_id(); }

__device__ __forceinline__ uint64_t lanemask_lt() {
    return (uint64_t(1) << lane_id()) - 1;  // lane 0 -> 0
}

__device__ __forceinline__ int popc64(uint64_t m) { return __popcll(m); }

// Orders LDS traffic of one wave: no instruction, only a compiler barrier;
// the LDS unit executes one wave's operations in issue order.
__device__ __forceinline__ void wave_sync() {
    __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
    __builtin_amdgcn_wave_barrier();
}

// ---------------------------------------------------------------------------
// top-k keys: a larger key ranks first.  High word: the logit mapped to an
// unsigned integer with the same order (-0 folded onto +0, so equal logits
// compare equal); low word: ~token, so that among equal logits the smaller
// token ranks first.  0 is "empty" (every real key is at least the key of
// -inf, 0x007FFFFF'xxxxxxxx).
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint32_t ord_f32(float f) {
    uint32_t u = __float_as_uint(f);
    u = (u == 0x80000000u) ? 0u : u;
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ float unord_f32(uint32_t o) {
    uint32_t u = (o & 0x80000000u) ? (o & 0x7FFFFFFFu) : ~o;
    return __uint_as_float(u);
}

__device__ __forceinline__ uint64_t topk_key(float v, uint32_t token) {
    return (uint64_t(ord_f32(v)) << 32) | uint64_t(~token);
}
__device__ __forceinline__ float topk_key_value(uint64_t key) {
    return unord_f32(uint32_t(key >> 32));
}
__device__ __forceinline__ int32_t topk_key_token(uint64_t key) {
    return int32_t(~uint32_t(key));
}

// ---------------------------------------------------------------------------
// Tree keys: a larger key pops first.  Fields, high to low:
//   [63:34] float32 bits of rho, plus 1 (rho < 2, so 30 bits suffice; the +1
//           keeps every real key above the empty key 0)
//   [33:29] 32 - depth       (depth 1..32: shallower first)
//   [28:10] 0x7FFFF - token  (token < 2^19: smaller token first)
//   [9:0]   1023 - parent    (parent index <= 1023: earlier parent first)
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint64_t tree_key(float rho, int depth, int token, int parent) {
    return ((uint64_t(__float_as_uint(rho)) + 1u) << 34) |
           (uint64_t(32 - depth) << 29) |
           (uint64_t(0x7FFFF - token) << 10) |
           uint64_t(1023 - parent);
}
__device__ __forceinline__ float tree_key_rho(uint64_t key) {
    return __uint_as_float(uint32_t((key >> 34) - 1u));
}
__device__ __forceinline__ int tree_key_depth(uint64_t key) {
    return 32 - int((key >> 29) & 31u);
}
__device__ __forceinline__ int tree_key_token(uint64_t key) {
    return 0x7FFFF - int((key >> 10) & 0x7FFFFu);
}
__device__ __forceinline__ int tree_key_parent(uint64_t key) {
    return 1023 - int(key & 1023u);
}

// ---------------------------------------------------------------------------
// Wave reductions (all 64 lanes active), as butterflies on the gfx950
// cross-lane paths: DPP quad permutes and row mirrors inside each 16-lane
// row, then v_permlane16_swap / v_permlane32_swap across rows.  After each
// step every lane of a group holds the group's value, so pairing a lane with
// any lane of the partner group completes the step.  Results are
// wave-uniform.
// ---------------------------------------------------------------------------
constexpr int kDppXor1 = 0xB1;        // quad_perm [1,0,3,2]
constexpr int kDppXor2 = 0x4E;        // quad_perm [2,3,0,1]
constexpr int kDppHalfMirror = 0x141; // row_half_mirror
constexpr int kDppMirror = 0x140;     // row_mirror

template <int CTRL>
__device__ __forceinline__ uint32_t dpp32(uint32_t v) {
    return uint32_t(__builtin_amdgcn_update_dpp(0, int(v), CTRL, 0xF, 0xF, false));
}

// v paired with a lane of the other 16-lane row (16) / other half-wave (32):
// both swap results together hold {own value, partner's value}.
__device__ __forceinline__ void swap16(uint32_t v, uint32_t &a, uint32_t &b) {
    auto r = __builtin_amdgcn_permlane16_swap(v, v, false, false);
    a = r[0];
    b = r[1];
}
__device__ __forceinline__ void swap32(uint32_t v, uint32_t &a, uint32_t &b) {
    auto r = __builtin_amdgcn_permlane32_swap(v, v, false, false);
    a = r[0];
    b = r[1];
}

__device__ __forceinline__ uint64_t max_u64(uint64_t a, uint64_t b) { return a > b ? a : b; }

template <int CTRL>
__device__ __forceinline__ uint64_t dpp64(uint64_t v) {
    return (uint64_t(dpp32<CTRL>(uint32_t(v >> 32))) << 32) | dpp32<CTRL>(uint32_t(v));
}

__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
    v = max_u64(v, dpp64<kDppXor1>(v));
    v = max_u64(v, dpp64<kDppXor2>(v));
    v = max_u64(v, dpp64<kDppHalfMirror>(v));
    v = max_u64(v, dpp64<kDppMirror>(v));
    uint32_t h0, h1, l0, l1;
    swap16(uint32_t(v >> 32), h0, h1);
    swap16(uint32_t(v), l0, l1);
    v = max_u64((uint64_t(h0) << 32) | l0, (uint64_t(h1) << 32) | l1);
    swap32(uint32_t(v >> 32), h0, h1);
    swap32(uint32_t(v), l0, l1);
    return max_u64((uint64_t(h0) << 32) | l0, (uint64_t(h1) << 32) | l1);
}

__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
    v = max(v, dpp32<kDppXor1>(v));
    v = max(v, dpp32<kDppXor2>(v));
    v = max(v, dpp32<kDppHalfMirror>(v));
    v = max(v, dpp32<kDppMirror>(v));
    uint32_t a, b;
    swap16(v, a, b);
    v = max(a, b);
    swap32(v, a, b);
    return max(a, b);
}

__device__ __forceinline__ float wave_max_f32(float v) {
    v = fmaxf(v, __uint_as_float(dpp32<kDppXor1>(__float_as_uint(v))));
    v = fmaxf(v, __uint_as_float(dpp32<kDppXor2>(__float_as_uint(v))));
    v = fmaxf(v, __uint_as_float(dpp32<kDppHalfMirror>(__float_as_uint(v))));
    v = fmaxf(v, __uint_as_float(dpp32<kDppMirror>(__float_as_uint(v))));
    uint32_t a, b;
    swap16(__float_as_uint(v), a, b);
    v = fmaxf(__uint_as_float(a), __uint_as_float(b));
    swap32(__float_as_uint(v), a, b);
    return fmaxf(__uint_as_float(a), __uint_as_float(b));
}

// Sum: IEEE addition is commutative, so the two lanes of each pair compute
// bit-identical partial sums and every lane ends with the same result.
__device__ __forceinline__ float wave_sum_f32(float v) {
    v += __uint_as_float(dpp32<kDppXor1>(__float_as_uint(v)));
    v += __uint_as_float(dpp32<kDppXor2>(__float_as_uint(v)));
    v += __uint_as_float(dpp32<kDppHalfMirror>(__float_as_uint(v)));
    v += __uint_as_float(dpp32<kDppMirror>(__float_as_uint(v)));
    uint32_t a, b;
    swap16(__float_as_uint(v), a, b);
    v = __uint_as_float(a) + __uint_as_float(b);
    swap32(__float_as_uint(v), a, b);
    return __uint_as_float(a) + __uint_as_float(b);
}

// k-th largest of the 64 lane values, ties counted (-inf if fewer than k
// values above -inf).  At most k wave-max rounds.
__device__ __forceinline__ float wave_kth_largest(float v, int k) {
    int found = 0;
    for (int r = 0; r < k; ++r) {
        const float m = wave_max_f32(v);
        if (!(m > -INFINITY)) break;
        found += popc64(__ballot(v == m));
        if (found >= k) return m;
        v = (v == m) ? -INFINITY : v;
    }
    return -INFINITY;
}

// Scale reference of the online softmax: c = fl(m * log2 e), kept finite so
// that rows (or lanes) that have only seen -inf contribute exactly 0.
__device__ __forceinline__ float scale_ref(float m) {
    return fmaxf(m * kLog2e, -3.402823466e38f);
}

// Number of the keys (all lanes, all registers) at or above t.
template <int PER_LANE>
__device__ __forceinline__ int count_ge(const uint64_t (&kv)[PER_LANE], uint64_t t) {
    int c = 0;
#pragma unroll
    for (int i = 0; i < PER_LANE; ++i) c += popc64(__ballot(kv[i] >= t));
    return c;
}

// Top-k by k rounds of a wave argmax, with the contract of wave_topk_keys
// below: less code, and for k <= 4 less time than its search.
template <int PER_LANE>
__device__ __forceinline__ int wave_rounds_topk(const uint64_t (&kv)[PER_LANE], int k,
                                                uint64_t *cand, uint64_t &kth) {
    const int lane = lane_id();
    const int count = count_ge(kv, 1);
    const int nsel = count < k ? count : k;
    uint64_t w[PER_LANE];
#pragma unroll
    for (int i = 0; i < PER_LANE; ++i) w[i] = kv[i];
    uint64_t mine = 0;
    kth = 0;
    for (int r = 0; r < nsel; ++r) {
        uint64_t lm = w[0];
#pragma unroll
        for (int i = 1; i < PER_LANE; ++i) lm = w[i] > lm ? w[i] : lm;
        const uint64_t wm = wave_max_u64(lm);
#pragma unroll
        for (int i = 0; i < PER_LANE; ++i) w[i] = w[i] == wm ? 0 : w[i];
        if (lane == r) mine = wm;
        if (r == k - 1) kth = wm;
    }
    wave_sync();
    if (lane < nsel) cand[lane] = mine;
    wave_sync();
    return nsel;
}

// ---------------------------------------------------------------------------
// Top-k selection inside one wave (k <= 32).  The candidate keys are unique
// and nonzero; kv[i] of lane l holds one of them or 0, PER_LANE per lane.
// Afterwards cand[0..nsel) (LDS, at least 64 slots) holds the best
// nsel = min(k, number of keys) in descending order, and kth the k-th best
// key (0 when there are fewer than k).  lb: a key that at least nsel of the
// keys reach (0 when none is known).
//
// A threshold T with k <= #{keys >= T} <= cap is found by bisecting the key
// range [lb, max] on ballot counts (one compare per register and scalar
// popcounts per probe); the keys at or above T are compacted into cand, and
// each finds its place by counting the larger ones, one wave-uniform key
// at a time.  Ties cannot occur, so the places are a permutation.  For
// k <= 4 the argmax rounds cost less.
// ---------------------------------------------------------------------------
template <int PER_LANE>
__device__ __forceinline__ int wave_topk_keys(const uint64_t (&kv)[PER_LANE], int k, uint64_t lb,
                                              uint64_t *cand, uint64_t &kth) {
    if (k <= 4) return wave_rounds_topk<PER_LANE>(kv, k, cand, kth);
    const int lane = lane_id();
    const int count = count_ge(kv, 1);
    const int nsel = count < k ? count : k;
    const int cap = k <= 8 ? 16 : (k <= 16 ? 32 : 64);
    uint64_t lo = 1;
    int c_lo = count;
    if (count > cap) {
        if (lb > 1) {
            const int c = count_ge(kv, lb);
            if (c >= nsel) {
                lo = lb;
                c_lo = c;
            }
        }
        if (c_lo > cap) {
            uint64_t lm = kv[0];
#pragma unroll
            for (int i = 1; i < PER_LANE; ++i) lm = kv[i] > lm ? kv[i] : lm;
            uint64_t hi = wave_max_u64(lm) + 1;   // no key reaches hi
            // invariant: count_ge(lo) = c_lo > cap >= k > count_ge(hi)
            while (c_lo > cap) {
                const uint64_t mid = lo + ((hi - lo) >> 1);
                const int c = count_ge(kv, mid);
                if (c >= k) {
                    lo = mid;
                    c_lo = c;
                } else {
                    hi = mid;
                }
            }
        }
    }
    // compact the keys >= lo (c_lo of them) into cand[0..c_lo)
    const uint64_t lt = lanemask_lt();
    int base = 0;
#pragma unroll
    for (int i = 0; i < PER_LANE; ++i) {
        const bool p = kv[i] >= lo;
        const uint64_t m = __ballot(p);
        if (p) cand[base + popc64(m & lt)] = kv[i];
        base += popc64(m);
    }
    wave_sync();
    const uint64_t mine = lane < c_lo ? cand[lane] : 0;
    wave_sync();
    // place = number of larger keys (readlane returns int: widen unsigned)
    const uint32_t mlo = uint32_t(mine), mhi = uint32_t(mine >> 32);
    int place = 0;
    for (int j = 0; j < c_lo; ++j) {
        const uint64_t x = (uint64_t(uint32_t(__builtin_amdgcn_readlane(mhi, j))) << 32) |
                           uint64_t(uint32_t(__builtin_amdgcn_readlane(mlo, j)));
        place += x > mine ? 1 : 0;
    }
    if (lane < c_lo && place < nsel) cand[place] = mine;
    const uint64_t km = __ballot(lane < c_lo && place == k - 1);
    kth = 0;
    if (km) {
        const int l = __builtin_amdgcn_readfirstlane(__ffsll((unsigned long long)km) - 1);
        kth = (uint64_t(uint32_t(__builtin_amdgcn_readlane(mhi, l))) << 32) |
              uint64_t(uint32_t(__builtin_amdgcn_readlane(mlo, l)));
    }
    wave_sync();
    return nsel;
}

// The same for `count` keys in cand[0..count) (LDS, count <= 64 * PER_LANE).
// ROUNDS: always the argmax rounds (the compactions inside the streaming
// loop, where the search's code would crowd the loop's registers).
template <int PER_LANE, bool ROUNDS = false>
__device__ __forceinline__ int wave_select_topk(uint64_t *cand, int count, int k, uint64_t &kth,
                                                uint64_t lb = 0) {
    const int lane = lane_id();
    uint64_t kv[PER_LANE];
#pragma unroll
    for (int i = 0; i < PER_LANE; ++i) {
        const int e = lane + kWave * i;
        kv[i] = e < count ? cand[e] : 0;
    }
    wave_sync();
    if (ROUNDS) return wave_rounds_topk<PER_LANE>(kv, k, cand, kth);
    return wave_topk_keys<PER_LANE>(kv, k, lb, cand, kth);
}

}  // namespace bastion
