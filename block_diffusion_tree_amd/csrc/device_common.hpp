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

// ---------------------------------------------------------------------------
// Top-k selection inside one wave.  `cand` (LDS) holds `count` unique keys;
// afterwards cand[0..min(k,count)) holds the best of them in descending
// order and the function returns that number.  `kth` receives the k-th key
// (0 when fewer than k keys exist).  Work: k rounds of a wave argmax over
// ceil(count/64) keys per lane.
// ---------------------------------------------------------------------------
template <int PER_LANE>
__device__ __forceinline__ int wave_select_topk(uint64_t *cand, int count, int k, uint64_t &kth) {
    const int lane = lane_id();
    uint64_t kv[PER_LANE];
#pragma unroll
    for (int i = 0; i < PER_LANE; ++i) {
        int e = lane + kWave * i;
        kv[i] = e < count ? cand[e] : 0;
    }
    wave_sync();
    const int nsel = count < k ? count : k;
    uint64_t mine = 0;
    for (int r = 0; r < nsel; ++r) {
        uint64_t lm = kv[0];
#pragma unroll
        for (int i = 1; i < PER_LANE; ++i) lm = kv[i] > lm ? kv[i] : lm;
        uint64_t wm = wave_max_u64(lm);
#pragma unroll
        for (int i = 0; i < PER_LANE; ++i) kv[i] = (kv[i] == wm) ? 0 : kv[i];
        if (lane == r) mine = wm;
    }
    if (lane < nsel) cand[lane] = mine;
    wave_sync();
    uint64_t t = __shfl(mine, (k - 1) & 63, kWave);
    kth = (nsel == k) ? t : 0;
    return nsel;
}

}  // namespace bastion
