// device_common.hpp -- small device helpers shared by the gfx950 kernels:
// order-preserving keys, 64-lane wave reductions and compaction.
//
// Everything here assumes wave64 (gfx950) and blocks whose size is a multiple
// of 64.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/bastion.h"

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
// Wave reductions (all 64 lanes active).  Results are wave-uniform.
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
        uint64_t o = __shfl_xor(v, off, kWave);
        v = o > v ? o : v;
    }
    return v;
}

__device__ __forceinline__ float wave_max_f32(float v) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, kWave));
    return v;
}

__device__ __forceinline__ float wave_sum_f32(float v) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, kWave);
    return v;
}

__device__ __forceinline__ double wave_sum_f64(double v) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, kWave);
    return v;
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
