// stream_probe.hip -- the practical HBM read ceiling that the tree-drafting
// kernels are compared against: a plain streaming read of a buffer, with the
// same 16-byte nontemporal loads and the same per-block layout as the
// logits stream (each block reads one contiguous chunk, four loads per
// thread in flight per tile, two tiles in flight), and nothing else.  Built
// into its own library (libbastion_probe.so): a measuring tool, not part of
// the method.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
constexpr int kU = 4;   // 16-byte loads per thread per tile

// Block x reads vectors [x * per, min((x + 1) * per, nvec)).  The XOR of
// everything read is stored only if it equals `magic`, which keeps every
// load alive without a store per block.
__global__ __launch_bounds__(kThreads) void stream_read_chunks(const u32x4 *p, int64_t nvec,
                                                               int64_t per, uint32_t magic,
                                                               uint32_t *sink) {
    const int64_t lo = int64_t(blockIdx.x) * per;
    int64_t hi = lo + per;
    hi = hi < nvec ? hi : nvec;
    uint32_t acc = 0;
    const int64_t span = int64_t(kThreads) * kU;
    int64_t v = lo + threadIdx.x;
    for (; v + (2 * kU - 1) * kThreads < hi; v += 2 * span) {
        u32x4 a[2 * kU];
#pragma unroll
        for (int u = 0; u < 2 * kU; ++u) a[u] = __builtin_nontemporal_load(p + v + u * kThreads);
#pragma unroll
        for (int u = 0; u < 2 * kU; ++u) acc ^= a[u][0] ^ a[u][1] ^ a[u][2] ^ a[u][3];
    }
    for (; v < hi; v += kThreads) {
        const u32x4 a = __builtin_nontemporal_load(p + v);
        acc ^= a[0] ^ a[1] ^ a[2] ^ a[3];
    }
    if (acc == magic) sink[blockIdx.x] = acc;
}

}  // namespace

extern "C" {

// Streams `bytes` (a multiple of 16) from the device buffer `buf` with
// `blocks` blocks of 256 threads, each reading one contiguous chunk.
// `sink` needs `blocks` uint32 words (written only on a one-in-2^32 XOR).
int32_t bastion_probe_stream_read(const void *buf, int64_t bytes, int32_t blocks, uint32_t *sink,
                                  void *stream) {
    if (!buf || !sink || bytes < 16 || (bytes & 15) != 0 || blocks < 1) return 1;
    const int64_t nvec = bytes / 16;
    const int64_t per = (nvec + blocks - 1) / blocks;
    hipLaunchKernelGGL(stream_read_chunks, dim3(unsigned(blocks)), dim3(kThreads), 0,
                       static_cast<hipStream_t>(stream), static_cast<const u32x4 *>(buf), nvec,
                       per, 0x9E3779B9u, sink);
    return hipGetLastError() == hipSuccess ? 0 : 3;
}

}  // extern "C"
