// noalloc.hip -- bastion_build_trees_noalloc: bastion_build_trees for
// callers that cannot allocate device memory (code under HIP graph capture,
// tight serving loops, harnesses that forbid hipMalloc).  Its scratch is a
// file-scope device array, one copy per GPU, held until the process ends.
#include <mutex>

#include "device_common.hpp"

#include "api_internal.hpp"

namespace {

constexpr size_t kScratchBytes = size_t(4) << 20;   // 4 MiB per GPU
constexpr int kMaxDevices = 64;

__device__ __align__(256) char scratch[kScratchBytes];

// Device address of `scratch` on each device, taken once per device with the
// device current.  Host code uses only these addresses: the array's name in
// host code is a host-side stand-in, not a device address.
std::mutex g_mu;
void *g_ptr[kMaxDevices];

int32_t scratch_source(size_t need, void **ws, size_t *ws_bytes) {
    if (need > kScratchBytes) return BASTION_EUNSUPPORTED;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return BASTION_EHIP;
    if (dev < 0 || dev >= kMaxDevices) return BASTION_EUNSUPPORTED;
    std::lock_guard<std::mutex> lock(g_mu);
    if (!g_ptr[dev]) {
        void *p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return BASTION_EHIP;
        g_ptr[dev] = p;
    }
    *ws = g_ptr[dev];
    *ws_bytes = kScratchBytes;
    return BASTION_OK;
}

}  // namespace

extern "C" {

int32_t bastion_build_trees_noalloc(const void *logits, int32_t dtype, int32_t B, int32_t b,
                                    int32_t V, int64_t row_stride, int32_t k, int32_t nmax,
                                    int32_t nmin, const double *cost, int64_t cost_qstride,
                                    double l_ar, const int32_t *pos_base,
                                    const bastion_tree_out *out, void *stream) {
    return bastion::build_trees_on(logits, dtype, B, b, V, row_stride, k, nmax, nmin, cost,
                                   cost_qstride, l_ar, pos_base, out, nullptr, 0, stream,
                                   scratch_source);
}

size_t bastion_noalloc_scratch_bytes(void) { return kScratchBytes; }

}  // extern "C"
