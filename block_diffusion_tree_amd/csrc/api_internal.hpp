// api_internal.hpp -- entry-point internals shared between the sources of
// libbastion.so (not part of the C ABI).
#pragma once

#include <stddef.h>
#include <stdint.h>

#include "bastion.h"

namespace bastion {

// Supplies the scratch of a call that brings none: given the bytes the call
// needs, sets *ws / *ws_bytes or returns a BASTION_* error.
typedef int32_t (*ScratchSource)(size_t need, void **ws, size_t *ws_bytes);

// bastion_build_trees on the caller's workspace (scratch == nullptr), or on
// the scratch `scratch` supplies, whose arrival counters it clears first.
int32_t build_trees_on(const void *logits, int32_t dtype, int32_t B, int32_t b, int32_t V,
                       int64_t row_stride, int32_t k, int32_t nmax, int32_t nmin,
                       const double *cost, int64_t cost_qstride, double l_ar,
                       const int32_t *pos_base, const bastion_tree_out *out, void *ws,
                       size_t ws_bytes, void *stream, ScratchSource scratch);

}  // namespace bastion
