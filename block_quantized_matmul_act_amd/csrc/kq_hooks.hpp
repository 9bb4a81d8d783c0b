// kq_hooks.hpp -- host-side launchers of test hooks that have no place in the
// GEMM launch path.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kq {

// Decode nblocks consecutive weight blocks with the tile kernel's loaders
// (kq_gemm.hip): q [nblocks][QK] int8 operands, scales [nblocks][16] int32
// (Q4_K: 8 scales then 8 mins; Q6_K: 16 scales; ternary: not written).
hipError_t launch_debug_unpack(int fmt, const void *W, int64_t nblocks, int8_t *q, int32_t *scales,
                               hipStream_t stream);

}  // namespace kq
