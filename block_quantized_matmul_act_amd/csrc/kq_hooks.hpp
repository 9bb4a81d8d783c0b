// kq_hooks.hpp -- host-side launchers outside the plain GEMM launch path: the
// loader test hook and the expert-indexed product.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kq {

// Decode nblocks consecutive weight blocks with the tile kernel's loaders
// (kq_gemm.hip): q [nblocks][QK] int8 operands, scales [nblocks][16] int32
// (Q4_K: 8 scales then 8 mins; Q6_K: 16 scales; ternary: not written).
hipError_t launch_debug_unpack(int fmt, const void *W, int64_t nblocks, int8_t *q, int32_t *scales,
                               hipStream_t stream);

// Expert-indexed product (kq_gemm_id) on the tile kernel of kq_gemm.hip
// (Q6_K and ternary formats).
hipError_t launch_gemm_id(int fmt, const void *W, int n_experts, int64_t expert_bytes,
                          const int8_t *qs, const float *da, const uint16_t *alpha,
                          const int32_t *exp_off, const int32_t *rows, int R, float *out, int M,
                          int N, int K, hipStream_t stream);

// Q4_K expert-indexed product on the register-unpack tile kernel
// (kq_gemm_q4k.hip, 64-row tiles in gather mode), for shapes where
// q4k_id_tile_ok(N, K) holds (the API declines the others); K == 0 writes
// zeros.
bool q4k_id_tile_ok(int N, int K);
hipError_t launch_gemm_q4k_id(const void *W, int n_experts, int64_t expert_bytes, const int8_t *qs,
                              const float *da, const uint16_t *alpha, const int32_t *exp_off,
                              const int32_t *rows, int R, float *out, int M, int N, int K,
                              hipStream_t stream);

}  // namespace kq
