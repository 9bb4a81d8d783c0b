// kq_launch.hpp -- host-side launchers of the kernels, and the shape rule
// that picks the Q4_K kernel (shared by the launcher and the variant query).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kq {

hipError_t launch_quant_act(int bs, const float *x, int8_t *qs, float *d, int16_t *bsums,
                            uint16_t *alpha, int64_t M, int64_t K, hipStream_t stream);
hipError_t launch_gemm(int fmt, const void *W, const int8_t *qs, const float *da,
                       const uint16_t *alpha, float *out, int M, int N, int K,
                       hipStream_t stream);
hipError_t launch_subsums(int fmt, const void *W, const int8_t *qs, int32_t *sums, int M, int N,
                          int K, hipStream_t stream);

// Q6_K and ternary shapes the matrix-vector kernels take (kq_gemv.hip), and
// their launcher.
bool gemv_choice(int fmt, int M, int N, int K);
hipError_t launch_gemv(int fmt, const void *W, const int8_t *qs, const float *da, float *out,
                       int M, int N, int K, hipStream_t stream);

// Q4_K kernels: one or two tokens with K a multiple of 2048 (and the staged
// activations within the LDS budget) -> matrix-vector kernel; up to 64 ->
// the Q4_K ring kernel on wide weights, the few-token kernel with K split
// over four waves (up to 16 tokens, mid widths) or the ring kernel of
// kq_gemm_ring.hip; otherwise the persistent tile kernel, 128 x 128 or (for
// shapes of at most 256 such tiles) 64 x 128.
// The 64-row tile also has an 8-wave build (one workgroup per CU, two
// superblocks per step) for tile counts that balance better over CUs.
// Ternary (base-3) products with K a multiple of 256 that neither the
// matrix-vector kernel nor the ring kernel (below) takes run on the
// register-unpack tile kernel (kq_gemm_tq.hip).
bool tq_tile_choice(int M, int N, int K);
// The 128 x 128 tile kernel with K in two parts on the grid's second
// dimension, each part adding into the zeroed output (Q6_K and ternary):
// shapes with at most half as many tiles as CUs, K of at least 1024, and
// half of K worth more than the zero fill and atomic adds.
bool tile_split_choice(int fmt, int M, int N, int K);
// Modelled cost of the 128 x 128 tile route (split or whole), in units of K:
// rounds x K, or the split's half K plus its zero fill and atomics.
int64_t tile_units(int fmt, int M, int N, int K);
// out[0, n) = 0, as a kernel (capturable in a graph)
hipError_t launch_zero_fill(float *out, int64_t n, hipStream_t stream);
hipError_t launch_gemm_tq_tile(const void *W, const int8_t *qs, const float *da, float *out, int M, int N,
                               int K, hipStream_t stream);

// Q6_K and ternary products of up to 64 tokens past the matrix-vector
// kernels, and of 65-512 tokens where 64-token slices beat the tile kernels
// (K a multiple of 256): the K-split ring kernel of kq_gemm_ring.hip (fmt:
// the API's format number; ring_slices_pay also takes Q4_K).
bool ring_choice(int fmt, int M, int N, int K);
int ring_parts(int M, int N, int K);
bool ring_slices_pay(int fmt, int M, int N, int K);
// (alpha: the Q4_K min-term operands of the activations; unused otherwise)
hipError_t launch_gemm_ring(int fmt, const void *W, const int8_t *qs, const float *da, const uint16_t *alpha,
                            float *out, int M, int N, int K, hipStream_t stream);

// Compute units of the current device (cached per device; persistent grids
// are sized from it).
int num_cus();

enum Q4KKernel {
    Q4K_TILE128 = 1,
    Q4K_MATVEC = 2,
    Q4K_TILE64 = 3,
    Q4K_TILE64_K2 = 4,
    Q4K_FEW_SPLIT = 5,
    Q4K_FEW_RING = 6,
    Q4K_RING_KP = 7
};
int q4k_kernel_choice(int M, int N, int K);

}  // namespace kq
