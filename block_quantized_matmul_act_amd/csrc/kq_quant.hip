// kq_quant.hip -- activation quantization to int8 blocks (gfx950).
//
// The activation-quant step of vllm.cpp PR 3036 ("cooperative-tile WMMA
// kernels"): fp32 rows become BlockQ8_K-style blocks (256 values, fp32 scale,
// int16 sums per 16) before the tile GEMM; the ternary path of llama.cpp PR
// 214 takes 128-value blocks with an fp32 scale.  Rule per block, in fp32:
// amax = max|x|; d = amax/127 and q = clamp(rint(x*127/amax), +-127), or all
// zero when amax is 0 or 127/amax is not finite.
//
// Layout: one block per group of BS/4 lanes, four consecutive values per lane
// (one 16-byte load), so a 64-lane wave covers one Q8_K block or two Q8_128
// blocks.  amax is a max-reduction across the group (exact, order-free).
// Scales are stored block-major (d[s][m]) so that the GEMM reads the scales
// of a 128-row tile as one contiguous run.  For Q8_K the kernel also writes
// the Q4_K min-term operand alpha = d * (sum of 32 qs) as a bf16 hi/lo pair
// per 32-value sub-block, once per activation instead of once per GEMM tile.
// The kernel is bound by HBM bandwidth: it reads 4 bytes and writes ~1.2
// bytes per value.
#include "kq_device.hpp"

namespace kq {

template <int BS, bool BSUMS>
__global__ __launch_bounds__(256) void quant_act_kernel(const float *__restrict__ x,
                                                        int8_t *__restrict__ qs,
                                                        float *__restrict__ d,
                                                        int16_t *__restrict__ bsums,
                                                        uint16_t *__restrict__ alpha,
                                                        int64_t nblocks_total,
                                                        int64_t blocks_per_row, int64_t M,
                                                        int64_t K) {
    constexpr int LANES = BS / 4;  // lanes per block
    const int lane = threadIdx.x & (LANES - 1);
    const int64_t blk = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) / LANES;
    // Every lane of the block runs the reductions, so no lane returns early.
    const bool valid = blk < nblocks_total;
    const int64_t b = valid ? blk : 0;
    const int64_t row = b / blocks_per_row;
    const int64_t col = (b % blocks_per_row) * BS + 4 * lane;

    v4f v = {0.f, 0.f, 0.f, 0.f};
    if (valid) v = *reinterpret_cast<const v4f *>(x + row * K + col);

    float amax = fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w)));
#pragma unroll
    for (int off = 1; off < LANES; off <<= 1) amax = fmaxf(amax, __shfl_xor(amax, off, 64));

    const float s = 127.0f / amax;
    const bool zero = !(amax > 0.0f) || !isfinite(s);
    int q0 = 0, q1 = 0, q2 = 0, q3 = 0;
    if (!zero) {
        q0 = (int)fminf(fmaxf(rintf(v.x * s), -127.f), 127.f);
        q1 = (int)fminf(fmaxf(rintf(v.y * s), -127.f), 127.f);
        q2 = (int)fminf(fmaxf(rintf(v.z * s), -127.f), 127.f);
        q3 = (int)fminf(fmaxf(rintf(v.w * s), -127.f), 127.f);
    }
    if (valid) {
        uint32_t packed = (uint32_t)(q0 & 0xFF) | ((uint32_t)(q1 & 0xFF) << 8) |
                          ((uint32_t)(q2 & 0xFF) << 16) | ((uint32_t)(q3 & 0xFF) << 24);
        *reinterpret_cast<uint32_t *>(qs + row * K + col) = packed;
    }
    const int64_t sblk = b % blocks_per_row;
    const float dv = zero ? 0.0f : amax / 127.0f;
    if (valid && lane == 0) d[sblk * M + row] = dv;
    if constexpr (BSUMS) {
        // 16 values = 4 lanes; reduce within aligned groups of 4 lanes
        int sum = q0 + q1 + q2 + q3;
        sum += __shfl_xor(sum, 1, 64);
        sum += __shfl_xor(sum, 2, 64);
        if (valid && (lane & 3) == 0) bsums[row * (K / 16) + col / 16] = (int16_t)sum;
        // 32 values = 8 lanes: alpha_j = d * sum32 in fp32, then a bf16 hi/lo pair
        const int sum32 = sum + __shfl_xor(sum, 4, 64);
        const float av = dv * (float)sum32;
        const __bf16 hi = (__bf16)av;
        const __bf16 lo = (__bf16)(av - (float)hi);
        if (valid && (lane & 7) == 0) {
            const int j = lane >> 3;
            alpha[((sblk * 2 + 0) * M + row) * 8 + j] = __builtin_bit_cast(uint16_t, hi);
            alpha[((sblk * 2 + 1) * M + row) * 8 + j] = __builtin_bit_cast(uint16_t, lo);
        }
    }
}

// Host-side launchers (called from kq_api.cpp after validation).
hipError_t launch_quant_act(int bs, const float *x, int8_t *qs, float *d, int16_t *bsums,
                            uint16_t *alpha, int64_t M, int64_t K, hipStream_t stream) {
    const int64_t blocks_per_row = K / bs;
    const int64_t nblocks = M * blocks_per_row;
    const int lanes = bs / 4;
    const int64_t threads = nblocks * lanes;
    const int64_t grid = (threads + 255) / 256;
    if (bs == 256)
        hipLaunchKernelGGL((quant_act_kernel<256, true>), dim3((unsigned)grid), dim3(256), 0,
                           stream, x, qs, d, bsums, alpha, nblocks, blocks_per_row, M, K);
    else
        hipLaunchKernelGGL((quant_act_kernel<128, false>), dim3((unsigned)grid), dim3(256), 0,
                           stream, x, qs, d, bsums, alpha, nblocks, blocks_per_row, M, K);
    return hipGetLastError();
}

}  // namespace kq
