// kq_quant.hip -- activation quantization to int8 blocks (gfx950).
//
// The activation-quant step of vllm.cpp PR 3036 ("cooperative-tile WMMA
// kernels"): fp32 rows become BlockQ8_K-style blocks (256 values, fp32 scale,
// int16 sums per 16) before the tile GEMM; the ternary path of llama.cpp PR
// 214 takes 128-value blocks with an fp32 scale.  Rule per block, in fp32:
// amax = max|x|; d = amax/127 and q = clamp(rint(x*127/amax), +-127), or all
// zero when amax is 0 or 127/amax is not finite.
//
// Layout: each lane owns 16 consecutive values (four 16-byte loads, all in
// flight at once), so a block is 16 lanes (Q8_K) or 8 lanes (Q8_128) and a
// per-16 sum is lane-local.  amax is a max across the block's lanes through
// DPP lane permutes (exact and order-free: |x| compared as bit patterns).  A
// wave covers 64 lanes' worth (1024 values) of one row, a workgroup the same
// columns of four rows: the grid is (column chunks x row groups), so no lane
// divides and no wave idles unless K is below 1024.
// Scales are stored block-major (d[s][m]) so that the GEMM reads the scales of
// a 128-row tile as one contiguous run.  For Q8_K the kernel also writes the
// Q4_K min-term operand: the sum B of the 32 qs of each sub-block, split into
// two parts that bf16 holds exactly (64 * floor(B / 64) and B mod 64), so
// that a bf16 matrix-core product with the 6-bit mins gives sum_j m_j B_j
// exactly; written once per activation instead of once per GEMM tile.  The
// kernel is bound by HBM bandwidth: it reads 4 bytes and writes ~1.2 bytes per
// value.
#include "kq_device.hpp"

namespace kq {

namespace {
// DPP controls: quad permutes (lane ^ 1, lane ^ 2 within a quad) and the
// half-row (lane i <- 7 - i in each 8) and row (lane i <- 15 - i in each 16)
// mirrors
constexpr int DPP_QUAD_XOR1 = 0xB1, DPP_QUAD_XOR2 = 0x4E;
constexpr int DPP_ROW_HALF_MIRROR = 0x141, DPP_ROW_MIRROR = 0x140;

template <int CTRL>
__device__ __forceinline__ uint32_t dpp(uint32_t v) {
    return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xF, 0xF, false);
}
}  // namespace

constexpr int QROWS_PER_WG = 4;                       // one row per wave
constexpr int QROWS_PER_LAUNCH = 65535 * QROWS_PER_WG;  // grid.y limit

template <int BS, bool BSUMS>
__global__ __launch_bounds__(256) void quant_act_kernel(const float *__restrict__ x,
                                                        int8_t *__restrict__ qs,
                                                        float *__restrict__ d,
                                                        int16_t *__restrict__ bsums,
                                                        uint16_t *__restrict__ alpha,
                                                        int64_t row0, int64_t M, int64_t K) {
    constexpr int G = BS / 16;  // lanes per block
    const int64_t row = row0 + (int64_t)blockIdx.y * QROWS_PER_WG + (threadIdx.x >> 6);
    const int t = blockIdx.x * 64 + (threadIdx.x & 63);
    const int sblk = t / G, gl = t & (G - 1);
    const int64_t bpr = K / BS;
    // Every lane runs the lane permutes, so no lane returns early.
    const bool valid = sblk < bpr && row < M;
    const int64_t col = (int64_t)sblk * BS + 16 * gl;

    v4f v[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] = v4f{0.f, 0.f, 0.f, 0.f};
    if (valid) {
        const v4f *p = reinterpret_cast<const v4f *>(x + row * K + col);
#pragma unroll
        for (int i = 0; i < 4; ++i) v[i] = p[i];
    }

    uint32_t m = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int e = 0; e < 4; ++e) m = max(m, __builtin_bit_cast(uint32_t, fabsf(v[i][e])));
    m = max(m, dpp<DPP_QUAD_XOR1>(m));
    m = max(m, dpp<DPP_QUAD_XOR2>(m));
    m = max(m, dpp<DPP_ROW_HALF_MIRROR>(m));
    if constexpr (G == 16) m = max(m, dpp<DPP_ROW_MIRROR>(m));
    const float amax = __builtin_bit_cast(float, m);

    const float s = 127.0f / amax;
    const bool zero = !(amax > 0.0f) || !isfinite(s);
    v4i packed = {0, 0, 0, 0};
    int sum = 0;
    if (!zero) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            uint32_t w = 0;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int q = (int)fminf(fmaxf(rintf(v[i][e] * s), -127.f), 127.f);
                sum += q;
                w |= (uint32_t)(q & 0xFF) << (8 * e);
            }
            packed[i] = (int)w;
        }
    }
    const float dv = zero ? 0.0f : amax / 127.0f;
    if (valid) {
        *reinterpret_cast<v4i *>(qs + row * K + col) = packed;
        if (gl == 0) d[sblk * M + row] = dv;
    }
    if constexpr (BSUMS) {
        // this lane's 16 values are one bsums group
        if (valid) bsums[row * (K / 16) + col / 16] = (int16_t)sum;
        // 32 values = lanes 2j, 2j+1: B_j = sum32 (|B_j| <= 4064), parts
        // 64 * floor(B_j / 64) (a 7-bit integer times 64) and B_j mod 64, both
        // exact in bf16
        const int sum32 = sum + (int)dpp<DPP_QUAD_XOR1>((uint32_t)sum);
        const __bf16 p0 = (__bf16)(float)(sum32 & ~63);
        const __bf16 p1 = (__bf16)(float)(sum32 & 63);
        if (valid && (gl & 1) == 0) {
            const int j = gl >> 1;
            alpha[((sblk * 2 + 0) * M + row) * 8 + j] = __builtin_bit_cast(uint16_t, p0);
            alpha[((sblk * 2 + 1) * M + row) * 8 + j] = __builtin_bit_cast(uint16_t, p1);
        }
    }
}

// Host-side launcher (called from kq_api.cpp after validation): rows in
// chunks of the grid's y limit.
hipError_t launch_quant_act(int bs, const float *x, int8_t *qs, float *d, int16_t *bsums,
                            uint16_t *alpha, int64_t M, int64_t K, hipStream_t stream) {
    const int64_t lanes_per_row = (K / bs) * (bs / 16);
    const unsigned gx = (unsigned)((lanes_per_row + 63) / 64);
    for (int64_t r0 = 0; r0 < M; r0 += QROWS_PER_LAUNCH) {
        const int64_t rows = M - r0 < QROWS_PER_LAUNCH ? M - r0 : QROWS_PER_LAUNCH;
        const unsigned gy = (unsigned)((rows + QROWS_PER_WG - 1) / QROWS_PER_WG);
        if (bs == 256)
            hipLaunchKernelGGL((quant_act_kernel<256, true>), dim3(gx, gy), dim3(256), 0, stream, x,
                               qs, d, bsums, alpha, r0, M, K);
        else
            hipLaunchKernelGGL((quant_act_kernel<128, false>), dim3(gx, gy), dim3(256), 0, stream,
                               x, qs, d, bsums, alpha, r0, M, K);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

}  // namespace kq
