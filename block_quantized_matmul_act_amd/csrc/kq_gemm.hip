// kq_gemm.hip -- cooperative-tile block-quantized GEMM on gfx950 int8 MFMA.
//
// out[m][n] = sum_k W^[n][k] * A^[m][k] for Q4_K / Q6_K weights against Q8_K
// activations and ternary weights against Q8_128 activations.
//
// Design (MI355X-first; prior art: the BigTile kernel of vllm.cpp PR 3036,
// which reuses staged activation rows across warps, and llama.cpp's
// mul_mat_q, which P1 describes as sharing one cooperatively loaded 128x128
// tile across all warps):
//   * One workgroup computes a BM x BN output tile.  Per K-chunk (256 values:
//     one Q4_K/Q6_K superblock or two ternary blocks) it stages ONE copy of
//     the activation tile and ONE unpacked copy of the weight tile in LDS;
//     every wave reads its MFMA fragments from those copies.
//   * Weights are unpacked once per workgroup into int8 "digit planes" so the
//     per-sub-block scales ride inside the int8 operands:
//       Q4_K: sc*q = 8*(sh*q) + (sl*q)      (sc = 8*sh + sl)
//       Q6_K: sc*(q-32) = 64*h + l          (l in [0,63], h in [-64,64])
//       ternary: t itself (one plane).
//     Two MFMA streams accumulate the two planes over the whole superblock
//     in int32, so the fp32 fold runs once per superblock per output instead
//     of once per sub-block.
//   * Q4_K mins: sum_j m_j * B_j (B_j = sub-block sums of the activations,
//     from the stored int16 bsums) is folded as -dmin*m_j x d_a*B_j through a
//     bf16 MFMA with hi/lo-split operands (~16 significant bits each),
//     accumulating straight into the fp32 output registers; two superblocks
//     share one K=16 MFMA (one per k-group).
//   * Rows >= M and >= N are never read: their LDS rows are zero-filled and
//     the epilogue masks the stores (the ragged-tail staging clamp of
//     vllm.cpp PR 3036).  No wave leaves before a barrier.
//   * blockIdx is remapped so consecutive tiles of one weight column-block
//     land on the same XCD (blocks are dealt round-robin to the 8 XCDs), so
//     a weight tile is fetched from HBM once per XCD L2.
#include "kq_device.hpp"

namespace kq {

enum { FMT_Q4K = 1, FMT_Q6K = 2, FMT_TQ = 3 };

template <int FMT>
struct Fmt;
template <>
struct Fmt<FMT_Q4K> {
    static constexpr int QK = 256, BB = 144, NDIG = 2, SHIFT = 3, SUB = 32;
};
template <>
struct Fmt<FMT_Q6K> {
    static constexpr int QK = 256, BB = 210, NDIG = 2, SHIFT = 6, SUB = 16;
};
template <>
struct Fmt<FMT_TQ> {
    static constexpr int QK = 128, BB = 28, NDIG = 1, SHIFT = 0, SUB = 128;
};

constexpr int KC = 256;         // K values per chunk
constexpr int PITCH = KC + 16;  // LDS row pitch in bytes (16-byte skew against bank conflicts)

struct GemmArgs {
    const uint8_t *W;
    const int8_t *qs;       // activation values  [M][K]
    const float *da;        // activation scales  [M][K/ABS]
    const int16_t *bsums;   // activation sums    [M][K/16]  (Q8_K only)
    void *out;              // fp32 [M][N], or int32 [M][N][K/SUB] for the sub-sum kernel
    int M, N, K;
    int nchunks;            // K / KC (ternary: K / 128 blocks rounded up to chunks)
    int nblk;               // weight blocks per row = K / QK
    int tiles_m, tiles_n;
};

// ---------------------------------------------------------------------------
// Per-thread staging: two threads per weight row, one 16-byte piece per
// activation load.  `unit` replaces the stored scales by 1 (sub-sum kernel).
// ---------------------------------------------------------------------------

template <int FMT>
struct WRaw;

template <>
struct WRaw<FMT_Q4K> {
    v4i hdr;     // d, dmin, 12 scale bytes
    v4i q[4];    // 64 nibble bytes of this thread's half
};
template <>
struct WRaw<FMT_Q6K> {
    uint32_t ql[17], qh[9], sc[3];
    uint32_t dbits;
    uint32_t shift;  // block start mod 4 (0 or 2)
};
template <>
struct WRaw<FMT_TQ> {
    uint32_t w[7];
};

__device__ __forceinline__ uint32_t ld_u32(const uint8_t *p) {
    return *reinterpret_cast<const uint32_t *>(p);
}

// Load this thread's part of weight row `n` (global row index, < N) for chunk c.
template <int FMT>
__device__ __forceinline__ void load_w(WRaw<FMT> &r, const GemmArgs &a, int n, int part,
                                       int c) {
    if constexpr (FMT == FMT_Q4K) {
        const uint8_t *blk = a.W + ((int64_t)n * a.nblk + c) * 144;
        r.hdr = *reinterpret_cast<const v4i *>(blk);
#pragma unroll
        for (int i = 0; i < 4; ++i)
            r.q[i] = *reinterpret_cast<const v4i *>(blk + 16 + 64 * part + 16 * i);
    } else if constexpr (FMT == FMT_Q6K) {
        const int64_t o = ((int64_t)n * a.nblk + c) * 210;
        const uint32_t sh = (uint32_t)(o & 3);
        const uint8_t *base = a.W + (o - sh);  // 4-byte aligned
        r.shift = sh;
        const int h = part;
        const int nq = sh ? 17 : 16, nh = sh ? 9 : 8, ns = sh ? 3 : 2;
#pragma unroll
        for (int i = 0; i < 17; ++i) r.ql[i] = i < nq ? ld_u32(base + 64 * h + 4 * i) : 0u;
#pragma unroll
        for (int i = 0; i < 9; ++i) r.qh[i] = i < nh ? ld_u32(base + 128 + 32 * h + 4 * i) : 0u;
#pragma unroll
        for (int i = 0; i < 3; ++i) r.sc[i] = i < ns ? ld_u32(base + 192 + 8 * h + 4 * i) : 0u;
        r.dbits = *reinterpret_cast<const unsigned short *>(a.W + o + 208);
    } else {
        const int blkidx = 2 * c + part;
        if (blkidx < a.nblk) {
            const uint8_t *blk = a.W + ((int64_t)n * a.nblk + blkidx) * 28;
#pragma unroll
            for (int i = 0; i < 7; ++i) r.w[i] = ld_u32(blk + 4 * i);
        } else {
#pragma unroll
            for (int i = 0; i < 7; ++i) r.w[i] = 0x79797979u;  // bytes 121: five zero trits
            r.w[6] = 0x00007979u;                               // and d = 0
        }
    }
}

// Unpack this thread's part into the LDS digit planes and per-row scalars.
// sw: digit planes [NDIG][rows][PITCH]; plane_stride = rows * PITCH.
// dw: weight block scales [NSC][rows]; beta: Q4_K min operands.
template <int FMT, bool UNIT>
__device__ __forceinline__ void unpack_w(const WRaw<FMT> &r, bool valid, int8_t *sw,
                                         int plane_stride, int nl, int part, float *dw,
                                         int rows, v8bf *beta, int parity, bool zero_odd) {
    int8_t *row0 = sw + nl * PITCH;
    int8_t *row1 = sw + plane_stride + nl * PITCH;
    if constexpr (FMT == FMT_Q4K) {
        const uint32_t w0 = (uint32_t)r.hdr[1], w1 = (uint32_t)r.hdr[2], w2 = (uint32_t)r.hdr[3];
        uint32_t sc[4], mn[4];
        q4k_fields(w0, w1, w2, 4 * part, 4, sc, mn);
        if (UNIT) {
#pragma unroll
            for (int i = 0; i < 4; ++i) sc[i] = 1u;
        }
        if (!valid) {
#pragma unroll
            for (int i = 0; i < 4; ++i) sc[i] = 0u;
        }
#pragma unroll
        for (int cc = 0; cc < 2; ++cc) {
            const int c = 2 * part + cc;  // nibble column: sub-blocks 2c (low) and 2c+1 (high)
#pragma unroll
            for (int g = 0; g < 2; ++g) {
                v4i raw = r.q[2 * cc + g];
                v4i hl, ll, hh, lh;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    uint32_t word = (uint32_t)raw[e];
                    uint32_t lo4 = word & 0x0F0F0F0Fu, hi4 = (word >> 4) & 0x0F0F0F0Fu;
                    uint32_t dh, dl;
                    q4k_digits(lo4, sc[2 * cc], dh, dl);
                    hl[e] = (int)dh;
                    ll[e] = (int)dl;
                    q4k_digits(hi4, sc[2 * cc + 1], dh, dl);
                    hh[e] = (int)dh;
                    lh[e] = (int)dl;
                }
                const int k0 = 64 * c + 16 * g;
                *reinterpret_cast<v4i *>(row0 + k0) = hl;
                *reinterpret_cast<v4i *>(row1 + k0) = ll;
                *reinterpret_cast<v4i *>(row0 + k0 + 32) = hh;
                *reinterpret_cast<v4i *>(row1 + k0 + 32) = lh;
            }
        }
        if (part == 0)
            dw[nl] = valid ? (UNIT ? 1.0f : f16_bits_to_f32((uint32_t)r.hdr[0])) : 0.0f;
        if (!UNIT && beta) {
            const float dmin = valid ? f16_bits_to_f32((uint32_t)r.hdr[0] >> 16) : 0.0f;
            __bf16 hi[4], lo[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) split_bf16(-dmin * (float)mn[i], hi[i], lo[i]);
            // beta[hl][row][parity] holds 8 bf16 (one per sub-block); this part owns 4
            __bf16 *bh = reinterpret_cast<__bf16 *>(&beta[(0 * rows + nl) * 2 + parity]) + 4 * part;
            __bf16 *bl = reinterpret_cast<__bf16 *>(&beta[(1 * rows + nl) * 2 + parity]) + 4 * part;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                bh[i] = hi[i];
                bl[i] = lo[i];
            }
            if (zero_odd) {
                __bf16 *zh = reinterpret_cast<__bf16 *>(&beta[(0 * rows + nl) * 2 + 1]) + 4 * part;
                __bf16 *zl = reinterpret_cast<__bf16 *>(&beta[(1 * rows + nl) * 2 + 1]) + 4 * part;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    zh[i] = (__bf16)0.0f;
                    zl[i] = (__bf16)0.0f;
                }
            }
        }
    } else if constexpr (FMT == FMT_Q6K) {
        const int h = part;
        const uint32_t sh = r.shift;
        // realign to the block's byte 0
        uint32_t ql[16], qh[8], scw[2];
#pragma unroll
        for (int i = 0; i < 16; ++i) ql[i] = sh ? __builtin_amdgcn_alignbyte(r.ql[i + 1], r.ql[i], 2) : r.ql[i];
#pragma unroll
        for (int i = 0; i < 8; ++i) qh[i] = sh ? __builtin_amdgcn_alignbyte(r.qh[i + 1], r.qh[i], 2) : r.qh[i];
#pragma unroll
        for (int i = 0; i < 2; ++i) scw[i] = sh ? __builtin_amdgcn_alignbyte(r.sc[i + 1], r.sc[i], 2) : r.sc[i];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
#pragma unroll
            for (int g = 0; g < 2; ++g) {
                const int j = 2 * u + g;  // sub-block within this half (0..7)
                int sc = (int)(int8_t)((scw[j >> 2] >> (8 * (j & 3))) & 0xFF);
                if (UNIT) sc = 1;
                if (!valid) sc = 0;
                v4i vh, vl;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int t4 = 4 * g + e;  // dword index within the 32-wide group
                    const uint32_t qlw = ql[8 * (u & 1) + t4];
                    const uint32_t lo4 = (u < 2) ? (qlw & 0x0F0F0F0Fu) : ((qlw >> 4) & 0x0F0F0F0Fu);
                    const uint32_t hi2 = (qh[t4] >> (2 * u)) & 0x03030303u;
                    const uint32_t q4 = lo4 | (hi2 << 4);
                    uint32_t dh, dl;
                    q6k_digits(q4, sc, dh, dl);
                    vh[e] = (int)dh;
                    vl[e] = (int)dl;
                }
                const int k0 = 128 * h + 32 * u + 16 * g;
                *reinterpret_cast<v4i *>(row0 + k0) = vh;
                *reinterpret_cast<v4i *>(row1 + k0) = vl;
            }
        }
        if (part == 0) dw[nl] = valid ? (UNIT ? 1.0f : f16_bits_to_f32(r.dbits)) : 0.0f;
    } else {
        // ternary: 26 digit bytes + fp16 d; this part is one 128-block
        uint32_t f[26];
#pragma unroll
        for (int b = 0; b < 26; ++b) f[b] = tq_fixed((r.w[b >> 2] >> (8 * (b & 3))) & 0xFFu);
        int8_t *dst = row0 + 128 * part;
#pragma unroll
        for (int q = 0; q < 8; ++q) {
            v4i v;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                uint32_t word = 0;
#pragma unroll
                for (int bb = 0; bb < 4; ++bb) {
                    const int k = 16 * q + 4 * e + bb;
                    const int byte = k / 5, pos = k % 5;
                    uint32_t dig;
                    switch (pos) {
                        case 0: dig = tq_digit<0>(f[byte]); break;
                        case 1: dig = tq_digit<1>(f[byte]); break;
                        case 2: dig = tq_digit<2>(f[byte]); break;
                        case 3: dig = tq_digit<3>(f[byte]); break;
                        default: dig = tq_digit<4>(f[byte]); break;
                    }
                    word |= dig << (8 * bb);
                }
                v[e] = valid ? (int)digits_to_trits(word) : 0;
            }
            *reinterpret_cast<v4i *>(dst + 16 * q) = v;
        }
        dw[part * rows + nl] = valid ? (UNIT ? 1.0f : f16_bits_to_f32(r.w[6] >> 16)) : 0.0f;
    }
}

// Activation staging for one 16-byte piece of row m, chunk c; zero for rows
// >= M and for the part of a ternary chunk past K (K % 256 == 128).
__device__ __forceinline__ v4i load_act_piece(const GemmArgs &a, int m, int c, int piece) {
    const int k = c * KC + 16 * piece;
    if (m >= a.M || k >= a.K) return v4i{0, 0, 0, 0};
    return *reinterpret_cast<const v4i *>(a.qs + (int64_t)m * a.K + k);
}

// ---------------------------------------------------------------------------
// Main kernel
// ---------------------------------------------------------------------------

template <int FMT>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1))) void gemm_kernel(
    GemmArgs a) {
    constexpr int BM = 128, BN = 128, NT = 256;
    constexpr int NDIG = Fmt<FMT>::NDIG;
    constexpr int NSC = (FMT == FMT_TQ) ? 2 : 1;  // scale sets per chunk
    constexpr int APIECES = BM * (KC / 16) / NT;  // 16-byte activation pieces per thread

    __shared__ __attribute__((aligned(16))) int8_t s_a[BM * PITCH];
    __shared__ __attribute__((aligned(16))) int8_t s_w[NDIG * BN * PITCH];
    __shared__ __attribute__((aligned(16))) float s_da[NSC * BM];
    __shared__ __attribute__((aligned(16))) float s_dw[NSC * BN];
    __shared__ v8bf s_alpha[(FMT == FMT_Q4K) ? 2 * BM * 2 : 1];
    __shared__ v8bf s_beta[(FMT == FMT_Q4K) ? 2 * BN * 2 : 1];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;

    // XCD-aware tile order: blocks are dealt round-robin over 8 XCDs, so give
    // XCD x the contiguous tile range [x*q, (x+1)*q); M-tiles vary fastest.
    const int nwg = gridDim.x;
    const int wg = blockIdx.x;
    const int q8 = nwg >> 3;
    const int tile = (wg < 8 * q8) ? ((wg & 7) * q8 + (wg >> 3)) : wg;
    const int tm = tile % a.tiles_m;
    const int tn = tile / a.tiles_m;
    const int m0 = tm * BM, n0 = tn * BN;

    // staging roles
    const int wn_row = tid >> 1, wpart = tid & 1;
    const bool wvalid = (n0 + wn_row) < a.N;
    const int wn_glob = wvalid ? (n0 + wn_row) : 0;

    // compute roles
    const int wm = wave >> 1, wnn = wave & 1;
    const int lrow = lane & 31, kgrp = lane >> 5;

    v16f acc_f[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc_f[i][j][r] = 0.0f;

    // register prefetch of one chunk
    v4i act[APIECES];
    float da_reg[NSC];
    v4i bs_reg;  // Q4_K: this thread's 8 int16 bsums
    float da_bs = 0.f;
    WRaw<FMT> wr;

    auto prefetch = [&](int c) {
#pragma unroll
        for (int i = 0; i < APIECES; ++i) {
            const int p = tid + NT * i;
            const int row = p >> 4, piece = p & 15;
            const int m = m0 + row;
            act[i] = load_act_piece(a, m, c, piece);
        }
        if (tid < BM) {
            const int m = m0 + tid;
            if constexpr (FMT == FMT_TQ) {
#pragma unroll
                for (int s = 0; s < 2; ++s) {
                    const int b = 2 * c + s;
                    da_reg[s] = (m < a.M && b < a.nblk) ? a.da[(int64_t)m * a.nblk + b] : 0.0f;
                }
            } else {
                da_reg[0] = (m < a.M) ? a.da[(int64_t)m * a.nchunks + c] : 0.0f;
            }
        }
        if constexpr (FMT == FMT_Q4K) {
            const int row = tid >> 1, half = tid & 1;
            const int m = m0 + row;
            if (m < a.M) {
                bs_reg = *reinterpret_cast<const v4i *>(a.bsums + (int64_t)m * (a.K / 16) +
                                                        16 * c + 8 * half);
                da_bs = a.da[(int64_t)m * a.nchunks + c];
            } else {
                bs_reg = v4i{0, 0, 0, 0};
                da_bs = 0.f;
            }
        }
        load_w<FMT>(wr, a, wn_glob, wpart, c);
    };

    auto stage = [&](int c) {
#pragma unroll
        for (int i = 0; i < APIECES; ++i) {
            const int p = tid + NT * i;
            const int row = p >> 4, piece = p & 15;
            *reinterpret_cast<v4i *>(s_a + row * PITCH + 16 * piece) = act[i];
        }
        if (tid < BM) {
#pragma unroll
            for (int s = 0; s < NSC; ++s) s_da[s * BM + tid] = da_reg[s];
        }
        const int parity = c & 1;
        const bool zero_odd = (parity == 0) && (c == a.nchunks - 1);
        if constexpr (FMT == FMT_Q4K) {
            // alpha_j = d_a * (bsums[2j] + bsums[2j+1]) for this thread's 4 sub-blocks
            const int row = tid >> 1, half = tid & 1;
            __bf16 *ah = reinterpret_cast<__bf16 *>(&s_alpha[(0 * BM + row) * 2 + parity]) + 4 * half;
            __bf16 *al = reinterpret_cast<__bf16 *>(&s_alpha[(1 * BM + row) * 2 + parity]) + 4 * half;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const uint32_t wv = (uint32_t)bs_reg[i];
                const int b = (int)(int16_t)(wv & 0xFFFF) + (int)(int16_t)(wv >> 16);
                __bf16 hi, lo;
                split_bf16(da_bs * (float)b, hi, lo);
                ah[i] = hi;
                al[i] = lo;
            }
            if (zero_odd) {
                __bf16 *zh = reinterpret_cast<__bf16 *>(&s_alpha[(0 * BM + row) * 2 + 1]) + 4 * half;
                __bf16 *zl = reinterpret_cast<__bf16 *>(&s_alpha[(1 * BM + row) * 2 + 1]) + 4 * half;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    zh[i] = (__bf16)0.0f;
                    zl[i] = (__bf16)0.0f;
                }
            }
        }
        unpack_w<FMT, false>(wr, wvalid, s_w, BN * PITCH, wn_row, wpart, s_dw, BN,
                             (FMT == FMT_Q4K) ? s_beta : nullptr, parity, zero_odd);
    };

    // int32 accumulators for the digit planes
    v16i acc_i[NDIG][2][2];

    auto fold = [&](int s) {
        // out += (T as fp32) * d_a[m] * d_w[n], T = (plane0 << SHIFT) + plane1
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const float dwv = s_dw[s * BN + 64 * wnn + 32 * j + lrow];
#pragma unroll
            for (int i = 0; i < 2; ++i) {
#pragma unroll
                for (int r4 = 0; r4 < 4; ++r4) {
                    const v4f dav = *reinterpret_cast<const v4f *>(
                        &s_da[s * BM + 64 * wm + 32 * i + 8 * r4 + 4 * kgrp]);
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int r = 4 * r4 + e;
                        int T;
                        if constexpr (NDIG == 2)
                            T = (acc_i[0][i][j][r] << Fmt<FMT>::SHIFT) + acc_i[1][i][j][r];
                        else
                            T = acc_i[0][i][j][r];
                        acc_f[i][j][r] = fmaf((float)T, dav[e] * dwv, acc_f[i][j][r]);
                    }
                }
            }
        }
    };

    if (a.nchunks > 0) prefetch(0);

    for (int c = 0; c < a.nchunks; ++c) {
        __syncthreads();
        stage(c);
        __syncthreads();
        if (c + 1 < a.nchunks) prefetch(c + 1);

        constexpr int KSTEPS = KC / 32;
        constexpr int FOLD_EVERY = (FMT == FMT_TQ) ? 4 : KSTEPS;  // K-steps per scale block
#pragma unroll
        for (int ks = 0; ks < KSTEPS; ++ks) {
            v4i A[2], B[NDIG][2];
#pragma unroll
            for (int i = 0; i < 2; ++i)
                A[i] = *reinterpret_cast<const v4i *>(
                    s_a + (64 * wm + 32 * i + lrow) * PITCH + 32 * ks + 16 * kgrp);
#pragma unroll
            for (int dg = 0; dg < NDIG; ++dg)
#pragma unroll
                for (int j = 0; j < 2; ++j)
                    B[dg][j] = *reinterpret_cast<const v4i *>(
                        s_w + dg * BN * PITCH + (64 * wnn + 32 * j + lrow) * PITCH + 32 * ks +
                        16 * kgrp);
            const bool first = (ks % FOLD_EVERY) == 0;
#pragma unroll
            for (int dg = 0; dg < NDIG; ++dg)
#pragma unroll
                for (int i = 0; i < 2; ++i)
#pragma unroll
                    for (int j = 0; j < 2; ++j) {
                        v16i cin;
                        if (first) {
#pragma unroll
                            for (int r = 0; r < 16; ++r) cin[r] = 0;
                        } else {
                            cin = acc_i[dg][i][j];
                        }
                        acc_i[dg][i][j] = mfma_i8_32x32x32(A[i], B[dg][j], cin);
                    }
            if ((ks % FOLD_EVERY) == FOLD_EVERY - 1) fold((FMT == FMT_TQ) ? (ks / 4) : 0);
        }

        if constexpr (FMT == FMT_Q4K) {
            if ((c & 1) || c == a.nchunks - 1) {
                v8bf ah[2], al[2], bh[2], bl[2];
#pragma unroll
                for (int i = 0; i < 2; ++i) {
                    const int row = 64 * wm + 32 * i + lrow;
                    ah[i] = s_alpha[(0 * BM + row) * 2 + kgrp];
                    al[i] = s_alpha[(1 * BM + row) * 2 + kgrp];
                }
#pragma unroll
                for (int j = 0; j < 2; ++j) {
                    const int col = 64 * wnn + 32 * j + lrow;
                    bh[j] = s_beta[(0 * BN + col) * 2 + kgrp];
                    bl[j] = s_beta[(1 * BN + col) * 2 + kgrp];
                }
#pragma unroll
                for (int i = 0; i < 2; ++i)
#pragma unroll
                    for (int j = 0; j < 2; ++j) {
                        acc_f[i][j] = mfma_bf16_32x32x16(ah[i], bh[j], acc_f[i][j]);
                        acc_f[i][j] = mfma_bf16_32x32x16(ah[i], bl[j], acc_f[i][j]);
                        acc_f[i][j] = mfma_bf16_32x32x16(al[i], bh[j], acc_f[i][j]);
                    }
            }
        }
    }

    // epilogue: masked fp32 stores
    float *out = reinterpret_cast<float *>(a.out);
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int n = n0 + 64 * wnn + 32 * j + lrow;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int m = m0 + 64 * wm + 32 * i + mfma32_row(r, lane);
                if (m < a.M && n < a.N) out[(int64_t)m * a.N + n] = acc_f[i][j][r];
            }
        }
}

// ---------------------------------------------------------------------------
// Sub-sum kernel (test hook): one wave per 32x32 tile, same staging code with
// unit scales, per-sub-block int32 sums written to out[m][n][j].
// ---------------------------------------------------------------------------

template <int FMT>
__global__ __launch_bounds__(64) void subsums_kernel(GemmArgs a) {
    constexpr int BM = 32, BN = 32, NT = 64;
    constexpr int NDIG = Fmt<FMT>::NDIG;
    constexpr int SUB = Fmt<FMT>::SUB;
    constexpr int APIECES = BM * (KC / 16) / NT;
    __shared__ __attribute__((aligned(16))) int8_t s_a[BM * PITCH];
    __shared__ __attribute__((aligned(16))) int8_t s_w[NDIG * BN * PITCH];
    __shared__ float s_dw[2 * BN];

    const int lane = threadIdx.x;
    const int tm = blockIdx.x % a.tiles_m, tn = blockIdx.x / a.tiles_m;
    const int m0 = tm * BM, n0 = tn * BN;
    const int wn_row = lane >> 1, wpart = lane & 1;
    const bool wvalid = (n0 + wn_row) < a.N;
    const int wn_glob = wvalid ? (n0 + wn_row) : 0;
    const int lrow = lane & 31, kgrp = lane >> 5;
    const int nsub = a.K / SUB;
    int32_t *S = reinterpret_cast<int32_t *>(a.out);

    for (int c = 0; c < a.nchunks; ++c) {
        WRaw<FMT> wr;
        load_w<FMT>(wr, a, wn_glob, wpart, c);
        v4i act[APIECES];
#pragma unroll
        for (int i = 0; i < APIECES; ++i) {
            const int p = lane + NT * i;
            const int row = p >> 4, piece = p & 15;
            const int m = m0 + row;
            act[i] = load_act_piece(a, m, c, piece);
        }
        __syncthreads();
#pragma unroll
        for (int i = 0; i < APIECES; ++i) {
            const int p = lane + NT * i;
            *reinterpret_cast<v4i *>(s_a + (p >> 4) * PITCH + 16 * (p & 15)) = act[i];
        }
        unpack_w<FMT, true>(wr, wvalid, s_w, BN * PITCH, wn_row, wpart, s_dw, BN, nullptr, 0,
                            false);
        __syncthreads();

        // K-steps of 32; sub-blocks of 32 (Q4_K), 16 (Q6_K: one per k-group),
        // 128 (ternary: four K-steps)
        v16i accb[NDIG];
        constexpr int KSTEPS = KC / 32;
#pragma unroll
        for (int ks = 0; ks < KSTEPS; ++ks) {
            v4i A = *reinterpret_cast<const v4i *>(s_a + lrow * PITCH + 32 * ks + 16 * kgrp);
            v4i B[NDIG];
#pragma unroll
            for (int dg = 0; dg < NDIG; ++dg)
                B[dg] = *reinterpret_cast<const v4i *>(s_w + dg * BN * PITCH + lrow * PITCH +
                                                       32 * ks + 16 * kgrp);
            if constexpr (FMT == FMT_Q6K) {
                // two 16-wide sub-blocks per K-step: isolate each by zeroing the
                // other k-group's activation operand
#pragma unroll
                for (int half = 0; half < 2; ++half) {
                    v4i Am = (kgrp == half) ? A : v4i{0, 0, 0, 0};
                    v16i z;
#pragma unroll
                    for (int r = 0; r < 16; ++r) z[r] = 0;
                    v16i s0 = mfma_i8_32x32x32(Am, B[0], z);
                    v16i s1 = mfma_i8_32x32x32(Am, B[1], z);
                    const int jg = (c * KC + 32 * ks) / 16 + half;
                    const int n = n0 + lrow;
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const int m = m0 + mfma32_row(r, lane);
                        if (m < a.M && n < a.N)
                            S[((int64_t)m * a.N + n) * nsub + jg] = (s0[r] << 6) + s1[r];
                    }
                }
            } else {
                const bool first = (32 * ks) % SUB == 0;
#pragma unroll
                for (int dg = 0; dg < NDIG; ++dg) {
                    v16i cin;
                    if (first) {
#pragma unroll
                        for (int r = 0; r < 16; ++r) cin[r] = 0;
                    } else {
                        cin = accb[dg];
                    }
                    accb[dg] = mfma_i8_32x32x32(A, B[dg], cin);
                }
                if ((32 * ks + 32) % SUB == 0) {
                    const int64_t kabs = (int64_t)c * KC + 32 * ks;
                    const int jg = (int)(kabs / SUB);
                    const int n = n0 + lrow;
                    if (jg < nsub) {
#pragma unroll
                        for (int r = 0; r < 16; ++r) {
                            const int m = m0 + mfma32_row(r, lane);
                            int v;
                            if constexpr (NDIG == 2)
                                v = (accb[0][r] << Fmt<FMT>::SHIFT) + accb[1][r];
                            else
                                v = accb[0][r];
                            if (m < a.M && n < a.N) S[((int64_t)m * a.N + n) * nsub + jg] = v;
                        }
                    }
                }
            }
        }
    }
}

// ---------------------------------------------------------------------------
// Launchers
// ---------------------------------------------------------------------------

static GemmArgs make_args(int fmt, const void *W, const int8_t *qs, const float *da,
                          const int16_t *bsums, void *out, int M, int N, int K, int bm,
                          int bn) {
    GemmArgs a;
    a.W = (const uint8_t *)W;
    a.qs = qs;
    a.da = da;
    a.bsums = bsums;
    a.out = out;
    a.M = M;
    a.N = N;
    a.K = K;
    a.nchunks = (K + KC - 1) / KC;
    a.nblk = (fmt == FMT_TQ) ? K / 128 : K / 256;
    a.tiles_m = (M + bm - 1) / bm;
    a.tiles_n = (N + bn - 1) / bn;
    return a;
}

hipError_t launch_gemm(int fmt, const void *W, const int8_t *qs, const float *da,
                       const int16_t *bsums, float *out, int M, int N, int K,
                       hipStream_t stream) {
    GemmArgs a = make_args(fmt, W, qs, da, bsums, out, M, N, K, 128, 128);
    const unsigned grid = (unsigned)(a.tiles_m * a.tiles_n);
    switch (fmt) {
        case FMT_Q4K:
            hipLaunchKernelGGL(gemm_kernel<FMT_Q4K>, dim3(grid), dim3(256), 0, stream, a);
            break;
        case FMT_Q6K:
            hipLaunchKernelGGL(gemm_kernel<FMT_Q6K>, dim3(grid), dim3(256), 0, stream, a);
            break;
        default:
            hipLaunchKernelGGL(gemm_kernel<FMT_TQ>, dim3(grid), dim3(256), 0, stream, a);
            break;
    }
    return hipGetLastError();
}

hipError_t launch_subsums(int fmt, const void *W, const int8_t *qs, int32_t *sums, int M, int N,
                          int K, hipStream_t stream) {
    GemmArgs a = make_args(fmt, W, qs, nullptr, nullptr, sums, M, N, K, 32, 32);
    const unsigned grid = (unsigned)(a.tiles_m * a.tiles_n);
    switch (fmt) {
        case FMT_Q4K:
            hipLaunchKernelGGL(subsums_kernel<FMT_Q4K>, dim3(grid), dim3(64), 0, stream, a);
            break;
        case FMT_Q6K:
            hipLaunchKernelGGL(subsums_kernel<FMT_Q6K>, dim3(grid), dim3(64), 0, stream, a);
            break;
        default:
            hipLaunchKernelGGL(subsums_kernel<FMT_TQ>, dim3(grid), dim3(64), 0, stream, a);
            break;
    }
    return hipGetLastError();
}

}  // namespace kq
