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

#include <type_traits>

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
// Main kernel.
//
// Workgroup: 512 threads (8 waves, two per SIMD), output tile 128 x 128.
// Wave w computes rows 64*(w/4) .. +64 and columns 32*(w%4) .. +32 as two
// 32x32 MFMA tiles.  K advances in chunks of 128 (half a Q4_K/Q6_K
// superblock, one ternary block).  Everything a chunk needs lives in one of
// two LDS buffers (activation tile, unpacked weight digit planes, scales), so
// the staging of chunk c+1 (global->register prefetch, unpack, LDS writes)
// and the MFMA work of chunk c run in the same iteration with one barrier.
// The two waves that share a SIMD take the two phases in opposite order, so
// one wave's unpack VALU work issues under the other wave's MFMAs.
//
// LDS rows are padded to 144 bytes: row r starts 36*r banks (mod 64) into
// the 64 four-byte banks, so the fragment reads of 16 consecutive rows hit 16
// different bank groups, and the piece for K-step ks is a constant offset.
//
// Q4_K / Q6_K keep two int32 accumulators per tile (high and low digit
// plane) across both halves of a superblock and fold once per superblock:
//   out += float((hi << SHIFT) + lo) * d_w[n] * d_a[m].
// Rows past M or N are clamped to the last valid row on load (their results
// are computed and never stored).
// ---------------------------------------------------------------------------

constexpr int MBM = 128, MBN = 128, MNT = 512, MKC = 128;
constexpr int MPITCH = MKC + 16;

// LDS byte offset of 16-byte piece c of row r (144-byte rows)
__device__ __forceinline__ int swz(int r, int c) { return r * MPITCH + 16 * c; }

template <int FMT>
struct WStage;
template <>
struct WStage<FMT_Q4K> {
    v4i hdr;
    v4i q;  // 16 nibble bytes
};
template <>
struct WStage<FMT_Q6K> {
    uint32_t ql[9], qh[9];
    uint32_t scbits, dbits, shift;
};
template <>
struct WStage<FMT_TQ> {
    uint32_t w[7];
};

// Ternary: trits [32*Q, 32*Q+32) of a block -> two 16-byte pieces.
template <int Q>
__device__ __forceinline__ void tq_unpack_part(const uint32_t *w, v4i *out) {
    constexpr int B0 = (32 * Q) / 5, B1 = (32 * Q + 31) / 5;
    uint32_t f[B1 - B0 + 1];
#pragma unroll
    for (int b = B0; b <= B1; ++b) f[b - B0] = tq_fixed((w[b >> 2] >> (8 * (b & 3))) & 0xFFu);
#pragma unroll
    for (int qq = 0; qq < 2; ++qq) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            uint32_t word = 0;
#pragma unroll
            for (int bb = 0; bb < 4; ++bb) {
                const int k = 32 * Q + 16 * qq + 4 * e + bb;
                const int byte = k / 5 - B0, pos = k % 5;
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
            out[qq][e] = (int)digits_to_trits(word);
        }
    }
}

template <int FMT>
__global__ __launch_bounds__(512) void gemm_kernel(GemmArgs a) {
    constexpr int BM = MBM, BN = MBN, KCH = MKC;
    constexpr int NDIG = Fmt<FMT>::NDIG;
    constexpr bool Q4 = FMT == FMT_Q4K;
    constexpr int CPS = (FMT == FMT_TQ) ? 1 : 2;  // chunks per scale block
    constexpr int ABUF = BM * MPITCH, WBUF = NDIG * BN * MPITCH;

    __shared__ __attribute__((aligned(16))) int8_t s_a[2 * ABUF];
    __shared__ __attribute__((aligned(16))) int8_t s_w[2 * WBUF];
    __shared__ __attribute__((aligned(16))) float s_da[2 * BM];
    __shared__ __attribute__((aligned(16))) float s_dw[2 * BN];
    // Q4_K min-term operands: [pair ring 2][hi/lo 2][row][superblock parity 2]
    __shared__ v8bf s_alpha[Q4 ? 2 * 2 * BM * 2 : 1];
    __shared__ v8bf s_beta[Q4 ? 2 * 2 * BN * 2 : 1];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;

    // XCD-aware tile order: workgroups are dealt round-robin to 8 XCDs, so
    // XCD x gets the contiguous tile range [x*q, (x+1)*q); M-tiles vary
    // fastest, so the workgroups sharing a weight tile share an L2.
    const int nwg = gridDim.x, wg = blockIdx.x, q8 = nwg >> 3;
    const int tile = (wg < 8 * q8) ? ((wg & 7) * q8 + (wg >> 3)) : wg;
    const int tm = tile % a.tiles_m, tn = tile / a.tiles_m;
    const int m0 = tm * BM, n0 = tn * BN;
    const int M = a.M, N = a.N, K = a.K;
    const int nch = (K + KCH - 1) / KCH;  // chunks
    const int nsa = (FMT == FMT_TQ) ? a.nblk : a.nchunks;  // activation scale blocks per row

    const int lrow = lane & 31, kgrp = lane >> 5;
    const int wm = wave >> 2, wn = wave & 3;

    // ---- staging roles --------------------------------------------------
    // activations: two 16-byte pieces per thread (row a_r0 + 64 i, piece a_pc)
    const int a_pc = tid & 7, a_r0 = tid >> 3;
    const int8_t *a_tile = a.qs + (int64_t)m0 * K;
    uint32_t a_off[2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
        a_off[i] = (uint32_t)(min(m0 + a_r0 + 64 * i, M - 1) - m0) * (uint32_t)K + 16u * a_pc;
    // scales / sums: threads < BM own row tid
    const float *da_tile = a.da + (int64_t)m0 * nsa;
    const uint32_t s_ml = (uint32_t)(min(m0 + (tid & (BM - 1)), M - 1) - m0);
    const uint32_t da_off = s_ml * (uint32_t)nsa;
    const int16_t *bs_tile = Q4 ? a.bsums + (int64_t)m0 * (K / 16) : nullptr;
    const uint32_t bs_off = s_ml * (uint32_t)(K / 16);
    // weights: four threads per row; ternary uses a wave-uniform quarter
    const int wq = (FMT == FMT_TQ) ? (tid >> 7) : (tid & 3);
    const int w_nl = (FMT == FMT_TQ) ? (tid & 127) : (tid >> 2);
    const int w_n = min(n0 + w_nl, N - 1);
    const int64_t w_rowbytes = (int64_t)a.nblk * Fmt<FMT>::BB;
    const uint8_t *w_tile = a.W + (int64_t)n0 * w_rowbytes;
    const uint32_t w_off = (uint32_t)(w_n - n0) * (uint32_t)w_rowbytes;

    // ---- prefetched chunks in registers: chunk j lives in set j % 2; it is
    // loaded at the start of iteration j-2 and staged in iteration j-1.
    constexpr int RING = 2;
    struct Regs {
        v4i act[2];
        float da_v;
        v4i bs_v;
        WStage<FMT> ws;
    };
    Regs rg[RING];

    auto prefetch = [&](Regs &R, int c) {
        v4i(&act)[2] = R.act;
        float &da_v = R.da_v;
        v4i &bs_v = R.bs_v;
        WStage<FMT> &ws = R.ws;
        const int8_t *ab = a_tile + (int64_t)c * KCH;
#pragma unroll
        for (int i = 0; i < 2; ++i) act[i] = *reinterpret_cast<const v4i *>(ab + a_off[i]);
        const int sblk = c / CPS;   // scale block of this chunk
        const int half = c % CPS;   // which half of the superblock
        // every thread loads (rows >= BM re-read a clamped row) so that all
        // paths issue the same number of loads and waits stay precise
        da_v = da_tile[da_off + sblk];
        if constexpr (Q4) bs_v = *reinterpret_cast<const v4i *>(bs_tile + bs_off + 16 * sblk + 8 * half);
        const uint8_t *blk = w_tile + w_off + (int64_t)sblk * Fmt<FMT>::BB;
        if constexpr (FMT == FMT_Q4K) {
            ws.hdr = *reinterpret_cast<const v4i *>(blk);
            ws.q = *reinterpret_cast<const v4i *>(blk + 16 + 64 * half + 16 * wq);
        } else if constexpr (FMT == FMT_Q6K) {
            const int64_t o = (int64_t)n0 * w_rowbytes + w_off + (int64_t)sblk * 210;
            const uint32_t sh = (uint32_t)(o & 3);
            const uint8_t *base = a.W + (o - sh);
            const int u = wq;
            ws.shift = sh;
            // nine dwords cover the 32 bytes for either alignment, and stay
            // inside the block (the ninth ends at byte 132 or 196 at most)
#pragma unroll
            for (int i = 0; i < 9; ++i) ws.ql[i] = ld_u32(base + 64 * half + 32 * (u & 1) + 4 * i);
#pragma unroll
            for (int i = 0; i < 9; ++i) ws.qh[i] = ld_u32(base + 128 + 32 * half + 4 * i);
            ws.scbits = *reinterpret_cast<const unsigned short *>(a.W + o + 192 + 8 * half + 2 * u);
            ws.dbits = *reinterpret_cast<const unsigned short *>(a.W + o + 208);
        } else {
#pragma unroll
            for (int i = 0; i < 7; ++i) ws.w[i] = ld_u32(blk + 4 * i);
        }
    };

    // stage chunk c (c & 1 == P) from register set R into LDS buffer P
    auto stage = [&](auto PP, const Regs &R, int c) {
        constexpr int buf = decltype(PP)::value;
        const v4i(&act)[2] = R.act;
        const float &da_v = R.da_v;
        const v4i &bs_v = R.bs_v;
        const WStage<FMT> &ws = R.ws;
        int8_t *sa = s_a + buf * ABUF;
        int8_t *p0 = s_w + buf * WBUF;
        int8_t *p1 = p0 + (NDIG - 1) * BN * MPITCH;
#pragma unroll
        for (int i = 0; i < 2; ++i) *reinterpret_cast<v4i *>(sa + swz(a_r0 + 64 * i, a_pc)) = act[i];
        if (tid < BM) s_da[buf * BM + tid] = da_v;
        const int sblk = c / CPS;
        constexpr int half = (CPS == 2) ? buf : 0;
        if constexpr (Q4) {
            const int pair = sblk >> 1, par = sblk & 1, ring = pair & 1;
            const bool zero_odd = (par == 0) && (sblk == a.nchunks - 1);
            if (tid < BM) {
                // alpha_j = d_a * (bsums[2j] + bsums[2j+1]) for j = 4*half .. +3
                __bf16 *ah = reinterpret_cast<__bf16 *>(&s_alpha[((ring * 2 + 0) * BM + tid) * 2 + par]) + 4 * half;
                __bf16 *al = reinterpret_cast<__bf16 *>(&s_alpha[((ring * 2 + 1) * BM + tid) * 2 + par]) + 4 * half;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const uint32_t wv = (uint32_t)bs_v[i];
                    const int b = (int)(int16_t)(wv & 0xFFFF) + (int)(int16_t)(wv >> 16);
                    __bf16 hi, lo;
                    split_bf16(da_v * (float)b, hi, lo);
                    ah[i] = hi;
                    al[i] = lo;
                }
                if (zero_odd) {
                    __bf16 *zh = reinterpret_cast<__bf16 *>(&s_alpha[((ring * 2 + 0) * BM + tid) * 2 + 1]) + 4 * half;
                    __bf16 *zl = reinterpret_cast<__bf16 *>(&s_alpha[((ring * 2 + 1) * BM + tid) * 2 + 1]) + 4 * half;
#pragma unroll
                    for (int i = 0; i < 4; ++i) zh[i] = zl[i] = (__bf16)0.0f;
                }
            }
            // weights: this thread's 16 nibble bytes hold column cl = 2*half + (wq>>1)
            const int cl = 2 * half + (wq >> 1);
            uint32_t sc[2], mn[2];
            q4k_fields((uint32_t)ws.hdr[1], (uint32_t)ws.hdr[2], (uint32_t)ws.hdr[3], 2 * cl, 2, sc, mn);
            v4i hl, ll, hh, lh;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const uint32_t word = (uint32_t)ws.q[e];
                uint32_t dh, dl;
                q4k_digits(word & 0x0F0F0F0Fu, sc[0], dh, dl);
                hl[e] = (int)dh;
                ll[e] = (int)dl;
                q4k_digits((word >> 4) & 0x0F0F0F0Fu, sc[1], dh, dl);
                hh[e] = (int)dh;
                lh[e] = (int)dl;
            }
            const int pl = 4 * (wq >> 1) + (wq & 1);   // piece of the low nibbles
            *reinterpret_cast<v4i *>(p0 + swz(w_nl, pl)) = hl;
            *reinterpret_cast<v4i *>(p1 + swz(w_nl, pl)) = ll;
            *reinterpret_cast<v4i *>(p0 + swz(w_nl, pl + 2)) = hh;
            *reinterpret_cast<v4i *>(p1 + swz(w_nl, pl + 2)) = lh;
            if (wq == 0) s_dw[buf * BN + w_nl] = f16_bits_to_f32((uint32_t)ws.hdr[0]);
            if ((wq & 1) == 0) {
                const float dmin = f16_bits_to_f32((uint32_t)ws.hdr[0] >> 16);
                __bf16 *bh = reinterpret_cast<__bf16 *>(&s_beta[((ring * 2 + 0) * BN + w_nl) * 2 + par]) + 2 * cl;
                __bf16 *bl = reinterpret_cast<__bf16 *>(&s_beta[((ring * 2 + 1) * BN + w_nl) * 2 + par]) + 2 * cl;
#pragma unroll
                for (int i = 0; i < 2; ++i) {
                    __bf16 hi, lo;
                    split_bf16(-dmin * (float)mn[i], hi, lo);
                    bh[i] = hi;
                    bl[i] = lo;
                }
                if (zero_odd) {
                    __bf16 *zh = reinterpret_cast<__bf16 *>(&s_beta[((ring * 2 + 0) * BN + w_nl) * 2 + 1]) + 2 * cl;
                    __bf16 *zl = reinterpret_cast<__bf16 *>(&s_beta[((ring * 2 + 1) * BN + w_nl) * 2 + 1]) + 2 * cl;
                    zh[0] = zh[1] = zl[0] = zl[1] = (__bf16)0.0f;
                }
            }
        } else if constexpr (FMT == FMT_Q6K) {
            const int u = wq;
            const uint32_t sh = ws.shift;
            const int sc_lo = (int)(int8_t)(ws.scbits & 0xFF), sc_hi = (int)(int8_t)(ws.scbits >> 8);
#pragma unroll
            for (int g = 0; g < 2; ++g) {
                const int sc = g ? sc_hi : sc_lo;
                v4i vh, vl;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int t4 = 4 * g + e;
                    const uint32_t qlw = sh ? __builtin_amdgcn_alignbyte(ws.ql[t4 + 1], ws.ql[t4], 2) : ws.ql[t4];
                    const uint32_t qhw = sh ? __builtin_amdgcn_alignbyte(ws.qh[t4 + 1], ws.qh[t4], 2) : ws.qh[t4];
                    const uint32_t lo4 = (qlw >> (4 * (u >> 1))) & 0x0F0F0F0Fu;
                    const uint32_t hi2 = (qhw >> (2 * u)) & 0x03030303u;
                    uint32_t dh, dl;
                    q6k_digits(lo4 | (hi2 << 4), sc, dh, dl);
                    vh[e] = (int)dh;
                    vl[e] = (int)dl;
                }
                *reinterpret_cast<v4i *>(p0 + swz(w_nl, 2 * u + g)) = vh;
                *reinterpret_cast<v4i *>(p1 + swz(w_nl, 2 * u + g)) = vl;
            }
            if (wq == 0) s_dw[buf * BN + w_nl] = f16_bits_to_f32(ws.dbits);
        } else {
            v4i pieces[2];
            switch (__builtin_amdgcn_readfirstlane(wq)) {  // wave-uniform
                case 0: tq_unpack_part<0>(ws.w, pieces); break;
                case 1: tq_unpack_part<1>(ws.w, pieces); break;
                case 2: tq_unpack_part<2>(ws.w, pieces); break;
                default: tq_unpack_part<3>(ws.w, pieces); break;
            }
            *reinterpret_cast<v4i *>(p0 + swz(w_nl, 2 * wq)) = pieces[0];
            *reinterpret_cast<v4i *>(p0 + swz(w_nl, 2 * wq + 1)) = pieces[1];
            if (wq == 0) s_dw[buf * BN + w_nl] = f16_bits_to_f32(ws.w[6] >> 16);
        }
    };

    v16f acc_f[2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc_f[i][r] = 0.0f;
    v16i acc[NDIG][2];

    // compute chunk c (c & 1 == P) from LDS buffer P
    auto compute = [&](auto PP, int c) {
        constexpr int buf = decltype(PP)::value;
        const int8_t *sa = s_a + buf * ABUF;
        const int8_t *sw = s_w + buf * WBUF;
        constexpr bool first = (CPS == 1) || (buf == 0);
        constexpr bool last = (CPS == 1) || (buf == 1);
#pragma unroll
        for (int ks = 0; ks < KCH / 32; ++ks) {
            const int pc = 2 * ks + kgrp;
            v4i A[2], B[NDIG];
#pragma unroll
            for (int i = 0; i < 2; ++i)
                A[i] = *reinterpret_cast<const v4i *>(sa + swz(64 * wm + 32 * i + lrow, pc));
#pragma unroll
            for (int dg = 0; dg < NDIG; ++dg)
                B[dg] = *reinterpret_cast<const v4i *>(sw + dg * BN * MPITCH + swz(32 * wn + lrow, pc));
#pragma unroll
            for (int dg = 0; dg < NDIG; ++dg)
#pragma unroll
                for (int i = 0; i < 2; ++i)
                    acc[dg][i] = (first && ks == 0) ? mfma_i8_32x32x32(A[i], B[dg], v16i{})
                                                    : mfma_i8_32x32x32(A[i], B[dg], acc[dg][i]);
        }
        if constexpr (last) {
            // fold: out += float(T) * d_w[n] * d_a[m]
            const float dwv = s_dw[buf * BN + 32 * wn + lrow];
#pragma unroll
            for (int i = 0; i < 2; ++i) {
#pragma unroll
                for (int r4 = 0; r4 < 4; ++r4) {
                    const v4f dav = *reinterpret_cast<const v4f *>(&s_da[buf * BM + 64 * wm + 32 * i + 8 * r4 + 4 * kgrp]);
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int r = 4 * r4 + e;
                        int T;
                        if constexpr (NDIG == 2)
                            T = (acc[0][i][r] << Fmt<FMT>::SHIFT) + acc[1][i][r];
                        else
                            T = acc[0][i][r];
                        acc_f[i][r] = fmaf((float)T * dwv, dav[e], acc_f[i][r]);
                    }
                }
            }
        }
        if constexpr (Q4) {
            const int sblk = c / CPS;
            // after the last chunk of each superblock pair (or of the row)
            if (last && ((sblk & 1) || sblk == a.nchunks - 1)) {
                const int ring = (sblk >> 1) & 1;
                const int col = 32 * wn + lrow;
                const v8bf bh = s_beta[((ring * 2 + 0) * BN + col) * 2 + kgrp];
                const v8bf bl = s_beta[((ring * 2 + 1) * BN + col) * 2 + kgrp];
#pragma unroll
                for (int i = 0; i < 2; ++i) {
                    const int row = 64 * wm + 32 * i + lrow;
                    const v8bf ah = s_alpha[((ring * 2 + 0) * BM + row) * 2 + kgrp];
                    const v8bf al = s_alpha[((ring * 2 + 1) * BM + row) * 2 + kgrp];
                    acc_f[i] = mfma_bf16_32x32x16(ah, bh, acc_f[i]);
                    acc_f[i] = mfma_bf16_32x32x16(ah, bl, acc_f[i]);
                    acc_f[i] = mfma_bf16_32x32x16(al, bh, acc_f[i]);
                }
            }
        }
    };

    // prologue: chunks 0..RING-1 in flight, chunk 0 staged
    // prefetches past the last chunk re-load the last chunk (harmless) so the
    // number of loads in flight is the same on every path
    const int clast = max(nch - 1, 0);
    using P0 = std::integral_constant<int, 0>;
    using P1 = std::integral_constant<int, 1>;
    if (nch > 0) {
        prefetch(rg[0], 0);
        prefetch(rg[1], min(1, clast));
        stage(P0{}, rg[0], 0);
    }
    __syncthreads();
    const bool stage_first = (wm == 0);
    // one iteration (c & 1 == P): refill the register set that held chunk c
    // with chunk c+2, stage chunk c+1 into the other LDS buffer, compute
    // chunk c, barrier.  The two waves of a SIMD take stage and compute in
    // opposite order.
    auto iteration = [&](auto PP, int c) {
        constexpr int P = decltype(PP)::value;
        using Q = std::integral_constant<int, 1 - P>;
        prefetch(rg[P], min(c + 2, clast));
        if (stage_first) {
            if (c + 1 < nch) stage(Q{}, rg[1 - P], c + 1);
            compute(PP, c);
        } else {
            compute(PP, c);
            if (c + 1 < nch) stage(Q{}, rg[1 - P], c + 1);
        }
        __syncthreads();
    };
    for (int c = 0; c < nch; c += 2) {
        iteration(P0{}, c);
        if (c + 1 < nch) iteration(P1{}, c + 1);
    }

    // ---- epilogue: fp32 stores (unmasked when the whole tile is inside) ----
    float *out = reinterpret_cast<float *>(a.out);
    const bool full = (m0 + BM <= M) && (n0 + BN <= N);
    const int n = n0 + 32 * wn + lrow;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int m = m0 + 64 * wm + 32 * i + mfma32_row(r, lane);
            if (full || (m < M && n < N)) out[(int64_t)m * N + n] = acc_f[i][r];
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
    GemmArgs a = make_args(fmt, W, qs, da, bsums, out, M, N, K, MBM, MBN);
    const unsigned grid = (unsigned)(a.tiles_m * a.tiles_n);
    switch (fmt) {
        case FMT_Q4K:
            hipLaunchKernelGGL(gemm_kernel<FMT_Q4K>, dim3(grid), dim3(MNT), 0, stream, a);
            break;
        case FMT_Q6K:
            hipLaunchKernelGGL(gemm_kernel<FMT_Q6K>, dim3(grid), dim3(MNT), 0, stream, a);
            break;
        default:
            hipLaunchKernelGGL(gemm_kernel<FMT_TQ>, dim3(grid), dim3(MNT), 0, stream, a);
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
