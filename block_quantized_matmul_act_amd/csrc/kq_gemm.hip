// kq_gemm.hip -- cooperative-tile block-quantized GEMM on gfx950 int8 MFMA.
//
// out[m][n] = sum_k W^[n][k] * A^[m][k] for Q4_K / Q6_K weights against Q8_K
// activations and ternary weights (base-3 at 1.6 bits per weight, or two bits
// per weight) against Q8_128 activations.
//
// Launched for Q6_K and ternary weights (shapes the matrix-vector kernels of
// kq_gemv.hip do not take; two-bit ternary always); Q4_K runs on the kernels
// of kq_gemm_q4k.hip, and gemm_kernel refuses to compile for it.  The two
// test hooks (subsums_kernel, debug_unpack_kernel) are a separate decoder:
// their own loaders (load_w / unpack_w) and a small 32 x 32 MFMA loop, for
// every format; the production kernels are checked exactly by the one-hot
// and unit-scale products of the tests instead.
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
//   * Q4_K mins: sum_j m_j * B_j (B_j = sub-block sums of the activations)
//     is folded as -dmin*m_j x d_a*B_j through a bf16 MFMA with hi/lo-split
//     operands (~16 significant bits each), accumulating straight into the
//     fp32 output registers; two superblocks share one K=16 MFMA (one per
//     k-group).  The activation operand d_a*B_j comes precomputed from the
//     quantizer (the alpha section).
//   * Rows >= M and >= N are never read: their LDS rows are zero-filled and
//     the epilogue masks the stores (the ragged-tail staging clamp of
//     vllm.cpp PR 3036).  No wave leaves before a barrier.
//   * blockIdx is remapped so consecutive tiles of one weight column-block
//     land on the same XCD (blocks are dealt round-robin to the 8 XCDs), so
//     a weight tile is fetched from HBM once per XCD L2.
#include "kq_device.hpp"
#include "kq_hooks.hpp"
#include "kq_launch.hpp"

#include <type_traits>

namespace kq {

enum { FMT_Q4K = 1, FMT_Q6K = 2, FMT_TQ = 3, FMT_TQ2 = 4 };

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
template <>
struct Fmt<FMT_TQ2> {
    static constexpr int QK = 128, BB = 34, NDIG = 1, SHIFT = 0, SUB = 128;
};
// formats whose scales cover 128 values (one block per 128-wide chunk half)
constexpr bool tri(int fmt) { return fmt == FMT_TQ || fmt == FMT_TQ2; }

constexpr int KC = 256;         // K values per chunk
constexpr int PITCH = KC + 16;  // LDS row pitch in bytes (16-byte skew against bank conflicts)

struct GemmArgs {
    const uint8_t *W;
    const int8_t *qs;       // activation values  [M][K]
    const float *da;        // activation scales  [K/ABS][M] (block-major)
    const uint16_t *alpha;  // Q4_K min operand   [K/256][2][M][8] bf16 (Q8_K only)
    void *out;              // fp32 [M][N], or int32 [M][N][K/SUB] for the sub-sum kernel
    int M, N, K;
    int nchunks;            // K / KC (ternary: K / 128 blocks rounded up to chunks)
    int nblk;               // weight blocks per row = K / QK
    int tiles_m, tiles_n;
    // expert-indexed product (gather mode of the tile kernel): routed row r of
    // expert e, r in [exp_off[e], exp_off[e+1]), is token rows[r]; expert e's
    // weights start expert_bytes * e bytes into W
    const int32_t *exp_off;
    const int32_t *rows;
    int n_experts, n_routed;
    int64_t expert_bytes;
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
template <>
struct WRaw<FMT_TQ2> {
    uint32_t w[9];   // the block from its dword boundary: 8 (aligned) or 9 dwords
    uint32_t dbits;  // fp16 d (aligned blocks; otherwise the top half of w[8])
    uint32_t shift;  // block start mod 4 (0 or 2)
};

// Four int8 trits t = c - 1 from four two-bit codes c <= 2, one per byte
// (adding 0x7F never carries out of a byte and flipping bit 7 gives c - 1).
__device__ __forceinline__ uint32_t codes_to_trits(uint32_t c4) {
    return (c4 + 0x7F7F7F7Fu) ^ 0x80808080u;
}

__device__ __forceinline__ uint32_t ld_u32(const uint8_t *p) {
    return *reinterpret_cast<const uint32_t *>(p);
}

// A Q6_K block starts 0 or 2 bytes into the dword its loads begin at; word i
// of the block is bytes [2, 4) of loaded word i and [0, 2) of word i + 1.
__device__ __forceinline__ uint32_t q6k_realign(uint32_t lo, uint32_t hi, uint32_t shift) {
    return shift ? __builtin_amdgcn_alignbyte(hi, lo, 2) : lo;
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
    } else if constexpr (FMT == FMT_TQ2) {
        // one 34-byte block per part; it starts 0 or 2 bytes past a dword
        // boundary, and no load reaches past its last byte
        const int blkidx = 2 * c + part;
        if (blkidx < a.nblk) {
            const int64_t o = ((int64_t)n * a.nblk + blkidx) * 34;
            const uint32_t sh = (uint32_t)(o & 3);
            const uint8_t *base = a.W + (o - sh);
            r.shift = sh;
#pragma unroll
            for (int i = 0; i < 9; ++i) r.w[i] = (i < 8 || sh) ? ld_u32(base + 4 * i) : 0u;
            r.dbits = sh ? (r.w[8] >> 16) : *reinterpret_cast<const unsigned short *>(a.W + o + 32);
        } else {
#pragma unroll
            for (int i = 0; i < 9; ++i) r.w[i] = 0x55555555u;  // code 1 everywhere: zero trits
            r.dbits = 0;
            r.shift = 0;
        }
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
        for (int i = 0; i < 16; ++i) ql[i] = q6k_realign(r.ql[i], r.ql[i + 1], sh);
#pragma unroll
        for (int i = 0; i < 8; ++i) qh[i] = q6k_realign(r.qh[i], r.qh[i + 1], sh);
#pragma unroll
        for (int i = 0; i < 2; ++i) scw[i] = q6k_realign(r.sc[i], r.sc[i + 1], sh);
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
    } else if constexpr (FMT == FMT_TQ2) {
        // two-bit ternary: this part is one 128-block; plane p of code dword i
        // is weights 4i .. 4i+3 + 32p
        int8_t *dst = row0 + 128 * part;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const uint32_t cw = __builtin_amdgcn_alignbyte(r.w[i + 1], r.w[i], r.shift);
#pragma unroll
            for (int pl = 0; pl < 4; ++pl) {
                const uint32_t v = codes_to_trits((cw >> (2 * pl)) & 0x03030303u);
                *reinterpret_cast<uint32_t *>(dst + 32 * pl + 4 * i) = valid ? v : 0u;
            }
        }
        dw[part * rows + nl] = valid ? (UNIT ? 1.0f : f16_bits_to_f32(r.dbits)) : 0.0f;
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
// superblock, one ternary block).  Each chunk has its own LDS buffer pair
// (activation tile, unpacked weight digit planes); scales live in a ring of
// four scale-block slots.  One iteration = one chunk, one barrier:
//   * global loads of chunk c+2 into one register set,
//   * unpack of chunk c+1 (loaded one iteration earlier) into the other LDS
//     buffer,
//   * the MFMAs of chunk c,
//   * the fold of one m-tile: at a superblock's last chunk, tile 0 is folded
//     right after its MFMAs (while tile 1's MFMAs run); tile 1 is folded at
//     the next chunk, before its accumulators restart (while tile 0's run).
// The body of an iteration is one basic block (compile-time chunk phase,
// clamped loads past the end, no divergent stores), so the scheduler can
// interleave the unpack and fold VALU work with the MFMAs.
//
// LDS rows are padded to 144 bytes: row r starts 36*r banks (mod 64) into
// the 64 four-byte banks, so the fragment reads of 16 consecutive rows hit 16
// different bank groups.
//
// Q4_K / Q6_K keep two int32 accumulators per tile (high and low digit
// plane) across both chunks of a superblock and fold once per superblock:
//   out += float((hi << SHIFT) + lo) * d_w[n] * d_a[m].
// Rows past M or N are clamped to the last valid row on load (their results
// are computed and never stored).
// ---------------------------------------------------------------------------

constexpr int MBM = 128, MBN = 128, MNT = 512, MKC = 128;
constexpr int MPITCH = MKC + 16;

// LDS byte offset of 16-byte piece c of row r (144-byte rows)
__device__ __forceinline__ int swz(int r, int c) { return r * MPITCH + 16 * c; }

// instruction classes of __builtin_amdgcn_sched_group_barrier
enum : int { SG_VALU = 0x002, SG_MFMA = 0x008, SG_VMEM = 0x020, SG_DSR = 0x100, SG_DSW = 0x200 };

// Per-thread registers of one chunk between its global loads and its unpack.
template <int FMT>
struct ChunkRegs;
template <>
struct ChunkRegs<FMT_Q4K> {
    v4i act[2];
    float da;
    uint32_t al;  // 4 bytes of the alpha section
    v4i hdr;      // d, dmin, 12 scale bytes (loaded with the superblock's first chunk)
    v4i q;        // 16 nibble bytes
};
template <>
struct ChunkRegs<FMT_Q6K> {
    v4i act[2];
    float da;
    uint32_t ql[6];  // two 8-byte runs of ql, each in 3 aligned dwords
    uint32_t qh[3];  // one 8-byte run of qh
    uint32_t sc[3];  // 8 scale bytes
    uint32_t d;
    uint32_t sh;     // block start mod 4 (0 or 2)
};
template <>
struct ChunkRegs<FMT_TQ> {
    v4i act[2];
    float da;
    uint32_t w[2];  // 8 trit bytes
};
template <>
struct ChunkRegs<FMT_TQ2> {
    v4i act[2];
    float da;
    uint32_t w[3];  // 8 code bytes from their dword boundary
    uint32_t sh;    // block start mod 4 (0 or 2)
    uint32_t d;     // fp16 d
};

// SPLIT: K in two parts on blockIdx.y (for shapes with at most half as many
// tiles as CUs), each a whole number of four-chunk groups so that both start
// at phase 0; each part adds its sums into the output, zeroed before the
// launch.  With exactly two addends onto zero the result does not depend on
// their order (0 + a + b = 0 + b + a in fp32), so it is deterministic.
template <int FMT, bool GATHER = false, bool SPLIT = false>
__global__ __launch_bounds__(MNT) void gemm_kernel(GemmArgs a) {
    constexpr int BM = MBM, BN = MBN, KCH = MKC;
    constexpr int NDIG = Fmt<FMT>::NDIG;
    // Q4_K runs on the register-unpack kernels of kq_gemm_q4k.hip; this
    // kernel's Q4_K branches (min term through the older alpha operand) are
    // never compiled
    static_assert(FMT != FMT_Q4K, "Q4_K products run on kq_gemm_q4k.hip");
    constexpr bool Q4 = FMT == FMT_Q4K, Q6 = FMT == FMT_Q6K, TQ = FMT == FMT_TQ, TQ2 = FMT == FMT_TQ2;
    constexpr bool TRI = tri(FMT);    // scales per 128 values, one block per chunk
    constexpr int CPS = TRI ? 1 : 2;  // chunks per scale block
    constexpr int PLANE = BN * MPITCH;

    // one array per buffer, so the compiler sees that staging writes and
    // fragment reads never alias
    __shared__ __attribute__((aligned(16))) int8_t s_a0[BM * MPITCH];
    __shared__ __attribute__((aligned(16))) int8_t s_a1[BM * MPITCH];
    __shared__ __attribute__((aligned(16))) int8_t s_w0[NDIG * PLANE];
    __shared__ __attribute__((aligned(16))) int8_t s_w1[NDIG * PLANE];
    // block scales: a ring of 4 scale-block slots
    __shared__ __attribute__((aligned(16))) float s_da[4 * BM];
    __shared__ __attribute__((aligned(16))) float s_dw[4 * BN + 64];  // + a junk row
    // Q4_K min-term operands: [pair ring 2][hi/lo 2][row][superblock parity 2]
    __shared__ v8bf s_alpha[Q4 ? 2 * 2 * BM * 2 : 1];
    __shared__ v8bf s_beta[Q4 ? 2 * 2 * BN * 2 : 1];
    __shared__ __attribute__((aligned(16))) uint32_t s_lut[TQ ? 2 * 256 : 2];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;

    // XCD-aware tile order: workgroups are dealt round-robin to 8 XCDs, so
    // XCD x gets the contiguous tile range [x*q, (x+1)*q).  Inside that range
    // tiles run in groups of GM M-tiles: down a group of GM M-tiles first,
    // then across N, so the ~32 workgroups resident on one XCD cover a GM x 8
    // block of tiles whose activation rows and weight rows both stay in that
    // XCD's L2 (M-fastest order re-fetched every activation row once per
    // N-tile; this order halves the L2 misses).
    constexpr int GM = 4;
    const int nwg = gridDim.x, wg = blockIdx.x, q8 = nwg >> 3;
    const int tile = (wg < 8 * q8) ? ((wg & 7) * q8 + (wg >> 3)) : wg;
    const int per_group = GM * a.tiles_n;
    const int first_m = (tile / per_group) * GM;
    const int gsize = min(a.tiles_m - first_m, GM);
    const int tm = first_m + (tile % per_group) % gsize, tn = (tile % per_group) / gsize;
    const int n0 = tn * BN;
    const int M = a.M, N = a.N, K = a.K;
    // m0: first activation row of the tile; mrows: tile rows holding data;
    // orow0: first output row; Wx: the weights this tile multiplies
    int m0, mrows, grb = 0;
    int64_t orow0;
    const uint8_t *Wx = a.W;
    if constexpr (!GATHER) {
        m0 = tm * BM;
        mrows = min(M - m0, BM);
        orow0 = m0;
    } else {
        // expert-indexed: M-tile tm is tile mt of expert e, counting each
        // expert's ceil(rows / BM) tiles in expert order; tiles past the last
        // one (the grid is an upper bound) leave before any barrier
        int e = -1, mt = 0, acc = 0;
        for (int x = 0; x < a.n_experts; ++x) {
            const int cnt = max(a.exp_off[x + 1] - a.exp_off[x], 0);
            const int te = (cnt + BM - 1) / BM;
            if (e < 0 && tm < acc + te) {
                e = x;
                mt = tm - acc;
            }
            acc += te;
        }
        if (e < 0) return;
        // (clamped, so that routing arrays that break their contract give
        // wrong values but never an access outside rows[] or out)
        grb = a.exp_off[e] + mt * BM;
        mrows = (grb < 0 || grb >= a.n_routed) ? 0 : min(min(a.exp_off[e + 1], a.n_routed) - grb, BM);
        m0 = 0;
        orow0 = grb;
        Wx = a.W + (int64_t)e * a.expert_bytes;
    }
    // token row of tile row r when gathering (rows past the expert's last
    // repeat it; indices are clamped into the activation buffer)
    auto token = [&](int r) KQ_INLINE {
        const int idx = min(max(grb + min(r, mrows - 1), 0), a.n_routed - 1);
        const int t = a.rows[idx];
        return min(max(t, 0), M - 1);
    };
    const int nch_all = (K + KCH - 1) / KCH;                // chunks
    const int cpp = SPLIT ? ((nch_all + 1) / 2 + 3) / 4 * 4 : nch_all;
    const int cb = SPLIT ? (int)blockIdx.y * cpp : 0;      // first chunk of this part
    const int nch = SPLIT ? max(min(nch_all - cb, cpp), 0) : nch_all;  // chunks of this part
    const int nsa = TRI ? a.nblk : a.nchunks;               // activation scale blocks per row

    const int lrow = lane & 31, kgrp = lane >> 5;
    const int wm = wave >> 2, wn = wave & 3;

    // ---- staging roles --------------------------------------------------
    // Every global read goes through a buffer resource of this tile (base in
    // SGPRs, 32-bit lane offsets fixed for the whole loop, the chunk advance
    // as a scalar offset), so the loads cost no per-iteration address
    // arithmetic.  Reads past a resource's end return zero: rows >= M or >= N
    // of a ragged tile read zeros and their results are never stored.
    constexpr int RSRC_FLAGS = 0x00020000;  // raw 32-bit dwords, gfx9 family
    // activations: two 16-byte pieces per thread (row a_r0 + 64 i, piece a_pc)
    const int a_pc = tid & 7, a_r0 = tid >> 3;
    const auto rs_a = __builtin_amdgcn_make_buffer_rsrc(
        (void *)(a.qs + (int64_t)m0 * K), (short)0, (GATHER ? M : min(M - m0, BM)) * K, RSRC_FLAGS);
    uint32_t a_off[2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
        a_off[i] = (uint32_t)(GATHER ? token(a_r0 + 64 * i) : a_r0 + 64 * i) * (uint32_t)K + 16u * a_pc;
    // activation scales (block-major [nsa][M]) and, for Q4_K, the alpha
    // section: thread t owns row t/4; of alpha it copies 4 bytes: part
    // (t%4)/2 (hi/lo), sub-blocks 2*(t%2) .. +1 of the chunk's four
    const int s_row = tid >> 2, s_j = tid & 3;
    const auto rs_d = __builtin_amdgcn_make_buffer_rsrc((void *)(a.da + m0), (short)0,
                                                        (nsa * M - m0) * 4, RSRC_FLAGS);
    const int s_tok = GATHER ? token(s_row) : s_row;  // activation row whose scales this thread stages
    const uint32_t d_off = 4u * s_tok;
    const auto rs_al = __builtin_amdgcn_make_buffer_rsrc(
        Q4 ? (void *)(a.alpha + (int64_t)m0 * 8) : (void *)a.da, (short)0,
        Q4 ? (a.nchunks * 2 * M - m0) * 16 : 0, RSRC_FLAGS);
    const uint32_t al_off = (uint32_t)(((s_j >> 1) * M + s_tok) * 16 + 4 * (s_j & 1));
    // weights: four threads per row
    const int wq = tid & 3, w_nl = tid >> 2;
    const int w_rowbytes = a.nblk * Fmt<FMT>::BB;
    const auto rs_w = __builtin_amdgcn_make_buffer_rsrc(
        (void *)(Wx + (int64_t)n0 * w_rowbytes), (short)0, min(N - n0, BN) * w_rowbytes,
        RSRC_FLAGS);
    const uint32_t w_off = (uint32_t)(w_nl * w_rowbytes);
    // ternary: this thread's 8 trit bytes start at byte 8*wq of the block
    // (20 for the last quarter, which decodes bytes 20..27 into row bytes
    // 100..139; bytes 128.. land in the row padding)
    const int tq_off = (wq == 3) ? 20 : 8 * wq;

    const int clast = max(nch - 1, 0);
    // chunk x, or past the end the last chunk with x's parity (the same half
    // of a superblock), so repeated loads and stages rewrite identical values
    auto clampc = [&](int x) KQ_INLINE {
        if (x <= clast) return x;
        return (CPS == 1) ? clast : clast - ((x - clast) & 1);
    };

    ChunkRegs<FMT> rg[2];

    // global loads of chunk c (c % 2 == H) into R
    auto prefetch = [&](auto HH, ChunkRegs<FMT> &R, int c) KQ_INLINE {
        constexpr int H = decltype(HH)::value;
        // (c counts this part's chunks; the global chunk is cb + c)
        const int cg = cb + c;
        const int sblk = cg / CPS;
#pragma unroll
        for (int i = 0; i < 2; ++i)
            R.act[i] = __builtin_bit_cast(v4i, __builtin_amdgcn_raw_buffer_load_b128(rs_a, (int)a_off[i], cg * KCH, 0));
        R.da = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rs_d, (int)d_off, sblk * M * 4, 0));
        const int wsoff = sblk * Fmt<FMT>::BB;
        if constexpr (Q4) {
            R.al = __builtin_amdgcn_raw_buffer_load_b32(rs_al, (int)al_off, sblk * 32 * M + 8 * H, 0);
            if constexpr (H == 0)  // the second chunk reuses the first chunk's header
                R.hdr = __builtin_bit_cast(v4i, __builtin_amdgcn_raw_buffer_load_b128(rs_w, (int)w_off, wsoff, 0));
            R.q = __builtin_bit_cast(v4i, __builtin_amdgcn_raw_buffer_load_b128(rs_w, (int)(w_off + 16 + 64 * H + 16 * wq), wsoff, 0));
        } else if constexpr (Q6) {
            // the 210-byte block starts 0 or 2 bytes past a dword boundary;
            // every window below lies inside the block or the block before it
            // (few wide loads: the address unit's cost is per instruction)
            const uint32_t o = w_off + (uint32_t)wsoff;
            const uint32_t sh = o & 3u;
            const int base = (int)(o - sh);
            const int bq = base + 8 * wq;
            R.sh = sh;
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                const v3u w3 = __builtin_amdgcn_raw_buffer_load_b96(rs_w, bq, 64 * H + 32 * j, 0);
                R.ql[3 * j + 0] = w3.x;
                R.ql[3 * j + 1] = w3.y;
                R.ql[3 * j + 2] = w3.z;
            }
            {
                const v3u w3 = __builtin_amdgcn_raw_buffer_load_b96(rs_w, bq, 128 + 32 * H, 0);
                R.qh[0] = w3.x;
                R.qh[1] = w3.y;
                R.qh[2] = w3.z;
            }
            const v2u s2 = __builtin_amdgcn_raw_buffer_load_b64(rs_w, base, 192 + 8 * H, 0);
            R.sc[0] = s2.x;
            R.sc[1] = s2.y;
            // third dword only needed when sh == 2; otherwise re-read the second
            R.sc[2] = __builtin_amdgcn_raw_buffer_load_b32(rs_w, base + (sh ? 4 : 0), 196 + 8 * H, 0);
            R.d = __builtin_amdgcn_raw_buffer_load_b16(rs_w, (int)o, 208, 0);
        } else if constexpr (TQ) {
            const v2u w2 = __builtin_amdgcn_raw_buffer_load_b64(rs_w, (int)(w_off + tq_off), wsoff, 0);
            R.w[0] = w2.x;
            R.w[1] = w2.y;
        } else {
            // code bytes 8wq .. 8wq+7 of the 34-byte block, from their dword
            // boundary (the block starts 0 or 2 bytes past one; a window may
            // run two bytes into the next block, or past the end, which reads
            // zero)
            const uint32_t o = w_off + (uint32_t)wsoff;
            const uint32_t sh = o & 3u;
            const v3u w3 = __builtin_amdgcn_raw_buffer_load_b96(rs_w, (int)(o - sh) + 8 * wq, 0, 0);
            R.w[0] = w3.x;
            R.w[1] = w3.y;
            R.w[2] = w3.z;
            R.sh = sh;
            R.d = __builtin_amdgcn_raw_buffer_load_b16(rs_w, (int)o, 32, 0);
        }
    };

    // ---- unpack of chunk c (c % 2 == B) from R into LDS buffer B, in eight
    // pieces that ride along the eight MFMA slots of one m-tile ------------
    struct StageTmp {
        uint32_t sc[2], mn[2];   // Q4_K sub-block scales / mins of this thread
        v4i hl, ll, hh, lh;      // Q4_K digit planes (low / high nibbles)
        uint32_t ql[2][2], qh[2], S0, S1, vh[2], vl[2];  // Q6_K
        uint32_t lo[8], hi[8];   // ternary table entries
    };
    // hdr: the Q4_K header of the chunk's superblock (held from its first chunk)
    auto stage_piece = [&](auto BB_, auto SS, const ChunkRegs<FMT> &R, const v4i &hdr, int c,
                           StageTmp &T) KQ_INLINE {
        constexpr int B = decltype(BB_)::value;
        constexpr int S = decltype(SS)::value;
        int8_t *sa = B ? s_a1 : s_a0;
        int8_t *p0 = B ? s_w1 : s_w0;
        int8_t *p1 = p0 + (NDIG - 1) * PLANE;
        const int sblk = c / CPS;
        const int slot = sblk & 3;
        if constexpr (S == 0) {
#pragma unroll
            for (int i = 0; i < 2; ++i)
                *reinterpret_cast<v4i *>(sa + swz(a_r0 + 64 * i, a_pc)) = R.act[i];
            s_da[slot * BM + s_row] = R.da;  // the four threads of a row store the same value
        }
        if constexpr (Q4) {
            constexpr int H = B;  // half of the superblock
            const int par = sblk & 1, ring = (sblk >> 1) & 1;
            const int cl = 2 * H + (wq >> 1);  // nibble column: 32-sub-blocks 2cl (low), 2cl+1 (high)
            if constexpr (S == 0) {
                // alpha: this thread's 4 bytes (part s_j/2, sub-blocks 4H + 2(s_j%2) .. +1)
                // go to the superblock's parity slot.  An even superblock also
                // clears its odd partner's slot (which stays zero if the row ends
                // there); an odd one writes its own slot twice.
                char *arow = reinterpret_cast<char *>(&s_alpha[(((ring * 2) + (s_j >> 1)) * BM + s_row) * 2]) +
                             8 * H + 4 * (s_j & 1);
                *reinterpret_cast<uint32_t *>(arow + 16 * par) = R.al;
                *reinterpret_cast<uint32_t *>(arow + 16) = par ? R.al : 0u;
            } else if constexpr (S == 1) {
                q4k_fields((uint32_t)hdr[1], (uint32_t)hdr[2], (uint32_t)hdr[3], 2 * cl, 2, T.sc, T.mn);
            } else if constexpr (S >= 2 && S <= 5) {
                constexpr int e = S - 2;
                const uint32_t word = (uint32_t)R.q[e];
                uint32_t dh, dl;
                q4k_digits(word & 0x0F0F0F0Fu, T.sc[0], dh, dl);
                T.hl[e] = (int)dh;
                T.ll[e] = (int)dl;
                q4k_digits((word >> 4) & 0x0F0F0F0Fu, T.sc[1], dh, dl);
                T.hh[e] = (int)dh;
                T.lh[e] = (int)dl;
            } else if constexpr (S == 6) {
                const int pl = 4 * (wq >> 1) + (wq & 1);  // piece of the low nibbles
                *reinterpret_cast<v4i *>(p0 + swz(w_nl, pl)) = T.hl;
                *reinterpret_cast<v4i *>(p1 + swz(w_nl, pl)) = T.ll;
                *reinterpret_cast<v4i *>(p0 + swz(w_nl, pl + 2)) = T.hh;
                *reinterpret_cast<v4i *>(p1 + swz(w_nl, pl + 2)) = T.lh;
                s_dw[slot * BN + w_nl] = f16_bits_to_f32((uint32_t)hdr[0]);
            } else {
                // beta_j = -dmin * m_j for j = 4*H + wq (field 2*cl + (wq & 1))
                const float dmin = f16_bits_to_f32((uint32_t)hdr[0] >> 16);
                const uint32_t mj = (wq & 1) ? T.mn[1] : T.mn[0];
                __bf16 hi, lo;
                split_bf16(-dmin * (float)mj, hi, lo);
                const int e = 4 * H + wq;
                __bf16 *bh = reinterpret_cast<__bf16 *>(&s_beta[((ring * 2 + 0) * BN + w_nl) * 2]);
                __bf16 *bl = reinterpret_cast<__bf16 *>(&s_beta[((ring * 2 + 1) * BN + w_nl) * 2]);
                bh[8 * par + e] = hi;
                bl[8 * par + e] = lo;
                bh[8 + e] = par ? hi : (__bf16)0.0f;
                bl[8 + e] = par ? lo : (__bf16)0.0f;
            }
        } else if constexpr (Q6) {
            // piece S unpacks dword e = S & 1 of quarter u = S >> 1: weights
            // 128H + 32u + 8wq + 4e .. +4, sub-block scale 8H + 2u + (wq >> 1)
            constexpr int u = S >> 1, e = S & 1;
            if constexpr (S == 0) {
                const uint32_t sh = R.sh;
#pragma unroll
                for (int j = 0; j < 2; ++j)
#pragma unroll
                    for (int k = 0; k < 2; ++k)
                        T.ql[j][k] = __builtin_amdgcn_alignbyte(R.ql[3 * j + k + 1], R.ql[3 * j + k], sh);
#pragma unroll
                for (int k = 0; k < 2; ++k) T.qh[k] = __builtin_amdgcn_alignbyte(R.qh[k + 1], R.qh[k], sh);
                T.S0 = __builtin_amdgcn_alignbyte(R.sc[1], R.sc[0], sh);
                T.S1 = __builtin_amdgcn_alignbyte(R.sc[2], R.sc[1], sh);
            }
            const uint32_t Sw = (u < 2) ? T.S0 : T.S1;
            const int sc = __builtin_amdgcn_sbfe((int)Sw, (int)(16u * (u & 1) + 8u * (uint32_t)(wq >> 1)), 8);
            const uint32_t qlw = T.ql[u & 1][e];
            const uint32_t lo4 = (u < 2) ? (qlw & 0x0F0F0F0Fu) : ((qlw >> 4) & 0x0F0F0F0Fu);
            const uint32_t hi2 = (T.qh[e] >> (2 * u)) & 0x03030303u;
            q6k_digits(lo4 | (hi2 << 4), sc, T.vh[e], T.vl[e]);
            if constexpr (e == 1) {
                const int off = w_nl * MPITCH + 32 * u + 8 * wq;
                *reinterpret_cast<uint2 *>(p0 + off) = make_uint2(T.vh[0], T.vh[1]);
                *reinterpret_cast<uint2 *>(p1 + off) = make_uint2(T.vl[0], T.vl[1]);
            }
            if constexpr (S == 7) s_dw[slot * BN + w_nl] = f16_bits_to_f32(R.d);
        } else if constexpr (TQ2) {
            // code bytes 8wq .. 8wq+7: piece S (1..4) writes plane p = S - 1,
            // weights 32p + 8wq .. +8; piece 5 the block scale
            if constexpr (S >= 1 && S <= 4) {
                constexpr int pl = S - 1;
                uint32_t v[2];
#pragma unroll
                for (int e = 0; e < 2; ++e) {
                    const uint32_t cw = __builtin_amdgcn_alignbyte(R.w[e + 1], R.w[e], R.sh);
                    v[e] = codes_to_trits((cw >> (2 * pl)) & 0x03030303u);
                }
                *reinterpret_cast<uint2 *>(p0 + w_nl * MPITCH + 32 * pl + 8 * wq) = make_uint2(v[0], v[1]);
            } else if constexpr (S == 5) {
                float *dwp = (wq == 0) ? &s_dw[slot * BN + w_nl] : &s_dw[4 * BN + lane];
                *dwp = f16_bits_to_f32(R.d);
            }
        } else {
            // trit byte v -> five int8 trits from the table; byte b of this
            // thread's window fills row bytes 5*(tq_off + b) .. +5
            if constexpr (S <= 1) {
#pragma unroll
                for (int b = 4 * S; b < 4 * S + 4; ++b) {
                    const uint32_t v = (R.w[b >> 2] >> (8 * (b & 3))) & 0xFFu;
                    const uint2 t = *reinterpret_cast<const uint2 *>(&s_lut[2 * v]);
                    T.lo[b] = t.x;
                    T.hi[b] = t.y;
                }
            } else if constexpr (S == 3 || S == 4) {
                constexpr int g = S - 3, b = 4 * g;
                uint32_t o[5];
                o[0] = T.lo[b];
                o[1] = perm_b32(T.lo[b + 1], T.hi[b], 0x06050400u);
                o[2] = __builtin_amdgcn_alignbyte(T.hi[b + 1], T.lo[b + 1], 3) | (T.lo[b + 2] << 16);
                o[3] = __builtin_amdgcn_alignbyte(T.hi[b + 2], T.lo[b + 2], 2) | (T.lo[b + 3] << 24);
                o[4] = __builtin_amdgcn_alignbyte(T.hi[b + 3], T.lo[b + 3], 1);
                uint32_t *dst = reinterpret_cast<uint32_t *>(p0 + w_nl * MPITCH + 5 * tq_off) + 5 * g;
#pragma unroll
                for (int i = 0; i < 5; ++i) dst[i] = o[i];
            } else if constexpr (S == 5) {
                // d is bytes 26..27, the high half of the last quarter's second dword
                float *dwp = (wq == 3) ? &s_dw[slot * BN + w_nl] : &s_dw[4 * BN + lane];
                *dwp = f16_bits_to_f32(R.w[1] >> 16);
            }
        }
    };

    v16f acc_f[2];
    v16i acc[NDIG][2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        acc_f[i] = v16f{};
#pragma unroll
        for (int dg = 0; dg < NDIG; ++dg) acc[dg][i] = v16i{};
    }

    constexpr int KS = KCH / 32;  // MFMA K-steps per chunk
    // weight fragments of K-step ks (shared by both m-tiles)
    auto ld_b = [&](auto BB_, v4i (&Bv)[KS][NDIG], int ks) KQ_INLINE {
        constexpr int B = decltype(BB_)::value;
        const int8_t *sw = B ? s_w1 : s_w0;
#pragma unroll
        for (int dg = 0; dg < NDIG; ++dg)
            Bv[ks][dg] = *reinterpret_cast<const v4i *>(sw + dg * PLANE + swz(32 * wn + lrow, 2 * ks + kgrp));
    };
    // activation fragment of m-tile I, K-step ks
    auto ld_a = [&](auto BB_, v4i (&Av)[2][KS], int I, int ks) KQ_INLINE {
        constexpr int B = decltype(BB_)::value;
        const int8_t *sa = B ? s_a1 : s_a0;
        Av[I][ks] = *reinterpret_cast<const v4i *>(sa + swz(64 * wm + 32 * I + lrow, 2 * ks + kgrp));
    };
    // one int8 MFMA: m-tile I, K-step ks, digit plane dg; ks == 0 of a
    // restarting chunk starts from zero
    auto mfma_one = [&](auto II, auto KK, auto DD, auto FF, const v4i (&Av)[2][KS],
                        const v4i (&Bv)[KS][NDIG]) KQ_INLINE {
        constexpr int I = decltype(II)::value, ks = decltype(KK)::value, dg = decltype(DD)::value;
        constexpr bool ZERO = decltype(FF)::value && ks == 0;
        acc[dg][I] = ZERO ? mfma_i8_32x32x32(Av[I][ks], Bv[ks][dg], v16i{})
                          : mfma_i8_32x32x32(Av[I][ks], Bv[ks][dg], acc[dg][I]);
    };

    // ---- fold of m-tile I of scale block sb: out += float(T) * d_w[n] * d_a[m]
    struct FoldTmp {
        float dw;
        v4f da[4];
    };
    struct MinTmp {
        v8bf ah, al, bh, bl;  // Q4_K min-term operands
    };
    auto fold_load = [&](auto II, int sb, FoldTmp &F) KQ_INLINE {
        constexpr int I = decltype(II)::value;
        const int slot = sb & 3;
        F.dw = s_dw[slot * BN + 32 * wn + lrow];
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4)
            F.da[r4] = *reinterpret_cast<const v4f *>(&s_da[slot * BM + 64 * wm + 32 * I + 8 * r4 + 4 * kgrp]);
    };
    auto min_load = [&](auto II, int sb, MinTmp &Mt) KQ_INLINE {
        constexpr int I = decltype(II)::value;
        const int ring = (sb >> 1) & 1;
        const int col = 32 * wn + lrow;
        const int row = 64 * wm + 32 * I + lrow;
        Mt.bh = s_beta[((ring * 2 + 0) * BN + col) * 2 + kgrp];
        Mt.bl = s_beta[((ring * 2 + 1) * BN + col) * 2 + kgrp];
        Mt.ah = s_alpha[((ring * 2 + 0) * BM + row) * 2 + kgrp];
        Mt.al = s_alpha[((ring * 2 + 1) * BM + row) * 2 + kgrp];
    };
    // piece S of NP: outputs r in [S*16/NP, (S+1)*16/NP)
    auto fold_piece = [&](auto II, auto SS, auto NPC, const FoldTmp &F) KQ_INLINE {
        constexpr int I = decltype(II)::value, S = decltype(SS)::value, NP = decltype(NPC)::value;
#pragma unroll
        for (int r = S * 16 / NP; r < (S + 1) * 16 / NP; ++r) {
            int T;
            if constexpr (NDIG == 2)
                T = (acc[0][I][r] << Fmt<FMT>::SHIFT) + acc[1][I][r];
            else
                T = acc[0][I][r];
            acc_f[I][r] = fmaf((float)T * F.dw, F.da[r >> 2][r & 3], acc_f[I][r]);
        }
    };
    // Q4_K min term of a superblock pair: out += alpha . beta (hi/lo split)
    auto fold_min = [&](auto II, const MinTmp &Mt) KQ_INLINE {
        constexpr int I = decltype(II)::value;
        acc_f[I] = mfma_bf16_32x32x16(Mt.ah, Mt.bh, acc_f[I]);
        acc_f[I] = mfma_bf16_32x32x16(Mt.ah, Mt.bl, acc_f[I]);
        acc_f[I] = mfma_bf16_32x32x16(Mt.al, Mt.bh, acc_f[I]);
    };
    auto fold_all = [&](auto II, int sb, auto MINC) KQ_INLINE {
        FoldTmp F;
        fold_load(II, sb, F);
        static_for<0, 4>([&](auto S) KQ_INLINE { fold_piece(II, S, IC<4>{}, F); });
        if constexpr (decltype(MINC)::value) {
            MinTmp Mt;
            min_load(II, sb, Mt);
            fold_min(II, Mt);
        }
    };

    // ---- prologue ---------------------------------------------------------
    // slot 3 and the min-term operands start zeroed: the first iteration
    // folds tile 1 of a "scale block -1" whose accumulators are zero
    for (int i = tid; i < BM; i += MNT) s_da[3 * BM + i] = 0.0f;
    for (int i = tid; i < BN; i += MNT) s_dw[3 * BN + i] = 0.0f;
    if constexpr (Q4) {
        for (int i = tid; i < 2 * 2 * BM * 2; i += MNT) s_alpha[i] = v8bf{};
        for (int i = tid; i < 2 * 2 * BN * 2; i += MNT) s_beta[i] = v8bf{};
    }
    if constexpr (TQ) {
        if (tid < 256) {
            uint32_t lo, hi;
            tq_lut_entry((uint32_t)tid, lo, hi);
            *reinterpret_cast<uint2 *>(&s_lut[2 * tid]) = make_uint2(lo, hi);
        }
    }
    if (nch > 0) {
        prefetch(IC<0>{}, rg[0], 0);
        prefetch(IC<1>{}, rg[1], clampc(1));
    }
    __syncthreads();
    if (nch > 0) {
        StageTmp T;
        v4i hdr = v4i{};
        if constexpr (Q4) hdr = rg[0].hdr;
        static_for<0, 8>([&](auto S) KQ_INLINE { stage_piece(IC<0>{}, S, rg[0], hdr, 0, T); });
    }
    __syncthreads();

    // ---- one iteration, chunk c with compile-time phase U (c % 4 for
    // Q4_K/Q6_K, c % 2 for ternary).  The body is a fixed sequence of slots
    // separated by scheduling fences: each slot issues one MFMA plus a share
    // of the unpack or fold work and of the fragment reads for later slots.
    auto iteration = [&](auto UU, int c) KQ_INLINE {
        constexpr int U = decltype(UU)::value;
        constexpr int P = U & 1;  // LDS buffer and register set of chunk c
        using BP = IC<P>;
        using BQ = IC<1 - P>;
        const int cs = clampc(c + 1);
        const ChunkRegs<FMT> &Rs = rg[1 - P];
        // Q4_K header of the staged chunk's superblock: in register set 0 either
        // way (when P == 0 the staged chunk is the superblock's second and set
        // 0 holds its first, which the prefetch below overwrites)
        v4i hdr = v4i{};
        if constexpr (Q4) hdr = rg[0].hdr;
        prefetch(BP{}, rg[P], clampc(c + 2));
        v4i Bv[KS][NDIG], Av[2][KS];
        StageTmp T;
        ld_b(BP{}, Bv, 0);
        ld_b(BP{}, Bv, 1);
        ld_a(BP{}, Av, 0, 0);
        ld_a(BP{}, Av, 0, 1);
        if constexpr (TRI) {
            FoldTmp F1, F0;
            fold_load(IC<1>{}, c - 1, F1);
            __builtin_amdgcn_sched_barrier(0);
            static_for<0, 4>([&](auto S) KQ_INLINE {
                constexpr int s = decltype(S)::value;
                mfma_one(IC<0>{}, S, IC<0>{}, std::true_type{}, Av, Bv);
                if constexpr (s == 0) { ld_b(BP{}, Bv, 2); ld_b(BP{}, Bv, 3); }
                if constexpr (s == 1) ld_a(BP{}, Av, 0, 2);
                if constexpr (s == 2) ld_a(BP{}, Av, 0, 3);
                if constexpr (s == 3) {
                    ld_a(BP{}, Av, 1, 0);
                    ld_a(BP{}, Av, 1, 1);
                    fold_load(IC<0>{}, c, F0);
                }
                stage_piece(BQ{}, S, Rs, hdr, cs, T);
                fold_piece(IC<1>{}, S, IC<4>{}, F1);
                __builtin_amdgcn_sched_barrier(0);
            });
            static_for<0, 4>([&](auto S) KQ_INLINE {
                constexpr int s = decltype(S)::value;
                mfma_one(IC<1>{}, S, IC<0>{}, std::true_type{}, Av, Bv);
                if constexpr (s < 2) ld_a(BP{}, Av, 1, 2 + s);
                stage_piece(BQ{}, IC<4 + s>{}, Rs, hdr, cs, T);
                fold_piece(IC<0>{}, S, IC<4>{}, F0);
                __builtin_amdgcn_sched_barrier(0);
            });
        } else if constexpr (P == 0) {
            // first chunk of superblock c/2: fold tile 1 of the superblock
            // before it (odd when U == 0) under tile 0's MFMAs, then restart
            // tile 1 under the unpack
            constexpr bool MIN = Q4 && U == 0;
            FoldTmp F;
            MinTmp Mt;
            fold_load(IC<1>{}, c / 2 - 1, F);
            __builtin_amdgcn_sched_barrier(0);
            static_for<0, 8>([&](auto S) KQ_INLINE {
                constexpr int s = decltype(S)::value;
                mfma_one(IC<0>{}, IC<(s >> 1)>{}, IC<(s & 1)>{}, std::true_type{}, Av, Bv);
                if constexpr (s == 0) ld_b(BP{}, Bv, 2);
                if constexpr (s == 1) ld_a(BP{}, Av, 0, 2);
                if constexpr (s == 2) ld_b(BP{}, Bv, 3);
                if constexpr (s == 3) ld_a(BP{}, Av, 0, 3);
                if constexpr (s >= 4) ld_a(BP{}, Av, 1, s - 4);
                if constexpr (MIN && s == 5) min_load(IC<1>{}, c / 2 - 1, Mt);
                fold_piece(IC<1>{}, S, IC<8>{}, F);
                __builtin_amdgcn_sched_barrier(0);
            });
            if constexpr (MIN) {
                fold_min(IC<1>{}, Mt);
                __builtin_amdgcn_sched_barrier(0);
            }
            static_for<0, 8>([&](auto S) KQ_INLINE {
                constexpr int s = decltype(S)::value;
                mfma_one(IC<1>{}, IC<(s >> 1)>{}, IC<(s & 1)>{}, std::true_type{}, Av, Bv);
                stage_piece(BQ{}, S, Rs, hdr, cs, T);
                __builtin_amdgcn_sched_barrier(0);
            });
        } else {
            // second chunk: tile 0's MFMAs under the unpack, then fold tile 0
            // (min term when the superblock is odd, U == 3) under tile 1's
            constexpr bool MIN = Q4 && U == 3;
            FoldTmp F;
            MinTmp Mt;
            __builtin_amdgcn_sched_barrier(0);
            static_for<0, 8>([&](auto S) KQ_INLINE {
                constexpr int s = decltype(S)::value;
                mfma_one(IC<0>{}, IC<(s >> 1)>{}, IC<(s & 1)>{}, std::false_type{}, Av, Bv);
                if constexpr (s == 0) ld_b(BP{}, Bv, 2);
                if constexpr (s == 1) ld_a(BP{}, Av, 0, 2);
                if constexpr (s == 2) ld_b(BP{}, Bv, 3);
                if constexpr (s == 3) ld_a(BP{}, Av, 0, 3);
                if constexpr (s >= 4) ld_a(BP{}, Av, 1, s - 4);
                if constexpr (s == 5) fold_load(IC<0>{}, c / 2, F);
                stage_piece(BQ{}, S, Rs, hdr, cs, T);
                __builtin_amdgcn_sched_barrier(0);
            });
            static_for<0, 8>([&](auto S) KQ_INLINE {
                constexpr int s = decltype(S)::value;
                mfma_one(IC<1>{}, IC<(s >> 1)>{}, IC<(s & 1)>{}, std::false_type{}, Av, Bv);
                if constexpr (MIN && s == 5) min_load(IC<0>{}, c / 2, Mt);
                fold_piece(IC<0>{}, S, IC<8>{}, F);
                __builtin_amdgcn_sched_barrier(0);
            });
            if constexpr (MIN) fold_min(IC<0>{}, Mt);
        }
        __syncthreads();
    };

    if constexpr (CPS == 2) {
        int c = 0;
        for (; c + 4 <= nch; c += 4) {
            iteration(IC<0>{}, c);
            iteration(IC<1>{}, c + 1);
            iteration(IC<2>{}, c + 2);
            iteration(IC<3>{}, c + 3);
        }
        if (c < nch) {  // nch is even
            iteration(IC<0>{}, c);
            iteration(IC<1>{}, c + 1);
        }
        if (nch > 0) {
            const int lastb = nch / 2 - 1;
            fold_all(IC<1>{}, lastb, std::integral_constant<bool, Q4>{});
            if constexpr (Q4) {
                if ((lastb & 1) == 0) {
                    // an even last superblock: its pair's min term is still due for tile 0
                    MinTmp Mt;
                    min_load(IC<0>{}, lastb, Mt);
                    fold_min(IC<0>{}, Mt);
                }
            }
        }
    } else {
        int c = 0;
        for (; c + 2 <= nch; c += 2) {
            iteration(IC<0>{}, c);
            iteration(IC<1>{}, c + 1);
        }
        if (c < nch) iteration(IC<0>{}, c);
        if (nch > 0) fold_all(IC<1>{}, nch - 1, std::false_type{});
    }


    // ---- epilogue: fp32 stores (unmasked when the whole tile is inside) ----
    float *out = reinterpret_cast<float *>(a.out);
    const bool full = (mrows == BM) && (n0 + BN <= N);
    const int n = n0 + 32 * wn + lrow;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int ml = 64 * wm + 32 * i + mfma32_row(r, lane);
            if (full || (ml < mrows && n < N)) {
                if constexpr (SPLIT) unsafeAtomicAdd(&out[(orow0 + ml) * N + n], acc_f[i][r]);
                else out[(orow0 + ml) * N + n] = acc_f[i][r];
            }
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
                          const uint16_t *alpha, void *out, int M, int N, int K, int bm,
                          int bn) {
    GemmArgs a;
    a.W = (const uint8_t *)W;
    a.qs = qs;
    a.da = da;
    a.alpha = alpha;
    a.out = out;
    a.M = M;
    a.N = N;
    a.K = K;
    a.nchunks = (K + KC - 1) / KC;
    a.nblk = (fmt == FMT_TQ || fmt == FMT_TQ2) ? K / 128 : K / 256;
    a.tiles_m = (M + bm - 1) / bm;
    a.tiles_n = (N + bn - 1) / bn;
    a.exp_off = nullptr;
    a.rows = nullptr;
    a.n_experts = 0;
    a.n_routed = 0;
    a.expert_bytes = 0;
    return a;
}

hipError_t launch_gemm_q4k(const void *W, const int8_t *qs, const float *da,
                           const uint16_t *alpha, float *out, int M, int N, int K,
                           hipStream_t stream);

// K in two parts where the tiles cover at most half the CUs (one round
// either way) and half of K outweighs the split's own cost: the zero fill
// and two atomic adds per output, which the L2 takes at about 0.3 per ns,
// modelled as M * N / 1536 in units of K (plus 256 for the second launch).
// Paired runs, us, whole K / split: Q6_K 512 x 4096 x 14336 143 / 96; 512 x
// 4096 x 4096 44.8 / 42.1; 128 x 14336 x 4096 46.5 / 41.0; 300 x 4000 x
// 2048 25.9 / 23.7; base-3 9 x 4096 x 5248 42.7 / 28.7; the whole-K kernel
// at half K (one part's share) on Q6_K 512 x 4096 x 14336: 76.
static int64_t split_units(int M, int N, int K) { return K / 2 + 256 + (int64_t)M * N / 1536; }

bool tile_split_choice(int fmt, int M, int N, int K) {
    if (fmt != FMT_Q6K && fmt != FMT_TQ && fmt != FMT_TQ2) return false;
    if (M <= 0 || N <= 0 || K < 1024) return false;
    const int64_t tiles = ((int64_t)M + MBM - 1) / MBM * (((int64_t)N + MBN - 1) / MBN);
    return 2 * tiles <= num_cus() && split_units(M, N, K) < K;
}

int64_t tile_units(int fmt, int M, int N, int K) {
    if (tile_split_choice(fmt, M, N, K)) return split_units(M, N, K);
    const int cus = num_cus();
    const int64_t tiles = ((int64_t)M + MBM - 1) / MBM * (((int64_t)N + MBN - 1) / MBN);
    return (tiles + cus - 1) / cus * K;
}

hipError_t launch_gemm(int fmt, const void *W, const int8_t *qs, const float *da,
                       const uint16_t *alpha, float *out, int M, int N, int K,
                       hipStream_t stream) {
    if (fmt == FMT_Q4K) return launch_gemm_q4k(W, qs, da, alpha, out, M, N, K, stream);
    if (gemv_choice(fmt, M, N, K)) return launch_gemv(fmt, W, qs, da, out, M, N, K, stream);
    if (ring_choice(fmt, M, N, K)) return launch_gemm_ring(fmt, W, qs, da, nullptr, out, M, N, K, stream);
    if (fmt == FMT_TQ && tq_tile_choice(M, N, K)) return launch_gemm_tq_tile(W, qs, da, out, M, N, K, stream);
    GemmArgs a = make_args(fmt, W, qs, da, alpha, out, M, N, K, MBM, MBN);
    const unsigned grid = (unsigned)(a.tiles_m * a.tiles_n);
    if (tile_split_choice(fmt, M, N, K)) {
        const hipError_t e = launch_zero_fill(out, (int64_t)M * N, stream);
        if (e != hipSuccess) return e;
        const dim3 g2(grid, 2);
        if (fmt == FMT_Q6K) hipLaunchKernelGGL((gemm_kernel<FMT_Q6K, false, true>), g2, dim3(MNT), 0, stream, a);
        else if (fmt == FMT_TQ2) hipLaunchKernelGGL((gemm_kernel<FMT_TQ2, false, true>), g2, dim3(MNT), 0, stream, a);
        else hipLaunchKernelGGL((gemm_kernel<FMT_TQ, false, true>), g2, dim3(MNT), 0, stream, a);
        return hipGetLastError();
    }
    switch (fmt) {
        case FMT_Q6K:
            hipLaunchKernelGGL(gemm_kernel<FMT_Q6K>, dim3(grid), dim3(MNT), 0, stream, a);
            break;
        case FMT_TQ2:
            hipLaunchKernelGGL(gemm_kernel<FMT_TQ2>, dim3(grid), dim3(MNT), 0, stream, a);
            break;
        default:
            hipLaunchKernelGGL(gemm_kernel<FMT_TQ>, dim3(grid), dim3(MNT), 0, stream, a);
            break;
    }
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Loader test hook: nblocks consecutive blocks of W, read as one weight row,
// go through load_w and unpack_w (unit scales) -- the loaders of the tile
// kernel above -- and the integer operand of every value is rebuilt from the
// digit planes as the MFMA accumulation does (high plane << SHIFT plus low
// plane).  The scale fields come from the same words the loader fetched:
// q4k_fields for the Q4_K 6-bit scales and mins, the realigned scale bytes for
// Q6_K.  One thread per chunk half (Q4_K, Q6_K: 128 values of a superblock;
// ternary: one 128-value block), 32 chunks per 64-thread workgroup.
// ---------------------------------------------------------------------------
constexpr int DBG_CHUNKS = 32;

template <int FMT>
__global__ __launch_bounds__(64) void debug_unpack_kernel(GemmArgs a, int8_t *q, int32_t *scales) {
    constexpr int NDIG = Fmt<FMT>::NDIG, SHIFT = Fmt<FMT>::SHIFT;
    __shared__ __attribute__((aligned(16))) int8_t s_w[NDIG * DBG_CHUNKS * PITCH];
    __shared__ float s_dw[2 * DBG_CHUNKS];
    const int nl = threadIdx.x >> 1, part = threadIdx.x & 1;
    const int c = blockIdx.x * DBG_CHUNKS + nl;
    // block holding this thread's values
    const int64_t b = tri(FMT) ? 2 * (int64_t)c + part : c;
    const bool valid = b < a.nblk;
    WRaw<FMT> wr;
    // past the end: Q4_K/Q6_K read block 0 instead (nothing is stored); the
    // ternary loader fills blocks past nblk itself without reading
    load_w<FMT>(wr, a, 0, part, (valid || tri(FMT)) ? c : 0);
    unpack_w<FMT, true>(wr, valid, s_w, DBG_CHUNKS * PITCH, nl, part, s_dw, DBG_CHUNKS, nullptr, 0,
                        false);
    __syncthreads();
    if (!valid) return;

    const int8_t *hi = s_w + nl * PITCH + 128 * part;
    int8_t *dst = q + (tri(FMT) ? b * 128 : b * 256 + 128 * part);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        v4i h = *reinterpret_cast<const v4i *>(hi + 16 * i), v;
        if constexpr (NDIG == 2) {
            const v4i l = *reinterpret_cast<const v4i *>(hi + DBG_CHUNKS * PITCH + 16 * i);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                uint32_t w = 0;
#pragma unroll
                for (int bb = 0; bb < 4; ++bb) {
                    const int hv = (int8_t)(h[e] >> (8 * bb)), lv = (int8_t)(l[e] >> (8 * bb));
                    w |= (uint32_t)((hv * (1 << SHIFT) + lv) & 0xFF) << (8 * bb);
                }
                v[e] = (int)w;
            }
        } else {
            v = h;
        }
        *reinterpret_cast<v4i *>(dst + 16 * i) = v;
    }
    if constexpr (FMT == FMT_Q4K) {
        uint32_t sc[4], mn[4];
        q4k_fields((uint32_t)wr.hdr[1], (uint32_t)wr.hdr[2], (uint32_t)wr.hdr[3], 4 * part, 4, sc, mn);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            scales[b * 16 + 4 * part + i] = (int32_t)sc[i];
            scales[b * 16 + 8 + 4 * part + i] = (int32_t)mn[i];
        }
    } else if constexpr (FMT == FMT_Q6K) {
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const uint32_t w = q6k_realign(wr.sc[j >> 2], wr.sc[(j >> 2) + 1], wr.shift);
            scales[b * 16 + 8 * part + j] = (int32_t)(int8_t)(w >> (8 * (j & 3)));
        }
    }
}

hipError_t launch_debug_unpack(int fmt, const void *W, int64_t nblocks, int8_t *q, int32_t *scales,
                               hipStream_t stream) {
    GemmArgs a{};
    a.W = (const uint8_t *)W;
    a.nblk = (int)nblocks;
    const int64_t chunks = (fmt == FMT_TQ || fmt == FMT_TQ2) ? (nblocks + 1) / 2 : nblocks;
    const unsigned grid = (unsigned)((chunks + DBG_CHUNKS - 1) / DBG_CHUNKS);
    switch (fmt) {
        case FMT_Q4K:
            hipLaunchKernelGGL(debug_unpack_kernel<FMT_Q4K>, dim3(grid), dim3(64), 0, stream, a, q, scales);
            break;
        case FMT_Q6K:
            hipLaunchKernelGGL(debug_unpack_kernel<FMT_Q6K>, dim3(grid), dim3(64), 0, stream, a, q, scales);
            break;
        case FMT_TQ2:
            hipLaunchKernelGGL(debug_unpack_kernel<FMT_TQ2>, dim3(grid), dim3(64), 0, stream, a, q, scales);
            break;
        default:
            hipLaunchKernelGGL(debug_unpack_kernel<FMT_TQ>, dim3(grid), dim3(64), 0, stream, a, q, scales);
            break;
    }
    return hipGetLastError();
}

// Expert-indexed product on the tile kernel (gather mode): out [R][N], row r =
// W[e(r)] x A[rows[r]].  The grid covers an upper bound of the M-tiles,
// ceil(R / BM) + n_experts; surplus workgroups return at once.
hipError_t launch_gemm_id(int fmt, const void *W, int n_experts, int64_t expert_bytes,
                          const int8_t *qs, const float *da, const uint16_t *alpha,
                          const int32_t *exp_off, const int32_t *rows, int R, float *out, int M,
                          int N, int K, hipStream_t stream) {
    GemmArgs a = make_args(fmt, W, qs, da, alpha, out, M, N, K, MBM, MBN);
    a.tiles_m = (R + MBM - 1) / MBM + n_experts;
    a.exp_off = exp_off;
    a.rows = rows;
    a.n_experts = n_experts;
    a.n_routed = R;
    a.expert_bytes = expert_bytes;
    const unsigned grid = (unsigned)(a.tiles_m * a.tiles_n);
    switch (fmt) {
        case FMT_Q6K:
            hipLaunchKernelGGL((gemm_kernel<FMT_Q6K, true>), dim3(grid), dim3(MNT), 0, stream, a);
            break;
        case FMT_TQ2:
            hipLaunchKernelGGL((gemm_kernel<FMT_TQ2, true>), dim3(grid), dim3(MNT), 0, stream, a);
            break;
        default:
            hipLaunchKernelGGL((gemm_kernel<FMT_TQ, true>), dim3(grid), dim3(MNT), 0, stream, a);
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
        case FMT_TQ2:
            hipLaunchKernelGGL(subsums_kernel<FMT_TQ2>, dim3(grid), dim3(64), 0, stream, a);
            break;
        default:
            hipLaunchKernelGGL(subsums_kernel<FMT_TQ>, dim3(grid), dim3(64), 0, stream, a);
            break;
    }
    return hipGetLastError();
}

}  // namespace kq
