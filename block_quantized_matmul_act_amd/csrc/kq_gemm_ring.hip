// kq_gemm_ring.hip -- few-token products (gfx950) for Q6_K and ternary
// weights: up to 64 tokens, past the matrix-vector kernels (the tile
// GEMM of vllm.cpp PR 3036 over Q6_K weights and BlockQ8_K activations, and
// the ternary MMQ path of llama.cpp PR 214, at the small-batch end of the
// mul_mat_q / mat-vec crossover).
//
// The 128 x 128 tile kernel leaves most of the chip idle here: 4096 weight
// rows are 32 tiles whatever the token count.  This kernel takes all tokens
// (a 16-, 32- or 64-row token tile, TM) in one workgroup and splits the
// weights over workgroups by rows and over waves by rows and K:
//   * A workgroup of NW = 8 waves owns 16 * (NW / KP) weight rows as 16-row
//     strips; the K-chunks of 256 values are cut into KP contiguous K-parts
//     (KP = 2, 4 or 8), and wave w takes strip w % (NW / KP) over K-part
//     w / (NW / KP).  Narrow weights take more K-parts so that the grid still
//     covers the CUs; where the LDS of 64 token rows stops at four K-parts, a
//     four-wave build (NW = 4, one strip per K-part) doubles the workgroups.
//   * Step x multiplies chunk pT + x of every K-part p (T = ceil(chunks /
//     KP)).  A step's activations (values and scales of every K-part, all
//     token rows) are copied global -> LDS into a ring of L + 1 slots, L
//     steps ahead; each wave loads its strip's weights for the same step into
//     a register ring in the same issue.  Vector-memory loads complete in
//     issue order, so the wait for a step's copies also waits for the weights
//     issued before them: those of the same step or earlier.
//   * The loop runs whole ring turns (steps past a part's end read through a
//     buffer resource with no records: zeros, no memory access), then the
//     T mod (L + 1) steps left over, which issue nothing.
//   * The K-parts are summed through LDS at the end, in a fixed order.
//
// A chunk is four K-steps of v_mfma_i32_16x16x64_i8: in K-step s, lane group
// kg (lane / 16) supplies 16 values of its token row (A) and of its weight
// row (B) in the same K order.  Per format:
//   * Q6_K (210 bytes per superblock of 256): lane group kg holds the values
//     128h + 32u + 16(s % 2) + i with h = kg/2, u = 2(kg % 2) + s/2, sub-block
//     4kg + s: the low (kg even) or high (kg odd) nibbles of ql bytes 64h +
//     16s + i, bits 4(kg % 2) + 2(s/2) of qh bytes 32h + 16(s % 2) + i, and
//     scale byte 4kg + s; so a lane reads 64 contiguous ql bytes, 32 qh bytes
//     and 4 scale bytes per superblock, and its A operand is the 16
//     activation bytes at 64kg + 16s.  W = sc (q - 32) = 64 h + l is split
//     into two int8 digits (q6k_digits), two MFMAs per K-step and m-tile, and
//     the superblock's sum T = 64 acc_h + acc_l is folded once:
//     out += d_a * d * T.
//   * Base-3 ternary (28 bytes per block of 128, 4-byte aligned; a chunk is
//     two blocks): K-steps 2b and 2b + 1 cover block b, lane group kg the
//     trits 32kg + 16(s % 2) + i of it, which lie in 4 bytes starting at byte
//     (32kg + 16(s % 2)) / 5, digit (32kg + 16(s % 2)) mod 5; a lane loads the
//     3 dwords that hold both its windows.  Each byte goes through a 256-entry
//     LDS table (its five trits as int8), the four 5-trit groups are packed
//     into 20 bytes and the 16 wanted taken from the digit offset.  The A
//     operand is the 16 activation bytes at 128b + 32kg + 16(s % 2).
//   * Two-bit ternary (34 bytes per block of 128; a chunk is two blocks):
//     K-steps 2b and 2b + 1 cover block b, lane group kg the values 64(s % 2)
//     + 16kg + i of it: plane 2(s % 2) + kg/2 of code bytes 16(kg % 2) + i,
//     so a lane reads 16 code bytes per block; its A operand is the 16
//     activation bytes at 64s + 16kg.  The trits are int8 operands as they
//     are (one MFMA per K-step and m-tile), and each block's sum is folded
//     after its two K-steps with the block's weight and activation scales.
// Blocks are 2-byte aligned: a lane loads aligned dwords and shifts them into
// place with v_alignbit; the fp16 weight scales come in 2-byte loads (their
// aligned dword can pass the buffer's end).
#include "kq_device.hpp"
#include "kq_launch.hpp"
#include "kq_tile.hpp"

namespace kq {
namespace rk {
using namespace tl;

enum { F_Q4K = 1, F_Q6K = 2, F_TQ = 3, F_TQ2 = 4 };  // the API's format numbers
constexpr int ROW = 256;         // LDS bytes per staged activation row (one chunk)

struct Args {
    const uint8_t *W;
    const int8_t *qs;
    const float *da;        // [K / (256 / NBLK)][M]
    const uint16_t *alpha;  // Q4_K: [K / 256][2][M][8] bf16, exact parts of the sub-block sums
    float *out;
    int M, N, K, nch;  // nch: 256-value chunks per row
};

template <int F>
struct Fmt;
template <>
struct Fmt<F_Q4K> {
    static constexpr int CB = 144;      // weight bytes per chunk of a row
    static constexpr int NBLK = 1;      // scale blocks per chunk
    static constexpr int NDIG = 2;      // int8 digits per weight
    static constexpr int SHIFT = 3;     // T = (digit-0 sum << SHIFT) + digit-1 sum
    static constexpr int WLOADS = 3;    // weight load instructions per lane and chunk
    __device__ static int piece(int s, int kg) { return 4 * kg + s; }
};
template <>
struct Fmt<F_Q6K> {
    static constexpr int CB = 210;
    static constexpr int NBLK = 1;
    static constexpr int NDIG = 2;
    static constexpr int SHIFT = 6;
    static constexpr int WLOADS = 10;
    __device__ static int piece(int s, int kg) { return 4 * kg + s; }
};
template <>
struct Fmt<F_TQ> {
    static constexpr int CB = 56;
    static constexpr int NBLK = 2;
    static constexpr int NDIG = 1;
    static constexpr int SHIFT = 0;
    static constexpr int WLOADS = 6;
    __device__ static int piece(int s, int kg) { return 8 * (s >> 1) + (s & 1) + 2 * kg; }
};
template <>
struct Fmt<F_TQ2> {
    static constexpr int CB = 68;
    static constexpr int NBLK = 2;
    static constexpr int NDIG = 1;
    static constexpr int SHIFT = 0;
    static constexpr int WLOADS = 6;
    __device__ static int piece(int s, int kg) { return 4 * s + kg; }
};

template <int F, int TM, int KP, int NW = 8>
struct Cfg {
    static_assert(TM == 16 || TM == 32 || TM == 64, "16, 32 or 64 token rows");
    static_assert(KP == 2 || KP == 4 || KP == 8, "two, four or eight K-parts");
    static_assert(NW == 8 || NW == 4, "eight or four waves");
    using FM = Fmt<F>;
    static constexpr int MT = TM / 16;            // 16-row m-tiles
    static constexpr int NS = NW / KP;            // 16-row strips per workgroup
    static_assert(NS >= 1, "a strip per K-part at least");
    static constexpr int ROWS = 16 * NS;          // weight rows per workgroup
    static constexpr int ACT = TM * ROW;          // values of one K-part: [row][256], swizzled
    // Q4_K min-term operands of one K-part: [hi, lo][TM][16] in 1 KiB copies
    static constexpr int NAL = F == F_Q4K ? (TM == 64 ? 2 : 1) : 0;
    static constexpr int ALO = ACT + 256 * FM::NBLK;   // ... after the scales (64-lane 4-byte copies)
    static constexpr int PART = ALO + 1024 * NAL;
    static constexpr int SLOT = KP * PART;
    // after the slots: the base-3 decode table, or the zeros lanes of
    // k-groups 2 and 3 read as their Q4_K min-term operand
    static constexpr int EXTRA = F == F_TQ ? 256 * 8 : F == F_Q4K ? 1024 : 0;
    static constexpr int LDS_MAX = 160 * 1024;
    // steps of lead: three with 16 token rows, two otherwise, one where two
    // do not fit the LDS
    static constexpr int L = TM == 16 && 4 * SLOT + EXTRA <= LDS_MAX ? 3 : (3 * SLOT + EXTRA <= LDS_MAX ? 2 : 1);
    static constexpr int S = L + 1;               // LDS slots and weight register sets
    static constexpr int LDS = S * SLOT + EXTRA;
    static_assert(LDS <= 160 * 1024, "LDS");
    static constexpr int NA = ACT / 1024;         // value copies per K-part
    static constexpr int CPV = NA / NS;           // ... per wave
    static_assert(CPV * NS == NA, "value copies split evenly over a part's waves");
    // vector-memory instructions per wave and step: value copies, scale
    // copies, min-term operand copies, weight loads
    static constexpr int LOADS = CPV + FM::NBLK + NAL + FM::WLOADS;
    static_assert(LOADS * (L - 1) < 64, "vmcnt range");
    // the K-parts' sums through LDS at the end
    static_assert((KP - 1) * NS * MT * 4 * 64 * 4 <= LDS, "reduction space");
};

// one chunk of a lane's weights, as loaded
template <int F>
struct WRaw;
template <>
struct WRaw<F_Q4K> {
    v4i hdr, q0, q1;      // block header; nibble bytes 32kg .. +15, 32kg + 16 .. +15
};
template <>
struct WRaw<F_Q6K> {
    v4i l0, l1, l2, l3;   // ql: 68 bytes from the aligned start of its 64
    uint32_t l4;
    v4i h0, h1;           // qh: 36 bytes from the aligned start of its 32
    uint32_t h2;
    v2u sc;               // the dwords holding its 4 scale bytes
    uint32_t dd;          // d
};
template <>
struct WRaw<F_TQ> {
    v2u w01[2];           // per block: the 3 dwords holding its trit windows
    uint32_t w2[2];
    uint32_t dd[2];       // per block: d
};
template <>
struct WRaw<F_TQ2> {
    v4i c[2];             // per block: 20 bytes from the aligned start of its 16 code bytes
    uint32_t c4[2];
    uint32_t dd[2];       // per block: d
};

template <int F, int TM, int KP, int NW = 8>
__global__ __launch_bounds__(64 * NW, 1) void gemm_ring_kernel(Args a) {
    using C = Cfg<F, TM, KP, NW>;
    using FM = Fmt<F>;
    constexpr int MT = C::MT, NS = C::NS, NBLK = FM::NBLK, NDIG = FM::NDIG;
    constexpr int KSB = 4 / NBLK;  // K-steps per scale block
    __shared__ __attribute__((aligned(16))) int8_t s_lds[C::LDS];

    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int strip = w % NS, part = w / NS;
    const int r16 = lane & 15, kg = lane >> 4;
    const int M = a.M, N = a.N, K = a.K, nch = a.nch;
    const int T = (nch + KP - 1) / KP;  // steps
    const int n0 = blockIdx.x * C::ROWS + 16 * strip;
    const int rowbytes = nch * FM::CB;

    // token slice: rows m0 .. m0 + TM - 1 (the resources start at row m0,
    // strides stay those of the whole M)
    const int m0 = blockIdx.y * TM;
    const auto rs_a = __builtin_amdgcn_make_buffer_rsrc((void *)(a.qs + (size_t)m0 * K), (short)0, (M - m0) * K,
                                                        RSRC_FLAGS);
    const auto rs_d = __builtin_amdgcn_make_buffer_rsrc((void *)(a.da + m0), (short)0, (nch * NBLK * M - m0) * 4,
                                                        RSRC_FLAGS);
    const auto rs_w = __builtin_amdgcn_make_buffer_rsrc((void *)a.W, (short)0, N * rowbytes, RSRC_FLAGS);
    const auto rs_o = __builtin_amdgcn_make_buffer_rsrc((void *)(a.out + (size_t)m0 * N), (short)0, (M - m0) * N * 4,
                                                        RSRC_FLAGS);
    const auto rs_l = __builtin_amdgcn_make_buffer_rsrc((void *)(F == F_Q4K ? a.alpha + (size_t)m0 * 8 : a.alpha), (short)0,
                                                        (nch * 2 * M - m0) * 16, RSRC_FLAGS);
    // no records: reads return zero without a memory access (copies and
    // loads of steps past a part's end, so that every step issues the same)
    const auto rs_nul = __builtin_amdgcn_make_buffer_rsrc((void *)a.W, (short)0, 0, RSRC_FLAGS);
    int8_t *const zero = s_lds + C::S * C::SLOT;
    if constexpr (F == F_Q4K) {
        for (int i = tid; i < 256; i += 64 * NW) reinterpret_cast<uint32_t *>(zero)[i] = 0u;
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    }

    // base-3 decode table: entry v = the five trits of byte v (t0..t3 in the
    // low word, t4 in the high word); the stores complete before the first
    // step's barrier (which carries no fence), so every wave sees them after
    uint32_t *const lut = reinterpret_cast<uint32_t *>(s_lds + C::S * C::SLOT);
    if constexpr (F == F_TQ) {
        if (tid < 256) {
            uint32_t lo, hi;
            tq_lut_entry((uint32_t)tid, lo, hi);
            lut[2 * tid] = lo;
            lut[2 * tid + 1] = hi;
        }
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    }

    // ---- copies of step x into slot x % S.  The NS waves of K-part p copy
    // its values (copy r: rows 4r .. 4r+3; lane l fills piece l%16 of row
    // 4r + l/16 with piece (l%16) ^ row), CPV copies each, and each copies
    // the part's scales (lane l: token l; the same bytes to the same place),
    // so every wave issues the same; for Q4_K each also copies the part's
    // min-term operands (TM = 64: copy j is part j, lane l token l; TM = 32:
    // lane l part l/32, token l%32; TM = 16: lane l part (l/16)%2, token
    // l%16, lanes 32..63 into padding).  Token rows past M read other rows'
    // data or zero; their outputs are dropped.
    int a_vo[C::CPV];
    int l_vo[C::NAL > 0 ? C::NAL : 1];
#pragma unroll
    for (int j = 0; j < C::NAL; ++j)
        l_vo[j] = TM == 64 ? (j * M + lane) * 16
                           : TM == 32 ? ((lane >> 5) * M + (lane & 31)) * 16 : (((lane >> 4) & 1) * M + (lane & 15)) * 16;
#pragma unroll
    for (int i = 0; i < C::CPV; ++i) {
        const int row = 4 * (C::CPV * strip + i) + (lane >> 4);
        a_vo[i] = row * K + 16 * ((lane & 15) ^ (row & 15));
    }
    auto copies = [&](int x) __attribute__((always_inline)) {
        int8_t *P = s_lds + (x % C::S) * C::SLOT + part * C::PART;
        const int ch = part * T + x;
        const bool real = x < T && ch < nch;
        const int chr = real ? ch : 0;
#pragma unroll
        for (int i = 0; i < C::CPV; ++i)
            copy16(real ? rs_a : rs_nul, P + (C::CPV * strip + i) * 1024, a_vo[i], chr * ROW);
#pragma unroll
        for (int bb = 0; bb < NBLK; ++bb)
            copy4(real ? rs_d : rs_nul, P + C::ACT + 256 * bb, 4 * lane, (chr * NBLK + bb) * M * 4);
#pragma unroll
        for (int j = 0; j < C::NAL; ++j) copy16(real ? rs_l : rs_nul, P + C::ALO + 1024 * j, l_vo[j], chr * 2 * M * 16);
    };
    // ---- this lane's weights: row n0 + r16 (row offsets as unsigned: rows
    // past N may pass 2^31, and the range check drops them)
    const uint32_t w_row = (uint32_t)(n0 + r16) * (uint32_t)rowbytes;
    WRaw<F> ring[C::S];
    auto wload = [&](int x, WRaw<F> &R) __attribute__((always_inline)) {
        const int ch = part * T + x;
        const bool real = x < T && ch < nch;
        const auto rw = real ? rs_w : rs_nul;
        const uint32_t b = w_row + (uint32_t)((real ? ch : 0) * FM::CB);  // chunk start
        if constexpr (F == F_Q4K) {
            // (blocks are 144 bytes: 16-byte aligned)
            R.hdr = ld16(rw, (int)b, 0);
            R.q0 = ld16(rw, (int)b + 16 + 32 * kg, 0);
            R.q1 = ld16(rw, (int)b + 32 + 32 * kg, 0);
        } else if constexpr (F == F_Q6K) {
            // the aligned dword at or below the block start (every field
            // offset used with it is a multiple of 4)
            const int b4 = (int)(b & ~3u);
            const int o_ql = 64 * (kg >> 1), o_qh = 128 + 32 * (kg >> 1), o_sc = 192 + 4 * kg;
            R.l0 = ld16(rw, b4 + o_ql, 0);
            R.l1 = ld16(rw, b4 + o_ql + 16, 0);
            R.l2 = ld16(rw, b4 + o_ql + 32, 0);
            R.l3 = ld16(rw, b4 + o_ql + 48, 0);
            R.l4 = ld4(rw, b4 + o_ql + 64, 0);
            R.h0 = ld16(rw, b4 + o_qh, 0);
            R.h1 = ld16(rw, b4 + o_qh + 16, 0);
            R.h2 = ld4(rw, b4 + o_qh + 32, 0);
            R.sc = ld8(rw, b4 + o_sc, 0);
            R.dd = (uint32_t)__builtin_amdgcn_raw_buffer_load_b16(rw, (int)b + 208, 0, 0);
        } else if constexpr (F == F_TQ) {
            // dwords {0, 1, 3, 4}[kg] .. +2 of each block
            const int o3 = kg == 0 ? 0 : kg == 1 ? 4 : kg == 2 ? 12 : 16;
#pragma unroll
            for (int bb = 0; bb < 2; ++bb) {
                R.w01[bb] = ld8(rw, (int)b + 28 * bb + o3, 0);
                R.w2[bb] = ld4(rw, (int)b + 28 * bb + o3 + 8, 0);
                R.dd[bb] = (uint32_t)__builtin_amdgcn_raw_buffer_load_b16(rw, (int)b + 28 * bb + 26, 0, 0);
            }
        } else {
#pragma unroll
            for (int bb = 0; bb < 2; ++bb) {
                const int c4 = (int)((b + 34u * bb + 16u * (kg & 1)) & ~3u);
                R.c[bb] = ld16(rw, c4, 0);
                R.c4[bb] = ld4(rw, c4 + 16, 0);
                R.dd[bb] = (uint32_t)__builtin_amdgcn_raw_buffer_load_b16(rw, (int)b + 34 * bb + 32, 0, 0);
            }
        }
    };

    v4f out[MT];
#pragma unroll
    for (int t = 0; t < MT; ++t) out[t] = v4f{};
    // LDS addresses: K-step s of m-tile t reads row 16t + r16 of this wave's
    // K-part, piece piece(s, kg) ^ r16; the scales of tokens 4kg .. 4kg+3 of
    // m-tile t and block bb follow the values
    uint32_t a_ad[4];
#pragma unroll
    for (int s = 0; s < 4; ++s)
        a_ad[s] = lds_addr(s_lds) + part * C::PART + r16 * ROW + ((FM::piece(s, kg) ^ r16) << 4);
    const uint32_t d_ad = lds_addr(s_lds) + part * C::PART + C::ACT + 16 * kg;
    // base-3: per half h of a block, the window's first byte as (dword q,
    // byte shift) within the lane's 3 dwords, and its first digit o
    uint32_t tq_q[2], tq_sh[2], tq_o[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const int k0 = 32 * kg + 16 * h;
        const int r = k0 / 5 - (kg == 0 ? 0 : kg == 1 ? 4 : kg == 2 ? 12 : 16);
        tq_q[h] = (uint32_t)(r >> 2);
        tq_sh[h] = (uint32_t)(r & 3);
        tq_o[h] = (uint32_t)(k0 % 5);
    }
    const uint32_t lut_ad = lds_addr(lut);
    // Q4_K min-term operands of m-tile t: part kg (hi, lo) of token 16t + r16
    // for kg < 2, zeros above (slot offsets apply to real operands only)
    const uint32_t l_ad = kg < 2 ? lds_addr(s_lds) + part * C::PART + C::ALO + kg * (TM * 16) + 16 * r16
                                 : lds_addr(zero) + 16 * r16;
    const uint32_t l_slot = kg < 2 ? 1u : 0u;

    auto compute = [&](const WRaw<F> &R, uint32_t so, int ch) __attribute__((always_inline)) {
        // LDS reads: the scales first, then K-step s (one per m-tile), two
        // K-steps in flight
        v4f da[NBLK][MT];
        v4i ap[MT];
        v4i av[2][MT];
        auto rd = [&](int s, v4i(&dst)[MT]) __attribute__((always_inline)) {
#pragma unroll
            for (int t = 0; t < MT; ++t) {
                switch (t) {
                    case 0: dst[t] = lds_read16<0>(a_ad[s] + so); break;
                    case 1: dst[t] = lds_read16<16 * ROW>(a_ad[s] + so); break;
                    case 2: dst[t] = lds_read16<32 * ROW>(a_ad[s] + so); break;
                    default: dst[t] = lds_read16<48 * ROW>(a_ad[s] + so); break;
                }
            }
        };
        __builtin_amdgcn_s_setprio(1);
#pragma unroll
        for (int bb = 0; bb < NBLK; ++bb)
#pragma unroll
            for (int t = 0; t < MT; ++t)
                da[bb][t] = __builtin_bit_cast(v4f, lds_read16<0>(d_ad + so + 256 * bb + 64 * t));
        if constexpr (F == F_Q4K) {
#pragma unroll
            for (int t = 0; t < MT; ++t) {
                switch (t) {
                    case 0: ap[t] = lds_read16<0>(l_ad + l_slot * so); break;
                    case 1: ap[t] = lds_read16<256>(l_ad + l_slot * so); break;
                    case 2: ap[t] = lds_read16<512>(l_ad + l_slot * so); break;
                    default: ap[t] = lds_read16<768>(l_ad + l_slot * so); break;
                }
            }
        }
        // base-3: the trits of all four K-steps through the decode table,
        // waited for before the values are read
        v4i tq_b[4];
        if constexpr (F == F_TQ) {
            v2u e[4][4];
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                const int bb = s >> 1, h = s & 1;
                const uint32_t w0 = R.w01[bb][0], w1 = R.w01[bb][1], w2 = R.w2[bb];
                const uint32_t x = __builtin_amdgcn_alignbyte(tq_q[h] ? w2 : w1, tq_q[h] ? w1 : w0, tq_sh[h]);
#pragma unroll
                for (int i = 0; i < 4; ++i) e[s][i] = lds_read8<0>(lut_ad + 8u * ((x >> (8 * i)) & 0xFFu));
            }
#pragma unroll
            for (int s = 0; s < 4; ++s)
#pragma unroll
                for (int i = 0; i < 4; ++i) lds_wait_n(15 - 4 * s - i, e[s][i]);
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                // 20 trits in order: D0 = t0..3, D1 = t4..7, ..., D4 = t16..19
                uint32_t D[5];
                D[0] = e[s][0].x;
                D[1] = perm_b32(e[s][1].x, e[s][0].y, 0x06050400u);
                D[2] = __builtin_amdgcn_alignbyte(e[s][1].y, e[s][1].x, 3) | (e[s][2].x << 16);
                D[3] = __builtin_amdgcn_alignbyte(e[s][2].y, e[s][2].x, 2) | (e[s][3].x << 24);
                D[4] = __builtin_amdgcn_alignbyte(e[s][3].y, e[s][3].x, 1);
                // the 16 from digit o on (o = 4: one dword on)
                const uint32_t o = tq_o[s & 1];
                const bool o4 = o >= 4;
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const uint32_t lo = o4 ? D[j + 1] : D[j];
                    const uint32_t hi = o4 ? D[j + 2 < 5 ? j + 2 : 4] : D[j + 1];
                    tq_b[s][j] = (int)__builtin_amdgcn_alignbyte(hi, lo, o & 3u);
                }
            }
        }
        rd(0, av[0]);
        rd(1, av[1]);
        const uint32_t b = w_row + (uint32_t)(ch * FM::CB);  // chunk start
        // ---- the chunk's weights, aligned, and the digits of K-step s
        float dw[NBLK];
        uint32_t q4x = 0;                            // Q4_K: this lane's scale fields
        float ndmin = 0.0f;
        v8bf bm;
        uint32_t q6l[17], q6h[8], q6s = 0, sh = 0;  // Q6_K
        uint32_t t2w[2][4];                          // two-bit ternary
        if constexpr (F == F_Q4K) {
            // scales of sub-blocks 2kg (K-steps 0, 1) and 2kg + 1 (2, 3):
            // fields 2kg, 2kg+1 of the 96-bit word, bits 12kg ..; mins m_j at
            // bits 48 + 6j
            const uint64_t f64 = (uint64_t)(uint32_t)R.hdr[1] | ((uint64_t)(uint32_t)R.hdr[2] << 32);
            q4x = (uint32_t)(f64 >> (12 * kg));
            dw[0] = f16_bits_to_f32((uint32_t)R.hdr[0]);
            ndmin = -f16_bits_to_f32((uint32_t)R.hdr[0] >> 16);
            const uint64_t mx = ((uint64_t)(uint32_t)R.hdr[2] | ((uint64_t)(uint32_t)R.hdr[3] << 32)) >> 16;
#pragma unroll
            for (int i = 0; i < 8; ++i) bm[i] = (__bf16)(float)(uint32_t)((mx >> (6 * i)) & 63u);
        } else if constexpr (F == F_Q6K) {
            // the block's offset past the aligned dword (0 or 2 bytes)
            sh = 8u * (b & 3u);
            const uint32_t l[17] = {(uint32_t)R.l0[0], (uint32_t)R.l0[1], (uint32_t)R.l0[2], (uint32_t)R.l0[3],
                                    (uint32_t)R.l1[0], (uint32_t)R.l1[1], (uint32_t)R.l1[2], (uint32_t)R.l1[3],
                                    (uint32_t)R.l2[0], (uint32_t)R.l2[1], (uint32_t)R.l2[2], (uint32_t)R.l2[3],
                                    (uint32_t)R.l3[0], (uint32_t)R.l3[1], (uint32_t)R.l3[2], (uint32_t)R.l3[3],
                                    R.l4};
            const uint32_t h[9] = {(uint32_t)R.h0[0], (uint32_t)R.h0[1], (uint32_t)R.h0[2], (uint32_t)R.h0[3],
                                   (uint32_t)R.h1[0], (uint32_t)R.h1[1], (uint32_t)R.h1[2], (uint32_t)R.h1[3],
                                   R.h2};
#pragma unroll
            for (int e = 0; e < 17; ++e) q6l[e] = l[e];
#pragma unroll
            for (int e = 0; e < 8; ++e) q6h[e] = __builtin_amdgcn_alignbit(h[e + 1], h[e], sh);
            q6s = __builtin_amdgcn_alignbit(R.sc[1], R.sc[0], sh);
            dw[0] = f16_bits_to_f32(R.dd);
        } else if constexpr (F == F_TQ) {
#pragma unroll
            for (int bb = 0; bb < 2; ++bb) dw[bb] = f16_bits_to_f32(R.dd[bb]);
        } else {
#pragma unroll
            for (int bb = 0; bb < 2; ++bb) {
                const uint32_t s2 = 8u * ((b + 34u * bb) & 3u);  // (16(kg % 2) keeps the phase)
                const uint32_t c[5] = {(uint32_t)R.c[bb][0], (uint32_t)R.c[bb][1], (uint32_t)R.c[bb][2],
                                       (uint32_t)R.c[bb][3], R.c4[bb]};
#pragma unroll
                for (int e = 0; e < 4; ++e) t2w[bb][e] = __builtin_amdgcn_alignbit(c[e + 1], c[e], s2);
                dw[bb] = f16_bits_to_f32(R.dd[bb]);
            }
        }
        auto digits = [&](int s, v4i(&dg)[NDIG]) __attribute__((always_inline)) {
            if constexpr (F == F_Q4K) {
                // the low (s < 2) or high nibbles of bytes 32kg + 16(s % 2) + i
                const uint32_t sc = (s < 2 ? q4x : q4x >> 6) & 63u;
                const v4i qw = (s & 1) ? R.q1 : R.q0;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const uint32_t nib = s < 2 ? (uint32_t)qw[e] & 0x0F0F0F0Fu : ((uint32_t)qw[e] >> 4) & 0x0F0F0F0Fu;
                    uint32_t dh, dl;
                    q4k_digits(nib, sc, dh, dl);
                    dg[0][e] = (int)dh;
                    dg[NDIG - 1][e] = (int)dl;
                }
            } else if constexpr (F == F_Q6K) {
                const uint32_t nib_sh = 4u * (uint32_t)(kg & 1);
                const int sc = (int)(int8_t)(uint8_t)(q6s >> (8 * s));
                const uint32_t hsh = nib_sh + 2u * (uint32_t)(s >> 1);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const uint32_t l4 =
                        (__builtin_amdgcn_alignbit(q6l[4 * s + e + 1], q6l[4 * s + e], sh) >> nib_sh) & 0x0F0F0F0Fu;
                    const uint32_t h2 = (q6h[4 * (s & 1) + e] >> hsh) & 0x03030303u;
                    uint32_t dh, dl;
                    q6k_digits(l4 | (h2 << 4), sc, dh, dl);
                    dg[0][e] = (int)dh;
                    dg[NDIG - 1][e] = (int)dl;
                }
            } else if constexpr (F == F_TQ) {
#pragma unroll
                for (int e = 0; e < 4; ++e) dg[0][e] = tq_b[s][e];
            } else {
                // code c = t + 1 in plane 2(s % 2) + kg/2; t bytewise without
                // borrows: (c | 0x80) - 1, bit 7 flipped back
                const uint32_t psh = 2u * (uint32_t)(2 * (s & 1) + (kg >> 1));
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const uint32_t code = (t2w[s >> 1][e] >> psh) & 0x03030303u;
                    dg[0][e] = (int)(((code | 0x80808080u) - 0x01010101u) ^ 0x80808080u);
                }
            }
        };
        v4i acc[NDIG][MT];
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            v4i dg[NDIG];
            digits(s, dg);
            // reads in flight behind m-tile t of K-step s: the rest of this
            // K-step's, then the next K-step's (none after K-step 3)
            v4i(&cur)[MT] = av[s & 1];
#pragma unroll
            for (int t = 0; t < MT; ++t) lds_wait_n(MT - 1 - t + (s < 3 ? MT : 0), cur[t]);
            const bool first = s % KSB == 0;
#pragma unroll
            for (int t = 0; t < MT; ++t)
#pragma unroll
                for (int d = 0; d < NDIG; ++d) acc[d][t] = mma16_i8(cur[t], dg[d], first ? v4i{} : acc[d][t]);
            if (s < 2) rd(s + 2, av[s & 1]);
            if (s % KSB == KSB - 1) {
                // fold of block bb: out += d_a[m] * d[n] * T, T = 64 acc_h +
                // acc_l (Q6_K) or acc (ternary); Q4_K: out += d_a[m] * (d[n] *
                // (8 acc_h + acc_l) - dmin[n] * sum_j m_j B_j), the min term on
                // one bf16 MFMA per m-tile (A row m = both exact parts of B_j
                // in k-groups 0 and 1, zeros in 2 and 3; B column n = the
                // mins).  Its operands were read before every K-step's values,
                // all of which are in by K-step 1's wait but the last two
                // K-steps' (2 MT)
                const int bb = s / KSB;
#pragma unroll
                for (int t = 0; t < MT; ++t) {
                    lds_wait_n(s < 3 ? 2 * MT : 0, da[bb][t]);
                    if constexpr (F == F_Q4K) {
                        lds_wait_n(0, ap[t]);
                        const v4f mt = mma16_bf16(__builtin_bit_cast(v8bf, ap[t]), bm, v4f{});
#pragma unroll
                        for (int i = 0; i < 4; ++i) {
                            const int Tq = (acc[0][t][i] << FM::SHIFT) + acc[1][t][i];
                            out[t][i] = fmaf(fmaf((float)Tq, dw[0], mt[i] * ndmin), da[0][t][i], out[t][i]);
                        }
                    } else {
#pragma unroll
                        for (int i = 0; i < 4; ++i) {
                            const int Tq = NDIG == 2 ? (acc[0][t][i] << FM::SHIFT) + acc[NDIG - 1][t][i] : acc[0][t][i];
                            out[t][i] = fmaf((float)Tq * dw[bb], da[bb][t][i], out[t][i]);
                        }
                    }
                }
            }
        }
        __builtin_amdgcn_s_setprio(0);
    };

    // step x: the copies and loads of step x + L go out once every wave is
    // past step x - 1 (their slot's last reader), then step x multiplies
    auto step = [&](auto KK, int x) __attribute__((always_inline)) {
        constexpr int k = decltype(KK)::value;
        __builtin_amdgcn_sched_barrier(0);
        wait_vmcnt<C::LOADS * (C::L - 1)>();
        barrier_nofence();
        copies(x + C::L);
        wload(x + C::L, ring[(k + C::L) % C::S]);
        __builtin_amdgcn_sched_barrier(0);
        const int ch = part * T + x;
        if (x < T && ch < nch) compute(ring[k], (uint32_t)(k * C::SLOT), ch);  // uniform
    };
#pragma unroll
    for (int x = 0; x < C::L; ++x) {
        copies(x);
        wload(x, ring[x]);
    }
    // whole ring turns, then the T mod S steps left over, which issue
    // nothing: in tail step j the loads of steps x .. nfull - 1 + L are
    // outstanding, L - j steps' worth, and step x's are the oldest
    const int nfull = T / C::S * C::S;
    for (int x0 = 0; x0 < nfull; x0 += C::S)
        static_for<0, C::S>([&](auto KK) KQ_INLINE { step(KK, x0 + decltype(KK)::value); });
    auto tail_step = [&](auto JJ) KQ_INLINE {
        constexpr int j = decltype(JJ)::value;
        __builtin_amdgcn_sched_barrier(0);
        wait_vmcnt<C::LOADS * (C::L - 1 - j)>();
        barrier_nofence();
        __builtin_amdgcn_sched_barrier(0);
        const int ch = part * T + nfull + j;
        if (ch < nch) compute(ring[j], (uint32_t)(j * C::SLOT), ch);  // uniform
    };
    const int rem = T - nfull;
    static_for<1, C::S>([&](auto RR) KQ_INLINE {
        if (rem == decltype(RR)::value) static_for<0, decltype(RR)::value>(tail_step);
    });
    // the copies and loads past the end (reading nothing) drain; then the
    // other parts' sums go through LDS to part 0's waves, added in part order
    wait_vmcnt<0>();
    barrier_nofence();
    float *red = reinterpret_cast<float *>(s_lds);
    if (part > 0) {
#pragma unroll
        for (int t = 0; t < MT; ++t)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                red[((((part - 1) * NS + strip) * MT + t) * 4 + i) * 64 + lane] = out[t][i];
    }
    barrier_nofence();
    if (part == 0) {
        // rows past M fall outside the resource; columns past N are sent out
        // of range
        const int n = n0 + r16;
        const int voff = n < N ? (4 * kg * N + n) * 4 : OOB_VOFF;
#pragma unroll
        for (int t = 0; t < MT; ++t) {
            v4f sum = out[t];
#pragma unroll
            for (int p = 1; p < KP; ++p)
#pragma unroll
                for (int i = 0; i < 4; ++i) sum[i] += red[((((p - 1) * NS + strip) * MT + t) * 4 + i) * 64 + lane];
            const v4i bits = __builtin_bit_cast(v4i, sum);
#pragma unroll
            for (int i = 0; i < 4; ++i)
                __builtin_amdgcn_raw_buffer_store_b32(bits[i], rs_o, voff, (16 * t + i) * N * 4, 0);
        }
    }
}

}  // namespace rk

// K-parts: one workgroup runs per CU at a time, each costing a fixed part
// (filling the rings, the reduction: about 4.5 us) plus its waves' share of
// K (about 0.0085-0.010 us per K value at 16-64 tokens), so the time goes as
// rounds * (512 + K / parts) in units of K, the workgroups of every 64-token
// slice counted.  The fewest parts among the best, within what the token
// tile's LDS allows (64 rows: at most four).  Measured (Q6_K) at 16 tokens,
// K = 4096, us for 2 / 4 / 8 parts: 4096 rows 21.4 / 14.1 / 9.3; 8192 rows
// 22.0 / 14.9 / 17.1; 11008 rows 22.4 / 27.0 / 24.5; 14336 rows 23.0 / 27.5 /
// 31.8; 28672 rows 44.2 / 53.1 / 55.4.
static int64_t ring_plan(int M, int N, int K, int *parts) {
    const int cus = num_cus();
    const int kmax = M > 32 ? 4 : 8;
    const int64_t slices = M > 64 ? (M + 63) / 64 : 1;
    int best = 2;
    int64_t best_cost = 0;
    for (int kp = 2; kp <= kmax; kp *= 2) {
        const int64_t wgs = ((int64_t)N + 16 * (8 / kp) - 1) / (16 * (8 / kp)) * slices;
        const int64_t cost = (wgs + cus - 1) / cus * (512 + K / kp);
        if (kp == 2 || cost < best_cost) {
            best = kp;
            best_cost = cost;
        }
    }
    *parts = best;
    return best_cost;
}

int ring_parts(int M, int N, int K) {
    int kp;
    ring_plan(M, N, K, &kp);
    return kp;
}

// Past 64 tokens the ring kernel runs one 64-token slice per grid row, each
// reading the whole weight matrix again (from L2 and the last-level cache
// when the slices run together).  It pays where the 128 x 128 tile kernels
// leave most CUs idle: narrow weights with a long K.  The tile kernels' time
// goes as rounds * K, their rounds counted in 128 x 128 tiles; the two
// models are weighed with the ratio of their fitted costs per unit (ring /
// tile: Q4_K 6/5, Q6_K 19/20, base-3 5/6, two-bit 4/5).  Paired runs, us,
// tile / ring: Q6_K 4096 x 14336 at 65 tokens 142 / 44, 128 144 / 45.5, 256
// 143 / 77, 384 143 / 124, 512 144 / 143, 1024 172 / 291; 4096 x 4096 at
// 128 45 / 15.8, 256 45 / 25, 512 45.6 / 45.6; 14336 x 4096 at 128 46.8 /
// 46.9, 256 51 / 90.  Base-3 4096 x 14336 at 128 / 256 / 512 tokens 111 /
// 31, 111 / 49, 112 / 91; 17408 x 5120 at 128 44 / 55.  Two-bit 4096 x
// 14336 101 / 33, 101 / 48, 102 / 86.5; 17408 x 5120 at 128 40 / 52.  Q4_K
// 4096 x 14336 at 65 / 128 / 256 / 512 tokens 71 / 31, 77 / 33, 77 / 50, 79
// / 93; 4096 x 4096 at 128 24 / 11.6, 256 24 / 16.8; 14336 x 4096 at 128 26
// / 31.
bool ring_slices_pay(int fmt, int M, int N, int K) {
    if (M <= 64 || M > 512) return false;
    const int cus = num_cus();
    const int64_t tiles = (int64_t)((M + 127) / 128) * (((int64_t)N + 127) / 128);
    // Q4_K's tile kernels take K whole; the others' split it where it pays
    const int64_t tile_cost = fmt == rk::F_Q4K ? (tiles + cus - 1) / cus * K : tile_units(fmt, M, N, K);
    int kp;
    const int64_t ring_units = ring_plan(M, N, K, &kp);
    int num = 4, den = 5;  // two-bit ternary
    if (fmt == rk::F_Q4K) num = 6, den = 5;
    else if (fmt == rk::F_Q6K) num = 19, den = 20;
    else if (fmt == rk::F_TQ) num = 5, den = 6;
    return ring_units * num < tile_cost * den;
}

// Shapes this kernel takes: Q6_K and ternary past the matrix-vector kernels,
// up to 64 tokens, and in 64-token slices where that pays; K a multiple of
// 256 (Q4_K comes through its own choice).
bool ring_choice(int fmt, int M, int N, int K) {
    if (fmt != rk::F_Q6K && fmt != rk::F_TQ && fmt != rk::F_TQ2) return false;
    if (M < 1 || N < 1 || K < 256 || K % 256 != 0) return false;
    if (M > 64) return ring_slices_pay(fmt, M, N, K);
    return !gemv_choice(fmt, M, N, K);
}

template <int F, int TM, int KP, int NW = 8>
static void launch_rk(const rk::Args &a, hipStream_t stream) {
    constexpr int R = rk::Cfg<F, TM, KP, NW>::ROWS;
    hipLaunchKernelGGL((rk::gemm_ring_kernel<F, TM, KP, NW>),
                       dim3((unsigned)((a.N + R - 1) / R), (unsigned)((a.M + TM - 1) / TM)), dim3(64 * NW), 0,
                       stream, a);
}

// Four-wave workgroups (one strip per K-part) for 64-row token tiles in four
// K-parts where the eight-wave ones would leave CUs idle and the four-wave
// ones take one round: twice the workgroups, each CU one of them.
static bool ring_four_waves(int M, int N, int kp) {
    if (M <= 32 || kp != 4) return false;
    const int64_t slices = M > 64 ? (M + 63) / 64 : 1;
    const int64_t wgs8 = ((int64_t)N + 31) / 32 * slices, wgs4 = ((int64_t)N + 15) / 16 * slices;
    const int cus = num_cus();
    return wgs8 < cus && wgs4 <= cus;
}

template <int F>
static void launch_rk_fmt(const rk::Args &a, int kp, hipStream_t stream) {
    if (a.M <= 16) {
        if (kp == 2) launch_rk<F, 16, 2>(a, stream);
        else if (kp == 4) launch_rk<F, 16, 4>(a, stream);
        else launch_rk<F, 16, 8>(a, stream);
    } else if (a.M <= 32) {
        if (kp == 2) launch_rk<F, 32, 2>(a, stream);
        else if (kp == 4) launch_rk<F, 32, 4>(a, stream);
        else launch_rk<F, 32, 8>(a, stream);
    } else {
        if (kp == 2) launch_rk<F, 64, 2>(a, stream);
        else if (ring_four_waves(a.M, a.N, kp)) launch_rk<F, 64, 4, 4>(a, stream);
        else launch_rk<F, 64, 4>(a, stream);
    }
}

hipError_t launch_gemm_ring(int fmt, const void *W, const int8_t *qs, const float *da, const uint16_t *alpha,
                            float *out, int M, int N, int K, hipStream_t stream) {
    rk::Args a;
    a.W = static_cast<const uint8_t *>(W);
    a.qs = qs;
    a.da = da;
    a.alpha = alpha;
    a.out = out;
    a.M = M;
    a.N = N;
    a.K = K;
    a.nch = K / 256;
    const int kp = ring_parts(M, N, K);
    if (fmt == rk::F_Q4K) launch_rk_fmt<rk::F_Q4K>(a, kp, stream);
    else if (fmt == rk::F_Q6K) launch_rk_fmt<rk::F_Q6K>(a, kp, stream);
    else if (fmt == rk::F_TQ) launch_rk_fmt<rk::F_TQ>(a, kp, stream);
    else launch_rk_fmt<rk::F_TQ2>(a, kp, stream);
    return hipGetLastError();
}

}  // namespace kq
