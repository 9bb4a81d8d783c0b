// kq_gemm_q4k.hip -- Q4_K x Q8_K GEMM on gfx950 int8 MFMA, weights unpacked
// straight into matrix-core operand registers.
//
// out[m][n] = sum_sb d_a[m,sb] * ( d[n,sb] * sum_k sc_j q_k a_k
//                                  - dmin[n,sb] * sum_j m_j * B_j[m,sb] )
// where B_j is the sum of the 32 quantized activations of sub-block j
// (the Q4_K dequantization w = d*sc_j*q - dmin*m_j, multiplied out).
//
// Work split (prior art: the BigTile kernel of vllm.cpp PR 3036 and
// llama.cpp's mul_mat_q share one staged activation tile among all warps of
// a block; here the weight side is not staged at all):
//   * A workgroup of 4 waves (one per SIMD) computes 128 x 128 output tiles,
//     persistently: the grid is two workgroups per CU and each walks a list
//     of tiles with one flat (tile, superblock) loop, so prefetching runs
//     across tile boundaries.
//   * Wave w owns 32 weight rows (output columns) and all 128 activation
//     rows.  Every weight is fetched and unpacked once per tile, by the wave
//     that multiplies it, directly into v_mfma_i32_32x32x32_i8 operand
//     registers (loaded one superblock ahead): no LDS round trip for weights.
//   * Each 256-wide superblock of activations (values, scales, min-term
//     operands) is copied global -> LDS by the buffer unit (no registers)
//     one superblock ahead, into the other of two slots; rows are 256 bytes
//     with 16-byte pieces XOR-swizzled by the row, which keeps fragment reads
//     conflict-free.
//   * The 6-bit sub-block scale rides in the int8 operand as two digits,
//     sc = 8*sh + sl with sh, sl in [0,7]:
//         sc*q = 8*(sh*q) + (sl*q),   sh*q, sl*q <= 105.
//     Pass 1 accumulates the sh digits over the whole superblock, the int32
//     sums are shifted left by 3, pass 2 adds the sl digits; the fp32 fold
//     then runs once per superblock and output.
//   * The min term is a rank-8 product per superblock, computed exactly:
//     M = sum_j m_j * B_j, with B_j the sum of a sub-block's 32 quantized
//     activations.  The quantizer stores B_j as two parts bf16 holds exactly
//     (the alpha section), so one bf16 MFMA against the 6-bit mins gives M
//     with every product and partial sum an integer below 2^24.  The fold is
//     then out += d_a * (d * T - dmin * M) in fp32, T the integer superblock
//     sum of sc*q*a.
//   * Reads past the last activation row or weight row return zero and
//     stores past the last output row are dropped (buffer resources over the
//     whole tensors); columns past N are sent out of range.
//   * The same kernel is built with 64-row tiles (two m-tiles per wave) for
//     shapes whose 128-row tiling would leave CUs idle, and, at that height,
//     in a gather mode for the expert-indexed product: a tile holds routed
//     rows of one expert, the copies take per-lane offsets of the gathered
//     token rows, and the weight and output resources are set per tile.
//
// MFMA operand convention (v_mfma_i32_32x32x32_i8, v_mfma_f32_32x32x16_bf16):
// lane l supplies row (l % 32) of A and column (l % 32) of B with k-group
// l / 32; the contraction sums over every (k-group, element) pair, so any K
// order works as long as both operands use the same one.  The 32x32 result
// is 16 registers per lane: register r of lane l holds row
// 8*(r/4) + 4*(l/32) + r%4, column l % 32.
#include "kq_device.hpp"
#include "kq_hooks.hpp"
#include "kq_launch.hpp"
#include "kq_tile.hpp"

#include <atomic>
#include <type_traits>

namespace kq {
namespace q4w {
using namespace tl;

constexpr int BN = 128, NWAVE = 4, NT = 64 * NWAVE;
constexpr int ROW = 256;              // LDS bytes per staged activation row
constexpr int BB = 144;               // Q4_K block bytes
// Tile heights: 128 rows (four 32-row m-tiles per wave), or 64 rows for
// shapes whose 128-row tiles would leave CUs idle.
template <int BM>
struct TileCfg {
    static constexpr int MT = BM / 32;                   // 32-row m-tiles per wave
    static constexpr int ABUF = BM * ROW;                // staged activation values of one superblock
    static constexpr int DBUF = 2 * BM > 256 ? 2 * BM : 256;  // staged scales (a 1 KiB copy lands here)
    static constexpr int LBUF = 2 * BM * 16;             // staged min-term operands (hi, lo)
    static constexpr int WG_PER_CU = 2;                   // workgroups sharing a CU
};
struct Args {
    const uint8_t *W;
    const int8_t *qs;
    const float *da;         // [nsb][M]
    const uint16_t *alpha;   // [nsb][2][M][8] bf16: exact parts of the sub-block sums B_j
    float *out;
    int M, N, K, nsb, tiles_m, tiles_n, ntiles;
    // expert-indexed product only: out has n_routed rows, routed row r
    // multiplies token rows[r] by the weights of the expert e with
    // exp_off[e] <= r < exp_off[e+1] (at W + e * expert_bytes); tiles_m is an
    // upper bound, the kernel counts the real M-tiles
    const int32_t *exp_off, *rows;
    int n_experts, n_routed;
    int64_t expert_bytes;
};

// four nibble bytes times a scale digit s < 8, bytewise (products < 128)
__device__ __forceinline__ int mul_digit(uint32_t nib4, uint32_t s) {
    v2u16 x = __builtin_bit_cast(v2u16, nib4);
    const unsigned short s16 = (unsigned short)s;
    return (int)__builtin_bit_cast(uint32_t, (v2u16)(x * (v2u16){s16, s16}));
}
// Tile t of the grouped order: GM M-tiles down, then across N.
// Expert-indexed tiles also carry the expert e, the first routed row grb
// and the number of routed rows mrows (0..BM) the tile holds.
struct TileXY {
    int m0, n0, e, grb, mrows;
};
// rows routed to expert x (clamped: routing that breaks its contract gives
// wrong values, never an access outside the buffers)
__device__ __forceinline__ int expert_rows(const Args &a, int x) {
    const int64_t c = (int64_t)a.exp_off[x + 1] - a.exp_off[x];
    return (int)min(max(c, (int64_t)0), (int64_t)a.n_routed);
}
template <int BM, bool GATHER>
__device__ __forceinline__ TileXY tile_xy(const Args &a, int tiles_m, int t) {
    constexpr int GM = 4;
    const int per_group = GM * a.tiles_n;
    const int first_m = (t / per_group) * GM;
    // (at least 1: the look-ahead tile of a workgroup's last tile may lie
    // past the list; its coordinates are then never used)
    const int gsize = max(min(tiles_m - first_m, GM), 1);
    const int r = t % per_group;
    const int tm = first_m + r % gsize, n0 = (r / gsize) * BN;
    if constexpr (!GATHER) {
        return {tm * BM, n0, 0, 0, 0};
    } else {
        // M-tile tm is tile mt of expert e, counting each expert's
        // ceil(rows / BM) tiles in expert order
        int e = 0, mt = 0, acc = 0;
        bool found = false;
        for (int x = 0; x < a.n_experts; ++x) {
            const int te = (expert_rows(a, x) + BM - 1) / BM;
            if (tm < acc + te) {
                e = x;
                mt = tm - acc;
                found = true;
                break;
            }
            acc += te;
        }
        int grb = a.exp_off[e] + mt * BM;
        int mrows = 0;
        if (found && grb >= 0 && grb < a.n_routed)
            mrows = min(min(a.exp_off[e + 1], a.n_routed) - grb, BM);
        if (mrows <= 0) {
            mrows = 0;
            grb = 0;
        }
        return {0, n0, e, grb, mrows};
    }
}

// One staging slot: distinct LDS arrays per slot, so the compiler can tell
// the copies into one slot from the reads of the other.
struct Slot {
    int8_t *a;      // [BM rows][256]: 16-byte piece p of row r at ((p ^ (r % 16)) * 16)
    float *d;       // [BM] activation scales
    int8_t *l;      // [2][BM][16]: min-term operands, hi then lo
};

// This lane's raw weight block: header and its 64 nibble bytes.
struct WRaw {
    v4i hdr, q[4];
};

// KS = 2: one workgroup of 8 waves per CU instead of two of 4.  Waves 4h ..
// 4h+3 (half h) take superblock 2i+h of superblock pair i, each half its own
// region of the staging slot; at the end of a tile half 1 hands its sums to
// half 0 through LDS.  A CU then owns whole tiles at twice the rate, so the
// tile count balances over CUs rather than over twice as many workgroups.
template <int BM, bool GATHER = false, int KS = 1>
__global__ __launch_bounds__(NT * KS, KS == 1 ? TileCfg<BM>::WG_PER_CU : 1) void gemm_q4k_kernel(Args a) {
    static_assert(!GATHER || (BM == 64 && KS == 1), "gather mode stages one routed row per lane");
    static_assert(KS == 1 || KS == 2, "one or two superblocks per step");
    using TC = TileCfg<BM>;
    constexpr int MT = TC::MT;
    // a slot holds KS superblocks, half h's at offset h * (ABUF, DBUF, LBUF)
    __shared__ __attribute__((aligned(16))) int8_t s_a0[KS * TC::ABUF], s_a1[KS * TC::ABUF];
    __shared__ __attribute__((aligned(16))) float s_d0[KS * TC::DBUF], s_d1[KS * TC::DBUF];
    __shared__ __attribute__((aligned(16))) int8_t s_l0[KS * TC::LBUF], s_l1[KS * TC::LBUF];
    const Slot slots[2] = {{s_a0, s_d0, s_l0}, {s_a1, s_d1, s_l1}};

    const int tid = threadIdx.x, lane = tid & 63;
    // weight strip of this wave (its 32 output columns) and its half
    const int wave = __builtin_amdgcn_readfirstlane((tid >> 6) & (NWAVE - 1));
    const int half = KS == 1 ? 0 : __builtin_amdgcn_readfirstlane(tid >> 8);
    const int ln = lane & 31, g = lane >> 5;
    const int M = a.M, N = a.N, K = a.K, nsb = a.nsb;
    const int npair = (nsb + KS - 1) / KS;  // steps per tile

    // ---- persistent tile list ----------------------------------------------
    // Workgroups are dealt round-robin to the 8 XCDs.  At step k the grid
    // covers grouped-order tiles [k*G, (k+1)*G); the workgroups of one XCD
    // take a contiguous run of them, so they share activation and weight
    // rows in that XCD's L2.
    const int G = gridDim.x, b = blockIdx.x;
    const int per_xcd = G >> 3;
    const int slot_in_step = (per_xcd > 0 && b < 8 * per_xcd) ? ((b & 7) * per_xcd + (b >> 3)) : b;
    int tiles_m = a.tiles_m;
    if constexpr (GATHER) {
        int acc = 0;
        for (int x = 0; x < a.n_experts; ++x) acc += (expert_rows(a, x) + BM - 1) / BM;
        tiles_m = min(acc, a.tiles_m);
    }
    const int ntiles = tiles_m * a.tiles_n;
    const int my_tiles = (ntiles - slot_in_step + G - 1) / G;    // tiles slot, slot+G, ...
    const int total = my_tiles * npair;                          // flat iterations
    const int rowbytes = nsb * BB;
    if (total <= 0) return;  // uniform: no barrier is ever reached

    // Buffer resources over whole tensors (built once): reads past the last
    // activation or weight row return zero and stores past the last output
    // row are dropped.  Every offset below stays under 2^31 (checked on the
    // host).
    const auto rs_a = __builtin_amdgcn_make_buffer_rsrc((void *)a.qs, (short)0, M * K, RSRC_FLAGS);
    const auto rs_d = __builtin_amdgcn_make_buffer_rsrc((void *)a.da, (short)0, nsb * M * 4, RSRC_FLAGS);
    const auto rs_l = __builtin_amdgcn_make_buffer_rsrc((void *)a.alpha, (short)0, nsb * 2 * M * 16, RSRC_FLAGS);
    const auto rs_w = __builtin_amdgcn_make_buffer_rsrc((void *)a.W, (short)0, N * rowbytes, RSRC_FLAGS);
    const auto rs_o = __builtin_amdgcn_make_buffer_rsrc((void *)a.out, (short)0, M * N * 4, RSRC_FLAGS);
    // expert-indexed: the weights of the tile's expert, and its output rows
    // (the range ends at the tile's last routed row, so stores past it drop)
    auto rs_w_of = [&](const TileXY &T) {
        if constexpr (!GATHER) return rs_w;
        else
            return __builtin_amdgcn_make_buffer_rsrc((void *)(a.W + (int64_t)T.e * a.expert_bytes), (short)0,
                                                     N * rowbytes, RSRC_FLAGS);
    };
    auto rs_o_of = [&](const TileXY &T) {
        if constexpr (!GATHER) return rs_o;
        else
            return __builtin_amdgcn_make_buffer_rsrc((void *)(a.out + (int64_t)T.grb * N), (short)0,
                                                     T.mrows * N * 4, RSRC_FLAGS);
    };

    // ---- staging of one superblock of activations: buffer -> LDS copies ----
    // Values: 1 KiB copy c holds rows 4c..4c+3; lane l fills position l%16 of
    // row 4c + l/16 with piece (l%16) ^ (row%16).  Wave w copies c = 8w..8w+7.
    // Each wave also copies a quarter of the min-term operands (1 KiB: part
    // w/2, rows 64*(w%2)..), and wave 0 the scales (one 1 KiB copy).
    const int st_row = lane >> 4, st_pos = lane & 15;
    // copy i covers rows (BM/4)w + 4(i%4) + 16(i/4) + l/16: its piece index
    // is (l%16) ^ (4(i%4) + l/16), i.e. base ^ (64*(i%4)) in bytes (K is a
    // multiple of 256, so the XOR stays inside the row), and copies i, i+4 are
    // 16 rows (16*K bytes) apart
    constexpr int CPW = BM / 16;  // value copies per wave
    const int a_vbase = ((BM / 4) * wave + st_row) * K + 16 * (st_pos ^ st_row);
    const int l_voff = 16 * lane + (BM == 128 ? (wave & 1) * 1024 : 0);  // 16 * lane for wave 0
    // Expert-indexed: the same copies with per-lane offsets of gathered token
    // rows: ga[i] for value copy i (row 16w + 4i + l/16, piece as above), gd
    // = 4 * token of tile row l (scales: one 4-byte copy per row; min-term
    // operands: 16 bytes per row).  Rows past the tile's last routed row
    // repeat it; indices are clamped into rows[] and the activation buffer.
    struct GOff {
        int ga[CPW], gd;
    };
    auto token = [&](const TileXY &T, int r) {
        const int idx = min(max(T.grb + min(r, T.mrows - 1), 0), a.n_routed - 1);
        return min(max(a.rows[idx], 0), M - 1);
    };
    auto goffs = [&](const TileXY &T, GOff &o) {
        if constexpr (GATHER) {
#pragma unroll
            for (int i = 0; i < CPW; ++i)
                o.ga[i] = token(T, (BM / 4) * wave + 4 * i + st_row) * K + 16 * (st_pos ^ (4 * i + st_row));
            o.gd = 4 * token(T, lane);
        }
    };
    auto stage = [&](const Slot &S0, TileXY T, int px, const GOff &o) {
        // this half's superblock of step px, into its region of the slot
        const int sbx = KS * px + half;
        if (KS > 1 && sbx >= nsb) return;  // uniform: an odd superblock count's last step
        const Slot S = KS == 1 ? S0 : Slot{S0.a + half * TC::ABUF, S0.d + half * TC::DBUF, S0.l + half * TC::LBUF};
        if constexpr (GATHER) {
#pragma unroll
            for (int i = 0; i < CPW; ++i) copy16(rs_a, S.a + (CPW * wave + i) * 1024, o.ga[i], sbx * ROW);
            if (wave < 2) copy16(rs_l, S.l + wave * 1024, 4 * o.gd, (sbx * 2 + wave) * M * 16);
            if (wave == 0) copy4(rs_d, S.d, o.gd, sbx * M * 4);
            return;
        }
#pragma unroll
        for (int i = 0; i < CPW; ++i)
            copy16(rs_a, S.a + (CPW * wave + i) * 1024, a_vbase ^ (64 * (i & 3)),
                   (T.m0 + 4 * (i & 3) + 16 * (i >> 2)) * K + sbx * ROW);
        if constexpr (BM == 128) {
            const int c = wave;  // min-term operands: part c/2, rows 64*(c%2) .. +64
            copy16(rs_l, S.l + c * 1024, l_voff, ((sbx * 2 + (c >> 1)) * M + T.m0) * 16);
        } else if (wave < 2) {
            // min-term operands: part w, all 64 rows
            copy16(rs_l, S.l + wave * 1024, l_voff, ((sbx * 2 + wave) * M + T.m0) * 16);
        }
        // scales of rows m0..m0+BM-1 (the rest of the 1 KiB copy fills an
        // unused part of the slot)
        if (wave == 0) copy16(rs_d, S.d, l_voff, (sbx * M + T.m0) * 4);
    };

    // ---- weights of this lane: row n0 + 32*wave + ln, straight to registers --
    // (constant offsets go to the scalar operand: one address register per lane)
    const int w_row = (32 * wave + ln) * rowbytes;
    const int w_nib = w_row + 64 * g;
    auto load_w = [&](TileXY T, int px, WRaw &R) {
        // (past an odd count's last superblock: a repeat of it, unused)
        const int so = T.n0 * rowbytes + (KS == 1 ? px : min(KS * px + half, nsb - 1)) * BB;
        const auto rw = rs_w_of(T);
        R.hdr = ld16(rw, w_row, so);
#pragma unroll
        for (int i = 0; i < 4; ++i) R.q[i] = ld16(rw, w_nib, so + 16 + 16 * i);
    };

    // ---- fragment addressing: row 32t + ln, piece p(g, s) swizzled by row ----
    // k-group g takes nibble bytes [64g, 64g+64) of the block: sub-blocks
    // 4g..4g+3.  K-step s uses the 16 bytes at 64g + 16*(s%4): their low
    // nibbles (s < 4) are weights 128g + 64*((s%4)/2) + 16*(s%2) + i of the
    // superblock, their high nibbles (s >= 4) the same plus 32.
    // p = 8g + c(s) with c < 8, so p ^ (ln % 16) splits into bit 3 (fixed
    // per lane) and bits 0..2: one XOR with a constant per K-step.
    const int frag_base = half * TC::ABUF + ln * ROW + (((8 * g) ^ (ln & 8)) << 4);
    const int d_lane = half * TC::DBUF + 4 * g;          // this half's scales, + 32t + 8q
    const int l_lane = half * TC::LBUF + ln * 16 + 8 * g;  // this half's min-term parts, + 32*16*t
    const int frag_x = (ln & 7) << 4;
    auto frag = [&](int s) {
        const int c = 4 * ((s & 3) >> 1) + (s & 1) + 2 * (s >> 2);
        return frag_base + ((c << 4) ^ frag_x);
    };

    v16i acc[MT];
    v16f out[MT];
#pragma unroll
    for (int t = 0; t < MT; ++t) out[t] = v16f{};

    WRaw wring[2];  // weights of iterations with slot parity 0 / 1

    // ---- one superblock; P = slot parity (compile-time) -----------------------
    // (k, sb): tile index in this workgroup's list and superblock of the
    // current iteration; T = tile k, TN = tile k+1 (computed once per tile)
    int k = 0, sb = 0;
    TileXY T = tile_xy<BM, GATHER>(a, tiles_m, slot_in_step);
    TileXY TN = tile_xy<BM, GATHER>(a, tiles_m, slot_in_step + G);
    GOff oT, oN;  // gathered offsets of tiles T and TN (expert-indexed only)
    goffs(T, oT);
    goffs(TN, oN);

    auto iteration = [&](auto PP, int it) {
        constexpr int P = decltype(PP)::value;
        // (this half's region of the slot: its offsets ride in the per-lane
        // read bases frag_base, d_lane and l_lane)
        const Slot &S = slots[P];
        // everything this wave copied or loaded for iteration it (one
        // iteration ago) has landed; after the barrier, so has every other
        // wave's, and every read of the other slot (iteration it-1) is done.
        wait_vmcnt<0>();
        barrier_nofence();
        const bool more = it + 1 < total;
        const bool last_sb = sb + 1 == npair;  // sb counts steps of KS superblocks
        const bool mine = KS == 1 || KS * sb + half < nsb;  // this half has a superblock this step
        const TileXY Tn = last_sb ? TN : T;
        const int sbn = last_sb ? 0 : sb + 1;
        // the next superblock's activations and weights, a whole iteration
        // ahead of their use
        const WRaw &wc = wring[P];
        __builtin_amdgcn_sched_barrier(0);
        if (more) {
            GOff on;
            if constexpr (GATHER) {
#pragma unroll
                for (int i = 0; i < CPW; ++i) on.ga[i] = last_sb ? oN.ga[i] : oT.ga[i];
                on.gd = last_sb ? oN.gd : oT.gd;
            }
            stage(slots[1 - P], Tn, sbn, on);
            load_w(Tn, sbn, wring[1 - P]);
        }
        __builtin_amdgcn_sched_barrier(0);
        if (mine) {  // uniform
            // scale digits of sub-blocks 4g..4g+3 (fields 4g.. of the 96-bit word)
            const uint32_t w1 = (uint32_t)wc.hdr[1], w2 = (uint32_t)wc.hdr[2], w3 = (uint32_t)wc.hdr[3];
            const uint32_t x24 = g ? __builtin_amdgcn_alignbit(w2, w1, 24) : w1;
            const float dw = f16_bits_to_f32((uint32_t)wc.hdr[0]);
            const float dmin = f16_bits_to_f32((uint32_t)wc.hdr[0] >> 16);

            // pass 1: high digits (sc >> 3) over the whole superblock; pass 2: low
            // digits (sc & 7) into the same accumulators after a shift by 3.  The
            // fragments of K-step s+1 are read while K-step s multiplies.
            // (scheduling fences pin the reads of K-step s+1 ahead of the MFMAs
            // of K-step s; left alone, the scheduler sinks each read to just
            // before its MFMA and every MFMA waits out a full LDS latency)
            // The two workgroups on a CU put one wave on each SIMD.  While this
            // wave multiplies it takes issue priority, so the other wave's fold
            // and unpacking fill the issue slots between its MFMAs.
            __builtin_amdgcn_s_setprio(2);
#pragma unroll
            for (int pass = 0; pass < 2; ++pass) {
                v4i av[2][MT];
#pragma unroll
                for (int t = 0; t < MT; ++t)
                    av[0][t] = *reinterpret_cast<const v4i *>(S.a + t * 32 * ROW + frag(0));
#pragma unroll
                for (int s = 0; s < 8; ++s) {
                    __builtin_amdgcn_sched_barrier(0);
                    if (s + 1 < 8) {
#pragma unroll
                        for (int t = 0; t < MT; ++t)
                            av[(s + 1) & 1][t] = *reinterpret_cast<const v4i *>(S.a + t * 32 * ROW + frag(s + 1));
                    }
                    __builtin_amdgcn_sched_barrier(0);
                    const int si = 2 * ((s & 3) >> 1) + (s >> 2);  // sub-block 4g + si
                    const uint32_t dig = pass == 0 ? (x24 >> (6 * si + 3)) & 7u : (x24 >> (6 * si)) & 7u;
                    v4i bq;
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const uint32_t q = (uint32_t)wc.q[s & 3][e];
                        bq[e] = mul_digit(s < 4 ? q & 0x0F0F0F0Fu : (q >> 4) & 0x0F0F0F0Fu, dig);
                    }
#pragma unroll
                    for (int t = 0; t < MT; ++t)
                        acc[t] = (pass == 0 && s == 0) ? mma_i8(av[s & 1][t], bq, v16i{})
                                                       : mma_i8(av[s & 1][t], bq, acc[t]);
                }
                if (pass == 0) {
#pragma unroll
                    for (int t = 0; t < MT; ++t)
#pragma unroll
                        for (int r = 0; r < 16; ++r) acc[t][r] <<= 3;
                    // re-read the operands in pass 2 rather than keeping all of
                    // pass 1's live (registers are the scarcer unit)
                    asm volatile("" ::: "memory");
                }
            }
            __builtin_amdgcn_s_setprio(0);
            // min term, exactly: M = sum_j m_j * B_j with B_j the sum of the
            // sub-block's 32 quantized activations (staged as two bf16 parts that
            // are exact, 64*floor(B_j/64) and B_j mod 64); one bf16 MFMA per
            // m-tile, all products and partial sums integers below 2^24.  k-group
            // g carries sub-blocks 4g..4g+3: A row m holds both parts of those, B
            // the mins m_j twice.
            // fold: out += d_a[m] * (d[n] * float(sum_k sc*q*a) - dmin[n] * M)
            {
                // mins m_j: bits 48 + 6j of the 96-bit word (words w1, w2, w3)
                const uint64_t hi64 = (uint64_t)w2 | ((uint64_t)w3 << 32);  // bits 32..95
                const uint32_t mx = (uint32_t)(hi64 >> (16 + 24 * g));      // fields 4g..4g+3
                v8bf bm;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const __bf16 m = (__bf16)(float)((mx >> (6 * i)) & 63u);
                    bm[i] = m;
                    bm[4 + i] = m;
                }
                const float ndmin = -dmin;
#pragma unroll
                for (int t = 0; t < MT; ++t) {
                    const int8_t *lp = S.l + 32 * 16 * t + l_lane;
                    const v2u ap0 = *reinterpret_cast<const v2u *>(lp);
                    const v2u ap1 = *reinterpret_cast<const v2u *>(lp + BM * 16);
                    const v4i avv = {(int)ap0.x, (int)ap0.y, (int)ap1.x, (int)ap1.y};
                    const v16f mt = mma_bf16(__builtin_bit_cast(v8bf, avv), bm, v16f{});
                    v4f da4[4];
#pragma unroll
                    for (int q = 0; q < 4; ++q)
                        da4[q] = *reinterpret_cast<const v4f *>(S.d + 32 * t + 8 * q + d_lane);
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
#pragma unroll
                        for (int i = 0; i < 4; ++i) {
                            const int r = 4 * q + i;
                            out[t][r] = fmaf(fmaf((float)acc[t][r], dw, mt[r] * ndmin), da4[q][i], out[t][r]);
                        }
                    }
                }
            }
        }

        if constexpr (KS == 2) {
            if (last_sb) {
                // half 1 hands its sums to half 0 through the activation
                // region of this slot, once every wave is done reading it
                // (the next step's copies into it wait for the next barrier)
                asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
                barrier_nofence();
                float *red = reinterpret_cast<float *>(slots[P].a);
                if (half == 1) {
#pragma unroll
                    for (int t = 0; t < MT; ++t)
#pragma unroll
                        for (int r = 0; r < 16; ++r) red[((wave * MT + t) * 16 + r) * 64 + lane] = out[t][r];
                }
                asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
                barrier_nofence();
                if (half == 0) {
#pragma unroll
                    for (int t = 0; t < MT; ++t)
#pragma unroll
                        for (int r = 0; r < 16; ++r) out[t][r] += red[((wave * MT + t) * 16 + r) * 64 + lane];
                }
            }
        }
        if (last_sb && half == 0) {
            // epilogue of tile T: rows past M fall outside the resource and
            // are dropped; columns past N are sent out of range
            const int n = T.n0 + 32 * wave + ln;
            const int voff = n < N ? (4 * g * N + n) * 4 : OOB_VOFF;
            const auto ro = rs_o_of(T);
            const int orow0 = GATHER ? 0 : T.m0;
#pragma unroll
            for (int t = 0; t < MT; ++t) {
                // cast the whole vector: storing a bit-cast of one element
                // directly miscompiles to a store of element 0 (ROCm 7.2 clang)
                const v16i bits = __builtin_bit_cast(v16i, out[t]);
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int row = 32 * t + 8 * (r >> 2) + (r & 3);  // minus the lane's 4g
                    __builtin_amdgcn_raw_buffer_store_b32(bits[r], ro, voff, (orow0 + row) * N * 4, 0);
                }
            }
        }
        if (last_sb) {
#pragma unroll
            for (int t = 0; t < MT; ++t) out[t] = v16f{};
        }
        // advance (k, sb); entering tile k+1 computes tile k+2 once
        if (last_sb) {
            ++k;
            sb = 0;
            T = TN;
            TN = tile_xy<BM, GATHER>(a, tiles_m, slot_in_step + (k + 1) * G);
            if constexpr (GATHER) {
                oT = oN;
                goffs(TN, oN);
            }
        } else {
            ++sb;
        }
    };

    // prologue: stage iteration 0, its weights
    stage(slots[0], T, 0, oT);
    load_w(T, 0, wring[0]);
    for (int it = 0; it < total; it += 2) {
        iteration(std::integral_constant<int, 0>{}, it);
        if (it + 1 < total) iteration(std::integral_constant<int, 1>{}, it + 1);
    }
}

// ---------------------------------------------------------------------------
// Few tokens, K split over the waves of a workgroup (M <= 16 in use).
// A workgroup of KW waves owns 32 weight rows; wave w takes superblocks w,
// w + KW, w + 2KW, ... for every token row (MT 16-row m-tiles), so the waves
// of a workgroup read neighbouring bytes of the same weight rows.  At the end
// the KW partial sums are added through LDS in a fixed order.  On 14336 x
// 4096 weights that is 448 workgroups of 4 waves: two waves on most SIMDs.
// Activation fragments go straight from memory into registers, half a
// superblock ahead: every workgroup reads the same few token rows, so they
// come from L2, and staging them in LDS per wave would cap the waves per CU.
// The 16 x 16 x 64 int8 MFMA keeps the wasted rows of a few-token product
// to one 16-row tile, and its A operand is 16 rows of 64 contiguous bytes: a
// fragment load touches 16 64-byte pieces where a 32-row operand touches 64
// half-used ones (a 32-row build measured three times the L1 accesses of
// the two-wave kernel, with the address unit stalled on the L1 40% of the
// time).
// The weights and the fold data (activation scales and min-term operands of
// a superblock) stream through a small per-wave LDS ring with coalesced
// buffer -> LDS copies.  No barrier is needed until the final sum.
// Past 16 tokens the kernel loses to the ring kernels below: its waves spend
// most of their time waiting on memory (the vector-memory counter counts in
// issue order, so waiting for the next half's activation loads also waits
// for every weight copy issued before them, and a weight stage gets at most
// two halves to arrive), and the m-tile registers leave no room to load the
// activations further ahead.
//
// v_mfma_i32_16x16x64_i8: lane l supplies row l % 16 of A and column l % 16
// of B with k-group l / 16 (16 values each); register i of the 4-register
// result holds row 4(l/16) + i, column l % 16.
// K order: K-step s (0..3) of a superblock covers values 64s .. 64s+63, lane
// group kg the 16 values k = 64s + 16kg + i, all in sub-block j = 2s + kg/2.
// In the Q4_K nibble layout (32-byte group u holds weights 64u + o in its
// low nibbles and 64u + 32 + o in its high nibbles, o = byte within the
// group) those are the low (kg < 2) or high (kg >= 2) nibbles of bytes 32s +
// 16(kg % 2) + i: piece 2(s % 2) + kg % 2 of the 64 nibble bytes of half s/2.
// ---------------------------------------------------------------------------
constexpr int SWN = 32 * 64;    // half the nibble bytes of 32 blocks
constexpr int SHD = 32 * 16;    // block headers of 32 rows
constexpr int SDS = 64 * 4;     // activation scales of 64 rows
constexpr int SLS = 2 * 64 * 16;  // min-term operands (hi, lo) of 64 rows
constexpr int KWS = SWN + SHD;  // weight stage: nibbles of one half of 32 blocks, their headers
constexpr int KFS = SDS + SLS;  // fold data of one superblock: scales and min-term parts of 64 rows

template <int MT, int KW, int DW>
struct SplitCfg {
    static_assert(MT == 1 || MT == 2 || MT == 4, "16-row m-tiles: up to 16, 32 or 64 tokens");
    static_assert(DW >= 2, "a weight stage is waited for two halves after its copies are issued");
    static_assert((8 * MT) % KW == 0, "the final sum deals output registers evenly over the waves");
    static constexpr int RING = (DW + 1) * KWS;
    static constexpr int LDS = RING + KFS;  // per wave
    static_assert(LDS >= 8 * MT * 64 * 4, "the final sum reuses each wave's stages");
    // buffer -> LDS copies of weight stage x: two of nibbles, plus two of
    // headers for a first half
    static constexpr int szW(int x) { return 2 + 2 * (1 - (x & 1)); }
};

template <int MT, int KW, int DW>
__global__ __launch_bounds__(64 * KW, 8 / KW) void gemm_q4k_split_kernel(Args a) {
    using C = SplitCfg<MT, KW, DW>;
    __shared__ __attribute__((aligned(16))) int8_t s_lds[KW][C::LDS];

    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int r16 = lane & 15, kg = lane >> 4;
    const int M = a.M, N = a.N, K = a.K, nsb = a.nsb;
    const int n0 = blockIdx.x * 32;
    const int rowbytes = nsb * BB;
    const int nk = (nsb - w + KW - 1) / KW;  // superblocks of this wave (0 if nsb <= w)

    const auto rs_a = __builtin_amdgcn_make_buffer_rsrc((void *)a.qs, (short)0, M * K, RSRC_FLAGS);
    const auto rs_d = __builtin_amdgcn_make_buffer_rsrc((void *)a.da, (short)0, nsb * M * 4, RSRC_FLAGS);
    const auto rs_l = __builtin_amdgcn_make_buffer_rsrc((void *)a.alpha, (short)0, nsb * 2 * M * 16, RSRC_FLAGS);
    const auto rs_w = __builtin_amdgcn_make_buffer_rsrc((void *)a.W, (short)0, N * rowbytes, RSRC_FLAGS);
    const auto rs_o = __builtin_amdgcn_make_buffer_rsrc((void *)a.out, (short)0, M * N * 4, RSRC_FLAGS);

    // activation fragment of m-tile t: row 16t + r16, bytes 64s + 16kg of the
    // superblock (rows past M read as zero)
    int a_vo[MT];
#pragma unroll
    for (int t = 0; t < MT; ++t) a_vo[t] = (16 * t + r16) * K + 16 * kg;
    // Weight stage: nibble copy i puts piece (l%4) ^ ((l/8)%4) of the 64
    // nibble bytes of row 16i + l/4 at LDS piece 64i + l, so that row r's
    // piece p sits at 4r + (p ^ ((r/2)%4)) and the 16-byte reads below, eight
    // consecutive rows at a time, hit all 32 banks; header copy i puts dword
    // l%4 of row 16i + l/4 at dword 64i + l.  (Row offsets as unsigned: rows
    // past N in the last strip may pass 2^31, and the range check drops them.)
    const uint32_t wr0 = (uint32_t)(n0 + (lane >> 2)) * (uint32_t)rowbytes;
    const uint32_t wr1 = wr0 + 16u * (uint32_t)rowbytes;
    const int wsw = 16 * ((lane & 3) ^ ((lane >> 3) & 3));
    const int w_vb0 = (int)(wr0 + 16 + wsw), w_vb1 = (int)(wr1 + 16 + wsw);
    const int h_vb0 = (int)(wr0 + 4 * (lane & 3)), h_vb1 = (int)(wr1 + 4 * (lane & 3));
    // this lane's pieces (K-step 2H + ss, n-tile nt): row 16nt + r16, piece
    // 2ss + kg%2
    uint32_t wo[2][2];
#pragma unroll
    for (int nt = 0; nt < 2; ++nt)
#pragma unroll
        for (int ss = 0; ss < 2; ++ss) {
            const int r = 16 * nt + r16;
            wo[nt][ss] = 16 * (4 * r + ((2 * ss + (kg & 1)) ^ ((r >> 1) & 3)));
        }
    const uint32_t nib_sh = 4 * (kg >> 1);  // high nibbles for k-groups 2, 3

    int8_t *const ring = &s_lds[w][0];
    int8_t *const fold = &s_lds[w][C::RING];
    const uint32_t ring_addr = lds_addr(ring), fold_addr = lds_addr(fold);
    // stage x: superblock w + KW * min(x/2, nk - 1) (past the end: a repeat
    // of the last, never used), half x % 2
    auto sb_of = [&](int x) { return w + KW * min(x >> 1, nk - 1); };

    v4i av[2][MT][2];  // activation fragments of the halves of parity 0 / 1
    // A stage: the activation fragments of half x; an odd x also brings the
    // superblock's fold data (the previous superblock's was read in full one
    // half earlier).  Copies are pinned between compiler memory barriers
    // (the LDS reads are asm the compiler does not see as memory accesses).
    auto issueA = [&](auto PP, int x) __attribute__((always_inline)) {
        constexpr int P = decltype(PP)::value;
        asm volatile("" ::: "memory");
        const int sb = sb_of(x);
#pragma unroll
        for (int t = 0; t < MT; ++t)
#pragma unroll
            for (int ss = 0; ss < 2; ++ss) av[P][t][ss] = ld16(rs_a, a_vo[t], sb * ROW + 128 * P + 64 * ss);
        if (P == 1) {
            copy4(rs_d, fold, 4 * lane, sb * M * 4);
            copy16(rs_l, fold + SDS, 16 * lane, sb * 2 * M * 16);
            copy16(rs_l, fold + SDS + 1024, 16 * lane, (sb * 2 + 1) * M * 16);
        }
        asm volatile("" ::: "memory");
    };
    auto issueW = [&](int x) __attribute__((always_inline)) {
        asm volatile("" ::: "memory");
        const int H = x & 1;
        const int sb = sb_of(x);
        int8_t *S = ring + (x % (DW + 1)) * KWS;
        copy16(rs_w, S, w_vb0, sb * BB + 64 * H);
        copy16(rs_w, S + 1024, w_vb1, sb * BB + 64 * H);
        if (H == 0) {
            copy4(rs_w, S + SWN, h_vb0, sb * BB);
            copy4(rs_w, S + SWN + 256, h_vb1, sb * BB);
        }
        asm volatile("" ::: "memory");
    };

    v4f out[2][MT];
#pragma unroll
    for (int nt = 0; nt < 2; ++nt)
#pragma unroll
        for (int t = 0; t < MT; ++t) out[nt][t] = v4f{};
    v4i acc_h[2][MT], acc_l[2][MT];
    v4i hdr[2];

    // half j (parity H): the weights of stage j landed DW halves after their
    // copies were issued; this half's activation fragments and fold data were
    // issued one half ago, followed only by the copies of weight stage
    // j - 1 + DW
    auto half = [&](auto HH, int j) __attribute__((always_inline)) {
        constexpr int H = decltype(HH)::value;
        // (scheduling fences keep each half's wait and copies in place: the
        // scheduler would otherwise hoist the next half's wait into this
        // half's multiplies, and the next activation loads ahead of this
        // half's weight copies, which shortens what the waits leave in flight)
        __builtin_amdgcn_sched_barrier(0);
        wait_vmcnt<C::szW((H + 1 + DW) & 1)>();
        issueA(std::integral_constant<int, 1 - H>{}, j + 1);
        issueW(j + DW);
        __builtin_amdgcn_sched_barrier(0);
        const uint32_t SW = ring_addr + (uint32_t)((j % (DW + 1)) * KWS);
        if (H == 0) {
            hdr[0] = lds_read16<SWN>(SW + 16 * r16);
            hdr[1] = lds_read16<SWN + 256>(SW + 16 * r16);
        }
        v4i wq[2][2];
        wq[0][0] = lds_read16<0>(SW + wo[0][0]);
        wq[0][1] = lds_read16<0>(SW + wo[0][1]);
        wq[1][0] = lds_read16<0>(SW + wo[1][0]);
        wq[1][1] = lds_read16<0>(SW + wo[1][1]);
        if (H == 0) {
            lds_wait<5>(hdr[0]);
            lds_wait<4>(hdr[1]);
        }
        lds_wait<3>(wq[0][0]);
        lds_wait<2>(wq[0][1]);
        lds_wait<1>(wq[1][0]);
        lds_wait<0>(wq[1][1]);
#pragma unroll
        for (int ss = 0; ss < 2; ++ss) {
#pragma unroll
            for (int nt = 0; nt < 2; ++nt) {
                // scale of sub-block j = 4H + 2ss + kg/2: field j, at bits
                // 12ss + 6(kg/2) of the fields from 4H on
                const uint32_t w1 = (uint32_t)hdr[nt][1], w2 = (uint32_t)hdr[nt][2];
                const uint32_t x = H == 0 ? w1 : __builtin_amdgcn_alignbit(w2, w1, 24);
                const uint32_t sc = (x >> (12 * ss + 6 * (kg >> 1))) & 63u;
                v4i bh, bl;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const uint32_t nib = ((uint32_t)wq[nt][ss][e] >> nib_sh) & 0x0F0F0F0Fu;
                    bh[e] = mul_digit(nib, sc >> 3);
                    bl[e] = mul_digit(nib, sc & 7u);
                }
#pragma unroll
                for (int t = 0; t < MT; ++t) {
                    if (H == 0 && ss == 0) {
                        acc_h[nt][t] = mma16_i8(av[H][t][ss], bh, v4i{});
                        acc_l[nt][t] = mma16_i8(av[H][t][ss], bl, v4i{});
                    } else {
                        acc_h[nt][t] = mma16_i8(av[H][t][ss], bh, acc_h[nt][t]);
                        acc_l[nt][t] = mma16_i8(av[H][t][ss], bl, acc_l[nt][t]);
                    }
                }
            }
        }
        if (H == 1) {
            // fold: out += d_a[m] * (d[n] * float(8*acc_h + acc_l) - dmin[n] * M)
            // with M = sum_j m_j B_j exact: one bf16 MFMA per output tile, A
            // row m = both exact parts of B_0..B_7 (k-groups 0 and 1; k-groups
            // 2 and 3 zero), B column n = m_0..m_7 (all products and partial
            // sums integers below 2^24)
            v4f da[MT];
            v4i ap[MT];
#pragma unroll
            for (int t = 0; t < MT; ++t) {
                da[t] = __builtin_bit_cast(v4f, lds_read16<0>(fold_addr + 64 * t + 16 * kg));
                ap[t] = lds_read16<0>(fold_addr + SDS + 1024 * (kg & 1) + 16 * (16 * t + r16));
            }
            v8bf bm[2];
            float dw[2], ndmin[2];
#pragma unroll
            for (int nt = 0; nt < 2; ++nt) {
                dw[nt] = f16_bits_to_f32((uint32_t)hdr[nt][0]);
                ndmin[nt] = -f16_bits_to_f32((uint32_t)hdr[nt][0] >> 16);
                // mins m_j: bits 48 + 6j of the 96-bit word
                const uint64_t hi64 = (uint64_t)(uint32_t)hdr[nt][2] | ((uint64_t)(uint32_t)hdr[nt][3] << 32);
                const uint64_t mx = hi64 >> 16;
#pragma unroll
                for (int i = 0; i < 8; ++i) bm[nt][i] = (__bf16)(float)(uint32_t)((mx >> (6 * i)) & 63u);
            }
            // (reads in flight after da[t]: 2(MT-1-t) + 1; after ap[t]: one fewer)
#pragma unroll
            for (int t = 0; t < MT; ++t) {
                lds_wait_n(2 * (MT - 1 - t) + 1, da[t]);
                lds_wait_n(2 * (MT - 1 - t), ap[t]);
            }
#pragma unroll
            for (int t = 0; t < MT; ++t) {
                const v4i avv = kg < 2 ? ap[t] : v4i{};
#pragma unroll
                for (int nt = 0; nt < 2; ++nt) {
                    const v4f mt = mma16_bf16(__builtin_bit_cast(v8bf, avv), bm[nt], v4f{});
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int T = (acc_h[nt][t][i] << 3) + acc_l[nt][t][i];
                        out[nt][t][i] = fmaf(fmaf((float)T, dw[nt], mt[i] * ndmin[nt]), da[t][i], out[nt][t][i]);
                    }
                }
            }
        }
    };

    if (nk > 0) {
        // Every loop pass is one superblock (two halves), so each wait sees
        // the same copies in flight.  The prologue issues what halves -DW ..
        // -1 would have: weight stages 0 .. DW-1 and, last but one, the
        // activations of half 0.
#pragma unroll
        for (int x = 0; x + 1 < DW; ++x) issueW(x);
        issueA(std::integral_constant<int, 0>{}, 0);
        issueW(DW - 1);
        for (int k = 0; k < nk; ++k) {
            half(std::integral_constant<int, 0>{}, 2 * k);
            half(std::integral_constant<int, 1>{}, 2 * k + 1);
        }
    }
    // no copy may still be writing this wave's stages, no read still pending
    wait_vmcnt<0>();
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");

    // Sum the KW partials in wave order.  Each wave parks its sums in its own
    // stages; wave w then adds and stores output registers w*PER .. +PER-1
    // (register u = 4(MT*nt + t) + i).
    constexpr int PER = 8 * MT / KW;
    {
        float *const mine = reinterpret_cast<float *>(&s_lds[w][0]);
#pragma unroll
        for (int nt = 0; nt < 2; ++nt)
#pragma unroll
            for (int t = 0; t < MT; ++t)
#pragma unroll
                for (int i = 0; i < 4; ++i) mine[(4 * (MT * nt + t) + i) * 64 + lane] = out[nt][t][i];
    }
    __syncthreads();
#pragma unroll
    for (int u = 0; u < PER; ++u) {
        const int idx = w * PER + u;
        float sum = 0.0f;
#pragma unroll
        for (int v = 0; v < KW; ++v) sum += reinterpret_cast<const float *>(&s_lds[v][0])[idx * 64 + lane];
        const int nt = idx / (4 * MT), t = (idx >> 2) % MT, i = idx & 3;
        const int n = n0 + 16 * nt + r16;
        const int voff = n < N ? n * 4 : OOB_VOFF;
        const int row = 16 * t + 4 * kg + i;
        __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(int, sum), rs_o, voff, row * N * 4, 0);
    }
}

// ---------------------------------------------------------------------------
// Matrix-vector kernel for one or two tokens (decode): the product is a stream of
// 33 MB of weights for a handful of dot products each, so it needs many waves
// with loads in flight rather than matrix cores.  Workgroups of 4 waves each
// own 8 weight rows (2 per wave: 8.4 us for one token on 14336 x 4096, against
// 8.9 and 9.0 with four and one); the activation buffer (values, scales,
// min-term operands of the few tokens) is copied once per workgroup into LDS.
//
// Load instruction i of a wave covers 8 consecutive superblocks of one of its
// rows (K is a multiple of 2048, so a row is a whole number of them); lane l
// takes 16-byte nibble chunk c8 = l % 8 of superblock l / 8 of them, a
// contiguous 1 KiB run apart from the block headers, which a second load
// brings (each lane its superblock's 16-byte header).  Chunk c8 holds the low
// nibbles of weights 64c + 16h + i (sub-block 2c) and the high nibbles of
// weights 64c + 32 + 16h + i (sub-block 2c + 1), c = c8 / 2, h = c8 % 2,
// i < 16.  Per token the lane forms the integer sums of those 32 products
// with v_dot4, scales them by the two sub-block scales, and folds
//   acc += d_a * (d * float(sc0 S0 + sc1 S1) - dmin * m_c8 * B_c8),
// the min term of sub-block c8 (one sub-block per lane covers all eight).
// A row's total is the sum over the 64 lanes of its load instructions, in a
// fixed butterfly order, stored by lane 0.
// ---------------------------------------------------------------------------
namespace mv {
constexpr int NW = 4;          // waves per workgroup
#ifndef MV_RPW
#define MV_RPW 2
#endif
constexpr int RPW = MV_RPW;    // weight rows per wave
constexpr int RPG = NW * RPW;  // weight rows per workgroup
// Load instructions in flight per row: two once a row has three or more
// (K >= 6144).  One token on 4096 rows: 5.48 against 6.27 us at K = 8192,
// 7.99 against 9.13 at 14336; at K = 4096 (two per row) the single one
// stays (8.40 against 8.59 us on 14336 rows).
__host__ __device__ constexpr int depth_for(int ipr) { return ipr >= 3 ? 2 : 1; }
// Up to two tokens: measured on 14336 x 4096 weights, 8.9 and 10.6 us
// against 14.6 us for the few-token kernel; at three and four tokens the two
// kernels tie, beyond that the per-token LDS reads and dot products lose.
constexpr int MAX_TOKENS = 2;

// LDS bytes of the staged activations for MT tokens (MT >= M); sections at
// 1 KiB multiples so every copy stays inside its own section
__host__ __device__ constexpr int lds_qs(int MT, int K) { return MT * K; }
__host__ __device__ constexpr int lds_d(int M, int nsb) { return (nsb * M * 4 + 1023) / 1024 * 1024; }
__host__ __device__ constexpr int lds_al(int M, int nsb) { return (nsb * 2 * M * 16 + 1023) / 1024 * 1024; }
// total, with room for the reads of token rows past M (never stored)
__host__ __device__ constexpr int lds_bytes(int MT, int M, int K, int nsb) {
    return lds_qs(MT, K) + lds_d(M, nsb) + lds_al(M, nsb) + 256;
}
}  // namespace mv

template <int MT, int D>
__global__ __launch_bounds__(64 * mv::NW) void gemv_q4k_kernel(Args a) {
    extern __shared__ __attribute__((aligned(16))) int8_t s_mv[];
    const int lane = threadIdx.x & 63;
    const int w = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
    const int M = a.M, N = a.N, K = a.K, nsb = a.nsb;
    const int rowbytes = nsb * BB;
    const int ipr = nsb >> 3;                  // load instructions per row
    const int row0 = blockIdx.x * mv::RPG + w * mv::RPW;

    int8_t *const s_qs = s_mv;
    float *const s_d = reinterpret_cast<float *>(s_mv + mv::lds_qs(MT, K));
    int8_t *const s_al = s_mv + mv::lds_qs(MT, K) + mv::lds_d(M, nsb);

    const auto rs_a = __builtin_amdgcn_make_buffer_rsrc((void *)a.qs, (short)0, M * K, RSRC_FLAGS);
    const auto rs_d = __builtin_amdgcn_make_buffer_rsrc((void *)a.da, (short)0, nsb * M * 4, RSRC_FLAGS);
    const auto rs_l = __builtin_amdgcn_make_buffer_rsrc((void *)a.alpha, (short)0, nsb * 2 * M * 16, RSRC_FLAGS);
    const auto rs_w = __builtin_amdgcn_make_buffer_rsrc((void *)a.W, (short)0, N * rowbytes, RSRC_FLAGS);

    // ---- activations -> LDS, shared by the workgroup's waves ----------------
    // (M*K is a multiple of 2048; the last scale and min-operand copies read
    // past their sections as zeros and stay inside their LDS sections)
    {
        const int nq = (M * K) >> 10, nd = (nsb * M * 4 + 255) >> 8, nl = (nsb * 2 * M * 16 + 1023) >> 10;
        // copy c holds superblocks 4c'..4c'+3 of one token row; lane l fills
        // slot l%16 of superblock l/16 with piece (l%16) ^ 2(sb%2), which
        // spreads the two superblocks one read instruction touches over
        // different banks
        const int aq = 16 * (lane ^ (2 * ((lane >> 4) & 1)));
        for (int c = w; c < nq; c += mv::NW) copy16(rs_a, s_qs + 1024 * c, 1024 * c + aq, 0);
        for (int c = w; c < nd; c += mv::NW) copy4(rs_d, reinterpret_cast<int8_t *>(s_d) + 256 * c, 256 * c + 4 * lane, 0);
        for (int c = w; c < nl; c += mv::NW) copy16(rs_l, s_al + 1024 * c, 1024 * c + 16 * lane, 0);
    }

    // ---- weights: D load instructions in flight per row -----------------------
    // Instruction (r, j) reads superblocks 8j .. 8j+7 of the wave's row r; the
    // wave walks j = 0 .. ipr-1 over its RPW rows in turn, keeping D
    // instructions per row in flight, and past the last group re-reads it
    // (unused, drained at the end), so every step has the same loads in
    // flight.
    const int c8 = lane & 7, sbl = lane >> 3;
    const int cq = c8 >> 1, hq = c8 & 1;
    v4i wq[mv::RPW][D], wh[mv::RPW][D];
    auto issue = [&](int r, int j, v4i &q, v4i &h) __attribute__((always_inline)) {
        const int off = (row0 + r) * rowbytes + (8 * min(j, ipr - 1) + sbl) * BB;  // < (N + 256) rows
        q = ld16(rs_w, off + 16 + 16 * c8, 0);
        h = ld16(rs_w, off, 0);
    };
#pragma unroll
    for (int jj = 0; jj < D; ++jj)
#pragma unroll
        for (int r = 0; r < mv::RPW; ++r) issue(r, jj, wq[r][jj], wh[r][jj]);
    // this wave's activation copies have landed once at most the weight loads
    // are in flight; the barrier covers the other waves' copies
    wait_vmcnt<2 * mv::RPW * D>();
    barrier_nofence();

    float acc[mv::RPW][MT];
#pragma unroll
    for (int r = 0; r < mv::RPW; ++r)
#pragma unroll
        for (int m = 0; m < MT; ++m) acc[r][m] = 0.0f;

    auto compute = [&](int j, const v4i &q, const v4i &h, float (&ac)[MT]) __attribute__((always_inline)) {
        const int sb = 8 * j + sbl;
        // header: d, dmin, scales sc_j (bits 6j) and mins m_j (bits 48 + 6j)
        const uint32_t w0 = (uint32_t)h[0], w1 = (uint32_t)h[1], w2 = (uint32_t)h[2], w3 = (uint32_t)h[3];
        const uint64_t lo64 = (uint64_t)w1 | ((uint64_t)w2 << 32);
        const uint64_t hi64 = (uint64_t)w2 | ((uint64_t)w3 << 32);
        const uint32_t scs = (uint32_t)(lo64 >> (12 * cq));
        const int sc0 = (int)(scs & 63u), sc1 = (int)((scs >> 6) & 63u);
        const float mn = (float)((uint32_t)(hi64 >> (16 + 6 * c8)) & 63u);
        const float dw = f16_bits_to_f32(w0);
        const float cmin = -f16_bits_to_f32(w0 >> 16) * mn;
        int lo[4], hi[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            lo[e] = q[e] & 0x0F0F0F0F;
            hi[e] = (int)(((uint32_t)q[e] >> 4) & 0x0F0F0F0Fu);
        }
        // pieces 4cq + hq (low nibbles' weights) and + 2 (high), swizzled
        const int sw = 2 * (sb & 1);
        const int k0 = sb * ROW + 16 * ((4 * cq + hq) ^ sw);
        const int k1 = sb * ROW + 16 * ((4 * cq + hq + 2) ^ sw);
        // every token's operands first, so the reads overlap
        v4i a0[MT], a1[MT];
        float da[MT];
        uint16_t ah[MT], al[MT];
#pragma unroll
        for (int m = 0; m < MT; ++m) {
            a0[m] = *reinterpret_cast<const v4i *>(s_qs + m * K + k0);
            a1[m] = *reinterpret_cast<const v4i *>(s_qs + m * K + k1);
            da[m] = s_d[sb * M + m];
            ah[m] = *reinterpret_cast<const uint16_t *>(s_al + ((sb * 2) * M + m) * 16 + 2 * c8);
            al[m] = *reinterpret_cast<const uint16_t *>(s_al + ((sb * 2 + 1) * M + m) * 16 + 2 * c8);
        }
#pragma unroll
        for (int m = 0; m < MT; ++m) {
            int s0 = 0, s1 = 0;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                s0 = __builtin_amdgcn_sdot4(lo[e], a0[m][e], s0, false);
                s1 = __builtin_amdgcn_sdot4(hi[e], a1[m][e], s1, false);
            }
            const int u = sc0 * s0 + sc1 * s1;
            // B of sub-block c8 from its two exact parts
            const float bj = __builtin_bit_cast(float, (uint32_t)ah[m] << 16) +
                             __builtin_bit_cast(float, (uint32_t)al[m] << 16);
            ac[m] = fmaf(fmaf((float)u, dw, cmin * bj), da[m], ac[m]);
        }
    };

    for (int j0 = 0; j0 < ipr; j0 += D) {
#pragma unroll
        for (int jj = 0; jj < D; ++jj) {
#pragma unroll
            for (int r = 0; r < mv::RPW; ++r) {
                // row r's instruction j0 + jj has landed once the RPW * D - 1
                // issued after it may still be in flight
                wait_vmcnt<2 * (mv::RPW * D - 1)>();
                if (j0 + jj < ipr) compute(j0 + jj, wq[r][jj], wh[r][jj], acc[r]);  // uniform
                issue(r, j0 + jj + D, wq[r][jj], wh[r][jj]);
            }
        }
    }

    // Each row's total: its 64 lanes summed in a fixed butterfly order (all
    // rows and tokens step together), stored by lane 0.
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1)
#pragma unroll
        for (int r = 0; r < mv::RPW; ++r)
#pragma unroll
            for (int m = 0; m < MT; ++m) acc[r][m] += __shfl_xor(acc[r][m], o, 64);
    if (lane == 0) {
#pragma unroll
        for (int r = 0; r < mv::RPW; ++r)
#pragma unroll
            for (int m = 0; m < MT; ++m)
                if (m < M && row0 + r < N) a.out[(int64_t)m * N + row0 + r] = acc[r][m];
    }
    wait_vmcnt<0>();
}

// ---------------------------------------------------------------------------
// Few tokens (3..64, weights wide enough to fill the CUs with 64-row
// workgroups): all tokens in one workgroup, K split in two halves.  The token
// rows form one, two or four 16-row m-tiles (TM = 16, 32 or 64).
// A workgroup owns 64 weight rows as four 16-row strips; wave w takes strip
// w % 4 over the superblocks of K-half w / 4, so two waves share each SIMD.
// Step t multiplies superblock t (first half) and T + t (second half),
// T = ceil(nsb / 2).  The activations of a step (values, scales, min-term
// operands of both halves, all token rows) are copied global -> LDS into a
// ring of L + 1 slots, L steps ahead; each wave loads its strip's weights
// for the same step into a register ring of L + 1 slots, in the same issue.  Vector-memory loads complete in issue order, so the wait for a
// step's copies is also a wait for the weights issued before them, but
// those are the weights of the same step or earlier: nothing is held up
// that is not needed.  (The kernels above stage activations one step ahead
// while weights run further, and there the in-order wait stalls.)  The two
// halves are summed through LDS at the end, in a fixed order.
//
// v_mfma_i32_16x16x64_i8 operands, in this kernel's K order: in K-step s of
// a superblock, lane group kg (lane / 16) holds the 16 values k = 64kg + 16s
// + i, sub-block j = 2kg + s/2.  Those are the low (s < 2) or high (s >= 2)
// nibbles of nibble bytes 32kg + 16(s % 2) + i (byte 32c + t holds weights
// 64c + t and 64c + 32 + t), so a lane loads 32 contiguous nibble bytes per
// superblock and uses each byte twice.  The A operand of K-step s is the 16
// contiguous activation bytes at 64kg + 16s of the token row.
// ---------------------------------------------------------------------------
constexpr int RING_ZERO = 1024;        // zero bytes read as the min-term operand of lanes 32..63

template <int TM>
struct RingCfg {
    static_assert(TM == 16 || TM == 32 || TM == 64, "16, 32 or 64 token rows");
    static constexpr int MT = TM / 16;             // 16-row m-tiles
    // steps of lead, and LDS slots / weight register sets.  Measured on
    // 14336 weight rows, K = 2048 .. 8192: with 32 or 64 token rows a lead
    // of two steps is 4-9% faster than three, and four is 10% slower than
    // three; one step is up to 3% faster with 64 rows at K <= 3072 but
    // 6-9% slower at K = 8192.  With 16 rows three steps are as fast as
    // two or slightly faster, and one is 6-35% slower.
    static constexpr int L = TM == 16 ? 3 : 2;
    static constexpr int S = L + 1;
    static constexpr int ACTH = TM * ROW;          // values of one half: [row][256], swizzled
    static constexpr int DAH = 256;                // scales of one half (a 64-lane 4-byte copy)
    // min-term operands of one half: [part][row][16] (at TM = 16 the 1 KiB
    // copy's second half lands in padding)
    static constexpr int ALH = 2 * TM * 16 > 1024 ? 2 * TM * 16 : 1024;
    static constexpr int O_DA = 2 * ACTH, O_AL = O_DA + 2 * DAH;
    static constexpr int SLOT = O_AL + 2 * ALH;
    static constexpr int LDS = S * SLOT + RING_ZERO;
    static constexpr int NA = ACTH / 1024;         // value copies per half
    static constexpr int NL = ALH / 1024;          // operand copies per half
    static_assert(NL <= 2 && NA % 4 == 0, "four value copies of a half per wave group, two operand parts");
    static constexpr int CPW = NA / 4 + 1;         // copies per wave and step
    static constexpr int LOADS = CPW + 3;          // vector-memory instructions per wave and step
    static_assert(LOADS * (L - 1) < 64, "vmcnt range");
};

struct RingW {
    v4i hdr, q0, q1;  // block header; nibble bytes 32kg .. +15, 32kg + 16 .. +15
};

template <int TM>
__global__ __launch_bounds__(512, 1) void gemm_q4k_ring_kernel(Args a) {
    using C = RingCfg<TM>;
    constexpr int MT = C::MT;
    __shared__ __attribute__((aligned(16))) int8_t s_lds[C::LDS];

    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int strip = w & 3, kh = w >> 2;
    const int r16 = lane & 15, kg = lane >> 4;
    const int M = a.M, N = a.N, K = a.K, nsb = a.nsb;
    const int T = (nsb + 1) >> 1;            // steps
    const int n0 = blockIdx.x * 64 + 16 * strip;
    const int rowbytes = nsb * BB;

    const auto rs_a = __builtin_amdgcn_make_buffer_rsrc((void *)a.qs, (short)0, M * K, RSRC_FLAGS);
    const auto rs_d = __builtin_amdgcn_make_buffer_rsrc((void *)a.da, (short)0, nsb * M * 4, RSRC_FLAGS);
    const auto rs_l = __builtin_amdgcn_make_buffer_rsrc((void *)a.alpha, (short)0, nsb * 2 * M * 16, RSRC_FLAGS);
    const auto rs_w = __builtin_amdgcn_make_buffer_rsrc((void *)a.W, (short)0, N * rowbytes, RSRC_FLAGS);
    const auto rs_o = __builtin_amdgcn_make_buffer_rsrc((void *)a.out, (short)0, M * N * 4, RSRC_FLAGS);
    // no records: reads return zero without a memory access (copies and
    // loads of steps past the end, so that every step issues the same)
    const auto rs_nul = __builtin_amdgcn_make_buffer_rsrc((void *)a.W, (short)0, 0, RSRC_FLAGS);

    // (the stores complete before the first step's barrier, which carries no
    // fence)
    int8_t *const zero = s_lds + C::S * C::SLOT;
    for (int i = tid; i < RING_ZERO / 4; i += 512) reinterpret_cast<uint32_t *>(zero)[i] = 0u;
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");

    // ---- copies of step x into slot x % S.  Wave w copies for its own
    // K-half kh: value copies CPV*(w%4) .. +CPV-1 (copy r: rows 4r .. 4r+3;
    // lane l fills piece l%16 of row 4r + l/16 with piece (l%16) ^ row), and
    // one more by w%4: the scales (lane l: token l), the min-term operands
    // (TM = 64: part w%4 - 1, lane l token l; TM = 32: lane l part l/32,
    // token l%32; TM = 16: lane l part (l/16)%2, token l%16, lanes 32..63
    // into padding), or a repeat of the last operand copy (the same bytes to
    // the same place).  Per-lane offsets are fixed; the superblock goes in
    // the scalar offset.  Token rows past M read other rows' data or zero;
    // their outputs are dropped.
    constexpr int CPV = C::NA / 4;
    const int wq = w & 3;
    int a_vo[CPV];
#pragma unroll
    for (int i = 0; i < CPV; ++i) {
        const int row = 4 * (CPV * wq + i) + (lane >> 4);
        a_vo[i] = row * K + 16 * ((lane & 15) ^ (row & 15));
    }
    const int x_part = TM == 64 ? min(max(wq - 1, 0), 1) : TM == 32 ? (lane >> 5) : ((lane >> 4) & 1);
    const int x_tok = TM == 64 ? lane : (lane & (TM - 1));
    const int x_vo = wq == 0 ? 4 * lane : (x_part * M + x_tok) * 16;
    const int x_lds = wq == 0 ? C::O_DA + kh * C::DAH
                              : C::O_AL + kh * C::ALH + (TM == 64 ? min(max(wq - 1, 0), 1) * 1024 : 0);
    auto copies = [&](int x) __attribute__((always_inline)) {
        int8_t *S = s_lds + (x % C::S) * C::SLOT;
        const int sb = kh ? T + x : x;
        const bool real = x < T && sb < nsb;
        const int sbr = real ? sb : 0;
        const auto ra = real ? rs_a : rs_nul;
#pragma unroll
        for (int i = 0; i < CPV; ++i)
            copy16(ra, S + kh * C::ACTH + (CPV * wq + i) * 1024, a_vo[i], sbr * ROW);
        if (wq == 0) copy4(real ? rs_d : rs_nul, S + x_lds, x_vo, sbr * M * 4);
        else copy16(real ? rs_l : rs_nul, S + x_lds, x_vo, sbr * 2 * M * 16);
    };
    // ---- this lane's weights: row n0 + r16, header and 32 nibble bytes ----
    // (row offsets as unsigned: rows past N may pass 2^31, and the range
    // check drops them)
    const int w_hdr = (int)((uint32_t)(n0 + r16) * (uint32_t)rowbytes);
    const int w_nib = w_hdr + 16 + 32 * kg;
    RingW ring[C::S];
    auto wload = [&](int x, RingW &R) __attribute__((always_inline)) {
        const int sb = kh ? T + x : x;
        const bool real = x < T && sb < nsb;
        const auto rw = real ? rs_w : rs_nul;
        const int so = (real ? sb : 0) * BB;
        R.hdr = ld16(rw, w_hdr, so);
        R.q0 = ld16(rw, w_nib, so);
        R.q1 = ld16(rw, w_nib + 16, so);
    };

    v4f out[MT];
#pragma unroll
    for (int t = 0; t < MT; ++t) out[t] = v4f{};
    // LDS addresses (the reads are instructions of our own with explicit
    // waits: the compiler's copy tracking would make them wait for every
    // load in flight).  K-step s of m-tile t: row 16t + r16, piece
    // (4kg + s) ^ r16; m-tile t is 16t rows (4096t bytes) on.
    uint32_t a_ad[4];
#pragma unroll
    for (int s = 0; s < 4; ++s)
        a_ad[s] = lds_addr(s_lds) + kh * C::ACTH + r16 * ROW + (((4 * kg + s) ^ r16) << 4);
    // min-term operands: part kg of row 16t + r16 for kg < 2, zeros above
    const uint32_t l_ad = kg < 2 ? lds_addr(s_lds) + C::O_AL + kh * C::ALH + (kg & 1) * (TM * 16) + 16 * r16
                                 : lds_addr(zero) + 16 * r16;
    const uint32_t l_slot = kg < 2 ? 1u : 0u;  // slot offsets apply to real operands only
    // scales of rows 4kg .. 4kg+3 of m-tile t
    const uint32_t d_ad = lds_addr(s_lds) + C::O_DA + kh * C::DAH + 16 * kg;

    auto compute = [&](const RingW &R, uint32_t so) __attribute__((always_inline)) {
        // LDS reads of K-step s (one per m-tile), two K-steps in flight; the
        // fold's reads go out under K-step 3
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
        // The two waves on a SIMD (one per K-half) leave each step's barrier
        // together; the one in its MFMA phase goes first, so the other's
        // fold tends to fall under those MFMAs (2-3% at 48-64 tokens).
        __builtin_amdgcn_s_setprio(1);
        rd(0, av[0]);
        rd(1, av[1]);
        // scales of sub-blocks 2kg (K-steps 0, 1) and 2kg + 1 (2, 3):
        // fields 2kg, 2kg+1 of the 96-bit word, bits 12kg ..
        const uint64_t f64 = (uint64_t)(uint32_t)R.hdr[1] | ((uint64_t)(uint32_t)R.hdr[2] << 32);
        const uint32_t x = (uint32_t)(f64 >> (12 * kg));
        v4i acc_h[MT], acc_l[MT];
        v4i ap[MT];
        v4f da[MT];
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            const uint32_t sc = (s < 2 ? x : x >> 6) & 63u;
            const v4i qw = (s & 1) ? R.q1 : R.q0;
            v4i bh, bl;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const uint32_t nib = s < 2 ? (uint32_t)qw[e] & 0x0F0F0F0Fu : ((uint32_t)qw[e] >> 4) & 0x0F0F0F0Fu;
                bh[e] = mul_digit(nib, sc >> 3);
                bl[e] = mul_digit(nib, sc & 7u);
            }
            // reads in flight behind m-tile t of K-step s: the rest of this
            // K-step's, then the next K-step's (MT) or, under K-step 3, the
            // fold's (2 MT)
            v4i(&cur)[MT] = av[s & 1];
            const int behind = s < 2 ? MT : (s == 2 ? MT : 2 * MT);
#pragma unroll
            for (int t = 0; t < MT; ++t) lds_wait_n(MT - 1 - t + behind, cur[t]);
#pragma unroll
            for (int t = 0; t < MT; ++t) {
                acc_h[t] = mma16_i8(cur[t], bh, s == 0 ? v4i{} : acc_h[t]);
                acc_l[t] = mma16_i8(cur[t], bl, s == 0 ? v4i{} : acc_l[t]);
            }
            if (s < 2) {
                rd(s + 2, av[s & 1]);
            } else if (s == 2) {
                // the fold's operands
#pragma unroll
                for (int t = 0; t < MT; ++t) {
                    switch (t) {
                        case 0: ap[t] = lds_read16<0>(l_ad + l_slot * so); break;
                        case 1: ap[t] = lds_read16<256>(l_ad + l_slot * so); break;
                        case 2: ap[t] = lds_read16<512>(l_ad + l_slot * so); break;
                        default: ap[t] = lds_read16<768>(l_ad + l_slot * so); break;
                    }
                }
#pragma unroll
                for (int t = 0; t < MT; ++t) da[t] = __builtin_bit_cast(v4f, lds_read16<0>(d_ad + so + 64 * t));
            }
        }
        __builtin_amdgcn_s_setprio(0);
        // fold: out += d_a[m] * (d[n] * float(8*acc_h + acc_l) - dmin[n] * M),
        // M = sum_j m_j B_j exact on one bf16 MFMA per m-tile (A row m =
        // both exact parts of B_0..B_7 in k-groups 0 and 1, k-groups 2 and 3
        // zero; B column n = m_0..m_7)
        const float dw = f16_bits_to_f32((uint32_t)R.hdr[0]);
        const float ndmin = -f16_bits_to_f32((uint32_t)R.hdr[0] >> 16);
        const uint64_t hi64 = (uint64_t)(uint32_t)R.hdr[2] | ((uint64_t)(uint32_t)R.hdr[3] << 32);
        const uint64_t mx = hi64 >> 16;  // mins m_j: bits 48 + 6j of the 96-bit word
        v8bf bm;
#pragma unroll
        for (int i = 0; i < 8; ++i) bm[i] = (__bf16)(float)(uint32_t)((mx >> (6 * i)) & 63u);
#pragma unroll
        for (int t = 0; t < MT; ++t) {
            lds_wait_n(2 * MT - 1 - t, ap[t]);
            lds_wait_n(MT - 1 - t, da[t]);
            const v4f mt = mma16_bf16(__builtin_bit_cast(v8bf, ap[t]), bm, v4f{});
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int Tq = (acc_h[t][i] << 3) + acc_l[t][i];
                out[t][i] = fmaf(fmaf((float)Tq, dw, mt[i] * ndmin), da[t][i], out[t][i]);
            }
        }
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
        const int sb = kh ? T + x : x;
        if (x < T && sb < nsb) compute(ring[k], (uint32_t)(k * C::SLOT));  // uniform
    };
#pragma unroll
    for (int x = 0; x < C::L; ++x) {
        copies(x);
        wload(x, ring[x]);
    }
    // Whole ring turns (every step issues the same loads, so the waits stay
    // partial), then the T mod S steps left over, which issue nothing: in
    // tail step j the loads of steps x .. nfull - 1 + L are outstanding,
    // L - j steps' worth, and step x's are the oldest.  (Padding T to whole
    // turns instead cost about half a step per padded step.)
    const int nfull = T / C::S * C::S;
    for (int x0 = 0; x0 < nfull; x0 += C::S)
        static_for<0, C::S>([&](auto KK) KQ_INLINE { step(KK, x0 + decltype(KK)::value); });
    auto tail_step = [&](auto JJ) KQ_INLINE {
        constexpr int j = decltype(JJ)::value;
        __builtin_amdgcn_sched_barrier(0);
        wait_vmcnt<C::LOADS * (C::L - 1 - j)>();
        barrier_nofence();
        __builtin_amdgcn_sched_barrier(0);
        const int sb = kh ? T + nfull + j : nfull + j;
        if (sb < nsb) compute(ring[j], (uint32_t)(j * C::SLOT));  // uniform
    };
    const int rem = T - nfull;
    static_for<1, C::S>([&](auto RR) KQ_INLINE {
        if (rem == decltype(RR)::value) static_for<0, decltype(RR)::value>(tail_step);
    });
    // the copies and loads past the end (reading nothing) drain; then the
    // second half's sums go through LDS to the first half's waves
    wait_vmcnt<0>();
    barrier_nofence();
    float *red = reinterpret_cast<float *>(s_lds);
    if (kh == 1) {
#pragma unroll
        for (int t = 0; t < MT; ++t)
#pragma unroll
            for (int i = 0; i < 4; ++i) red[((strip * MT + t) * 4 + i) * 64 + lane] = out[t][i];
    }
    barrier_nofence();
    if (kh == 0) {
        // rows past M fall outside the resource; columns past N are sent out
        // of range
        const int n = n0 + r16;
        const int voff = n < N ? (4 * kg * N + n) * 4 : OOB_VOFF;
#pragma unroll
        for (int t = 0; t < MT; ++t) {
            v4f sum;
#pragma unroll
            for (int i = 0; i < 4; ++i) sum[i] = out[t][i] + red[((strip * MT + t) * 4 + i) * 64 + lane];
            // (the whole vector is bit-cast: see the tile kernel's epilogue)
            const v4i bits = __builtin_bit_cast(v4i, sum);
#pragma unroll
            for (int i = 0; i < 4; ++i)
                __builtin_amdgcn_raw_buffer_store_b32(bits[i], rs_o, voff, (16 * t + i) * N * 4, 0);
        }
    }
}

// out[0, n) = 0 (the product over an empty K, or before the two K-parts of
// the tile kernel add into it); a kernel rather than a memset so that the
// call stays capturable in a graph.  out is 16-byte aligned: four floats per
// lane, the last lane's group cut at n.
__global__ __launch_bounds__(256) void zero_fill_kernel(float *out, int64_t n) {
    const int64_t i = 4 * ((int64_t)blockIdx.x * 256 + threadIdx.x);
    if (i + 4 <= n) {
        *reinterpret_cast<v4f *>(out + i) = v4f{0.f, 0.f, 0.f, 0.f};
    } else {
        for (int64_t j = i; j < n; ++j) out[j] = 0.0f;
    }
}
static unsigned zero_fill_blocks(int64_t n) { return (unsigned)((n + 1023) / 1024); }

}  // namespace q4w

// Compute units of the current device, cached per device (the persistent
// grids are sized from it).  Concurrent first calls may both query; they
// store the same value.
int num_cus() {
    constexpr int MAX_DEV = 64;
    static std::atomic<int> cache[MAX_DEV];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 256;
    if (dev < MAX_DEV) {
        const int c = cache[dev].load(std::memory_order_relaxed);
        if (c > 0) return c;
    }
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
        cus = 256;
    if (dev < MAX_DEV) cache[dev].store(cus, std::memory_order_relaxed);
    return cus;
}

static int mv_tokens(int M) { return M <= 1 ? 1 : 2; }
constexpr int MV_LDS_BUDGET = 40 * 1024;  // four workgroups (16 waves) per CU

// Which Q4_K kernel a shape gets: one or two tokens -> the matrix-vector
// kernel; up to 64 -> a ring kernel or, on mid-width weights up to 16
// tokens, the four-wave K-split kernel (the rules below); otherwise the
// persistent tile kernel (two workgroups per CU), 128 x 128 when that tiling
// has more tiles than the chip has CUs (256), else 64 x 128: below that the
// taller tile leaves CUs idle, above it the shorter tile's extra unpacking
// (twice the weight work per output) and tail cost more than they gain.
constexpr int TILE64_MAX_TILES128 = 256;
// Persistent grids: two 4-wave workgroups per CU (KS = 1) or one 8-wave
// workgroup per CU that works on two superblocks at a time (KS = 2), which
// finishes a tile in about half the time.  The tiles are dealt in rounds of
// one tile per workgroup; the last round may be partly empty.  In units of
// one KS = 1 tile time, KS = 1 takes ceil(tiles / 2c) and KS = 2 takes
// ceil(tiles / c) / 2 for c CUs: KS = 2 wins when the tile count leaves the
// last KS = 1 round at most half full.  Measured for the 64-row tile on
// K = 4096: 512 x 4096 (256 tiles) 27.3 against 32.4 us, 200 x 4096 22.8
// against 27.4 us; 1024 x 4096 and 256 x 14336 (448-512 tiles) keep KS = 1
// (43.8 / 45.8 us against 50.3 / 52.5).  The 128-row tile at KS = 2 needs
// more than 256 VGPRs per lane and spills: it ran 420 against 308 us on
// 2048 x 14336, so that tile height keeps KS = 1 everywhere.
static bool split_pays(int64_t tiles, int cus) {
    const int64_t r1 = (tiles + 2 * cus - 1) / (2 * cus), r2 = (tiles + cus - 1) / cus;
    return r2 < 2 * r1;
}
int q4k_kernel_choice(int M, int N, int K) {
    if (M <= q4w::mv::MAX_TOKENS && K % 2048 == 0 && K <= (1 << 20) &&
        q4w::mv::lds_bytes(mv_tokens(M), M, K, K / 256) <= MV_LDS_BUDGET)
        return Q4K_MATVEC;
    const int cus = num_cus();
    // The K-split ring kernel (one 64-row workgroup per CU) once the 32-row
    // workgroups of the split and (former) two-wave kernels would need a
    // second round on some CUs: those kernels jump by a quarter to a half
    // there, and the ring kernel wins from that point on.  K = 4096, us, ring against the
    // other: 9216 rows 10.0 / 11.0 at 3 tokens, 10.8 / 13.0 at 16, 11.6 /
    // 14.6 at 32, 15.6 / 17.7 at 64; 14336 rows 11.2 / 13.6 at 16, 16.5 /
    // 19.9 at 64; K = 2048 and 8192 alike (8448-10240 rows: 5-25% faster).
    // At 8192 rows (one round) the other kernels win: 9.8 / 7.5 at 3 tokens,
    // 15.4 / 14.3 at 64.
    if (M <= 64 && ((int64_t)N + 31) / 32 > cus) return Q4K_FEW_RING;
    // Narrower weights: the four-wave split kernel up to 16 tokens while its
    // 32-row workgroups cover more than half the CUs, else the ring kernel
    // with K in 2, 4 or 8 parts (kq_gemm_ring.hip).  Paired runs, us, split
    // / ring: 8192 x 4096 at 16 tokens 8.1 / 9.2, 5120 x 4096 7.5 / 8.7,
    // 4096 x 4096 7.3 / 5.8, 4096 x 14336 at 3 tokens 17.1 / 12.1.  From 17
    // tokens the ring kernel beat the former two-wave kernel at every width
    // measured (8192 x 4096: 9.2 / 11.1 at 17 tokens, 12.6 / 14.1 at 64;
    // 4096 x 14336: 18.0 / 31.9 at 32 tokens, 32.2 / 41.3 at 64).  Past 64
    // tokens, the ring kernel in 64-token slices where the tile kernels
    // would leave most CUs idle (4096 x 14336 at 128 tokens: 33 against 77
    // us).
    if (M <= 16 && 2 * (((int64_t)N + 31) / 32) > cus) return Q4K_FEW_SPLIT;
    if (M <= 64 || ring_slices_pay(1, M, N, K)) return Q4K_RING_KP;
    const int64_t tiles128 = (((int64_t)M + 127) / 128) * (((int64_t)N + 127) / 128);
    if (tiles128 > TILE64_MAX_TILES128) return Q4K_TILE128;
    const int64_t tiles64 = (((int64_t)M + 63) / 64) * (((int64_t)N + 127) / 128);
    return split_pays(tiles64, cus) ? Q4K_TILE64_K2 : Q4K_TILE64;
}

hipError_t launch_zero_fill(float *out, int64_t n, hipStream_t stream) {
    if (n <= 0) return hipSuccess;
    hipLaunchKernelGGL(q4w::zero_fill_kernel, dim3(q4w::zero_fill_blocks(n)), dim3(256), 0, stream, out, n);
    return hipGetLastError();
}

bool q4k_id_tile_ok(int N, int K) {
    // per-tile output offsets (64 rows of N floats) stay below 2^31
    (void)K;
    return (int64_t)64 * N * 4 < ((int64_t)1 << 31);
}

hipError_t launch_gemm_q4k_id(const void *W, int n_experts, int64_t expert_bytes, const int8_t *qs,
                              const float *da, const uint16_t *alpha, const int32_t *exp_off,
                              const int32_t *rows, int R, float *out, int M, int N, int K,
                              hipStream_t stream) {
    const int cus = num_cus();
    if (K == 0) {
        const int64_t n = (int64_t)R * N;
        hipLaunchKernelGGL(q4w::zero_fill_kernel, dim3(q4w::zero_fill_blocks(n)), dim3(256), 0,
                           stream, out, n);
        return hipGetLastError();
    }
    q4w::Args a;
    a.W = static_cast<const uint8_t *>(W);
    a.qs = qs;
    a.da = da;
    a.alpha = alpha;
    a.out = out;
    a.M = M;
    a.N = N;
    a.K = K;
    a.nsb = K / 256;
    // upper bound on the M-tiles: each expert's count rounded up to 64 rows
    a.tiles_m = (R + 63) / 64 + n_experts;
    a.tiles_n = (N + q4w::BN - 1) / q4w::BN;
    a.ntiles = a.tiles_m * a.tiles_n;
    a.exp_off = exp_off;
    a.rows = rows;
    a.n_experts = n_experts;
    a.n_routed = R;
    a.expert_bytes = expert_bytes;
    const unsigned grid = (unsigned)min(a.ntiles, q4w::TileCfg<64>::WG_PER_CU * cus);
    hipLaunchKernelGGL((q4w::gemm_q4k_kernel<64, true>), dim3(grid), dim3(q4w::NT), 0, stream, a);
    return hipGetLastError();
}

hipError_t launch_gemm_q4k(const void *W, const int8_t *qs, const float *da,
                           const uint16_t *alpha, float *out, int M, int N, int K,
                           hipStream_t stream) {
    const int cus = num_cus();
    if (K == 0) {
        const int64_t n = (int64_t)M * N;
        hipLaunchKernelGGL(q4w::zero_fill_kernel, dim3(q4w::zero_fill_blocks(n)), dim3(256), 0,
                           stream, out, n);
        return hipGetLastError();
    }
    q4w::Args a;
    a.W = static_cast<const uint8_t *>(W);
    a.qs = qs;
    a.da = da;
    a.alpha = alpha;
    a.out = out;
    a.M = M;
    a.N = N;
    a.K = K;
    a.nsb = K / 256;
    const int choice = q4k_kernel_choice(M, N, K);
    const int bm = (choice == Q4K_TILE64 || choice == Q4K_TILE64_K2) ? 64 : 128;
    a.tiles_m = (M + bm - 1) / bm;
    a.tiles_n = (N + q4w::BN - 1) / q4w::BN;
    a.ntiles = a.tiles_m * a.tiles_n;
    switch (choice) {
        case Q4K_MATVEC: {
            const dim3 grid((unsigned)((N + q4w::mv::RPG - 1) / q4w::mv::RPG)), block(64 * q4w::mv::NW);
            const int mt = mv_tokens(M);
            const size_t lds = (size_t)q4w::mv::lds_bytes(mt, M, K, a.nsb);
            const bool deep = q4w::mv::depth_for(a.nsb / 8) == 2;
            switch (mt) {
                case 1:
                    if (deep) hipLaunchKernelGGL((q4w::gemv_q4k_kernel<1, 2>), grid, block, lds, stream, a);
                    else hipLaunchKernelGGL((q4w::gemv_q4k_kernel<1, 1>), grid, block, lds, stream, a);
                    break;
                default:
                    if (deep) hipLaunchKernelGGL((q4w::gemv_q4k_kernel<2, 2>), grid, block, lds, stream, a);
                    else hipLaunchKernelGGL((q4w::gemv_q4k_kernel<2, 1>), grid, block, lds, stream, a);
                    break;
            }
            break;
        }
        case Q4K_FEW_SPLIT:
            hipLaunchKernelGGL((q4w::gemm_q4k_split_kernel<1, 4, 2>), dim3((unsigned)((N + 31) / 32)), dim3(64 * 4),
                               0, stream, a);
            break;
        case Q4K_RING_KP:
            return launch_gemm_ring(1, W, qs, da, alpha, out, M, N, K, stream);
        case Q4K_FEW_RING:
            if (M <= 16)
                hipLaunchKernelGGL(q4w::gemm_q4k_ring_kernel<16>, dim3((unsigned)((N + 63) / 64)), dim3(512), 0,
                                   stream, a);
            else if (M <= 32)
                hipLaunchKernelGGL(q4w::gemm_q4k_ring_kernel<32>, dim3((unsigned)((N + 63) / 64)), dim3(512), 0,
                                   stream, a);
            else
                hipLaunchKernelGGL(q4w::gemm_q4k_ring_kernel<64>, dim3((unsigned)((N + 63) / 64)), dim3(512), 0,
                                   stream, a);
            break;
        case Q4K_TILE64: {
            const unsigned grid = (unsigned)min(a.ntiles, q4w::TileCfg<64>::WG_PER_CU * cus);
            hipLaunchKernelGGL(q4w::gemm_q4k_kernel<64>, dim3(grid), dim3(q4w::NT), 0, stream, a);
            break;
        }
        case Q4K_TILE64_K2: {
            const unsigned grid = (unsigned)min(a.ntiles, cus);
            hipLaunchKernelGGL((q4w::gemm_q4k_kernel<64, false, 2>), dim3(grid), dim3(2 * q4w::NT), 0, stream, a);
            break;
        }

        default: {
            const unsigned grid = (unsigned)min(a.ntiles, q4w::TileCfg<128>::WG_PER_CU * cus);
            hipLaunchKernelGGL(q4w::gemm_q4k_kernel<128>, dim3(grid), dim3(q4w::NT), 0, stream, a);
            break;
        }
    }
    return hipGetLastError();
}

}  // namespace kq
