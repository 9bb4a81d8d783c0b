// kq_gemm_tq.hip -- ternary (base-3, five trits per byte) x Q8_128 products
// on a persistent tile kernel that unpacks the weights in registers.
//
// out[m][n] = sum_b d_a[b][m] * d_w[n][b] * sum_{k in block b} t[n][k] * qs[m][k]
// for 128-value blocks b (llama.cpp PR 214: a 26-byte base-3 trit array and
// an fp16 scale per 128 weights; the activations carry one fp32 scale per 128
// values).  The integer sums run on v_mfma_i32_32x32x32_i8, one MFMA per
// algorithmic one (trits are int8 operands as they are); each block's sums
// are folded into the fp32 output as soon as its four K-steps are done.
// The fold, out += float(sum) * s with s = d_a[m] * d_w[n], costs two VALU
// operations per output: s comes for a whole 32 x 32 tile from one bf16
// MFMA, with d_a split exactly into three bf16 parts (staged once per
// workgroup) and d_w into two, so the six part products and their sum are
// d_a * d_w to within an ulp or two (exactly so for unit scales).
//
// Structure (the Q4_K tile kernel's, see kq_gemm_q4k.hip): persistent
// workgroups of 4 waves, two per CU, each owning 128 x 128 output tiles in
// turn; per step of 256 values (two blocks) the workgroup stages one copy of
// the activation tile (and the two blocks' activation scales) in LDS with
// buffer -> LDS copies, one step ahead, and every wave reads its fragments
// from it.  Wave w owns the 32 weight columns 32w .. 32w+31 of the tile, all
// four 32-row m-tiles, and loads its weight bytes straight into registers,
// one step ahead.  Compared with the generic tile kernel (kq_gemm.hip), which
// unpacks each chunk once per workgroup into LDS digit planes that every wave
// then re-reads, this drops the plane writes and half the fragment reads, and
// one barrier covers 256 values instead of 128.
//
// K order of a block: lane group g takes the 64 values 64g .. 64g+63, 16 per
// K-step s (values 64g + 16s + i), so each lane decodes trits from its own
// half of the block: bytes 0..15 (g = 0) or 12..27 (g = 1, which also holds
// the scale).  The 16 trits of a K-step start at trit k0 = 64g + 16s, i.e.
// at digit o = k0 mod 5 of byte k0 / 5, and span four bytes.  Each byte goes
// through a 256-entry LDS table (five int8 trits per byte value); the four
// 5-trit groups are packed into 20 consecutive bytes and the 16 wanted ones
// taken from offset o.
#include "kq_device.hpp"
#include "kq_hooks.hpp"
#include "kq_launch.hpp"
#include "kq_tile.hpp"

#include <type_traits>

namespace kq {
namespace tqt {
using namespace tl;

constexpr int BM = 128, BN = 128, NWAVE = 4, NT = 64 * NWAVE, MT = BM / 32;
constexpr int TB = 28;            // bytes per 128-weight block
constexpr int ROW = 256;          // staged activation bytes per row and step (two blocks)
constexpr int ABUF = BM * ROW;    // staged activation values of one step
constexpr int DBUF = 2 * BM;      // staged activation scales: [block of the step][row]
constexpr int PBUF = 2 * BM * 4;  // their bf16 parts as MFMA operands: [block][row][4 dwords]
constexpr int WG_PER_CU = 2;

struct Args {
    const uint8_t *W;
    const int8_t *qs;
    const float *da;  // [K/128][M]
    float *out;
    int M, N, K, nblk, nst, tiles_m, tiles_n, ntiles;
};

// Tile t of the grouped order: GM M-tiles down, then across N.
struct TileXY {
    int m0, n0;
};
__device__ __forceinline__ TileXY tile_xy(const Args &a, int t) {
    constexpr int GM = 4;
    const int per_group = GM * a.tiles_n;
    const int first_m = (t / per_group) * GM;
    // (at least 1: the look-ahead tile of a workgroup's last tile may lie
    // past the list; its coordinates are then never used)
    const int gsize = max(min(a.tiles_m - first_m, GM), 1);
    const int r = t % per_group;
    return {(first_m + r % gsize) * BM, (r / gsize) * BN};
}

struct Slot {
    int8_t *a;     // [BM rows][256]: 16-byte piece p of row r at ((p ^ (r % 16)) * 16)
    float *d;      // [2][BM] activation scales, staged two steps ahead
    uint32_t *p;   // [2][BM][4]: bf16 parts of those scales, formed one step ahead
};

// This lane's weights for one step: per block, 16 trit bytes of its half and
// the dword holding the block's scale (bytes 24..27: two trit bytes, fp16 d).
struct WRaw {
    v4i q[2];
    uint32_t dw[2];
};

__global__ __launch_bounds__(NT, WG_PER_CU) void gemm_tq_tile_kernel(Args a) {
    __shared__ __attribute__((aligned(16))) int8_t s_a0[ABUF], s_a1[ABUF];
    __shared__ __attribute__((aligned(16))) float s_d0[DBUF], s_d1[DBUF];
    __shared__ __attribute__((aligned(16))) uint32_t s_p0[PBUF], s_p1[PBUF];
    __shared__ __attribute__((aligned(16))) uint32_t s_lut[2 * 256];
    const Slot slots[2] = {{s_a0, s_d0, s_p0}, {s_a1, s_d1, s_p1}};

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int ln = lane & 31, g = lane >> 5;
    const int M = a.M, N = a.N, K = a.K, nst = a.nst;

    // decode table: entry v = the five trits of byte v (t0..t3 in the low
    // word, t4 in the high word); visible to every wave after the first
    // iteration's barrier
    {
        uint32_t lo, hi;
        tq_lut_entry((uint32_t)tid, lo, hi);
        s_lut[2 * tid] = lo;
        s_lut[2 * tid + 1] = hi;
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    }

    // ---- persistent tile list (as in the Q4_K tile kernel) ------------------
    // Workgroups are dealt round-robin to the 8 XCDs; at step k the grid
    // covers grouped-order tiles [k*G, (k+1)*G) and the workgroups of one XCD
    // take a contiguous run of them.
    const int G = gridDim.x, b = blockIdx.x;
    const int per_xcd = G >> 3;
    const int slot_in_step = (per_xcd > 0 && b < 8 * per_xcd) ? ((b & 7) * per_xcd + (b >> 3)) : b;
    const int my_tiles = (a.ntiles - slot_in_step + G - 1) / G;
    const int total = my_tiles * nst;  // flat iterations
    const int rowbytes = a.nblk * TB;
    if (total <= 0) return;  // uniform: no barrier is ever reached

    // Buffer resources over whole tensors: reads past the last activation or
    // weight row return zero, stores past the last output row are dropped
    // (every offset stays under 2^31, checked on the host).
    const auto rs_a = __builtin_amdgcn_make_buffer_rsrc((void *)a.qs, (short)0, M * K, RSRC_FLAGS);
    const auto rs_d = __builtin_amdgcn_make_buffer_rsrc((void *)a.da, (short)0, a.nblk * M * 4, RSRC_FLAGS);
    const auto rs_w = __builtin_amdgcn_make_buffer_rsrc((void *)a.W, (short)0, N * rowbytes, RSRC_FLAGS);
    const auto rs_o = __builtin_amdgcn_make_buffer_rsrc((void *)a.out, (short)0, M * N * 4, RSRC_FLAGS);

    // ---- staging: buffer -> LDS copies ---------------------------------------
    // Values of a step, one step ahead: 1 KiB copy c holds rows 4c..4c+3, lane
    // l filling position l%16 of row 4c + l/16 with piece (l%16) ^ (row%16);
    // wave w copies c = 8w .. 8w+7.  Scales of a step, two steps ahead (their
    // bf16 parts are formed the step in between): wave 0, lanes 0..31 the
    // first block's 128 rows, lanes 32..63 the second's, four rows per lane.
    const int st_row = lane >> 4, st_pos = lane & 15;
    constexpr int CPW = BM / 16;  // value copies per wave
    const int a_vbase = ((BM / 4) * wave + st_row) * K + 16 * (st_pos ^ st_row);
    const int d_voff = (g * M + 4 * ln) * 4;
    auto stage = [&](const Slot &S, TileXY T, int st) {
#pragma unroll
        for (int i = 0; i < CPW; ++i)
            copy16(rs_a, S.a + (CPW * wave + i) * 1024, a_vbase ^ (64 * (i & 3)),
                   (T.m0 + 4 * (i & 3) + 16 * (i >> 2)) * K + st * ROW);
    };
    auto stage_d = [&](float *D, TileXY T, int st) {
        if (wave == 0) copy16(rs_d, D, d_voff, (2 * st * M + T.m0) * 4);
    };
    // Parts of the staged scales (wave w: rows 32w .. 32w+31 of both blocks,
    // one per lane): x = h + m + l with h = x with its low 16 bits cleared, m
    // the same of x - h, l = x - h - m; each has at most 8 significant bits,
    // so it is exact in bf16 and the subtractions are exact.  Stored as the
    // A operand row [h, h, m, m, l, l, 0, 0] of the scale MFMA.
    auto make_parts = [&](const float *D, uint32_t *Pp) {
        const int bb = lane >> 5, r = 32 * wave + ln;
        const uint32_t x = __builtin_bit_cast(uint32_t, D[bb * BM + r]);
        const uint32_t h = x & 0xFFFF0000u;
        const float x1 = __builtin_bit_cast(float, x) - __builtin_bit_cast(float, h);
        const uint32_t m = __builtin_bit_cast(uint32_t, x1) & 0xFFFF0000u;
        const uint32_t l = __builtin_bit_cast(uint32_t, x1 - __builtin_bit_cast(float, m)) & 0xFFFF0000u;
        *reinterpret_cast<v4i *>(Pp + (bb * BM + r) * 4) =
            v4i{(int)(h | (h >> 16)), (int)(m | (m >> 16)), (int)(l | (l >> 16)), 0};
    };
    // flat iteration j's tile and step (for the scales two steps ahead)
    auto tile_of = [&](int j) { return tile_xy(a, slot_in_step + (j / nst) * G); };

    // ---- weights of this lane: row n0 + 32*wave + ln, straight to registers --
    const int w_row = (32 * wave + ln) * rowbytes;
    const int w_q = w_row + 12 * g, w_d = w_row + 24;
    auto load_w = [&](TileXY T, int st, WRaw &R) {
        const int so = T.n0 * rowbytes + st * (2 * TB);
#pragma unroll
        for (int bb = 0; bb < 2; ++bb) {
            R.q[bb] = ld16(rs_w, w_q, so + bb * TB);
            R.dw[bb] = __builtin_amdgcn_raw_buffer_load_b32(rs_w, w_d, so + bb * TB, 0);
        }
    };

    // ---- fragment addressing: lane (ln, g), block bb, K-step s reads piece
    // p = 8bb + 4g + s of row 32t + ln; p ^ (row % 16) = (8bb + s) ^ L with
    // L = 4g ^ (ln % 16) (the three terms of p occupy disjoint bits)
    const int Lx = (4 * g) ^ (ln & 15);
    int foff[2][4];
#pragma unroll
    for (int bb = 0; bb < 2; ++bb)
#pragma unroll
        for (int s = 0; s < 4; ++s) foff[bb][s] = ln * ROW + (((8 * bb + s) ^ Lx) << 4);
    // decode constants: byte shifts of the K-step's first trit byte within
    // the lane's 16 bytes, and the digit offset o of its first trit
    const bool hi_half = g != 0;
    const uint32_t sh1 = hi_half ? 0u : 3u, sh2 = hi_half ? 3u : 2u, sh3 = hi_half ? 2u : 1u;
    const uint32_t o1 = hi_half ? 0u : 1u, o2 = hi_half ? 1u : 2u, o3 = hi_half ? 2u : 3u;
    const uint32_t lo_mask = hi_half ? 0u : ~0u;  // the scale MFMA's B operand: k-group 0 only

    // the 16 trits of K-step s of block bb as an int8 MFMA operand
    auto decode = [&](const v4i &q, int s) __attribute__((always_inline)) {
        const uint32_t q0 = (uint32_t)q[0], q1 = (uint32_t)q[1], q2 = (uint32_t)q[2], q3 = (uint32_t)q[3];
        uint32_t x;
        if (s == 0)
            x = q0;
        else if (s == 1)
            x = __builtin_amdgcn_alignbyte(hi_half ? q2 : q1, hi_half ? q1 : q0, sh1);
        else if (s == 2)
            x = __builtin_amdgcn_alignbyte(q2, q1, sh2);
        else
            x = __builtin_amdgcn_alignbyte(q3, q2, sh3);
        v2u e[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) e[i] = *reinterpret_cast<const v2u *>(&s_lut[2 * ((x >> (8 * i)) & 0xFFu)]);
        // 20 trits in order: D0 = t0..3, D1 = t4..7, D2 = t8..11, D3 = t12..15, D4 = t16..19
        uint32_t D[5];
        D[0] = e[0].x;
        D[1] = perm_b32(e[1].x, e[0].y, 0x06050400u);
        D[2] = __builtin_amdgcn_alignbyte(e[1].y, e[1].x, 3) | (e[2].x << 16);
        D[3] = __builtin_amdgcn_alignbyte(e[2].y, e[2].x, 2) | (e[3].x << 24);
        D[4] = __builtin_amdgcn_alignbyte(e[3].y, e[3].x, 1);
        v4i bq;
        if (s == 0) {
            // o = 0 (low half) or 4 (high half: the group starts one dword on)
#pragma unroll
            for (int j = 0; j < 4; ++j) bq[j] = (int)(hi_half ? D[j + 1] : D[j]);
        } else {
            const uint32_t o = s == 1 ? o1 : s == 2 ? o2 : o3;
#pragma unroll
            for (int j = 0; j < 4; ++j) bq[j] = (int)__builtin_amdgcn_alignbyte(D[j + 1], D[j], o);
        }
        return bq;
    };

    v16i acc[MT];
    v16f out[MT];
#pragma unroll
    for (int t = 0; t < MT; ++t) out[t] = v16f{};

    WRaw wring[2];  // weights of iterations with slot parity 0 / 1

    int k = 0, st = 0;
    TileXY T = tile_xy(a, slot_in_step);
    TileXY TN = tile_xy(a, slot_in_step + G);

    auto iteration = [&](auto PP, int it) {
        constexpr int P = decltype(PP)::value;
        const Slot &S = slots[P];
        // everything this wave copied or loaded for iteration it has landed;
        // after the barrier, so has every other wave's, and every read of the
        // other slot (iteration it-1) is done
        wait_vmcnt<0>();
        barrier_nofence();
        const bool more = it + 1 < total;
        const bool last = st + 1 == nst;
        const TileXY Tn = last ? TN : T;
        const int stn = last ? 0 : st + 1;
        const WRaw &wc = wring[P];
        __builtin_amdgcn_sched_barrier(0);
        if (more) {
            stage(slots[1 - P], Tn, stn);
            load_w(Tn, stn, wring[1 - P]);
            // the scales of iteration it+2 into this slot (this iteration's
            // were turned into parts one iteration ago)
            if (it + 2 < total) stage_d(slots[P].d, tile_of(it + 2), (it + 2) % nst);
            // the parts of iteration it+1's scales (landed before the barrier)
            make_parts(slots[1 - P].d, slots[1 - P].p);
        }
        __builtin_amdgcn_sched_barrier(0);
        __builtin_amdgcn_s_setprio(2);
#pragma unroll
        for (int bb = 0; bb < 2; ++bb) {
            // the fragments of K-step s+1 are read while K-step s multiplies
            v4i av[2][MT];
#pragma unroll
            for (int t = 0; t < MT; ++t)
                av[0][t] = *reinterpret_cast<const v4i *>(S.a + t * 32 * ROW + foff[bb][0]);
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                __builtin_amdgcn_sched_barrier(0);
                if (s + 1 < 4) {
#pragma unroll
                    for (int t = 0; t < MT; ++t)
                        av[(s + 1) & 1][t] = *reinterpret_cast<const v4i *>(S.a + t * 32 * ROW + foff[bb][s + 1]);
                }
                __builtin_amdgcn_sched_barrier(0);
                const v4i bq = decode(wc.q[bb], s);
#pragma unroll
                for (int t = 0; t < MT; ++t)
                    acc[t] = s == 0 ? mma_i8(av[s & 1][t], bq, v16i{}) : mma_i8(av[s & 1][t], bq, acc[t]);
            }
            // fold block bb: out += float(sum) * s, s = d_a[m] * d_w[n] from one
            // bf16 MFMA per m-tile: A row m = parts of d_a[m] (k-group 0),
            // B column n = [q0, q1] x 3 with d_w[n] = q0 + q1 (q0 = d_w with its
            // low 16 bits cleared; d_w has 11 significant bits, so q1 has at
            // most 3) in k-group 0, zero in k-group 1
            // (masked per lane: a branch or a select on the lane group here
            // made the register allocator spill)
            v4i bw;
            {
                const uint32_t f = __builtin_bit_cast(uint32_t, f16_bits_to_f32(wc.dw[bb] >> 16));
                const uint32_t q0 = f & 0xFFFF0000u;
                const uint32_t q1 = __builtin_bit_cast(
                    uint32_t, __builtin_bit_cast(float, f) - __builtin_bit_cast(float, q0));
                const int pair = (int)(((q0 >> 16) | (q1 & 0xFFFF0000u)) & lo_mask);
                bw = v4i{pair, pair, pair, 0};
            }
#pragma unroll
            for (int t = 0; t < MT; ++t) {
                const v4i ap = *reinterpret_cast<const v4i *>(S.p + (bb * BM + 32 * t + ln) * 4);
                const v16f sc = mma_bf16(__builtin_bit_cast(v8bf, ap), __builtin_bit_cast(v8bf, bw), v16f{});
#pragma unroll
                for (int r = 0; r < 16; ++r) out[t][r] = fmaf((float)acc[t][r], sc[r], out[t][r]);
            }
        }
        __builtin_amdgcn_s_setprio(0);

        if (last) {
            // epilogue of tile T: rows past M fall outside the resource and
            // are dropped; columns past N are sent out of range
            const int n = T.n0 + 32 * wave + ln;
            const int voff = n < N ? (4 * g * N + n) * 4 : OOB_VOFF;
#pragma unroll
            for (int t = 0; t < MT; ++t) {
                // cast the whole vector: storing a bit-cast of one element
                // directly miscompiles to a store of element 0 (ROCm 7.2 clang)
                const v16i bits = __builtin_bit_cast(v16i, out[t]);
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int row = 32 * t + 8 * (r >> 2) + (r & 3);  // minus the lane's 4g
                    __builtin_amdgcn_raw_buffer_store_b32(bits[r], rs_o, voff, (T.m0 + row) * N * 4, 0);
                }
            }
#pragma unroll
            for (int t = 0; t < MT; ++t) out[t] = v16f{};
            ++k;
            st = 0;
            T = TN;
            TN = tile_xy(a, slot_in_step + (k + 1) * G);
        } else {
            ++st;
        }
    };

    // prologue: stage iteration 0, its weights, the scales of iterations 0
    // and 1, and the parts of iteration 0's (visible after the first barrier)
    stage(slots[0], T, 0);
    load_w(T, 0, wring[0]);
    stage_d(slots[0].d, T, 0);
    if (total > 1) stage_d(slots[1].d, tile_of(1), 1 % nst);
    wait_vmcnt<0>();
    barrier_nofence();
    make_parts(slots[0].d, slots[0].p);
    for (int it = 0; it < total; it += 2) {
        iteration(std::integral_constant<int, 0>{}, it);
        if (it + 1 < total) iteration(std::integral_constant<int, 1>{}, it + 1);
    }
}

}  // namespace tqt

bool tq_tile_choice(int M, int N, int K) {
    // two blocks per step; the matrix-vector kernel keeps what it takes; the
    // (tile, step) count of a workgroup is an int.  With fewer tiles than CUs
    // the digit-plane kernel's eight waves per tile win (200 x 4096 x 5120:
    // 43 against 48 us).
    if (M <= 0 || N <= 0 || K <= 0 || K % 256 != 0 || gemv_choice(3, M, N, K)) return false;
    const int64_t tiles = (((int64_t)M + tqt::BM - 1) / tqt::BM) * (((int64_t)N + tqt::BN - 1) / tqt::BN);
    return tiles >= num_cus() && tiles * (K / 256) <= INT32_MAX;
}

hipError_t launch_gemm_tq_tile(const void *W, const int8_t *qs, const float *da, float *out, int M, int N,
                               int K, hipStream_t stream) {
    tqt::Args a;
    a.W = static_cast<const uint8_t *>(W);
    a.qs = qs;
    a.da = da;
    a.out = out;
    a.M = M;
    a.N = N;
    a.K = K;
    a.nblk = K / 128;
    a.nst = K / 256;
    a.tiles_m = (M + tqt::BM - 1) / tqt::BM;
    a.tiles_n = (N + tqt::BN - 1) / tqt::BN;
    a.ntiles = a.tiles_m * a.tiles_n;
    const unsigned grid = (unsigned)min(a.ntiles, tqt::WG_PER_CU * num_cus());
    hipLaunchKernelGGL(tqt::gemm_tq_tile_kernel, dim3(grid), dim3(tqt::NT), 0, stream, a);
    return hipGetLastError();
}

}  // namespace kq
