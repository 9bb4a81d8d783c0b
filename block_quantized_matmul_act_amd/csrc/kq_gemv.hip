// kq_gemv.hip -- matrix-vector kernels for Q6_K and ternary weights (a
// handful of tokens, decode).
//
// A token's product with a weight row is a stream of the row's blocks: a
// handful of tokens need many waves with loads in flight, not matrix cores.
// Workgroups of 4 waves own 8 weight rows (2 per wave); the tokens'
// activation values and scales are copied once per workgroup into LDS.  A
// load instruction covers 8 consecutive superblocks of one row, one 32-value
// piece per lane; each wave keeps one instruction per row in flight and walks
// its rows in turn (two rows per wave beat one and four: 12.5 against 13.1
// and 16.3 us for one token on 4096 x 14336).  Every lane keeps its rows'
// sums in registers, and one butterfly over the 64 lanes at the end (a fixed
// order) gives each row's total, which lane 0 stores.  Integer sums come from
// v_dot4_i32_i8 and are folded per 16-value sub-block with the block scales.
#include "kq_device.hpp"
#include "kq_launch.hpp"

namespace kq {
namespace gv {

constexpr int NW = 4;          // waves per workgroup
#ifndef GV_RPW
#define GV_RPW 2
#endif
constexpr int RPW = GV_RPW;    // weight rows per wave
constexpr int RPG = NW * RPW;  // weight rows per workgroup
constexpr int RSRC_FLAGS = 0x00020000;
constexpr int Q6B = 210;       // Q6_K block bytes
// staged activations: values of MT tokens, then the scales (1 KiB multiple so
// the last 256-byte scale copy stays inside)
__host__ __device__ constexpr int lds_qs(int MT, int K) { return MT * K; }
__host__ __device__ constexpr int lds_d(int M, int nsb) { return (nsb * M * 4 + 1023) / 1024 * 1024; }
__host__ __device__ constexpr int lds_bytes(int MT, int M, int K) {
    return lds_qs(MT, K) + lds_d(M, K / 256) + 256;  // + room for reads of token rows past M
}
constexpr int LDS_BUDGET = 120 * 1024;  // one workgroup per CU at most

typedef __attribute__((address_space(3))) void *lds_ptr_t;

struct Args {
    const uint8_t *W;
    const int8_t *qs;  // [M][K]
    const float *da;   // [K/256][M]
    float *out;        // [M][N]
    int M, N, K;
};

__device__ __forceinline__ void copy16(__amdgpu_buffer_rsrc_t rs, void *lds, int voff) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_ptr_t)lds, 16, voff, 0, 0, 0);
}
__device__ __forceinline__ void copy4(__amdgpu_buffer_rsrc_t rs, void *lds, int voff) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_ptr_t)lds, 4, voff, 0, 0, 0);
}
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}
__device__ __forceinline__ uint32_t ld4(__amdgpu_buffer_rsrc_t rs, int voff) {
    return __builtin_amdgcn_raw_buffer_load_b32(rs, voff, 0, 0);
}
__device__ __forceinline__ v4i ld16(__amdgpu_buffer_rsrc_t rs, int voff) {
    return __builtin_bit_cast(v4i, __builtin_amdgcn_raw_buffer_load_b128(rs, voff, 0, 0));
}

// Stage the activations of a workgroup (values [M][K], scales [K/256][M]).
// The 16-byte pieces of odd superblocks are stored with their index's low bit
// flipped, which puts the two superblocks a read instruction touches on
// different banks.
__device__ __forceinline__ void stage_acts(const Args &a, int8_t *s_qs, float *s_d, int w, int lane) {
    const int M = a.M, K = a.K, nsb = K / 256;
    const auto rs_a = __builtin_amdgcn_make_buffer_rsrc((void *)a.qs, (short)0, M * K, RSRC_FLAGS);
    const auto rs_d = __builtin_amdgcn_make_buffer_rsrc((void *)a.da, (short)0, nsb * M * 4, RSRC_FLAGS);
    const int nq = (M * K) >> 10, nd = (nsb * M * 4 + 255) >> 8;
    const int aq = 16 * (lane ^ ((lane >> 4) & 1));
    for (int c = w; c < nq; c += NW) copy16(rs_a, s_qs + 1024 * c, 1024 * c + aq);
    for (int c = w; c < nd; c += NW) copy4(rs_d, reinterpret_cast<int8_t *>(s_d) + 256 * c, 256 * c + 4 * lane);
}

// ---------------------------------------------------------------------------
// Q6_K.  Lane l of a load instruction takes superblock l/8 of the instruction's
// eight and, within it, the 32 values 128h + 32u + t (t < 32) with h = (l%8)/4,
// u = l%4: low 4 bits from ql[64h + 32(u%2) + t] (low nibble for u < 2, high
// for u >= 2), high 2 bits from bits 2u of qh[32h + t], sub-blocks 8h + 2u
// and 8h + 2u + 1.  Blocks are 210 bytes, so a block is 2-byte aligned: the
// lane loads whole aligned dwords and shifts them into place with v_alignbit.
// q - 32 is formed per byte without borrows: (q | 0x80) - 0x20, then bit 7
// flipped back.
// ---------------------------------------------------------------------------
template <int MT, int D>
__global__ __launch_bounds__(64 * NW) void gemv_q6k_kernel(Args a) {
    extern __shared__ __attribute__((aligned(16))) int8_t s_gv[];
    const int lane = threadIdx.x & 63;
    const int w = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
    const int M = a.M, N = a.N, K = a.K, nsb = K / 256;
    const int rowbytes = nsb * Q6B;
    const int ipr = nsb >> 3;  // load instructions per row
    const int row0 = blockIdx.x * RPG + w * RPW;
    int8_t *const s_qs = s_gv;
    float *const s_d = reinterpret_cast<float *>(s_gv + lds_qs(MT, K));
    const auto rs_w = __builtin_amdgcn_make_buffer_rsrc((void *)a.W, (short)0, N * rowbytes, RSRC_FLAGS);

    stage_acts(a, s_qs, s_d, w, lane);

    const int sbl = lane >> 3, h = (lane >> 2) & 1, u = lane & 3;
    struct Raw {
        v4i ql0, ql1;
        uint32_t ql2;
        v4i qh0, qh1;
        uint32_t qh2, sc, dd;
    };
    // (rows past N: offsets stay below (N + 256) rows, the host's limit)
    auto issue = [&](int r, int j, Raw &R) __attribute__((always_inline)) {
        const int base = (row0 + r) * rowbytes + (8 * min(j, ipr - 1) + sbl) * Q6B;
        const int b4 = base & ~3;
        const int oq = b4 + 64 * h + 32 * (u & 1), oh = b4 + 128 + 32 * h;
        R.ql0 = ld16(rs_w, oq);
        R.ql1 = ld16(rs_w, oq + 16);
        R.ql2 = ld4(rs_w, oq + 32);
        R.qh0 = ld16(rs_w, oh);
        R.qh1 = ld16(rs_w, oh + 16);
        R.qh2 = ld4(rs_w, oh + 32);
        R.sc = ld4(rs_w, (base + 192 + 8 * h + 2 * u) & ~3);
        R.dd = ld4(rs_w, (base + 208) & ~3);
    };
    constexpr int LOADS = 8;  // per issue
    // D groups of loads in flight per row (past the last group a re-read of
    // it, unused and drained at the end, so every step has the same loads in
    // flight)
    Raw raw[RPW][D];
#pragma unroll
    for (int jj = 0; jj < D; ++jj)
#pragma unroll
        for (int r = 0; r < RPW; ++r) issue(r, jj, raw[r][jj]);
    // this wave's activation copies have landed once at most the weight loads
    // are in flight; the barrier covers the other waves' copies
    wait_vmcnt<LOADS * RPW * D>();
    __builtin_amdgcn_s_barrier();

    float acc[RPW][MT];
#pragma unroll
    for (int r = 0; r < RPW; ++r)
#pragma unroll
        for (int m = 0; m < MT; ++m) acc[r][m] = 0.0f;

    auto compute = [&](int j, const Raw &R, float (&ac)[MT]) __attribute__((always_inline)) {
        const int sb = 8 * j + sbl;
        const int mis = (2 * sb) & 3;  // block offset mod 4 (rows are 16-byte multiples)
        const uint32_t sh = 8 * mis;
        const uint32_t ql[9] = {(uint32_t)R.ql0[0], (uint32_t)R.ql0[1], (uint32_t)R.ql0[2], (uint32_t)R.ql0[3],
                                (uint32_t)R.ql1[0], (uint32_t)R.ql1[1], (uint32_t)R.ql1[2], (uint32_t)R.ql1[3], R.ql2};
        const uint32_t qh[9] = {(uint32_t)R.qh0[0], (uint32_t)R.qh0[1], (uint32_t)R.qh0[2], (uint32_t)R.qh0[3],
                                (uint32_t)R.qh1[0], (uint32_t)R.qh1[1], (uint32_t)R.qh1[2], (uint32_t)R.qh1[3], R.qh2};
        int q[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const uint32_t l4 = (__builtin_amdgcn_alignbit(ql[i + 1], ql[i], sh) >> (4 * (u >> 1))) & 0x0F0F0F0Fu;
            const uint32_t h2 = (__builtin_amdgcn_alignbit(qh[i + 1], qh[i], sh) >> (2 * u)) & 0x03030303u;
            const uint32_t v = l4 | (h2 << 4);
            q[i] = (int)(((v | 0x80808080u) - 0x20202020u) ^ 0x80808080u);
        }
        const uint32_t scw = R.sc >> (8 * ((mis + 2 * u) & 3));
        const int sc0 = (int)(int8_t)(scw & 0xFFu), sc1 = (int)(int8_t)((scw >> 8) & 0xFFu);
        const float dw = f16_bits_to_f32(R.dd >> (8 * mis));
        // values 128h + 32u + t: pieces 8h + 2u (t < 16) and 8h + 2u + 1, swizzled
        const int sw = sb & 1;
        const int k0 = sb * 256 + 16 * ((8 * h + 2 * u) ^ sw);
        const int k1 = sb * 256 + 16 * ((8 * h + 2 * u + 1) ^ sw);
        v4i a0[MT], a1[MT];
        float da[MT];
#pragma unroll
        for (int m = 0; m < MT; ++m) {
            a0[m] = *reinterpret_cast<const v4i *>(s_qs + m * K + k0);
            a1[m] = *reinterpret_cast<const v4i *>(s_qs + m * K + k1);
            da[m] = s_d[sb * M + m];
        }
#pragma unroll
        for (int m = 0; m < MT; ++m) {
            int s0 = 0, s1 = 0;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                s0 = __builtin_amdgcn_sdot4(q[e], a0[m][e], s0, false);
                s1 = __builtin_amdgcn_sdot4(q[4 + e], a1[m][e], s1, false);
            }
            ac[m] = fmaf((float)(sc0 * s0 + sc1 * s1), da[m] * dw, ac[m]);
        }
    };

    for (int j0 = 0; j0 < ipr; j0 += D) {
#pragma unroll
        for (int jj = 0; jj < D; ++jj) {
#pragma unroll
            for (int r = 0; r < RPW; ++r) {
                // row r's loads for group j0 + jj have landed once the
                // RPW * D - 1 groups issued after them may still be in flight
                wait_vmcnt<LOADS * (RPW * D - 1)>();
                if (j0 + jj < ipr) compute(j0 + jj, raw[r][jj], acc[r]);  // uniform
                issue(r, j0 + jj + D, raw[r][jj]);
            }
        }
    }

#pragma unroll
    for (int o = 32; o >= 1; o >>= 1)
#pragma unroll
        for (int r = 0; r < RPW; ++r)
#pragma unroll
            for (int m = 0; m < MT; ++m) acc[r][m] += __shfl_xor(acc[r][m], o, 64);
    if (lane == 0) {
#pragma unroll
        for (int r = 0; r < RPW; ++r)
#pragma unroll
            for (int m = 0; m < MT; ++m)
                if (m < M && row0 + r < N) a.out[(int64_t)m * N + row0 + r] = acc[r][m];
    }
    wait_vmcnt<0>();
}

// ---------------------------------------------------------------------------
// Ternary (TWO = false: base-3; TWO = true: two bits per trit).
// Base-3 blocks are 28 bytes (26 trit bytes, fp16 scale), 4-byte aligned.
// A load instruction covers 8 consecutive blocks of each of the wave's 8 rows:
// lane l takes block l%8 of row l/8, all 128 values.  Byte b holds the digits
// e = t + 1 of values 5b .. 5b+4 (value 5b + p at base-3 position p).  The
// trits come from an LDS table with four phases: entry (phi, v) holds the five
// trits of byte value v as int8 at byte offsets phi .. phi+4 of 8 bytes.  Byte
// b's values start at byte 5b of the block's natural order, i.e. at offset
// 5b mod 4 = b mod 4 of dword floor(5b/4), so the phase-(b mod 4) entry ORs
// straight into natural-order dwords 5b/4 and 5b/4 + 1 (the two padding
// positions past value 127 are dropped).
// Two-bit blocks are 34 bytes (32 code bytes, fp16 scale), 2-byte aligned;
// a lane loads the 9 aligned dwords around its block and shifts them into
// place with v_alignbit (rows are a multiple of 8 blocks, so an odd block
// ends 4-aligned and no dword it needs passes the buffer's end).  Code byte
// j holds weights j + 32p in bits 2p, 2p+1, so natural-order dword d (values
// 4d .. 4d+3) is plane d/8 of code dword d % 8, trits bytewise without
// borrows: (c | 0x80) - 1, bit 7 flipped back.
// Then 32 v_dot4 per token, one fold per block with the block scale.  The 8
// lanes of a row are summed at the end in a fixed order.
// ---------------------------------------------------------------------------
constexpr int TQB = 28;         // ternary block bytes (base-3)
constexpr int TQ2B = 34;        // ... (two bits per trit)
constexpr int TRPW = 8;         // rows per wave
constexpr int TRPG = NW * TRPW; // rows per workgroup
#ifndef GV_TQ_DEPTH
#define GV_TQ_DEPTH 2
#endif
constexpr int TQ_DEPTH = GV_TQ_DEPTH;  // load instructions in flight per wave
constexpr int LUT_BYTES = 4 * 256 * 8;
__host__ __device__ constexpr int tq_lds_d(int M, int nblk) { return (nblk * M * 4 + 1023) / 1024 * 1024; }
__host__ __device__ constexpr int tq_lds_bytes(int MT, int M, int K, bool two = false) {
    return MT * K + tq_lds_d(M, K / 128) + (two ? 0 : LUT_BYTES) + 256;
}

template <int MT, bool TWO>
__global__ __launch_bounds__(64 * NW) void gemv_tq_kernel(Args a) {
    constexpr int BB = TWO ? TQ2B : TQB;
    extern __shared__ __attribute__((aligned(16))) int8_t s_gv[];
    const int lane = threadIdx.x & 63;
    const int w = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
    const int M = a.M, N = a.N, K = a.K, nblk = K / 128;
    const int rowbytes = nblk * BB;
    const int ipr = nblk >> 3;  // load instructions per row
    const int r = lane >> 3, bl = lane & 7;
    const int row = blockIdx.x * TRPG + w * TRPW + r;
    int8_t *const s_qs = s_gv;
    float *const s_d = reinterpret_cast<float *>(s_gv + MT * K);
    int8_t *const s_lut = s_gv + MT * K + tq_lds_d(M, nblk);

    // ---- activations -> LDS (piece i of block b at slot i ^ (b % 8): the 8
    // blocks one read instruction touches fall on different banks) ----------
    {
        const auto rs_a = __builtin_amdgcn_make_buffer_rsrc((void *)a.qs, (short)0, M * K, RSRC_FLAGS);
        const auto rs_d = __builtin_amdgcn_make_buffer_rsrc((void *)a.da, (short)0, nblk * M * 4, RSRC_FLAGS);
        const int nq = (M * K) >> 10, nd = (nblk * M * 4 + 255) >> 8;
        const int aq = 128 * (lane >> 3) + 16 * ((lane & 7) ^ (lane >> 3));
        for (int c = w; c < nq; c += NW) copy16(rs_a, s_qs + 1024 * c, 1024 * c + aq);
        for (int c = w; c < nd; c += NW) copy4(rs_d, reinterpret_cast<int8_t *>(s_d) + 256 * c, 256 * c + 4 * lane);
    }
    // ---- weights: TQ_DEPTH instructions in flight (7 dwords per lane) ---------
    const auto rs_w = __builtin_amdgcn_make_buffer_rsrc((void *)a.W, (short)0, N * rowbytes, RSRC_FLAGS);
    struct Raw {
        v4i w0;
        v3u w1;   // base-3: dwords 4..6
        v4i w1b;  // two bits per trit: dwords 4..7, then w3
        uint32_t w3;
    };
    // (rows past N: offsets stay below (N + 256) rows, the host's limit)
    auto issue = [&](int j, Raw &R) __attribute__((always_inline)) {
        const int off = row * rowbytes + (8 * min(j, ipr - 1) + bl) * BB;
        if constexpr (TWO) {
            const int off4 = off & ~3;
            R.w0 = __builtin_bit_cast(v4i, __builtin_amdgcn_raw_buffer_load_b128(rs_w, off4, 0, 0));
            R.w1b = __builtin_bit_cast(v4i, __builtin_amdgcn_raw_buffer_load_b128(rs_w, off4 + 16, 0, 0));
            R.w3 = __builtin_amdgcn_raw_buffer_load_b32(rs_w, off4 + 32, 0, 0);
        } else {
            R.w0 = __builtin_bit_cast(v4i, __builtin_amdgcn_raw_buffer_load_b128(rs_w, off, 0, 0));
            R.w1 = __builtin_bit_cast(v3u, __builtin_amdgcn_raw_buffer_load_b96(rs_w, off + 16, 0, 0));
        }
    };
    constexpr int WLOADS = TWO ? 3 : 2;  // load instructions per issue
    Raw raw[TQ_DEPTH];
#pragma unroll
    for (int s = 0; s < TQ_DEPTH; ++s) issue(s, raw[s]);

    // ---- the trit table: entry (phi, v), 8 bytes, at 8 * (256 phi + v) ----
    for (int e = threadIdx.x; !TWO && e < 4 * 256; e += 64 * NW) {
        const int phi = e >> 8, v = e & 255;
        uint64_t ent = 0;
        if (v < 243) {
            int x = v;
#pragma unroll
            for (int p = 0; p < 5; ++p) {
                const int t = x % 3 - 1;
                x /= 3;
                ent |= (uint64_t)(uint8_t)(int8_t)t << (8 * (phi + p));
            }
        }
        *reinterpret_cast<uint64_t *>(s_lut + 8 * e) = ent;
    }
    // this wave's activation copies have landed once at most the weight loads
    // are in flight, and its table entries once its LDS writes are done; the
    // barrier covers the other waves'
    wait_vmcnt<WLOADS * TQ_DEPTH>();
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    __builtin_amdgcn_s_barrier();

    float acc[MT];
#pragma unroll
    for (int m = 0; m < MT; ++m) acc[m] = 0.0f;
    const uint32_t lut = (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void *)s_lut;

    auto compute = [&](int j, const Raw &R) __attribute__((always_inline)) {
        const int b = 8 * j + bl;
        int nat[32];
        float dw;
        if constexpr (TWO) {
            // the block's offset past the aligned dword: 2 bytes for odd
            // blocks (rows start 4-aligned)
            const uint32_t sh = 16u * (uint32_t)(b & 1);
            const uint32_t wv[9] = {(uint32_t)R.w0[0],  (uint32_t)R.w0[1],  (uint32_t)R.w0[2],
                                    (uint32_t)R.w0[3],  (uint32_t)R.w1b[0], (uint32_t)R.w1b[1],
                                    (uint32_t)R.w1b[2], (uint32_t)R.w1b[3], R.w3};
            uint32_t cw[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) cw[e] = __builtin_amdgcn_alignbit(wv[e + 1], wv[e], sh);
#pragma unroll
            for (int d = 0; d < 32; ++d) {
                const uint32_t c = (cw[d & 7] >> (2 * (d >> 3))) & 0x03030303u;
                nat[d] = (int)(((c | 0x80808080u) - 0x01010101u) ^ 0x80808080u);
            }
            dw = f16_bits_to_f32((R.w3 >> sh) & 0xFFFFu);
        } else {
            const uint32_t wv[7] = {(uint32_t)R.w0[0], (uint32_t)R.w0[1], (uint32_t)R.w0[2], (uint32_t)R.w0[3],
                                    R.w1[0], R.w1[1], R.w1[2]};
            // table lookups for the 26 trit bytes
            uint64_t ent[26];
#pragma unroll
            for (int by = 0; by < 26; ++by) {
                const uint32_t v = (wv[by >> 2] >> (8 * (by & 3))) & 0xFFu;
                const uint32_t addr = lut + 2048u * (uint32_t)(by & 3) + 8u * v;
                ent[by] = *reinterpret_cast<const __attribute__((address_space(3))) uint64_t *>(
                    (__attribute__((address_space(3))) void *)(uintptr_t)addr);
            }
            // natural-order int8 trits: byte by ORs into dwords 5by/4 and 5by/4 + 1
#pragma unroll
            for (int d = 0; d < 32; ++d) nat[d] = 0;
#pragma unroll
            for (int by = 0; by < 26; ++by) {
                const int d0 = (5 * by) >> 2;
                nat[d0] |= (int)(uint32_t)ent[by];
                if (d0 + 1 < 32) nat[d0 + 1] |= (int)(uint32_t)(ent[by] >> 32);
            }
            dw = f16_bits_to_f32(wv[6] >> 16);
        }
        const int kb = b * 128;
        v4i av[MT][8];
        float da[MT];
#pragma unroll
        for (int m = 0; m < MT; ++m) {
#pragma unroll
            for (int i = 0; i < 8; ++i)
                av[m][i] = *reinterpret_cast<const v4i *>(s_qs + m * K + kb + 16 * (i ^ (b & 7)));
            da[m] = s_d[b * M + m];
        }
#pragma unroll
        for (int m = 0; m < MT; ++m) {
            int sacc = 0;
#pragma unroll
            for (int i = 0; i < 8; ++i)
#pragma unroll
                for (int e = 0; e < 4; ++e) sacc = __builtin_amdgcn_sdot4(nat[4 * i + e], av[m][i][e], sacc, false);
            acc[m] = fmaf((float)sacc, da[m] * dw, acc[m]);
        }
    };

    for (int j0 = 0; j0 < ipr; j0 += TQ_DEPTH) {
#pragma unroll
        for (int s = 0; s < TQ_DEPTH; ++s) {
            // instruction j0 + s has landed once the TQ_DEPTH - 1 issued after
            // it may still be in flight (past the last, re-reads are harmless)
            wait_vmcnt<WLOADS * (TQ_DEPTH - 1)>();
            if (j0 + s < ipr) compute(j0 + s, raw[s]);
            issue(j0 + s + TQ_DEPTH, raw[s]);
        }
    }
    // a row's total: its 8 lanes summed in a fixed order, stored by lane 8r
#pragma unroll
    for (int o = 1; o < 8; o <<= 1)
#pragma unroll
        for (int m = 0; m < MT; ++m) acc[m] += __shfl_xor(acc[m], o, 64);
    if (bl == 0) {
#pragma unroll
        for (int m = 0; m < MT; ++m)
            if (m < M && row < N) a.out[(int64_t)m * N + row] = acc[m];
    }
    wait_vmcnt<0>();
}

}  // namespace gv

static int gv_tokens(int M) { return M <= 1 ? 1 : M <= 2 ? 2 : 4; }

// Which Q6_K / ternary shapes the matrix-vector kernels take: up to 4
// tokens, K a multiple of 2048 (Q6_K) or 1024 (ternary), so that a row is a
// whole number of load instructions, and the staged activations within the
// LDS budget.  From 5 tokens the ring kernel of kq_gemm_ring.hip is faster
// (Q6_K 4096 x 14336: 20.3 against 28.0 us at 5 tokens, 20.7 against 29.0 at
// 8, and 16.5 against 20.1 us for this kernel at 4; ternary 17408 x 5120:
// 18.1 against 27.9 us at 5 tokens, 13.3 against 18.0 for this kernel at 4).
bool gemv_choice(int fmt, int M, int N, int K) {
    (void)N;
    // (the staged activations cap K far below 2^20; the bound keeps the LDS
    // arithmetic below in int range for any K the API accepts)
    if (M < 1 || M > 4 || K > (1 << 20)) return false;
    if (fmt == 2) return K % 2048 == 0 && gv::lds_bytes(gv_tokens(M), M, K) <= gv::LDS_BUDGET;
    if (fmt == 3) return K % 1024 == 0 && gv::tq_lds_bytes(gv_tokens(M), M, K) <= gv::LDS_BUDGET;
    if (fmt == 4) return K % 1024 == 0 && gv::tq_lds_bytes(gv_tokens(M), M, K, true) <= gv::LDS_BUDGET;
    return false;
}

hipError_t launch_gemv(int fmt, const void *W, const int8_t *qs, const float *da, float *out,
                       int M, int N, int K, hipStream_t stream) {
    gv::Args a;
    a.W = static_cast<const uint8_t *>(W);
    a.qs = qs;
    a.da = da;
    a.out = out;
    a.M = M;
    a.N = N;
    a.K = K;
    const dim3 block(64 * gv::NW);
    const int mt = gv_tokens(M);
    if (fmt == 3 || fmt == 4) {
        const dim3 grid((unsigned)((N + gv::TRPG - 1) / gv::TRPG));
        const bool two = fmt == 4;
        const size_t lds = (size_t)gv::tq_lds_bytes(mt, M, K, two);
        switch (mt) {
            case 1:
                if (two) hipLaunchKernelGGL((gv::gemv_tq_kernel<1, true>), grid, block, lds, stream, a);
                else hipLaunchKernelGGL((gv::gemv_tq_kernel<1, false>), grid, block, lds, stream, a);
                break;
            case 2:
                if (two) hipLaunchKernelGGL((gv::gemv_tq_kernel<2, true>), grid, block, lds, stream, a);
                else hipLaunchKernelGGL((gv::gemv_tq_kernel<2, false>), grid, block, lds, stream, a);
                break;
            default:
                if (two) hipLaunchKernelGGL((gv::gemv_tq_kernel<4, true>), grid, block, lds, stream, a);
                else hipLaunchKernelGGL((gv::gemv_tq_kernel<4, false>), grid, block, lds, stream, a);
                break;
        }
        return hipGetLastError();
    }
    const dim3 grid((unsigned)((N + gv::RPG - 1) / gv::RPG));
    const size_t lds = (size_t)gv::lds_bytes(mt, M, K);
    // two groups of loads in flight per row for four tokens once a row has
    // three or more groups (4096 x 14336: 16.7 against 17.7 us; at one and
    // two tokens one group in flight is faster, 12.8 against 14.5 us)
    if (K / 2048 >= 3 && mt >= 4) {
        hipLaunchKernelGGL((gv::gemv_q6k_kernel<4, 2>), grid, block, lds, stream, a);
    } else {
        switch (mt) {
            case 1: hipLaunchKernelGGL((gv::gemv_q6k_kernel<1, 1>), grid, block, lds, stream, a); break;
            case 2: hipLaunchKernelGGL((gv::gemv_q6k_kernel<2, 1>), grid, block, lds, stream, a); break;
            default: hipLaunchKernelGGL((gv::gemv_q6k_kernel<4, 1>), grid, block, lds, stream, a); break;
        }
    }
    return hipGetLastError();
}

}  // namespace kq
