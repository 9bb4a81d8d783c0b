/*
 * kq.h -- C ABI of the block-quantized weight x quantized-activation GEMM
 * for AMD Instinct MI355X (gfx950).
 *
 * The path (vllm.cpp PR 3036 "cooperative-tile WMMA kernels -- Shared
 * rejected, BigTile accepted": activation-quant scratch, then a tile GEMM over
 * Q4_K/Q6_K weights and BlockQ8_K activations; PrismML llama.cpp PR 214
 * "branch-free PTQ1_0 MMQ tile loader": the ternary MMQ path):
 *
 *   1. kq_quantize_act: fp32 activations -> int8 blocks with an fp32 scale
 *      (Q8_K: 256 per block plus int16 sums per 16; Q8_128: 128 per block).
 *   2. kq_gemm: out[m][n] = sum_k W^[n][k] * A^[m][k], where W^ is the
 *      dequantized stored weight and A^[m][k] = d[m][block] * qs[m][k].
 *      The contraction runs on int8 matrix cores; block scales and mins are
 *      folded in afterwards.
 *
 * Conventions (all entry points):
 *   - Every pointer argument is a DEVICE pointer except where noted.  The
 *     caller allocates and frees all memory; the library allocates nothing,
 *     keeps no handles and needs no scratch.
 *   - Work is enqueued asynchronously on `stream` (NULL = the default
 *     stream).  Device faults surface at the caller's next synchronization.
 *   - Arguments are validated on the host before any HIP call.  On any error
 *     nothing is launched and a negative KQ_ERR_* code is returned; a shape
 *     with no verified kernel variant is declined with KQ_ERR_UNSUPPORTED
 *     rather than computed wrongly.  M == 0 or N == 0 returns KQ_OK with no
 *     launch.
 *   - Output buffers must not overlap inputs.  Calls are thread-safe; the only
 *     global state is a set of atomic per-variant dispatch counters and a
 *     per-device cache of the compute-unit count (atomic; it sizes the
 *     persistent grids).
 *   - Every launch goes to the caller's stream and the library records no
 *     memset (outputs that must start at zero are cleared by a kernel), so
 *     kq_quantize_act, kq_gemm and kq_gemm_id can be captured in a HIP graph;
 *     dispatch counters count the capture, not the replays.
 *
 * Data layouts (this library's own; the pages fix only the block sizes:
 * 292 bytes per 256 activations for BlockQ8_K in vllm.cpp PR 3036, a 28-byte
 * block per 128 ternary weights in llama.cpp PR 214):
 *
 *   Q8_K activations (KQ_ACT_Q8_K), one buffer of kq_act_bytes() bytes with
 *   four sections, each at a 256-byte-aligned offset from the start:
 *     qs    int8  [M][K]        quantized values
 *     d     fp32  [K/256][M]    block scales, block-major: the scales of block
 *                               s of all M rows are contiguous
 *     bsums int16 [M][K/16]     sums of qs over each 16 consecutive values
 *     alpha bf16  [K/256][2][M][8]
 *                               per block s, row m and 32-value sub-block j,
 *                               with B the sum of the sub-block's 32 qs
 *                               (|B| <= 4064): part 0 = 64 * floor(B / 64),
 *                               part 1 = B - part 0 (in [0, 63]); both are
 *                               integers bf16 represents exactly.  This is
 *                               the activation operand of the Q4_K min term
 *                               sum_j m_j * B_j, which the GEMM forms exactly
 *                               from it instead of re-summing qs per tile.
 *   Q8_128 activations (KQ_ACT_Q8_128): sections qs int8 [M][K] and
 *   d fp32 [K/128][M] (block-major); no bsums, no alpha.
 *   Quantization rule per block, in fp32: amax = max|x|; if amax == 0 or
 *   127/amax is not finite then d = 0 and qs = 0; otherwise d = amax/127,
 *   s = 127/amax, qs = clamp(rint(x*s), -127, 127) (round half to even, one
 *   fp32 multiply).  Inputs must be finite.
 *
 *   Weights W: row n (output feature) is K/QK consecutive blocks, rows are
 *   consecutive, so W is [N][K/QK] blocks.
 *   KQ_Q4_K, 144 bytes per 256 weights (8 sub-blocks of 32):
 *     [0,2) fp16 d; [2,4) fp16 dmin; [4,16) a little-endian 96-bit integer
 *     whose bits [6f, 6f+6) hold field f: f < 8 scale sc_f, f >= 8 min m_(f-8);
 *     [16,144) byte 32c+t (c < 4, t < 32) holds weight 64c+t in its low nibble
 *     and weight 64c+32+t in its high nibble.
 *     W^_k = d * sc_j * q_k - dmin * m_j, j = k/32.
 *   KQ_Q6_K, 210 bytes per 256 weights (16 sub-blocks of 16):
 *     [0,128) byte 64h+t (h < 2, t < 64): low 4 bits of weight 128h+t (bits
 *     0..3) and of weight 128h+64+t (bits 4..7); [128,192) bits 2u..2u+1 of
 *     byte 128+32h+t (t < 32, u < 4) are the high 2 bits of weight
 *     128h+32u+t; [192,208) int8 scales; [208,210) fp16 d.
 *     W^_k = d * sc_j * (q_k - 32), j = k/16.
 *   KQ_TQ (ternary), 28 bytes per 128 weights:
 *     [0,26) weight k is base-3 digit t_k+1 at position k mod 5 of byte k/5
 *     (least significant digit first; the two spare digits of byte 25 must
 *     be 1, so every byte is <= 242); [26,28) fp16 d.  W^_k = d * t_k.
 *     Bytes 24..27 read as a little-endian word are qh0 | qh1<<8 | d<<16,
 *     the word layout of llama.cpp PR 214's loader.
 *   KQ_TQ2 (ternary at two bits per weight: the PQ2_0 packing llama.cpp PR
 *   214 names, the same trits), 34 bytes per 128 weights:
 *     [0,32) byte j holds the codes c = t + 1 of weights j, j+32, j+64 and
 *     j+96 in bits 0-1, 2-3, 4-5 and 6-7 (code 3 must not occur); [32,34)
 *     fp16 d.  W^_k = d * t_k.  Blocks start 2-byte aligned only.
 *   Q4_K and Q6_K weights take Q8_K activations; both ternary formats take
 *   Q8_128.
 *
 *   out: fp32 [M][N] row-major, fully overwritten (never accumulated).
 */
#ifndef KQ_H
#define KQ_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define KQ_VERSION 2

/* weight formats */
#define KQ_Q4_K 1
#define KQ_Q6_K 2
#define KQ_TQ 3
#define KQ_TQ2 4

/* activation formats */
#define KQ_ACT_Q8_K 1
#define KQ_ACT_Q8_128 2

/* activation buffer sections */
#define KQ_SEC_QS 0
#define KQ_SEC_D 1
#define KQ_SEC_BSUMS 2
#define KQ_SEC_ALPHA 3

/* status codes */
#define KQ_OK 0
#define KQ_ERR_FMT (-1)         /* unknown format */
#define KQ_ERR_SHAPE (-2)       /* negative size, K not a multiple of the block, size overflow */
#define KQ_ERR_NULL (-3)        /* NULL pointer with nonzero work */
#define KQ_ERR_ALIGN (-4)       /* a pointer is not 16-byte aligned */
#define KQ_ERR_UNSUPPORTED (-5) /* no verified kernel variant for this case */
#define KQ_ERR_HIP (-6)         /* the HIP runtime reported an error at launch */

/* Size queries.  Return 0 for invalid arguments. */
size_t kq_weight_bytes(int fmt, int64_t N, int64_t K);
size_t kq_act_bytes(int act_fmt, int64_t M, int64_t K);
/* Byte offset of a section (KQ_SEC_*) inside an activation buffer; -1 when the
 * section does not exist for this format or the arguments are invalid. */
int64_t kq_act_section_offset(int act_fmt, int section, int64_t M, int64_t K);
/* The activation format a weight format consumes; KQ_ERR_FMT if unknown. */
int kq_act_fmt_for(int fmt);

/*
 * Quantize fp32 activations x [M][K] (device, row-major, contiguous, 16-byte
 * aligned) into a_q8 (device, kq_act_bytes(act_fmt, M, K) bytes, 16-byte
 * aligned) in the layout above.  K must be a multiple of 256 (Q8_K) or 128
 * (Q8_128).  Defined by the activation-quant step of vllm.cpp PR 3036
 * (EnsureQuantScratch filling qact with BlockQ8_K rows; no padding rows).
 */
int kq_quantize_act(int act_fmt, const float *x, int64_t M, int64_t K, void *a_q8,
                    hipStream_t stream);

/*
 * out [M][N] = product of the quantized activations a_q8 (from
 * kq_quantize_act with kq_act_fmt_for(fmt); exactly M rows, no padding) and
 * the stored weights W [N][K/QK blocks].  K must be a multiple of 256 (Q4_K,
 * Q6_K) or 128 (ternary).  All pointers device, 16-byte aligned.  Defined by
 * the tile GEMM of vllm.cpp PR 3036 (per-sub-block int8 dot products with the
 * Q4_K/Q6_K scales and mins folded in) and the PTQ1_0 MMQ path of llama.cpp
 * PR 214.  The fp32 result agrees with the exact product of the dequantized
 * operands to within 1e-4 * sum_k |W^ A^| + 1e-6 per element, and the same
 * call on the same inputs gives the same bits (where a product runs K in two
 * parts, each adds into out, zeroed first, and two addends onto zero round
 * alike in either order; out is written in full whatever it held).  Calls
 * on one stream run in order; out must not be read or written by other work
 * until the call completes.  The kernels
 * address every operand with 32-bit byte offsets: shapes where the weight
 * tensor plus 256 rows, or an activation section (qs, d, alpha) or the
 * output plus 128 (scales: 256) rows, reaches 2^31 bytes are declined with
 * KQ_ERR_UNSUPPORTED.
 */
int kq_gemm(int fmt, const void *W, const void *a_q8, int64_t M, int64_t N, int64_t K,
            float *out, hipStream_t stream);

/*
 * Test hook: per-sub-block integer dot sums, written out.  sums (device,
 * int32 [M][N][K/SB]) receives
 *   S[m][n][j] = sum_{k in sub-block j} qint[n][k] * qs[m][k]
 * with SB = 32 and qint = q (Q4_K), SB = 16 and qint = q - 32 (Q6_K),
 * SB = 128 and qint = t (ternary).  This runs a separate small decoder (its
 * own weight loaders and a 32 x 32 int8 MFMA loop, for every format), not
 * the kq_gemm kernels, which never materialize S: those are held to the same
 * sums exactly by products whose scales expose them (unit scales, a single
 * nonzero sub-block scale), so the hook is a reference implementation on the
 * device rather than a view into production code.  Defined by the
 * per-sub-block int8 dot products of vllm.cpp PR 3036's tile GEMM.
 */
int kq_gemm_subsums(int fmt, const void *W, const void *a_q8, int64_t M, int64_t N,
                    int64_t K, int32_t *sums, hipStream_t stream);

/*
 * Test hook: decode nblocks consecutive weight blocks of W (device, 16-byte
 * aligned, kq_weight_bytes(fmt, 1, nblocks * QK) bytes) with the loaders of
 * the sub-sum hook above (the loader fuzz test of llama.cpp PR 214, which ran
 * its unpack on thousands of random packed blocks against the scalar codec;
 * the kq_gemm kernels' own unpacking is checked through identity activations
 * and the exact-sum products instead).  Writes, for block b:
 *   q [b][QK] int8 (device, 16-byte aligned): the integer operand of every
 *     value in storage order, q in [0,15] (Q4_K), q - 32 (Q6_K), t (ternary);
 *   scales [b][16] int32 (device, 4-byte aligned): Q4_K sc_0..sc_7 then
 *     m_0..m_7 (the 6-bit fields); Q6_K the 16 int8 scales, sign-extended.
 *     Not written for the ternary formats, where scales may be NULL.
 * The fp16 d / dmin fields are not decoded here.  nblocks may be at most
 * KQ_DEBUG_UNPACK_MAX_BLOCKS (KQ_ERR_SHAPE beyond, or when negative); 0 returns
 * KQ_OK with no launch.  Unknown fmt -> KQ_ERR_FMT; W or q NULL (or scales for
 * Q4_K / Q6_K) -> KQ_ERR_NULL; misaligned pointers -> KQ_ERR_ALIGN.
 */
#define KQ_DEBUG_UNPACK_MAX_BLOCKS (1 << 24)
int kq_debug_unpack(int fmt, const void *W, int64_t nblocks, int8_t *q, int32_t *scales,
                    hipStream_t stream);

/*
 * Expert-indexed product (a mixture-of-experts layer's GEMM; llama.cpp's
 * MUL_MAT_ID, which the pages test next to MUL_MAT): every routed row r
 * multiplies one expert's weights with one token's quantized activations,
 *   out[r][n] = sum_k W^_e[n][k] * A^[rows[r]][k],  e the expert of row r,
 * through the same loaders and tile kernels as kq_gemm: Q4_K on the
 * register-unpack tile kernel with 64-row tiles (N < 2^23; wider Q4_K shapes
 * are declined with KQ_ERR_UNSUPPORTED), the other formats on the 128 x 128
 * tile kernel, each gathering the token rows of one expert per tile.  Every
 * routed row gets the bits kq_gemm gives its token where kq_gemm runs the
 * same tile kernel.
 *   W               device, n_experts consecutive weight tensors of N rows of
 *                   K/QK blocks (expert e starts e * kq_weight_bytes(fmt, N, K)
 *                   bytes in), 16-byte aligned
 *   a_q8            device, M tokens from kq_quantize_act (kq_act_fmt_for(fmt))
 *   expert_offsets  device int32 [n_experts + 1], non-decreasing, [0] = 0,
 *                   [n_experts] = R: the routed rows of expert e are
 *                   [expert_offsets[e], expert_offsets[e + 1])
 *   rows            device int32 [R]: the token (row of a_q8, 0 <= t < M) of
 *                   each routed row; a token may appear any number of times
 *   out             device fp32 [R][N], fully overwritten
 * The routing arrays live on the device and are not checked on the host:
 * arrays that break the contract give undefined values in out, but every
 * access stays inside W, a_q8, rows and out.  R == 0 or N == 0 returns KQ_OK
 * with no launch; M == 0 with R > 0 is KQ_ERR_SHAPE; n_experts must be in
 * 1 .. KQ_GEMM_ID_MAX_EXPERTS (each tile locates its expert by walking the
 * offsets, so the walk is kept short).  Other errors and limits as kq_gemm
 * (one expert's weights and the activation sections within 2^31 bytes, and
 * the per-workgroup loop count of the persistent tile kernel within int32).
 */
#define KQ_GEMM_ID_MAX_EXPERTS 1024
int kq_gemm_id(int fmt, const void *W, int64_t n_experts, const void *a_q8, int64_t M, int64_t N,
               int64_t K, const int32_t *expert_offsets, const int32_t *rows, int64_t R, float *out,
               hipStream_t stream);

/* Per-variant dispatch counters (incremented on each successful launch) and
 * their names, so tests can prove which kernel variant ran (vllm.cpp PR 3036
 * added such counters after finding tests that never reached a variant). */
int kq_num_variants(void);
const char *kq_variant_name(int variant);
uint64_t kq_dispatch_count(int variant);
void kq_dispatch_reset(void);

/*
 * Calibration kernels (measurement hooks): the device's own int8 matrix-core,
 * fp32 VALU and HBM read rates, against which the GEMM's fractions of peak are
 * also reported (the published peaks assume a clock the chip does not hold
 * under load).  One call launches one kernel on `stream` that does a fixed
 * amount of work and stores *work (host pointer): int8 ops for the matrix-core
 * kinds, fp32 flops for KQ_CALIB_VALU_F32, bytes read for KQ_CALIB_HBM_READ.
 * The caller times the launch with events on the same stream.
 *   KQ_CALIB_MFMA_I8        independent v_mfma_i32_32x32x32_i8 chains, two
 *                           waves per SIMD, constant operands
 *   KQ_CALIB_MFMA_I8_TOGGLE the same with operands that change every iteration
 *                           (two VALU adds per MFMA)
 *   KQ_CALIB_VALU_F32       independent v_fma_f32 chains (not packed)
 *   KQ_CALIB_MFMA_I8_VALU   KQ_CALIB_MFMA_I8_TOGGLE plus `param` (2, 4, 6 or
 *                           8) v_fma_f32 between consecutive MFMAs
 *   KQ_CALIB_HBM_READ       16-byte loads over buf [bytes] (device, 16-byte
 *                           aligned, bytes a positive multiple of 16); use a
 *                           buffer well beyond the 256 MB Infinity Cache
 * Errors: unknown kind -> KQ_ERR_FMT; work NULL, or buf NULL for the read ->
 * KQ_ERR_NULL; bad param or bytes -> KQ_ERR_SHAPE; misaligned buf ->
 * KQ_ERR_ALIGN; a launch failure -> KQ_ERR_HIP.
 */
#define KQ_CALIB_MFMA_I8 0
#define KQ_CALIB_MFMA_I8_TOGGLE 1
#define KQ_CALIB_VALU_F32 2
#define KQ_CALIB_MFMA_I8_VALU 3
#define KQ_CALIB_HBM_READ 4
int kq_calib_launch(int kind, int param, const void *buf, int64_t bytes, double *work,
                    hipStream_t stream);

/* The variant kq_gemm would launch for this case, or a negative KQ_ERR_*. */
int kq_select_variant(int fmt, int64_t M, int64_t N, int64_t K);

const char *kq_strerror(int status);
int kq_version(void);

#ifdef __cplusplus
}
#endif

#endif /* KQ_H */
