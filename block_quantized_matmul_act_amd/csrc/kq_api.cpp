// kq_api.cpp -- the C ABI of include/kq.h: host-side validation, size
// queries, variant selection and launch.  Every argument check happens before
// the first HIP call, so invalid calls return a status without touching the
// runtime (and can be tested on a machine without a GPU).
#include "../../include/kq.h"

#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdint>

#include "kq_calib.hpp"
#include "kq_hooks.hpp"
#include "kq_launch.hpp"

namespace {

enum Variant {
    V_QUANT_Q8K = 0,
    V_QUANT_Q8_128,
    V_GEMM_Q4K_128x128,
    V_GEMM_Q4K_MATVEC,
    V_GEMM_Q6K_128x128,
    V_GEMM_Q6K_MATVEC,
    V_GEMM_TQ_128x128,
    V_GEMM_TQ_MATVEC,
    V_SUBSUMS_Q4K,
    V_SUBSUMS_Q6K,
    V_SUBSUMS_TQ,
    V_GEMM_TQ2_128x128,
    V_SUBSUMS_TQ2,
    V_GEMM_ID_128x128,
    V_GEMM_Q4K_64x128,
    V_GEMM_ID_Q4K_64x128,
    V_GEMM_Q4K_64x128_K2,
    V_GEMM_Q4K_M16,
    V_GEMM_TQ_128x128_REG,
    V_GEMM_Q4K_M64_RING,
    V_GEMM_Q6K_RING,
    V_GEMM_TQ2_RING,
    V_GEMM_TQ_RING,
    V_GEMM_Q4K_RING_KP,
    V_GEMM_TQ2_MATVEC,
    V_GEMM_Q6K_128x128_K2,
    V_GEMM_TQ_128x128_K2,
    V_GEMM_TQ2_128x128_K2,
    V_COUNT
};

const char *const kVariantNames[V_COUNT] = {
    "quant_q8_k",        "quant_q8_128",    "gemm_q4_k_128x128", "gemm_q4_k_matvec",
    "gemm_q6_k_128x128", "gemm_q6_k_matvec", "gemm_tq_128x128", "gemm_tq_matvec", "subsums_q4_k",  "subsums_q6_k",
    "subsums_tq",        "gemm_tq2_128x128", "subsums_tq2",   "gemm_id_128x128", "gemm_q4_k_64x128",
    "gemm_id_q4_k_64x128", "gemm_q4_k_64x128_k2", "gemm_q4_k_m16", "gemm_tq_128x128_reg", "gemm_q4_k_m64_ring",
    "gemm_q6_k_ring", "gemm_tq2_ring", "gemm_tq_ring", "gemm_q4_k_ring_kp", "gemm_tq2_matvec",
    "gemm_q6_k_128x128_k2", "gemm_tq_128x128_k2", "gemm_tq2_128x128_k2",
};

std::atomic<uint64_t> g_count[V_COUNT];

constexpr int64_t kMaxDim = INT32_MAX;  // kernels index rows and columns with int
constexpr int64_t kMaxBytes = (int64_t)1 << 46;

int qk_of(int fmt) {
    return fmt == KQ_Q4_K || fmt == KQ_Q6_K ? 256 : fmt == KQ_TQ || fmt == KQ_TQ2 ? 128 : 0;
}
int bb_of(int fmt) {
    return fmt == KQ_Q4_K ? 144 : fmt == KQ_Q6_K ? 210 : fmt == KQ_TQ ? 28 : fmt == KQ_TQ2 ? 34 : 0;
}
int bs_of(int act_fmt) {
    return act_fmt == KQ_ACT_Q8_K ? 256 : act_fmt == KQ_ACT_Q8_128 ? 128 : 0;
}
int64_t align256(int64_t v) { return (v + 255) & ~(int64_t)255; }
bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

// Section offsets of an activation buffer; false when invalid.
struct ActLayout {
    int64_t d, bsums, alpha, total;  // byte offsets; -1 for absent sections
};
bool act_layout(int act_fmt, int64_t M, int64_t K, ActLayout *L) {
    const int bs = bs_of(act_fmt);
    if (!bs || M < 0 || K < 0 || K % bs || M > kMaxDim || K > kMaxDim) return false;
    if (M != 0 && K > kMaxBytes / M) return false;
    const int64_t qs_bytes = align256(M * K);
    const int64_t d_bytes = align256(M * (K / bs) * 4);
    L->d = qs_bytes;
    if (act_fmt == KQ_ACT_Q8_K) {
        L->bsums = qs_bytes + d_bytes;
        L->alpha = L->bsums + align256(M * (K / 16) * 2);
        L->total = L->alpha + align256((K / 256) * 2 * M * 8 * 2);
    } else {
        L->bsums = -1;
        L->alpha = -1;
        L->total = qs_bytes + d_bytes;
    }
    return true;
}

// Shared validation of kq_gemm / kq_gemm_subsums arguments.
int check_gemm(int fmt, const void *W, const void *a_q8, int64_t M, int64_t N, int64_t K,
               const void *out) {
    if (!qk_of(fmt)) return KQ_ERR_FMT;
    if (M < 0 || N < 0 || K < 0 || K % qk_of(fmt)) return KQ_ERR_SHAPE;
    if (M > kMaxDim || N > kMaxDim || K > kMaxDim) return KQ_ERR_SHAPE;
    if ((M && K > kMaxBytes / M) || (N && K > kMaxBytes / N) || (M && N > kMaxBytes / M))
        return KQ_ERR_SHAPE;
    if (M == 0 || N == 0) return KQ_OK;
    if (!W || !a_q8 || !out) return KQ_ERR_NULL;
    if (!aligned16(W) || !aligned16(a_q8) || !aligned16(out)) return KQ_ERR_ALIGN;
    // grid limits: tiles must fit a 1-D grid
    const int64_t tiles = ((M + 31) / 32) * ((N + 31) / 32);
    if (tiles > INT32_MAX) return KQ_ERR_UNSUPPORTED;
    // the Q4_K persistent kernels count (tile, superblock) steps per
    // workgroup in int32 (64-row tiles at the most)
    if (fmt == KQ_Q4_K && ((M + 63) / 64) * ((N + 127) / 128) * (K / 256) > INT32_MAX)
        return KQ_ERR_UNSUPPORTED;
    // the GEMM kernels address whole tensors (W, the qs, d and alpha sections,
    // out) with 32-bit buffer offsets, including the rows and columns a last
    // tile hangs past M (up to 128) and N (up to 256): every such offset stays
    // below 2^31, so adding the 2^31 "drop this store" offset cannot wrap
    const int64_t lim = (int64_t)1 << 31;
    const int64_t rowbytes = (K / qk_of(fmt)) * bb_of(fmt);
    if ((M + 128) * K >= lim || (N + 256) * rowbytes >= lim || (M + 128) * N * 4 >= lim ||
        (K / qk_of(fmt)) * (M + 256) * 4 >= lim || (K / 256) * 2 * (M + 256) * 16 >= lim)
        return KQ_ERR_UNSUPPORTED;
    return 1;  // proceed
}

int variant_for(int fmt, int64_t M, int64_t N, int64_t K) {
    if (fmt == KQ_Q4_K) {
        switch (kq::q4k_kernel_choice((int)M, (int)N, (int)K)) {
            case kq::Q4K_MATVEC: return V_GEMM_Q4K_MATVEC;
            case kq::Q4K_FEW_RING: return V_GEMM_Q4K_M64_RING;
            case kq::Q4K_RING_KP: return V_GEMM_Q4K_RING_KP;
            case kq::Q4K_TILE64: return V_GEMM_Q4K_64x128;
            case kq::Q4K_TILE64_K2: return V_GEMM_Q4K_64x128_K2;
            case kq::Q4K_FEW_SPLIT: return V_GEMM_Q4K_M16;
            default: return V_GEMM_Q4K_128x128;
        }
    }
    if (kq::gemv_choice(fmt, (int)M, (int)N, (int)K))
        return fmt == KQ_Q6_K ? V_GEMM_Q6K_MATVEC : fmt == KQ_TQ ? V_GEMM_TQ_MATVEC : V_GEMM_TQ2_MATVEC;
    if (kq::ring_choice(fmt, (int)M, (int)N, (int)K))
        return fmt == KQ_Q6_K ? V_GEMM_Q6K_RING : fmt == KQ_TQ ? V_GEMM_TQ_RING : V_GEMM_TQ2_RING;
    if (fmt == KQ_TQ && kq::tq_tile_choice((int)M, (int)N, (int)K)) return V_GEMM_TQ_128x128_REG;
    if (kq::tile_split_choice(fmt, (int)M, (int)N, (int)K))
        return fmt == KQ_Q6_K ? V_GEMM_Q6K_128x128_K2 : fmt == KQ_TQ ? V_GEMM_TQ_128x128_K2 : V_GEMM_TQ2_128x128_K2;
    if (fmt == KQ_TQ2) return V_GEMM_TQ2_128x128;
    return fmt == KQ_Q6_K ? V_GEMM_Q6K_128x128 : V_GEMM_TQ_128x128;
}

}  // namespace

extern "C" {

size_t kq_weight_bytes(int fmt, int64_t N, int64_t K) {
    const int qk = qk_of(fmt);
    if (!qk || N < 0 || K < 0 || K % qk || N > kMaxDim || K > kMaxDim) return 0;
    if (N && K > kMaxBytes / N) return 0;
    return (size_t)(N * (K / qk) * bb_of(fmt));
}

size_t kq_act_bytes(int act_fmt, int64_t M, int64_t K) {
    ActLayout L;
    if (!act_layout(act_fmt, M, K, &L)) return 0;
    return (size_t)L.total;
}

int64_t kq_act_section_offset(int act_fmt, int section, int64_t M, int64_t K) {
    ActLayout L;
    if (!act_layout(act_fmt, M, K, &L)) return -1;
    if (section == KQ_SEC_QS) return 0;
    if (section == KQ_SEC_D) return L.d;
    if (section == KQ_SEC_BSUMS) return L.bsums;
    if (section == KQ_SEC_ALPHA) return L.alpha;
    return -1;
}

int kq_act_fmt_for(int fmt) {
    if (fmt == KQ_Q4_K || fmt == KQ_Q6_K) return KQ_ACT_Q8_K;
    if (fmt == KQ_TQ || fmt == KQ_TQ2) return KQ_ACT_Q8_128;
    return KQ_ERR_FMT;
}

int kq_quantize_act(int act_fmt, const float *x, int64_t M, int64_t K, void *a_q8,
                    hipStream_t stream) {
    const int bs = bs_of(act_fmt);
    if (!bs) return KQ_ERR_FMT;
    ActLayout L;
    if (!act_layout(act_fmt, M, K, &L)) return KQ_ERR_SHAPE;
    if (M == 0 || K == 0) return KQ_OK;
    if (!x || !a_q8) return KQ_ERR_NULL;
    if (!aligned16(x) || !aligned16(a_q8)) return KQ_ERR_ALIGN;
    char *base = static_cast<char *>(a_q8);
    hipError_t e = kq::launch_quant_act(
        bs, x, reinterpret_cast<int8_t *>(base), reinterpret_cast<float *>(base + L.d),
        L.bsums >= 0 ? reinterpret_cast<int16_t *>(base + L.bsums) : nullptr,
        L.alpha >= 0 ? reinterpret_cast<uint16_t *>(base + L.alpha) : nullptr, M, K, stream);
    if (e != hipSuccess) return KQ_ERR_HIP;
    g_count[act_fmt == KQ_ACT_Q8_K ? V_QUANT_Q8K : V_QUANT_Q8_128].fetch_add(1);
    return KQ_OK;
}

int kq_select_variant(int fmt, int64_t M, int64_t N, int64_t K) {
    if (!qk_of(fmt)) return KQ_ERR_FMT;
    if (M < 0 || N < 0 || K < 0 || K % qk_of(fmt)) return KQ_ERR_SHAPE;
    if (M > kMaxDim || N > kMaxDim || K > kMaxDim) return KQ_ERR_SHAPE;
    return variant_for(fmt, M, N, K);
}

int kq_gemm(int fmt, const void *W, const void *a_q8, int64_t M, int64_t N, int64_t K,
            float *out, hipStream_t stream) {
    int rc = check_gemm(fmt, W, a_q8, M, N, K, out);
    if (rc <= 0) return rc;
    ActLayout L;
    act_layout(kq_act_fmt_for(fmt), M, K, &L);
    const char *base = static_cast<const char *>(a_q8);
    hipError_t e = kq::launch_gemm(
        fmt, W, reinterpret_cast<const int8_t *>(base), reinterpret_cast<const float *>(base + L.d),
        L.alpha >= 0 ? reinterpret_cast<const uint16_t *>(base + L.alpha) : nullptr, out, (int)M,
        (int)N, (int)K, stream);
    if (e != hipSuccess) return KQ_ERR_HIP;
    g_count[variant_for(fmt, M, N, K)].fetch_add(1);
    return KQ_OK;
}

int kq_gemm_subsums(int fmt, const void *W, const void *a_q8, int64_t M, int64_t N, int64_t K,
                    int32_t *sums, hipStream_t stream) {
    int rc = check_gemm(fmt, W, a_q8, M, N, K, sums);
    if (rc <= 0) return rc;
    const char *base = static_cast<const char *>(a_q8);
    hipError_t e = kq::launch_subsums(fmt, W, reinterpret_cast<const int8_t *>(base), sums,
                                      (int)M, (int)N, (int)K, stream);
    if (e != hipSuccess) return KQ_ERR_HIP;
    g_count[fmt == KQ_Q4_K ? V_SUBSUMS_Q4K : fmt == KQ_Q6_K ? V_SUBSUMS_Q6K
            : fmt == KQ_TQ ? V_SUBSUMS_TQ : V_SUBSUMS_TQ2]
        .fetch_add(1);
    return KQ_OK;
}

int kq_debug_unpack(int fmt, const void *W, int64_t nblocks, int8_t *q, int32_t *scales,
                    hipStream_t stream) {
    if (!qk_of(fmt)) return KQ_ERR_FMT;
    if (nblocks < 0 || nblocks > KQ_DEBUG_UNPACK_MAX_BLOCKS) return KQ_ERR_SHAPE;
    if (nblocks == 0) return KQ_OK;
    const bool ternary = fmt == KQ_TQ || fmt == KQ_TQ2;  // no scale fields
    if (!W || !q || (!ternary && !scales)) return KQ_ERR_NULL;
    if (!aligned16(W) || !aligned16(q) || ((uintptr_t)scales & 3u)) return KQ_ERR_ALIGN;
    return kq::launch_debug_unpack(fmt, W, nblocks, q, ternary ? nullptr : scales, stream) ==
                   hipSuccess
               ? KQ_OK
               : KQ_ERR_HIP;
}

int kq_gemm_id(int fmt, const void *W, int64_t n_experts, const void *a_q8, int64_t M, int64_t N,
               int64_t K, const int32_t *expert_offsets, const int32_t *rows, int64_t R, float *out,
               hipStream_t stream) {
    if (!qk_of(fmt)) return KQ_ERR_FMT;
    if (M < 0 || N < 0 || K < 0 || R < 0 || K % qk_of(fmt)) return KQ_ERR_SHAPE;
    if (n_experts < 1 || n_experts > KQ_GEMM_ID_MAX_EXPERTS) return KQ_ERR_SHAPE;
    if (M > kMaxDim || N > kMaxDim || K > kMaxDim || R > kMaxDim) return KQ_ERR_SHAPE;
    if ((M && K > kMaxBytes / M) || (N && K > kMaxBytes / N) || (R && N > kMaxBytes / R))
        return KQ_ERR_SHAPE;
    const int64_t rowbytes = (K / qk_of(fmt)) * bb_of(fmt);
    if (N && rowbytes && n_experts > kMaxBytes / (N * rowbytes)) return KQ_ERR_SHAPE;
    if (R == 0 || N == 0) return KQ_OK;
    if (M == 0) return KQ_ERR_SHAPE;  // routed rows but no token to read
    if (!W || !a_q8 || !expert_offsets || !rows || !out) return KQ_ERR_NULL;
    if (!aligned16(W) || !aligned16(a_q8) || !aligned16(out) || ((uintptr_t)expert_offsets & 3u) ||
        ((uintptr_t)rows & 3u))
        return KQ_ERR_ALIGN;
    // the tile kernel addresses one expert's weights and the activation
    // sections with 32-bit offsets (activation rows are gathered, never past M)
    const int64_t lim = (int64_t)1 << 31;
    if ((N + 256) * rowbytes >= lim || M * K >= lim || (K / qk_of(fmt)) * M * 4 >= lim ||
        (K / 256) * 2 * M * 16 >= lim)
        return KQ_ERR_UNSUPPORTED;
    const int64_t tiles = ((R + 63) / 64 + n_experts) * ((N + 127) / 128);
    if (tiles > INT32_MAX) return KQ_ERR_UNSUPPORTED;
    // the Q4_K persistent kernel counts (tile, superblock) steps per
    // workgroup in int32; a workgroup may own every tile
    if (fmt == KQ_Q4_K && tiles * (K / 256) > INT32_MAX) return KQ_ERR_UNSUPPORTED;
    ActLayout L;
    act_layout(kq_act_fmt_for(fmt), M, K, &L);
    const char *base = static_cast<const char *>(a_q8);
    const int8_t *qs = reinterpret_cast<const int8_t *>(base);
    const float *da = reinterpret_cast<const float *>(base + L.d);
    const uint16_t *alpha = L.alpha >= 0 ? reinterpret_cast<const uint16_t *>(base + L.alpha) : nullptr;
    // Q4_K runs only on the register-unpack tile kernel (per-tile output
    // offsets within 2^31 bytes); wider Q4_K shapes are declined
    if (fmt == KQ_Q4_K && !kq::q4k_id_tile_ok((int)N, (int)K)) return KQ_ERR_UNSUPPORTED;
    const bool q4k_tile = fmt == KQ_Q4_K;
    hipError_t e = q4k_tile ? kq::launch_gemm_q4k_id(W, (int)n_experts, N * rowbytes, qs, da, alpha,
                                                     expert_offsets, rows, (int)R, out, (int)M, (int)N,
                                                     (int)K, stream)
                            : kq::launch_gemm_id(fmt, W, (int)n_experts, N * rowbytes, qs, da, alpha,
                                                 expert_offsets, rows, (int)R, out, (int)M, (int)N,
                                                 (int)K, stream);
    if (e != hipSuccess) return KQ_ERR_HIP;
    g_count[q4k_tile ? V_GEMM_ID_Q4K_64x128 : V_GEMM_ID_128x128].fetch_add(1);
    return KQ_OK;
}

int kq_calib_launch(int kind, int param, const void *buf, int64_t bytes, double *work,
                    hipStream_t stream) {
    if (kind < KQ_CALIB_MFMA_I8 || kind > KQ_CALIB_HBM_READ) return KQ_ERR_FMT;
    if (!work) return KQ_ERR_NULL;
    if (kind == KQ_CALIB_MFMA_I8_VALU && param != 2 && param != 4 && param != 6 && param != 8)
        return KQ_ERR_SHAPE;
    if (kind == KQ_CALIB_HBM_READ) {
        if (!buf) return KQ_ERR_NULL;
        if (bytes < 16 || bytes % 16 || bytes > kMaxBytes) return KQ_ERR_SHAPE;
        if (!aligned16(buf)) return KQ_ERR_ALIGN;
    }
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
        return KQ_ERR_HIP;
    return kq::launch_calib(kind, param, buf, bytes, cus, work, stream) == hipSuccess ? KQ_OK
                                                                                      : KQ_ERR_HIP;
}

int kq_num_variants(void) { return V_COUNT; }

const char *kq_variant_name(int variant) {
    return (variant >= 0 && variant < V_COUNT) ? kVariantNames[variant] : nullptr;
}

uint64_t kq_dispatch_count(int variant) {
    return (variant >= 0 && variant < V_COUNT) ? g_count[variant].load() : 0;
}

void kq_dispatch_reset(void) {
    for (auto &c : g_count) c.store(0);
}

const char *kq_strerror(int status) {
    switch (status) {
        case KQ_OK: return "ok";
        case KQ_ERR_FMT: return "unknown weight or activation format";
        case KQ_ERR_SHAPE: return "invalid shape (negative size, K not a multiple of the block, or size overflow)";
        case KQ_ERR_NULL: return "null pointer with nonzero work";
        case KQ_ERR_ALIGN: return "pointer not 16-byte aligned";
        case KQ_ERR_UNSUPPORTED: return "no verified kernel variant for this case";
        case KQ_ERR_HIP: return "HIP runtime error at launch";
        default: return "unknown status";
    }
}

int kq_version(void) { return KQ_VERSION; }

}  // extern "C"
