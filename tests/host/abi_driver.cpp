// Host-side driver for the C ABI's argument handling (kq_api.cpp), built with
// AddressSanitizer and UndefinedBehaviorSanitizer by
// tests/test_host_sanitizers.py.  The kernel launchers and the two HIP runtime
// calls kq_api.cpp makes are replaced by stubs that record their arguments,
// so every entry point runs on extreme sizes (signed overflow in a size
// computation is reported) and the pointers handed to the launchers can be
// checked against the documented section offsets.  Prints "ok" and exits 0
// when every expectation holds.
#include "../../include/kq.h"

#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstdio>

#include "../../block_quantized_matmul_act_amd/csrc/kq_calib.hpp"
#include "../../block_quantized_matmul_act_amd/csrc/kq_hooks.hpp"
#include "../../block_quantized_matmul_act_amd/csrc/kq_launch.hpp"

namespace {
int failures = 0;
#define EXPECT(c)                                                       \
    do {                                                                \
        if (!(c)) {                                                     \
            std::fprintf(stderr, "%s:%d: %s\n", __FILE__, __LINE__, #c); \
            ++failures;                                                 \
        }                                                               \
    } while (0)

struct Rec {
    int calls = 0;
    const void *p[4] = {};
    int64_t n[3] = {};
} rq, rg, rs, rd, ri, rx;
}  // namespace

namespace kq {
hipError_t launch_quant_act(int, const float *x, int8_t *qs, float *d, int16_t *bsums, uint16_t *alpha,
                            int64_t M, int64_t K, hipStream_t) {
    ++rq.calls;
    rq.p[0] = qs;
    rq.p[1] = d;
    rq.p[2] = bsums;
    rq.p[3] = alpha;
    rq.n[0] = M;
    rq.n[1] = K;
    (void)x;
    return hipSuccess;
}
hipError_t launch_gemm(int, const void *, const int8_t *qs, const float *da, const uint16_t *alpha, float *,
                       int M, int N, int K, hipStream_t) {
    ++rg.calls;
    rg.p[0] = qs;
    rg.p[1] = da;
    rg.p[2] = alpha;
    rg.n[0] = M;
    rg.n[1] = N;
    rg.n[2] = K;
    return hipSuccess;
}
hipError_t launch_subsums(int, const void *, const int8_t *, int32_t *, int, int, int, hipStream_t) {
    ++rs.calls;
    return hipSuccess;
}
bool gemv_choice(int fmt, int M, int, int) { return fmt >= 2 && fmt <= 4 && M <= 4; }
hipError_t launch_gemv(int, const void *, const int8_t *, const float *, float *, int, int, int, hipStream_t) {
    return hipSuccess;
}
bool tq_tile_choice(int M, int, int K) { return M > 8 && K % 256 == 0; }
hipError_t launch_gemm_tq_tile(const void *, const int8_t *, const float *, float *, int, int, int, hipStream_t) {
    return hipSuccess;
}
bool ring_choice(int fmt, int M, int N, int K) {
    return fmt >= 2 && fmt <= 4 && M >= 1 && M <= 64 && K >= 256 && K % 256 == 0 && !gemv_choice(fmt, M, N, K);
}
int num_cus() { return 256; }
bool tile_split_choice(int fmt, int M, int N, int K) {
    return fmt >= 2 && fmt <= 4 && M > 0 && K >= 1024 &&
           2 * (((int64_t)M + 127) / 128) * (((int64_t)N + 127) / 128) <= 256 &&
           K / 2 + 256 + (int64_t)M * N / 1536 < K;
}
int q4k_kernel_choice(int M, int, int) {
    return M <= 2 ? Q4K_MATVEC : M <= 16 ? Q4K_FEW_SPLIT : M <= 64 ? Q4K_RING_KP : Q4K_TILE128;
}
hipError_t launch_calib(int, int, const void *, int64_t, int, double *work, hipStream_t) {
    *work = 1.0;
    return hipSuccess;
}
hipError_t launch_gemm_id(int, const void *, int n_experts, int64_t expert_bytes, const int8_t *qs,
                          const float *da, const uint16_t *alpha, const int32_t *, const int32_t *, int R,
                          float *, int M, int N, int K, hipStream_t) {
    ++ri.calls;
    ri.p[0] = qs;
    ri.p[1] = da;
    ri.p[2] = alpha;
    ri.n[0] = n_experts;
    ri.n[1] = expert_bytes;
    ri.n[2] = (int64_t)R * 1000000 + M;
    (void)N;
    (void)K;
    return hipSuccess;
}
bool q4k_id_tile_ok(int N, int K) { (void)K; return (int64_t)64 * N * 4 < ((int64_t)1 << 31); }
hipError_t launch_gemm_q4k_id(const void *, int n_experts, int64_t expert_bytes, const int8_t *qs, const float *da,
                              const uint16_t *alpha, const int32_t *, const int32_t *, int R, float *, int M, int,
                              int, hipStream_t) {
    ++rx.calls;
    rx.p[0] = qs;
    rx.p[1] = da;
    rx.p[2] = alpha;
    rx.n[0] = n_experts;
    rx.n[1] = expert_bytes;
    rx.n[2] = (int64_t)R * 1000000 + M;
    return hipSuccess;
}
hipError_t launch_debug_unpack(int, const void *, int64_t nblocks, int8_t *, int32_t *, hipStream_t) {
    ++rd.calls;
    rd.n[0] = nblocks;
    return hipSuccess;
}
}  // namespace kq

extern "C" hipError_t hipGetDevice(int *d) {
    *d = 0;
    return hipSuccess;
}
extern "C" hipError_t hipDeviceGetAttribute(int *v, hipDeviceAttribute_t, int) {
    *v = 256;
    return hipSuccess;
}

int main() {
    const int64_t big[] = {-(int64_t)1 << 62, -1, 0, 1, 7, 128, 255, 256, 4096, 14336, INT32_MAX,
                           (int64_t)INT32_MAX + 1, (int64_t)1 << 40, INT64_MAX, INT64_MIN};
    char *A = reinterpret_cast<char *>((uintptr_t)1 << 20);  // never dereferenced
    hipStream_t s = nullptr;

    // every entry point on every combination of extreme sizes
    for (int fmt = -1; fmt <= 4; ++fmt)
        for (int64_t M : big)
            for (int64_t N : big)
                for (int64_t K : big) {
                    (void)kq_weight_bytes(fmt, N, K);
                    (void)kq_act_bytes(fmt, M, K);
                    for (int sec = -1; sec <= 4; ++sec) (void)kq_act_section_offset(fmt, sec, M, K);
                    (void)kq_select_variant(fmt, M, N, K);
                    // only shapes the library accepts reach a launcher; all
                    // others return a status first
                    const int rc = kq_gemm(fmt, A, A, M, N, K, reinterpret_cast<float *>(A), s);
                    EXPECT(rc == KQ_OK || rc == KQ_ERR_FMT || rc == KQ_ERR_SHAPE || rc == KQ_ERR_UNSUPPORTED);
                    if (rc == KQ_OK && M > 0 && N > 0) {
                        EXPECT(M <= INT32_MAX && N <= INT32_MAX && K <= INT32_MAX);
                        EXPECT((M + 128) * K < ((int64_t)1 << 31));
                    }
                    (void)kq_gemm_subsums(fmt, A, A, M, N, K, reinterpret_cast<int32_t *>(A), s);
                    for (int64_t E : {(int64_t)-1, (int64_t)0, (int64_t)1, (int64_t)8, (int64_t)65537, INT64_MAX}) {
                        const int rc2 = kq_gemm_id(fmt, A, E, A, M, N, K, reinterpret_cast<int32_t *>(A),
                                                   reinterpret_cast<int32_t *>(A), K, reinterpret_cast<float *>(A), s);
                        EXPECT(rc2 == KQ_OK || rc2 == KQ_ERR_FMT || rc2 == KQ_ERR_SHAPE || rc2 == KQ_ERR_UNSUPPORTED);
                    }
                    (void)kq_quantize_act(fmt, reinterpret_cast<float *>(A), M, K, A, s);
                }
    for (int fmt = -1; fmt <= 4; ++fmt)
        for (int64_t n : big) (void)kq_debug_unpack(fmt, A, n, reinterpret_cast<int8_t *>(A), reinterpret_cast<int32_t *>(A), s);

    // pointers handed to the launchers are the documented sections
    for (int64_t M : {1, 7, 64, 513})
        for (int64_t K : {256, 768, 4096}) {
            rq = Rec{};
            rg = Rec{};
            EXPECT(kq_quantize_act(KQ_ACT_Q8_K, reinterpret_cast<float *>(A), M, K, A, s) == KQ_OK);
            EXPECT(rq.calls == 1 && rq.n[0] == M && rq.n[1] == K);
            EXPECT(rq.p[0] == A);
            EXPECT(rq.p[1] == A + kq_act_section_offset(KQ_ACT_Q8_K, KQ_SEC_D, M, K));
            EXPECT(rq.p[2] == A + kq_act_section_offset(KQ_ACT_Q8_K, KQ_SEC_BSUMS, M, K));
            EXPECT(rq.p[3] == A + kq_act_section_offset(KQ_ACT_Q8_K, KQ_SEC_ALPHA, M, K));
            EXPECT(kq_gemm(KQ_Q4_K, A, A, M, 96, K, reinterpret_cast<float *>(A), s) == KQ_OK);
            EXPECT(rg.calls == 1 && rg.n[0] == M && rg.n[1] == 96 && rg.n[2] == K);
            EXPECT(rg.p[0] == A);
            EXPECT(rg.p[1] == A + kq_act_section_offset(KQ_ACT_Q8_K, KQ_SEC_D, M, K));
            EXPECT(rg.p[2] == A + kq_act_section_offset(KQ_ACT_Q8_K, KQ_SEC_ALPHA, M, K));
            // Q8_128: no sums, no min operands
            rq = Rec{};
            EXPECT(kq_quantize_act(KQ_ACT_Q8_128, reinterpret_cast<float *>(A), M, K, A, s) == KQ_OK);
            EXPECT(rq.p[1] == A + kq_act_section_offset(KQ_ACT_Q8_128, KQ_SEC_D, M, K));
            EXPECT(rq.p[2] == nullptr && rq.p[3] == nullptr);
            rg = Rec{};
            EXPECT(kq_gemm(KQ_TQ, A, A, M, 96, K, reinterpret_cast<float *>(A), s) == KQ_OK);
            EXPECT(rg.p[2] == nullptr);
        }
    // the expert-indexed product hands the launcher the documented sections
    // and the byte stride of one expert's weights
    ri = Rec{};
    EXPECT(kq_gemm_id(KQ_Q6_K, A, 8, A, 100, 96, 512, reinterpret_cast<int32_t *>(A),
                      reinterpret_cast<int32_t *>(A), 300, reinterpret_cast<float *>(A), s) == KQ_OK);
    EXPECT(ri.calls == 1 && ri.n[0] == 8 && ri.n[1] == 96 * 2 * 210 && ri.n[2] == 300 * 1000000 + 100);
    EXPECT(ri.p[1] == A + kq_act_section_offset(KQ_ACT_Q8_K, KQ_SEC_D, 100, 512));
    EXPECT(ri.p[2] == A + kq_act_section_offset(KQ_ACT_Q8_K, KQ_SEC_ALPHA, 100, 512));
    // Q4_K goes to the register-unpack tile kernel's gather mode, with the same
    // sections, K = 0 included (its launcher writes the zeros)
    ri = Rec{};
    rx = Rec{};
    EXPECT(kq_gemm_id(KQ_Q4_K, A, 8, A, 100, 96, 512, reinterpret_cast<int32_t *>(A),
                      reinterpret_cast<int32_t *>(A), 300, reinterpret_cast<float *>(A), s) == KQ_OK);
    EXPECT(ri.calls == 0 && rx.calls == 1 && rx.n[0] == 8 && rx.n[1] == 96 * 2 * 144 &&
           rx.n[2] == 300 * 1000000 + 100);
    EXPECT(rx.p[1] == A + kq_act_section_offset(KQ_ACT_Q8_K, KQ_SEC_D, 100, 512));
    EXPECT(rx.p[2] == A + kq_act_section_offset(KQ_ACT_Q8_K, KQ_SEC_ALPHA, 100, 512));
    EXPECT(kq_gemm_id(KQ_Q4_K, A, 8, A, 100, 96, 0, reinterpret_cast<int32_t *>(A),
                      reinterpret_cast<int32_t *>(A), 300, reinterpret_cast<float *>(A), s) == KQ_OK);
    EXPECT(ri.calls == 0 && rx.calls == 2);
    // N >= 2^23 (64 output rows of N floats past 2^31 bytes) is declined
    EXPECT(kq_gemm_id(KQ_Q4_K, A, 8, A, 100, (int64_t)1 << 23, 256, reinterpret_cast<int32_t *>(A),
                      reinterpret_cast<int32_t *>(A), 300, reinterpret_cast<float *>(A), s) == KQ_ERR_UNSUPPORTED);
    EXPECT(ri.calls == 0 && rx.calls == 2);
    EXPECT(kq_gemm_id(KQ_Q4_K, A, 8, A, 100, ((int64_t)1 << 23) - 1, 256, reinterpret_cast<int32_t *>(A),
                      reinterpret_cast<int32_t *>(A), 300, reinterpret_cast<float *>(A), s) == KQ_OK);
    EXPECT(ri.calls == 0 && rx.calls == 3);
    // the loader hook reaches its launcher only with a valid count
    rd = Rec{};
    EXPECT(kq_debug_unpack(KQ_Q4_K, A, 10, reinterpret_cast<int8_t *>(A), reinterpret_cast<int32_t *>(A), s) == KQ_OK);
    EXPECT(rd.calls == 1 && rd.n[0] == 10);
    EXPECT(kq_debug_unpack(KQ_Q4_K, A, KQ_DEBUG_UNPACK_MAX_BLOCKS + 1, reinterpret_cast<int8_t *>(A),
                           reinterpret_cast<int32_t *>(A), s) == KQ_ERR_SHAPE);
    EXPECT(rd.calls == 1);
    double w = 0;
    EXPECT(kq_calib_launch(KQ_CALIB_MFMA_I8, 0, nullptr, 0, &w, s) == KQ_OK && w == 1.0);

    if (failures) {
        std::fprintf(stderr, "%d failures\n", failures);
        return 1;
    }
    std::printf("ok\n");
    return 0;
}
