"""CPU tests of the C ABI: the library loads, exports every symbol the header
declares, and rejects invalid arguments with its status codes before any HIP
call (so they run without a GPU)."""
from __future__ import annotations

import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kq.h")


@pytest.fixture(scope="module")
def kq():
    import block_quantized_matmul_act_amd as kq
    if not os.path.exists(kq.LIB_PATH):
        from block_quantized_matmul_act_amd import build
        build.build()
    kq.lib()
    return kq


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(kq_\w+)\s*\(", text)))


def test_header_declares_the_boundary():
    names = declared_functions()
    for required in ("kq_quantize_act", "kq_gemm", "kq_weight_bytes", "kq_act_bytes",
                     "kq_gemm_subsums", "kq_dispatch_count", "kq_strerror", "kq_version"):
        assert required in names


def test_every_declared_symbol_is_exported(kq):
    L = kq.lib()
    names = declared_functions()
    assert set(names) == set(kq.SIGNATURES), "binding and header disagree"
    for name in names:
        assert hasattr(L, name), name


def test_version_and_strings(kq):
    assert kq.kq_version() == 2
    for st in (kq.KQ_OK, kq.KQ_ERR_FMT, kq.KQ_ERR_SHAPE, kq.KQ_ERR_NULL, kq.KQ_ERR_ALIGN,
               kq.KQ_ERR_UNSUPPORTED, kq.KQ_ERR_HIP):
        s = kq.kq_strerror(st)
        assert s and s != "unknown status"
    assert kq.kq_strerror(12345) == "unknown status"


def _a256(v):
    return (v + 255) // 256 * 256


@pytest.mark.parametrize("M,K", [(1, 256), (8, 512), (7, 768), (513, 4096), (0, 256)])
def test_act_layout_q8k(kq, M, K):
    # four sections at 256-byte-aligned offsets: qs [M][K], d [K/256][M],
    # bsums [M][K/16], alpha bf16 [K/256][2][M][8]
    off_d = _a256(M * K)
    off_b = off_d + _a256(M * (K // 256) * 4)
    off_a = off_b + _a256(M * (K // 16) * 2)
    total = off_a + _a256((K // 256) * 2 * M * 8 * 2)
    assert kq.kq_act_section_offset(kq.KQ_ACT_Q8_K, kq.KQ_SEC_QS, M, K) == 0
    assert kq.kq_act_section_offset(kq.KQ_ACT_Q8_K, kq.KQ_SEC_D, M, K) == off_d
    assert kq.kq_act_section_offset(kq.KQ_ACT_Q8_K, kq.KQ_SEC_BSUMS, M, K) == off_b
    assert kq.kq_act_section_offset(kq.KQ_ACT_Q8_K, kq.KQ_SEC_ALPHA, M, K) == off_a
    assert kq.kq_act_section_offset(kq.KQ_ACT_Q8_K, 4, M, K) == -1
    assert kq.kq_act_bytes(kq.KQ_ACT_Q8_K, M, K) == total


@pytest.mark.parametrize("M,K", [(1, 128), (9, 384), (2048, 5120)])
def test_act_layout_q8_128(kq, M, K):
    off_d = _a256(M * K)
    assert kq.kq_act_section_offset(kq.KQ_ACT_Q8_128, kq.KQ_SEC_D, M, K) == off_d
    assert kq.kq_act_section_offset(kq.KQ_ACT_Q8_128, kq.KQ_SEC_BSUMS, M, K) == -1
    assert kq.kq_act_section_offset(kq.KQ_ACT_Q8_128, kq.KQ_SEC_ALPHA, M, K) == -1
    assert kq.kq_act_bytes(kq.KQ_ACT_Q8_128, M, K) == off_d + _a256(M * (K // 128) * 4)


def test_size_queries(kq):
    assert kq.kq_weight_bytes(kq.KQ_Q4_K, 14336, 4096) == 14336 * 16 * 144 == 33030144
    assert kq.kq_weight_bytes(kq.KQ_Q6_K, 4096, 14336) == 4096 * 56 * 210 == 48168960
    assert kq.kq_weight_bytes(kq.KQ_TQ, 17408, 5120) == 17408 * 40 * 28 == 19496960
    assert kq.kq_weight_bytes(kq.KQ_Q4_K, 10, 100) == 0          # K not a multiple of 256
    assert kq.kq_weight_bytes(kq.KQ_TQ, 10, 384) == 10 * 3 * 28
    assert kq.kq_weight_bytes(99, 10, 256) == 0
    assert kq.kq_weight_bytes(kq.KQ_Q4_K, -1, 256) == 0
    assert kq.kq_act_bytes(kq.KQ_ACT_Q8_K, 4, 128) == 0           # K not a multiple of 256
    assert kq.kq_act_bytes(7, 4, 256) == 0
    assert kq.kq_act_fmt_for(kq.KQ_Q4_K) == kq.KQ_ACT_Q8_K
    assert kq.kq_act_fmt_for(kq.KQ_Q6_K) == kq.KQ_ACT_Q8_K
    assert kq.kq_act_fmt_for(kq.KQ_TQ) == kq.KQ_ACT_Q8_128
    assert kq.kq_act_fmt_for(kq.KQ_TQ2) == kq.KQ_ACT_Q8_128
    assert kq.kq_weight_bytes(kq.KQ_TQ2, 17408, 5120) == 17408 * 40 * 34
    assert kq.kq_weight_bytes(kq.KQ_TQ2, 3, 200) == 0             # K not a multiple of 128
    assert kq.kq_act_fmt_for(0) == kq.KQ_ERR_FMT


def _raw(kq):
    return kq.lib()


def test_gemm_validation_without_hip(kq):
    L = _raw(kq)
    A = 1 << 20   # a fake, aligned "device address": never dereferenced on these paths
    s = None
    assert L.kq_gemm(0, A, A, 8, 8, 256, A, s) == kq.KQ_ERR_FMT
    assert L.kq_gemm(kq.KQ_Q4_K, A, A, 8, 8, 300, A, s) == kq.KQ_ERR_SHAPE
    assert L.kq_gemm(kq.KQ_TQ, A, A, 8, 8, 200, A, s) == kq.KQ_ERR_SHAPE
    assert L.kq_gemm(kq.KQ_Q4_K, A, A, -1, 8, 256, A, s) == kq.KQ_ERR_SHAPE
    assert L.kq_gemm(kq.KQ_Q4_K, A, A, 8, -3, 256, A, s) == kq.KQ_ERR_SHAPE
    assert L.kq_gemm(kq.KQ_Q4_K, A, A, 8, 8, -256, A, s) == kq.KQ_ERR_SHAPE
    assert L.kq_gemm(kq.KQ_Q4_K, A, A, 1 << 33, 8, 256, A, s) == kq.KQ_ERR_SHAPE
    assert L.kq_gemm(kq.KQ_Q4_K, A, A, 1 << 30, 1 << 30, 1 << 20, A, s) == kq.KQ_ERR_SHAPE
    assert L.kq_gemm(kq.KQ_Q4_K, None, A, 8, 8, 256, A, s) == kq.KQ_ERR_NULL
    assert L.kq_gemm(kq.KQ_Q4_K, A, None, 8, 8, 256, A, s) == kq.KQ_ERR_NULL
    assert L.kq_gemm(kq.KQ_Q4_K, A, A, 8, 8, 256, None, s) == kq.KQ_ERR_NULL
    assert L.kq_gemm(kq.KQ_Q4_K, A + 4, A, 8, 8, 256, A, s) == kq.KQ_ERR_ALIGN
    assert L.kq_gemm(kq.KQ_Q4_K, A, A + 8, 8, 8, 256, A, s) == kq.KQ_ERR_ALIGN
    assert L.kq_gemm(kq.KQ_Q4_K, A, A, 8, 8, 256, A + 2, s) == kq.KQ_ERR_ALIGN
    # 32-bit tile offsets: 128*K must stay below 2^31 bytes
    assert L.kq_gemm(kq.KQ_Q4_K, A, A, 8, 8, 1 << 24, A, s) == kq.KQ_ERR_UNSUPPORTED
    # ... and so must the output plus the 128 rows a last tile hangs past M:
    # 131000 x 4096 fp32 is below 2^31 bytes, 131128 x 4096 is not
    assert 131000 * 4096 * 4 < 1 << 31 <= (131000 + 128) * 4096 * 4
    assert L.kq_gemm(kq.KQ_Q4_K, A, A, 131000, 4096, 256, A, s) == kq.KQ_ERR_UNSUPPORTED
    # ... and the weights plus 256 overhanging rows (Q4_K, K = 4096: 2304 B a row)
    n = (1 << 31) // 2304 - 100
    assert n * 2304 < 1 << 31 <= (n + 256) * 2304
    assert L.kq_gemm(kq.KQ_Q4_K, A, A, 8, n, 4096, A, s) == kq.KQ_ERR_UNSUPPORTED
    # empty problems are a no-op that succeeds, even with null pointers
    assert L.kq_gemm(kq.KQ_Q4_K, None, None, 0, 8, 256, None, s) == kq.KQ_OK
    assert L.kq_gemm(kq.KQ_Q6_K, None, None, 8, 0, 256, None, s) == kq.KQ_OK
    assert L.kq_gemm_subsums(kq.KQ_TQ, None, None, 0, 0, 128, None, s) == kq.KQ_OK
    assert L.kq_gemm_subsums(kq.KQ_TQ, A, A, 4, 4, 100, A, s) == kq.KQ_ERR_SHAPE
    assert L.kq_gemm_subsums(9, A, A, 4, 4, 128, A, s) == kq.KQ_ERR_FMT


def test_quantize_validation_without_hip(kq):
    L = _raw(kq)
    A = 1 << 20
    assert L.kq_quantize_act(3, A, 4, 256, A, None) == kq.KQ_ERR_FMT
    assert L.kq_quantize_act(kq.KQ_ACT_Q8_K, A, 4, 128, A, None) == kq.KQ_ERR_SHAPE
    assert L.kq_quantize_act(kq.KQ_ACT_Q8_128, A, 4, 64, A, None) == kq.KQ_ERR_SHAPE
    assert L.kq_quantize_act(kq.KQ_ACT_Q8_K, A, -4, 256, A, None) == kq.KQ_ERR_SHAPE
    assert L.kq_quantize_act(kq.KQ_ACT_Q8_K, None, 4, 256, A, None) == kq.KQ_ERR_NULL
    assert L.kq_quantize_act(kq.KQ_ACT_Q8_K, A, 4, 256, None, None) == kq.KQ_ERR_NULL
    assert L.kq_quantize_act(kq.KQ_ACT_Q8_K, A + 4, 4, 256, A, None) == kq.KQ_ERR_ALIGN
    assert L.kq_quantize_act(kq.KQ_ACT_Q8_K, None, 0, 256, None, None) == kq.KQ_OK


def test_variants_and_counters(kq):
    n = kq.kq_num_variants()
    names = [kq.kq_variant_name(v) for v in range(n)]
    assert len(set(names)) == n and all(names)
    assert kq.kq_variant_name(n) is None and kq.kq_variant_name(-1) is None
    kq.kq_dispatch_reset()
    assert all(kq.kq_dispatch_count(v) == 0 for v in range(n))
    for fmt in (kq.KQ_Q4_K, kq.KQ_Q6_K, kq.KQ_TQ, kq.KQ_TQ2):
        for M in (1, 8, 64, 65, 2048):
            v = kq.kq_select_variant(fmt, M, 4096, 4096 if fmt < kq.KQ_TQ else 5120)
            assert 0 <= v < n
    # Q4_K tile heights: 128 x 128 above 256 such tiles, else 64 x 128; the
    # 8-wave 64 x 128 build when the 64-row tiles are at most one per CU
    # (the CU count without a device is taken as 256)
    q4 = lambda M, N, K: kq.kq_variant_name(kq.kq_select_variant(kq.KQ_Q4_K, M, N, K))
    assert q4(2048, 2048, 4096) == "gemm_q4_k_64x128"    # 16 x 16 tiles (32 x 16 of 64 rows)
    assert q4(2048, 2049, 4096) == "gemm_q4_k_128x128"   # 16 x 17
    assert q4(1536, 4096, 4096) == "gemm_q4_k_128x128"   # 12 x 32
    assert q4(512, 4096, 4096) == "gemm_q4_k_64x128_k2"  # 8 x 32 tiles of 64 rows
    assert q4(576, 4096, 4096) == "gemm_q4_k_64x128"     # 9 x 32
    assert q4(2048, 14336, 4096) == "gemm_q4_k_128x128"
    assert q4(65, 4000, 512) == "gemm_q4_k_64x128_k2"
    # 3 .. 64 tokens: the Q4_K ring kernel once 32-row workgroups would
    # outnumber the CUs (256 here); below that the four-wave split kernel up
    # to 16 tokens while 32-row workgroups cover more than half the CUs, and
    # the ring kernel with 2, 4 or 8 K-parts otherwise
    assert q4(64, 4096, 4096) == "gemm_q4_k_ring_kp"
    assert q4(17, 4096, 4096) == "gemm_q4_k_ring_kp"
    assert q4(16, 4096, 4096) == "gemm_q4_k_ring_kp"    # 128 workgroups of 32 rows
    assert q4(16, 4128, 4096) == "gemm_q4_k_m16"        # 129
    assert q4(64, 14336, 4096) == "gemm_q4_k_m64_ring"
    assert q4(17, 8224, 4096) == "gemm_q4_k_m64_ring"   # 257 row pairs of 32
    assert q4(17, 8192, 4096) == "gemm_q4_k_ring_kp"    # 256
    assert q4(16, 8224, 4096) == "gemm_q4_k_m64_ring"   # its 16-row build
    assert q4(16, 8192, 4096) == "gemm_q4_k_m16"
    assert q4(64, 10880, 4096) == "gemm_q4_k_m64_ring"
    assert q4(3, 14336, 4096) == "gemm_q4_k_m64_ring"
    # Q6_K: the matrix-vector kernel up to 4 tokens (K a multiple of 2048),
    # the K-split ring kernel past it up to 64, the tile kernel above
    q6 = lambda M, N, K: kq.kq_variant_name(kq.kq_select_variant(kq.KQ_Q6_K, M, N, K))
    assert q6(4, 4096, 14336) == "gemm_q6_k_matvec"
    assert q6(5, 4096, 14336) == "gemm_q6_k_ring"
    assert q6(9, 4096, 14336) == "gemm_q6_k_ring"
    assert q6(64, 4096, 14336) == "gemm_q6_k_ring"
    # 65 .. 512 tokens: the ring kernel in 64-token slices where the 128 x
    # 128 tile kernels leave most CUs idle (narrow weights, long K)
    for M in (65, 128, 200, 256):
        assert q6(M, 4096, 14336) == "gemm_q6_k_ring"
    # ... and the tile kernel with K in two parts where its tiles cover at
    # most half the CUs and the ring kernel would need more rounds
    assert q6(512, 4096, 14336) == "gemm_q6_k_128x128_k2"  # 128 tiles over 14336 of K
    assert q6(513, 1024, 4096) == "gemm_q6_k_128x128_k2"   # past 512 tokens (40 tiles)
    assert q6(1024, 4096, 14336) == "gemm_q6_k_128x128"    # 256 tiles
    assert q6(512, 1024, 4096) == "gemm_q6_k_ring"
    assert q6(128, 14336, 4096) == "gemm_q6_k_128x128_k2"  # 112 tiles
    assert q6(256, 14336, 4096) == "gemm_q6_k_128x128"     # 224 tiles
    assert q6(300, 4000, 512) == "gemm_q6_k_128x128"       # K under 1024
    assert q6(300, 4000, 2048) == "gemm_q6_k_128x128"      # half of K under the split's cost
    assert q6(130, 72, 512) == "gemm_q6_k_128x128"      # one tile, short K
    assert q4(128, 4096, 14336) == "gemm_q4_k_ring_kp"
    assert q4(256, 4096, 14336) == "gemm_q4_k_ring_kp"
    assert q4(384, 4096, 14336) == "gemm_q4_k_64x128_k2"
    assert q4(128, 14336, 4096) != "gemm_q4_k_ring_kp"
    assert q6(4, 4096, 14336 + 256) == "gemm_q6_k_ring"  # K not a multiple of 2048
    assert q6(1, 100, 256) == "gemm_q6_k_ring"
    # base-3 ternary: the register-unpack tile kernel when K is a multiple of
    # 256, the digit-plane tile kernel otherwise
    tq = lambda M, N, K: kq.kq_variant_name(kq.kq_select_variant(kq.KQ_TQ, M, N, K))
    assert tq(2048, 17408, 5120) == "gemm_tq_128x128_reg"
    assert tq(2048, 17408, 5248) == "gemm_tq_128x128"
    # ... and the K-split ring kernel past the matrix-vector kernel up to 64
    # tokens (K a multiple of 256)
    assert tq(4, 17408, 5120) == "gemm_tq_matvec"
    assert tq(5, 17408, 5120) == "gemm_tq_ring"
    assert tq(9, 17408, 5120) == "gemm_tq_ring"
    assert tq(64, 17408, 5120) == "gemm_tq_ring"
    assert tq(1, 17408, 5120 + 256) == "gemm_tq_ring"   # K not a multiple of 1024
    assert tq(9, 17408, 5120 + 128) == "gemm_tq_128x128"
    for M in (65, 256):
        assert tq(M, 4096, 14336) == "gemm_tq_ring"
    assert tq(128, 17408, 5120) == "gemm_tq_128x128"     # 136 tiles: whole K
    assert tq(512, 4096, 14336) == "gemm_tq_128x128_k2"
    assert tq(9, 4096, 5120 + 128) == "gemm_tq_128x128_k2"
    # two-bit ternary: the matrix-vector kernel up to 4 tokens (K a multiple
    # of 1024), the K-split ring kernel up to 64 (K a multiple of 256), the
    # tile kernel otherwise
    tq2 = lambda M, N, K: kq.kq_variant_name(kq.kq_select_variant(kq.KQ_TQ2, M, N, K))
    for M in (1, 4):
        assert tq2(M, 4096, 5120) == "gemm_tq2_matvec"
    for M in (5, 8, 64):
        assert tq2(M, 4096, 5120) == "gemm_tq2_ring"
    assert tq2(1, 4096, 5120 + 256) == "gemm_tq2_ring"
    assert tq2(65, 4096, 5120) == "gemm_tq2_ring"
    assert tq2(256, 4096, 14336) == "gemm_tq2_ring"
    assert tq2(512, 4096, 14336) == "gemm_tq2_128x128_k2"
    assert tq2(128, 17408, 5120) == "gemm_tq2_128x128"
    assert tq2(2048, 4096, 5120) == "gemm_tq2_128x128"
    assert tq2(8, 4096, 5120 + 128) == "gemm_tq2_128x128_k2"  # 32 tiles: K in two parts
    assert tq2(8, 16384, 5120 + 128) == "gemm_tq2_128x128_k2"  # 128 tiles: two parts fill the CUs
    assert tq2(8, 16512, 5120 + 128) == "gemm_tq2_128x128"     # 129 tiles
    assert kq.kq_select_variant(0, 1, 1, 256) == kq.KQ_ERR_FMT
    assert kq.kq_select_variant(kq.KQ_Q4_K, 1, 1, 100) == kq.KQ_ERR_SHAPE


def test_calib_rejects_bad_arguments(kq):
    L = kq.lib()
    import ctypes
    w = ctypes.c_double(0.0)
    assert L.kq_calib_launch(5, 0, None, 0, ctypes.byref(w), None) == kq.KQ_ERR_FMT
    assert L.kq_calib_launch(-1, 0, None, 0, ctypes.byref(w), None) == kq.KQ_ERR_FMT
    assert L.kq_calib_launch(kq.KQ_CALIB_MFMA_I8, 0, None, 0, None, None) == kq.KQ_ERR_NULL
    for p in (0, 1, 3, 10):
        assert L.kq_calib_launch(kq.KQ_CALIB_MFMA_I8_VALU, p, None, 0, ctypes.byref(w), None) == kq.KQ_ERR_SHAPE
    R = kq.KQ_CALIB_HBM_READ
    assert L.kq_calib_launch(R, 0, None, 1024, ctypes.byref(w), None) == kq.KQ_ERR_NULL
    assert L.kq_calib_launch(R, 0, 4096, 0, ctypes.byref(w), None) == kq.KQ_ERR_SHAPE
    assert L.kq_calib_launch(R, 0, 4096, 24, ctypes.byref(w), None) == kq.KQ_ERR_SHAPE
    assert L.kq_calib_launch(R, 0, 4104, 1024, ctypes.byref(w), None) == kq.KQ_ERR_ALIGN


def test_debug_unpack_rejects_bad_arguments(kq):
    L = kq.lib()
    Q4, Q6, TQ = kq.KQ_Q4_K, kq.KQ_Q6_K, kq.KQ_TQ
    # unknown format, bad counts, zero work
    assert L.kq_debug_unpack(0, 4096, 1, 8192, 16384, None) == kq.KQ_ERR_FMT
    assert L.kq_debug_unpack(Q4, 4096, -1, 8192, 16384, None) == kq.KQ_ERR_SHAPE
    assert L.kq_debug_unpack(Q4, 4096, kq.KQ_DEBUG_UNPACK_MAX_BLOCKS + 1, 8192, 16384,
                             None) == kq.KQ_ERR_SHAPE
    for fmt in (Q4, Q6, TQ):
        assert L.kq_debug_unpack(fmt, None, 0, None, None, None) == kq.KQ_OK
    # null pointers: scales may be NULL only for ternary
    assert L.kq_debug_unpack(Q4, None, 1, 8192, 16384, None) == kq.KQ_ERR_NULL
    assert L.kq_debug_unpack(Q6, 4096, 1, None, 16384, None) == kq.KQ_ERR_NULL
    assert L.kq_debug_unpack(Q4, 4096, 1, 8192, None, None) == kq.KQ_ERR_NULL
    assert L.kq_debug_unpack(Q6, 4096, 1, 8192, None, None) == kq.KQ_ERR_NULL
    # alignment: W and q 16 bytes, scales 4 bytes
    assert L.kq_debug_unpack(Q4, 4100, 1, 8192, 16384, None) == kq.KQ_ERR_ALIGN
    assert L.kq_debug_unpack(TQ, 4096, 1, 8200, None, None) == kq.KQ_ERR_ALIGN
    assert L.kq_debug_unpack(Q6, 4096, 1, 8192, 16386, None) == kq.KQ_ERR_ALIGN
    assert L.kq_debug_unpack(5, 4096, 1, 8192, 16384, None) == kq.KQ_ERR_FMT
    assert L.kq_debug_unpack(kq.KQ_TQ2, 4096, 0, None, None, None) == kq.KQ_OK


def test_gemm_id_rejects_bad_arguments(kq):
    L = kq.lib()
    A, P4 = 1 << 20, (1 << 20) + 4096   # fake aligned addresses, never dereferenced
    Q4, TQ2 = kq.KQ_Q4_K, kq.KQ_TQ2
    f = lambda *a: L.kq_gemm_id(*a, None)
    assert f(0, A, 8, A, 10, 64, 256, P4, P4, 20, A) == kq.KQ_ERR_FMT
    assert f(Q4, A, 8, A, 10, 64, 300, P4, P4, 20, A) == kq.KQ_ERR_SHAPE     # K % 256
    assert f(Q4, A, 0, A, 10, 64, 256, P4, P4, 20, A) == kq.KQ_ERR_SHAPE     # no expert
    assert f(Q4, A, kq.KQ_GEMM_ID_MAX_EXPERTS + 1, A, 10, 64, 256, P4, P4, 20, A) == kq.KQ_ERR_SHAPE
    assert f(Q4, A, 8, A, 10, 64, 256, P4, P4, -1, A) == kq.KQ_ERR_SHAPE
    assert f(Q4, A, 8, A, 0, 64, 256, P4, P4, 20, A) == kq.KQ_ERR_SHAPE      # rows but no token
    assert f(Q4, None, 8, None, 10, 64, 256, None, None, 0, None) == kq.KQ_OK  # R == 0
    assert f(TQ2, None, 8, None, 10, 0, 256, None, None, 20, None) == kq.KQ_OK  # N == 0
    assert f(Q4, A, 8, A, 10, 64, 256, None, P4, 20, A) == kq.KQ_ERR_NULL
    assert f(Q4, A, 8, A, 10, 64, 256, P4, None, 20, A) == kq.KQ_ERR_NULL
    assert f(Q4, A + 8, 8, A, 10, 64, 256, P4, P4, 20, A) == kq.KQ_ERR_ALIGN
    assert f(Q4, A, 8, A, 10, 64, 256, P4 + 2, P4, 20, A) == kq.KQ_ERR_ALIGN
    assert f(Q4, A, 8, A, 10, 64, 256, P4, P4, 20, A + 4) == kq.KQ_ERR_ALIGN
    # one expert's weights must stay within 2^31 bytes
    n = (1 << 31) // 2304
    assert f(Q4, A, 2, A, 10, n, 4096, P4, P4, 20, A) == kq.KQ_ERR_UNSUPPORTED


def test_binding_checks_tensor_arguments(kq):
    """The torch conveniences refuse host tensors, wrong element types,
    non-contiguous tensors and buffers smaller than the size queries give,
    before any address reaches the library."""
    torch = pytest.importorskip("torch")
    cpu = torch.zeros(16, dtype=torch.float32)
    with pytest.raises(ValueError, match="device tensor"):
        kq.kq_quantize_act(kq.KQ_ACT_Q8_K, cpu, 1, 256, cpu)
    with pytest.raises(ValueError, match="device tensor"):
        kq.kq_gemm(kq.KQ_Q4_K, cpu, 0, 1, 1, 256, 0)

    class FakeDev:  # duck-typed device tensor for the size and type checks
        is_cuda = True

        def __init__(self, n, dtype="uint8", size=1, contiguous=True):
            self.n, self.dtype, self.size, self.c = n, "torch." + dtype, size, contiguous

        def is_contiguous(self):
            return self.c

        def numel(self):
            return self.n

        def element_size(self):
            return self.size

        def data_ptr(self):
            raise AssertionError("an address escaped the check")

    M, N, K = 3, 5, 256
    wb, ab = kq.kq_weight_bytes(kq.KQ_Q4_K, N, K), kq.kq_act_bytes(kq.KQ_ACT_Q8_K, M, K)
    W, A = FakeDev(wb), FakeDev(ab)
    with pytest.raises(ValueError, match="W"):
        kq.kq_gemm(kq.KQ_Q4_K, FakeDev(wb - 1), A, M, N, K, FakeDev(M * N, "float32", 4))
    with pytest.raises(ValueError, match="a_q8"):
        kq.kq_gemm(kq.KQ_Q4_K, W, FakeDev(ab - 16), M, N, K, FakeDev(M * N, "float32", 4))
    with pytest.raises(ValueError, match="out"):
        kq.kq_gemm(kq.KQ_Q4_K, W, A, M, N, K, FakeDev(M * N - 1, "float32", 4))
    with pytest.raises(ValueError, match="dtype"):
        kq.kq_gemm(kq.KQ_Q4_K, W, A, M, N, K, FakeDev(M * N, "float16", 2))
    with pytest.raises(ValueError, match="contiguous"):
        kq.kq_gemm(kq.KQ_Q4_K, W, A, M, N, K, FakeDev(M * N, "float32", 4, contiguous=False))
    with pytest.raises(ValueError, match="dtype"):
        kq.kq_quantize_act(kq.KQ_ACT_Q8_K, FakeDev(M * K, "float16", 2), M, K, A)
    with pytest.raises(ValueError, match="rows"):
        kq.kq_gemm_id(kq.KQ_Q4_K, FakeDev(2 * wb), 2, A, M, N, K, FakeDev(3, "int32", 4),
                      FakeDev(6, "int32", 4), 7, FakeDev(7 * N, "float32", 4))
