"""GPU tests of the weight loaders against the oracle's codec.

1. kq_debug_unpack runs the tile kernel's loaders on fuzzed blocks (the loader
   fuzz test of llama.cpp PR 214: thousands of arbitrary packed blocks through
   the unpack, compared value by value with the scalar codec) and on blocks
   built so that every field position takes every value.  Integer results must
   match bit for bit.
2. Identity activations through every GEMM kernel variant: with unit
   activation scales and qs = I, row m of the product is column m of the
   dequantized weights, so each kernel's own loader (registers, LDS digit
   planes, trit table) is checked at every K position.  Q6_K and ternary
   results are exact in fp32; Q4_K's min term goes through bf16 hi/lo operands
   (16 significant bits), so it is checked against a bound derived from that
   split instead.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import datagen
from oracle import kqref

pytestmark = pytest.mark.gpu

Q4_K, Q6_K, TQ, TQ2 = 1, 2, 3, 4
QK = {Q4_K: 256, Q6_K: 256, TQ: 128, TQ2: 128}
BB = {Q4_K: 144, Q6_K: 210, TQ: 28, TQ2: 34}
TERNARY = (TQ, TQ2)
DEV = "cuda:0"


def say(*a):
    print(*a, flush=True)


@pytest.fixture(scope="module")
def kq():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import block_quantized_matmul_act_amd as kq
    kq.lib()
    return kq


def dev(a: np.ndarray):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


# ------------------------------------------------------------ block sets

def fuzz_blocks(fmt: int, n: int, seed: int) -> np.ndarray:
    """n arbitrary blocks: every byte pattern is a valid Q4_K / Q6_K block; a
    ternary block takes digit bytes <= 242 and a last digit byte whose two
    spare digits are 1 (108..134)."""
    rng = np.random.default_rng(seed)
    if fmt == TQ2:  # two-bit codes 0..2 only
        b = np.empty((n, 34), np.uint8)
        c = rng.integers(0, 3, size=(n, 32, 4))
        b[:, :32] = (c[..., 0] | (c[..., 1] << 2) | (c[..., 2] << 4) | (c[..., 3] << 6)).astype(np.uint8)
        b[:, 32:] = rng.integers(0, 256, size=(n, 2))
        return b
    if fmt != TQ:
        return rng.integers(0, 256, size=(n, BB[fmt]), dtype=np.uint8)
    b = np.empty((n, 28), np.uint8)
    b[:, :25] = rng.integers(0, 243, size=(n, 25))
    b[:, 25] = 108 + rng.integers(0, 27, size=n)
    b[:, 26:] = rng.integers(0, 256, size=(n, 2))
    return b


def exhaustive_blocks(fmt: int) -> np.ndarray:
    """Blocks in which every field position takes every value it can hold."""
    if fmt == Q4_K:
        # 6-bit scale/min fields: field f of block b is (b + 5f) mod 64; nibble
        # bytes: byte i of block b is (b + i) mod 256
        B = 256
        b = np.arange(B)[:, None]
        fields = (b + 5 * np.arange(16)[None, :]) % 64
        bits = ((fields[:, :, None] >> np.arange(6)) & 1).reshape(B, 96).astype(np.uint8)
        out = np.zeros((B, 144), np.uint8)
        out[:, 0:4] = (b + np.arange(4)) % 256
        out[:, 4:16] = np.packbits(bits, axis=1, bitorder="little")
        out[:, 16:] = (b + np.arange(128)) % 256
        return out
    if fmt == TQ2:
        # every code byte of the block takes all 81 values made of valid
        # codes (byte i of block b is the (b + 7i) mod 81-th of them)
        valid = np.array([v for v in range(256) if all((v >> (2 * p)) & 3 != 3 for p in range(4))],
                         np.uint8)
        assert len(valid) == 81
        b = np.arange(81)[:, None]
        out = np.zeros((81, 34), np.uint8)
        out[:, :32] = valid[(b + 7 * np.arange(32)[None, :]) % 81]
        out[:, 32:] = (b + np.arange(2)) % 256
        return out
    if fmt == Q6_K:
        # every byte of the block, quant and scale bytes alike, takes all 256
        # values across the set (byte i of block b is (b + 3i) mod 256)
        b = np.arange(256)[:, None]
        return ((b + 3 * np.arange(210)[None, :]) % 256).astype(np.uint8)
    # ternary: digit byte i of block b is (b + 7i) mod 243; the last digit byte
    # runs through its 27 valid values
    b = np.arange(243)[:, None]
    out = np.zeros((243, 28), np.uint8)
    out[:, :25] = (b + 7 * np.arange(25)[None, :]) % 243
    out[:, 25] = 108 + (np.arange(243) % 27)
    out[:, 26:] = (b + np.arange(2)) % 256
    return out


def oracle_scales(fmt: int, blocks: np.ndarray) -> np.ndarray:
    out = np.zeros((blocks.shape[0], 16), np.int32)
    for i, blk in enumerate(blocks):
        if fmt == Q4_K:
            _, _, sc, mn, _ = kqref.decode_q4k(blk)
            out[i, :8], out[i, 8:] = sc, mn
        else:
            _, sc, _ = kqref.decode_q6k(blk)
            out[i] = sc
    return out


# ------------------------------------------------------------ 1. kq_debug_unpack

@pytest.mark.parametrize("fmt", (Q4_K, Q6_K, TQ, TQ2))
def test_debug_unpack_matches_codec(kq, fmt):
    blocks = np.concatenate([exhaustive_blocks(fmt), fuzz_blocks(fmt, 10007, 900 + fmt)])
    B = blocks.shape[0]
    say(f"debug_unpack fmt={fmt} blocks={B}")
    q, scales = kq.debug_unpack(fmt, dev(blocks.reshape(-1)), B)
    torch.cuda.synchronize()
    want_q = kqref.int_operands(fmt, blocks.reshape(1, -1), B * QK[fmt]).reshape(B, QK[fmt])
    got_q = q.cpu().numpy().astype(np.int32)
    bad = np.argwhere(got_q != want_q)
    assert bad.size == 0, f"{len(bad)} values differ, first at block/value {tuple(bad[0])}"
    if fmt not in TERNARY:
        got_s = scales.cpu().numpy()
        want_s = oracle_scales(fmt, blocks)
        bad = np.argwhere(got_s != want_s)
        assert bad.size == 0, f"{len(bad)} scale fields differ, first at {tuple(bad[0])}"


@pytest.mark.parametrize("fmt", (Q4_K, Q6_K, TQ, TQ2))
@pytest.mark.parametrize("B", [1, 2, 31, 33, 65])
def test_debug_unpack_ragged_counts(kq, fmt, B):
    """Counts that leave workgroups partly empty; bytes past the last block are
    never written (canaries after q and scales stay intact)."""
    blocks = fuzz_blocks(fmt, B, 77 + B)
    q = torch.full((B + 4, QK[fmt]), 99, dtype=torch.int8, device=DEV)
    sc = torch.full((B + 4, 16), -7, dtype=torch.int32, device=DEV)
    kq.kq_debug_unpack(fmt, dev(blocks.reshape(-1)), B, q, sc)
    torch.cuda.synchronize()
    want = kqref.int_operands(fmt, blocks.reshape(1, -1), B * QK[fmt]).reshape(B, QK[fmt])
    qn = q.cpu().numpy()
    assert np.array_equal(qn[:B].astype(np.int32), want)
    assert np.all(qn[B:] == 99)
    scn = sc.cpu().numpy()
    if fmt not in TERNARY:
        assert np.array_equal(scn[:B], oracle_scales(fmt, blocks))
    assert np.all(scn[B:] == -7) and (fmt not in TERNARY or np.all(scn == -7))


# ------------------------------------------------------------ 2. identity activations

def unit_act(kq, fmt, qs):
    """Activation buffer with unit scales (and, for Q8_K, the sums and min
    operands that go with qs), built on the host."""
    M, K = qs.shape
    act = kq.kq_act_fmt_for(fmt)
    bs = 256 if act == kq.KQ_ACT_Q8_K else 128
    buf = np.zeros(kq.kq_act_bytes(act, M, K), np.uint8)
    buf[:M * K] = qs.view(np.uint8).reshape(-1)
    od = kq.kq_act_section_offset(act, kq.KQ_SEC_D, M, K)
    buf[od:od + M * (K // bs) * 4] = np.ones(M * (K // bs), np.float32).view(np.uint8)
    if act == kq.KQ_ACT_Q8_K:
        ob = kq.kq_act_section_offset(act, kq.KQ_SEC_BSUMS, M, K)
        bsums = qs.astype(np.int32).reshape(M, K // 16, 16).sum(-1).astype(np.int16)
        buf[ob:ob + bsums.nbytes] = bsums.view(np.uint8).reshape(-1)
        # alpha: the sum B of each sub-block's 32 qs as 64 * floor(B / 64) and
        # B mod 64, both exact in bf16 (the low 16 bits of their fp32 are 0)
        s32 = qs.astype(np.int32).reshape(M, K // 256, 8, 32).sum(-1)
        p0 = ((s32 // 64) * 64).astype(np.float32)
        p1 = (s32 - (s32 // 64) * 64).astype(np.float32)
        parts = [(p.view(np.uint32) >> 16).astype(np.uint16) for p in (p0, p1)]
        for p, b in zip((p0, p1), parts):
            assert np.array_equal((b.astype(np.uint32) << 16).view(np.float32), p)
        al = np.stack(parts, 0).transpose(2, 0, 1, 3)                      # [S][2][M][8]
        oa = kq.kq_act_section_offset(act, kq.KQ_SEC_ALPHA, M, K)
        buf[oa:oa + al.nbytes] = np.ascontiguousarray(al).view(np.uint8).reshape(-1)
    return dev(buf)


def finite_weights(fmt: int, N: int, K: int, seed: int) -> np.ndarray:
    """Fuzzed fields with finite fp16 scales, packed as [N][K/QK] blocks."""
    rng = np.random.default_rng(seed)
    B = N * K // QK[fmt]
    if fmt == Q4_K:
        W = datagen.pack_q4k(*datagen.random_fields_q4k(rng, B))
    elif fmt == Q6_K:
        W = datagen.pack_q6k(*datagen.random_fields_q6k(rng, B))
    elif fmt == TQ2:
        d, t = datagen.random_fields_tq2(rng, B)
        W = datagen.pack_tq2(t, d)
    else:
        d, t = datagen.random_fields_tq(rng, B)
        W = datagen.pack_tq(t, d)
    return W.reshape(N, -1)


# (fmt, K, variant, token rows per launch, weight rows); the 128 x 128 Q4_K
# kernel takes shapes of more than 256 such tiles, hence its 2100 weight rows,
# the 4-wave 64 x 128 build more than 256 of its own (1100 rows), and the
# K-split ring kernel more than 256 32-row pieces (11016 rows, ragged); the
# 128 x 128 tile kernel of the other formats takes K in two parts where its
# tiles cover at most half the CUs (72 rows) and whole at 4200 rows
IDENTITY_CASES = [
    (Q4_K, 2048, "gemm_q4_k_matvec", 2, 72),
    (Q4_K, 2048, "gemm_q4_k_ring_kp", 64, 72),
    (Q4_K, 2048, "gemm_q4_k_ring_kp", 32, 4104),
    (Q4_K, 2048, "gemm_q4_k_m64_ring", 64, 11016),
    (Q4_K, 2048, "gemm_q4_k_m64_ring", 16, 11016),
    (Q4_K, 2048, "gemm_q4_k_m16", 16, 4200),
    (Q4_K, 2048, "gemm_q4_k_64x128_k2", 2048, 72),
    (Q4_K, 2048, "gemm_q4_k_64x128", 2048, 1100),
    (Q4_K, 2048, "gemm_q4_k_128x128", 2048, 2100),
    (Q6_K, 2048, "gemm_q6_k_matvec", 4, 72),
    (Q6_K, 2048, "gemm_q6_k_ring", 16, 72),
    (Q6_K, 2304, "gemm_q6_k_ring", 64, 4104),
    (Q6_K, 2048, "gemm_q6_k_128x128_k2", 2048, 72),
    (Q6_K, 2048, "gemm_q6_k_128x128", 2048, 4200),
    (TQ, 1024, "gemm_tq_matvec", 4, 72),
    (TQ, 1152, "gemm_tq_128x128_k2", 1152, 72),
    (TQ, 1152, "gemm_tq_128x128", 1152, 4200),
    (TQ, 1024, "gemm_tq_ring", 16, 72),
    (TQ, 1280, "gemm_tq_ring", 64, 4104),
    (TQ, 1024, "gemm_tq_128x128_reg", 1024, 4200),
    (TQ2, 1152, "gemm_tq2_128x128_k2", 8, 72),
    (TQ2, 1024, "gemm_tq2_matvec", 4, 72),
    (TQ2, 1024, "gemm_tq2_ring", 8, 72),
    (TQ2, 1280, "gemm_tq2_ring", 64, 4104),
    (TQ2, 1024, "gemm_tq2_128x128_k2", 1024, 72),
    (TQ2, 1024, "gemm_tq2_128x128", 1024, 4200),
]


@pytest.mark.parametrize("fmt,K,variant,MT,N", IDENTITY_CASES,
                         ids=[c[2] for c in IDENTITY_CASES])
def test_identity_activations_decode_every_position(kq, fmt, K, variant, MT, N):
    # N = 72: two and a bit 32-row groups, a ragged column tile; N = 2100:
    # 16 full column tiles and a ragged one
    W = finite_weights(fmt, N, K, 300 + fmt)
    ref = kqref.dequant_rows(fmt, W, K).T            # out[m][n] = W^[n][m]
    Wd = dev(W)
    out = np.empty((K, N), np.float32)
    names = [kq.kq_variant_name(v) for v in range(kq.kq_num_variants())]
    assert kq.kq_variant_name(kq.kq_select_variant(fmt, MT, N, K)) == variant
    kq.kq_dispatch_reset()
    say(f"identity {variant}: K={K} N={N}, {K // MT} launches of {MT} rows")
    for m0 in range(0, K, MT):
        qs = np.zeros((MT, K), np.int8)
        qs[np.arange(MT), m0 + np.arange(MT)] = 1
        o = torch.full((MT, N), float("nan"), dtype=torch.float32, device=DEV)
        kq.kq_gemm(fmt, Wd, unit_act(kq, fmt, qs), MT, N, K, o)
        out[m0:m0 + MT] = o.cpu().numpy()
    assert kq.kq_dispatch_count(names.index(variant)) == K // MT
    assert np.all(np.isfinite(out))
    if fmt == Q4_K:
        # the bound the product is held to: 1e-4 * sum_k |W^ A^| + 1e-6, here
        # 1e-4 * |W^[n][m]| + 1e-6 (one unit activation per row); the kernels
        # form d * (sc*q) - dmin * m_j * 1 with two fp32 roundings
        bound = 1e-4 * np.abs(ref) + 1e-6
        err = np.abs(out.astype(np.float64) - ref)
        worst = np.unravel_index(np.argmax(err / bound), err.shape)
        say(f"  max err/tol {(err / bound).max():.3g}")
        assert np.all(err <= bound), f"{variant}: err/tol {(err / bound).max():.3g} at k,n={worst}"
    else:
        bad = np.argwhere(out != ref.astype(np.float32))
        assert bad.size == 0, f"{variant}: {len(bad)} values differ, first at k,n={tuple(bad[0])}"
