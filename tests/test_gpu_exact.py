"""Exact integer checks through every production kernel variant.

The products must reproduce each per-sub-block int32 dot sum
S[m][n][j] = sum_{k in sub-block j} qint[n][k] * qs[m][k] bit for bit.  The
production kernels never write S out, so these tests choose inputs that make
the fp32 output an exact integer combination of the S values:

* unit activation scales (d_a = 1) and weight scale d = 1, no mins (dmin = 0);
* Q4_K sub-block scales c * e_j (c = 1, 8, 63: the high and low scale digits
  and the shift between them are each exercised alone and together) and
  random scales in [0, 63]; Q6_K signed scales c * e_j (c = 1, -1, 127,
  -128) and random ones; ternary rows whose trits are zero outside one block.

The output is then sum_j sc_j S_j summed over superblocks, an integer below
2^24 (asserted on the drawn data), which fp32 holds exactly.  Every launch
asserts the dispatch counter of the variant it targets.

The last test measures how far inside the tolerance the Q4_K min term stays
on weights built to stress it (outlier-heavy sub-blocks, and sub-blocks whose
weights nearly cancel against a large min).
"""
from __future__ import annotations

import numpy as np
import pytest

import datagen
from oracle import kqref

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

Q4_K, Q6_K, TQ, TQ2 = 1, 2, 3, 4
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


def bf16_bits_exact(v: np.ndarray) -> np.ndarray:
    """bf16 bit patterns of values bf16 holds exactly (checked)."""
    f = v.astype(np.float32)
    b = (f.view(np.uint32) >> 16).astype(np.uint16)
    assert np.array_equal((b.astype(np.uint32) << 16).view(np.float32), f)
    return b


def unit_act(kq, act_fmt, qs):
    """Activation buffer for qs with unit scales (plus, for Q8_K, the sums and
    the min-term operand parts that belong to qs), built on the host."""
    M, K = qs.shape
    bs = 256 if act_fmt == kq.KQ_ACT_Q8_K else 128
    buf = np.zeros(kq.kq_act_bytes(act_fmt, M, K), np.uint8)
    buf[:M * K] = qs.view(np.uint8).reshape(-1)
    od = kq.kq_act_section_offset(act_fmt, kq.KQ_SEC_D, M, K)
    buf[od:od + M * (K // bs) * 4] = np.ones(M * (K // bs), np.float32).view(np.uint8)
    if act_fmt == kq.KQ_ACT_Q8_K:
        ob = kq.kq_act_section_offset(act_fmt, kq.KQ_SEC_BSUMS, M, K)
        bsums = qs.astype(np.int32).reshape(M, K // 16, 16).sum(-1).astype(np.int16)
        buf[ob:ob + bsums.nbytes] = bsums.view(np.uint8).reshape(-1)
        s32 = qs.astype(np.int64).reshape(M, K // 256, 8, 32).sum(-1)
        p0 = (s32 // 64) * 64
        al = np.stack([bf16_bits_exact(p0), bf16_bits_exact(s32 - p0)], 0).transpose(2, 0, 1, 3)
        oa = kq.kq_act_section_offset(act_fmt, kq.KQ_SEC_ALPHA, M, K)
        buf[oa:oa + al.nbytes] = np.ascontiguousarray(al).view(np.uint8).reshape(-1)
    return dev(buf)


def variant_index(kq, name):
    names = [kq.kq_variant_name(v) for v in range(kq.kq_num_variants())]
    return names.index(name)


def run_checked(kq, variant, fmt, W, a_q8, M, N, K):
    """kq_gemm, asserting that exactly the named variant ran."""
    v = variant_index(kq, variant)
    assert kq.kq_select_variant(fmt, M, N, K) == v, (variant, M, N, K)
    before = kq.kq_dispatch_count(v)
    out = torch.full((M, N), float("nan"), dtype=torch.float32, device=DEV)
    kq.kq_gemm(fmt, W, a_q8, M, N, K, out)
    torch.cuda.synchronize()
    assert kq.kq_dispatch_count(v) == before + 1
    return out.cpu().numpy()


def assert_exact(out, want, what):
    assert np.abs(want).max() < 2 ** 24, what + ": expected sums leave the exact fp32 range"
    bad = np.argwhere(out != want.astype(np.float32))
    assert bad.size == 0, f"{what}: {len(bad)} outputs differ, first at {tuple(bad[0])}: " \
                          f"{out[tuple(bad[0])]} != {want[tuple(bad[0])]}"


# ------------------------------------------------------------------ Q4_K

# (variant, M, N, K): the 128 x 128 tile needs more than 256 such tiles
# (3 x 86); the 4-wave 64 x 128 tile more than 256 of its own (3 x 100); the
# 8-wave 64 x 128 build takes the smaller counts (K = 768: an odd number of
# superblocks, so one half of its waves sits out the last step); the Q4_K
# ring kernel takes 3 .. 64 tokens when N / 32 exceeds the CU count, in 16-,
# 32- and 64-row builds (one superblock: the second K-half has none; three:
# its second step is empty; 11016 columns: a ragged last workgroup); below
# that the four-wave split kernel takes up to 16 tokens while N / 32 is more
# than half the CU count (4104-4200 rows), and the ring kernel with K-parts
# the rest (K-parts without a superblock at 200 and 100 rows); the
# matrix-vector kernel takes one or two tokens with K a multiple of 2048
Q4K_CASES = [
    ("gemm_q4_k_128x128", 300, 11000, 256),
    ("gemm_q4_k_64x128", 192, 12800, 256),
    ("gemm_q4_k_64x128_k2", 70, 96, 256),
    ("gemm_q4_k_64x128_k2", 129, 200, 768),
    ("gemm_q4_k_ring_kp", 64, 200, 256),
    ("gemm_q4_k_ring_kp", 20, 200, 512),
    ("gemm_q4_k_ring_kp", 3, 100, 256),
    ("gemm_q4_k_ring_kp", 20, 4104, 768),
    # ... in 64-token slices (two, three ragged, five)
    ("gemm_q4_k_ring_kp", 128, 72, 2048),
    ("gemm_q4_k_ring_kp", 150, 200, 2048),
    ("gemm_q4_k_ring_kp", 300, 72, 2048),
    ("gemm_q4_k_m64_ring", 64, 11008, 256),
    ("gemm_q4_k_m64_ring", 20, 11016, 768),
    ("gemm_q4_k_m64_ring", 9, 11008, 512),
    ("gemm_q4_k_m16", 16, 4200, 512), ("gemm_q4_k_m16", 3, 4200, 256), ("gemm_q4_k_m16", 9, 4104, 1280),
    ("gemm_q4_k_matvec", 1, 100, 2048),
    ("gemm_q4_k_matvec", 2, 100, 2048),
]


def q4k_patterns(rng, N, nsb):
    """(name, sc [N][nsb][8]) scale patterns: c * e_j in one superblock (the
    others all-zero scales) for c = 1, 8, 63, and random scales everywhere."""
    pats = []
    for c in (1, 8, 63):
        for j in range(8):
            sc = np.zeros((N, nsb, 8), np.int64)
            s0 = (j + c) % nsb
            sc[:, s0, j] = c
            pats.append((f"{c}*e_{j} in superblock {s0}", sc))
    pats.append(("random scales", rng.integers(0, 64, size=(N, nsb, 8))))
    return pats


@pytest.mark.parametrize("variant,M,N,K", Q4K_CASES, ids=[f"{c[0]}-M{c[1]}" for c in Q4K_CASES])
def test_q4k_subsums_exact_through_variant(kq, variant, M, N, K):
    rng = np.random.default_rng(M * 7 + N + K)
    nsb = K // 256
    qs = rng.integers(-127, 128, size=(M, K)).astype(np.int8)
    a_q8 = unit_act(kq, kq.KQ_ACT_Q8_K, qs)
    q = rng.integers(0, 16, size=(N * nsb, 256))
    mn = rng.integers(0, 64, size=(N * nsb, 8))        # mins present, dmin = 0
    ones = np.ones(N * nsb, np.float16)
    zeros = np.zeros(N * nsb, np.float16)
    # S does not depend on the scales: compute it once from unit scales
    W1 = datagen.pack_q4k(ones, zeros, np.ones((N * nsb, 8), np.int64), mn, q).reshape(N, -1)
    S = kqref.subsums(Q4_K, W1, qs, K).reshape(M, N, nsb, 8).astype(np.int64)
    for name, sc in q4k_patterns(rng, N, nsb):
        say(f"{variant} M={M} N={N} K={K}: {name}")
        W = datagen.pack_q4k(ones, zeros, sc.reshape(N * nsb, 8), mn, q).reshape(N, -1)
        out = run_checked(kq, variant, Q4_K, dev(W), a_q8, M, N, K)
        want = np.einsum("mnsj,nsj->mn", S, sc)
        assert_exact(out, want, f"{variant} {name}")


def test_q4k_subsums_exact_through_gather(kq):
    """The expert-indexed product's gather mode of the Q4_K tile kernel: every
    routed row gets exactly its token's sums against its expert's scales."""
    E, M, N, K = 3, 40, 96, 512
    nsb = K // 256
    rng = np.random.default_rng(97)
    counts = (0, 70, 5)
    off = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    rows = rng.integers(0, M, size=int(off[-1])).astype(np.int32)
    R = int(off[-1])
    qs = rng.integers(-127, 128, size=(M, K)).astype(np.int8)
    a_q8 = unit_act(kq, kq.KQ_ACT_Q8_K, qs)
    ones = np.ones(N * nsb, np.float16)
    zeros = np.zeros(N * nsb, np.float16)
    v = variant_index(kq, "gemm_id_q4_k_64x128")
    for c in (1, 8, 63, None):
        Ws, wants = [], []
        for e in range(E):
            q = rng.integers(0, 16, size=(N * nsb, 256))
            mn = rng.integers(0, 64, size=(N * nsb, 8))
            sc = rng.integers(0, 64, size=(N, nsb, 8)) if c is None else np.zeros((N, nsb, 8), np.int64)
            if c is not None:
                sc[:, e % nsb, (3 * e + c) % 8] = c
            W = datagen.pack_q4k(ones, zeros, sc.reshape(N * nsb, 8), mn, q).reshape(N, -1)
            S = kqref.subsums(Q4_K, W, np.ascontiguousarray(qs[rows[off[e]:off[e + 1]]]), K)
            Ws.append(W)
            wants.append(np.einsum("mnsj,nsj->mn", S.reshape(-1, N, nsb, 8).astype(np.int64), sc))
        say(f"gemm_id Q4_K gather: scales {c if c is not None else 'random'}")
        out = torch.full((R, N), float("nan"), dtype=torch.float32, device=DEV)
        before = kq.kq_dispatch_count(v)
        kq.kq_gemm_id(Q4_K, dev(np.concatenate([w.reshape(-1) for w in Ws])), E, a_q8, M, N, K,
                      dev(off), dev(rows), R, out)
        torch.cuda.synchronize()
        assert kq.kq_dispatch_count(v) == before + 1
        assert_exact(out.cpu().numpy(), np.concatenate(wants, 0), f"gemm_id scales {c}")


# ------------------------------------------------------------------ Q6_K

Q6K_CASES = [
    ("gemm_q6_k_128x128", 70, 96, 512),
    ("gemm_q6_k_128x128", 130, 260, 256),
    ("gemm_q6_k_matvec", 1, 72, 2048),
    ("gemm_q6_k_matvec", 4, 72, 2048),
    # the K-split ring kernel: 16-, 32- and 64-row token tiles; eight K-parts
    # (72 rows), four (4104 rows and 64 tokens' 200 rows) and two (14344
    # rows); K-parts with no superblock; one to four superblocks
    ("gemm_q6_k_ring", 3, 72, 256),
    ("gemm_q6_k_ring", 9, 72, 512),
    ("gemm_q6_k_ring", 5, 72, 2048),
    ("gemm_q6_k_ring", 20, 4104, 1024),
    ("gemm_q6_k_ring", 33, 200, 768),
    ("gemm_q6_k_ring", 16, 14344, 512),
    # ... in 64-token slices (two, three ragged, five)
    ("gemm_q6_k_ring", 128, 72, 2048),
    ("gemm_q6_k_ring", 150, 200, 2048),
    ("gemm_q6_k_ring", 300, 72, 2048),
    # the tile kernel with K in two parts (4 / 4 and 8 / 2 chunks of 128)
    ("gemm_q6_k_128x128_k2", 600, 130, 1024),
    ("gemm_q6_k_128x128_k2", 600, 130, 1280),
]


@pytest.mark.parametrize("variant,M,N,K", Q6K_CASES, ids=[f"{c[0]}-M{c[1]}" for c in Q6K_CASES])
def test_q6k_subsums_exact_through_variant(kq, variant, M, N, K):
    rng = np.random.default_rng(M * 5 + N + K)
    nsb = K // 256
    # |qs| <= 40 keeps the random-scale sums (16 sub-blocks per superblock,
    # scales up to 128) inside the exact fp32 range
    qs = rng.integers(-40, 41, size=(M, K)).astype(np.int8)
    a_q8 = unit_act(kq, kq.KQ_ACT_Q8_K, qs)
    q = rng.integers(0, 64, size=(N * nsb, 256))
    ones = np.ones(N * nsb, np.float16)
    W1 = datagen.pack_q6k(ones, np.ones((N * nsb, 16), np.int64), q).reshape(N, -1)
    S = kqref.subsums(Q6_K, W1, qs, K).reshape(M, N, nsb, 16).astype(np.int64)
    pats = []
    for c in (1, -1, 127, -128):
        for j in (0, 5, 15):
            sc = np.zeros((N, nsb, 16), np.int64)
            sc[:, (j + 1) % nsb, j] = c
            pats.append((f"{c}*e_{j}", sc))
    pats.append(("random scales", rng.integers(-128, 128, size=(N, nsb, 16))))
    for name, sc in pats:
        say(f"{variant} M={M} N={N} K={K}: {name}")
        W = datagen.pack_q6k(ones, sc.reshape(N * nsb, 16), q).reshape(N, -1)
        out = run_checked(kq, variant, Q6_K, dev(W), a_q8, M, N, K)
        assert_exact(out, np.einsum("mnsj,nsj->mn", S, sc), f"{variant} {name}")


# ------------------------------------------------------------------ ternary

TQ_CASES = [
    ("gemm_tq_128x128", TQ, 67, 90, 640),
    ("gemm_tq_128x128_reg", TQ, 300, 11000, 512), ("gemm_tq_128x128_reg", TQ, 129, 16500, 256),
    ("gemm_tq_matvec", TQ, 1, 40, 1024),
    ("gemm_tq_matvec", TQ, 4, 40, 1024),
    # the K-split ring kernel (eight, four and two K-parts)
    ("gemm_tq_ring", TQ, 9, 40, 1024),
    ("gemm_tq_ring", TQ, 3, 72, 768),
    ("gemm_tq_ring", TQ, 20, 4104, 768),
    ("gemm_tq_ring", TQ, 64, 200, 512),
    ("gemm_tq_ring", TQ, 16, 14344, 512),
    ("gemm_tq_ring", TQ, 150, 200, 2048),  # three 64-token slices, ragged
    ("gemm_tq2_128x128", TQ2, 67, 90, 640),
    ("gemm_tq2_128x128_k2", TQ2, 5, 40, 1152),
    # the K-split ring kernel: 16-, 32- and 64-row token tiles; eight K-parts
    # (40 and 72 rows), four (4104 rows; 64 tokens' 200), two (14344 rows)
    ("gemm_tq2_matvec", TQ2, 1, 40, 1024),
    ("gemm_tq2_matvec", TQ2, 4, 40, 2048),
    ("gemm_tq2_ring", TQ2, 1, 40, 256),
    ("gemm_tq2_ring", TQ2, 5, 72, 1024),
    ("gemm_tq2_ring", TQ2, 20, 4104, 768),
    ("gemm_tq2_ring", TQ2, 64, 200, 512),
    ("gemm_tq2_ring", TQ2, 16, 14344, 512),
    ("gemm_tq2_ring", TQ2, 150, 200, 2048),
    # the tile kernel with K in two parts (8 / 1 chunks of 128)
    ("gemm_tq_128x128_k2", TQ, 600, 130, 1152),
    ("gemm_tq2_128x128_k2", TQ2, 600, 130, 1152),
]


@pytest.mark.parametrize("variant,fmt,M,N,K", TQ_CASES, ids=[f"{c[0]}-M{c[2]}" for c in TQ_CASES])
def test_ternary_block_sums_exact_through_variant(kq, variant, fmt, M, N, K):
    """Unit scales and trits that are zero outside block b: the output is
    exactly the block sum S[:, :, b]; then all blocks at once."""
    rng = np.random.default_rng(M * 3 + N + K + fmt)
    nb = K // 128
    qs = rng.integers(-127, 128, size=(M, K)).astype(np.int8)
    a_q8 = unit_act(kq, kq.KQ_ACT_Q8_128, qs)
    t = rng.integers(-1, 2, size=(N, K)).astype(np.int8)
    d = np.ones((N, nb), np.float16)
    enc = datagen.encode_tq if fmt == TQ else datagen.encode_tq2
    S = kqref.subsums(fmt, enc(t, d), qs, K).astype(np.int64)      # [M][N][nb]
    for b in sorted({0, 1, nb - 1}) + [None]:
        tb = t.copy()
        if b is not None:
            mask = np.zeros(K, bool)
            mask[128 * b:128 * (b + 1)] = True
            tb[:, ~mask] = 0
        say(f"{variant} M={M} N={N} K={K}: block {b if b is not None else 'all'}")
        out = run_checked(kq, variant, fmt, dev(enc(tb, d)), a_q8, M, N, K)
        want = S.sum(-1) if b is None else S[:, :, b]
        assert_exact(out, want, f"{variant} block {b}")


# ------------------------------------------------------------------ min-term headroom

def stress_weights(N, K, seed, kind):
    """fp32 weights that stress the Q4_K min term.  'outliers': N(0, 0.02) with
    10% of the weights times 10.  'cancel': per 32-wide sub-block, tiny weights
    and one large negative one, so the quantizer's large min nearly cancels
    d*sc*q for most weights."""
    rng = np.random.default_rng(seed)
    if kind == "outliers":
        w = rng.normal(0.0, 0.02, size=(N, K))
        w *= np.where(rng.random((N, K)) < 0.1, 10.0, 1.0)
    else:
        w = rng.normal(0.0, 1e-4, size=(N, K // 32, 32))
        pos = rng.integers(0, 32, size=(N, K // 32))
        big = -rng.uniform(0.5, 1.0, size=(N, K // 32))
        np.put_along_axis(w, pos[:, :, None], big[:, :, None], axis=2)
        w = w.reshape(N, K)
    return w.astype(np.float32)


HEADROOM_CASES = [
    ("gemm_q4_k_128x128", 300, 11000, 512),
    ("gemm_q4_k_64x128_k2", 129, 4000, 1024),
    ("gemm_q4_k_ring_kp", 129, 640, 1024),  # three 64-token slices
    ("gemm_q4_k_ring_kp", 64, 640, 1024),
    ("gemm_q4_k_m64_ring", 64, 11008, 1024),
    ("gemm_q4_k_m64_ring", 16, 11008, 1024),
    ("gemm_q4_k_m16", 16, 4200, 1024),
    ("gemm_q4_k_ring_kp", 16, 640, 1024),
    ("gemm_q4_k_matvec", 2, 640, 2048),
]


@pytest.mark.parametrize("kind", ["outliers", "cancel"])
@pytest.mark.parametrize("variant,M,N,K", HEADROOM_CASES, ids=[c[0] for c in HEADROOM_CASES])
def test_q4k_min_term_headroom(kq, variant, M, N, K, kind):
    """Held to the product's tolerance with 10x to spare (err/tol <= 0.1) on
    weights that stress the min term, real quantized activations (N(0, 1)
    with LogNormal channel scales)."""
    W = datagen.encode_q4k(stress_weights(N, K, 71 + K, kind))
    x = datagen.draw_activations(M, K, 72 + M, "outlier_lognormal")
    a_q8 = kq.quantize_act(dev(x), kq.KQ_ACT_Q8_K)
    qs, d, _ = kqref.quantize_act(kq.KQ_ACT_Q8_K, x)
    out = run_checked(kq, variant, Q4_K, dev(W), a_q8, M, N, K)
    rows = None if N <= 1024 else np.unique(np.concatenate(
        [np.arange(0, N, 97), [N - 1], np.random.default_rng(5).choice(N, 64, replace=False)]))
    ref, tol = kqref.gemm(Q4_K, W, qs, d, K, rows=rows)
    got = out if rows is None else out[:, rows]
    ratio = float((np.abs(got.astype(np.float64) - ref) / tol).max())
    say(f"{variant} {kind} M={M} N={N} K={K}: max err/tol {ratio:.3g}")
    assert ratio <= 0.1, f"{variant} {kind}: max err/tol {ratio:.3g} (headroom under 10x)"
