"""GPU parity: the HIP path (through the C ABI) against the CPU oracle.

Integers are compared bit for bit (quantized activations, their scales and
sums, per-sub-block dot sums); fp32 outputs must satisfy
|out - ref| <= 1e-4 * sum_k |W^ A^| + 1e-6 on every element checked.
"""
from __future__ import annotations

import os

import numpy as np
import pytest

import datagen
from oracle import kqref

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

Q4_K, Q6_K, TQ, TQ2 = 1, 2, 3, 4
FMTS = (Q4_K, Q6_K, TQ, TQ2)
FMT_NAME = {Q4_K: "q4_k", Q6_K: "q6_k", TQ: "tq", TQ2: "tq2"}
QK = {Q4_K: 256, Q6_K: 256, TQ: 128, TQ2: 128}
SUB = {Q4_K: 32, Q6_K: 16, TQ: 128, TQ2: 128}


def say(*a):
    print(*a, flush=True)


@pytest.fixture(scope="module")
def kq():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import block_quantized_matmul_act_amd as kq
    kq.lib()
    return kq


DEV = "cuda:0"


def dev(a: np.ndarray):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def run_quant(kq, act_fmt, x):
    M, K = x.shape
    a_q8 = kq.quantize_act(dev(x), act_fmt)
    torch.cuda.synchronize()
    return a_q8


def bf16_bits_rne(a: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit patterns, round to nearest even (finite inputs)."""
    b = a.astype(np.float32).view(np.uint32).astype(np.uint64)
    return ((b + 0x7FFF + ((b >> 16) & 1)) >> 16).astype(np.uint16)


def expected_alpha(qs: np.ndarray, d=None) -> np.ndarray:
    """The alpha section [K/256][2][M][8] (bf16 bits) that the Q8_K layout
    defines: for the sum B of the 32 qs of each sub-block, part 0 = 64 *
    floor(B / 64) and part 1 = B - part 0, both integers bf16 holds exactly
    (the scales d do not enter)."""
    M, K = qs.shape
    s32 = qs.astype(np.int64).reshape(M, K // 256, 8, 32).sum(-1)          # [M][S][8]
    p0 = (s32 // 64) * 64
    p1 = s32 - p0
    assert np.all((p1 >= 0) & (p1 < 64)) and np.all(np.abs(p0) <= 4096)
    parts = [bf16_bits_rne(p.astype(np.float32)) for p in (p0, p1)]
    for p, b in zip((p0, p1), parts):   # exact: the bits decode to the integer
        assert np.array_equal((b.astype(np.uint32) << 16).view(np.float32), p.astype(np.float32))
    return np.stack(parts, 0).transpose(2, 0, 1, 3).view(np.int16)         # [S][2][M][8]


def check_act_exact(kq, act_fmt, x, a_q8):
    M, K = x.shape
    qs, d, bs = kqref.quantize_act(act_fmt, x)
    gq, gd, gb = kq.act_views(a_q8, act_fmt, M, K)
    assert np.array_equal(gq.cpu().numpy(), qs)
    assert np.array_equal(gd.cpu().numpy().view(np.uint32), d.view(np.uint32))
    if bs is not None:
        assert np.array_equal(gb.cpu().numpy(), bs)
        ga = kq.alpha_view(a_q8, M, K).cpu().numpy()
        assert np.array_equal(ga, expected_alpha(qs, d)), "alpha section differs"
    return qs, d, bs


def run_gemm(kq, fmt, W, a_q8, M, N, K):
    out = torch.full((M, N), float("nan"), dtype=torch.float32, device=DEV)
    kq.kq_gemm(fmt, dev(W) if isinstance(W, np.ndarray) else W, a_q8, M, N, K, out)
    torch.cuda.synchronize()
    return out.cpu().numpy()


def assert_within_tol(out, ref, tol, what):
    assert np.all(np.isfinite(out)), what + ": non-finite output"
    err = np.abs(out.astype(np.float64) - ref.astype(np.float64))
    ratio = err / tol
    worst = np.unravel_index(np.argmax(ratio), ratio.shape)
    assert np.all(err <= tol), f"{what}: max err/tol {ratio.max():.3g} at {worst}"
    return float(ratio.max())


# ---------------------------------------------------------------- activations

@pytest.mark.parametrize("act_fmt,M,K", [(1, 8, 512), (1, 37, 4096), (1, 3, 14336),
                                         (2, 5, 5120), (2, 64, 384)])
def test_quantize_bit_exact(kq, act_fmt, M, K):
    say(f"quantize act_fmt={act_fmt} M={M} K={K}")
    x = datagen.draw_activations(M, K, 1000 + K, "outlier_lognormal" if M % 2 else "plain")
    a_q8 = run_quant(kq, act_fmt, x)
    check_act_exact(kq, act_fmt, x, a_q8)


def test_quantize_special_blocks(kq):
    say("quantize special blocks")
    K = 1024
    x = np.random.default_rng(3).standard_normal((6, K)).astype(np.float32)
    x[0] = 0.0                                         # all-zero row
    x[1, :256] = np.float32(1e-45)                     # subnormal amax: zero block
    x[2, :256] = 0.0
    x[2, 0] = 127.0
    x[2, 1:8] = [0.5, 1.5, 2.5, -2.5, 126.5, -0.5, 3.5]   # ties
    x[3] *= np.float32(2.0 ** 60)                      # large but finite
    x[4] *= np.float32(2.0 ** -60)                     # tiny but normal
    x[5, 256:512] = -x[5, 256:512]
    for act_fmt in (1, 2):
        a_q8 = run_quant(kq, act_fmt, x)
        check_act_exact(kq, act_fmt, x, a_q8)


# ---------------------------------------------------------------- sub-sums

def run_subsums(kq, fmt, W, a_q8, M, N, K):
    S = torch.full((M, N, K // SUB[fmt]), -7, dtype=torch.int32, device=DEV)
    kq.kq_gemm_subsums(fmt, dev(W), a_q8, M, N, K, S)
    torch.cuda.synchronize()
    return S.cpu().numpy()


@pytest.mark.parametrize("fmt,M,N,K", [(Q4_K, 8, 256, 512), (Q4_K, 33, 70, 768),
                                       (Q6_K, 8, 96, 512), (Q6_K, 40, 33, 256),
                                       (TQ, 8, 64, 384), (TQ, 35, 50, 640),
                                       (TQ2, 8, 64, 384), (TQ2, 35, 50, 640)])
def test_subsums_bit_exact(kq, fmt, M, N, K):
    say(f"subsums fmt={fmt} M={M} N={N} K={K}")
    W = datagen.make_weights(fmt, N, K, 1001)
    x = datagen.draw_activations(M, K, 1001)
    act_fmt = kq.kq_act_fmt_for(fmt)
    a_q8 = run_quant(kq, act_fmt, x)
    qs, d, bs = check_act_exact(kq, act_fmt, x, a_q8)
    S = run_subsums(kq, fmt, W, a_q8, M, N, K)
    assert np.array_equal(S, kqref.subsums(fmt, W, qs, K))


@pytest.mark.parametrize("name", ["proj_q4k_4096", "ffn_up_q4k_2048", "ffn_down_q6k_2048",
                                  "tern_5120_2048"])
def test_subsums_workload_slices(kq, workloads, name):
    """First 64 tokens x 256 rows x all K of each large workload."""
    say(f"subsums slice {name}")
    wl = datagen.WORKLOADS[name]
    W, x = workloads(name)
    W = np.ascontiguousarray(W[:256])
    x = np.ascontiguousarray(x[:64])
    act_fmt = kq.kq_act_fmt_for(wl.fmt)
    a_q8 = run_quant(kq, act_fmt, x)
    qs, _, _ = check_act_exact(kq, act_fmt, x, a_q8)
    S = run_subsums(kq, wl.fmt, W, a_q8, 64, 256, wl.K)
    assert np.array_equal(S, kqref.subsums(wl.fmt, W, qs, wl.K))


# ---------------------------------------------------------------- GEMM parity

@pytest.fixture(scope="module")
def workloads():
    cache = {}

    def get(name):
        if name not in cache:
            say(f"generating {name}")
            cache[name] = datagen.make_workload(name)
        return cache[name]
    return get


def gemm_vs_oracle(kq, fmt, W, x, M, N, K, rows=None, what=""):
    act_fmt = kq.kq_act_fmt_for(fmt)
    a_q8 = run_quant(kq, act_fmt, x)
    qs, d, _ = check_act_exact(kq, act_fmt, x, a_q8)
    out = run_gemm(kq, fmt, W, a_q8, M, N, K)
    ref, tol = kqref.gemm(fmt, W, qs, d, K, rows=rows)
    got = out if rows is None else out[:, rows]
    return assert_within_tol(got, ref, tol, what or f"fmt={fmt} M={M} N={N} K={K}")


def test_tiny_workload_full(kq, workloads):
    say("gemm tiny_q4k full")
    wl = datagen.WORKLOADS["tiny_q4k"]
    W, x = workloads("tiny_q4k")
    gemm_vs_oracle(kq, wl.fmt, W, x, wl.M, wl.N, wl.K)


SWEEP_M = (1, 7, 8, 24, 40, 63, 64, 65, 80, 128, 129, 300)
SWEEP_N = (48, 128, 200, 256)


@pytest.mark.parametrize("fmt", FMTS)
def test_shape_sweep(kq, fmt):
    Ks = (256, 512, 768) if fmt not in (TQ, TQ2) else (128, 384, 640)
    rng = np.random.default_rng(fmt)
    for K in Ks:
        Wfull = datagen.make_weights(fmt, max(SWEEP_N), K, 2000 + K)
        xfull = datagen.draw_activations(max(SWEEP_M), K, 3000 + K)
        for M in SWEEP_M:
            for N in SWEEP_N:
                if rng.random() < 0.5 and not (M in (1, 65) or N == 200):
                    continue
                say(f"sweep fmt={fmt} M={M} N={N} K={K}")
                gemm_vs_oracle(kq, fmt, np.ascontiguousarray(Wfull[:N]),
                               np.ascontiguousarray(xfull[:M]), M, N, K)


@pytest.mark.parametrize("name", ["proj_q4k_4096", "ffn_up_q4k_1", "ffn_up_q4k_64", "ffn_up_q4k_2048",
                                  "ffn_down_q6k_1", "ffn_down_q6k_16", "ffn_down_q6k_512", "tern_5120_1",
                                  "ffn_down_q6k_2048", "tern_5120_2048"])
def test_workload_full_size_sampled(kq, workloads, name):
    """Full-size problem in the benchmarked launch; the oracle checks a sample
    of output rows (all tokens) spread over every tile position."""
    wl = datagen.WORKLOADS[name]
    W, x = workloads(name)
    rng = np.random.default_rng(77)
    nrows = 48
    rows = np.unique(np.concatenate([[0, 1, 127, 128, wl.N - 1],
                                     rng.choice(wl.N, nrows, replace=False)]))
    say(f"gemm full-size {name} (M={wl.M} N={wl.N} K={wl.K}), {len(rows)} sampled rows")
    r = gemm_vs_oracle(kq, wl.fmt, W, x, wl.M, wl.N, wl.K, rows=rows, what=name)
    say(f"  max err/tol {r:.3g}")


def test_large_ragged_tiles(kq, workloads):
    """The persistent 128 x 128 kernel on a large shape ragged in both M (2000
    = 15 tiles + 80 rows) and N (13999 = 109 tiles + 47 columns, odd), sliced
    from the FFN draw; sampled output columns cover the first, last and
    tile-edge columns."""
    wl = datagen.WORKLOADS["ffn_up_q4k_2048"]
    W, x = workloads("ffn_up_q4k_2048")
    M, N, K = 2000, 13999, wl.K
    v = kq.kq_select_variant(Q4_K, M, N, K)
    assert kq.kq_variant_name(v) == "gemm_q4_k_128x128"
    rng = np.random.default_rng(78)
    edges = [0, 1, 31, 32, 127, 128, 255, 256, 13823, 13824, 13951, 13952, N - 1]
    rows = np.unique(np.concatenate([edges, rng.choice(N, 40, replace=False)]))
    say(f"gemm large ragged M={M} N={N} K={K}, {len(rows)} sampled columns")
    before = kq.kq_dispatch_count(v)
    r = gemm_vs_oracle(kq, Q4_K, np.ascontiguousarray(W[:N]), np.ascontiguousarray(x[:M]),
                       M, N, K, rows=rows, what="large ragged")
    assert kq.kq_dispatch_count(v) == before + 1
    say(f"  max err/tol {r:.3g}")


def test_q4k_tile_heights(kq):
    """The Q4_K tile kernel in both heights at shapes ragged in M and N: 128 x
    128 (a shape of more than 256 such tiles: 3 x 86), 64 x 128 just below
    that count (3 x 85), and the 8-wave 64 x 128 build for shapes of at most
    one 64 x 128 tile per CU, with a short K so the full output is compared."""
    K = 512
    W = datagen.make_weights(Q4_K, 11000, K, 4848)
    x = datagen.draw_activations(300, K, 4949)
    for M, N, name in ((300, 11000, "gemm_q4_k_128x128"), (300, 10880, "gemm_q4_k_64x128"),
                       (65, 4000, "gemm_q4_k_64x128_k2"), (129, 200, "gemm_q4_k_64x128_k2")):
        v = kq.kq_select_variant(Q4_K, M, N, K)
        assert kq.kq_variant_name(v) == name, (M, N)
        say(f"q4k tile {name} M={M} N={N} K={K}")
        before = kq.kq_dispatch_count(v)
        gemm_vs_oracle(kq, Q4_K, np.ascontiguousarray(W[:N]), np.ascontiguousarray(x[:M]), M, N, K)
        assert kq.kq_dispatch_count(v) == before + 1


def test_q4k_few_token_ring(kq):
    """The K-split ring kernel of 3 .. 64 tokens: its choice rule, then
    products in full against the oracle at a ragged width (11016 columns:
    the last workgroup has two 16-row strips past N and 8 columns) for all
    three token-tile builds (16, 32 and 64 rows) and odd and even superblock
    counts.  Steps per K-half T = 2, 3, 5, 7 against rings of 3 slots (32
    and 64 rows) and 4 (16 rows): tails of 1 .. 3 steps with and without
    whole ring turns before them, and none; with an odd superblock count
    the second half's last step is empty, in the turns or in the tail."""
    name = lambda M, N, K: kq.kq_variant_name(kq.kq_select_variant(Q4_K, M, N, K))
    assert name(64, 14336, 4096) == "gemm_q4_k_m64_ring"
    assert name(33, 8224, 1280) == "gemm_q4_k_m64_ring"
    assert name(64, 8192, 4096) == "gemm_q4_k_ring_kp"
    assert name(3, 14336, 4096) == "gemm_q4_k_m64_ring"
    assert name(16, 8192, 4096) == "gemm_q4_k_m16"
    N = 11016
    v = kq.kq_select_variant(Q4_K, 64, N, 768)
    for K in (768, 1280, 2304, 3584):
        W = datagen.make_weights(Q4_K, N, K, 5100 + K)
        x = datagen.draw_activations(64, K, 5200 + K)
        for M in (3, 16, 17, 32, 33, 64):
            say(f"ring M={M} N={N} K={K}")
            before = kq.kq_dispatch_count(v)
            gemm_vs_oracle(kq, Q4_K, W, np.ascontiguousarray(x[:M]), M, N, K, what=f"ring M={M} K={K}")
            assert kq.kq_dispatch_count(v) == before + 1


def test_q4k_ring_kparts(kq):
    """The ring kernel of kq_gemm_ring.hip on Q4_K (narrower weights, up to
    64 tokens): every token-tile build; on 256 CUs 4008 weight rows take
    eight K-parts (four at 64 rows) and 8192 rows four.  K = 2304 and 3584:
    tails after whole ring turns, empty K-parts; one token with K not a
    multiple of 2048 (the matrix-vector kernel declines it)."""
    name = lambda M, N, K: kq.kq_variant_name(kq.kq_select_variant(Q4_K, M, N, K))
    v = kq.kq_select_variant(Q4_K, 64, 4008, 2304)
    assert kq.kq_variant_name(v) == "gemm_q4_k_ring_kp"
    for N in (4008, 8192):
        for K in (2304, 3584):
            W = datagen.make_weights(Q4_K, N, K, 9100 + K + N)
            x = datagen.draw_activations(64, K, 9200 + K)
            for M in (1, 3, 16, 17, 32, 33, 64):
                if name(M, N, K) != "gemm_q4_k_ring_kp":
                    assert M <= 16 and N == 8192
                    continue
                say(f"q4k ring_kp M={M} N={N} K={K}")
                before = kq.kq_dispatch_count(v)
                gemm_vs_oracle(kq, Q4_K, W, np.ascontiguousarray(x[:M]), M, N, K,
                               what=f"q4k ring_kp M={M} N={N} K={K}")
                assert kq.kq_dispatch_count(v) == before + 1


def test_q6k_few_token_ring(kq):
    """The K-split Q6_K ring kernel (past the matrix-vector kernel, up to 64
    tokens): products in full against the oracle for every token-tile build
    (16, 32, 64 rows) and K-part count.  On 256 CUs, 14344 weight rows take
    two K-parts (225 workgroups of 64 rows, the last with 8), 8192 rows four
    and 4008 rows eight (four at 64 rows; the last workgroup ragged).  K =
    2304 and 3584 (9 and 14 superblocks): tails after whole ring turns, steps
    and whole K-parts past the end, blocks at both 4-byte phases.  Then the
    FFN-down shape itself at 16 tokens."""
    name = lambda M, N, K: kq.kq_variant_name(kq.kq_select_variant(Q6_K, M, N, K))
    v = kq.kq_select_variant(Q6_K, 16, 4096, 2304)
    assert kq.kq_variant_name(v) == "gemm_q6_k_ring"
    for N in (14344, 8192, 4008):
        for K in (2304, 3584):
            W = datagen.make_weights(Q6_K, N, K, 6100 + K + N)
            x = datagen.draw_activations(64, K, 6200 + K)
            for M in (3, 5, 16, 17, 32, 33, 64):
                assert name(M, N, K) == "gemm_q6_k_ring"
                say(f"q6k ring M={M} N={N} K={K}")
                before = kq.kq_dispatch_count(v)
                gemm_vs_oracle(kq, Q6_K, W, np.ascontiguousarray(x[:M]), M, N, K,
                               what=f"q6k ring M={M} N={N} K={K}")
                assert kq.kq_dispatch_count(v) == before + 1
    W = datagen.make_weights(Q6_K, 4096, 14336, 6300)
    x = datagen.draw_activations(16, 14336, 6400)
    say("q6k ring M=16 N=4096 K=14336")
    gemm_vs_oracle(kq, Q6_K, W, x, 16, 4096, 14336, what="q6k ring FFN down")


def test_tq_few_token_ring(kq):
    """The K-split ring kernel for base-3 ternary (past the matrix-vector
    kernel, up to 64 tokens, K a multiple of 256): every token-tile build and
    K-part count (14344, 8192 and 4008 weight rows), K = 2304 and 3584; with
    K = 2304 the matrix-vector kernel declines even one token."""
    name = lambda M, N, K: kq.kq_variant_name(kq.kq_select_variant(TQ, M, N, K))
    v = kq.kq_select_variant(TQ, 16, 4096, 2304)
    assert kq.kq_variant_name(v) == "gemm_tq_ring"
    for N in (14344, 8192, 4008):
        for K in (2304, 3584):
            W = datagen.make_weights(TQ, N, K, 8100 + K + N)
            x = datagen.draw_activations(64, K, 8200 + K)
            for M in (1, 3, 16, 17, 32, 33, 64):
                if name(M, N, K) != "gemm_tq_ring":
                    assert M <= 4 and K % 1024 == 0
                    continue
                say(f"tq ring M={M} N={N} K={K}")
                before = kq.kq_dispatch_count(v)
                gemm_vs_oracle(kq, TQ, W, np.ascontiguousarray(x[:M]), M, N, K,
                               what=f"tq ring M={M} N={N} K={K}")
                assert kq.kq_dispatch_count(v) == before + 1


def test_tq2_few_token_ring(kq):
    """The K-split ring kernel for two-bit ternary (1 to 64 tokens, K a
    multiple of 256): every token-tile build and K-part count as in the Q6_K
    test (14344, 8192 and 4008 weight rows), K = 2304 and 3584 (9 and 14
    chunks of two blocks), blocks at both 4-byte phases."""
    name = lambda M, N, K: kq.kq_variant_name(kq.kq_select_variant(TQ2, M, N, K))
    v = kq.kq_select_variant(TQ2, 16, 4096, 2304)
    assert kq.kq_variant_name(v) == "gemm_tq2_ring"
    for N in (14344, 8192, 4008):
        for K in (2304, 3584):
            W = datagen.make_weights(TQ2, N, K, 7100 + K + N)
            x = datagen.draw_activations(64, K, 7200 + K)
            for M in (1, 3, 16, 17, 32, 33, 64):
                assert name(M, N, K) == "gemm_tq2_ring"
                say(f"tq2 ring M={M} N={N} K={K}")
                before = kq.kq_dispatch_count(v)
                gemm_vs_oracle(kq, TQ2, W, np.ascontiguousarray(x[:M]), M, N, K,
                               what=f"tq2 ring M={M} N={N} K={K}")
                assert kq.kq_dispatch_count(v) == before + 1


SPLIT_TILE = {Q6_K: "gemm_q6_k_128x128_k2", TQ: "gemm_tq_128x128_k2", TQ2: "gemm_tq2_128x128_k2"}
SPLIT_SHAPES = {
    # (M, N, K): chunks of 128 values per part in the comments
    Q6_K: ((300, 4000, 4096),    # 16 / 16
           (300, 4000, 2304),    # 12 / 6
           (65, 4099, 1280)),    # 8 / 2; an output count that is not a multiple of 4
    TQ: ((300, 4000, 4096), (129, 2000, 1152),   # 8 / 1
         (70, 4000, 5248),                        # 24 / 17
         (5, 4095, 5248)),                        # a few tokens, K not a multiple of 256
}
SPLIT_SHAPES[TQ2] = SPLIT_SHAPES[TQ]


@pytest.mark.parametrize("fmt", sorted(SPLIT_TILE))
def test_tile_split_k(kq, fmt):
    """The 128 x 128 tile kernel with K in two parts (grid row 0 and 1),
    each adding into the zeroed output, on shapes whose tiles cover at most
    half the CUs: full products against the oracle (the output starts as NaN,
    so a missed zero fill fails) with parts of equal and unequal length, a
    part of one chunk, ragged M and N; then sampled columns of 512 x 4096 x
    14336; and the same product twice, bit for bit (two addends onto zero
    commute in fp32)."""
    name = SPLIT_TILE[fmt]
    for M, N, K in SPLIT_SHAPES[fmt]:
        v = kq.kq_select_variant(fmt, M, N, K)
        assert kq.kq_variant_name(v) == name, (M, N, K)
        W = datagen.make_weights(fmt, N, K, 9500 + N + K + fmt)
        x = datagen.draw_activations(M, K, 9600 + K + fmt)
        say(f"{name} M={M} N={N} K={K}")
        before = kq.kq_dispatch_count(v)
        gemm_vs_oracle(kq, fmt, W, x, M, N, K, what=f"{name} M={M} N={N} K={K}")
        assert kq.kq_dispatch_count(v) == before + 1
    M, N, K = 512, 4096, 14336
    assert kq.kq_variant_name(kq.kq_select_variant(fmt, M, N, K)) == name
    W = datagen.make_weights(fmt, N, K, 9700 + fmt)
    x = datagen.draw_activations(M, K, 9800 + fmt)
    rows = np.unique(np.concatenate([[0, 127, 128, N - 1], np.random.default_rng(9900).choice(N, 48, replace=False)]))
    say(f"{name} M={M} N={N} K={K}, {len(rows)} sampled columns")
    gemm_vs_oracle(kq, fmt, W, x, M, N, K, rows=rows, what=f"{name} 512 x 4096 x 14336")
    a_q8 = kq.quantize_act(dev(x), kq.kq_act_fmt_for(fmt))
    Wd = dev(W)
    o1 = run_gemm(kq, fmt, Wd, a_q8, M, N, K)
    o2 = run_gemm(kq, fmt, Wd, a_q8, M, N, K)
    assert np.array_equal(o1.view(np.uint32), o2.view(np.uint32)), f"{name}: two runs differ"


@pytest.mark.parametrize("fmt", FMTS)
def test_random_shapes_every_route(kq, fmt):
    """Seeded random shapes across the routing boundaries (mat-vec, ring
    kernels with and without slices and in both wave counts, tile kernels
    whole and with K in two parts): 16 products per format with M in 1..700,
    N in 1..8000 and K up to 8192, the oracle's work bounded, each against
    the oracle in full; the variants reached are printed."""
    rng = np.random.default_rng(4242 + fmt)
    qk = 256 if fmt in (Q4_K, Q6_K) else 128
    seen = {}
    done = 0
    while done < 16:
        M = int(rng.choice([rng.integers(1, 5), rng.integers(5, 65), rng.integers(65, 700)]))
        N = int(rng.integers(1, 8000))
        K = qk * int(rng.integers(1, 8192 // qk + 1))
        if M * N * K > 2e9:
            continue
        name = kq.kq_variant_name(kq.kq_select_variant(fmt, M, N, K))
        W = datagen.make_weights(fmt, N, K, 7700 + 31 * done + fmt)
        x = datagen.draw_activations(M, K, 7800 + 31 * done + fmt)
        say(f"random {name} M={M} N={N} K={K}")
        gemm_vs_oracle(kq, fmt, W, x, M, N, K, what=f"random {name} M={M} N={N} K={K}")
        seen[name] = seen.get(name, 0) + 1
        done += 1
    say(f"  variants reached: {seen}")


GRAPH_CASES = [
    (Q4_K, 300, 11000, 512, "gemm_q4_k_128x128"),
    (Q4_K, 64, 11008, 512, "gemm_q4_k_m64_ring"),
    (Q4_K, 2, 1000, 2048, "gemm_q4_k_matvec"),
    (Q4_K, 40, 1000, 2048, "gemm_q4_k_ring_kp"),      # four-wave build
    (Q6_K, 300, 4000, 4096, "gemm_q6_k_128x128_k2"),  # zero fill, then two parts adding
    (Q6_K, 128, 1024, 4096, "gemm_q6_k_ring"),         # two 64-token slices
    (TQ, 1, 1000, 2048, "gemm_tq_matvec"),
    (TQ2, 600, 130, 1152, "gemm_tq2_128x128_k2"),
]


def test_graph_capture_replays(kq):
    """Quantize + product captured in one HIP graph (the library records no
    memset and allocates nothing), replayed three times with eager work
    between the replays (the buffers refilled, the device synchronized): every
    replay equals the eager call bit for bit, on each kernel family,
    including the two-part tile kernel with its zero fill."""
    import torch
    for fmt, M, N, K, name in GRAPH_CASES:
        assert kq.kq_variant_name(kq.kq_select_variant(fmt, M, N, K)) == name, (fmt, M, N, K)
        act = kq.kq_act_fmt_for(fmt)
        W = dev(datagen.make_weights(fmt, N, K, 9950 + fmt + M))
        x = dev(datagen.draw_activations(M, K, 9960 + fmt + M))
        a_q8 = torch.empty(kq.kq_act_bytes(act, M, K), dtype=torch.uint8, device=DEV)
        out = torch.full((M, N), float("nan"), dtype=torch.float32, device=DEV)
        kq.kq_quantize_act(act, x, M, K, a_q8)
        kq.kq_gemm(fmt, W, a_q8, M, N, K, out)
        torch.cuda.synchronize()
        ref = out.clone()
        say(f"graph {name} M={M} N={N} K={K}")
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=side):
            kq.kq_quantize_act(act, x, M, K, a_q8)
            kq.kq_gemm(fmt, W, a_q8, M, N, K, out)
        torch.cuda.synchronize()
        for r in range(3):
            out.fill_(float("nan"))
            a_q8.zero_()
            torch.cuda.synchronize()
            g.replay()
            torch.cuda.synchronize()
            assert torch.equal(out.view(torch.int32), ref.view(torch.int32)), f"{name}: replay {r} differs"
        del g


SLICE_RING = {Q4_K: "gemm_q4_k_ring_kp", Q6_K: "gemm_q6_k_ring", TQ: "gemm_tq_ring", TQ2: "gemm_tq2_ring"}


@pytest.mark.parametrize("fmt", sorted(SLICE_RING))
def test_ring_token_slices(kq, fmt):
    """Past 64 tokens the ring kernel runs one 64-token slice per grid row,
    each slice's activations, scales, min-term operands and output rows at
    its own offset: full products against the oracle at 65 tokens (one in
    the second slice), 128, 200 (ragged), 320 and 512, on 1000 weight rows
    (ragged against the 32- and 64-row workgroups) and 1024, K = 2304 (a
    tail after whole ring turns) and 4096.  Then 128 tokens on the FFN-down
    shape 4096 x 14336."""
    name = SLICE_RING[fmt]
    for N in (1000, 1024):
        for K in (2304, 4096):
            W = datagen.make_weights(fmt, N, K, 9100 + N + K + fmt)
            x = datagen.draw_activations(512, K, 9200 + K + fmt)
            for M in (65, 128, 200, 320, 512):
                v = kq.kq_select_variant(fmt, M, N, K)
                assert kq.kq_variant_name(v) == name, (M, N, K)
                say(f"{name} slices M={M} N={N} K={K}")
                before = kq.kq_dispatch_count(v)
                gemm_vs_oracle(kq, fmt, W, np.ascontiguousarray(x[:M]), M, N, K,
                               what=f"{name} slices M={M} N={N} K={K}")
                assert kq.kq_dispatch_count(v) == before + 1
    M, N, K = 128, 4096, 14336
    assert kq.kq_variant_name(kq.kq_select_variant(fmt, M, N, K)) == name
    W = datagen.make_weights(fmt, N, K, 9300 + fmt)
    x = datagen.draw_activations(M, K, 9400 + fmt)
    say(f"{name} slices M={M} N={N} K={K}")
    gemm_vs_oracle(kq, fmt, W, x, M, N, K, what=f"{name} slices FFN down")


MATVEC = {Q4_K: ("gemm_q4_k_matvec", (1, 2)), Q6_K: ("gemm_q6_k_matvec", (1, 2, 3, 4)),
          TQ: ("gemm_tq_matvec", (1, 2, 3, 4)), TQ2: ("gemm_tq2_matvec", (1, 2, 3, 4))}


@pytest.mark.parametrize("fmt", sorted(MATVEC))
@pytest.mark.parametrize("K", [2048, 4096])
def test_matvec_path(kq, fmt, K):
    """The matrix-vector kernels (a handful of tokens, K a multiple of 2048):
    every token count each is built for, N ragged against their 16-row
    workgroups, full output against the oracle."""
    name, tokens = MATVEC[fmt]
    Wfull = datagen.make_weights(fmt, 1000, K, 4000 + K)
    xfull = datagen.draw_activations(max(tokens), K, 5000 + K)
    for M in tokens:
        for N in (16, 40, 1000):
            v = kq.kq_select_variant(fmt, M, N, K)
            assert kq.kq_variant_name(v) == name
            say(f"matvec fmt={fmt} M={M} N={N} K={K}")
            before = kq.kq_dispatch_count(v)
            gemm_vs_oracle(kq, fmt, np.ascontiguousarray(Wfull[:N]),
                           np.ascontiguousarray(xfull[:M]), M, N, K)
            assert kq.kq_dispatch_count(v) == before + 1


def test_matvec_boundaries(kq):
    """Shapes just outside the matrix-vector kernels' rules go to the
    tile kernels; inside them the long-K projection still takes them."""
    name = lambda M, N, K: kq.kq_variant_name(kq.kq_select_variant(Q4_K, M, N, K))
    assert name(3, 4200, 4096) == "gemm_q4_k_m16"
    assert name(2, 4200, 1792) == "gemm_q4_k_m16"      # K not a multiple of 2048
    assert name(2, 4200, 2048 * 9) == "gemm_q4_k_m16"  # staged activations past the budget
    assert name(2, 4096, 1792) == "gemm_q4_k_ring_kp"  # ... on narrower weights
    assert name(16, 4200, 4096) == "gemm_q4_k_m16"
    assert name(17, 4200, 4096) == "gemm_q4_k_ring_kp"
    Ws = datagen.make_weights(Q4_K, 4200, 4096, 4141)
    xs = datagen.draw_activations(16, 4096, 4040)
    say("split M=16 N=4200 K=4096")
    gemm_vs_oracle(kq, Q4_K, Ws, xs, 16, 4200, 4096)
    assert name(2, 4096, 14336) == "gemm_q4_k_matvec"
    W = datagen.make_weights(Q4_K, 48, 14336, 4242)
    x = datagen.draw_activations(2, 14336, 4343)
    say("matvec M=2 N=48 K=14336")
    gemm_vs_oracle(kq, Q4_K, W, x, 2, 48, 14336)
    q6 = lambda M, N, K: kq.kq_variant_name(kq.kq_select_variant(Q6_K, M, N, K))
    assert q6(5, 4096, 14336) == "gemm_q6_k_ring"
    assert q6(4, 4096, 14336 + 256) == "gemm_q6_k_ring"  # K not a multiple of 2048
    assert q6(4, 4096, 14336) == "gemm_q6_k_matvec"
    assert q6(65, 4096, 14336) == "gemm_q6_k_ring"       # 64-token slices
    assert q6(520, 4096, 14336) == "gemm_q6_k_128x128"
    tq = lambda M, N, K: kq.kq_variant_name(kq.kq_select_variant(TQ, M, N, K))
    assert tq(9, 17408, 5120) == "gemm_tq_ring"           # past the matrix-vector kernel
    assert tq(65, 17408, 5120) == "gemm_tq_128x128"       # fewer 128 x 128 tiles than CUs
    assert tq(256, 17408, 5120) == "gemm_tq_128x128_reg"
    assert tq(4, 17408, 5120 + 128) == "gemm_tq_128x128"  # K not a multiple of 1024 (nor of 256)
    assert tq(4, 17408, 5120) == "gemm_tq_matvec"
    assert tq(5, 17408, 5120) == "gemm_tq_ring"
    Wt = datagen.make_weights(TQ, 40, 5120, 4646)
    xt = datagen.draw_activations(4, 5120, 4747)
    say("matvec ternary M=4 N=40 K=5120")
    gemm_vs_oracle(kq, TQ, Wt, xt, 4, 40, 5120)
    W6 = datagen.make_weights(Q6_K, 40, 14336, 4444)
    x6 = datagen.draw_activations(4, 14336, 4545)
    say("matvec Q6_K M=4 N=40 K=14336")
    gemm_vs_oracle(kq, Q6_K, W6, x6, 4, 40, 14336)


def test_other_reading_of_distributions(kq):
    """Config text 'same value distributions as config 1' read 0-based: outlier
    weights and LogNormal channel scales on the FFN shape (sliced)."""
    say("gemm ffn shape under the outlier/LogNormal distributions")
    M, N, K = 256, 512, 4096
    W = datagen.make_weights(Q4_K, N, K, 1003, "outlier_lognormal")
    x = datagen.draw_activations(M, K, 1003, "outlier_lognormal")
    gemm_vs_oracle(kq, Q4_K, W, x, M, N, K)
    W6 = datagen.make_weights(Q6_K, 256, 2048, 1004, "outlier_lognormal")
    x6 = datagen.draw_activations(200, 2048, 1004, "outlier_lognormal")
    gemm_vs_oracle(kq, Q6_K, W6, x6, 200, 256, 2048)


# ------------------------------------------------- exact special cases of the real kernel

def hand_act_q8k(kq, qs):
    """Q8_K buffer with unit scales and consistent sums, built on the host."""
    M, K = qs.shape
    buf = np.zeros(kq.kq_act_bytes(1, M, K), np.uint8)
    od = kq.kq_act_section_offset(1, 1, M, K)
    ob = kq.kq_act_section_offset(1, 2, M, K)
    buf[:M * K] = qs.view(np.uint8).reshape(-1)
    buf[od:od + M * (K // 256) * 4] = np.ones((M, K // 256), np.float32).view(np.uint8).reshape(-1)
    bs = qs.astype(np.int32).reshape(M, K // 16, 16).sum(axis=2).astype(np.int16)
    buf[ob:ob + M * (K // 16) * 2] = bs.view(np.uint8).reshape(-1)
    oa = kq.kq_act_section_offset(1, 3, M, K)
    al = expected_alpha(qs, np.ones((M, K // 256), np.float32))
    buf[oa:oa + al.nbytes] = al.view(np.uint8).reshape(-1)
    return dev(buf)


def hand_act_q8_128(kq, qs):
    M, K = qs.shape
    buf = np.zeros(kq.kq_act_bytes(2, M, K), np.uint8)
    od = kq.kq_act_section_offset(2, 1, M, K)
    buf[:M * K] = qs.view(np.uint8).reshape(-1)
    buf[od:od + M * (K // 128) * 4] = np.ones((M, K // 128), np.float32).view(np.uint8).reshape(-1)
    return dev(buf)


@pytest.mark.parametrize("fmt", (Q4_K, Q6_K))
def test_onehot_scales_expose_subsums(kq, fmt):
    """d = d_a = 1, no mins, scale vector e_j: the production kernel's output is
    exactly the sub-block sum S[:, :, j]."""
    rng = np.random.default_rng(31 + fmt)
    M, N, K = 70, 96, 512
    qs = rng.integers(-127, 128, size=(M, K)).astype(np.int8)
    a_q8 = hand_act_q8k(kq, qs)
    nsub = 8 if fmt == Q4_K else 16
    for j in range(nsub):
        say(f"one-hot fmt={fmt} j={j}")
        B = N * (K // 256)
        one = np.zeros((B, nsub), np.int64)
        one[:, j] = 1
        if fmt == Q4_K:
            q = rng.integers(0, 16, size=(B, 256))
            mn = rng.integers(0, 64, size=(B, 8))
            W = datagen.pack_q4k(np.ones(B, np.float16), np.zeros(B, np.float16), one, mn, q)
        else:
            q = rng.integers(0, 64, size=(B, 256))
            W = datagen.pack_q6k(np.ones(B, np.float16), one, q)
        W = W.reshape(N, -1)
        out = run_gemm(kq, fmt, W, a_q8, M, N, K)
        S = kqref.subsums(fmt, W, qs, K)
        want = np.stack([S[:, :, j + nsub * s] for s in range(K // 256)]).sum(axis=0)
        assert np.array_equal(out, want.astype(np.float32)), f"one-hot j={j}"


def test_unit_scale_ternary_is_integer_matmul(kq):
    say("ternary unit scales")
    rng = np.random.default_rng(41)
    M, N, K = 67, 90, 640
    qs = rng.integers(-127, 128, size=(M, K)).astype(np.int8)
    t = rng.integers(-1, 2, size=(N, K))
    W = datagen.encode_tq(t.astype(np.int8), np.ones((N, K // 128), np.float16))
    out = run_gemm(kq, TQ, W, hand_act_q8_128(kq, qs), M, N, K)
    want = qs.astype(np.int64) @ t.astype(np.int64).T
    assert np.array_equal(out, want.astype(np.float32))


@pytest.mark.parametrize("fmt", FMTS)
def test_zero_and_negated_activations(kq, fmt):
    say(f"x=0 and x->-x fmt={fmt}")
    M, N, K = 96, 160, 768 if fmt not in (TQ, TQ2) else 640
    W = datagen.make_weights(fmt, N, K, 55)
    x = datagen.draw_activations(M, K, 56)
    act_fmt = kq.kq_act_fmt_for(fmt)
    out = run_gemm(kq, fmt, W, run_quant(kq, act_fmt, x), M, N, K)
    neg = run_gemm(kq, fmt, W, run_quant(kq, act_fmt, -x), M, N, K)
    if fmt == Q4_K:
        # The Q4_K min term goes through a bf16 MFMA whose internal fp32
        # accumulation is not exactly sign-symmetric (measured: differences of
        # about one ulp of the partial sums); everything else negates exactly.
        qs, d, _ = kqref.quantize_act(act_fmt, x)
        _, tol = kqref.gemm(fmt, W, qs, d, K)
        assert np.all(np.abs(neg.astype(np.float64) + out) <= 0.01 * tol)
    else:
        assert np.array_equal(neg, -out)
    zero = run_gemm(kq, fmt, W, run_quant(kq, act_fmt, np.zeros_like(x)), M, N, K)
    assert np.all(zero == 0)


# ------------------------------------------------- expert-indexed product

def routing(rng, M, counts):
    """Synthetic routing: expert e takes counts[e] routed rows of random tokens
    (repeats allowed); returns int32 offsets [E+1] and rows [R]."""
    off = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    rows = np.concatenate([rng.integers(0, M, size=c) for c in counts]).astype(np.int32)
    return off, rows


@pytest.mark.parametrize("fmt", FMTS)
def test_gemm_id_matches_oracle(kq, fmt):
    """Every routed row against the oracle on its expert and token; experts
    with no row, one row, and more rows than a tile; canaries after out."""
    E, M, N = 8, 97, 200
    K = 640 if fmt in (TQ, TQ2) else 512
    rng = np.random.default_rng(60 + fmt)
    counts = [0, 1, 129, 7, 40, 0, 64, 33]
    off, rows = routing(rng, M, counts)
    R = int(off[-1])
    Ws = [datagen.make_weights(fmt, N, K, 900 + e) for e in range(E)]
    W = np.concatenate([w.reshape(-1) for w in Ws])
    x = datagen.draw_activations(M, K, 61)
    act_fmt = kq.kq_act_fmt_for(fmt)
    a_q8 = run_quant(kq, act_fmt, x)
    qs, d, _ = check_act_exact(kq, act_fmt, x, a_q8)
    say(f"gemm_id fmt={fmt} E={E} M={M} N={N} K={K} R={R}")
    ob = torch.full((R + 3, N), 12345.0, dtype=torch.float32, device=DEV)
    variant = "gemm_id_q4_k_64x128" if fmt == Q4_K else "gemm_id_128x128"
    before = kq.dispatch_counts()[variant]
    kq.kq_gemm_id(fmt, dev(W), E, a_q8, M, N, K, dev(off), dev(rows), R, ob)
    torch.cuda.synchronize()
    assert kq.dispatch_counts()[variant] == before + 1
    out = ob.cpu().numpy()
    assert np.all(out[R:] == 12345.0), "rows past R written"
    for e in range(E):
        r0, r1 = int(off[e]), int(off[e + 1])
        if r0 == r1:
            continue
        toks = rows[r0:r1]
        ref, tol = kqref.gemm(fmt, Ws[e], np.ascontiguousarray(qs[toks]), np.ascontiguousarray(d[toks]), K)
        assert_within_tol(out[r0:r1], ref, tol, f"gemm_id fmt={fmt} expert {e}")
        same = {Q4_K: ("gemm_q4_k_64x128", "gemm_q4_k_128x128")}.get(fmt, (f"gemm_{FMT_NAME[fmt]}_128x128",))
        if kq.kq_variant_name(kq.kq_select_variant(fmt, r1 - r0, N, K)) in same:
            # the plain product of the same tile kernel on the gathered tokens
            # (Q4_K: a 4-wave tile kernel, either height): identical
            # arithmetic, identical bits (the 8-wave build adds its two
            # superblock streams in another order)
            xg = np.ascontiguousarray(x[toks])
            plain = run_gemm(kq, fmt, Ws[e], run_quant(kq, act_fmt, xg), r1 - r0, N, K)
            assert np.array_equal(out[r0:r1], plain), f"expert {e} differs from kq_gemm"


def test_gemm_id_many_experts(kq):
    """Q4_K gather kernel with 300 experts, most of them empty and a few
    spanning several 64-row tiles (the kernel counts the tiles and finds
    each tile's expert from the offsets): sampled experts against the oracle,
    every expert's rows finite, canaries after out."""
    E, M, N, K = 300, 150, 96, 256
    rng = np.random.default_rng(303)
    counts = np.zeros(E, np.int64)
    busy = rng.choice(E, 12, replace=False)
    counts[busy] = rng.integers(1, 200, size=12)
    counts[busy[0]], counts[E - 1] = 129, 64
    off, rows = routing(rng, M, counts)
    R = int(off[-1])
    W = datagen.make_weights(Q4_K, E * N, K, 304)
    x = datagen.draw_activations(M, K, 305)
    a_q8 = run_quant(kq, kq.KQ_ACT_Q8_K, x)
    qs, d, _ = check_act_exact(kq, kq.KQ_ACT_Q8_K, x, a_q8)
    say(f"gemm_id many experts E={E} R={R}")
    ob = torch.full((R + 2, N), 12345.0, dtype=torch.float32, device=DEV)
    before = kq.dispatch_counts()["gemm_id_q4_k_64x128"]
    kq.kq_gemm_id(Q4_K, dev(W), E, a_q8, M, N, K, dev(off), dev(rows), R, ob)
    torch.cuda.synchronize()
    assert kq.dispatch_counts()["gemm_id_q4_k_64x128"] == before + 1
    out = ob.cpu().numpy()
    assert np.all(out[R:] == 12345.0) and np.all(np.isfinite(out[:R]))
    for e in sorted(set(busy[:6].tolist()) | {E - 1}):
        r0, r1 = int(off[e]), int(off[e + 1])
        toks = rows[r0:r1]
        ref, tol = kqref.gemm(Q4_K, W[e * N:(e + 1) * N], np.ascontiguousarray(qs[toks]),
                              np.ascontiguousarray(d[toks]), K)
        assert_within_tol(out[r0:r1], ref, tol, f"gemm_id many experts: expert {e}")


@pytest.mark.parametrize("fmt", (Q6_K, Q4_K))
def test_gemm_id_routing_out_of_contract_stays_in_bounds(kq, fmt):
    """Offsets past R, decreasing offsets and token indices past M give
    undefined values but no access outside the buffers: canaries around out
    stay intact and the call completes (both gather kernels)."""
    E, M, N, K = 4, 20, 64, 256
    rng = np.random.default_rng(77)
    W = np.concatenate([datagen.make_weights(fmt, N, K, 70 + e).reshape(-1) for e in range(E)])
    a_q8 = run_quant(kq, kq.KQ_ACT_Q8_K, datagen.draw_activations(M, K, 71))
    R = 50
    off = np.array([0, 30, 10, 60, 1000], np.int32)     # decreasing, then past R
    rows = rng.integers(-5, M + 5, size=R).astype(np.int32)
    pad = 4096
    ob = torch.full((R * N + 2 * pad,), 7.0, dtype=torch.float32, device=DEV)
    view = ob[pad:pad + R * N].view(R, N)
    kq.kq_gemm_id(fmt, dev(W), E, a_q8, M, N, K, dev(off), dev(rows), R, view)
    torch.cuda.synchronize()
    assert torch.all(ob[:pad] == 7.0).item() and torch.all(ob[pad + R * N:] == 7.0).item()


# ------------------------------------------------- the gate is not vacuous

# (fmt, field, byte offset inside the block, xor mask): one stored field of
# one block changed in the copy of the weights the GPU gets
MUTATIONS = [
    (Q4_K, "nibble", 16 + 40, 0x08),            # bit 3 of a 4-bit quant
    (Q4_K, "scale", 4 + 2, 0x02),               # bit 5 of the 6-bit scale field 2
    (Q4_K, "min", 4 + 8, 0x40),                 # bit 4 of the 6-bit min field 3
    (Q6_K, "low bits", 10, 0x08),               # bit 3 of a quant's low nibble
    (Q6_K, "high bits", 128 + 5, 0x02),         # the high bit of a quant's top pair
    (Q6_K, "scale", 192 + 3, 0x40),             # bit 6 of an int8 scale
    (TQ, "trit", 7, None),                      # one base-3 digit of byte 7
    (TQ2, "code", 9, 0x30),                     # the code of weight 73 (bits 4-5 of byte 9)
]


@pytest.mark.parametrize("fmt,field,off,mask", MUTATIONS,
                         ids=[f"{f}-{w}" for f, w, _, _ in MUTATIONS])
def test_gate_fails_on_a_flipped_field(kq, fmt, field, off, mask):
    """One field flipped in the GPU's copy of the weights must fail the
    comparison with the oracle run on the original, in exactly the output
    column of the changed weight row."""
    say(f"mutation fmt={fmt} {field}")
    M, N = 64, 96
    K = 384 if fmt in (TQ, TQ2) else 512
    W = datagen.make_weights(fmt, N, K, 71)
    x = datagen.draw_activations(M, K, 72)
    act_fmt = kq.kq_act_fmt_for(fmt)
    qs, d, _ = kqref.quantize_act(act_fmt, x)
    ref, tol = kqref.gemm(fmt, W, qs, d, K)
    a_q8 = run_quant(kq, act_fmt, x)
    assert_within_tol(run_gemm(kq, fmt, W, a_q8, M, N, K), ref, tol, "unmutated")

    n, bb = 37, {Q4_K: 144, Q6_K: 210, TQ: 28, TQ2: 34}[fmt]
    Wm = W.copy()
    i = bb + off                                   # second block of row n
    if mask is None:                               # next base-3 value of the lowest digit
        v = int(Wm[n, i])
        Wm[n, i] = v + 1 if v % 3 != 2 else v - 2
    elif fmt == TQ2:                               # next valid code (0 -> 1 -> 2 -> 0)
        c = (int(Wm[n, i]) >> 4) & 3
        Wm[n, i] = (int(Wm[n, i]) & ~0x30) | (((c + 1) % 3) << 4)
    else:
        Wm[n, i] ^= mask
    changed = np.argwhere(kqref.dequant_rows(fmt, Wm, K) != kqref.dequant_rows(fmt, W, K))
    assert changed.size and set(changed[:, 0]) == {n}, "the mutation must change row n only"
    out = run_gemm(kq, fmt, Wm, a_q8, M, N, K)
    bad = np.abs(out.astype(np.float64) - ref) > tol
    assert bad.any(), f"{field} flip not caught by the gate"
    assert set(np.nonzero(bad)[1]) == {n}


# ------------------------------------------------- out-of-bounds canaries

@pytest.mark.parametrize("fmt", FMTS)
def test_canaries_and_poisoned_tails(kq, fmt):
    """Inputs end at the last valid byte of larger buffers whose tails hold
    garbage; the output is a view followed by NaN canaries.  Results must equal
    the clean run and the canaries must be untouched."""
    say(f"canaries fmt={fmt}")
    M, N, K = 77, 131, 512 if fmt not in (TQ, TQ2) else 384
    W = datagen.make_weights(fmt, N, K, 91)
    x = datagen.draw_activations(M, K, 92)
    act_fmt = kq.kq_act_fmt_for(fmt)
    a_clean = run_quant(kq, act_fmt, x)
    ref = run_gemm(kq, fmt, W, a_clean, M, N, K)

    pad = 4096
    wb = np.full(W.nbytes + pad, 0xFF, np.uint8)
    wb[:W.nbytes] = W.reshape(-1)
    Wd = dev(wb)
    ab = torch.full((a_clean.numel() + pad,), 0x7F, dtype=torch.uint8, device=DEV)
    ab[:a_clean.numel()] = a_clean
    ob = torch.full((M * N + pad,), float("nan"), dtype=torch.float32, device=DEV)
    ob[M * N:] = 12345.0
    kq.kq_gemm(fmt, Wd, ab, M, N, K, ob)
    torch.cuda.synchronize()
    got = ob[:M * N].cpu().numpy().reshape(M, N)
    assert np.array_equal(got, ref)
    assert torch.all(ob[M * N:] == 12345.0).item()


def test_empty_problems_are_noops(kq):
    say("empty problems")
    out = torch.full((4, 4), 7.0, device=DEV)
    a = torch.zeros(4096, dtype=torch.uint8, device=DEV)
    kq.kq_gemm(Q4_K, a, a, 0, 4, 256, out)
    kq.kq_gemm(Q4_K, a, a, 4, 0, 256, out)
    torch.cuda.synchronize()
    assert torch.all(out == 7.0).item()


def test_zero_k_gives_zero(kq):
    say("K = 0")
    out = torch.full((5, 6), 7.0, device=DEV)
    a = torch.zeros(4096, dtype=torch.uint8, device=DEV)
    for fmt in FMTS:
        out.fill_(7.0)
        kq.kq_gemm(fmt, a, a, 5, 6, 0, out)
        torch.cuda.synchronize()
        assert torch.all(out == 0.0).item()


@pytest.mark.parametrize("M,N,K,variant", [
    (512, 16384, 5120, "gemm_tq_128x128_reg"),       # 512 tiles: one full round of two per CU
    (1024, 17408, 5376, "gemm_tq_128x128_reg"),      # 1088 tiles, 2.1 rounds; 21 steps per tile
])
def test_ternary_register_kernels(kq, M, N, K, variant):
    """The ternary register-unpack tile kernel against the oracle on sampled
    weight rows (the first, last and random ones)."""
    assert kq.kq_variant_name(kq.kq_select_variant(TQ, M, N, K)) == variant
    say(f"{variant}: M={M} N={N} K={K}")
    rng = np.random.default_rng(M + N + K)
    t = rng.choice(np.array([-1, 0, 1], np.int8), size=(N, K), p=[0.3, 0.4, 0.3])
    d = rng.uniform(0.01, 0.05, size=(N, K // 128)).astype(np.float16)
    W = datagen.encode_tq(t, d)
    x = datagen.draw_activations(M, K, M + 7)
    rows = np.unique(np.concatenate([[0, 1, 127, 128, N - 2, N - 1], rng.choice(N, 24, replace=False)]))
    names = [kq.kq_variant_name(v) for v in range(kq.kq_num_variants())]
    before = kq.kq_dispatch_count(names.index(variant))
    gemm_vs_oracle(kq, TQ, W, x, M, N, K, rows=rows, what=variant)
    assert kq.kq_dispatch_count(names.index(variant)) == before + 1


def test_zz_every_variant_dispatched(kq):
    """Runs last in this file: every kernel variant in the table was launched by
    the tests above (the counters prove which kernel ran)."""
    counts = kq.dispatch_counts()
    say(f"dispatch counts: {counts}")
    missing = [name for name, c in counts.items() if c == 0]
    assert not missing, f"variants never dispatched: {missing}"
