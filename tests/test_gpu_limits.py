"""GPU tests at the largest shapes the library accepts.

The kernels address each operand with 32-bit byte offsets, and the host
declines any shape where an operand plus the rows a last tile hangs past it
reaches 2^31 bytes (KQ_ERR_UNSUPPORTED; checked without a GPU in
test_abi.py).  These tests run shapes just inside that limit: about 2 GiB of
weights through every kernel family, and about 2 GiB of output, and compare
sampled outputs (first, last and random weight rows) with the oracle.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

from oracle import kqref

pytestmark = pytest.mark.gpu

Q4_K, Q6_K, TQ, TQ2 = 1, 2, 3, 4
QK = {Q4_K: 256, Q6_K: 256, TQ: 128, TQ2: 128}
BB = {Q4_K: 144, Q6_K: 210, TQ: 28, TQ2: 34}
DEV = "cuda:0"
LIMIT = 1 << 31


def say(*a):
    print(*a, flush=True)


@pytest.fixture(scope="module")
def kq():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import block_quantized_matmul_act_amd as kq
    kq.lib()
    return kq


def random_blocks(fmt: int, nblocks: int, seed: int) -> np.ndarray:
    """nblocks valid blocks of random content with small finite fp16 scales."""
    rng = np.random.default_rng(seed)
    b = rng.integers(0, 256, size=(nblocks, BB[fmt]), dtype=np.uint8)
    if fmt == Q4_K:
        b[:, 0:2] = np.array([0.004], np.float16).view(np.uint8)
        b[:, 2:4] = np.array([0.002], np.float16).view(np.uint8)
    elif fmt == Q6_K:
        b[:, 208:210] = np.array([0.003], np.float16).view(np.uint8)
    elif fmt == TQ2:
        b[:, :32] &= 0x55  # codes 0 or 1 in every field: valid
        b[:, 32:34] = np.array([0.01], np.float16).view(np.uint8)
    else:
        b[:, :25] %= 243
        b[:, 25] = 108 + b[:, 25] % 27
        b[:, 26:28] = np.array([0.01], np.float16).view(np.uint8)
    return b


def quantize(kq, fmt, x):
    M, K = x.shape
    act = kq.kq_act_fmt_for(fmt)
    a_q8 = kq.quantize_act(torch.from_numpy(x).to(DEV), act)
    qs, d, _ = kqref.quantize_act(act, x)
    return a_q8, qs, d


def check_columns(out, ref, tol, what):
    err = np.abs(out.astype(np.float64) - ref)
    assert np.all(np.isfinite(out)), what + ": non-finite output"
    assert np.all(err <= tol), f"{what}: max err/tol {(err / tol).max():.3g}"


# (fmt, K, token counts: one per kernel family)
WEIGHT_CASES = [
    (Q4_K, 4096, (1, 40, 200)),     # matrix-vector, few-token, 128 x 128
    (Q4_K, 131072, (100,)),         # 64 x 128 (226 column tiles)
    (Q6_K, 4096, (1, 40)),          # matrix-vector, 128 x 128 tile
    (Q6_K, 589824, (128, 200)),     # ring kernel in 64-token slices, tile kernel with K in two parts
    (TQ, 5120, (1, 40)),            # matrix-vector, 128 x 128 tile
    (TQ2, 5120, (1, 40)),           # 128 x 128 tile
]


@pytest.mark.parametrize("fmt,K,Ms", WEIGHT_CASES, ids=["q4_k", "q4_k_long_k", "q6_k", "q6_k_long_k", "tq", "tq2"])
def test_weights_just_below_2gib(kq, fmt, K, Ms):
    rowbytes = (K // QK[fmt]) * BB[fmt]
    N = LIMIT // rowbytes - 256           # largest N with (N + 256) * rowbytes < 2^31
    if (N + 256) * rowbytes >= LIMIT:
        N -= 1
    assert (N + 256) * rowbytes < LIMIT <= (N + 257) * rowbytes
    say(f"weights near 2 GiB: fmt={fmt} N={N} K={K} ({N * rowbytes / 2**30:.3f} GiB)")
    W = random_blocks(fmt, N * (K // QK[fmt]), 500 + fmt).reshape(N, rowbytes)
    Wd = torch.from_numpy(W).to(DEV)
    rng = np.random.default_rng(600 + fmt)
    rows = np.unique(np.concatenate([[0, 1, 2, N - 3, N - 2, N - 1], rng.choice(N, 10, replace=False)]))
    for M in Ms:
        x = rng.standard_normal((M, K)).astype(np.float32)
        a_q8, qs, d = quantize(kq, fmt, x)
        variant = kq.kq_variant_name(kq.kq_select_variant(fmt, M, N, K))
        say(f"  M={M} {variant}")
        out = torch.full((M, N), float("nan"), dtype=torch.float32, device=DEV)
        kq.kq_gemm(fmt, Wd, a_q8, M, N, K, out)
        torch.cuda.synchronize()
        got = out[:, torch.from_numpy(rows).to(DEV)].cpu().numpy()
        ref, tol = kqref.gemm(fmt, W, qs, d, K, rows=rows)
        check_columns(got, ref, tol, f"{variant} N={N}")
        del out


@pytest.mark.parametrize("fmt", (Q4_K, Q6_K, TQ, TQ2), ids=["q4_k", "q6_k", "tq", "tq2"])
def test_output_just_below_2gib(kq, fmt):
    M, K = 4096, 256
    N = LIMIT // (4 * (M + 128))          # largest N with (M + 128) * N * 4 < 2^31
    if (M + 128) * N * 4 >= LIMIT:
        N -= 1
    assert (M + 128) * N * 4 < LIMIT
    say(f"output near 2 GiB: fmt={fmt} M={M} N={N} K={K} ({M * N * 4 / 2**30:.3f} GiB)")
    rowbytes = (K // QK[fmt]) * BB[fmt]
    W = random_blocks(fmt, N * (K // QK[fmt]), 700 + fmt).reshape(N, rowbytes)
    rng = np.random.default_rng(800 + fmt)
    x = rng.standard_normal((M, K)).astype(np.float32)
    a_q8, qs, d = quantize(kq, fmt, x)
    variant = kq.kq_variant_name(kq.kq_select_variant(fmt, M, N, K))
    say(f"  {variant}")
    out = torch.full((M, N), float("nan"), dtype=torch.float32, device=DEV)
    kq.kq_gemm(fmt, torch.from_numpy(W).to(DEV), a_q8, M, N, K, out)
    torch.cuda.synchronize()
    rows = np.unique(np.concatenate([[0, 1, N - 2, N - 1], rng.choice(N, 8, replace=False)]))
    got = out[:, torch.from_numpy(rows).to(DEV)].cpu().numpy()
    ref, tol = kqref.gemm(fmt, W, qs, d, K, rows=rows)
    check_columns(got, ref, tol, f"{variant} M={M} N={N}")
    # the last output row, every column: the end of the buffer
    last = out[M - 1].cpu().numpy()
    assert np.all(np.isfinite(last))


def test_gemm_id_experts_beyond_2gib(kq):
    """Four Q4_K experts of about 0.9 GiB each: the last ones start past 2^31
    bytes into W (the per-expert base is 64-bit; each expert's own offsets stay
    32-bit).  A few routed rows per expert, sampled weight rows checked."""
    fmt, E, K = Q4_K, 4, 4096
    rowbytes = (K // 256) * 144
    N = 400_000
    assert E * N * rowbytes > LIMIT and (N + 256) * rowbytes < LIMIT
    say(f"gemm_id: {E} experts x {N * rowbytes / 2**30:.2f} GiB")
    W = random_blocks(fmt, E * N * (K // 256), 900).reshape(E * N, rowbytes)
    rng = np.random.default_rng(901)
    M = 12
    x = rng.standard_normal((M, K)).astype(np.float32)
    a_q8, qs, d = quantize(kq, fmt, x)
    counts = [3, 5, 4, 6]
    off = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    rows = rng.integers(0, M, size=int(off[-1])).astype(np.int32)
    R = int(off[-1])
    out = torch.full((R, N), float("nan"), dtype=torch.float32, device=DEV)
    kq.kq_gemm_id(fmt, torch.from_numpy(W).to(DEV), E, a_q8, M, N, K,
                  torch.from_numpy(off).to(DEV), torch.from_numpy(rows).to(DEV), R, out)
    torch.cuda.synchronize()
    cols = np.unique(np.concatenate([[0, N - 1], rng.choice(N, 6, replace=False)]))
    got = out[:, torch.from_numpy(cols).to(DEV)].cpu().numpy()
    for e in range(E):
        r0, r1 = int(off[e]), int(off[e + 1])
        toks = rows[r0:r1]
        ref, tol = kqref.gemm(fmt, W[e * N:(e + 1) * N], np.ascontiguousarray(qs[toks]),
                              np.ascontiguousarray(d[toks]), K, rows=cols)
        check_columns(got[r0:r1], ref, tol, f"gemm_id expert {e}")
