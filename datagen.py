"""Seeded synthetic inputs for the block-quantized GEMM path.

This module is input preparation only. It draws fp32 weights and activations
with numpy's PCG64 generator and encodes the weights into the stored block
formats (Q4_K, Q6_K, ternary).  It holds none of the path's arithmetic: it does
not quantize activations, does not decode blocks and does not multiply.  Both
the HIP path and the CPU oracle consume the arrays it returns; neither is
imported here.

Block layouts (our own definitions; the pages fix only the block sizes):

* Q4_K, 144 bytes per 256 weights: fp16 d, fp16 dmin, 12 bytes holding sixteen
  6-bit fields as one little-endian 96-bit integer (field j < 8 is the scale of
  32-wide sub-block j, field 8+j its min), then 128 nibble bytes.  Byte 32c+t
  carries weight 64c+t in its low nibble and weight 64c+32+t in its high one.
  Dequantized weight: d*sc_j*q - dmin*m_j.
* Q6_K, 210 bytes per 256 weights: 128 bytes of low nibbles, 64 bytes of high
  bit pairs, 16 signed 8-bit scales (one per 16 weights), fp16 d.
  Dequantized weight: d*sc_j*(q-32).
* Ternary, 28 bytes per 128 weights: 26 bytes with five base-3 digits each
  (digit = trit+1, least significant first; the two spare digits of byte 25
  are 1), then fp16 d.  Dequantized weight: d*t.

Workloads (token count M, output rows N, reduction K) follow the five
configurations of the vllm.cpp / llama.cpp prefill shapes: a tiny Q4_K case,
a 4096x4096 Q4_K projection at 512 tokens, the 4096->14336 FFN gate/up at
2048 and 64 tokens, the 14336->4096 Q6_K FFN down at 2048 tokens and a
5120->17408 ternary projection at 2048 tokens.
"""
from __future__ import annotations

import dataclasses

import numpy as np

Q4_K, Q6_K, TQ, TQ2 = 1, 2, 3, 4
FMT_NAMES = {Q4_K: "q4_k", Q6_K: "q6_k", TQ: "tq", TQ2: "tq2"}
QK = {Q4_K: 256, Q6_K: 256, TQ: 128, TQ2: 128}             # weights per block
BLOCK_BYTES = {Q4_K: 144, Q6_K: 210, TQ: 28, TQ2: 34}      # bytes per block


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    fmt: int
    M: int
    N: int
    K: int
    seed: int
    dist: str          # "plain" or "outlier_lognormal"
    note: str
    experts: int = 0   # > 0: an expert-indexed product over this many experts
    topk: int = 0      # experts per token


WORKLOADS = {
    "tiny_q4k": Workload("tiny_q4k", Q4_K, 8, 256, 512, 1001, "plain",
                         "Q4_K x Q8_K, 8 tokens, 256 rows, K=512"),
    "proj_q4k_4096": Workload("proj_q4k_4096", Q4_K, 512, 4096, 4096, 1002,
                              "outlier_lognormal",
                              "Q4_K x Q8_K projection, 512 tokens, 4096x4096, "
                              "1% weight outliers x10, LogNormal channel scales"),
    "ffn_up_q4k_2048": Workload("ffn_up_q4k_2048", Q4_K, 2048, 14336, 4096, 1003,
                                "plain", "Q4_K x Q8_K FFN gate/up, 2048 tokens"),
    "ffn_up_q4k_64": Workload("ffn_up_q4k_64", Q4_K, 64, 14336, 4096, 1003,
                              "plain", "Q4_K x Q8_K FFN gate/up, 64 tokens "
                              "(first 64 token rows of the 2048-token draw)"),
    "ffn_up_q4k_1": Workload("ffn_up_q4k_1", Q4_K, 1, 14336, 4096, 1003,
                             "plain", "Q4_K x Q8_K FFN gate/up, one token (decode; "
                             "first token row of the 2048-token draw)"),
    "ffn_down_q6k_2048": Workload("ffn_down_q6k_2048", Q6_K, 2048, 4096, 14336, 1004,
                                  "plain", "Q6_K x Q8_K FFN down, 2048 tokens"),
    "tern_5120_2048": Workload("tern_5120_2048", TQ, 2048, 17408, 5120, 1005,
                               "plain", "ternary x Q8_128, 2048 tokens, 17408x5120"),
    "ffn_down_q6k_1": Workload("ffn_down_q6k_1", Q6_K, 1, 4096, 14336, 1004,
                               "plain", "Q6_K x Q8_K FFN down, one token (decode; first "
                               "token row of the 2048-token draw)"),
    "ffn_down_q6k_16": Workload("ffn_down_q6k_16", Q6_K, 16, 4096, 14336, 1004,
                                "plain", "Q6_K x Q8_K FFN down, 16 tokens (a small decode batch; "
                                "first 16 token rows of the 2048-token draw)"),
    "ffn_down_q6k_512": Workload("ffn_down_q6k_512", Q6_K, 512, 4096, 14336, 1004,
                                 "plain", "Q6_K x Q8_K FFN down, 512 tokens (a prefill chunk; "
                                 "first 512 token rows of the 2048-token draw)"),
    "tern_5120_1": Workload("tern_5120_1", TQ, 1, 17408, 5120, 1005,
                            "plain", "ternary x Q8_128, one token (decode; first token row "
                            "of the 2048-token draw), 17408x5120"),
    "moe_q4k_8x2_512": Workload("moe_q4k_8x2_512", Q4_K, 512, 14336, 4096, 1006, "plain",
                                "Q4_K x Q8_K expert-indexed FFN gate/up: 8 experts of 14336x4096, "
                                "512 tokens routed to 2 experts each (1024 routed rows)",
                                experts=8, topk=2),
    "tern2_5120_2048": Workload("tern2_5120_2048", TQ2, 2048, 17408, 5120, 1005,
                                "plain", "ternary at two bits per weight x Q8_128, 2048 "
                                "tokens, 17408x5120 (the same trits as tern_5120_2048)"),
}


def _streams(seed: int):
    """Three independent PCG64 streams: weights, activations, extra."""
    ss = np.random.SeedSequence(seed)
    return [np.random.Generator(np.random.PCG64(s)) for s in ss.spawn(3)]


# ----------------------------------------------------------------------------
# fp32 draws
# ----------------------------------------------------------------------------

def draw_weights(N: int, K: int, seed: int, dist: str = "plain") -> np.ndarray:
    """fp32 [N][K] weights ~ N(0, 0.02); with dist='outlier_lognormal' an
    independent Bernoulli(0.01) mask multiplies 1% of them by 10."""
    gw, _, gx = _streams(seed)
    w = gw.normal(0.0, 0.02, size=(N, K))
    if dist == "outlier_lognormal":
        mask = gx.random(size=(N, K)) < 0.01
        w = np.where(mask, w * 10.0, w)
    return w.astype(np.float32)


def draw_activations(M: int, K: int, seed: int, dist: str = "plain",
                     rows: int | None = None) -> np.ndarray:
    """fp32 [M][K] activations ~ N(0, 1); with dist='outlier_lognormal' each
    K-channel k is scaled by c_k ~ LogNormal(0, 0.5).  `rows` draws that many
    rows and returns the first M (so a 64-token case is a prefix of the
    2048-token one)."""
    _, ga, _ = _streams(seed)
    total = rows if rows is not None else M
    z = ga.normal(0.0, 1.0, size=(total, K))
    if dist == "outlier_lognormal":
        c = ga.lognormal(0.0, 0.5, size=(K,))
        z = z * c[None, :]
    return np.ascontiguousarray(z[:M].astype(np.float32))


def draw_ternary(N: int, K: int, seed: int):
    """Ternary weights t in {-1,0,1} with p=(0.3,0.4,0.3) and per-128-block
    fp16 scales d ~ U(0.01, 0.05).  Returns (t int8 [N][K], d fp16 [N][K/128])."""
    gw, _, gx = _streams(seed)
    u = gw.random(size=(N, K))
    t = np.where(u < 0.3, -1, np.where(u < 0.7, 0, 1)).astype(np.int8)
    d = gx.uniform(0.01, 0.05, size=(N, K // 128)).astype(np.float16)
    return t, d


# ----------------------------------------------------------------------------
# Field packers: integer fields -> block bytes
# ----------------------------------------------------------------------------

def pack_q4k(d: np.ndarray, dmin: np.ndarray, sc: np.ndarray, mn: np.ndarray,
             q: np.ndarray) -> np.ndarray:
    """Pack Q4_K fields for B blocks into uint8 [B][144].

    d, dmin: fp16 [B]; sc, mn: ints [B][8] in [0,63]; q: ints [B][256] in [0,15].
    """
    B = d.shape[0]
    out = np.zeros((B, 144), dtype=np.uint8)
    out[:, 0:2] = np.asarray(d, dtype=np.float16).reshape(B, 1).view(np.uint8)
    out[:, 2:4] = np.asarray(dmin, dtype=np.float16).reshape(B, 1).view(np.uint8)
    fields = np.concatenate([np.asarray(sc), np.asarray(mn)], axis=1).astype(np.int64)
    assert fields.min(initial=0) >= 0 and fields.max(initial=0) <= 63
    bits = ((fields[:, :, None] >> np.arange(6)[None, None, :]) & 1).reshape(B, 96)
    out[:, 4:16] = np.packbits(bits.astype(np.uint8), axis=1, bitorder="little")
    q = np.asarray(q).astype(np.uint8).reshape(B, 4, 2, 32)
    assert q.max(initial=0) <= 15
    out[:, 16:144] = (q[:, :, 0, :] | (q[:, :, 1, :] << 4)).reshape(B, 128)
    return out


def pack_q6k(d: np.ndarray, sc: np.ndarray, q: np.ndarray) -> np.ndarray:
    """Pack Q6_K fields for B blocks into uint8 [B][210].

    d: fp16 [B]; sc: ints [B][16] in [-128,127]; q: ints [B][256] in [0,63].
    """
    B = d.shape[0]
    out = np.zeros((B, 210), dtype=np.uint8)
    q = np.asarray(q).astype(np.uint8).reshape(B, 2, 128)
    assert q.max(initial=0) <= 63
    lo = q & 15
    hi = q >> 4
    ql = lo[:, :, 0:64] | (lo[:, :, 64:128] << 4)                  # [B][2][64]
    h4 = hi.reshape(B, 2, 4, 32)                                    # [B][half][u][t]
    qh = (h4[:, :, 0] | (h4[:, :, 1] << 2) | (h4[:, :, 2] << 4) | (h4[:, :, 3] << 6))
    out[:, 0:128] = ql.reshape(B, 128)
    out[:, 128:192] = qh.reshape(B, 64)
    sc = np.asarray(sc).astype(np.int64)
    assert sc.min(initial=0) >= -128 and sc.max(initial=0) <= 127
    out[:, 192:208] = sc.astype(np.int8).view(np.uint8)
    out[:, 208:210] = np.asarray(d, dtype=np.float16).reshape(B, 1).view(np.uint8)
    return out


_POW3 = np.array([1, 3, 9, 27, 81], dtype=np.int64)


def pack_tq(t: np.ndarray, d: np.ndarray) -> np.ndarray:
    """Pack ternary blocks: t int [B][128] in {-1,0,1}, d fp16 [B] -> uint8 [B][28]."""
    t = np.asarray(t).astype(np.int64)
    B = t.shape[0]
    assert t.shape[1] == 128 and t.min(initial=0) >= -1 and t.max(initial=0) <= 1
    e = np.ones((B, 130), dtype=np.int64)          # two spare digits hold 1
    e[:, :128] = t + 1
    out = np.zeros((B, 28), dtype=np.uint8)
    out[:, 0:26] = (e.reshape(B, 26, 5) * _POW3).sum(axis=2).astype(np.uint8)
    out[:, 26:28] = np.asarray(d, dtype=np.float16).reshape(B, 1).view(np.uint8)
    return out


def pack_tq2(t: np.ndarray, d: np.ndarray) -> np.ndarray:
    """Pack ternary blocks at two bits per weight: t int [B][128] in {-1,0,1},
    d fp16 [B] -> uint8 [B][34]; byte j holds the codes t+1 of weights j,
    j+32, j+64, j+96 from its low bits up."""
    t = np.asarray(t).astype(np.int64)
    B = t.shape[0]
    assert t.shape[1] == 128 and t.min(initial=0) >= -1 and t.max(initial=0) <= 1
    c = (t + 1).reshape(B, 4, 32)
    out = np.zeros((B, 34), dtype=np.uint8)
    out[:, 0:32] = (c[:, 0] | (c[:, 1] << 2) | (c[:, 2] << 4) | (c[:, 3] << 6)).astype(np.uint8)
    out[:, 32:34] = np.asarray(d, dtype=np.float16).reshape(B, 1).view(np.uint8)
    return out


# ----------------------------------------------------------------------------
# Weight encoders: fp32 weights -> block bytes (fp64 arithmetic)
# ----------------------------------------------------------------------------

def _rne(x):
    return np.rint(x)     # numpy rounds half to even


def encode_q4k(w: np.ndarray) -> np.ndarray:
    """Per-sub-block min/max Q4_K encoder.  w fp32 [N][K] -> uint8 [N][K/256*144].

    For each 32-wide sub-block j: lo = min(0, min w), hi = max w,
    s_j = (hi-lo)/15, mn_j = -lo; d = fp16(max_j s_j/63), dmin = fp16(max_j mn_j/63);
    sc_j = rne(s_j/d), m_j = rne(mn_j/dmin) clamped to [0,63];
    q = rne((w + dmin*m_j)/(d*sc_j)) clamped to [0,15].
    """
    N, K = w.shape
    assert K % 256 == 0
    x = w.astype(np.float64).reshape(N, K // 256, 8, 32)
    lo = np.minimum(0.0, x.min(axis=3))
    hi = x.max(axis=3)
    s = (hi - lo) / 15.0
    mn = -lo
    d = (s.max(axis=2) / 63.0).astype(np.float16)
    dmin = (mn.max(axis=2) / 63.0).astype(np.float16)
    d64 = d.astype(np.float64)[..., None]
    dm64 = dmin.astype(np.float64)[..., None]
    with np.errstate(divide="ignore", invalid="ignore"):
        sc = np.where(d64 > 0, np.clip(_rne(s / d64), 0, 63), 0).astype(np.int64)
        m = np.where(dm64 > 0, np.clip(_rne(mn / dm64), 0, 63), 0).astype(np.int64)
        step = (d64 * sc)[..., None]
        q = np.where(step > 0,
                     np.clip(_rne((x + (dm64 * m)[..., None]) / step), 0, 15), 0)
    B = N * (K // 256)
    blocks = pack_q4k(d.reshape(B), dmin.reshape(B), sc.reshape(B, 8),
                      m.reshape(B, 8), q.astype(np.int64).reshape(B, 256))
    return blocks.reshape(N, (K // 256) * 144)


def encode_q6k(w: np.ndarray) -> np.ndarray:
    """Symmetric Q6_K encoder.  w fp32 [N][K] -> uint8 [N][K/256*210].

    For each 16-wide sub-block j: s_j = max|w|/31; d = fp16(max_j s_j/127);
    sc_j = rne(s_j/d) clamped to [0,127]; q = rne(w/(d*sc_j)) clamped to
    [-32,31], stored +32.
    """
    N, K = w.shape
    assert K % 256 == 0
    x = w.astype(np.float64).reshape(N, K // 256, 16, 16)
    s = np.abs(x).max(axis=3) / 31.0
    d = (s.max(axis=2) / 127.0).astype(np.float16)
    d64 = d.astype(np.float64)[..., None]
    with np.errstate(divide="ignore", invalid="ignore"):
        sc = np.where(d64 > 0, np.clip(_rne(s / d64), 0, 127), 0).astype(np.int64)
        step = (d64 * sc)[..., None]
        q = np.where(step > 0, np.clip(_rne(x / step), -32, 31), 0) + 32
    B = N * (K // 256)
    blocks = pack_q6k(d.reshape(B), sc.reshape(B, 16), q.astype(np.int64).reshape(B, 256))
    return blocks.reshape(N, (K // 256) * 210)


def encode_tq(t: np.ndarray, d: np.ndarray) -> np.ndarray:
    """Ternary encoder. t int8 [N][K], d fp16 [N][K/128] -> uint8 [N][K/128*28]."""
    N, K = t.shape
    assert K % 128 == 0
    B = N * (K // 128)
    return pack_tq(t.reshape(B, 128), d.reshape(B)).reshape(N, (K // 128) * 28)


def encode_tq2(t: np.ndarray, d: np.ndarray) -> np.ndarray:
    """Two-bit ternary encoder. t int8 [N][K], d fp16 [N][K/128] -> uint8 [N][K/128*34]."""
    N, K = t.shape
    assert K % 128 == 0
    B = N * (K // 128)
    return pack_tq2(t.reshape(B, 128), d.reshape(B)).reshape(N, (K // 128) * 34)


# ----------------------------------------------------------------------------
# Whole workloads
# ----------------------------------------------------------------------------

def draw_routing(M: int, experts: int, topk: int, seed: int):
    """Synthetic top-k routing: each token picks topk distinct experts
    uniformly.  Returns int32 expert offsets [experts + 1] and the token of
    each routed row [M * topk], grouped by expert (tokens ascending within an
    expert)."""
    _, _, gx = _streams(seed)
    choice = np.argsort(gx.random((M, experts)), axis=1)[:, :topk]     # [M][topk]
    tok = np.repeat(np.arange(M), topk)
    exp = choice.reshape(-1)
    order = np.lexsort((tok, exp))
    counts = np.bincount(exp, minlength=experts)
    off = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    return off, tok[order].astype(np.int32)


def make_weights(fmt: int, N: int, K: int, seed: int, dist: str = "plain") -> np.ndarray:
    """Stored weight blocks uint8 [N][K/QK*block_bytes] for a seeded draw."""
    if fmt == Q4_K:
        return encode_q4k(draw_weights(N, K, seed, dist))
    if fmt == Q6_K:
        return encode_q6k(draw_weights(N, K, seed, dist))
    if fmt == TQ:
        t, d = draw_ternary(N, K, seed)
        return encode_tq(t, d)
    if fmt == TQ2:
        t, d = draw_ternary(N, K, seed)
        return encode_tq2(t, d)
    raise ValueError(f"unknown format {fmt}")


# token-prefix workloads: their activations are the first rows of the 2048-token draw
_PREFIX_OF_2048 = ("ffn_up_q4k_2048", "ffn_up_q4k_64", "ffn_up_q4k_1", "ffn_down_q6k_1", "ffn_down_q6k_16",
                   "ffn_down_q6k_512", "tern_5120_1")


def make_workload(wl: Workload | str, n_rows: int | None = None, m_rows: int | None = None):
    """(W blocks, x fp32) for a named workload.  n_rows / m_rows take a prefix
    of the output rows / tokens (the draws are made at full size, so a prefix
    equals the same rows of the full problem)."""
    if isinstance(wl, str):
        wl = WORKLOADS[wl]
    # an expert-indexed workload: experts x N consecutive weight rows
    W = make_weights(wl.fmt, wl.N * max(wl.experts, 1), wl.K, wl.seed, wl.dist)
    full_rows = 2048 if wl.name in _PREFIX_OF_2048 else wl.M
    x = draw_activations(wl.M, wl.K, wl.seed, wl.dist, rows=full_rows)
    if n_rows is not None:
        W = np.ascontiguousarray(W[:n_rows])
    if m_rows is not None:
        x = np.ascontiguousarray(x[:m_rows])
    return W, x


def random_fields_q4k(rng: np.random.Generator, B: int):
    """Uniformly random Q4_K fields for fuzzing: finite fp16 d/dmin, 6-bit
    scales and mins, 4-bit quants."""
    d = rng.uniform(-2.0, 2.0, size=B).astype(np.float16)
    dmin = rng.uniform(-2.0, 2.0, size=B).astype(np.float16)
    sc = rng.integers(0, 64, size=(B, 8))
    mn = rng.integers(0, 64, size=(B, 8))
    q = rng.integers(0, 16, size=(B, 256))
    return d, dmin, sc, mn, q


def random_fields_q6k(rng: np.random.Generator, B: int):
    d = rng.uniform(-2.0, 2.0, size=B).astype(np.float16)
    sc = rng.integers(-128, 128, size=(B, 16))
    q = rng.integers(0, 64, size=(B, 256))
    return d, sc, q


def random_fields_tq(rng: np.random.Generator, B: int):
    d = rng.uniform(-2.0, 2.0, size=B).astype(np.float16)
    t = rng.integers(-1, 2, size=(B, 128))
    return d, t


def random_fields_tq2(rng: np.random.Generator, B: int):
    d = rng.uniform(-2.0, 2.0, size=B).astype(np.float16)
    t = rng.integers(-1, 2, size=(B, 128))
    return d, t
