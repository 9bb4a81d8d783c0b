"""Checks that pin the CPU oracle to facts that do not come from the oracle.

Each check_* function raises AssertionError on a mismatch.  They are run by
test_oracle_pins.py against the oracle as built, and against copies of the
oracle with planted mistakes (each mutant must fail at least one check).

What pins what:
* fp16 -> fp64 conversion: numpy's float16, exhaustively.
* Block decoders: hand-built blocks whose dequantized values follow a closed
  form, packed here with Python integers (not with datagen, not with the
  oracle); every 6-bit field position and every nibble / bit-pair position;
  every valid base-3 byte against numpy.base_repr.
* Q8 activation rule: printed tie cases, exact power-of-two scaling, sign
  symmetry, the half-step error bound and the zero / non-finite-scale rule.
* The product: exact rational arithmetic (fractions) on tiny shapes, via the
  factored form d*sum_j sc_j S_j - dmin*sum_j m_j B_j, which is algebra the
  oracle never uses; unit-scale blocks reduce to numpy's integer matmul;
  one-hot scales expose single sub-block sums; x=0, x->-x and joint
  superblock permutations.
* Tolerance bound: exact rational sum of |W^ A^|.
* Encoder / decoder round trip: the datagen encoders against the oracle
  decoders with the half-step error bounds of each format.
"""
from __future__ import annotations

from fractions import Fraction

import numpy as np

import datagen
from oracle import kqref

Q4_K, Q6_K, TQ, TQ2 = kqref.Q4_K, kqref.Q6_K, kqref.TQ, kqref.TQ2
ACT_Q8_K, ACT_Q8_128 = kqref.ACT_Q8_K, kqref.ACT_Q8_128


# ---------------------------------------------------------------------------
# Independent block packers (Python integers, written from the layout text)
# ---------------------------------------------------------------------------

def f16_bits(v: float) -> int:
    return int(np.array([v], dtype=np.float16).view(np.uint16)[0])


def q4k_by_hand(d_bits: int, dmin_bits: int, sc, mn, q) -> np.ndarray:
    S = 0
    for j in range(8):
        S |= int(sc[j]) << (6 * j)
        S |= int(mn[j]) << (48 + 6 * j)
    b = bytearray(144)
    b[0:2] = d_bits.to_bytes(2, "little")
    b[2:4] = dmin_bits.to_bytes(2, "little")
    b[4:16] = S.to_bytes(12, "little")
    for c in range(4):
        for t in range(32):
            b[16 + 32 * c + t] = int(q[64 * c + t]) | (int(q[64 * c + 32 + t]) << 4)
    return np.frombuffer(bytes(b), dtype=np.uint8).copy()


def q6k_by_hand(d_bits: int, sc, q) -> np.ndarray:
    b = bytearray(210)
    for h in range(2):
        for t in range(64):
            b[64 * h + t] = (int(q[128 * h + t]) & 15) | ((int(q[128 * h + 64 + t]) & 15) << 4)
        for t in range(32):
            v = 0
            for u in range(4):
                v |= (int(q[128 * h + 32 * u + t]) >> 4) << (2 * u)
            b[128 + 32 * h + t] = v
    for j in range(16):
        b[192 + j] = int(sc[j]) & 0xFF
    b[208:210] = d_bits.to_bytes(2, "little")
    return np.frombuffer(bytes(b), dtype=np.uint8).copy()


def tq_by_hand(d_bits: int, t) -> np.ndarray:
    e = [int(v) + 1 for v in t] + [1, 1]
    b = bytearray(28)
    for i in range(26):
        b[i] = sum(e[5 * i + p] * 3 ** p for p in range(5))
    b[26:28] = d_bits.to_bytes(2, "little")
    return np.frombuffer(bytes(b), dtype=np.uint8).copy()


def tq2_by_hand(d_bits: int, t) -> np.ndarray:
    # byte j: codes t+1 of weights j, j+32, j+64, j+96, from the low bits up
    b = bytearray(34)
    for j in range(32):
        b[j] = sum((int(t[j + 32 * p]) + 1) << (2 * p) for p in range(4))
    b[32:34] = d_bits.to_bytes(2, "little")
    return np.frombuffer(bytes(b), dtype=np.uint8).copy()


# ---------------------------------------------------------------------------
# fp16
# ---------------------------------------------------------------------------

def check_f16_exhaustive():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    want = bits.view(np.float16).astype(np.float64)
    got = np.array([kqref.f16_to_f64(int(b)) for b in bits])
    fin = np.isfinite(want)
    assert np.array_equal(got[fin], want[fin])
    assert np.array_equal(np.isnan(got), np.isnan(want))
    assert np.array_equal(np.isinf(got), np.isinf(want))


# ---------------------------------------------------------------------------
# Q4_K decoder
# ---------------------------------------------------------------------------

def check_q4k_closed_form():
    # d = 1, dmin = 0.5, sc_j = j+1, m_j = 2j, q_k = k mod 16
    # => W^_k = (j+1)(k mod 16) - j.
    sc = [j + 1 for j in range(8)]
    mn = [2 * j for j in range(8)]
    q = [k % 16 for k in range(256)]
    blk = q4k_by_hand(f16_bits(1.0), f16_bits(0.5), sc, mn, q)
    w = kqref.dequant_rows(Q4_K, blk[None], 256)[0]
    want = np.array([(k // 32 + 1) * (k % 16) - (k // 32) for k in range(256)], np.float64)
    assert np.array_equal(w, want)
    d, dmin, dsc, dmn, dq = kqref.decode_q4k(blk)
    assert (d, dmin) == (1.0, 0.5)
    assert list(dsc) == sc and list(dmn) == mn and list(dq) == q


def check_q4k_field_positions():
    zero_q = [0] * 256
    for f in range(16):
        sc = [0] * 8
        mn = [0] * 8
        (sc if f < 8 else mn)[f % 8] = 63
        blk = q4k_by_hand(0, 0, sc, mn, zero_q)
        _, _, dsc, dmn, _ = kqref.decode_q4k(blk)
        assert list(dsc) == sc and list(dmn) == mn, f
    # every single bit of the 96-bit field word
    for bit in range(96):
        S = 1 << bit
        b = bytearray(144)
        b[4:16] = S.to_bytes(12, "little")
        _, _, dsc, dmn, _ = kqref.decode_q4k(np.frombuffer(bytes(b), np.uint8))
        fields = list(dsc) + list(dmn)
        want = [0] * 16
        want[bit // 6] = 1 << (bit % 6)
        assert fields == want, bit


def check_q4k_nibble_positions():
    for k in range(256):
        q = [0] * 256
        q[k] = 9
        blk = q4k_by_hand(f16_bits(1.0), 0, [1] * 8, [0] * 8, q)
        w = kqref.dequant_rows(Q4_K, blk[None], 256)[0]
        want = np.zeros(256)
        want[k] = 9.0
        assert np.array_equal(w, want), k


# ---------------------------------------------------------------------------
# Q6_K decoder
# ---------------------------------------------------------------------------

def check_q6k_closed_form():
    # d = 0.25, sc_j = (-1)^j (j+1), q_k = k mod 64  => W^_k = 0.25 sc_j (k mod 64 - 32)
    sc = [(-1) ** j * (j + 1) for j in range(16)]
    q = [k % 64 for k in range(256)]
    blk = q6k_by_hand(f16_bits(0.25), sc, q)
    w = kqref.dequant_rows(Q6_K, blk[None], 256)[0]
    want = np.array([0.25 * sc[k // 16] * (k % 64 - 32) for k in range(256)])
    assert np.array_equal(w, want)
    # extreme scales
    sc2 = [-128, 127] * 8
    q2 = [0 if (k // 7) % 2 else 63 for k in range(256)]
    blk2 = q6k_by_hand(f16_bits(1.0), sc2, q2)
    w2 = kqref.dequant_rows(Q6_K, blk2[None], 256)[0]
    want2 = np.array([sc2[k // 16] * (q2[k] - 32) for k in range(256)], np.float64)
    assert np.array_equal(w2, want2)


def check_q6k_positions():
    # every position with every 6-bit value class: put value v at position k
    for k in range(256):
        for v in (1, 16, 33, 63):
            q = [32] * 256
            q[k] = v
            blk = q6k_by_hand(f16_bits(1.0), [1] * 16, q)
            w = kqref.dequant_rows(Q6_K, blk[None], 256)[0]
            want = np.zeros(256)
            want[k] = v - 32
            assert np.array_equal(w, want), (k, v)


# ---------------------------------------------------------------------------
# Ternary decoder
# ---------------------------------------------------------------------------

def check_tq_bytes():
    def trits_of_byte(v):
        blk = np.zeros(28, np.uint8)
        blk[0] = v
        blk[26:28] = np.array([f16_bits(1.0)], np.uint16).view(np.uint8)
        _, t = kqref.decode_tq(blk)
        return list(t[:5])

    assert trits_of_byte(0) == [-1] * 5
    assert trits_of_byte(121) == [0] * 5
    assert trits_of_byte(242) == [1] * 5
    assert trits_of_byte(5) == [1, 0, -1, -1, -1]
    for v in range(243):
        digits = [int(c) for c in np.base_repr(v, 3).zfill(5)[::-1]]
        assert trits_of_byte(v) == [dg - 1 for dg in digits], v


def check_tq_block():
    rng = np.random.default_rng(7)
    for _ in range(50):
        t = rng.integers(-1, 2, size=128)
        dval = float(rng.uniform(0.01, 0.05))
        blk = tq_by_hand(f16_bits(dval), t)
        d, dt = kqref.decode_tq(blk)
        assert d == float(np.float16(dval))
        assert np.array_equal(dt, t)
        w = kqref.dequant_rows(TQ, blk[None], 128)[0]
        assert np.array_equal(w, d * t.astype(np.float64))


def check_tq2_codes():
    # every code at every position, the other weights at code 1 (zero)
    one = f16_bits(1.0)
    for k in range(128):
        for c in range(3):
            t = [0] * 128
            t[k] = c - 1
            blk = tq2_by_hand(one, t)
            assert (int(blk[k % 32]) >> (2 * (k // 32))) & 3 == c
            d, dt = kqref.decode_tq2(blk)
            assert d == 1.0
            assert list(dt) == t, (k, c)


def check_tq2_block():
    rng = np.random.default_rng(8)
    for _ in range(50):
        t = rng.integers(-1, 2, size=128)
        dval = float(rng.uniform(-0.05, 0.05))
        blk = tq2_by_hand(f16_bits(dval), t)
        d, dt = kqref.decode_tq2(blk)
        assert d == float(np.float16(dval))
        assert np.array_equal(dt, t)
        w = kqref.dequant_rows(TQ2, blk[None], 128)[0]
        assert np.array_equal(w, d * t.astype(np.float64))


def check_tq2_same_trits_as_tq():
    # the two packings of the same trits and scales are the same weights:
    # dequantized values, products and integer sub-sums all agree exactly
    rng = np.random.default_rng(9)
    N, K, M = 5, 640, 4
    t = rng.integers(-1, 2, size=(N, K // 128, 128))
    d = rng.uniform(-0.1, 0.1, size=(N, K // 128))
    W3 = np.stack([np.concatenate([tq_by_hand(f16_bits(float(d[n, s])), t[n, s]) for s in range(K // 128)])
                   for n in range(N)])
    W4 = np.stack([np.concatenate([tq2_by_hand(f16_bits(float(d[n, s])), t[n, s]) for s in range(K // 128)])
                   for n in range(N)])
    assert W4.shape == (N, (K // 128) * 34)
    assert np.array_equal(kqref.dequant_rows(TQ, W3, K), kqref.dequant_rows(TQ2, W4, K))
    qs, d_a = _random_acts(rng, M, K, 128)
    o3, t3 = kqref.gemm(TQ, W3, qs, d_a, K)
    o4, t4 = kqref.gemm(TQ2, W4, qs, d_a, K)
    assert np.array_equal(o3, o4) and np.array_equal(t3, t4)
    assert np.array_equal(kqref.subsums(TQ, W3, qs, K), kqref.subsums(TQ2, W4, qs, K))


# ---------------------------------------------------------------------------
# Q8 activation rule
# ---------------------------------------------------------------------------

def check_q8_ties():
    # amax = 127 -> d = 1, s = 1, q = rint(x): half-way cases go to even.
    x = np.zeros((1, 256), np.float32)
    x[0, :8] = [127.0, 0.5, 1.5, 2.5, -2.5, 126.5, -0.5, 3.5]
    qs, d, bs = kqref.quantize_act(ACT_Q8_K, x)
    assert d[0, 0] == 1.0
    assert list(qs[0, :8]) == [127, 0, 2, 2, -2, 126, 0, 4]
    # amax = 254 -> d = 2, s = 0.5, q = rint(x/2)
    x2 = np.zeros((1, 256), np.float32)
    x2[0, :6] = [254.0, 1.0, 3.0, 5.0, -7.0, -254.0]
    qs2, d2, _ = kqref.quantize_act(ACT_Q8_K, x2)
    assert d2[0, 0] == 2.0
    assert list(qs2[0, :6]) == [127, 0, 2, 2, -4, -127]
    # the same rule per 128 for Q8_128
    qs3, d3, bs3 = kqref.quantize_act(ACT_Q8_128, x[:, :128].copy())
    assert bs3 is None and d3[0, 0] == 1.0 and list(qs3[0, :8]) == [127, 0, 2, 2, -2, 126, 0, 4]


def check_q8_zero_and_tiny():
    x = np.zeros((2, 512), np.float32)
    x[1, 256:] = np.float32(1e-45)          # subnormal amax: 127/amax overflows
    x[1, 0] = 3.0
    qs, d, bs = kqref.quantize_act(ACT_Q8_K, x)
    assert np.all(qs[0] == 0) and np.all(d[0] == 0) and np.all(bs[0] == 0)
    assert d[1, 1] == 0.0 and np.all(qs[1, 256:] == 0) and np.all(bs[1, 16:] == 0)
    assert d[1, 0] == np.float32(3.0) / np.float32(127.0) and qs[1, 0] == 127


def check_q8_properties():
    rng = np.random.default_rng(11)
    for act_fmt, bsz in ((ACT_Q8_K, 256), (ACT_Q8_128, 128)):
        x = (rng.standard_normal((16, 4 * bsz)) * rng.lognormal(0, 2, (16, 1))).astype(np.float32)
        qs, d, bs = kqref.quantize_act(act_fmt, x)
        xb = x.reshape(16, 4, bsz).astype(np.float64)
        qb = qs.reshape(16, 4, bsz).astype(np.float64)
        amax = np.abs(xb).max(axis=2)
        # d is the fp32 quotient amax/127
        assert np.array_equal(d, (amax.astype(np.float32) / np.float32(127.0)))
        # half-step bound
        err = np.abs(xb - d.astype(np.float64)[..., None] * qb)
        assert np.all(err <= 0.5 * d[..., None] + 2.0 ** -20 * amax[..., None])
        # the largest element maps to +-127
        assert np.all(np.abs(qb).max(axis=2) == 127)
        # sign symmetry
        qn, dn, bn = kqref.quantize_act(act_fmt, -x)
        assert np.array_equal(qn, -qs) and np.array_equal(dn, d)
        # exact power-of-two scaling
        for e in (-7, 5):
            qe, de, _ = kqref.quantize_act(act_fmt, (x * np.float32(2.0 ** e)).astype(np.float32))
            assert np.array_equal(qe, qs) and np.array_equal(de, d * np.float32(2.0 ** e))
        if bs is not None:
            assert np.array_equal(bs.astype(np.int64),
                                  qs.reshape(16, -1, 16).astype(np.int64).sum(axis=2))


# ---------------------------------------------------------------------------
# The product: exact rational brute force on tiny shapes
# ---------------------------------------------------------------------------

def _cr_f32(F: Fraction) -> np.float32:
    """Correctly rounded fp32 of an exact rational (ties to even)."""
    f = np.float32(float(F))
    cands = [np.nextafter(f, np.float32(-np.inf)), f, np.nextafter(f, np.float32(np.inf))]
    best = min(cands, key=lambda c: (abs(Fraction(float(c)) - F),
                                     int(np.array([c], np.float32).view(np.uint32)[0]) & 1))
    return np.float32(best)


def _random_acts(rng, M, K, bs):
    qs = rng.integers(-127, 128, size=(M, K)).astype(np.int8)
    d = rng.uniform(0.001, 0.1, size=(M, K // bs)).astype(np.float32)
    d[rng.random(d.shape) < 0.1] = 0.0
    return qs, d


def _fields_to_blocks(fmt, fields):
    """Pack fields for one row of blocks by hand."""
    if fmt == Q4_K:
        d, dmin, sc, mn, q = fields
        return np.concatenate([q4k_by_hand(f16_bits(float(d[b])), f16_bits(float(dmin[b])),
                                           sc[b], mn[b], q[b]) for b in range(len(d))])
    if fmt == Q6_K:
        d, sc, q = fields
        return np.concatenate([q6k_by_hand(f16_bits(float(d[b])), sc[b], q[b])
                               for b in range(len(d))])
    d, t = fields
    pack = tq2_by_hand if fmt == TQ2 else tq_by_hand
    return np.concatenate([pack(f16_bits(float(d[b])), t[b]) for b in range(len(d))])


def _exact_factored(fmt, fields_rows, qs, d_a):
    """Exact value of each output via the factored form, and exact sub-sums."""
    M, K = qs.shape
    N = len(fields_rows)
    Q = {Q4_K: 256, Q6_K: 256, TQ: 128, TQ2: 128}[fmt]
    sub = {Q4_K: 32, Q6_K: 16, TQ: 128, TQ2: 128}[fmt]
    exact = [[Fraction(0)] * N for _ in range(M)]
    mag = [[Fraction(0)] * N for _ in range(M)]
    S = np.zeros((M, N, K // sub), np.int64)
    for n, fields in enumerate(fields_rows):
        for s in range(K // Q):
            if fmt == Q4_K:
                d, dmin, sc, mn, q = (fields[0][s], fields[1][s], fields[2][s], fields[3][s],
                                      fields[4][s])
                qint = [int(v) for v in q]
            elif fmt == Q6_K:
                d, sc, q = fields[0][s], fields[1][s], fields[2][s]
                qint = [int(v) - 32 for v in q]
            else:
                d, t = fields[0][s], fields[1][s]
                qint = [int(v) for v in t]
            Fd = Fraction(float(d))
            for m in range(M):
                a = [int(v) for v in qs[m, s * Q:(s + 1) * Q]]
                Fda = Fraction(float(d_a[m, s]))
                Sj = [sum(qint[k] * a[k] for k in range(j * sub, (j + 1) * sub))
                      for j in range(Q // sub)]
                S[m, n, s * (Q // sub):(s + 1) * (Q // sub)] = Sj
                if fmt == Q4_K:
                    Bj = [sum(a[k] for k in range(32 * j, 32 * j + 32)) for j in range(8)]
                    val = Fd * sum(int(sc[j]) * Sj[j] for j in range(8)) - \
                        Fraction(float(dmin)) * sum(int(mn[j]) * Bj[j] for j in range(8))
                    wk = [Fd * int(sc[k // 32]) * qint[k] - Fraction(float(dmin)) * int(mn[k // 32])
                          for k in range(256)]
                elif fmt == Q6_K:
                    val = Fd * sum(int(sc[j]) * Sj[j] for j in range(16))
                    wk = [Fd * int(sc[k // 16]) * qint[k] for k in range(256)]
                else:
                    val = Fd * Sj[0]
                    wk = [Fd * qint[k] for k in range(128)]
                exact[m][n] += Fda * val
                mag[m][n] += sum(abs(wk[k] * Fda * a[k]) for k in range(Q))
    return exact, mag, S


def _tiny_case(fmt, rng, M, N, K):
    Q = {Q4_K: 256, Q6_K: 256, TQ: 128, TQ2: 128}[fmt]
    nb = K // Q
    rows = []
    for _ in range(N):
        if fmt == Q4_K:
            rows.append(datagen.random_fields_q4k(rng, nb))
        elif fmt == Q6_K:
            rows.append(datagen.random_fields_q6k(rng, nb))
        else:
            d, t = datagen.random_fields_tq(rng, nb)
            rows.append((d, t))
    W = np.stack([_fields_to_blocks(fmt, f) for f in rows])
    qs, d_a = _random_acts(rng, M, K, 128 if fmt in (TQ, TQ2) else 256)
    return rows, W, qs, d_a


def check_bruteforce_exact():
    rng = np.random.default_rng(2024)
    for fmt, Ks in ((Q4_K, (256, 512)), (Q6_K, (256, 512)), (TQ, (128, 384)), (TQ2, (128, 384))):
        for K in Ks:
            M, N = 3, 4
            rows, W, qs, d_a = _tiny_case(fmt, rng, M, N, K)
            exact, mag, S = _exact_factored(fmt, rows, qs, d_a)
            out, tol = kqref.gemm(fmt, W, qs, d_a, K)
            for m in range(M):
                for n in range(N):
                    cr = _cr_f32(exact[m][n])
                    if out[m, n] != cr:
                        ulp = abs(float(np.nextafter(cr, np.float32(np.inf))) - float(cr))
                        assert abs(Fraction(float(out[m, n])) - exact[m][n]) <= \
                            Fraction(ulp) + mag[m][n] * Fraction(1, 2 ** 40), (fmt, K, m, n)
                    want_tol = 1e-4 * float(mag[m][n]) + 1e-6
                    assert abs(tol[m, n] - want_tol) <= 1e-12 * want_tol, (fmt, K, m, n)
            got_S = kqref.subsums(fmt, W, qs, K)
            assert np.array_equal(got_S.astype(np.int64), S), (fmt, K)


def check_integer_special_case():
    # unit scales, no mins, unit activation scales: the product is numpy's integer matmul
    rng = np.random.default_rng(5)
    M, N, K = 5, 6, 512
    q = rng.integers(0, 16, size=(N, 2, 256))
    mn = rng.integers(0, 64, size=(N, 2, 8))
    W = np.stack([np.concatenate([q4k_by_hand(f16_bits(1.0), 0, [1] * 8, mn[n, s], q[n, s])
                                  for s in range(2)]) for n in range(N)])
    qs = rng.integers(-127, 128, size=(M, K)).astype(np.int8)
    ones = np.ones((M, K // 256), np.float32)
    out, _ = kqref.gemm(Q4_K, W, qs, ones, K)
    want = qs.astype(np.int64) @ q.reshape(N, K).astype(np.int64).T
    assert np.array_equal(out, want.astype(np.float32))
    # Q6_K: q - 32
    q6 = rng.integers(0, 64, size=(N, 2, 256))
    W6 = np.stack([np.concatenate([q6k_by_hand(f16_bits(1.0), [1] * 16, q6[n, s])
                                   for s in range(2)]) for n in range(N)])
    out6, _ = kqref.gemm(Q6_K, W6, qs, ones, K)
    want6 = qs.astype(np.int64) @ (q6.reshape(N, K).astype(np.int64) - 32).T
    assert np.array_equal(out6, want6.astype(np.float32))
    # ternary
    tt = rng.integers(-1, 2, size=(N, 4, 128))
    WT = np.stack([np.concatenate([tq_by_hand(f16_bits(1.0), tt[n, s]) for s in range(4)])
                   for n in range(N)])
    outT, _ = kqref.gemm(TQ, WT, qs, np.ones((M, K // 128), np.float32), K)
    wantT = qs.astype(np.int64) @ tt.reshape(N, K).astype(np.int64).T
    assert np.array_equal(outT, wantT.astype(np.float32))
    # ternary at two bits per weight
    W2 = np.stack([np.concatenate([tq2_by_hand(f16_bits(1.0), tt[n, s]) for s in range(4)])
                   for n in range(N)])
    out2, _ = kqref.gemm(TQ2, W2, qs, np.ones((M, K // 128), np.float32), K)
    assert np.array_equal(out2, wantT.astype(np.float32))


def check_onehot_scales():
    # sc = e_j: the product is the single sub-block sum S[:, :, j]
    rng = np.random.default_rng(9)
    M, N, K = 4, 3, 256
    qs = rng.integers(-127, 128, size=(M, K)).astype(np.int8)
    ones = np.ones((M, 1), np.float32)
    for fmt, nsub in ((Q4_K, 8), (Q6_K, 16)):
        for j in range(nsub):
            sc = [0] * nsub
            sc[j] = 1
            if fmt == Q4_K:
                q = rng.integers(0, 16, size=(N, 256))
                W = np.stack([q4k_by_hand(f16_bits(1.0), 0, sc, [0] * 8, q[n]) for n in range(N)])
                qint = q
                sub = 32
            else:
                q = rng.integers(0, 64, size=(N, 256))
                W = np.stack([q6k_by_hand(f16_bits(1.0), sc, q[n]) for n in range(N)])
                qint = q - 32
                sub = 16
            out, _ = kqref.gemm(fmt, W, qs, ones, K)
            Sj = qs[:, j * sub:(j + 1) * sub].astype(np.int64) @ \
                qint[:, j * sub:(j + 1) * sub].astype(np.int64).T
            assert np.array_equal(out, Sj.astype(np.float32)), (fmt, j)
            S = kqref.subsums(fmt, W, qs, K)
            assert np.array_equal(S[:, :, j].astype(np.int64), Sj), (fmt, j)


def check_invariants():
    rng = np.random.default_rng(13)
    M, N, K = 6, 5, 1024
    w = (rng.standard_normal((N, K)) * 0.02).astype(np.float32)
    W = datagen.encode_q4k(w)
    x = rng.standard_normal((M, K)).astype(np.float32)
    qs, d, _ = kqref.quantize_act(ACT_Q8_K, x)
    out, tol = kqref.gemm(Q4_K, W, qs, d, K)
    # x = 0 -> out = 0
    qz, dz, _ = kqref.quantize_act(ACT_Q8_K, np.zeros_like(x))
    oz, _ = kqref.gemm(Q4_K, W, qz, dz, K)
    assert np.all(oz == 0)
    # x -> -x -> out -> -out exactly
    qn, dn, _ = kqref.quantize_act(ACT_Q8_K, -x)
    on, _ = kqref.gemm(Q4_K, W, qn, dn, K)
    assert np.array_equal(on, -out)
    # joint permutation of superblocks along K
    perm = np.array([2, 0, 3, 1])
    Wp = W.reshape(N, 4, 144)[:, perm].reshape(N, -1)
    xp = x.reshape(M, 4, 256)[:, perm].reshape(M, K)
    qp, dp, _ = kqref.quantize_act(ACT_Q8_K, xp)
    op, _ = kqref.gemm(Q4_K, Wp, qp, dp, K)
    assert np.all(np.abs(op.astype(np.float64) - out) <= 1e-3 * tol)
    # output row selection returns the same columns
    rows = np.array([4, 1])
    osel, tsel = kqref.gemm(Q4_K, W, qs, d, K, rows=rows)
    assert np.array_equal(osel, out[:, rows]) and np.array_equal(tsel, tol[:, rows])


# ---------------------------------------------------------------------------
# Encoders (datagen) against decoders (oracle): round-trip bounds
# ---------------------------------------------------------------------------

def check_roundtrip_q4k():
    rng = np.random.default_rng(17)
    for scale, outl in ((0.02, False), (0.02, True), (3.0, False)):
        w = rng.standard_normal((8, 1024)) * scale
        if outl:
            w = np.where(rng.random(w.shape) < 0.01, w * 10, w)
        w = w.astype(np.float32)
        W = datagen.encode_q4k(w)
        wh = kqref.dequant_rows(Q4_K, W, 1024)
        for n in range(8):
            for s in range(4):
                d, dmin, sc, mn, q = kqref.decode_q4k(W[n, 144 * s:144 * (s + 1)])
                for j in range(8):
                    sl = slice(256 * s + 32 * j, 256 * s + 32 * (j + 1))
                    err = np.abs(w[n, sl].astype(np.float64) - wh[n, sl])
                    bound = 0.5 * d * sc[j] + 7.5 * d + 0.5 * dmin
                    assert np.all(err <= bound * (1 + 1e-9)), (n, s, j)


def check_roundtrip_q6k():
    rng = np.random.default_rng(19)
    for scale in (0.02, 3.0):
        w = (rng.standard_normal((8, 512)) * scale).astype(np.float32)
        W = datagen.encode_q6k(w)
        wh = kqref.dequant_rows(Q6_K, W, 512)
        for n in range(8):
            for s in range(2):
                d, sc, q = kqref.decode_q6k(W[n, 210 * s:210 * (s + 1)])
                for j in range(16):
                    sl = slice(256 * s + 16 * j, 256 * s + 16 * (j + 1))
                    err = np.abs(w[n, sl].astype(np.float64) - wh[n, sl])
                    bound = 0.5 * d * abs(sc[j]) + 15.5 * d
                    assert np.all(err <= bound * (1 + 1e-9)), (n, s, j)


def check_roundtrip_tq():
    t, d = datagen.draw_ternary(4, 640, 99)
    W = datagen.encode_tq(t, d)
    wh = kqref.dequant_rows(TQ, W, 640)
    want = t.astype(np.float64) * np.repeat(d.astype(np.float64), 128, axis=1)
    assert np.array_equal(wh, want)


def check_packers_agree():
    """datagen's vectorised packers (used by the GPU tests) emit exactly the
    bytes of the hand packers above."""
    rng = np.random.default_rng(23)
    d, dmin, sc, mn, q = datagen.random_fields_q4k(rng, 6)
    a = datagen.pack_q4k(d, dmin, sc, mn, q)
    b = np.stack([q4k_by_hand(f16_bits(float(d[i])), f16_bits(float(dmin[i])), sc[i], mn[i], q[i])
                  for i in range(6)])
    assert np.array_equal(a, b)
    d6, sc6, q6 = datagen.random_fields_q6k(rng, 6)
    a6 = datagen.pack_q6k(d6, sc6, q6)
    b6 = np.stack([q6k_by_hand(f16_bits(float(d6[i])), sc6[i], q6[i]) for i in range(6)])
    assert np.array_equal(a6, b6)
    dt, tt = datagen.random_fields_tq(rng, 6)
    at = datagen.pack_tq(tt, dt)
    bt = np.stack([tq_by_hand(f16_bits(float(dt[i])), tt[i]) for i in range(6)])
    assert np.array_equal(at, bt)
    d2, t2 = datagen.random_fields_tq2(rng, 6)
    a2 = datagen.pack_tq2(t2, d2)
    b2 = np.stack([tq2_by_hand(f16_bits(float(d2[i])), t2[i]) for i in range(6)])
    assert np.array_equal(a2, b2)


ALL_CHECKS = [
    check_f16_exhaustive,
    check_q4k_closed_form,
    check_q4k_field_positions,
    check_q4k_nibble_positions,
    check_q6k_closed_form,
    check_q6k_positions,
    check_tq_bytes,
    check_tq_block,
    check_tq2_codes,
    check_tq2_block,
    check_tq2_same_trits_as_tq,
    check_q8_ties,
    check_q8_zero_and_tiny,
    check_q8_properties,
    check_bruteforce_exact,
    check_integer_special_case,
    check_onehot_scales,
    check_invariants,
    check_roundtrip_q4k,
    check_roundtrip_q6k,
    check_roundtrip_tq,
    check_packers_agree,
]
