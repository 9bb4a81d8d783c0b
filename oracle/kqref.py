"""ctypes front end of the plain CPU oracle (oracle/kqref.c).

TEST INFRASTRUCTURE ONLY: imported by the test suite, the smoke check and the
CPU-baseline leg of the benchmark.  The HIP path never imports it.  This file
only marshals numpy arrays into the C routines; all arithmetic is in kqref.c.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "kqref.c")
LIB = os.path.join(HERE, "libkqref.so")

Q4_K, Q6_K, TQ, TQ2 = 1, 2, 3, 4
ACT_Q8_K, ACT_Q8_128 = 1, 2
QK = {Q4_K: 256, Q6_K: 256, TQ: 128, TQ2: 128}
BLOCK_BYTES = {Q4_K: 144, Q6_K: 210, TQ: 28, TQ2: 34}
SUB = {Q4_K: 32, Q6_K: 16, TQ: 128, TQ2: 128}
ACT_FOR = {Q4_K: ACT_Q8_K, Q6_K: ACT_Q8_K, TQ: ACT_Q8_128, TQ2: ACT_Q8_128}
ACT_BS = {ACT_Q8_K: 256, ACT_Q8_128: 128}

CFLAGS = ["-O2", "-fopenmp", "-ffp-contract=off", "-fPIC", "-shared", "-Wall"]


def build(force: bool = False) -> str:
    """Compile kqref.c with gcc (plain C, no fast-math)."""
    if force or not os.path.exists(LIB) or os.path.getmtime(LIB) < os.path.getmtime(SRC):
        tmp = LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", *CFLAGS, "-o", tmp, SRC, "-lm"])
        os.replace(tmp, LIB)
    return LIB


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB):
            build()
        _lib = _bind(ctypes.CDLL(LIB))
    return _lib


class use_library:
    """Context manager that points this module at another build of kqref.c
    (used by the tests that plant mistakes in a copy of the oracle)."""

    def __init__(self, path: str):
        self.path = path

    def __enter__(self):
        global _lib
        self.saved = _lib
        _lib = _bind(ctypes.CDLL(self.path))
        return self

    def __exit__(self, *exc):
        global _lib
        _lib = self.saved
        return False


def _bind(L):
    P = ctypes.c_void_p
    I64 = ctypes.c_int64
    L.kqref_f16_to_f64.restype = ctypes.c_double
    L.kqref_f16_to_f64.argtypes = [ctypes.c_uint16]
    L.kqref_decode_q4k.argtypes = [P, P, P, P, P, P]
    L.kqref_decode_q6k.argtypes = [P, P, P, P]
    L.kqref_decode_tq.argtypes = [P, P, P]
    L.kqref_decode_tq2.argtypes = [P, P, P]
    L.kqref_dequant_rows.argtypes = [ctypes.c_int, P, I64, I64, P]
    L.kqref_int_operands.argtypes = [ctypes.c_int, P, I64, I64, P]
    L.kqref_quantize_act.argtypes = [ctypes.c_int, P, I64, I64, P, P, P]
    L.kqref_gemm_rows.argtypes = [ctypes.c_int, P, P, P, I64, I64, I64, P, I64, P, P]
    L.kqref_subsums.argtypes = [ctypes.c_int, P, P, I64, I64, I64, P]
    return L


def _p(a: np.ndarray):
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data_as(ctypes.c_void_p)


def f16_to_f64(bits: int) -> float:
    return lib().kqref_f16_to_f64(bits)


def decode_q4k(block: np.ndarray):
    b = np.ascontiguousarray(block, dtype=np.uint8)
    d = np.zeros(1, np.float64); dm = np.zeros(1, np.float64)
    sc = np.zeros(8, np.int32); mn = np.zeros(8, np.int32); q = np.zeros(256, np.int32)
    lib().kqref_decode_q4k(_p(b), _p(d), _p(dm), _p(sc), _p(mn), _p(q))
    return float(d[0]), float(dm[0]), sc, mn, q


def decode_q6k(block: np.ndarray):
    b = np.ascontiguousarray(block, dtype=np.uint8)
    d = np.zeros(1, np.float64); sc = np.zeros(16, np.int32); q = np.zeros(256, np.int32)
    lib().kqref_decode_q6k(_p(b), _p(d), _p(sc), _p(q))
    return float(d[0]), sc, q


def decode_tq(block: np.ndarray):
    b = np.ascontiguousarray(block, dtype=np.uint8)
    d = np.zeros(1, np.float64); t = np.zeros(128, np.int32)
    lib().kqref_decode_tq(_p(b), _p(d), _p(t))
    return float(d[0]), t


def decode_tq2(block: np.ndarray):
    b = np.ascontiguousarray(block, dtype=np.uint8)
    d = np.zeros(1, np.float64); t = np.zeros(128, np.int32)
    lib().kqref_decode_tq2(_p(b), _p(d), _p(t))
    return float(d[0]), t


def dequant_rows(fmt: int, W: np.ndarray, K: int) -> np.ndarray:
    W = np.ascontiguousarray(W, dtype=np.uint8)
    N = W.shape[0]
    out = np.zeros((N, K), np.float64)
    rc = lib().kqref_dequant_rows(fmt, _p(W), N, K, _p(out))
    assert rc == 0, rc
    return out


def int_operands(fmt: int, W: np.ndarray, K: int) -> np.ndarray:
    W = np.ascontiguousarray(W, dtype=np.uint8)
    N = W.shape[0]
    out = np.zeros((N, K), np.int32)
    rc = lib().kqref_int_operands(fmt, _p(W), N, K, _p(out))
    assert rc == 0, rc
    return out


def quantize_act(act_fmt: int, x: np.ndarray):
    """x fp32 [M][K] -> (qs int8 [M][K], d fp32 [M][K/bs], bsums int16 [M][K/16] or None)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    M, K = x.shape
    bs = ACT_BS[act_fmt]
    qs = np.zeros((M, K), np.int8)
    d = np.zeros((M, K // bs), np.float32)
    bsums = np.zeros((M, K // 16), np.int16) if act_fmt == ACT_Q8_K else None
    rc = lib().kqref_quantize_act(act_fmt, _p(x), M, K, _p(qs), _p(d),
                                  _p(bsums) if bsums is not None else None)
    assert rc == 0, rc
    return qs, d, bsums


def gemm(fmt: int, W: np.ndarray, qs: np.ndarray, d_a: np.ndarray, K: int,
         rows: np.ndarray | None = None, want_tol: bool = True):
    """fp32 out [M][N] (or [M][len(rows)]) and fp64 tol of the same shape."""
    W = np.ascontiguousarray(W, dtype=np.uint8)
    qs = np.ascontiguousarray(qs, dtype=np.int8)
    d_a = np.ascontiguousarray(d_a, dtype=np.float32)
    M = qs.shape[0]
    N = W.shape[0]
    if rows is not None:
        rows = np.ascontiguousarray(rows, dtype=np.int64)
        ncols = rows.shape[0]
    else:
        ncols = N
    out = np.zeros((M, ncols), np.float32)
    tol = np.zeros((M, ncols), np.float64) if want_tol else None
    rc = lib().kqref_gemm_rows(fmt, _p(W), _p(qs), _p(d_a), M, N, K,
                               _p(rows) if rows is not None else None,
                               ncols if rows is not None else 0,
                               _p(out), _p(tol) if tol is not None else None)
    assert rc == 0, rc
    return out, tol


def subsums(fmt: int, W: np.ndarray, qs: np.ndarray, K: int) -> np.ndarray:
    W = np.ascontiguousarray(W, dtype=np.uint8)
    qs = np.ascontiguousarray(qs, dtype=np.int8)
    M, N = qs.shape[0], W.shape[0]
    S = np.zeros((M, N, K // SUB[fmt]), np.int32)
    rc = lib().kqref_subsums(fmt, _p(W), _p(qs), M, N, K, _p(S))
    assert rc == 0, rc
    return S
