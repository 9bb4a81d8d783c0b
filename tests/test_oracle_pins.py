"""CPU tests: the oracle against its pins, and planted mistakes against the pins.

The planted-mistake test compiles copies of oracle/kqref.c with one plausible
error each (a dropped term, a wrong sign or index, a swapped nibble, the wrong
rounding rule, ...) and requires every copy to fail at least one pin.
"""
from __future__ import annotations

import json
import os
import subprocess

import numpy as np
import pytest

import oracle_pins as pins
from oracle import kqref

HERE = os.path.dirname(os.path.abspath(__file__))


@pytest.mark.parametrize("check", pins.ALL_CHECKS, ids=lambda f: f.__name__)
def test_pin(ref, check):
    check()


def test_page_facts(ref):
    facts = json.load(open(os.path.join(HERE, "golden", "page_facts.json")))
    q8 = facts["q8k_block_bytes_per_256"]
    assert sum(q8["parts"].values()) == q8["value"] == 292
    # our Q8_K sections carry exactly these parts per 256 activations
    M, K = 1, 256
    qs, d, bs = kqref.quantize_act(kqref.ACT_Q8_K, np.ones((M, K), np.float32))
    assert qs.nbytes == q8["parts"]["qs_int8"]
    assert d.nbytes == q8["parts"]["d_fp32"]
    assert bs.nbytes == q8["parts"]["bsums_int16_per_16"]
    tb = facts["ternary_block"]
    assert kqref.BLOCK_BYTES[kqref.TQ] == tb["bytes"] and kqref.QK[kqref.TQ] == tb["weights"]
    # word 6 of a ternary block is qh[0] | qh[1] << 8 | d << 16, where the two
    # bytes after the six qs words are the page's qh bytes
    blk = pins.tq_by_hand(pins.f16_bits(0.03125), [1, -1, 0, 0] * 32)
    words = blk.view(np.uint32)
    assert len(words) == tb["qs_words"] + 1
    d_bits = pins.f16_bits(0.03125)
    assert int(words[6]) == int(blk[24]) | (int(blk[25]) << 8) | (d_bits << 16)


MUTANTS = [
    ("q4k high nibble read as low", "q[64 * c + 32 + t] = (byte >> 4) & 15;",
     "q[64 * c + 32 + t] = byte & 15;"),
    ("q4k min added instead of subtracted", "if (w) w[k] = d * sc[j] * q[k] - dmin * mn[j];",
     "if (w) w[k] = d * sc[j] * q[k] + dmin * mn[j];"),
    ("q4k min fields shifted by one bit", "int pos = 6 * f + bit;",
     "int pos = 6 * f + bit + (f >= 8);"),
    ("q4k scale and min fields swapped",
     "if (f < 8)\n            sc[f] = v;\n        else\n            mn[f - 8] = v;",
     "if (f < 8)\n            mn[f] = v;\n        else\n            sc[f - 8] = v;"),
    ("q6k integer operand offset 31", "if (qint) qint[k] = q[k] - 32;",
     "if (qint) qint[k] = q[k] - 31;"),
    ("q6k dequant offset 31", "if (w) w[k] = d * sc[j] * (q[k] - 32);",
     "if (w) w[k] = d * sc[j] * (q[k] - 31);"),
    ("q6k scales read unsigned", "sc[j] = (int8_t)b[192 + j];", "sc[j] = (uint8_t)b[192 + j];"),
    ("q6k high bits at the wrong shift", "q[128 * h + 32 * u + t] |= ((v >> (2 * u)) & 3) << 4;",
     "q[128 * h + 32 * u + t] |= ((v >> (2 * u)) & 3) << 2;"),
    ("q6k sub-block of 32", "int j = k / 16;\n            if (w) w[k] = d * sc[j]",
     "int j = k / 32;\n            if (w) w[k] = d * sc[j]"),
    ("ternary digits most significant first", "for (int p = 0; p < k % 5; p++)",
     "for (int p = 0; p < 4 - k % 5; p++)"),
    ("ternary trit not centred", "t[k] = v % 3 - 1;", "t[k] = v % 3 - (k % 7 != 0);"),
    ("q8 ties away from zero", "float v = rintf(x[i] * s);", "float v = roundf(x[i] * s);"),
    ("q8 scale over 128", "*d = amax / 127.0f;", "*d = amax / 128.0f;"),
    ("q8 amax without abs", "float a = fabsf(x[i]);", "float a = x[i];"),
    ("q8 bsums drop one element", "for (int i = 0; i < 16; i++) sum += qs[16 * g + i];",
     "for (int i = 0; i < 15; i++) sum += qs[16 * g + i];"),
    ("gemm activation scale without block index",
     "A[m * K + k] = (double)d_a[m * na + k / abs_] * (double)qs[m * K + k];",
     "A[m * K + k] = (double)d_a[m * na] * (double)qs[m * K + k];"),
    ("gemm activation reversed along K", "double p = w[k] * a[k];",
     "double p = w[k] * a[K - 1 - k];"),
    ("ternary with 256-wide activation scales", "int abs_ = ternary(fmt) ? 128 : 256;",
     "int abs_ = 256;"),
    ("tq2 code planes in reverse", "int c = (b[k % 32] >> (2 * (k / 32))) & 3;",
     "int c = (b[k % 32] >> (6 - 2 * (k / 32))) & 3;"),
    ("tq2 codes of consecutive weights in one byte", "int c = (b[k % 32] >> (2 * (k / 32))) & 3;",
     "int c = (b[k / 4] >> (2 * (k % 4))) & 3;"),
    ("tq2 code not centred", "        t[k] = c - 1;\n", "        t[k] = c - (k != 5);\n"),
    ("tq2 scale read from the code bytes", "*d = kqref_f16_to_f64(rd16(b + 32));",
     "*d = kqref_f16_to_f64(rd16(b + 30));"),
    ("tolerance without abs", "mag += fabs(p);", "mag += p;"),
    ("subsums activation index restarts per sub-block",
     "acc += (int64_t)qi[k] * (int64_t)qs[m * K + k];",
     "acc += (int64_t)qi[k] * (int64_t)qs[m * K + k - j * sub];"),
    ("fp16 exponent bias off by one", "v = ldexp((double)(1024 + frac), e - 25);",
     "v = ldexp((double)(1024 + frac), e - 24);"),
    ("fp16 subnormal scale", "v = ldexp((double)frac, -24);", "v = ldexp((double)frac, -25);"),
]


def _first_failure(libpath):
    with kqref.use_library(libpath):
        for check in pins.ALL_CHECKS:
            try:
                check()
            except AssertionError:
                return check.__name__
    return None


@pytest.mark.parametrize("name,orig,mut", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_planted_mistake_is_caught(ref, tmp_path, name, orig, mut):
    src = open(kqref.SRC).read()
    assert src.count(orig) == 1, "mutation site not found: " + name
    path = tmp_path / "kqref_mut.c"
    path.write_text(src.replace(orig, mut))
    lib = str(tmp_path / "libkqref_mut.so")
    subprocess.check_call(["gcc", *kqref.CFLAGS, "-o", lib, str(path), "-lm"])
    failed = _first_failure(lib)
    assert failed is not None, "no pin caught: " + name


def test_unmutated_copy_passes(ref, tmp_path):
    path = tmp_path / "kqref_copy.c"
    path.write_text(open(kqref.SRC).read())
    lib = str(tmp_path / "libkqref_copy.so")
    subprocess.check_call(["gcc", *kqref.CFLAGS, "-o", lib, str(path), "-lm"])
    assert _first_failure(lib) is None
