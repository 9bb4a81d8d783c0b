"""GPU tests of the calibration kernels: each launch runs, reports its work,
and the rate it implies lies between a tenth of and just above the published
MI355X peak (int8 matrix core 5.0 POP/s, fp32 vector 157.3 TFLOP/s, which
plain v_fma_f32 reaches on gfx950 without packed math, HBM 8 TB/s)."""
from __future__ import annotations

import pytest

pytestmark = pytest.mark.gpu


def rate(kq, kind, param=0, buf=None, nbytes=0):
    import torch
    s = torch.cuda.current_stream()
    kq.kq_calib_launch(kind, param, buf, nbytes, s.cuda_stream)  # warm-up
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(s)
    work = kq.kq_calib_launch(kind, param, buf, nbytes, s.cuda_stream)
    e1.record(s)
    torch.cuda.synchronize()
    return work / (e0.elapsed_time(e1) * 1e-3)


@pytest.fixture(scope="module")
def kq():
    import block_quantized_matmul_act_amd as kq
    kq.lib()
    return kq


def test_matrix_core_rates(kq):
    toggle = None
    for kind in (kq.KQ_CALIB_MFMA_I8, kq.KQ_CALIB_MFMA_I8_TOGGLE):
        r = rate(kq, kind) / 1e12
        print(f"calib kind {kind}: {r:.0f} TOP/s int8", flush=True)
        assert 500 < r < 5100
        toggle = r
    for p in (2, 4, 6, 8):
        r = rate(kq, kq.KQ_CALIB_MFMA_I8_VALU, p) / 1e12
        print(f"calib MFMA with {p} more VALU/MFMA: {r:.0f} TOP/s int8", flush=True)
        assert 200 < r < 5100
    # the most VALU work between MFMAs never runs faster than none (single
    # launches vary by a few percent with the clock)
    assert r < toggle * 1.1


def test_valu_rate(kq):
    r = rate(kq, kq.KQ_CALIB_VALU_F32) / 1e12
    print(f"calib VALU: {r:.1f} TFLOP/s fp32", flush=True)
    assert 15.7 < r < 160


def test_hbm_read_rate(kq):
    import torch
    nbytes = 1 << 30
    buf = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    buf.fill_(3)
    r = rate(kq, kq.KQ_CALIB_HBM_READ, 0, buf, nbytes) / 1e9
    print(f"calib HBM read: {r:.0f} GB/s", flush=True)
    assert 800 < r < 8200
