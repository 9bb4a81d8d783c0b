"""Python binding of libkq (include/kq.h): block-quantized GEMM for MI355X.

Argument marshalling only.  Every step of the path runs in the HIP kernels of
libkq.so; there is no CPU fallback.  If the library is missing the first call
raises.  The kq_* functions mirror the C ABI one to one and accept torch
tensors (their data_ptr() is passed) or plain integer addresses.  `stream`
defaults to torch's current HIP stream.
"""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libkq.so")

KQ_Q4_K, KQ_Q6_K, KQ_TQ, KQ_TQ2 = 1, 2, 3, 4
KQ_ACT_Q8_K, KQ_ACT_Q8_128 = 1, 2
KQ_SEC_QS, KQ_SEC_D, KQ_SEC_BSUMS, KQ_SEC_ALPHA = 0, 1, 2, 3
KQ_OK = 0
KQ_DEBUG_UNPACK_MAX_BLOCKS = 1 << 24
KQ_GEMM_ID_MAX_EXPERTS = 1024
KQ_ERR_FMT, KQ_ERR_SHAPE, KQ_ERR_NULL, KQ_ERR_ALIGN, KQ_ERR_UNSUPPORTED, KQ_ERR_HIP = (
    -1, -2, -3, -4, -5, -6)
(KQ_CALIB_MFMA_I8, KQ_CALIB_MFMA_I8_TOGGLE, KQ_CALIB_VALU_F32, KQ_CALIB_MFMA_I8_VALU,
 KQ_CALIB_HBM_READ) = 0, 1, 2, 3, 4

# Every symbol include/kq.h declares, with its ctypes signature.
_P, _I, _I64, _SZ = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_size_t
SIGNATURES = {
    "kq_weight_bytes": (_SZ, [_I, _I64, _I64]),
    "kq_act_bytes": (_SZ, [_I, _I64, _I64]),
    "kq_act_section_offset": (_I64, [_I, _I, _I64, _I64]),
    "kq_act_fmt_for": (_I, [_I]),
    "kq_quantize_act": (_I, [_I, _P, _I64, _I64, _P, _P]),
    "kq_gemm": (_I, [_I, _P, _P, _I64, _I64, _I64, _P, _P]),
    "kq_gemm_subsums": (_I, [_I, _P, _P, _I64, _I64, _I64, _P, _P]),
    "kq_debug_unpack": (_I, [_I, _P, _I64, _P, _P, _P]),
    "kq_gemm_id": (_I, [_I, _P, _I64, _P, _I64, _I64, _I64, _P, _P, _I64, _P, _P]),
    "kq_num_variants": (_I, []),
    "kq_variant_name": (ctypes.c_char_p, [_I]),
    "kq_dispatch_count": (ctypes.c_uint64, [_I]),
    "kq_dispatch_reset": (None, []),
    "kq_select_variant": (_I, [_I, _I64, _I64, _I64]),
    "kq_calib_launch": (_I, [_I, _I, _P, _I64, ctypes.POINTER(ctypes.c_double), _P]),
    "kq_strerror": (ctypes.c_char_p, [_I]),
    "kq_version": (_I, []),
}


class KQError(RuntimeError):
    def __init__(self, status: int, where: str):
        super().__init__(f"{where}: {kq_strerror(status)} (status {status})")
        self.status = status


_lib = None


def lib():
    """Load libkq.so (built in-tree by __graft_entry__.build())."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with __graft_entry__.build() "
                               "(hipcc --offload-arch=gfx950); there is no fallback path")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


def _ptr(t):
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream):
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _check(status: int, where: str) -> int:
    if status != KQ_OK:
        raise KQError(status, where)
    return status


def _need(t, nbytes, what, dtype=None):
    """Host-side check of a torch tensor argument before its address goes to the
    library (plain integer addresses are passed through unchecked): a
    contiguous device tensor of the right element type holding at least
    nbytes bytes.  Raises ValueError; nothing is launched."""
    if t is None or isinstance(t, int):
        return
    if not getattr(t, "is_cuda", False):
        raise ValueError(f"{what}: expected a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{what}: expected a contiguous tensor")
    if dtype is not None and str(t.dtype) != "torch." + dtype:
        raise ValueError(f"{what}: expected dtype {dtype}, got {t.dtype}")
    have = t.numel() * t.element_size()
    if have < nbytes:
        raise ValueError(f"{what}: {have} bytes, {nbytes} needed")


def _sub_block(fmt):
    return {KQ_Q4_K: 32, KQ_Q6_K: 16}.get(fmt, 128)


# ---------------------------------------------------------------- C ABI mirror

def kq_weight_bytes(fmt, N, K):
    return lib().kq_weight_bytes(fmt, N, K)


def kq_act_bytes(act_fmt, M, K):
    return lib().kq_act_bytes(act_fmt, M, K)


def kq_act_section_offset(act_fmt, section, M, K):
    return lib().kq_act_section_offset(act_fmt, section, M, K)


def kq_act_fmt_for(fmt):
    return lib().kq_act_fmt_for(fmt)


def kq_quantize_act(act_fmt, x, M, K, a_q8, stream=None):
    _need(x, 4 * max(M, 0) * max(K, 0), "kq_quantize_act x", "float32")
    _need(a_q8, kq_act_bytes(act_fmt, M, K), "kq_quantize_act a_q8")
    return _check(lib().kq_quantize_act(act_fmt, _ptr(x), M, K, _ptr(a_q8), _stream(stream)),
                  "kq_quantize_act")


def _need_gemm_inputs(fmt, W, a_q8, M, N, K, where, n_experts=1):
    _need(W, n_experts * kq_weight_bytes(fmt, N, K), where + " W")
    act = kq_act_fmt_for(fmt)
    if act > 0:
        _need(a_q8, kq_act_bytes(act, M, K), where + " a_q8")


def kq_gemm(fmt, W, a_q8, M, N, K, out, stream=None):
    _need_gemm_inputs(fmt, W, a_q8, M, N, K, "kq_gemm")
    _need(out, 4 * max(M, 0) * max(N, 0), "kq_gemm out", "float32")
    return _check(lib().kq_gemm(fmt, _ptr(W), _ptr(a_q8), M, N, K, _ptr(out), _stream(stream)),
                  "kq_gemm")


def kq_gemm_subsums(fmt, W, a_q8, M, N, K, sums, stream=None):
    _need_gemm_inputs(fmt, W, a_q8, M, N, K, "kq_gemm_subsums")
    _need(sums, 4 * max(M, 0) * max(N, 0) * max(K, 0) // _sub_block(fmt), "kq_gemm_subsums sums", "int32")
    return _check(lib().kq_gemm_subsums(fmt, _ptr(W), _ptr(a_q8), M, N, K, _ptr(sums),
                                        _stream(stream)), "kq_gemm_subsums")


def kq_num_variants():
    return lib().kq_num_variants()


def kq_variant_name(v):
    s = lib().kq_variant_name(v)
    return s.decode() if s else None


def kq_dispatch_count(v):
    return lib().kq_dispatch_count(v)


def kq_dispatch_reset():
    lib().kq_dispatch_reset()


def kq_select_variant(fmt, M, N, K):
    return lib().kq_select_variant(fmt, M, N, K)


def kq_debug_unpack(fmt, W, nblocks, q, scales, stream=None):
    return _check(lib().kq_debug_unpack(fmt, _ptr(W), nblocks, _ptr(q), _ptr(scales),
                                        _stream(stream)), "kq_debug_unpack")


def kq_gemm_id(fmt, W, n_experts, a_q8, M, N, K, expert_offsets, rows, R, out, stream=None):
    if 1 <= n_experts <= KQ_GEMM_ID_MAX_EXPERTS:
        _need_gemm_inputs(fmt, W, a_q8, M, N, K, "kq_gemm_id", n_experts)
        _need(expert_offsets, 4 * (n_experts + 1), "kq_gemm_id expert_offsets", "int32")
    _need(rows, 4 * max(R, 0), "kq_gemm_id rows", "int32")
    _need(out, 4 * max(R, 0) * max(N, 0), "kq_gemm_id out", "float32")
    return _check(lib().kq_gemm_id(fmt, _ptr(W), n_experts, _ptr(a_q8), M, N, K, _ptr(expert_offsets),
                                   _ptr(rows), R, _ptr(out), _stream(stream)), "kq_gemm_id")


def kq_calib_launch(kind, param=0, buf=None, nbytes=0, stream=None):
    """Launch one calibration kernel; returns the work it does (int8 ops, fp32
    flops or bytes)."""
    work = ctypes.c_double(0.0)
    _check(lib().kq_calib_launch(kind, param, _ptr(buf), nbytes, ctypes.byref(work), _stream(stream)),
           "kq_calib_launch")
    return work.value


def kq_strerror(status):
    return lib().kq_strerror(status).decode()


def kq_version():
    return lib().kq_version()


# ------------------------------------------------- torch conveniences (allocation)

def dispatch_counts() -> dict:
    return {kq_variant_name(v): kq_dispatch_count(v) for v in range(kq_num_variants())}


def quantize_act(x, act_fmt=KQ_ACT_Q8_K, stream=None):
    """fp32 [M][K] device tensor -> uint8 device tensor holding the activation buffer."""
    import torch
    M, K = x.shape
    a_q8 = torch.empty(kq_act_bytes(act_fmt, M, K), dtype=torch.uint8, device=x.device)
    kq_quantize_act(act_fmt, x, M, K, a_q8, stream)
    return a_q8


def act_views(a_q8, act_fmt, M, K):
    """(qs int8 [M][K], d fp32 [M][K/bs], bsums int16 [M][K/16] or None) views of a
    buffer.  d is stored block-major ([K/bs][M]); the view is its transpose."""
    import torch
    bs = 256 if act_fmt == KQ_ACT_Q8_K else 128
    od = kq_act_section_offset(act_fmt, KQ_SEC_D, M, K)
    qs = a_q8[:M * K].view(torch.int8).view(M, K)
    d = a_q8[od:od + M * (K // bs) * 4].view(torch.float32).view(K // bs, M).t()
    bsums = None
    if act_fmt == KQ_ACT_Q8_K:
        ob = kq_act_section_offset(act_fmt, KQ_SEC_BSUMS, M, K)
        bsums = a_q8[ob:ob + M * (K // 16) * 2].view(torch.int16).view(M, K // 16)
    return qs, d, bsums


def alpha_view(a_q8, M, K):
    """The Q8_K alpha section as int16 bit patterns of bf16 values, [K/256][2][M][8]."""
    import torch
    oa = kq_act_section_offset(KQ_ACT_Q8_K, KQ_SEC_ALPHA, M, K)
    n = (K // 256) * 2 * M * 8
    return a_q8[oa:oa + 2 * n].view(torch.int16).view(K // 256, 2, M, 8)


def gemm(fmt, W, a_q8, M, N, K, out=None, stream=None):
    """out fp32 [M][N] = W x A (device tensors)."""
    import torch
    if out is None:
        out = torch.empty((M, N), dtype=torch.float32, device=a_q8.device)
    kq_gemm(fmt, W, a_q8, M, N, K, out, stream)
    return out


def debug_unpack(fmt, W, nblocks, stream=None):
    """Decode nblocks weight blocks (uint8 device tensor) with the tile kernel's
    loaders: (q int8 [nblocks][QK], scales int32 [nblocks][16] or None)."""
    import torch
    ternary = fmt in (KQ_TQ, KQ_TQ2)
    qk = 128 if ternary else 256
    q = torch.empty((nblocks, qk), dtype=torch.int8, device=W.device)
    scales = None if ternary else torch.empty((nblocks, 16), dtype=torch.int32, device=W.device)
    kq_debug_unpack(fmt, W, nblocks, q, scales, stream)
    return q, scales


def gemm_id(fmt, W, n_experts, a_q8, M, N, K, expert_offsets, rows, out=None, stream=None):
    """out fp32 [R][N]: routed row r = expert e's weights x token rows[r]
    (expert_offsets int32 [n_experts + 1], rows int32 [R]; device tensors)."""
    import torch
    R = rows.numel()
    if out is None:
        out = torch.empty((R, N), dtype=torch.float32, device=a_q8.device)
    kq_gemm_id(fmt, W, n_experts, a_q8, M, N, K, expert_offsets, rows, R, out, stream)
    return out
