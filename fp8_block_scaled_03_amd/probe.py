"""ctypes binding of libfp8bs_probe.so (measurement and test support; see
include/fp8bs_probe.h).  Argument marshalling only; raises Fp8bsError when the
library is missing or a call is rejected."""

from __future__ import annotations

import ctypes
import os
import threading

import torch

from .binding import Fp8bsError, _stream_ptr

_PKG = os.path.dirname(os.path.abspath(__file__))
_lock = threading.Lock()
_lib = None


def load_probe_library() -> ctypes.CDLL:
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        path = os.path.join(_PKG, "libfp8bs_probe.so")
        if not os.path.exists(path):
            raise Fp8bsError(f"{path} not found: build it first (python -m fp8_block_scaled_03_amd.build)")
        lib = ctypes.CDLL(path)
        vp, i32 = ctypes.c_void_p, ctypes.c_int
        lib.fp8bs_probe_gemm.argtypes = [vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, vp]
        lib.fp8bs_probe_gemm.restype = i32
        lib.fp8bs_probe_mfma_scale.argtypes = [vp, vp, vp, vp, vp, vp, i32, vp]
        lib.fp8bs_probe_mfma_scale.restype = i32
        lib.fp8bs_probe_promote_ceiling.argtypes = [vp, i32, i32, i32, vp]
        lib.fp8bs_probe_promote_ceiling.restype = i32
        lib.fp8bs_probe_stream_read.argtypes = [vp, ctypes.c_longlong, vp, i32, vp]
        lib.fp8bs_probe_stream_read.restype = i32
        _lib = lib
        return lib


def _dev(t: torch.Tensor, dtype, shape, name):
    if t.dtype != dtype or tuple(t.shape) != tuple(shape) or not t.is_contiguous() or not t.is_cuda:
        raise Fp8bsError(f"{name}: need contiguous {dtype} {tuple(shape)} on the GPU, got {t.dtype} {tuple(t.shape)}")
    return t.data_ptr()


def _ok(rc: int, what: str) -> None:
    if rc != 0:
        raise Fp8bsError(f"{what} rejected (status {rc})")


def gemm(qa, sa, qb, sb, fp8_form: bool, with_partials: bool = False):
    """C (bf16 [M, N]) and optionally the K-block partials (fp32 [K/32, M, N])."""
    M, K = qa.shape
    N = qb.shape[1]
    c = torch.empty((M, N), dtype=torch.bfloat16, device=qa.device)
    parts = torch.empty((K // 32, M, N), dtype=torch.float32, device=qa.device) if with_partials else None
    rc = load_probe_library().fp8bs_probe_gemm(
        _dev(qa, torch.uint8, (M, K), "a"), _dev(sa, torch.float32, (M // 32, K // 32), "sa"),
        _dev(qb, torch.uint8, (K, N), "b"), _dev(sb, torch.float32, (K // 32, N // 32), "sb"),
        c.data_ptr(), parts.data_ptr() if parts is not None else None, M, N, K, 1 if fp8_form else 0,
        _stream_ptr(qa))
    _ok(rc, "fp8bs_probe_gemm")
    return c, parts


def mfma_scale(a, bt, ea, eb, cin):
    """d [count, 16, 16] fp32 from one scaled MFMA per problem."""
    count = a.shape[0]
    d = torch.empty((count, 16, 16), dtype=torch.float32, device=a.device)
    rc = load_probe_library().fp8bs_probe_mfma_scale(
        _dev(a, torch.uint8, (count, 16, 128), "a"), _dev(bt, torch.uint8, (count, 16, 128), "bt"),
        _dev(ea, torch.uint8, (count, 16, 4), "ea"), _dev(eb, torch.uint8, (count, 16, 4), "eb"),
        _dev(cin, torch.float32, (count, 16, 16), "cin"), d.data_ptr(), count, _stream_ptr(a))
    _ok(rc, "fp8bs_probe_mfma_scale")
    return d


def promote_ceiling(out, workgroups: int, iters: int, mode: int = 0):
    """Enqueue the register-only MFMA + promotion loop (out: fp32 [workgroups * 8]);
    mode 0 = MFMA + four FMAs per step, 1 = the MFMAs alone, 2 = the FMAs alone,
    3 = the FP8 form of the MFMA alone (iters x 8 steps); 4-7 = the mix in
    bursts of PROMOTE_BURSTS[mode] MFMAs, each followed by the previous burst's
    FMAs (iters x 12 steps, iters even); 8 = the hardware-scaled f8f6f4 MFMA
    alone (iters x 8 instructions of SCALED_MFMA_FLOPS each)."""
    rc = load_probe_library().fp8bs_probe_promote_ceiling(
        _dev(out, torch.float32, (workgroups * 8,), "out"), workgroups, iters, mode, _stream_ptr(out))
    _ok(rc, "fp8bs_probe_promote_ceiling")


PROMOTE_CEILING_FLOPS_PER_STEP = 2 * 16 * 16 * 32   # one 16x16x32 MFMA
PROMOTE_BURSTS = {4: 2, 5: 3, 6: 4, 7: 6}             # burst modes -> MFMAs per burst
PROMOTE_STEPS_PER_ITER = {0: 8, 1: 8, 2: 8, 3: 8, 4: 12, 5: 12, 6: 12, 7: 12, 8: 8}
SCALED_MFMA_FLOPS = 2 * 16 * 16 * 128              # one 16x16x128 scaled MFMA


def stream_read(buf, out, workgroups: int):
    """Enqueue one streaming read of the whole of `buf` (any contiguous GPU
    tensor, size a multiple of 16 bytes); out: int32 [workgroups * 8]."""
    if not buf.is_cuda or not buf.is_contiguous():
        raise Fp8bsError("stream_read: need a contiguous GPU tensor")
    rc = load_probe_library().fp8bs_probe_stream_read(
        buf.data_ptr(), buf.numel() * buf.element_size(), _dev(out, torch.int32, (workgroups * 8,), "out"),
        workgroups, _stream_ptr(buf))
    _ok(rc, "fp8bs_probe_stream_read")
