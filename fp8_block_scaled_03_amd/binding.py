"""ctypes binding of libfp8bs.so (argument marshalling only).

Every function here checks torch dtypes, shapes, contiguity and devices, then
passes raw device pointers and the current HIP stream to the C ABI declared in
include/fp8bs.h.  No arithmetic of the method happens in Python; if the library
is missing the call raises ``Fp8bsError`` - there is no fallback path.
"""

from __future__ import annotations

import ctypes
import os
import threading

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
_LIB_NAME = "libfp8bs.so"
_lock = threading.Lock()
_lib = None

BLOCK = 32
E4M3_DTYPES = (torch.uint8, torch.float8_e4m3fn)
STATUS = {0: "FP8BS_OK", 1: "FP8BS_EINVAL", 2: "FP8BS_ESHAPE", 3: "FP8BS_EALIGN", 4: "FP8BS_EHIP",
          5: "FP8BS_ENOSYS"}


class Fp8bsError(RuntimeError):
    """Raised for a non-OK status from the library or a missing library."""


def library_path() -> str:
    return os.environ.get("FP8BS_LIBRARY", os.path.join(_PKG, _LIB_NAME))


def load_library() -> ctypes.CDLL:
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        path = library_path()
        if not os.path.exists(path):
            raise Fp8bsError(f"{path} not found: build it first (python -m fp8_block_scaled_03_amd.build)")
        lib = ctypes.CDLL(path)
        vp, i64, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32
        lib.fp8bs_quantize.argtypes = [vp, i64, i64, vp, vp, vp]
        lib.fp8bs_quantize.restype = ctypes.c_int
        lib.fp8bs_gemm.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, vp]
        lib.fp8bs_gemm.restype = ctypes.c_int
        lib.fp8bs_grouped_gemm.argtypes = [vp, vp, vp, vp, vp, i32, vp, i64, i64, i64, vp]
        lib.fp8bs_grouped_gemm.restype = ctypes.c_int
        lib.fp8bs_gemm_nt.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, vp]
        lib.fp8bs_gemm_nt.restype = ctypes.c_int
        lib.fp8bs_quantize_tg.argtypes = [vp, i64, i64, vp, vp, vp]
        lib.fp8bs_quantize_tg.restype = ctypes.c_int
        lib.fp8bs_gemm_tg.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, vp]
        lib.fp8bs_gemm_tg.restype = ctypes.c_int
        lib.fp8bs_gemm_tg_nt.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, vp]
        lib.fp8bs_gemm_tg_nt.restype = ctypes.c_int
        lib.fp8bs_grouped_gemm_nt.argtypes = [vp, vp, vp, vp, vp, i32, vp, i64, i64, i64, vp]
        lib.fp8bs_grouped_gemm_nt.restype = ctypes.c_int
        lib.fp8bs_rmsnorm_quantize_tg.argtypes = [vp, vp, vp, ctypes.c_float, i64, i64, vp, vp, vp, vp]
        lib.fp8bs_rmsnorm_quantize_tg.restype = ctypes.c_int
        lib.fp8bs_quantize_e8m0.argtypes = [vp, i64, i64, vp, vp, vp]
        lib.fp8bs_quantize_e8m0.restype = ctypes.c_int
        lib.fp8bs_gemm_e8m0_nt.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, vp]
        lib.fp8bs_gemm_e8m0_nt.restype = ctypes.c_int
        lib.fp8bs_status_str.argtypes = [ctypes.c_int]
        lib.fp8bs_status_str.restype = ctypes.c_char_p
        _lib = lib
        return lib


def _check(status: int) -> None:
    if status != 0:
        msg = load_library().fp8bs_status_str(status).decode()
        raise Fp8bsError(msg)


def _stream_ptr(t: torch.Tensor) -> int:
    return torch.cuda.current_stream(t.device).cuda_stream


def _ptr(t: torch.Tensor | None) -> int | None:
    return None if t is None or t.numel() == 0 else t.data_ptr()


def _need(t: torch.Tensor, name: str, dtypes, ndim: int) -> None:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype not in (dtypes if isinstance(dtypes, tuple) else (dtypes,)):
        raise TypeError(f"{name}: dtype {t.dtype} not accepted ({dtypes})")
    if t.dim() != ndim:
        raise ValueError(f"{name}: expected {ndim} dims, got {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be on a GPU")


def _same_device(*ts: torch.Tensor) -> None:
    dev = ts[0].device
    for t in ts[1:]:
        if t.device != dev:
            raise ValueError("all tensors must be on the same device")


# ---- raw pointer entry points (used by tests of the ABI itself) ------------------------
def quantize_raw(x_ptr, rows, cols, q_ptr, s_ptr, stream=None) -> int:
    return load_library().fp8bs_quantize(x_ptr, rows, cols, q_ptr, s_ptr, stream)


def gemm_raw(a_ptr, sa_ptr, b_ptr, sb_ptr, c_ptr, M, N, K, stream=None) -> int:
    return load_library().fp8bs_gemm(a_ptr, sa_ptr, b_ptr, sb_ptr, c_ptr, M, N, K, stream)


def quantize_tg_raw(x_ptr, rows, cols, q_ptr, s_ptr, stream=None) -> int:
    return load_library().fp8bs_quantize_tg(x_ptr, rows, cols, q_ptr, s_ptr, stream)


def gemm_tg_raw(a_ptr, sa_ptr, b_ptr, sb_ptr, c_ptr, M, N, K, stream=None) -> int:
    return load_library().fp8bs_gemm_tg(a_ptr, sa_ptr, b_ptr, sb_ptr, c_ptr, M, N, K, stream)


def gemm_tg_nt_raw(a_ptr, sa_ptr, bt_ptr, sbt_ptr, c_ptr, M, N, K, stream=None) -> int:
    return load_library().fp8bs_gemm_tg_nt(a_ptr, sa_ptr, bt_ptr, sbt_ptr, c_ptr, M, N, K, stream)


def rmsnorm_quantize_tg_raw(x_ptr, res_ptr, gamma_ptr, eps, rows, d, q_ptr, s_ptr, y_ptr, stream=None) -> int:
    return load_library().fp8bs_rmsnorm_quantize_tg(x_ptr, res_ptr, gamma_ptr, eps, rows, d, q_ptr, s_ptr, y_ptr,
                                                    stream)


def quantize_e8m0_raw(x_ptr, rows, cols, q_ptr, e_ptr, stream=None) -> int:
    return load_library().fp8bs_quantize_e8m0(x_ptr, rows, cols, q_ptr, e_ptr, stream)


def gemm_e8m0_nt_raw(a_ptr, ea_ptr, bt_ptr, ebt_ptr, c_ptr, M, N, K, stream=None) -> int:
    return load_library().fp8bs_gemm_e8m0_nt(a_ptr, ea_ptr, bt_ptr, ebt_ptr, c_ptr, M, N, K, stream)


def gemm_nt_raw(a_ptr, sa_ptr, bt_ptr, sbt_ptr, c_ptr, M, N, K, stream=None) -> int:
    return load_library().fp8bs_gemm_nt(a_ptr, sa_ptr, bt_ptr, sbt_ptr, c_ptr, M, N, K, stream)


def grouped_gemm_nt_raw(a_ptr, sa_ptr, bt_ptr, sbt_ptr, off_ptr, G, c_ptr, M_total, N, K, stream=None) -> int:
    return load_library().fp8bs_grouped_gemm_nt(a_ptr, sa_ptr, bt_ptr, sbt_ptr, off_ptr, G, c_ptr, M_total, N, K,
                                                stream)


def grouped_gemm_raw(a_ptr, sa_ptr, b_ptr, sb_ptr, off_ptr, G, c_ptr, M_total, N, K, stream=None) -> int:
    return load_library().fp8bs_grouped_gemm(a_ptr, sa_ptr, b_ptr, sb_ptr, off_ptr, G, c_ptr, M_total, N, K, stream)


# ---- tensor entry points -----------------------------------------------------------------
def quantize(x: torch.Tensor, q: torch.Tensor | None = None, scales: torch.Tensor | None = None):
    """bf16 [R, C] -> (E4M3 codes uint8 [R, C], fp32 scales [ceil(R/32), C/32])."""
    _need(x, "x", torch.bfloat16, 2)
    R, C = x.shape
    if q is None:
        q = torch.empty((R, C), dtype=torch.uint8, device=x.device)
    if scales is None:
        scales = torch.empty(((R + BLOCK - 1) // BLOCK, C // BLOCK), dtype=torch.float32, device=x.device)
    _need(q, "q", E4M3_DTYPES, 2)
    _need(scales, "scales", torch.float32, 2)
    _same_device(x, q, scales)
    if tuple(q.shape) != (R, C) or tuple(scales.shape) != ((R + BLOCK - 1) // BLOCK, C // BLOCK):
        raise ValueError("output shapes do not match the input")
    _check(quantize_raw(_ptr(x), R, C, _ptr(q), _ptr(scales), _stream_ptr(x)))
    return q, scales


def gemm(a: torch.Tensor, sa: torch.Tensor, b: torch.Tensor, sb: torch.Tensor, out: torch.Tensor | None = None):
    """E4M3 a [M, K], sa [ceil(M/32), K/32], b [K, N], sb [K/32, N/32] -> bf16 [M, N]."""
    _need(a, "a", E4M3_DTYPES, 2)
    _need(b, "b", E4M3_DTYPES, 2)
    _need(sa, "sa", torch.float32, 2)
    _need(sb, "sb", torch.float32, 2)
    M, K = a.shape
    K2, N = b.shape
    if K2 != K:
        raise ValueError(f"inner dimensions differ: {K} vs {K2}")
    if tuple(sa.shape) != ((M + BLOCK - 1) // BLOCK, K // BLOCK) or tuple(sb.shape) != (K // BLOCK, N // BLOCK):
        raise ValueError("scale grid shapes do not match the operands")
    if out is None:
        out = torch.empty((M, N), dtype=torch.bfloat16, device=a.device)
    _need(out, "out", torch.bfloat16, 2)
    if tuple(out.shape) != (M, N):
        raise ValueError("out has the wrong shape")
    _same_device(a, sa, b, sb, out)
    _check(gemm_raw(_ptr(a), _ptr(sa), _ptr(b), _ptr(sb), _ptr(out), M, N, K, _stream_ptr(a)))
    return out


def grouped_gemm(a: torch.Tensor, sa: torch.Tensor, b: torch.Tensor, sb: torch.Tensor, offsets: torch.Tensor,
                 out: torch.Tensor | None = None):
    """a [M_total, K], sa [M_total/32, K/32], b [G, K, N], sb [G, K/32, N/32], offsets int32 [G+1] on device."""
    _need(a, "a", E4M3_DTYPES, 2)
    _need(b, "b", E4M3_DTYPES, 3)
    _need(sa, "sa", torch.float32, 2)
    _need(sb, "sb", torch.float32, 3)
    _need(offsets, "offsets", torch.int32, 1)
    M, K = a.shape
    G, K2, N = b.shape
    if K2 != K or offsets.shape[0] != G + 1:
        raise ValueError("shape mismatch between a, b and offsets")
    if tuple(sa.shape) != (M // BLOCK, K // BLOCK) or tuple(sb.shape) != (G, K // BLOCK, N // BLOCK):
        raise ValueError("scale grid shapes do not match the operands")
    if out is None:
        out = torch.empty((M, N), dtype=torch.bfloat16, device=a.device)
    _need(out, "out", torch.bfloat16, 2)
    if tuple(out.shape) != (M, N):
        raise ValueError("out has the wrong shape")
    _same_device(a, sa, b, sb, offsets, out)
    _check(grouped_gemm_raw(_ptr(a), _ptr(sa), _ptr(b), _ptr(sb), _ptr(offsets), G, _ptr(out), M, N, K,
                            _stream_ptr(a)))
    return out


def gemm_nt(a: torch.Tensor, sa: torch.Tensor, bt: torch.Tensor, sbt: torch.Tensor,
            out: torch.Tensor | None = None):
    """K-major weight: E4M3 a [M, K], sa [ceil(M/32), K/32], bt [N, K], sbt [N/32, K/32] -> bf16 [M, N]."""
    _need(a, "a", E4M3_DTYPES, 2)
    _need(bt, "bt", E4M3_DTYPES, 2)
    _need(sa, "sa", torch.float32, 2)
    _need(sbt, "sbt", torch.float32, 2)
    M, K = a.shape
    N, K2 = bt.shape
    if K2 != K:
        raise ValueError(f"inner dimensions differ: {K} vs {K2}")
    if tuple(sa.shape) != ((M + BLOCK - 1) // BLOCK, K // BLOCK) or tuple(sbt.shape) != (N // BLOCK, K // BLOCK):
        raise ValueError("scale grid shapes do not match the operands")
    if out is None:
        out = torch.empty((M, N), dtype=torch.bfloat16, device=a.device)
    _need(out, "out", torch.bfloat16, 2)
    if tuple(out.shape) != (M, N):
        raise ValueError("out has the wrong shape")
    _same_device(a, sa, bt, sbt, out)
    _check(gemm_nt_raw(_ptr(a), _ptr(sa), _ptr(bt), _ptr(sbt), _ptr(out), M, N, K, _stream_ptr(a)))
    return out


def grouped_gemm_nt(a: torch.Tensor, sa: torch.Tensor, bt: torch.Tensor, sbt: torch.Tensor, offsets: torch.Tensor,
                    out: torch.Tensor | None = None):
    """a [M_total, K], sa [M_total/32, K/32], bt [G, N, K], sbt [G, N/32, K/32], offsets int32 [G+1] on device."""
    _need(a, "a", E4M3_DTYPES, 2)
    _need(bt, "bt", E4M3_DTYPES, 3)
    _need(sa, "sa", torch.float32, 2)
    _need(sbt, "sbt", torch.float32, 3)
    _need(offsets, "offsets", torch.int32, 1)
    M, K = a.shape
    G, N, K2 = bt.shape
    if K2 != K or offsets.shape[0] != G + 1:
        raise ValueError("shape mismatch between a, bt and offsets")
    if tuple(sa.shape) != (M // BLOCK, K // BLOCK) or tuple(sbt.shape) != (G, N // BLOCK, K // BLOCK):
        raise ValueError("scale grid shapes do not match the operands")
    if out is None:
        out = torch.empty((M, N), dtype=torch.bfloat16, device=a.device)
    _need(out, "out", torch.bfloat16, 2)
    if tuple(out.shape) != (M, N):
        raise ValueError("out has the wrong shape")
    _same_device(a, sa, bt, sbt, offsets, out)
    _check(grouped_gemm_nt_raw(_ptr(a), _ptr(sa), _ptr(bt), _ptr(sbt), _ptr(offsets), G, _ptr(out), M, N, K,
                               _stream_ptr(a)))
    return out


def quantize_tg(x: torch.Tensor, q: torch.Tensor | None = None, scales: torch.Tensor | None = None):
    """bf16 [R, C] -> (E4M3 codes uint8 [R, C], fp32 per-token-group scales [R, C/32])."""
    _need(x, "x", torch.bfloat16, 2)
    R, C = x.shape
    if q is None:
        q = torch.empty((R, C), dtype=torch.uint8, device=x.device)
    if scales is None:
        scales = torch.empty((R, C // BLOCK), dtype=torch.float32, device=x.device)
    _need(q, "q", E4M3_DTYPES, 2)
    _need(scales, "scales", torch.float32, 2)
    _same_device(x, q, scales)
    if tuple(q.shape) != (R, C) or tuple(scales.shape) != (R, C // BLOCK):
        raise ValueError("output shapes do not match the input")
    _check(quantize_tg_raw(_ptr(x), R, C, _ptr(q), _ptr(scales), _stream_ptr(x)))
    return q, scales


def _gemm_tg_checked(raw, a, sa_rows, w, sw, out, k_major):
    _need(a, "a", E4M3_DTYPES, 2)
    _need(w, "b", E4M3_DTYPES, 2)
    _need(sa_rows, "sa_rows", torch.float32, 2)
    _need(sw, "sb", torch.float32, 2)
    M, K = a.shape
    if k_major:
        N, K2 = w.shape
        sw_shape = (N // BLOCK, K // BLOCK)
    else:
        K2, N = w.shape
        sw_shape = (K // BLOCK, N // BLOCK)
    if K2 != K:
        raise ValueError(f"inner dimensions differ: {K} vs {K2}")
    if tuple(sa_rows.shape) != (M, K // BLOCK) or tuple(sw.shape) != sw_shape:
        raise ValueError("scale grid shapes do not match the operands")
    if out is None:
        out = torch.empty((M, N), dtype=torch.bfloat16, device=a.device)
    _need(out, "out", torch.bfloat16, 2)
    if tuple(out.shape) != (M, N):
        raise ValueError("out has the wrong shape")
    _same_device(a, sa_rows, w, sw, out)
    _check(raw(_ptr(a), _ptr(sa_rows), _ptr(w), _ptr(sw), _ptr(out), M, N, K, _stream_ptr(a)))
    return out


def gemm_tg(a: torch.Tensor, sa_rows: torch.Tensor, b: torch.Tensor, sb: torch.Tensor,
            out: torch.Tensor | None = None):
    """E4M3 a [M, K] with per-token-group scales sa_rows [M, K/32], b [K, N], sb [K/32, N/32] -> bf16 [M, N]."""
    return _gemm_tg_checked(gemm_tg_raw, a, sa_rows, b, sb, out, False)


def gemm_tg_nt(a: torch.Tensor, sa_rows: torch.Tensor, bt: torch.Tensor, sbt: torch.Tensor,
               out: torch.Tensor | None = None):
    """As gemm_tg with the weight K-major: bt [N, K], sbt [N/32, K/32]."""
    return _gemm_tg_checked(gemm_tg_nt_raw, a, sa_rows, bt, sbt, out, True)


def rmsnorm_quantize_tg(x: torch.Tensor, gamma: torch.Tensor, eps: float, residual: torch.Tensor | None = None,
                        q: torch.Tensor | None = None, scales: torch.Tensor | None = None,
                        y: torch.Tensor | None = None, want_y: bool = False):
    """Residual add (in place on ``residual`` when given) + RMSNorm + per-token-group
    quantization of bf16 x [R, d] with weight gamma [d].

    Returns (q uint8 [R, d], scales fp32 [R, d/32]), plus the bf16 normalised rows
    [R, d] as a third element when ``want_y`` is true or ``y`` is given."""
    _need(x, "x", torch.bfloat16, 2)
    _need(gamma, "gamma", torch.bfloat16, 1)
    R, d = x.shape
    if gamma.shape[0] != d:
        raise ValueError(f"gamma has {gamma.shape[0]} entries, rows have {d}")
    if residual is not None:
        _need(residual, "residual", torch.bfloat16, 2)
        if tuple(residual.shape) != (R, d):
            raise ValueError("residual has the wrong shape")
    if q is None:
        q = torch.empty((R, d), dtype=torch.uint8, device=x.device)
    if scales is None:
        scales = torch.empty((R, d // BLOCK), dtype=torch.float32, device=x.device)
    if y is None and want_y:
        y = torch.empty((R, d), dtype=torch.bfloat16, device=x.device)
    _need(q, "q", E4M3_DTYPES, 2)
    _need(scales, "scales", torch.float32, 2)
    if tuple(q.shape) != (R, d) or tuple(scales.shape) != (R, d // BLOCK):
        raise ValueError("output shapes do not match the input")
    if y is not None:
        _need(y, "y", torch.bfloat16, 2)
        if tuple(y.shape) != (R, d):
            raise ValueError("y has the wrong shape")
    _same_device(*[t for t in (x, gamma, residual, q, scales, y) if t is not None])
    _check(rmsnorm_quantize_tg_raw(_ptr(x), _ptr(residual), _ptr(gamma), float(eps), R, d, _ptr(q), _ptr(scales),
                                   _ptr(y), _stream_ptr(x)))
    return (q, scales) if y is None else (q, scales, y)


def quantize_e8m0(x: torch.Tensor, q: torch.Tensor | None = None, e8m0: torch.Tensor | None = None):
    """bf16 [R, C] -> (E4M3 codes uint8 [R, C], E8M0 exponent bytes uint8 [ceil(R/32), C/32])."""
    _need(x, "x", torch.bfloat16, 2)
    R, C = x.shape
    if q is None:
        q = torch.empty((R, C), dtype=torch.uint8, device=x.device)
    if e8m0 is None:
        e8m0 = torch.empty(((R + BLOCK - 1) // BLOCK, C // BLOCK), dtype=torch.uint8, device=x.device)
    _need(q, "q", E4M3_DTYPES, 2)
    _need(e8m0, "e8m0", torch.uint8, 2)
    _same_device(x, q, e8m0)
    if tuple(q.shape) != (R, C) or tuple(e8m0.shape) != ((R + BLOCK - 1) // BLOCK, C // BLOCK):
        raise ValueError("output shapes do not match the input")
    _check(quantize_e8m0_raw(_ptr(x), R, C, _ptr(q), _ptr(e8m0), _stream_ptr(x)))
    return q, e8m0


def gemm_e8m0_nt(a: torch.Tensor, ea: torch.Tensor, bt: torch.Tensor, ebt: torch.Tensor,
                 out: torch.Tensor | None = None):
    """E4M3 a [M, K] with E8M0 bytes ea [ceil(M/32), K/32], bt [N, K] with ebt [N/32, K/32] -> bf16 [M, N]."""
    _need(a, "a", E4M3_DTYPES, 2)
    _need(bt, "bt", E4M3_DTYPES, 2)
    _need(ea, "ea", torch.uint8, 2)
    _need(ebt, "ebt", torch.uint8, 2)
    M, K = a.shape
    N, K2 = bt.shape
    if K2 != K:
        raise ValueError(f"inner dimensions differ: {K} vs {K2}")
    if tuple(ea.shape) != ((M + BLOCK - 1) // BLOCK, K // BLOCK) or tuple(ebt.shape) != (N // BLOCK, K // BLOCK):
        raise ValueError("exponent grid shapes do not match the operands")
    if out is None:
        out = torch.empty((M, N), dtype=torch.bfloat16, device=a.device)
    _need(out, "out", torch.bfloat16, 2)
    if tuple(out.shape) != (M, N):
        raise ValueError("out has the wrong shape")
    _same_device(a, ea, bt, ebt, out)
    _check(gemm_e8m0_nt_raw(_ptr(a), _ptr(ea), _ptr(bt), _ptr(ebt), _ptr(out), M, N, K, _stream_ptr(a)))
    return out
