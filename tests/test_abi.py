"""The C ABI loads, exports what include/fp8bs.h declares, and rejects bad
arguments on the host before any launch (CPU only: no GPU call is made)."""

import ctypes
import os
import re

import pytest

from fp8_block_scaled_03_amd import binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
OK, EINVAL, ESHAPE, EALIGN = 0, 1, 2, 3
A16 = 0x10000          # fake, 16-byte aligned "device" addresses: never dereferenced
A4 = 0x10004


def _declared_functions():
    text = open(os.path.join(ROOT, "include", "fp8bs.h")).read()
    return sorted(set(re.findall(r"\b(fp8bs_[a-z0-9_]+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    lib = binding.load_library()
    names = _declared_functions()
    assert names == ["fp8bs_gemm", "fp8bs_gemm_e8m0_nt", "fp8bs_gemm_nt", "fp8bs_gemm_tg", "fp8bs_gemm_tg_nt",
                     "fp8bs_grouped_gemm", "fp8bs_grouped_gemm_nt", "fp8bs_quantize", "fp8bs_quantize_e8m0",
                     "fp8bs_quantize_tg", "fp8bs_rmsnorm_quantize_tg", "fp8bs_status_str"]
    for n in names:
        assert hasattr(lib, n), n


def test_probe_library_exports_every_declared_symbol_and_checks_arguments():
    """libfp8bs_probe.so (measurement and test support) exports what
    include/fp8bs_probe.h declares and rejects bad sizes before any launch."""
    from fp8_block_scaled_03_amd import probe
    lib = probe.load_probe_library()
    text = open(os.path.join(ROOT, "include", "fp8bs_probe.h")).read()
    names = sorted(set(re.findall(r"\b(fp8bs_probe_[a-z0-9_]+)\s*\(", text)))
    assert names == ["fp8bs_probe_gemm", "fp8bs_probe_mfma_scale", "fp8bs_probe_promote_ceiling",
                     "fp8bs_probe_stream_read"]
    for n in names:
        assert hasattr(lib, n), n
    assert lib.fp8bs_probe_gemm(A16, A4, A16, A4, A16, None, 48, 64, 64, 0, None) == 2     # M % 32
    assert lib.fp8bs_probe_gemm(None, A4, A16, A4, A16, None, 64, 64, 64, 0, None) == 1
    assert lib.fp8bs_probe_mfma_scale(A16, A16, A16, A16, A4, A4, 0, None) == 2
    assert lib.fp8bs_probe_promote_ceiling(None, 1, 1, 0, None) == 1
    assert lib.fp8bs_probe_promote_ceiling(A4, 1, 1, 4, None) == 2                        # burst mode, odd iters
    assert lib.fp8bs_probe_promote_ceiling(A4, 1, 2, 9, None) == 2                        # no mode 9
    assert lib.fp8bs_probe_stream_read(A16, 24, A4, 1, None) == 2                          # bytes % 16


def test_status_strings():
    lib = binding.load_library()
    for code in range(6):
        s = lib.fp8bs_status_str(code).decode()
        assert s.startswith(binding.STATUS[code])
    assert lib.fp8bs_status_str(99).decode()


@pytest.mark.parametrize("q", [binding.quantize_raw, binding.quantize_tg_raw])
def test_quantize_argument_checks(q):
    assert q(A16, 0, 64, A16, A4) == OK            # empty: no-op
    assert q(A16, 5, 0, A16, A4) == OK
    assert q(A16, -1, 64, A16, A4) == EINVAL
    assert q(A16, 4, 48, A16, A4) == ESHAPE         # cols % 32
    assert q(None, 4, 64, A16, A4) == EINVAL
    assert q(A16, 4, 64, None, A4) == EINVAL
    assert q(A16, 4, 64, A16, None) == EINVAL
    assert q(A16 + 8, 4, 64, A16, A4) == EALIGN
    assert q(A16, 4, 64, A16 + 4, A4) == EALIGN
    assert q(A16, 4, 64, A16, A4 + 1) == EALIGN
    assert q(A16, 1 << 31, 64, A16, A4) == ESHAPE


def test_gemm_argument_checks():
    g = binding.gemm_raw
    assert g(A16, A4, A16, A4, A16, 0, 64, 64) == OK      # M == 0: no-op
    assert g(A16, A4, A16, A4, A16, 4, 0, 64) == OK       # N == 0: no-op
    assert g(A16, A4, A16, A4, A16, -4, 64, 64) == EINVAL
    assert g(A16, A4, A16, A4, A16, 4, 64, 48) == ESHAPE  # K % 32
    assert g(A16, A4, A16, A4, A16, 4, 40, 64) == ESHAPE  # N % 32
    assert g(None, A4, A16, A4, A16, 4, 64, 64) == EINVAL
    assert g(A16, None, A16, A4, A16, 4, 64, 64) == EINVAL
    assert g(A16, A4, None, A4, A16, 4, 64, 64) == EINVAL
    assert g(A16, A4, A16, None, A16, 4, 64, 64) == EINVAL
    assert g(A16, A4, A16, A4, None, 4, 64, 64) == EINVAL
    assert g(A16 + 1, A4, A16, A4, A16, 4, 64, 64) == EALIGN
    assert g(A16, A4 + 2, A16, A4, A16, 4, 64, 64) == EALIGN
    assert g(A16, A4, A16, A4, A16 + 8, 4, 64, 64) == EALIGN
    assert g(A16, A4, A16, A4, A16, 4, 64, (1 << 30) + 32) == ESHAPE


@pytest.mark.parametrize("g", [binding.gemm_raw, binding.gemm_nt_raw, binding.gemm_tg_raw, binding.gemm_tg_nt_raw])
def test_gemm_argument_checks_all_variants(g):
    assert g(A16, A4, A16, A4, A16, 0, 64, 64) == OK
    assert g(A16, A4, A16, A4, A16, 4, 64, 48) == ESHAPE
    assert g(A16, A4, A16, A4, A16, 4, 40, 64) == ESHAPE
    assert g(A16, A4, None, A4, A16, 4, 64, 64) == EINVAL
    assert g(A16, A4, A16, None, A16, 4, 64, 64) == EINVAL
    assert g(A16, A4, A16 + 8, A4, A16, 4, 64, 64) == EALIGN
    assert g(A16, A4, A16, A4 + 1, A16, 4, 64, 64) == EALIGN


@pytest.mark.parametrize("g", [binding.grouped_gemm_raw, binding.grouped_gemm_nt_raw])
def test_grouped_argument_checks(g):
    assert g(A16, A4, A16, A4, A4, 0, A16, 64, 64, 64) == EINVAL      # G < 1
    assert g(A16, A4, A16, A4, A4, 1025, A16, 64, 64, 64) == EINVAL   # G > max
    assert g(A16, A4, A16, A4, None, 2, A16, 64, 64, 64) == EINVAL    # no offsets
    assert g(A16, A4, A16, A4, A4 + 1, 2, A16, 64, 64, 64) == EALIGN
    assert g(A16, A4, A16, A4, A4, 2, A16, 48, 64, 64) == ESHAPE      # M_total % 32
    assert g(A16, A4, A16, A4, A4, 2, A16, 64, 40, 64) == ESHAPE
    assert g(A16, A4, A16, A4, A4, 2, A16, 0, 64, 64) == OK           # empty
    assert g(A16, A4, A16, A4, A4, 2, None, 64, 64, 64) == EINVAL


def test_e8m0_argument_checks():
    q = binding.quantize_e8m0_raw
    assert q(A16, 0, 64, A16, A4) == OK
    assert q(A16, 4, 48, A16, A4) == ESHAPE
    assert q(None, 4, 64, A16, A4) == EINVAL
    assert q(A16, 4, 64, A16, None) == EINVAL
    assert q(A16 + 8, 4, 64, A16, A4) == EALIGN
    g = binding.gemm_e8m0_nt_raw
    assert g(A16, A4, A16, A4, A16, 0, 64, 128) == OK
    assert g(A16, A4, A16, A4, A16, 4, 64, 96) == ESHAPE      # K % 128
    assert g(A16, A4, A16, A4, A16, 4, 40, 128) == ESHAPE     # N % 32
    assert g(A16, None, A16, A4, A16, 4, 64, 128) == EINVAL
    assert g(A16, A4, A16, A4 + 1, A16, 4, 64, 128) == EALIGN
    assert g(A16 + 4, A4, A16, A4, A16, 4, 64, 128) == EALIGN


def test_rmsnorm_quantize_argument_checks():
    r = binding.rmsnorm_quantize_tg_raw
    # x, residual, gamma, eps, rows, d, q, scales, y
    assert r(A16, None, A16, 1e-6, 0, 64, A16, A4, None) == OK            # empty: no-op
    assert r(A16, None, A16, 1e-6, 4, 0, A16, A4, None) == OK
    assert r(A16, None, A16, 1e-6, -1, 64, A16, A4, None) == EINVAL
    assert r(A16, None, A16, -1.0, 4, 64, A16, A4, None) == EINVAL        # eps < 0
    assert r(A16, None, A16, float("nan"), 4, 64, A16, A4, None) == EINVAL
    assert r(A16, None, A16, float("inf"), 4, 64, A16, A4, None) == EINVAL
    assert r(A16, None, A16, 1e-6, 4, 48, A16, A4, None) == ESHAPE        # d % 32
    assert r(A16, None, A16, 1e-6, 4, 16384 + 32, A16, A4, None) == ESHAPE  # d too large
    assert r(None, None, A16, 1e-6, 4, 64, A16, A4, None) == EINVAL
    assert r(A16, None, None, 1e-6, 4, 64, A16, A4, None) == EINVAL
    assert r(A16, None, A16, 1e-6, 4, 64, None, A4, None) == EINVAL
    assert r(A16, None, A16, 1e-6, 4, 64, A16, None, None) == EINVAL
    assert r(A16 + 2, None, A16, 1e-6, 4, 64, A16, A4, None) == EALIGN
    assert r(A16, A16 + 8, A16, 1e-6, 4, 64, A16, A4, None) == EALIGN     # residual
    assert r(A16, None, A16 + 4, 1e-6, 4, 64, A16, A4, None) == EALIGN
    assert r(A16, None, A16, 1e-6, 4, 64, A16 + 8, A4, None) == EALIGN
    assert r(A16, None, A16, 1e-6, 4, 64, A16, A4 + 2, None) == EALIGN
    assert r(A16, None, A16, 1e-6, 4, 64, A16, A4, A16 + 8) == EALIGN     # y


def test_tensor_api_rejects_bad_inputs_without_gpu():
    import torch
    with pytest.raises(TypeError):
        binding.quantize(torch.zeros(4, 32, dtype=torch.float32))
    with pytest.raises(ValueError):
        binding.quantize(torch.zeros(4, 32, dtype=torch.bfloat16))   # not on a GPU


def test_missing_library_fails_loudly(monkeypatch):
    monkeypatch.setattr(binding, "_lib", None)
    monkeypatch.setenv("FP8BS_LIBRARY", "/nonexistent/libfp8bs.so")
    with pytest.raises(binding.Fp8bsError):
        binding.load_library()
