"""FP8 (E4M3) GEMM with 32x32 block scales for AMD MI355X (gfx950).

The compute path is the C-ABI library ``libfp8bs.so`` (HIP kernels); the
functions exported here only marshal torch tensors into it.  Importing this
package loads nothing; the first call loads the library and raises
``Fp8bsError`` if it is missing.
"""

_BINDING_NAMES = ("Fp8bsError", "quantize", "gemm", "grouped_gemm", "gemm_nt", "grouped_gemm_nt", "quantize_tg",
                  "gemm_tg", "gemm_tg_nt", "library_path", "load_library", "quantize_raw", "gemm_raw",
                  "grouped_gemm_raw", "gemm_nt_raw", "grouped_gemm_nt_raw", "quantize_tg_raw", "gemm_tg_raw",
                  "gemm_tg_nt_raw", "rmsnorm_quantize_tg", "rmsnorm_quantize_tg_raw",
                  "quantize_e8m0", "gemm_e8m0_nt", "quantize_e8m0_raw", "gemm_e8m0_nt_raw")

__all__ = list(_BINDING_NAMES)


def __getattr__(name):
    if name in _BINDING_NAMES:
        from . import binding
        return getattr(binding, name)
    raise AttributeError(name)
