"""CPU oracle for the FP8 (E4M3) GEMM with 32x32 block scales.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package.  The product path
(the HIP library and its Python binding) never imports, calls or links it, and
this package never imports the product package: the two share no code.

Everything here is plain numpy (fp64 where the arithmetic is floating point,
exact integers / fractions where the result must be exact).  Each function
cites the passage of the source pages it follows:

* "DeepGEMM write-up" = the featured DeepGEMM FP8 article on hncyxsy.com
  (news item 241433), sections 2.1-2.3 (E4M3 format, 32x32 block scales, scale
  applied inside the GEMM), 4.1-4.3 (grouped GEMM), 5.2 (absmax scaling) and 6
  (call interface).
* "Determinism article" = "AI Infra 进阶：如何让大模型输出确定的结果"
  (aif.amtbbs.org, post 29992): introduction (FP16 encoding table and the
  round-half-to-even example), part 一 (GEMM batch invariance) and part 三
  (RMSNorm, its residual-add form and the per-token-group quantizer fused
  with it).
* "Triton-cutlass article" = "Triton内核命名嵌入Cutlass：自动调用FP8 Tensor
  Core GEMM路径..." (blog.hotdry.top, 2025-10-04): the tiled GEMM listing in the
  section on deployable parameters (a plain GEMM with fp32 accumulation).

Pins (tests marked ``not gpu``) tie every function to something other than
itself; no function here is "parity unpinned".
"""

from .minifloat import Minifloat, E4M3FN, FP16, BF16
from .e4m3 import decode_e4m3, encode_e4m3, FINITE_E4M3_CODES
from .quantize import quantize_blocks, quantize_token_groups, bf16_bits_to_f32, BLOCK
from .gemm import (dequantize, dequantize_token_groups, gemm_ref, gemm_ref_at, gemm_ref_nt, gemm_ref_tg,
                   gemm_ref_tg_nt, grouped_gemm_ref, grouped_gemm_ref_at, grouped_gemm_ref_nt, tolerance_ok,
                   tolerance_bound, bf16_bits_to_f64)
from .exact import gemm_exact
from .rmsnorm import residual_add, rmsnorm_ref, rmsnorm_tolerance_ok, RMS_REL_TOL, RMS_ABS_TOL
from .e8m0 import (e8m0_exponent, quantize_blocks_e8m0, dequantize_e8m0, gemm_ref_e8m0_nt, gemm_e8m0_bound_nt,
                   emulate_gemm_e8m0_nt, code_exponents, step_bound)

__all__ = [
    "Minifloat", "E4M3FN", "FP16", "BF16",
    "decode_e4m3", "encode_e4m3", "FINITE_E4M3_CODES",
    "quantize_blocks", "quantize_token_groups", "bf16_bits_to_f32", "BLOCK",
    "dequantize", "dequantize_token_groups", "gemm_ref", "gemm_ref_at", "gemm_ref_nt", "gemm_ref_tg",
    "gemm_ref_tg_nt", "grouped_gemm_ref", "grouped_gemm_ref_at",
    "grouped_gemm_ref_nt",
    "tolerance_ok", "tolerance_bound", "bf16_bits_to_f64",
    "gemm_exact",
    "residual_add", "rmsnorm_ref", "rmsnorm_tolerance_ok", "RMS_REL_TOL", "RMS_ABS_TOL",
    "e8m0_exponent", "quantize_blocks_e8m0", "dequantize_e8m0", "gemm_ref_e8m0_nt", "gemm_e8m0_bound_nt",
    "emulate_gemm_e8m0_nt", "code_exponents", "step_bound",
]
