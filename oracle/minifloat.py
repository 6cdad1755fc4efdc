"""Generic binary floating-point formats from their bit fields (test oracle only).

One small class describes a sign / exponent / mantissa format.  ``decode`` turns
codes into exact fp64 values straight from the bit-field formula; ``encode``
rounds fp32/fp64 values to the nearest representable value, ties going to the
code whose last mantissa bit is 0 (round half to even).  Three instances exist:

* ``E4M3FN`` - 4 exponent bits, 3 mantissa bits, largest finite value 448, no
  infinity (DeepGEMM write-up, section 2.1: the forward-pass FP8 format with a
  448 ceiling).  Only S.1111.111 is NaN.  Overflow saturates to +-448.
* ``FP16``   - IEEE binary16, used only to pin the rounding rule against the
  Determinism article's FP16 encoding table and its 2048 + 1 -> 2048 example.
* ``BF16``   - bfloat16, used only to pin the encoder against a bit-level
  fp32 -> bf16 rounding written independently in the tests.

Nothing here is fast; everything is exact (all compared quantities are exactly
representable in fp64 for these formats).
"""

from __future__ import annotations

import numpy as np


class Minifloat:
    def __init__(self, name: str, exp_bits: int, man_bits: int, bias: int, ieee_specials: bool):
        self.name = name
        self.e = exp_bits
        self.m = man_bits
        self.bias = bias
        # ieee_specials: all-ones exponent is inf/NaN (IEEE).  Otherwise (the
        # "FN" convention) only all-ones exponent AND all-ones mantissa is NaN.
        self.ieee = ieee_specials
        self.nbits = 1 + exp_bits + man_bits
        self.sign_bit = 1 << (exp_bits + man_bits)
        # table of non-negative finite magnitudes in code order (monotone)
        codes = np.arange(self.sign_bit, dtype=np.int64)
        vals = self.decode(codes)
        finite = np.isfinite(vals)
        self._pos_codes = codes[finite]
        self._pos_vals = vals[finite]
        assert np.all(np.diff(self._pos_vals) > 0), "codes must be monotone in value"
        self.max_finite = float(self._pos_vals[-1])

    # ---- decode: the bit-field formula -------------------------------------------------
    def decode(self, codes) -> np.ndarray:
        c = np.asarray(codes, dtype=np.int64)
        s = np.where(c & self.sign_bit, -1.0, 1.0)
        E = (c >> self.m) & ((1 << self.e) - 1)
        M = c & ((1 << self.m) - 1)
        frac = M.astype(np.float64) / float(1 << self.m)
        normal = (1.0 + frac) * np.exp2((E - self.bias).astype(np.float64))
        subnormal = frac * np.exp2(float(1 - self.bias))
        v = s * np.where(E == 0, subnormal, normal)
        emax = (1 << self.e) - 1
        if self.ieee:
            v = np.where((E == emax) & (M == 0), s * np.inf, v)
            v = np.where((E == emax) & (M != 0), np.nan, v)
        else:
            v = np.where((E == emax) & (M == (1 << self.m) - 1), np.nan, v)
        return v

    # ---- encode: nearest representable value, ties to even ------------------------------
    def encode(self, x, overflow: str = "saturate") -> np.ndarray:
        """Round ``x`` (fp32 or fp64 array) to this format; returns integer codes.

        ``overflow='saturate'`` clamps magnitudes beyond the largest finite value to
        it; ``overflow='inf'`` (IEEE formats only) lets them round to infinity by the
        usual rule (the halfway point above the largest finite value rounds up, since
        the largest finite value has an odd mantissa).
        """
        x = np.asarray(x, dtype=np.float64)
        neg = np.signbit(x)
        a = np.abs(x)
        vals, codes = self._pos_vals, self._pos_codes
        if overflow == "saturate":
            a = np.minimum(a, self.max_finite)
            top_val = None
        elif overflow == "inf":
            assert self.ieee
            # the next power of two above max_finite plays the role of the next value
            top_val = float(2.0 ** ((1 << self.e) - 1 - self.bias))
        else:
            raise ValueError(overflow)
        # index of the largest table value <= a
        lo = np.searchsorted(vals, a, side="right") - 1
        lo = np.clip(lo, 0, len(vals) - 1)
        v_lo = vals[lo]
        c_lo = codes[lo]
        at_top = lo == len(vals) - 1
        hi = np.minimum(lo + 1, len(vals) - 1)
        v_hi = np.where(at_top, top_val if top_val is not None else vals[-1], vals[hi])
        inf_code = ((1 << self.e) - 1) << self.m
        c_hi = np.where(at_top, inf_code if top_val is not None else codes[-1], codes[hi])
        mid = (v_lo + v_hi) / 2.0  # exact: both are short binary fractions
        pick_hi = (a > mid) | ((a == mid) & ((c_lo & 1) == 1))
        pick_hi &= v_hi > v_lo
        out = np.where(pick_hi, c_hi, c_lo)
        out = np.where(neg, out | self.sign_bit, out)
        nan_code = ((1 << (self.e + self.m)) - 1) | self.sign_bit
        out = np.where(np.isnan(x), nan_code, out)
        return out.astype(np.int64)


E4M3FN = Minifloat("e4m3fn", 4, 3, 7, ieee_specials=False)
FP16 = Minifloat("fp16", 5, 10, 15, ieee_specials=True)
BF16 = Minifloat("bf16", 8, 7, 127, ieee_specials=True)
