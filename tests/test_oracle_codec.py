"""Pins for the oracle's floating-point codecs (CPU only).

Each test ties the oracle to something other than its own code: values printed
on the source pages, a library routine, an independent brute force, or a
closed form derived by hand.
"""

import os

import numpy as np
import pytest

from oracle import BF16, E4M3FN, FP16, FINITE_E4M3_CODES, decode_e4m3, encode_e4m3

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _read_fp16_table():
    rows, ties = [], []
    for line in open(os.path.join(GOLDEN, "fp16_encoding_table.txt")):
        line = line.split("#")[0].strip()
        if not line:
            continue
        f = line.split()
        if f[0] == "tie":
            ties.append((float(f[1]), float(f[2])))
        else:
            rows.append((float(f[0]), int(f[1]), f[2]))
    return rows, ties


def test_fp16_encoding_table_from_determinism_article():
    rows, ties = _read_fp16_table()
    assert len(rows) == 7 and len(ties) == 1
    for value, stored_exp, mant_bits in rows:
        code = int(FP16.encode(np.array([value]), overflow="inf")[0])
        assert (code >> 10) & 0x1F == stored_exp, value
        assert format(code & 0x3FF, "010b") == mant_bits, value
        assert FP16.decode(np.array([code]))[0] == value
    for exact, expected in ties:
        code = int(FP16.encode(np.array([exact]), overflow="inf")[0])
        assert FP16.decode(np.array([code]))[0] == expected


def test_fp16_matches_numpy_conversion():
    """The generic encoder instantiated as IEEE binary16 equals numpy's cast."""
    g = np.random.default_rng(1)
    x = (g.standard_normal(200000) * np.exp2(g.integers(-30, 20, 200000))).astype(np.float32)
    # every fp16 midpoint and its fp32 neighbours, both signs
    codes = np.arange(0x7C00, dtype=np.int64)
    v = FP16.decode(codes)
    mids = ((v[:-1] + v[1:]) / 2).astype(np.float32)
    x = np.concatenate([x, mids, np.nextafter(mids, 0), np.nextafter(mids, np.inf), -mids,
                        np.float32([65504, 65519.99, 65520, 65536, 1e9, 0.0, -0.0])])
    ours = FP16.encode(x.astype(np.float64), overflow="inf").astype(np.uint16)
    with np.errstate(over="ignore"):   # the values past 65519.99 overflow to inf on purpose
        ref = x.astype(np.float16).view(np.uint16)
    assert np.array_equal(ours, ref)


def _bf16_bits_rne(x):
    """Independent fp32 -> bf16 rounding done on the bit pattern."""
    u = x.astype(np.float32).view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    return ((u + 0x7FFF + lsb) >> 16).astype(np.uint16)


def test_bf16_matches_bit_rounding():
    g = np.random.default_rng(2)
    x = (g.standard_normal(200000) * np.exp2(g.integers(-120, 120, 200000))).astype(np.float32)
    x = np.concatenate([x, np.float32([1.00390625, 1.01171875, -1.00390625, 0.0, -0.0])])
    ours = BF16.encode(x.astype(np.float64), overflow="inf").astype(np.uint16)
    assert np.array_equal(ours, _bf16_bits_rne(x))


def test_e4m3_closed_form_values():
    # largest finite value 448 is printed (DeepGEMM write-up 2.1); the rest
    # follow from the 4/3 bit split with bias 7.
    v = decode_e4m3(np.arange(256))
    assert v[0x7E] == 448.0
    assert v[0x38] == 1.0
    assert v[0x01] == 2.0 ** -9            # smallest subnormal
    assert v[0x07] == 7 * 2.0 ** -9        # largest subnormal
    assert v[0x08] == 2.0 ** -6            # smallest normal
    assert v[0x7D] == 416.0
    assert v[0x80] == 0.0 and np.signbit(v[0x80])
    assert np.isnan(v[0x7F]) and np.isnan(v[0xFF])
    finite = np.isfinite(v)
    assert finite.sum() == 254 == len(FINITE_E4M3_CODES)
    assert np.nanmax(v) == 448.0 and np.nanmin(v) == -448.0
    # every value is an integer multiple of 2**-9
    units = v[finite] * 512
    assert np.array_equal(units, np.round(units))
    # positive codes are ordered by value
    assert np.all(np.diff(v[0:0x7F]) > 0)
    # sign symmetry
    assert np.array_equal(v[0x80:0xFF], -v[0x00:0x7F])


def test_e4m3_roundtrip_all_codes():
    vals = decode_e4m3(FINITE_E4M3_CODES).astype(np.float32)
    assert np.array_equal(encode_e4m3(vals), FINITE_E4M3_CODES)


def _e4m3_brute(t):
    """Nearest finite E4M3 code by scanning all 254 codes; ties -> even code.

    Saturates beyond +-448.  Distances are exact in fp64 for the inputs used.
    """
    t = np.asarray(t, dtype=np.float64)
    codes = np.arange(0, 0x7F)                 # non-negative finite codes
    vals = decode_e4m3(codes)
    a = np.minimum(np.abs(t), 448.0)
    d = np.abs(a[:, None] - vals[None, :])
    dmin = d.min(axis=1, keepdims=True)
    cand = d == dmin
    # among the nearest (at most two), prefer an even code
    even = cand & ((codes[None, :] & 1) == 0)
    pick = np.where(even.any(axis=1), even.argmax(axis=1), cand.argmax(axis=1))
    out = codes[pick]
    return np.where(np.signbit(t), out | 0x80, out).astype(np.uint8)


def test_e4m3_encode_matches_brute_force_on_all_bf16():
    # every bf16 bit pattern with magnitude <= 500 (exhaustive, both signs)
    bits = np.arange(0, 1 << 16, dtype=np.uint32)
    x = (bits << 16).view(np.float32)
    x = x[np.isfinite(x) & (np.abs(x) <= 500) & (np.abs(x) >= 2.0 ** -20)]
    x = np.concatenate([x, np.float32([0.0, -0.0, 2.0 ** -21, -(2.0 ** -21)])])
    assert np.array_equal(encode_e4m3(x), _e4m3_brute(x))


def test_e4m3_encode_matches_brute_force_near_midpoints():
    vals = decode_e4m3(np.arange(0, 0x7F))
    mids = ((vals[:-1] + vals[1:]) / 2).astype(np.float32)
    near = np.concatenate([mids, np.nextafter(mids, np.float32(0)), np.nextafter(mids, np.float32(1e9))])
    near = np.concatenate([near, -near, np.float32([448, 449, 463.99, 464, 464.01, 480, 1e6, -1e6])])
    assert np.array_equal(encode_e4m3(near), _e4m3_brute(near))


def test_e4m3_ties_go_to_even():
    # 1.0625 sits halfway between 1.0 (0x38, even) and 1.125 (0x39)
    assert encode_e4m3(np.float32([1.0625]))[0] == 0x38
    # 1.1875 sits halfway between 1.125 (0x39) and 1.25 (0x3A, even)
    assert encode_e4m3(np.float32([1.1875]))[0] == 0x3A
    # 464 sits halfway between 448 (0x7E) and the non-existent 480: saturates
    assert encode_e4m3(np.float32([464.0, -464.0, 1e30])).tolist() == [0x7E, 0xFE, 0x7E]


def test_e4m3_rejects_non_fp32():
    with pytest.raises(TypeError):
        encode_e4m3(np.array([1.0]))
