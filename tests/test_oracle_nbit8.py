"""Pins for the oracle's 8-bit storage modes, int8 and fp8 e4m3 (CPU only).

e4m3 values against the format's landmarks and an independent float32
bit-pattern construction; the quantisers against closed forms, exact ties and
brute force; round-trip bounds; the fidelity ordering of all modes.
"""

import numpy as np
import pytest

import oracle


def _e4m3_via_float32_bits(code):
    """Decode by building the float32 bit pattern (normals) or m * 2^-9."""
    c = int(code)
    s, e, m = c >> 7, (c >> 3) & 15, c & 7
    if e == 15 and m == 7:
        return np.nan
    if e == 0:
        v = m * 2.0 ** -9
    else:
        bits = np.uint32(((e - 7 + 127) << 23) | (m << 20))
        v = float(np.array([bits], dtype=np.uint32).view(np.float32)[0])
    return -v if s else v


def test_e4m3_values():
    got = oracle.e4m3_value(np.arange(256))
    want = np.array([_e4m3_via_float32_bits(c) for c in range(256)])
    assert np.array_equal(np.isnan(got), np.isnan(want))
    ok = ~np.isnan(want)
    assert np.array_equal(got[ok], want[ok])
    # landmarks of the format: 448 largest, 2^-6 smallest normal, 2^-9 the
    # smallest subnormal, 1.0 at 0x38, NaN at 0x7F / 0xFF
    assert got[0x7E] == 448.0 and got[0x08] == 2.0 ** -6 and got[0x01] == 2.0 ** -9
    assert got[0x38] == 1.0 and np.isnan(got[0x7F]) and np.isnan(got[0xFF])
    assert np.all(np.diff(got[:127]) > 0)


def test_int8_codes_closed_forms_and_ties():
    xn = np.array([1.0, -1.0, 0.0, -0.0, 0.5 / 127, 1.5 / 127, -2.5 / 127], dtype=np.float32)
    codes = oracle.int8_code(xn).view(np.int8)
    y = xn * np.float32(127)
    # ties of y itself go to even (y is exactly k + 0.5 only where fp32 says so)
    want = np.rint(y.astype(np.float64)).astype(np.int8)
    assert codes.tolist() == want.tolist()
    assert codes[0] == 127 and codes[1] == -127 and codes[2] == 0 and codes[3] == 0


def test_fp8_codes_brute_force_and_ties():
    rng = np.random.default_rng(0)
    xn = rng.uniform(-1, 1, 4000).astype(np.float32)
    codes = oracle.fp8_code(xn)
    vals = oracle.e4m3_value(codes)
    y = (xn * np.float32(448)).astype(np.float64)
    allv = oracle.e4m3_value(np.arange(256))
    fin = ~np.isnan(allv)
    for yy, v in zip(y, vals):
        assert abs(v - yy) == np.min(np.abs(allv[fin] - yy))
    # exact midpoints between neighbours: the even code wins
    pos = oracle.e4m3_value(np.arange(127))
    for c in range(126):
        mid = (pos[c] + pos[c + 1]) / 2
        xn_mid = np.float32(mid / 448.0)
        if float(np.float32(xn_mid * np.float32(448))) != mid:
            continue  # not an exact tie after the fp32 multiply
        got = int(oracle.fp8_code(np.array([xn_mid]))[0])
        assert got == (c if c % 2 == 0 else c + 1), (c, got)
    assert int(oracle.fp8_code(np.array([1.0], np.float32))[0]) == 0x7E
    assert int(oracle.fp8_code(np.array([-0.0], np.float32))[0]) == 0


@pytest.mark.parametrize("qt", ["int8", "fp8"])
def test_round_trip_within_half_a_step(qt):
    rng = np.random.default_rng(1)
    w = rng.standard_normal((3, 8, 256), dtype=np.float32) * np.float32(0.02)
    w[0, 0, :64] = 0.0
    codes, absmax = oracle.quantize_blockwise8(w, qt)
    assert codes.shape == w.shape and absmax.shape == (3, 8, 4)
    assert np.all(codes[0, 0, :64] == 0) and absmax[0, 0, 0] == 0
    deq = oracle.dequantize_blockwise8(codes, absmax, qt)
    a = np.repeat(absmax.astype(np.float64), 64, axis=-1)
    err = np.abs(deq - w)
    if qt == "int8":
        assert np.all(err <= a / 254 * (1 + 1e-6) + 1e-12)
    else:
        # half the e4m3 spacing at the value, scaled back by absmax / 448
        y = np.abs(w / np.where(a == 0, 1, a) * 448)
        _, ex = np.frexp(np.maximum(y, 2.0 ** -6))
        half = np.ldexp(1.0, ex - 1 - 4)  # 3 mantissa bits
        assert np.all(err <= half * a / 448 * (1 + 1e-6) + 1e-12)
    # the block's extreme is exact
    k = np.argmax(np.abs(w[1, 2, :64]))
    assert deq[1, 2, k] == w[1, 2, k]


def test_fidelity_ordering_of_all_modes():
    """Mean squared reconstruction error on N(0,1)-like blocks:
    int8 < fp8 < nf4 < fp4."""
    rng = np.random.default_rng(2)
    w = rng.standard_normal((4, 64, 512), dtype=np.float32)
    err = {}
    for qt in ("nf4", "fp4"):
        p, a = oracle.quantize_blockwise(w, quant_type=qt)
        err[qt] = float(np.mean((oracle.dequantize_blockwise(p, a, quant_type=qt) - w) ** 2))
    for qt in ("int8", "fp8"):
        c, a = oracle.quantize_blockwise8(w, qt)
        err[qt] = float(np.mean((oracle.dequantize_blockwise8(c, a, qt) - w) ** 2))
    assert err["int8"] < err["fp8"] < err["nf4"] < err["fp4"], err


def test_grouped_gemm_accepts_8bit_stacks():
    rng = np.random.default_rng(3)
    w = rng.standard_normal((2, 16, 128), dtype=np.float32) * np.float32(0.05)
    for qt in ("int8", "fp8"):
        c, a = oracle.quantize_blockwise8(w, qt)
        x = rng.standard_normal((5, 128))
        off = np.array([0, 2, 5], dtype=np.int32)
        got = oracle.grouped_gemm(x, c, a, off, quant_type=qt)
        W = oracle.dequantize_blockwise8(c, a, qt)
        want = np.concatenate([x[0:2] @ W[0].T, x[2:5] @ W[1].T])
        assert np.allclose(got, want, rtol=1e-13, atol=1e-15)
