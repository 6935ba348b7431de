"""Pins of the oracle's fp4 storage mode (CPU only).

The pages list fp4 beside nf4 as the 4-bit packed storage modes, with a
fidelity ordering in which nf4 reconstructs with less error than fp4
(experts4bit-qlora 0.22.0 README, "The problem").  Their fp4 values are not
printed; the oracle reads fp4 as the OCP e2m1 element format scaled by
absmax / 6.  These tests pin that reading against an independent decoding of
the e2m1 bit fields, brute force, exact ties, closed forms and the pages'
ordering.
"""

import numpy as np
import pytest

import oracle



def _e2m1_value(code: int) -> float:
    """e2m1 from its bit fields: sign, 2 exponent bits (bias 1), 1 mantissa
    bit; exponent 0 is subnormal (m/2), else 2^(e-1) * (1 + m/2)."""
    s, e, m = code >> 3, (code >> 1) & 3, code & 1
    v = (m / 2.0) if e == 0 else (2.0 ** (e - 1)) * (1.0 + m / 2.0)
    return -v if s else v


def test_fp4_codebook_is_e2m1_over_six():
    lv = oracle.fp4_codebook()
    assert lv.dtype == np.float32 and lv.shape == (16,)
    for c in range(16):
        want = np.float32(_e2m1_value(c) / 6.0)
        assert lv[c] == want, c
    assert lv[7] == np.float32(1.0) and lv[15] == np.float32(-1.0)
    assert lv[0] == 0.0 and np.signbit(lv[8]) and lv[8] == 0.0  # +0 and -0


def _brute_code(xn: np.float32) -> int:
    """Independent nearest-code search over all 16 codes: the sign must match
    (xn < 0 <-> sign bit), then the smallest |xn - level| in fp64, ties to
    the code whose magnitude index is even."""
    lv = oracle.fp4_codebook().astype(np.float64)
    want_sign = 1 if xn < 0 else 0
    best = None
    for c in range(16):
        if (c >> 3) != want_sign:
            continue
        d = abs(float(xn) - lv[c])
        key = (d, (c & 7) % 2)  # on a tie the even magnitude index wins
        if best is None or key < best[0]:
            best = (key, c)
    return best[1]


def test_fp4_code_brute_force_random():
    rng = np.random.default_rng(1)
    xn = rng.uniform(-1, 1, size=4000).astype(np.float32)
    got = oracle.fp4_code(xn)
    want = np.array([_brute_code(v) for v in xn], dtype=np.uint8)
    assert np.array_equal(got, want)


def test_fp4_exact_tie_goes_to_even_magnitude():
    lv = oracle.fp4_codebook()
    # midpoint of +0 and the smallest magnitude is exactly representable
    mid = np.float32(lv[1] / np.float32(2))
    assert float(mid) == (float(lv[0]) + float(lv[1])) / 2
    assert oracle.fp4_code(np.array([mid], np.float32))[0] == 0
    assert oracle.fp4_code(np.array([-mid], np.float32))[0] == 8
    # just above the midpoint rounds up to magnitude index 1
    up = np.nextafter(mid, np.float32(1))
    assert oracle.fp4_code(np.array([up], np.float32))[0] == 1
    # 2/3 and 1: their fp64 midpoint is not an fp32 value, so the fp32
    # values just below and above it go to the lower and upper level
    m64 = (float(lv[6]) + float(lv[7])) / 2
    below = np.float32(m64)
    if float(below) > m64:
        below = np.nextafter(below, np.float32(0))
    above = np.nextafter(below, np.float32(1))
    assert float(below) < m64 < float(above)
    assert oracle.fp4_code(np.array([below, above], np.float32)).tolist() == [6, 7]


def test_fp4_quantize_closed_forms():
    # every element an exact multiple of absmax/6 at an e2m1 magnitude
    a = np.float32(3.0)
    mags = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6], np.float32) / np.float32(6) * a
    row = np.concatenate([mags, -mags[1:], np.zeros(64 - 15, np.float32)])
    w = row.reshape(1, 1, 64).astype(np.float32)
    packed, absmax = oracle.quantize_blockwise(w, quant_type="fp4")
    assert absmax[0, 0, 0] == a
    back = oracle.dequantize_blockwise(packed, absmax, quant_type="fp4")
    assert np.array_equal(back, w)
    codes = oracle.unpack_codes(packed)[0, 0]
    assert list(codes[:8]) == list(range(8)) and list(codes[8:15]) == list(range(9, 16))


def test_fp4_zero_block_and_extremes():
    w = np.zeros((1, 2, 64), np.float32)
    w[0, 1, 5] = -2.5
    w[0, 1, 6] = 1.0
    packed, absmax = oracle.quantize_blockwise(w, quant_type="fp4")
    codes = oracle.unpack_codes(packed)
    assert absmax[0, 0, 0] == 0 and np.all(codes[0, 0] == 0)
    assert codes[0, 1, 5] == 15  # -absmax -> -1 exactly
    back = oracle.dequantize_blockwise(packed, absmax, quant_type="fp4")
    assert back[0, 1, 5] == np.float32(-2.5)


def test_fp4_round_trip_error_bound():
    rng = np.random.default_rng(2)
    w = rng.standard_normal((3, 8, 256)).astype(np.float32)
    packed, absmax = oracle.quantize_blockwise(w, quant_type="fp4")
    back = oracle.dequantize_blockwise(packed, absmax, quant_type="fp4").astype(np.float64)
    bound = np.repeat(oracle.block_error_bound(absmax, "fp4"), 64, axis=-1)
    # half the widest gap (1/3 -> 1/2 and 2/3 -> 1 are 1/6 and 1/3 wide)
    assert np.all(np.abs(back - w) <= bound * (1 + 1e-6))


def test_fidelity_ordering_nf4_better_than_fp4():
    """The pages' ordering: nf4 reconstructs with less error than fp4."""
    rng = np.random.default_rng(3)
    w = (rng.standard_normal((4, 64, 512)) * 0.02).astype(np.float32)
    errs = {}
    for qt in ("nf4", "fp4"):
        p, a = oracle.quantize_blockwise(w, quant_type=qt)
        back = oracle.dequantize_blockwise(p, a, quant_type=qt).astype(np.float64)
        errs[qt] = float(np.linalg.norm(back - w) / np.linalg.norm(w))
    assert errs["nf4"] < errs["fp4"], errs


def test_fp4_nibble_packing_shared_with_nf4():
    rng = np.random.default_rng(4)
    w = rng.standard_normal((2, 3, 128)).astype(np.float32)
    packed, absmax = oracle.quantize_blockwise(w, quant_type="fp4")
    codes = oracle.unpack_codes(packed)
    xn = (w.reshape(2, 3, 2, 64) / absmax[..., None]).astype(np.float32).reshape(2, 3, 128)
    assert np.array_equal(codes, oracle.fp4_code(xn))
    assert np.array_equal(oracle.pack_codes(codes), packed)
