"""Pins for the oracle's NF4 codebook, quantiser and dequantiser (CPU only).

Each test checks the oracle against something other than itself: a second
quantile implementation and the normal CDF, byte totals printed on the pages,
brute force in exact rational arithmetic, exact special cases and the
round-trip error bound.
"""

import json
import math
import os
import statistics
from fractions import Fraction

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
DELTA = 0.9677083333333334  # ((1 - 1/32) + (1 - 1/30)) / 2, written out


# ----------------------------------------------------------------- codebook

def test_codebook_structure():
    q = oracle.nf4_codebook()
    assert q.dtype == np.float32 and q.shape == (16,)
    assert np.all(np.diff(q.astype(np.float64)) > 0), "strictly increasing"
    assert q[0] == -1.0 and q[7] == 0.0 and q[15] == 1.0
    assert np.sum(q < 0) == 7 and np.sum(q > 0) == 8
    # asymmetric: 8 positive levels, so the smallest positive level sits
    # closer to zero than the smallest negative one
    assert q[8] < -q[6]


def test_codebook_points_are_normal_quantiles():
    """Phi(v) (via math.erf, not the quantile routine) lands on the grid."""
    v = oracle.nf4_levels_unnormalised()
    phi = [0.5 * (1.0 + math.erf(t / math.sqrt(2.0))) for t in v]
    pos = sorted(p for p, t in zip(phi, v) if t > 0)
    neg = sorted(1.0 - p for p, t in zip(phi, v) if t < 0)
    want_pos = [0.5 + (DELTA - 0.5) * i / 8 for i in range(1, 9)]
    want_neg = [0.5 + (DELTA - 0.5) * i / 7 for i in range(1, 8)]
    assert np.allclose(pos, want_pos, rtol=0, atol=1e-12)
    assert np.allclose(neg, want_neg, rtol=0, atol=1e-12)
    assert v[7] == 0.0


def test_codebook_second_quantile_implementation_agrees():
    nd = statistics.NormalDist()
    alt = oracle.nf4_codebook_f64(ppf=nd.inv_cdf).astype(np.float32)
    assert np.array_equal(alt.view(np.uint32), oracle.nf4_codebook().view(np.uint32))


# ------------------------------------------------------------------ format

def test_byte_totals_printed_on_the_pages():
    with open(os.path.join(GOLDEN, "page_byte_totals.json")) as f:
        cases = json.load(f)["cases"]
    for c in cases:
        E, H, I = c["experts"], c["hidden"], c["intermediate"]
        per_layer = oracle.packed_bytes(E, 2 * I, H) + oracle.packed_bytes(E, H, I)
        assert c["layers"] * per_layer == c["bytes"], c["cite"]
        if c["round_to_GB_decimals"]:
            gb = round(c["bytes"] / 1e9, c["round_to_GB_decimals"])
            assert f"{gb:.2f} GB" == c["printed_as"]


def test_buffer_sizes_match_the_byte_formula():
    rng = np.random.default_rng(1)
    w = rng.standard_normal((3, 5, 128), dtype=np.float32)
    packed, absmax = oracle.quantize_blockwise(w)
    assert packed.shape == (3, 5, 64) and packed.dtype == np.uint8
    assert absmax.shape == (3, 5, 2) and absmax.dtype == np.float32
    assert packed.nbytes + absmax.nbytes == oracle.packed_bytes(3, 5, 128)


def test_nibble_order_even_element_high():
    """Reading: byte = (code[2i] << 4) | code[2i+1]."""
    q = oracle.nf4_codebook()
    a = np.float32(0.25)
    codes = np.array([15, 0] + [7] * 62, dtype=np.uint8)
    w = (q[codes] * a).astype(np.float32)[None, None, :]
    packed, absmax = oracle.quantize_blockwise(w)
    assert packed[0, 0, 0] == 0xF0 and packed[0, 0, 1] == 0x77
    assert absmax[0, 0, 0] == a


# --------------------------------------------------------------- quantise

def _brute_code(xn: np.float32, q: np.ndarray) -> int:
    """Nearest level in exact rational arithmetic, ties to the lower index."""
    x = Fraction(float(xn))
    best, best_d = None, None
    for i, qi in enumerate(q):
        d = abs(x - Fraction(float(qi)))
        if best_d is None or d < best_d:
            best, best_d = i, d
    return best


def test_nearest_code_brute_force_random():
    q = oracle.nf4_codebook()
    rng = np.random.default_rng(7)
    xn = rng.uniform(-1, 1, 4000).astype(np.float32)
    got = oracle.nearest_code(xn, q)
    want = [_brute_code(v, q) for v in xn]
    assert list(got) == want


def test_nearest_code_at_and_around_midpoints():
    q = oracle.nf4_codebook()
    cases = []
    for j in range(15):
        mid = (Fraction(float(q[j])) + Fraction(float(q[j + 1]))) / 2
        m32 = np.float32(float(mid))
        # the fp32 neighbours of the midpoint and the nearest fp32 value
        for v in (np.nextafter(m32, np.float32(-2)), m32, np.nextafter(m32, np.float32(2))):
            cases.append(np.float32(v))
        if Fraction(float(m32)) == mid:  # exactly representable: a true tie
            assert oracle.nearest_code(np.array([m32]), q)[0] == j
    xn = np.array(cases, dtype=np.float32)
    assert list(oracle.nearest_code(xn, q)) == [_brute_code(v, q) for v in xn]
    # at least a few midpoints are exact fp32 ties, so the tie rule is exercised
    exact = sum(
        Fraction(float(np.float32(float((Fraction(float(q[j])) + Fraction(float(q[j + 1]))) / 2))))
        == (Fraction(float(q[j])) + Fraction(float(q[j + 1]))) / 2
        for j in range(15))
    assert exact >= 1


def test_quantize_brute_force_small_stack():
    rng = np.random.default_rng(3)
    w = (rng.standard_normal((2, 3, 128), dtype=np.float32) * np.float32(0.02))
    packed, absmax = oracle.quantize_blockwise(w)
    q = oracle.nf4_codebook()
    codes = oracle.unpack_codes(packed)
    for e in range(2):
        for n in range(3):
            for b in range(2):
                blk = w[e, n, 64 * b: 64 * (b + 1)]
                a = np.float32(max(abs(float(v)) for v in blk))
                assert absmax[e, n, b] == a
                for i, v in enumerate(blk):
                    xn = np.float32(v) / a  # IEEE fp32 division
                    assert codes[e, n, 64 * b + i] == _brute_code(xn, q)


def test_exact_levels_round_trip():
    """Values a*level with a = 2^-3 quantise to their own codes exactly."""
    rng = np.random.default_rng(11)
    q = oracle.nf4_codebook()
    codes = rng.integers(0, 16, size=(4, 6, 256)).astype(np.uint8)
    codes[..., ::64] = 15  # every block holds a +1 element, so absmax = a
    a = np.float32(0.125)
    w = (q[codes] * a).astype(np.float32)
    packed, absmax = oracle.quantize_blockwise(w)
    assert np.all(absmax == a)
    assert np.array_equal(oracle.unpack_codes(packed), codes)
    assert np.array_equal(oracle.dequantize_blockwise(packed, absmax), w)


def test_round_trip_error_bound_and_max_element():
    rng = np.random.default_rng(5)
    w = rng.standard_normal((4, 16, 512), dtype=np.float32) * np.float32(0.02)
    packed, absmax = oracle.quantize_blockwise(w)
    d = oracle.dequantize_blockwise(packed, absmax)
    q = oracle.nf4_codebook().astype(np.float64)
    half_gap = np.max(np.diff(q)) / 2.0
    assert abs(half_gap - 0.15190) < 1e-4
    bound = np.repeat(absmax.astype(np.float64), 64, axis=-1) * half_gap
    ulp = np.spacing(np.abs(w)).astype(np.float64)
    err = np.abs(d.astype(np.float64) - w.astype(np.float64))
    assert np.all(err <= bound + ulp)
    # the element of largest magnitude in each block is reproduced exactly
    blocks = w.reshape(4, 16, 8, 64)
    dblk = d.reshape(4, 16, 8, 64)
    idx = np.argmax(np.abs(blocks), axis=-1)[..., None]
    assert np.array_equal(np.take_along_axis(dblk, idx, -1),
                          np.take_along_axis(blocks, idx, -1))


def test_zero_and_negative_zero_blocks():
    w = np.zeros((1, 2, 128), dtype=np.float32)
    w[0, 1, :64] = -0.0
    w[0, 1, 64:] = np.linspace(-1, 1, 64, dtype=np.float32)
    packed, absmax = oracle.quantize_blockwise(w)
    codes = oracle.unpack_codes(packed)
    assert np.all(codes[0, 0] == 7) and np.all(absmax[0, 0] == 0)
    assert np.all(codes[0, 1, :64] == 7) and absmax[0, 1, 0] == 0
    d = oracle.dequantize_blockwise(packed, absmax)
    assert np.all(d[0, 0] == 0) and np.all(d[0, 1, :64] == 0)


def test_quantize_is_idempotent():
    rng = np.random.default_rng(9)
    w = rng.standard_normal((2, 8, 256), dtype=np.float32)
    p1, a1 = oracle.quantize_blockwise(w)
    p2, a2 = oracle.quantize_blockwise(oracle.dequantize_blockwise(p1, a1))
    assert np.array_equal(p1, p2) and np.array_equal(a1, a2)


def test_blocks_never_cross_rows_or_experts():
    rng = np.random.default_rng(2)
    w = rng.standard_normal((3, 4, 192), dtype=np.float32)
    p, a = oracle.quantize_blockwise(w)
    for e in range(3):
        for n in range(4):
            pr, ar = oracle.quantize_blockwise(w[e:e + 1, n:n + 1])
            assert np.array_equal(pr[0, 0], p[e, n]) and np.array_equal(ar[0, 0], a[e, n])


def test_denormal_inputs_are_not_flushed():
    tiny = np.float32(1e-40)  # an fp32 subnormal
    w = np.full((1, 1, 64), 0, dtype=np.float32)
    w[0, 0, 0] = tiny
    w[0, 0, 1] = -tiny
    p, a = oracle.quantize_blockwise(w)
    assert a[0, 0, 0] == tiny
    c = oracle.unpack_codes(p)[0, 0]
    assert c[0] == 15 and c[1] == 0 and np.all(c[2:] == 7)


def test_gaussian_code_histogram_is_roughly_balanced():
    """NF4 levels are normal quantiles: Gaussian data fills every code."""
    rng = np.random.default_rng(4)
    w = rng.standard_normal((8, 64, 1024), dtype=np.float32)
    p, _ = oracle.quantize_blockwise(w)
    h = np.bincount(oracle.unpack_codes(p).ravel(), minlength=16) / w.size
    assert h.min() > 0.01 and h.max() < 0.12
    # mirror-image bins on the two sides hold similar mass
    assert abs(h[1] - h[14]) < 0.03
