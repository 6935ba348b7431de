"""The comparison rule itself (CPU only): a correctly rounded output passes
with zero error beyond rounding, and a real deviation is seen."""

import numpy as np

from grouped_nf4_gemm_quantize_amd import synth
from parity import half_spacing, metrics


def test_correctly_rounded_bf16_has_no_error_beyond_rounding():
    rng = np.random.default_rng(0)
    y = rng.standard_normal(200000) * np.exp(rng.uniform(-20, 5, 200000))
    y = y.astype(np.float32).astype(np.float64)  # so bf16 rounding is a single rounding
    yb = synth.round_to_bf16(y.astype(np.float32)).astype(np.float64)
    m = metrics(yb, y)
    assert m["maxabs_beyond_rounding"] == 0.0
    assert m["maxabs"] > 0 and m["floor"] == m["maxabs"]


def test_half_spacing_values():
    assert half_spacing(np.array([1.0]), "bf16")[0] == 2.0 ** -8
    assert half_spacing(np.array([1.99]), "bf16")[0] == 2.0 ** -8
    assert half_spacing(np.array([2.0]), "bf16")[0] == 2.0 ** -7
    assert half_spacing(np.array([0.75]), "f16")[0] == 2.0 ** -12
    assert half_spacing(np.array([0.0]), "f16")[0] == 2.0 ** -25


def test_a_deviation_beyond_rounding_is_reported():
    y = np.linspace(-3, 3, 10001)
    yb = synth.round_to_bf16(y.astype(np.float32)).astype(np.float64)
    rms = np.sqrt(np.mean(y ** 2))
    bad = yb.copy()
    bad[1234] += 0.05 * rms
    m = metrics(bad, y)
    assert m["maxabs_beyond_rounding"] > 0.04


def test_literal_clause_has_no_rounding_allowance():
    """The literal check fails an fp32 result whose only deviation is a bf16
    rounding the relaxed rule forgives, and passes the exact result."""
    import pytest

    from parity import assert_parity_literal

    rng = np.random.default_rng(3)
    y = rng.standard_normal(4096) * 3.0
    y[7] = 123.4  # one large output: its bf16 rounding error is ~0.2 * RMS
    assert_parity_literal(y.astype(np.float32), y)
    yb = synth.round_to_bf16(y.astype(np.float32)).astype(np.float64)
    with pytest.raises(AssertionError):
        assert_parity_literal(yb, y)
