"""Pins for the oracle's bf16 / fp16 passthrough storage (CPU only).

The rounding is checked against torch's own conversions (independent
implementations of the same IEEE / bf16 rounding), on random values and on
constructed exact ties; the bit decode against the formats' known patterns;
the GEMM against brute force, an exact integer case and a library matmul;
the storage modes' reconstruction errors against the expected fidelity
order.
"""

import numpy as np
import pytest
import torch

import oracle


def _spread(rng, n):
    """Random fp32 values over many binades, both signs."""
    mant = rng.uniform(1.0, 2.0, n)
    exp = rng.integers(-30, 16, n)
    sign = rng.choice([-1.0, 1.0], n)
    return (sign * mant * np.exp2(exp)).astype(np.float32)


def test_bf16_store_matches_torch_rounding():
    rng = np.random.default_rng(0)
    w = np.concatenate([_spread(rng, 20000), rng.standard_normal(20000).astype(np.float32)])
    want = torch.from_numpy(w).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(oracle.bf16_store(w), want)


def test_bf16_store_exact_ties_go_to_even():
    # 1 + 2^-8 lies exactly between the bf16 values 1 and 1 + 2^-7
    # (last bit 0 / 1): it rounds down; 1 + 3 * 2^-8 lies between 1 + 2^-7
    # (odd) and 1 + 2^-6 (even): it rounds up
    w = np.array([1 + 2.0 ** -8, 1 + 3 * 2.0 ** -8, -(1 + 2.0 ** -8)], dtype=np.float32)
    got = oracle.bf16_value(oracle.bf16_store(w))
    assert got.tolist() == [1.0, 1 + 2.0 ** -6, -1.0]
    want = torch.from_numpy(w).to(torch.bfloat16).float().numpy()
    assert np.array_equal(got, want.astype(np.float64))


def test_fp16_store_matches_torch_rounding():
    rng = np.random.default_rng(1)
    w = np.concatenate([_spread(rng, 20000), rng.standard_normal(20000).astype(np.float32)])
    w = w[np.abs(w) < 60000]
    want = torch.from_numpy(w).half().view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(oracle.fp16_store(w), want)
    # a tie at 1 + 2^-11 (between 1 and 1 + 2^-10) goes to 1; subnormals kept
    t = np.array([1 + 2.0 ** -11, 2.0 ** -20, -3 * 2.0 ** -24], dtype=np.float32)
    assert oracle.fp16_value(oracle.fp16_store(t)).tolist() == [1.0, 2.0 ** -20, -3 * 2.0 ** -24]


def test_bit_decode_known_patterns():
    assert oracle.bf16_value(np.array([0x3F80, 0xC000, 0x0000, 0x8000], np.uint16)).tolist() \
        == [1.0, -2.0, 0.0, -0.0]
    assert oracle.fp16_value(np.array([0x3C00, 0xC000, 0x7BFF, 0x0001], np.uint16)).tolist() \
        == [1.0, -2.0, 65504.0, 2.0 ** -24]


@pytest.mark.parametrize("qt", ["bf16", "fp16"])
def test_grouped_gemm16_brute_force(qt):
    rng = np.random.default_rng(2)
    E, N, K, P = 3, 8, 64, 9
    bits = oracle.store16(rng.standard_normal((E, N, K)).astype(np.float32) * 0.1, qt)
    a = rng.standard_normal((5, K))
    offsets = np.array([0, 4, 4, 9], dtype=np.int32)
    gather = rng.integers(0, 10, size=P).astype(np.int32)
    rs = rng.uniform(0.5, 1.5, P)
    for swiglu in (False, True):
        got = oracle.grouped_gemm16(a, bits, offsets, qt, gather=gather, gather_div=2,
                                    swiglu=swiglu, row_scale=rs)
        W = oracle.value16(bits, qt)
        for i in range(P):
            e = 0 if i < 4 else 2
            row = a[gather[i] // 2]
            g = [sum(row[k] * W[e, n, k] for k in range(K)) for n in range(N)]
            if swiglu:
                g = [g[n] / (1 + np.exp(-g[n])) * g[n + N // 2] for n in range(N // 2)]
            assert np.allclose(got[i], np.array(g) * rs[i], rtol=1e-12, atol=1e-14)


@pytest.mark.parametrize("qt", ["bf16", "fp16"])
def test_grouped_gemm16_exact_integer_case(qt):
    """Small integers are exact in both formats: the product is exact."""
    rng = np.random.default_rng(3)
    E, N, K = 2, 16, 128
    w = rng.integers(-8, 9, size=(E, N, K)).astype(np.float32)
    bits = oracle.store16(w, qt)
    assert np.array_equal(oracle.value16(bits, qt), w.astype(np.float64))
    a = rng.integers(-4, 5, size=(6, K)).astype(np.float64)
    offsets = np.array([0, 2, 6], dtype=np.int32)
    got = oracle.grouped_gemm16(a, bits, offsets, qt)
    want = np.concatenate([a[:2] @ w[0].T, a[2:] @ w[1].T])
    assert np.array_equal(got, want)


def test_layer_with_one_expert_is_the_dense_mlp():
    rng = np.random.default_rng(4)
    H, I, T = 64, 64, 5
    gu = oracle.store16(rng.standard_normal((1, 2 * I, H)).astype(np.float32) * 0.05, "fp16")
    dn = oracle.store16(rng.standard_normal((1, H, I)).astype(np.float32) * 0.05, "fp16")
    x = rng.standard_normal((T, H))
    lg = np.zeros((T, 1), dtype=np.float32)
    y = oracle.moe_forward16(x, lg, 1, gu, dn, "fp16")
    Wg = torch.from_numpy(oracle.fp16_value(gu[0]))
    Wd = torch.from_numpy(oracle.fp16_value(dn[0]))
    g = torch.from_numpy(x) @ Wg.T
    want = (torch.nn.functional.silu(g[:, :I]) * g[:, I:]) @ Wd.T
    assert np.allclose(y, want.numpy(), rtol=1e-12, atol=1e-14)


def test_storage_modes_fidelity_order():
    """Relative RMS reconstruction error on Gaussian weights: fp16 < bf16 <
    int8 < fp8 < nf4 < fp4 (the selectable-precision stack is ordered by
    fidelity)."""
    rng = np.random.default_rng(5)
    w = (rng.standard_normal((4, 64, 512)) * 0.02).astype(np.float32)

    def rel(q):
        if q in oracle.PASSTHROUGH:
            v = oracle.value16(oracle.store16(w, q), q)
        elif q in ("int8", "fp8"):
            v = oracle.dequantize_blockwise(*oracle.quantize_blockwise8(w, q), quant_type=q)
        else:
            v = oracle.dequantize_blockwise(*oracle.quantize_blockwise(w, quant_type=q),
                                            quant_type=q)
        d = np.asarray(v, np.float64) - w
        return np.sqrt(np.mean(d * d) / np.mean(w.astype(np.float64) ** 2))

    errs = [rel(q) for q in ("fp16", "bf16", "int8", "fp8", "nf4", "fp4")]
    assert errs == sorted(errs), errs
    assert errs[0] < 5e-4 and errs[1] < 3e-3
