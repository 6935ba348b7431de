"""Pins for the oracle's MXFP4 weights (e2m1 + e8m0) and GEMM (CPU only).

The element and scale decodes are checked against the values the OCP
microscaling format defines (a literal table and a float32 bit-pattern
construction), against the independently written fp4 codebook, and the GEMM
against brute force and a library matmul.
"""

import numpy as np
import torch

import oracle

# e2m1 values by code: the format's table (sign bit 3)
E2M1 = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0,
        -0.0, -0.5, -1.0, -1.5, -2.0, -3.0, -4.0, -6.0]


def test_e2m1_values_match_the_format_table():
    got = oracle.e2m1_value(np.arange(16))
    assert got.tolist() == E2M1
    assert np.signbit(got[8])


def test_e2m1_agrees_with_the_fp4_codebook():
    """The fp4 storage mode's levels are the same e2m1 values over 6."""
    assert np.array_equal(oracle.e2m1_value(np.arange(16)) / 6.0,
                          oracle.fp4_codebook_f64())


def test_e8m0_is_a_float32_exponent_field():
    s = np.arange(1, 255)
    bits = (s.astype(np.uint32) << 23).view(np.float32).astype(np.float64)
    assert np.array_equal(oracle.e8m0_value(s), bits)
    assert oracle.e8m0_value(0) == 2.0 ** -127
    assert oracle.e8m0_value(127) == 1.0
    assert np.isnan(oracle.e8m0_value(255))


def test_nibble_order_is_low_first():
    codes = np.array([[1, 2, 15, 8]], dtype=np.uint8)
    packed = oracle.pack_mx(codes)
    assert packed.tolist() == [[0x21, 0x8F]]
    assert np.array_equal(oracle.unpack_mx(packed), codes)


def test_dequantize_brute_force():
    rng = np.random.default_rng(0)
    E, N, K = 2, 3, 96
    codes = rng.integers(0, 16, size=(E, N, K)).astype(np.uint8)
    scales = rng.integers(100, 140, size=(E, N, K // 32)).astype(np.uint8)
    w = oracle.dequantize_mxfp4(oracle.pack_mx(codes), scales)
    for e in range(E):
        for n in range(N):
            for k in range(K):
                want = E2M1[codes[e, n, k]] * 2.0 ** (int(scales[e, n, k // 32]) - 127)
                assert w[e, n, k] == want


def test_grouped_gemm_exact_integer_case():
    """Scales 2^0 and 2^1, small-integer rows: exact, by brute force."""
    rng = np.random.default_rng(1)
    E, N, K, P = 3, 16, 64, 11
    codes = rng.integers(0, 16, size=(E, N, K)).astype(np.uint8)
    scales = (127 + rng.integers(0, 2, size=(E, N, K // 32))).astype(np.uint8)
    blocks = oracle.pack_mx(codes)
    a = rng.integers(-3, 4, size=(6, K)).astype(np.float64)
    offsets = np.array([0, 5, 5, 11], dtype=np.int32)
    gather = rng.integers(0, 12, size=P).astype(np.int32)
    got = oracle.grouped_gemm_mxfp4(a, blocks, scales, offsets, gather=gather, gather_div=2)
    for i in range(P):
        e = 0 if i < 5 else 2
        row = a[gather[i] // 2]
        for n in range(N):
            want = sum(row[k] * E2M1[codes[e, n, k]] * 2.0 ** (int(scales[e, n, k // 32]) - 127)
                       for k in range(K))
            assert got[i, n] == want


def test_grouped_gemm_matches_torch_matmul():
    rng = np.random.default_rng(2)
    E, N, K = 2, 40, 128
    blocks = rng.integers(0, 256, size=(E, N, K // 2)).astype(np.uint8)
    scales = rng.integers(118, 124, size=(E, N, K // 32)).astype(np.uint8)
    a = rng.standard_normal((9, K))
    offsets = np.array([0, 4, 9], dtype=np.int32)
    got = oracle.grouped_gemm_mxfp4(a, blocks, scales, offsets)
    W = torch.from_numpy(oracle.dequantize_mxfp4(blocks, scales))
    for e in range(E):
        lo, hi = offsets[e], offsets[e + 1]
        want = torch.matmul(torch.from_numpy(a[lo:hi]), W[e].T).numpy()
        assert np.allclose(got[lo:hi], want, rtol=1e-12, atol=1e-14)


def test_layer_with_one_expert_is_the_dense_mlp():
    """E = 1, k = 1: y = down(silu(gate x) * up x) with the dequantised
    weights, written with torch ops."""
    rng = np.random.default_rng(3)
    H, I, T = 64, 64, 5
    gb = rng.integers(0, 256, size=(1, 2 * I, H // 2)).astype(np.uint8)
    gs = rng.integers(118, 122, size=(1, 2 * I, H // 32)).astype(np.uint8)
    db = rng.integers(0, 256, size=(1, H, I // 2)).astype(np.uint8)
    ds = rng.integers(118, 122, size=(1, H, I // 32)).astype(np.uint8)
    x = rng.standard_normal((T, H))
    lg = np.zeros((T, 1), dtype=np.float32)
    y = oracle.moe_forward_mxfp4(x, lg, 1, gb, gs, db, ds)
    Wg = torch.from_numpy(oracle.dequantize_mxfp4(gb, gs)[0])
    Wd = torch.from_numpy(oracle.dequantize_mxfp4(db, ds)[0])
    g = torch.from_numpy(x) @ Wg.T
    want = (torch.nn.functional.silu(g[:, :I]) * g[:, I:]) @ Wd.T
    assert np.allclose(y, want.numpy(), rtol=1e-12, atol=1e-14)
