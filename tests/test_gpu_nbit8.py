"""GPU parity of the 8-bit storage modes (int8, fp8 e4m3) on the grouped GEMM.

Codes and absmax must match the oracle bit for bit; exactly representable
GEMMs must match bit for bit; everything else meets ``parity.py``.
"""

import numpy as np
import pytest
import torch

import oracle
from grouped_nf4_gemm_quantize_amd import synth
from parity import assert_parity

pytestmark = pytest.mark.gpu
DEV = "cuda"


def gpu(a, dtype=None):
    t = torch.from_numpy(np.ascontiguousarray(a)).to(DEV)
    return t.to(dtype) if dtype is not None else t


def host(t):
    return t.detach().float().cpu().numpy() if t.dtype in (torch.bfloat16, torch.float16) \
        else t.detach().cpu().numpy()


def _edge_case_stack(qt):
    rng = np.random.default_rng(51)
    w = rng.standard_normal((2, 24, 256), dtype=np.float32) * np.float32(0.03)
    w[0, 0, :64] = 0.0
    w[0, 1, 64:128] = -0.0
    # a block with absmax 1 holding exact ties of the rounding
    if qt == "fp8":
        pos = oracle.e4m3_value(np.arange(127))
        mids = [np.float32(((pos[c] + pos[c + 1]) / 2) / 448.0) for c in range(126)]
    else:
        mids = [np.float32((k + 0.5) / 127.0) for k in range(126)]
    blk = np.array([1.0] + mids[:63], dtype=np.float32)
    w[1, 3, :64] = blk
    w[1, 4, 64:128] = -blk
    return w


@pytest.mark.parametrize("qt", ["int8", "fp8"])
def test_8bit_quantize_bit_exact(gpu_lib, qt):
    w = _edge_case_stack(qt)
    c_ref, a_ref = oracle.quantize_blockwise8(w, qt)
    c, a = gpu_lib.quantize(gpu(w), quant_type=qt)
    assert c.shape == w.shape
    assert np.array_equal(host(c), c_ref)
    assert np.array_equal(host(a).view(np.uint32), a_ref.view(np.uint32))
    # bf16 input
    wb = synth.round_to_bf16(w)
    c_ref, a_ref = oracle.quantize_blockwise8(wb, qt)
    c, a = gpu_lib.quantize(gpu(wb, torch.bfloat16), quant_type=qt)
    assert np.array_equal(host(c), c_ref) and np.array_equal(host(a), a_ref)


def _integer_codes(rng, qt, shape):
    if qt == "int8":
        return rng.integers(-127, 128, size=shape).astype(np.int8).view(np.uint8)
    vals = oracle.e4m3_value(np.arange(256))
    ok = [c for c in range(256) if np.isfinite(vals[c]) and vals[c] == np.round(vals[c])
          and abs(vals[c]) <= 64]
    return rng.choice(np.array(ok, dtype=np.uint8), size=shape)


@pytest.mark.parametrize("qt", ["int8", "fp8"])
def test_8bit_gemm_exact_integer_case(gpu_lib, qt):
    """absmax = 127 (448): the scale is 1, weights are the integer codes."""
    rng = np.random.default_rng(52)
    E, N, K = 3, 544, 640
    counts = [70, 0, 200]
    P = sum(counts)
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    codes = _integer_codes(rng, qt, (E, N, K))
    absmax = np.full((E, N, K // 64), 127.0 if qt == "int8" else 448.0, dtype=np.float32)
    a = rng.integers(-4, 5, size=(P // 2 + 3, K)).astype(np.float16)
    gather = rng.integers(0, 2 * a.shape[0], size=P).astype(np.int32)
    out = gpu_lib.grouped_gemm(gpu(a), gpu(codes), gpu(absmax), gpu(offsets), P,
                               gather=gpu(gather), gather_div=2, out_dtype=torch.float32,
                               quant_type=qt)
    want = oracle.grouped_gemm(a.astype(np.float64), codes, absmax, offsets, gather=gather,
                               gather_div=2, quant_type=qt)
    assert np.array_equal(host(out), want.astype(np.float32))


@pytest.mark.parametrize("qt", ["int8", "fp8"])
@pytest.mark.parametrize("swiglu", [False, True])
def test_8bit_gemm_matches_oracle(gpu_lib, qt, swiglu):
    rng = np.random.default_rng(53 + swiglu)
    E, N, K = 4, 640, 320
    counts = [130, 1, 0, 260]
    P = sum(counts)
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    w = rng.standard_normal((E, N, K), dtype=np.float32) * np.float32(0.05)
    codes, absmax = oracle.quantize_blockwise8(w, qt)
    a = rng.standard_normal((200, K)).astype(np.float16)
    gather = rng.integers(0, 400, size=P).astype(np.int32)
    scatter = rng.permutation(P).astype(np.int32)
    out = gpu_lib.grouped_gemm(gpu(a), gpu(codes), gpu(absmax), gpu(offsets), P,
                               gather=gpu(gather), gather_div=2, swiglu=swiglu,
                               scatter=gpu(scatter), out_dtype=torch.float32, quant_type=qt)
    ref = oracle.grouped_gemm(a.astype(np.float64), codes, absmax, offsets, gather=gather,
                              gather_div=2, swiglu=swiglu, quant_type=qt)
    # the fp16 roundings of the scale and of code x scale remain
    assert_parity(host(out)[scatter], ref, fro_tol=2e-3, maxabs_tol=2e-2, what=qt,
                  out_dtype="f32")


@pytest.mark.parametrize("qt", ["int8", "fp8"])
@pytest.mark.parametrize("name,T,E", [("tiny", None, None), ("olmoe", 256, 16)])
def test_8bit_forward_matches_oracle(gpu_lib, qt, name, T, E):
    cfg = synth.config(name, **({} if T is None else dict(T=T, E=E)))
    gu = synth.stack_weights(cfg, "gu")
    dn = synth.stack_weights(cfg, "dn")
    gc, ga = gpu_lib.quantize(gpu(gu), quant_type=qt)
    dc, da = gpu_lib.quantize(gpu(dn), quant_type=qt)
    gc_r, ga_r = oracle.quantize_blockwise8(gu, qt)
    dc_r, da_r = oracle.quantize_blockwise8(dn, qt)
    assert np.array_equal(host(gc), gc_r) and np.array_equal(host(dc), dc_r)
    x = synth.activations(cfg)
    lg = synth.router_logits(cfg)
    y = gpu_lib.moe_forward(gpu(x, torch.bfloat16), gpu(lg), cfg.k, gc, ga, dc, da,
                            quant_type=qt)
    ref, _ = oracle.moe_forward(x, lg, cfg.k, gc_r, ga_r, dc_r, da_r, quant_type=qt)
    print(qt, name, assert_parity(host(y), ref, what=f"{qt} {name}"))


def test_fidelity_ordering_of_all_modes_through_the_kernels(gpu_lib):
    """The same fp32 weights stored in each mode, one GEMM each on the GPU:
    error against the unquantised product orders int8 < fp8 < nf4 < fp4."""
    rng = np.random.default_rng(55)
    E, N, K = 2, 256, 512
    w = rng.standard_normal((E, N, K), dtype=np.float32) * np.float32(0.02)
    a = rng.standard_normal((96, K)).astype(np.float16)
    offsets = np.array([0, 40, 96], dtype=np.int32)
    exact = np.concatenate([a[:40].astype(np.float64) @ w[0].T.astype(np.float64),
                            a[40:].astype(np.float64) @ w[1].T.astype(np.float64)])
    err = {}
    for qt in ("int8", "fp8", "nf4", "fp4"):
        p, s = gpu_lib.quantize(gpu(w), quant_type=qt)
        out = gpu_lib.grouped_gemm(gpu(a), p, s, gpu(offsets), 96, out_dtype=torch.float32,
                                   quant_type=qt)
        err[qt] = float(np.linalg.norm(host(out) - exact) / np.linalg.norm(exact))
    assert err["int8"] < err["fp8"] < err["nf4"] < err["fp4"], err
