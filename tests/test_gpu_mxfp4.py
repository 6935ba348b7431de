"""GPU parity of the MXFP4 path (released e2m1 blocks + e8m0 scales).

The HIP grouped GEMM and layer forward on MXFP4 stacks against the oracle
(``oracle/mxfp4.py``).  Decoded MXFP4 weights are exact in fp16, so exactly
representable inputs must give bit-exact results.
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


def _mx_stack(rng, E, N, K, s_lo=118, s_hi=124):
    blocks = rng.integers(0, 256, size=(E, N, K // 2)).astype(np.uint8)
    scales = rng.integers(s_lo, s_hi, size=(E, N, K // 32)).astype(np.uint8)
    return blocks, scales


def test_mxfp4_gemm_exact_integer_case(gpu_lib):
    """Scales 2^0 / 2^1, small-integer rows: bit-exact over three 8-step scale
    groups (K = 1152), a ragged weight-row tile and several row tiles."""
    rng = np.random.default_rng(41)
    E, N, K = 3, 1056, 1152
    counts = [130, 0, 257]
    P = sum(counts)
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    blocks, scales = _mx_stack(rng, E, N, K, 127, 129)
    a = rng.integers(-4, 5, size=(P // 2 + 3, K)).astype(np.float16)
    gather = rng.integers(0, 2 * a.shape[0], size=P).astype(np.int32)
    out = gpu_lib.grouped_gemm_mxfp4(gpu(a), gpu(blocks), gpu(scales), gpu(offsets), P,
                                     gather=gpu(gather), gather_div=2, out_dtype=torch.float32)
    want = oracle.grouped_gemm_mxfp4(a.astype(np.float64), blocks, scales, offsets,
                                     gather=gather, gather_div=2)
    assert np.array_equal(host(out), want.astype(np.float32))


@pytest.mark.parametrize("swiglu", [False, True])
def test_mxfp4_gemm_matches_oracle(gpu_lib, swiglu):
    rng = np.random.default_rng(42 + swiglu)
    E, N, K = 4, 640, 768
    counts = [200, 1, 0, 90]
    P = sum(counts)
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    blocks, scales = _mx_stack(rng, E, N, K)
    a = rng.standard_normal((150, K)).astype(np.float16)
    gather = rng.integers(0, 300, size=P).astype(np.int32)
    rs = rng.uniform(0.2, 1.0, size=P).astype(np.float32)
    scatter = rng.permutation(P).astype(np.int32)
    out = gpu_lib.grouped_gemm_mxfp4(gpu(a), gpu(blocks), gpu(scales), gpu(offsets), P,
                                     gather=gpu(gather), gather_div=2, swiglu=swiglu,
                                     row_scale=gpu(rs), scatter=gpu(scatter),
                                     out_dtype=torch.float32)
    ref = oracle.grouped_gemm_mxfp4(a.astype(np.float64), blocks, scales, offsets,
                                    gather=gather, gather_div=2, swiglu=swiglu, row_scale=rs)
    # weights decode exactly; only the fp32 summation order differs
    assert_parity(host(out)[scatter], ref, fro_tol=1e-4, maxabs_tol=1e-3, what="mxfp4",
                  out_dtype="f32")


@pytest.mark.parametrize("name,T,E", [("tiny", None, None), ("olmoe", 256, 16),
                                      ("decode", 1, 32)])
def test_mxfp4_forward_matches_oracle(gpu_lib, name, T, E):
    over = {}
    if T is not None:
        over = dict(T=T, E=E)
    cfg = synth.config(name, **over)
    gb, gs = synth.mxfp4_stack(cfg, "gu")
    db, ds = synth.mxfp4_stack(cfg, "dn")
    x = synth.activations(cfg)
    lg = synth.router_logits(cfg)
    y = gpu_lib.moe_forward_mxfp4(gpu(x, torch.bfloat16), gpu(lg), cfg.k, gpu(gb), gpu(gs),
                                  gpu(db), gpu(ds), cfg.renormalize)
    ref = oracle.moe_forward_mxfp4(x, lg, cfg.k, gb, gs, db, ds, cfg.renormalize)
    m = assert_parity(host(y), ref, what=f"mxfp4 {name}")
    print(name, m)


def test_mxfp4_decode_scales_beyond_fp16_range(gpu_lib):
    """T = 1 runs the decode GEMVs, which apply each block's e8m0 scale in
    fp32: down weights up to 6 * 2^20 (beyond fp16's 65504) stay exact.  (h
    between the projections is fp16, so the gate_up scales stay moderate.)"""
    cfg = synth.config("decode", E=16)
    rng = np.random.default_rng(44)
    gb, _ = synth.mxfp4_stack(cfg, "gu")
    db, _ = synth.mxfp4_stack(cfg, "dn")
    gs = rng.integers(114, 118, size=(cfg.E, 2 * cfg.I, cfg.H // 32)).astype(np.uint8)  # 2^-13..-10
    ds = rng.integers(143, 148, size=(cfg.E, cfg.H, cfg.I // 32)).astype(np.uint8)      # 2^16..2^20
    x = synth.activations(cfg)
    lg = synth.router_logits(cfg)
    y = gpu_lib.moe_forward_mxfp4(gpu(x, torch.bfloat16), gpu(lg), cfg.k, gpu(gb), gpu(gs),
                                  gpu(db), gpu(ds), y_dtype=torch.float32)
    ref = oracle.moe_forward_mxfp4(x, lg, cfg.k, gb, gs, db, ds)
    assert_parity(host(y), ref, fro_tol=2e-3, maxabs_tol=2e-2, what="mx decode range",
                  out_dtype="f32")
