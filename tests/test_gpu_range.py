"""Observability of the fp16 range the grouped GEMMs compute in: the range
check of activations / gradients and the quantiser's absmax flag, against
NumPy's own float16 conversion (round to nearest even), and a layer whose
input leaves fp16's range."""

import numpy as np
import pytest
import torch

import oracle
from grouped_nf4_gemm_quantize_amd import synth

pytestmark = pytest.mark.gpu
DEV = "cuda"


def expected_flags(v):
    """The flag bits from NumPy's float16 conversion of the fp32 values."""
    v = np.asarray(v, dtype=np.float32)
    with np.errstate(over="ignore"):
        h = v.astype(np.float16)
    f = 0
    if np.any(~np.isfinite(h)):
        f |= 1
    if np.any((v != 0) & (h == 0)):
        f |= 2
    if np.any((v != 0) & (np.abs(v) < np.float32(2.0 ** -14))):
        f |= 4
    return f


def run_check(gpu_lib, v, dtype):
    t = torch.from_numpy(np.ascontiguousarray(v, dtype=np.float32)).to(DEV).to(dtype)
    flags = torch.zeros(1, dtype=torch.int32, device=DEV)
    gpu_lib.f16_range_check(t, flags)
    return int(flags.item())


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_range_check_matches_numpy_float16(gpu_lib, dtype):
    rng = np.random.default_rng(11)
    cases = {
        "normal": [1.0, -2.5, 0.0, -0.0, 1000.0, 2.0 ** -14],
        "overflow": [1.0, 7.0e4],
        "inf": [np.inf, 1.0],
        "nan": [np.nan],
        "flush": [1e-9, 1.0],
        "subnormal": [3e-5, -1.0],
        "edge_max": [65504.0, 65519.0],    # both round to 65504 (fp32 input)
        "edge_inf": [65520.0],             # ties to the even code: inf
        "edge_flush": [2.0 ** -25],        # ties to 0
        "edge_keep": [2.0 ** -24],         # the smallest subnormal
    }
    for name, vals in cases.items():
        for n in (len(vals), 1000, 4097):  # ragged tails beyond one vector
            v = rng.standard_normal(n).astype(np.float32)
            v[np.abs(v) < 1e-3] = 1.0      # keep the background in the normal range
            v[-len(vals):] = np.asarray(vals, dtype=np.float32)[:n]
            if dtype == torch.bfloat16:
                v = synth.round_to_bf16(v)
            assert run_check(gpu_lib, v, dtype) == expected_flags(v), (name, n, dtype)


@pytest.mark.parametrize("quant_type,div", [("nf4", 1.0), ("fp4", 1.0), ("int8", 127.0),
                                            ("fp8", 448.0)])
def test_quantiser_flags_absmax_outside_fp16(gpu_lib, quant_type, div):
    rng = np.random.default_rng(5)
    w = rng.standard_normal((2, 8, 128), dtype=np.float32) * np.float32(0.02)
    flag = torch.zeros(1, dtype=torch.int32, device=DEV)
    gpu_lib.quantize(torch.from_numpy(w).to(DEV), nonfinite_flag=flag, quant_type=quant_type)
    ok_flag = int(flag.item())
    for scale in (1e8 * div, 1e-6 * div):
        bad = w.copy()
        bad[1, 3, 64:128] *= np.float32(scale)
        flag.zero_()
        gpu_lib.quantize(torch.from_numpy(bad).to(DEV), nonfinite_flag=flag, quant_type=quant_type)
        got = int(flag.item())
        blocks = np.abs(bad.reshape(-1, 64)).max(axis=1).astype(np.float32) / np.float32(div)
        with np.errstate(over="ignore"):
            h = blocks.astype(np.float16)
        out = np.any((blocks != 0) & (~np.isfinite(h) | (blocks < np.float32(2.0 ** -14))))
        assert out, (quant_type, scale)  # the case does leave the range
        assert got == 2, (quant_type, scale, got)
    assert ok_flag == 0


def test_layer_input_beyond_fp16_is_observable(gpu_lib):
    """An activation past fp16's range: the check flags it before the
    forward, and the forward's output row carries non-finite values instead
    of a silently wrong finite result."""
    cfg = synth.config("tiny")
    gp, ga = oracle.quantize_blockwise(synth.stack_weights(cfg, "gu"))
    dp, da = oracle.quantize_blockwise(synth.stack_weights(cfg, "dn"))
    x = synth.activations(cfg).copy()
    x[5, 17] = 1.0e5
    xt = torch.from_numpy(x).to(DEV).to(torch.bfloat16)
    flags = torch.zeros(1, dtype=torch.int32, device=DEV)
    gpu_lib.f16_range_check(xt, flags)
    assert int(flags.item()) & 1
    st = [torch.from_numpy(a).to(DEV) for a in (gp, ga, dp, da)]
    y = gpu_lib.moe_forward(xt, torch.from_numpy(synth.router_logits(cfg)).to(DEV), cfg.k, *st,
                            y_dtype=torch.float32).cpu().numpy()
    assert not np.all(np.isfinite(y[5]))
    assert np.all(np.isfinite(np.delete(y, 5, axis=0)))
