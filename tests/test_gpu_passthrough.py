"""GPU parity of the bf16 / fp16 passthrough storage modes.

The stack conversion must give the oracle's bits; the grouped GEMM is exact
on integer-valued inputs and within fp32 summation error otherwise (weights
and activations enter the MFMAs as fp16: exact for fp16 stacks and for bf16
values in fp16's normal range); the layer forward meets the layer tolerance.
"""

import numpy as np
import pytest
import torch

import oracle
from grouped_nf4_gemm_quantize_amd import synth
from parity import assert_parity

pytestmark = pytest.mark.gpu
DEV = "cuda"
QTS = ["bf16", "fp16"]
TORCH_DT = {"bf16": torch.bfloat16, "fp16": torch.float16}


def gpu(a, dtype=None):
    t = torch.from_numpy(np.ascontiguousarray(a)).to(DEV)
    return t.to(dtype) if dtype is not None else t


def host(t):
    return t.detach().float().cpu().numpy() if t.dtype in (torch.bfloat16, torch.float16) \
        else t.detach().cpu().numpy()


def stack(bits, qt):
    """Oracle-stored uint16 patterns as a GPU tensor of the storage type."""
    return gpu(np.ascontiguousarray(bits).view(np.int16)).view(TORCH_DT[qt])


def bits_of(t):
    return t.detach().cpu().view(torch.int16).numpy().view(np.uint16)


@pytest.mark.parametrize("qt", QTS)
@pytest.mark.parametrize("src", ["f32", "bf16"])
def test_passthrough_store_is_bit_exact(gpu_lib, qt, src):
    rng = np.random.default_rng(10 + (qt == "fp16") + 2 * (src == "bf16"))
    mant = rng.uniform(1.0, 2.0, (3, 48, 320))
    exp = rng.integers(-26, 15, (3, 48, 320))
    w = (rng.choice([-1.0, 1.0], mant.shape) * mant * np.exp2(exp)).astype(np.float32)
    if src == "bf16":
        w = synth.round_to_bf16(w)
        wt = gpu(w, torch.bfloat16)
    else:
        wt = gpu(w)
    packed, absmax = gpu_lib.quantize(wt, quant_type=qt)
    assert absmax is None and packed.dtype == TORCH_DT[qt]
    assert np.array_equal(bits_of(packed), oracle.store16(w, qt))


@pytest.mark.parametrize("qt", QTS)
@pytest.mark.parametrize("K", [64, 128, 320])
def test_passthrough_gemm_exact_integer_case(gpu_lib, qt, K):
    """Integer weights and activations: every product and sum is exact in
    fp32, so the result is bit-exact; one, two and five k-steps, a ragged
    last N-tile (N = 656) and row tiles across three experts."""
    rng = np.random.default_rng(20 + K + (qt == "fp16"))
    E, N = 3, 656
    counts = [130, 0, 257]
    P = sum(counts)
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    bits = oracle.store16(rng.integers(-8, 9, size=(E, N, K)).astype(np.float32), qt)
    a = rng.integers(-4, 5, size=(P // 2 + 3, K)).astype(np.float16)
    gather = rng.integers(0, 2 * a.shape[0], size=P).astype(np.int32)
    out = gpu_lib.grouped_gemm(gpu(a), stack(bits, qt), None, gpu(offsets), P,
                               gather=gpu(gather), gather_div=2, out_dtype=torch.float32,
                               quant_type=qt)
    want = oracle.grouped_gemm16(a.astype(np.float64), bits, offsets, qt, gather=gather,
                                 gather_div=2)
    assert np.array_equal(host(out), want.astype(np.float32))


@pytest.mark.parametrize("qt", QTS)
@pytest.mark.parametrize("swiglu", [False, True])
@pytest.mark.parametrize("a_dt", ["fp16", "bf16"])
def test_passthrough_gemm_matches_oracle(gpu_lib, qt, swiglu, a_dt):
    rng = np.random.default_rng(30 + (qt == "fp16") + 2 * swiglu + 4 * (a_dt == "bf16"))
    E, N, K = 4, 640, 768
    counts = [200, 1, 0, 90]
    P = sum(counts)
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    bits = oracle.store16(rng.standard_normal((E, N, K)).astype(np.float32) * 0.05, qt)
    a = rng.standard_normal((150, K)).astype(np.float32)
    a = synth.round_to_bf16(a) if a_dt == "bf16" else a.astype(np.float16).astype(np.float32)
    gather = rng.integers(0, 300, size=P).astype(np.int32)
    rs = rng.uniform(0.2, 1.0, size=P).astype(np.float32)
    scatter = rng.permutation(P).astype(np.int32)
    out = gpu_lib.grouped_gemm(gpu(a, TORCH_DT[a_dt]), stack(bits, qt), None, gpu(offsets), P,
                               gather=gpu(gather), gather_div=2, swiglu=swiglu,
                               row_scale=gpu(rs), scatter=gpu(scatter),
                               out_dtype=torch.float32, quant_type=qt)
    ref = oracle.grouped_gemm16(a.astype(np.float64), bits, offsets, qt, gather=gather,
                                gather_div=2, swiglu=swiglu, row_scale=rs)
    # operands reach the MFMAs exactly (bf16 weights below fp16's normal
    # range aside); only the fp32 summation order differs
    assert_parity(host(out)[scatter], ref, fro_tol=1e-4, maxabs_tol=1e-3,
                  what=f"{qt} gemm", out_dtype="f32")


@pytest.mark.parametrize("qt", QTS)
@pytest.mark.parametrize("name,T,E", [("tiny", None, None), ("olmoe", 256, 16),
                                      ("decode", 1, 32)])
def test_passthrough_forward_matches_oracle(gpu_lib, qt, name, T, E):
    over = {} if T is None else dict(T=T, E=E)
    cfg = synth.config(name, **over)
    gu = oracle.store16(synth.stack_weights(cfg, "gu"), qt)
    dn = oracle.store16(synth.stack_weights(cfg, "dn"), qt)
    x = synth.activations(cfg)
    lg = synth.router_logits(cfg)
    y = gpu_lib.moe_forward(gpu(x, torch.bfloat16), gpu(lg), cfg.k, stack(gu, qt), None,
                            stack(dn, qt), None, renormalize=cfg.renormalize, quant_type=qt)
    ref = oracle.moe_forward16(x, lg, cfg.k, gu, dn, qt, cfg.renormalize)
    m = assert_parity(host(y), ref, what=f"{qt} forward {name}")
    print(qt, name, m)


def test_passthrough_rejects_adapters(gpu_lib):
    cfg = synth.config("tiny")
    gu = stack(oracle.store16(synth.stack_weights(cfg, "gu"), "bf16"), "bf16")
    dn = stack(oracle.store16(synth.stack_weights(cfg, "dn"), "bf16"), "bf16")
    x = gpu(synth.activations(cfg), torch.bfloat16)
    lg = gpu(synth.router_logits(cfg))
    A = torch.zeros((cfg.E, 8, cfg.H), dtype=torch.bfloat16, device=DEV)
    B = torch.zeros((cfg.E, 2 * cfg.I, 8), dtype=torch.bfloat16, device=DEV)
    with pytest.raises(Exception, match="adapters"):
        gpu_lib.moe_forward(x, lg, cfg.k, gu, None, dn, None, gu_lora=(A, B, 2.0),
                            quant_type="bf16")
