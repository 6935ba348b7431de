"""The allocation-free layer forward (moe_expert_forward_noalloc) through the
C ABI: the same result, bit for bit, as moe_expert_forward with a workspace,
on consecutive calls whose second input is smaller (so it reuses the scratch
memory the first left behind), on the prefill and the single-token decode
paths; refused sizes; a captured graph replayed several times.

The expected values come from moe_expert_forward, whose own parity with the
oracle is tested elsewhere; one case here is also checked against the oracle.
"""

import numpy as np
import pytest
import torch

import oracle
from grouped_nf4_gemm_quantize_amd import binding, synth
from parity import assert_parity

pytestmark = pytest.mark.gpu
DEV = "cuda"


def gpu(a, dtype=None):
    t = torch.from_numpy(np.ascontiguousarray(a)).to(DEV)
    return t.to(dtype) if dtype is not None else t


def _case(cfg, lora=False):
    gu = synth.stack_weights(cfg, "gu")
    dn = synth.stack_weights(cfg, "dn")
    gp, ga = oracle.quantize_blockwise(gu)
    dp, da = oracle.quantize_blockwise(dn)
    x = synth.activations(cfg)
    lg = synth.router_logits(cfg)
    args = [gpu(x, torch.bfloat16), gpu(lg), cfg.k, gpu(gp), gpu(ga), gpu(dp), gpu(da)]
    lo = (None, None)
    lo_ref = (None, None)
    if lora:
        lw = synth.lora_weights(cfg)
        s = cfg.lora_scale
        lo = ((gpu(lw["a_gu"], torch.bfloat16), gpu(lw["b_gu"], torch.bfloat16), s),
              (gpu(lw["a_dn"], torch.bfloat16), gpu(lw["b_dn"], torch.bfloat16), s))
        lo_ref = ((lw["a_gu"], lw["b_gu"], s), (lw["a_dn"], lw["b_dn"], s))
    ref = (x, lg, cfg.k, gp, ga, dp, da) + lo_ref
    return args, lo, ref


@pytest.mark.parametrize("first,second", [
    (dict(name="qwen3_zipf", T=96, E=16), dict(name="decode", E=16)),
    (dict(name="qlora", T=80, E=16), dict(name="qlora", T=17, E=16)),
    (dict(name="olmoe", T=64, E=8), dict(name="tiny", T=5)),
])
def test_noalloc_matches_the_workspace_forward(gpu_lib, first, second):
    for spec in (first, second):
        spec = dict(spec)
        cfg = synth.config(spec.pop("name"), **spec)
        args, lo, ref = _case(cfg, lora=cfg.lora_r > 0)
        for y_dtype in (torch.bfloat16, torch.float32):
            want = gpu_lib.moe_forward(*args, *lo, cfg.renormalize, y_dtype=y_dtype)
            got = torch.full_like(want, float("nan"))
            gpu_lib.moe_forward_noalloc(*args, *lo, cfg.renormalize, y=got)
            torch.cuda.synchronize()
            assert torch.equal(got, want), (cfg, y_dtype)
        y_ref, _ = oracle.moe_forward(*ref, renormalize=cfg.renormalize)
        assert_parity(got.cpu().numpy(), y_ref, 2e-3, 2e-2, what=f"noalloc {cfg}", out_dtype="f32")


def test_noalloc_refuses_sizes_beyond_its_scratch(gpu_lib):
    cfg = synth.config("qwen3_zipf", T=1024, E=16)
    need = gpu_lib.forward_workspace_bytes(cfg.T, cfg.H, cfg.I, cfg.E, cfg.k)
    assert need > binding.NOALLOC_SCRATCH_BYTES
    args, lo, _ = _case(cfg)
    y = torch.zeros((cfg.T, cfg.H), dtype=torch.bfloat16, device=DEV)
    with pytest.raises(binding.Nf4MoeError) as err:
        gpu_lib.moe_forward_noalloc(*args, y=y)
    assert err.value.status == -6 and "scratch" in str(err.value)
    torch.cuda.synchronize()
    assert torch.count_nonzero(y) == 0  # nothing was launched


def test_noalloc_graph_replays(gpu_lib):
    cfg = synth.config("qwen3_zipf", T=48, E=16)
    args, lo, _ = _case(cfg)
    y = torch.empty((cfg.T, cfg.H), dtype=torch.float32, device=DEV)
    eager = gpu_lib.moe_forward(*args, y_dtype=torch.float32).clone()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        gpu_lib.moe_forward_noalloc(*args, y=y)
    torch.cuda.current_stream().wait_stream(s)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        gpu_lib.moe_forward_noalloc(*args, y=y)
    small = synth.config("decode", E=16)
    sargs, _, _ = _case(small)
    for _ in range(3):
        y.fill_(7.0)
        gpu_lib.moe_forward_noalloc(*sargs)  # other eager work on the same scratch
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y, eager)
