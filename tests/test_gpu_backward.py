"""GPU parity of the backward path: grouped dgrad and the layer backward.

The HIP kernels (through the C ABI) against the CPU oracle's backward
(``oracle/backward.py``, pinned by finite differences and fp64 autograd).
Exactly representable cases must match bit for bit; everything else meets
the tolerance in ``parity.py``.
"""

import numpy as np
import pytest
import torch

import oracle
from grouped_nf4_gemm_quantize_amd import synth
from fullsize import full_stacks
from parity import assert_parity, assert_parity_literal, metrics

pytestmark = pytest.mark.gpu
DEV = "cuda"


def gpu(a, dtype=None):
    t = torch.from_numpy(np.ascontiguousarray(a)).to(DEV)
    return t.to(dtype) if dtype is not None else t


def host(t):
    return t.detach().float().cpu().numpy() if t.dtype in (torch.bfloat16, torch.float16) \
        else t.detach().cpu().numpy()


def _int_stack(rng, E, N, K):
    codes = rng.choice(np.array([0, 7, 15], dtype=np.uint8), size=(E, N, K))
    codes[..., ::64] = 15
    packed = oracle.pack_codes(codes)
    shifts = rng.integers(-3, 2, size=(E, N, K // 64))
    absmax = np.ldexp(np.ones_like(shifts, dtype=np.float32), shifts).astype(np.float32)
    ints = np.where(codes == 15, 1, np.where(codes == 0, -1, 0)).astype(np.float64)
    w = ints * np.repeat(absmax.astype(np.float64), 64, axis=-1)
    return packed, absmax, w


def _random_stack(rng, E, N, K, quant_type="nf4"):
    w = rng.standard_normal((E, N, K), dtype=np.float32) * np.float32(0.05)
    return oracle.quantize_blockwise(w, quant_type=quant_type)


# -------------------------------------------------------------- grouped dgrad

def test_dgrad_exact_integer_case(gpu_lib):
    """Exactly representable operands: bit-exact, over several row tiles, a
    ragged last column tile (K = 640) and three contraction steps."""
    rng = np.random.default_rng(21)
    E, N, K = 4, 192, 640
    counts = [5, 0, 145, 300]
    P = sum(counts)
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    packed, absmax, w = _int_stack(rng, E, N, K)
    a = rng.integers(-4, 5, size=(P // 2 + 7, N)).astype(np.float16)
    gather = rng.integers(0, 2 * a.shape[0], size=P).astype(np.int32)
    out = gpu_lib.grouped_dgrad(gpu(a), gpu(packed), gpu(absmax), gpu(offsets), P,
                                gather=gpu(gather), gather_div=2, out_dtype=torch.float32)
    got = host(out)
    want = np.zeros((P, K))
    for e in range(E):
        lo, hi = offsets[e], offsets[e + 1]
        want[lo:hi] = a[gather[lo:hi] // 2].astype(np.float64) @ w[e]
    assert np.array_equal(got, want.astype(np.float32))


@pytest.mark.parametrize("quant_type", ["nf4", "fp4"])
def test_dgrad_matches_oracle(gpu_lib, quant_type):
    rng = np.random.default_rng(22 if quant_type == "nf4" else 23)
    E, N, K = 5, 320, 768
    counts = [130, 1, 0, 77, 260]
    P = sum(counts)
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    packed, absmax = _random_stack(rng, E, N, K, quant_type)
    a = rng.standard_normal((300, N)).astype(np.float16)
    gather = rng.integers(0, 300 * 3, size=P).astype(np.int32)
    rs = rng.uniform(0.1, 1.0, size=300 * 3).astype(np.float32)  # indexed by gather[i]
    scatter = rng.permutation(P).astype(np.int32)
    out = gpu_lib.grouped_dgrad(gpu(a), gpu(packed), gpu(absmax), gpu(offsets), P,
                                gather=gpu(gather), gather_div=3, row_scale=gpu(rs),
                                scatter=gpu(scatter), out_dtype=torch.float32,
                                quant_type=quant_type)
    ref = oracle.grouped_dgrad(a.astype(np.float64), packed, absmax, offsets, gather=gather,
                               gather_div=3, row_scale=rs[gather], quant_type=quant_type)
    got = host(out)[scatter]
    # the only roundings are the fp16 weight operands (level, absmax, product)
    assert_parity(got, ref, fro_tol=2e-3, maxabs_tol=2e-2, what="dgrad", out_dtype="f32")


def test_dgrad_bf16_rows_and_outputs(gpu_lib):
    rng = np.random.default_rng(24)
    E, N, K = 3, 256, 512
    counts = [40, 200, 17]
    P = sum(counts)
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    packed, absmax = _random_stack(rng, E, N, K)
    a = synth.round_to_bf16(rng.standard_normal((P, N), dtype=np.float32))
    ref = oracle.grouped_dgrad(a.astype(np.float64), packed, absmax, offsets)
    for out_dt, name in ((torch.bfloat16, "bf16"), (torch.float16, "f16"), (torch.float32, "f32")):
        out = gpu_lib.grouped_dgrad(gpu(a, torch.bfloat16), gpu(packed), gpu(absmax),
                                    gpu(offsets), P, out_dtype=out_dt)
        tol = 5e-3 if name == "bf16" else 2e-3
        assert_parity(host(out), ref, fro_tol=tol, maxabs_tol=2e-2, what=name, out_dtype=name)


def test_dgrad_single_expert_is_a_dense_matmul(gpu_lib):
    """E = 1: a @ W against torch.matmul on the fp16-rounded dequantised
    weights (the kernel's operands), leaving only summation order."""
    rng = np.random.default_rng(25)
    N, K, P = 448, 384, 333
    packed, absmax = _random_stack(rng, 1, N, K)
    offsets = np.array([0, P], dtype=np.int32)
    a = rng.standard_normal((P, N)).astype(np.float16)
    w16 = (oracle.nf4_codebook()[oracle.unpack_codes(packed)].astype(np.float16).astype(np.float32)
           * np.repeat(absmax.astype(np.float16).astype(np.float32), 64, axis=-1))[0]
    w16 = w16.astype(np.float16).astype(np.float32)
    out = gpu_lib.grouped_dgrad(gpu(a), gpu(packed), gpu(absmax), gpu(offsets), P,
                                out_dtype=torch.float32)
    want = torch.matmul(gpu(a).float(), gpu(w16))
    assert torch.allclose(out, want, rtol=1e-5, atol=1e-4)


def test_dgrad_is_the_adjoint_of_the_forward_kernel(gpu_lib):
    """<gemm(a), b> = <a, dgrad(b)>, both sides computed by the HIP kernels."""
    rng = np.random.default_rng(26)
    E, N, K = 3, 256, 320
    counts = [100, 3, 190]
    P = sum(counts)
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    packed, absmax = _random_stack(rng, E, N, K)
    a = rng.standard_normal((P, K)).astype(np.float16)
    b = rng.standard_normal((P, N)).astype(np.float16)
    fwd = gpu_lib.grouped_gemm(gpu(a), gpu(packed), gpu(absmax), gpu(offsets), P,
                               out_dtype=torch.float32)
    bwd = gpu_lib.grouped_dgrad(gpu(b), gpu(packed), gpu(absmax), gpu(offsets), P,
                                out_dtype=torch.float32)
    lhs = float((fwd.double() * gpu(b).double()).sum())
    rhs = float((gpu(a).double() * bwd.double()).sum())
    assert abs(lhs - rhs) <= 1e-5 * (abs(lhs) + np.sqrt(P * N))


def test_dgrad_swiglu_backward_epilogue(gpu_lib):
    rng = np.random.default_rng(27)
    E, H, I = 4, 256, 320   # the down stack [E, H, I]: contraction H, output I
    counts = [70, 0, 200, 33]
    P = sum(counts)
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    packed, absmax = _random_stack(rng, E, H, I)
    dy = rng.standard_normal((P // 2 + 5, H)).astype(np.float16)
    gather = rng.integers(0, 2 * dy.shape[0], size=P).astype(np.int32)
    rs = rng.uniform(0.1, 1.0, size=2 * dy.shape[0]).astype(np.float32)
    g = (rng.standard_normal((P, 2 * I)) * 1.5).astype(np.float16)
    out = gpu_lib.grouped_dgrad(gpu(dy), gpu(packed), gpu(absmax), gpu(offsets), P,
                                gather=gpu(gather), gather_div=2, g_pre=gpu(g),
                                row_scale=gpu(rs), out_dtype=torch.float32)
    dh = oracle.grouped_dgrad(dy.astype(np.float64), packed, absmax, offsets, gather=gather,
                              gather_div=2, row_scale=rs[gather])
    ref = oracle.swiglu_backward(g.astype(np.float64), dh)
    assert out.shape == (P, 2 * I)
    assert_parity(host(out), ref, fro_tol=2e-3, maxabs_tol=2e-2, what="swiglu bwd",
                  out_dtype="f32")


@pytest.mark.parametrize("lora", [False, True])
def test_swiglu_bwd_gemm_matches_oracle(gpu_lib, lora):
    """The gate_up GEMM recomputed with the SwiGLU backward as its epilogue:
    dG = [dh * up * silu'(gate) | dh * silu(gate)] and h = silu(gate) * up,
    against the oracle's fp64 G from the same bytes (several row tiles, an
    empty expert, a one-row expert, I = 272 so the last column tile is
    ragged)."""
    rng = np.random.default_rng(300 + lora)
    E, I, K = 5, 272, 320
    N = 2 * I
    counts = [130, 1, 0, 77, 260]
    P = sum(counts)
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    packed, absmax = _random_stack(rng, E, N, K)
    a = rng.standard_normal((300, K)).astype(np.float16)
    gather = rng.integers(0, 300 * 3, size=P).astype(np.int32)
    dh = rng.standard_normal((P, I)).astype(np.float16)
    lo = lo_ref = None
    if lora:
        r = 8
        A = synth.round_to_bf16(rng.standard_normal((E, r, K), dtype=np.float32) * 0.05)
        B = synth.round_to_bf16(rng.standard_normal((E, N, r), dtype=np.float32) * 0.05)
        lo = (gpu(A, torch.bfloat16), gpu(B, torch.bfloat16), 2.0)
        lo_ref = (A, B, 2.0)
    h = torch.full((P, I), float("nan"), dtype=torch.float16, device=DEV)
    out = gpu_lib.grouped_gemm_swiglu_bwd(gpu(a), gpu(packed), gpu(absmax), gpu(offsets), P,
                                          gpu(dh), gather=gpu(gather), gather_div=3, lora=lo,
                                          h_out=h)
    G = oracle.grouped_gemm(a.astype(np.float64), packed, absmax, offsets, gather=gather,
                            gather_div=3, lora=lo_ref)
    ref = oracle.swiglu_backward(G, dh.astype(np.float64))
    assert_parity(host(out), ref, what="SwiGLU-backward GEMM dG", out_dtype="f16")
    href = oracle.silu(G[:, :I]) * G[:, I:]
    assert_parity(host(h), href, what="SwiGLU-backward GEMM h", out_dtype="f16")
    # without h_out the same dG, bit for bit
    out2 = gpu_lib.grouped_gemm_swiglu_bwd(gpu(a), gpu(packed), gpu(absmax), gpu(offsets), P,
                                           gpu(dh), gather=gpu(gather), gather_div=3, lora=lo)
    assert torch.equal(out, out2)


def test_swiglu_bwd_gemm_leaves_rows_beyond_offsets_untouched(gpu_lib):
    """Rows at and past offsets[E] of dG and h are not written."""
    rng = np.random.default_rng(33)
    E, I, K = 3, 128, 128
    counts = [40, 0, 90]
    P = sum(counts) + 30
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    packed, absmax = _random_stack(rng, E, 2 * I, K)
    a = rng.standard_normal((P, K)).astype(np.float16)
    dh = rng.standard_normal((P, I)).astype(np.float16)
    out = torch.full((P, 2 * I), float("nan"), dtype=torch.float16, device=DEV)
    h = torch.full((P, I), float("nan"), dtype=torch.float16, device=DEV)
    gpu_lib.grouped_gemm_swiglu_bwd(gpu(a), gpu(packed), gpu(absmax), gpu(offsets), P, gpu(dh),
                                    out=out, h_out=h)
    n = int(offsets[-1])
    assert torch.isnan(out[n:]).all() and torch.isnan(h[n:]).all()
    assert not torch.isnan(out[:n]).any() and not torch.isnan(h[:n]).any()


def test_dgrad_leaves_rows_beyond_offsets_untouched(gpu_lib):
    rng = np.random.default_rng(28)
    packed, absmax = _random_stack(rng, 2, 64, 64)
    offsets = np.array([0, 3, 7], dtype=np.int32)
    a = rng.standard_normal((7, 64)).astype(np.float16)
    out = torch.full((12, 64), 7.0, dtype=torch.float32, device=DEV)
    gpu_lib.grouped_dgrad(gpu(a), gpu(packed), gpu(absmax), gpu(offsets), 12, out=out)
    assert torch.all(out[7:] == 7.0)


# ------------------------------------------------------------ layer backward

def _stacks(cfg, quant_type="nf4"):
    gu = synth.stack_weights(cfg, "gu")
    dn = synth.stack_weights(cfg, "dn")
    return (oracle.quantize_blockwise(gu, quant_type=quant_type)
            + oracle.quantize_blockwise(dn, quant_type=quant_type))


def _lora(cfg):
    lw = synth.lora_weights(cfg)
    if lw is None:
        return None, None, None, None
    s = cfg.lora_scale
    return ((gpu(lw["a_gu"], torch.bfloat16), gpu(lw["b_gu"], torch.bfloat16), s),
            (gpu(lw["a_dn"], torch.bfloat16), gpu(lw["b_dn"], torch.bfloat16), s),
            (lw["a_gu"], lw["b_gu"], s), (lw["a_dn"], lw["b_dn"], s))


def _backward_case(gpu_lib, cfg, dx_dtype=torch.bfloat16, x_dtype=torch.bfloat16,
                   quant_type="nf4"):
    gp, ga, dp, da = _stacks(cfg, quant_type)
    x = synth.activations(cfg)
    lg = synth.router_logits(cfg)
    dy = synth.output_grad(cfg)
    glo, dlo, glo_r, dlo_r = _lora(cfg)
    dx, grads = gpu_lib.moe_backward(gpu(x, x_dtype), gpu(lg), gpu(dy, torch.bfloat16), cfg.k,
                                     gpu(gp), gpu(ga), gpu(dp), gpu(da), glo, dlo,
                                     cfg.renormalize, dx_dtype=dx_dtype,
                                     quant_type=quant_type)
    ref = oracle.moe_backward(x, lg, dy, cfg.k, gp, ga, dp, da, glo_r, dlo_r, cfg.renormalize,
                              quant_type=quant_type)
    return host(dx), {k: host(v) for k, v in grads.items()}, ref


def _check_lora_grads(grads, ref, what):
    """Adapter gradients: each expert's block is its own output, so the
    tolerance applies per expert that received rows (relative to that
    expert's RMS); an expert without rows must get exact zeros."""
    for name in ("dA_gu", "dB_gu", "dA_dn", "dB_dn"):
        if name not in grads:
            continue
        g, r = grads[name], ref[name]
        assert metrics(g, r, "f32")["fro"] <= 5e-3, (what, name)
        for e in range(r.shape[0]):
            if not np.any(r[e]):
                assert not np.any(g[e]), (what, name, e)
                continue
            assert_parity(g[e], r[e], fro_tol=5e-3, maxabs_tol=2e-2,
                          what=f"{what} {name} expert {e}", out_dtype="f32")


@pytest.mark.parametrize("variant", ["plain", "lora", "norenorm", "f16_in_f32_out"])
def test_backward_tiny(gpu_lib, variant):
    over = {}
    if variant == "lora":
        over = dict(lora_r=8, lora_alpha=16.0)
    if variant == "norenorm":
        over = dict(renormalize=False)
    cfg = synth.config("tiny", **over)
    if variant == "f16_in_f32_out":
        dx, grads, ref = _backward_case(gpu_lib, cfg, torch.float32, torch.float16)
        assert_parity(dx, ref["dx"], what=variant, out_dtype="f32")
    else:
        dx, grads, ref = _backward_case(gpu_lib, cfg)
        assert_parity(dx, ref["dx"], what=variant)
    _check_lora_grads(grads, ref, variant)


@pytest.mark.parametrize("name,T,E", [("olmoe", 320, 16), ("qwen3_zipf", 600, 24),
                                      ("qlora", 256, 16)])
def test_backward_real_widths(gpu_lib, name, T, E):
    """Full H and I of the configs with fewer experts/tokens (oracle in seconds)."""
    cfg = synth.config(name, T=T, E=E)
    dx, grads, ref = _backward_case(gpu_lib, cfg)
    m = assert_parity(dx, ref["dx"], what=name)
    print(name, m)
    _check_lora_grads(grads, ref, name)


def test_backward_fp4_storage(gpu_lib):
    cfg = synth.config("tiny", lora_r=8, lora_alpha=16.0)
    dx, grads, ref = _backward_case(gpu_lib, cfg, quant_type="fp4")
    assert_parity(dx, ref["dx"], what="fp4")
    _check_lora_grads(grads, ref, "fp4")


def test_backward_is_deterministic(gpu_lib):
    cfg = synth.config("tiny", T=200, lora_r=8, lora_alpha=16.0)
    gp, ga, dp, da = _stacks(cfg)
    x = gpu(synth.activations(cfg), torch.bfloat16)
    lg = gpu(synth.router_logits(cfg))
    dy = gpu(synth.output_grad(cfg), torch.bfloat16)
    glo, dlo, _, _ = _lora(cfg)
    args = (x, lg, dy, cfg.k, gpu(gp), gpu(ga), gpu(dp), gpu(da), glo, dlo)
    dx1, g1 = gpu_lib.moe_backward(*args)
    dx2, g2 = gpu_lib.moe_backward(*args)
    assert torch.equal(dx1, dx2)
    for k in g1:
        assert torch.equal(g1[k], g2[k]), k


def test_backward_bf16_adapters_match_their_f16_copies_bitwise(gpu_lib):
    """bf16 adapters are rounded to fp16 (nearest even) for the recomputed
    gate_up and the adapter passes; handing in the same adapters already
    rounded by torch gives the same dx and adapter gradients, bit for bit."""
    cfg = synth.config("tiny", T=200, lora_r=8, lora_alpha=16.0)
    gp, ga, dp, da = _stacks(cfg)
    x = gpu(synth.activations(cfg), torch.bfloat16)
    lg = gpu(synth.router_logits(cfg))
    dy = gpu(synth.output_grad(cfg), torch.bfloat16)
    glo, dlo, _, _ = _lora(cfg)
    half = lambda lo: (lo[0].half(), lo[1].half(), lo[2])
    st = (gpu(gp), gpu(ga), gpu(dp), gpu(da))
    dx1, g1 = gpu_lib.moe_backward(x, lg, dy, cfg.k, *st, glo, dlo, dx_dtype=torch.float32)
    dx2, g2 = gpu_lib.moe_backward(x, lg, dy, cfg.k, *st, half(glo), half(dlo),
                                   dx_dtype=torch.float32)
    assert torch.equal(dx1, dx2)
    for k in g1:
        assert torch.equal(g1[k], g2[k]), k
    assert torch.count_nonzero(g1["dA_gu"]) > 0


def test_backward_with_zero_b_has_zero_a_gradient(gpu_lib):
    """B = 0 adapters: dA is exactly zero and dx equals the adapter-free dx
    bit for bit (every adapter term adds exact zeros), with the gate_up
    adapter alone and with both."""
    cfg = synth.config("tiny", lora_r=8, lora_alpha=16.0)
    gp, ga, dp, da = _stacks(cfg)
    x = gpu(synth.activations(cfg), torch.bfloat16)
    lg = gpu(synth.router_logits(cfg))
    dy = gpu(synth.output_grad(cfg), torch.bfloat16)
    glo, dlo, _, _ = _lora(cfg)
    glo = (glo[0], torch.zeros_like(glo[1]), glo[2])
    dlo = (dlo[0], torch.zeros_like(dlo[1]), dlo[2])
    st = (gpu(gp), gpu(ga), gpu(dp), gpu(da))
    dx0, _ = gpu_lib.moe_backward(x, lg, dy, cfg.k, *st, dx_dtype=torch.float32)
    dxg, gg = gpu_lib.moe_backward(x, lg, dy, cfg.k, *st, glo, None, dx_dtype=torch.float32)
    assert torch.count_nonzero(gg["dA_gu"]) == 0 and torch.count_nonzero(gg["dB_gu"]) > 0
    assert torch.equal(dxg, dx0)
    dx, g = gpu_lib.moe_backward(x, lg, dy, cfg.k, *st, glo, dlo, dx_dtype=torch.float32)
    assert torch.count_nonzero(g["dA_gu"]) == 0 and torch.count_nonzero(g["dA_dn"]) == 0
    assert torch.count_nonzero(g["dB_gu"]) > 0 and torch.count_nonzero(g["dB_dn"]) > 0
    assert torch.equal(dx, dx0)


@pytest.mark.slow
@pytest.mark.parametrize("name", ["olmoe", "qlora"])
def test_backward_full_size(gpu_lib, name):
    """The full-size layer backward on the GPU against the oracle's on every
    token: dx of all T tokens (bf16, and fp32 under the clause as written)
    and, with adapters, every expert's adapter gradients.  The stacks are the
    full-size ones whose every expert was checked bit for bit."""
    cfg = synth.config(name)
    (gp, ga, dp, da), (gpr, gar, dpr, dar) = full_stacks(gpu_lib, cfg)
    x = synth.activations(cfg)
    lg = synth.router_logits(cfg)
    dy = synth.output_grad(cfg)
    glo, dlo, glo_r, dlo_r = _lora(cfg)
    args = (gpu(x, torch.bfloat16), gpu(lg), gpu(dy, torch.bfloat16), cfg.k, gp, ga, dp, da,
            glo, dlo, cfg.renormalize)
    dx, grads = gpu_lib.moe_backward(*args)
    dx, grads = host(dx), {n: host(v) for n, v in grads.items()}
    dxf, _ = gpu_lib.moe_backward(*args, dx_dtype=torch.float32)
    ref = oracle.moe_backward(x, lg, dy, cfg.k, gpr, gar, dpr, dar, glo_r, dlo_r,
                              cfg.renormalize)
    m = assert_parity(dx, ref["dx"], what=f"{name} dx")
    mf = assert_parity_literal(host(dxf), ref["dx"], what=f"{name} dx f32")
    print(name, "dx bf16", m, "f32", mf)
    if glo is not None:
        _check_lora_grads(grads, ref, f"{name} full size")


@pytest.mark.parametrize("T,E,k,skew", [(40, 300, 4, False), (96, 8, 2, True), (1, 16, 4, False)])
def test_backward_degenerate_routings(gpu_lib, T, E, k, skew):
    """Many empty experts; every token on the same experts (one expert holds
    all rows); a single token.  dx and the adapter gradients vs the oracle."""
    cfg = synth.config("tiny", T=T, E=E, k=k, lora_r=8, lora_alpha=16.0)
    gp, ga, dp, da = _stacks(cfg)
    x = synth.activations(cfg)
    lg = synth.router_logits(cfg)
    if skew:
        lg = lg.copy()
        lg[:, 3] += 50.0
        lg[:, 5] += 40.0
    dy = synth.output_grad(cfg)
    glo, dlo, glo_r, dlo_r = _lora(cfg)
    dx, grads = gpu_lib.moe_backward(gpu(x, torch.bfloat16), gpu(lg), gpu(dy, torch.bfloat16),
                                     cfg.k, gpu(gp), gpu(ga), gpu(dp), gpu(da), glo, dlo,
                                     dx_dtype=torch.float32)
    ref = oracle.moe_backward(x, lg, dy, cfg.k, gp, ga, dp, da, glo_r, dlo_r)
    assert_parity(host(dx), ref["dx"], what=f"degenerate T={T} E={E}", out_dtype="f32")
    _check_lora_grads({n: host(v) for n, v in grads.items()}, ref, "degenerate")
    used = set(ref["info"]["ids"].reshape(-1).tolist())
    for e in range(E):
        if e not in used:
            assert torch.count_nonzero(grads["dA_gu"][e]) == 0


def test_dgrad_minimal_contraction_and_width(gpu_lib):
    """N = K = 64: one contraction step, one absmax block per row."""
    rng = np.random.default_rng(29)
    packed, absmax = _random_stack(rng, 2, 64, 64)
    offsets = np.array([0, 5, 9], dtype=np.int32)
    a = rng.standard_normal((9, 64)).astype(np.float16)
    out = gpu_lib.grouped_dgrad(gpu(a), gpu(packed), gpu(absmax), gpu(offsets), 9,
                                out_dtype=torch.float32)
    ref = oracle.grouped_dgrad(a.astype(np.float64), packed, absmax, offsets)
    assert_parity(host(out), ref, fro_tol=2e-3, maxabs_tol=2e-2, what="N=K=64", out_dtype="f32")


def test_backward_in_hip_graph_replays(gpu_lib):
    """The layer backward (with adapters) captured once and replayed, with
    eager work and clearing of every buffer between replays: each replay
    equals the eager result bit for bit."""
    cfg = synth.config("tiny", lora_r=8, lora_alpha=16.0)
    gp, ga, dp, da = _stacks(cfg)
    x = gpu(synth.activations(cfg), torch.bfloat16)
    lg = gpu(synth.router_logits(cfg))
    dy = gpu(synth.output_grad(cfg), torch.bfloat16)
    glo, dlo, _, _ = _lora(cfg)
    st = (gpu(gp), gpu(ga), gpu(dp), gpu(da))
    dx_e, g_e = gpu_lib.moe_backward(x, lg, dy, cfg.k, *st, glo, dlo)
    dx_e, g_e = dx_e.clone(), {k_: v.clone() for k_, v in g_e.items()}
    nbytes = gpu_lib.backward_workspace_bytes(cfg.T, cfg.H, cfg.I, cfg.E, cfg.k, 8)
    ws = torch.empty(nbytes, dtype=torch.uint8, device=DEV)
    dx = torch.empty_like(dx_e)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        _, grads = gpu_lib.moe_backward(x, lg, dy, cfg.k, *st, glo, dlo, dx=dx, workspace=ws)
    torch.cuda.current_stream().wait_stream(s)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        _, grads = gpu_lib.moe_backward(x, lg, dy, cfg.k, *st, glo, dlo, dx=dx, workspace=ws)
    for _ in range(3):
        dx.zero_()
        ws.zero_()
        for v in grads.values():
            v.fill_(7.0)
        gpu_lib.moe_backward(x, lg, dy, cfg.k, *st, glo, dlo)  # eager work in between
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(dx, dx_e)
        for k_, v in grads.items():
            assert torch.equal(v, g_e[k_]), k_
