"""Pins for the oracle's backward of the routed-expert layer (CPU only).

The backward is pinned to things other than its own formulas:

* central finite differences of the (separately pinned) oracle forward, for
  the input and each of the four adapter matrices;
* PyTorch autograd in fp64 through an independent dense formulation of the
  forward (all experts evaluated for every token, masked by the routing);
* the adjoint identity between the grouped GEMM and the grouped dgrad, and an
  exact integer case of the dgrad checked by brute force;
* closed forms of silu's derivative, zero and linearity properties.
"""

import numpy as np
import pytest
import torch

import oracle


def _stack(rng, E, N, K, scale=0.05):
    w = rng.standard_normal((E, N, K), dtype=np.float32) * np.float32(scale)
    return oracle.quantize_blockwise(w)


def _lora(rng, E, r, n_in, n_out, scale=2.0, amp=0.1):
    A = rng.standard_normal((E, r, n_in)) * amp
    B = rng.standard_normal((E, n_out, r)) * amp
    return (A, B, scale)


def _problem(seed=0, E=4, H=64, I=64, k=2, T=6, r=4, lora=True):
    rng = np.random.default_rng(seed)
    gu = _stack(rng, E, 2 * I, H)
    dn = _stack(rng, E, H, I)
    x = rng.standard_normal((T, H))
    logits = rng.standard_normal((T, E)).astype(np.float32)
    dy = rng.standard_normal((T, H))
    lgu = _lora(rng, E, r, H, 2 * I) if lora else None
    ldn = _lora(rng, E, r, I, H) if lora else None
    return dict(x=x, logits=logits, dy=dy, k=k, gu=gu, dn=dn, lgu=lgu, ldn=ldn)


def _loss(p, x=None, lgu=None, ldn=None):
    y, _ = oracle.moe_forward(x if x is not None else p["x"], p["logits"], p["k"],
                              p["gu"][0], p["gu"][1], p["dn"][0], p["dn"][1],
                              lgu if lgu is not None else p["lgu"],
                              ldn if ldn is not None else p["ldn"])
    return float(np.sum(p["dy"] * y))


def _backward(p):
    return oracle.moe_backward(p["x"], p["logits"], p["dy"], p["k"], p["gu"][0],
                               p["gu"][1], p["dn"][0], p["dn"][1], p["lgu"], p["ldn"])


def _with(lora, which, value):
    A, B, s = lora
    return (value, B, s) if which == 0 else (A, value, s)


@pytest.mark.parametrize("target", ["x", "A_gu", "B_gu", "A_dn", "B_dn"])
def test_backward_matches_central_differences(target):
    p = _problem(seed=3)
    g = _backward(p)
    rng = np.random.default_rng(11)
    eps = 1e-5
    if target == "x":
        d = rng.standard_normal(p["x"].shape)
        plus, minus = _loss(p, x=p["x"] + eps * d), _loss(p, x=p["x"] - eps * d)
        analytic = float(np.sum(g["dx"] * d))
    else:
        name = "lgu" if target.endswith("gu") else "ldn"
        which = 0 if target.startswith("A") else 1
        base = p[name][which]
        d = rng.standard_normal(base.shape)
        kw_p = {name: _with(p[name], which, base + eps * d)}
        kw_m = {name: _with(p[name], which, base - eps * d)}
        plus, minus = _loss(p, **kw_p), _loss(p, **kw_m)
        analytic = float(np.sum(g["d" + target] * d))
    numeric = (plus - minus) / (2 * eps)
    assert abs(analytic - numeric) <= 1e-6 * max(1.0, abs(numeric)), (analytic, numeric)


def test_backward_matches_autograd_of_a_dense_formulation():
    """Every expert on every token, masked by a dense routing-weight matrix."""
    p = _problem(seed=5, E=5, T=7, k=3)
    g = _backward(p)
    E = p["gu"][0].shape[0]
    I = p["dn"][0].shape[2] * 2
    W_gu = torch.from_numpy(oracle.dequantize_blockwise(*p["gu"]).astype(np.float64))
    W_dn = torch.from_numpy(oracle.dequantize_blockwise(*p["dn"]).astype(np.float64))
    # dense [T, E] routing weights from a softmax over each token's top-k
    lg = torch.from_numpy(p["logits"].astype(np.float64))
    top = torch.topk(lg, p["k"], dim=1)
    dense_w = torch.zeros_like(lg).scatter(1, top.indices, torch.softmax(top.values, dim=1))
    x = torch.tensor(p["x"], requires_grad=True)
    Ag = torch.tensor(p["lgu"][0], requires_grad=True)
    Bg = torch.tensor(p["lgu"][1], requires_grad=True)
    Ad = torch.tensor(p["ldn"][0], requires_grad=True)
    Bd = torch.tensor(p["ldn"][1], requires_grad=True)
    s = p["lgu"][2]
    y = torch.zeros_like(x)
    for e in range(E):
        gg = x @ W_gu[e].T + s * (x @ Ag[e].T) @ Bg[e].T
        h = torch.nn.functional.silu(gg[:, :I]) * gg[:, I:]
        o = h @ W_dn[e].T + s * (h @ Ad[e].T) @ Bd[e].T
        y = y + dense_w[:, e : e + 1] * o
    (y * torch.from_numpy(p["dy"])).sum().backward()
    for name, t in (("dx", x), ("dA_gu", Ag), ("dB_gu", Bg), ("dA_dn", Ad), ("dB_dn", Bd)):
        assert np.allclose(g[name], t.grad.numpy(), rtol=1e-10, atol=1e-12), name


def test_dgrad_is_the_adjoint_of_the_grouped_gemm():
    """<gemm(a), b> == <a, dgrad(b)> per expert group, with row scales."""
    rng = np.random.default_rng(2)
    E, N, K = 3, 96, 128
    packed, absmax = _stack(rng, E, N, K)
    offsets = np.array([0, 9, 9, 23], dtype=np.int32)
    P = 23
    a = rng.standard_normal((P, K))
    b = rng.standard_normal((P, N))
    rs = rng.uniform(0.5, 2.0, size=P)
    fwd = oracle.grouped_gemm(a, packed, absmax, offsets, row_scale=rs)
    bwd = oracle.grouped_dgrad(b, packed, absmax, offsets, row_scale=rs)
    assert fwd.shape == (P, N) and bwd.shape == (P, K)
    lhs, rhs = float(np.sum(fwd * b)), float(np.sum(a * bwd))
    assert abs(lhs - rhs) <= 1e-10 * max(1.0, abs(lhs))


def test_dgrad_exact_integer_case():
    """Weights in {-2, 0, 2}, small-integer rows, gathered: brute force."""
    rng = np.random.default_rng(4)
    E, N, K, P = 3, 32, 128, 14
    codes = rng.choice(np.array([0, 7, 15], dtype=np.uint8), size=(E, N, K))
    codes[..., ::64] = 15
    packed = oracle.pack_codes(codes)
    absmax = np.full((E, N, K // 64), np.float32(2.0), dtype=np.float32)
    ints = np.where(codes == 15, 1, np.where(codes == 0, -1, 0)).astype(np.int64)
    a = rng.integers(-3, 4, size=(5, N)).astype(np.float64)
    offsets = np.array([0, 4, 4, 14], dtype=np.int32)
    gather = rng.integers(0, 15, size=P).astype(np.int32)
    got = oracle.grouped_dgrad(a, packed, absmax, offsets, gather=gather, gather_div=3)
    for i in range(P):
        e = 0 if i < 4 else 2
        row = a[gather[i] // 3].astype(np.int64)
        want = [int(sum(int(row[n]) * int(ints[e, n, kk]) * 2 for n in range(N)))
                for kk in range(K)]
        assert got[i].tolist() == want


def test_silu_grad_closed_forms():
    assert oracle.silu_grad(np.array([0.0]))[0] == 0.5
    big = oracle.silu_grad(np.array([40.0, -40.0]))
    assert abs(big[0] - 1.0) < 1e-12 and abs(big[1]) < 1e-12
    z = np.linspace(-6, 6, 25)
    eps = 1e-6
    fd = (oracle.silu(z + eps) - oracle.silu(z - eps)) / (2 * eps)
    assert np.allclose(oracle.silu_grad(z), fd, atol=1e-9)
    # silu' has its minimum where z = -2.3994 (a root of 2 + z tanh-free form)
    zz = np.linspace(-3, -2, 100001)
    zmin = zz[np.argmin(oracle.silu_grad(zz))]
    assert abs(zmin - (-2.39936)) < 1e-4


def test_zero_adapter_b_gives_zero_a_gradient():
    p = _problem(seed=6)
    p["lgu"] = (p["lgu"][0], np.zeros_like(p["lgu"][1]), p["lgu"][2])
    p["ldn"] = (p["ldn"][0], np.zeros_like(p["ldn"][1]), p["ldn"][2])
    g = _backward(p)
    assert not np.any(g["dA_gu"]) and not np.any(g["dA_dn"])
    assert np.any(g["dB_gu"]) and np.any(g["dB_dn"])
    # and the input gradient equals the adapter-free one
    q = dict(p, lgu=None, ldn=None)
    g0 = oracle.moe_backward(q["x"], q["logits"], q["dy"], q["k"], q["gu"][0],
                             q["gu"][1], q["dn"][0], q["dn"][1])
    assert np.allclose(g["dx"], g0["dx"], rtol=1e-13, atol=1e-15)


def test_backward_is_linear_in_dy_and_zero_at_zero():
    p = _problem(seed=7)
    g1 = _backward(p)
    p2 = dict(p, dy=-3.0 * p["dy"])
    g2 = _backward(p2)
    for name in ("dx", "dA_gu", "dB_gu", "dA_dn", "dB_dn"):
        assert np.allclose(g2[name], -3.0 * g1[name], rtol=1e-12, atol=1e-14)
    g0 = _backward(dict(p, dy=np.zeros_like(p["dy"])))
    for name in ("dx", "dA_gu", "dB_gu", "dA_dn", "dB_dn"):
        assert not np.any(g0[name])


def test_unrouted_expert_gets_no_adapter_gradient():
    p = _problem(seed=8, E=6, T=3, k=1)
    g = _backward(p)
    used = set(g["info"]["ids"].reshape(-1).tolist())
    for e in range(6):
        if e not in used:
            assert not np.any(g["dA_gu"][e]) and not np.any(g["dB_dn"][e])


def test_token_subset_matches_full_backward():
    p = _problem(seed=9, T=8, lora=True)
    g = _backward(p)
    toks = [0, 5, 7]
    sub = oracle.moe_backward_tokens(toks, p["x"], p["logits"], p["dy"], p["k"],
                                     p["gu"][0], p["gu"][1], p["dn"][0], p["dn"][1],
                                     p["lgu"], p["ldn"])
    assert np.allclose(sub, g["dx"][toks], rtol=1e-12, atol=1e-14)
