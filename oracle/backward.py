"""Backward of the routed-expert layer for QLoRA training (oracle).

TEST INFRASTRUCTURE ONLY -- see ``oracle/__init__.py``.

What the pages fix:

* experts4bit-qlora 0.22.0 README, "Which training path?" (the dgrad=True
  paragraph): the training backward runs through the frozen 4-bit stack in a
  single dgrad launch that materialises no dequantised expert weights.
* experts4bit-qlora 0.22.0 README, "Training + expert offload": nothing
  dequantised is kept for backward; the frozen projections are decoded again
  from the packed bytes inside backward (recompute), so the forward
  activations the backward needs are recomputed from x.
* Solutions index, "How do I QLoRA-train the fused experts": only the
  per-expert low-rank adapters train; the packed stack is frozen.

Readings taken where the pages are silent:

* The backward is the exact gradient of the forward in ``oracle.moe`` (same
  readings: gate = first I rows, h = silu(gate) * up, LoRA delta
  (alpha/r) B (A x) before the activation, y_t = sum_j w_tj o_tj).
* Given dL/dy the layer returns dL/dx (the expert path's contribution; the
  router logits are an input, so no gradient flows through the routing) and,
  for each adapter, dL/dA and dL/dB.  The frozen stack receives no gradient.
* All arithmetic is fp64.  Every gradient is the plain chain rule written
  out: no blocking, fusion or reordering beyond it.
"""

from __future__ import annotations

import numpy as np

from .moe import _deq64, silu
from .routing import permute_pairs, route_topk


def silu_grad(z: np.ndarray) -> np.ndarray:
    """d/dz [z * sigmoid(z)] = sigmoid(z) * (1 + z * (1 - sigmoid(z))), fp64."""
    z = np.asarray(z, dtype=np.float64)
    with np.errstate(over="ignore"):
        s = 1.0 / (1.0 + np.exp(-z))
    return s * (1.0 + z * (1.0 - s))


def swiglu_backward(g: np.ndarray, dh: np.ndarray) -> np.ndarray:
    """Gradient of h = silu(g[:, :I]) * g[:, I:] with respect to g.

    Returns dg [M, 2I]: the gate half is dh * up * silu'(gate), the up half
    dh * silu(gate).
    """
    g = np.asarray(g, dtype=np.float64)
    dh = np.asarray(dh, dtype=np.float64)
    I = g.shape[1] // 2
    gate, up = g[:, :I], g[:, I:]
    return np.concatenate([dh * up * silu_grad(gate), dh * silu(gate)], axis=1)


def grouped_dgrad(a, packed, absmax, offsets, gather=None, gather_div=1,
                  row_scale=None, quant_type="nf4"):
    """Rows of ``a`` times each expert's dequantised weight, untransposed.

    The backward of ``oracle.moe.grouped_gemm`` with respect to its input:
    row i of expert e (``offsets[e] <= i < offsets[e+1]``) is
    ``row_scale[i] * a[src(i)] @ W_e`` with ``W_e`` [N, K] the dequantised
    matrix of ``packed[e]``/``absmax[e]``, so it contracts over the N axis
    along which the 64-blocks do *not* run.  ``a`` [rows, N];
    ``src(i) = gather[i] // gather_div`` or i.  fp64 result [P, K].
    """
    a = np.asarray(a, dtype=np.float64)
    offsets = np.asarray(offsets, dtype=np.int64)
    E, N = packed.shape[0], packed.shape[1]
    K = packed.shape[2] * 2
    P = int(offsets[E])
    out = np.zeros((P, K), dtype=np.float64)
    for e in range(E):
        lo, hi = int(offsets[e]), int(offsets[e + 1])
        if hi == lo:
            continue
        idx = np.arange(lo, hi)
        src = idx if gather is None else np.asarray(gather)[idx] // gather_div
        out[lo:hi] = a[src] @ _deq64(packed[e], absmax[e], quant_type)
    if row_scale is not None:
        out *= np.asarray(row_scale, dtype=np.float64)[:P, None]
    return out


def _lora_parts(lora, e):
    A, B, scale = lora
    return (np.asarray(A[e], dtype=np.float64), np.asarray(B[e], dtype=np.float64),
            float(scale))


def expert_backward(x_rows, w_gu, w_dn, dO, lora_gu=None, lora_dn=None, e=0):
    """Backward of one expert's MLP (``oracle.moe.expert_mlp``) on M rows.

    ``dO`` [M, H] is dL/d(expert output) (the routing weight already
    applied).  The forward is recomputed from ``x_rows``.  Returns a dict
    with ``dx`` [M, H] and, per present adapter, ``dA_gu`` [r, H],
    ``dB_gu`` [2I, r], ``dA_dn`` [r, I], ``dB_dn`` [H, r], plus the
    intermediate ``g`` [M, 2I], ``h`` [M, I] and ``dg`` [M, 2I].
    """
    x_rows = np.asarray(x_rows, dtype=np.float64)
    dO = np.asarray(dO, dtype=np.float64)
    w_gu = np.asarray(w_gu, np.float64)
    w_dn = np.asarray(w_dn, np.float64)
    I = w_dn.shape[1]
    res = {}

    # recompute: g = x W_gu^T (+ s (x A_gu^T) B_gu^T), h = silu(gate) * up
    g = x_rows @ w_gu.T
    if lora_gu is not None:
        A, B, s = _lora_parts(lora_gu, e)
        u_gu = x_rows @ A.T
        g = g + s * (u_gu @ B.T)
    h = silu(g[:, :I]) * g[:, I:]

    # down: o = h W_dn^T (+ s (h A_dn^T) B_dn^T)
    dh = dO @ w_dn
    if lora_dn is not None:
        A, B, s = _lora_parts(lora_dn, e)
        u_dn = h @ A.T            # [M, r]
        v_dn = dO @ B             # [M, r]
        dh = dh + s * (v_dn @ A)
        res["dB_dn"] = s * (dO.T @ u_dn)
        res["dA_dn"] = s * (v_dn.T @ h)

    dg = swiglu_backward(g, dh)

    # gate_up: g = x W_gu^T (+ LoRA)
    dx = dg @ w_gu
    if lora_gu is not None:
        A, B, s = _lora_parts(lora_gu, e)
        v_gu = dg @ B             # [M, r]
        dx = dx + s * (v_gu @ A)
        res["dB_gu"] = s * (dg.T @ u_gu)
        res["dA_gu"] = s * (v_gu.T @ x_rows)

    res.update(dx=dx, g=g, h=h, dg=dg)
    return res


def moe_backward(x, logits, dy, k, gu_packed, gu_absmax, dn_packed, dn_absmax,
                 lora_gu=None, lora_dn=None, renormalize=True, quant_type="nf4"):
    """Backward of ``oracle.moe.moe_forward`` for a given dL/dy, in fp64.

    Returns a dict: ``dx`` [T, H]; ``dA_gu`` [E, r, H], ``dB_gu`` [E, 2I, r]
    when ``lora_gu`` is given; ``dA_dn`` [E, r, I], ``dB_dn`` [E, H, r] when
    ``lora_dn`` is given (zero for experts no token picked); and ``info``
    with the routing.  Per pair p = (t, j) with expert e and weight w:
    dL/d o_p = w * dy_t, and dx_t sums the k pairs' input gradients.
    """
    x = np.asarray(x, dtype=np.float64)
    dy = np.asarray(dy, dtype=np.float64)
    T, H = x.shape
    E = gu_packed.shape[0]
    I = dn_packed.shape[2] * 2
    ids, w = route_topk(logits, k, renormalize)
    sorted_pair, pair_pos, offsets = permute_pairs(ids, E)
    w_flat = w.reshape(-1).astype(np.float64)
    out = {"dx": np.zeros((T, H), dtype=np.float64)}
    if lora_gu is not None:
        r = np.asarray(lora_gu[0]).shape[1]
        out["dA_gu"] = np.zeros((E, r, H))
        out["dB_gu"] = np.zeros((E, 2 * I, r))
    if lora_dn is not None:
        r = np.asarray(lora_dn[0]).shape[1]
        out["dA_dn"] = np.zeros((E, r, I))
        out["dB_dn"] = np.zeros((E, H, r))
    for e in range(E):
        lo, hi = int(offsets[e]), int(offsets[e + 1])
        if hi == lo:
            continue
        pairs = sorted_pair[lo:hi].astype(np.int64)
        toks = pairs // k  # each token appears at most once per expert
        dO = w_flat[pairs][:, None] * dy[toks]
        res = expert_backward(x[toks], _deq64(gu_packed[e], gu_absmax[e], quant_type),
                              _deq64(dn_packed[e], dn_absmax[e], quant_type), dO,
                              lora_gu, lora_dn, e)
        out["dx"][toks] += res["dx"]
        for name in ("dA_gu", "dB_gu", "dA_dn", "dB_dn"):
            if name in res:
                out[name][e] = res[name]
    out["info"] = dict(ids=ids, w=w, sorted_pair=sorted_pair, pair_pos=pair_pos,
                       offsets=offsets)
    return out


def moe_backward_tokens(tokens, x, logits, dy, k, gu_packed, gu_absmax, dn_packed,
                        dn_absmax, lora_gu=None, lora_dn=None, renormalize=True,
                        quant_type="nf4"):
    """dx[t] (fp64 [len(tokens), H]) for the listed tokens only.

    Used to check full-size runs on a sample of tokens: a token's input
    gradient depends only on its own row of x, logits and dy.
    """
    x = np.asarray(x, dtype=np.float64)
    dy = np.asarray(dy, dtype=np.float64)
    lg = np.asarray(logits, dtype=np.float32)
    cache = {}

    def weights(e):
        if e not in cache:
            cache[e] = (_deq64(gu_packed[e], gu_absmax[e], quant_type),
                        _deq64(dn_packed[e], dn_absmax[e], quant_type))
        return cache[e]

    out = np.zeros((len(tokens), x.shape[1]), dtype=np.float64)
    for n, t in enumerate(tokens):
        ids, w = route_topk(lg[t : t + 1], k, renormalize)
        for j in range(k):
            e = int(ids[0, j])
            w_gu, w_dn = weights(e)
            res = expert_backward(x[t : t + 1], w_gu, w_dn, w[0, j] * dy[t : t + 1],
                                  lora_gu, lora_dn, e)
            out[n] += res["dx"][0]
    return out
