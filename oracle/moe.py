"""Grouped expert GEMM and the full routed-expert forward (oracle).

TEST INFRASTRUCTURE ONLY -- see ``oracle/__init__.py``.

What the pages fix:

* experts4bit-qlora 0.22.0 README, "The problem" / "Quickstart":
  ``gate_up_proj [E, 2I, H]`` and ``down_proj [E, H, I]``, stored [out, in],
  so each projection contracts over the last axis.
* experts4bit-qlora 0.22.0 README, "Which door?": the expert projections of
  each expert run on its frozen NF4 weights with fp32 accumulation; modules
  with activations other than SwiGLU are not handled.
* experts4bit-qlora 0.22.0 README, "Scope": the supported families are SwiGLU
  fused-MoE architectures.
* Solutions index, "How do I QLoRA-train the fused experts": a trainable
  per-expert low-rank delta is added before each routed expert's activation;
  experts4bit-qlora 0.22.0 "Quickstart" gives r=8, alpha=16.
* experts4bit-qlora 0.22.0 README, "Which training path?": pairs are sorted by
  expert and the per-pair outputs are summed back per token.

Readings taken where the pages are silent:

* Of the 2I rows of gate_up, the first I are the gate and the next I the up
  projection (the name order).  h = silu(gate) * up, silu(z) = z/(1+e^-z).
* LoRA: delta = (alpha/r) * B (A x) with A [E, r, in] and B [E, out, r]; it is
  added to the gate_up output before SwiGLU and to the down output.
* Combine: y_t = sum_j w_tj * o_tj over the k slots of token t.
* All arithmetic after dequantisation is fp64 (summation order is then
  immaterial to the comparison tolerance).
"""

from __future__ import annotations

import numpy as np

from .nf4 import dequantize_blockwise
from .routing import permute_pairs, route_topk


def silu(z: np.ndarray) -> np.ndarray:
    """z * sigmoid(z) in fp64."""
    z = np.asarray(z, dtype=np.float64)
    with np.errstate(over="ignore"):
        return z / (1.0 + np.exp(-z))


def _deq64(packed_e: np.ndarray, absmax_e: np.ndarray, quant_type: str = "nf4") -> np.ndarray:
    return dequantize_blockwise(packed_e, absmax_e, quant_type=quant_type).astype(np.float64)


def _lora_delta(a_rows: np.ndarray, lora, e: int) -> np.ndarray:
    """(alpha/r) * (a A_e^T) B_e^T in fp64, or 0 when there is no adapter."""
    if lora is None:
        return 0.0
    A, B, scale = lora
    A_e = np.asarray(A[e], dtype=np.float64)  # [r, in]
    B_e = np.asarray(B[e], dtype=np.float64)  # [out, r]
    return float(scale) * ((a_rows @ A_e.T) @ B_e.T)


def expert_mlp(x_rows, w_gu, w_dn, lora_gu=None, lora_dn=None, e=0):
    """One expert's SwiGLU MLP on dequantised fp64 weights.

    ``w_gu`` [2I, H] and ``w_dn`` [H, I] are the expert's dequantised
    matrices; the optional adapters are ``(A, B, scale)`` triples indexed by
    expert ``e``.  Returns ``(o [M, H], h [M, I], g [M, 2I])``.
    """
    x_rows = np.asarray(x_rows, dtype=np.float64)
    I = w_dn.shape[1]
    g = x_rows @ np.asarray(w_gu, np.float64).T + _lora_delta(x_rows, lora_gu, e)
    h = silu(g[:, :I]) * g[:, I:]
    o = h @ np.asarray(w_dn, np.float64).T + _lora_delta(h, lora_dn, e)
    return o, h, g


def grouped_gemm(a, packed, absmax, offsets, gather=None, gather_div=1,
                 lora=None, swiglu=False, row_scale=None, quant_type="nf4"):
    """Rows of ``a`` times each expert's dequantised weight, per group.

    Row i of the output belongs to expert e when
    ``offsets[e] <= i < offsets[e+1]`` and reads input row
    ``gather[i] // gather_div`` (or row i when ``gather`` is None).
    ``packed`` [E, N, K/2], ``absmax`` [E, N, K/64].  With ``swiglu`` the
    N = 2I outputs become I outputs silu(first half) * second half.
    ``row_scale`` [P] multiplies output row i.  fp64 result [P, N or N/2].
    """
    a = np.asarray(a, dtype=np.float64)
    offsets = np.asarray(offsets, dtype=np.int64)
    E = packed.shape[0]
    N = packed.shape[1]
    P = int(offsets[E])
    n_out = N // 2 if swiglu else N
    out = np.zeros((P, n_out), dtype=np.float64)
    for e in range(E):
        lo, hi = int(offsets[e]), int(offsets[e + 1])
        if hi == lo:
            continue
        idx = np.arange(lo, hi)
        src = idx if gather is None else np.asarray(gather)[idx] // gather_div
        rows = a[src]
        g = rows @ _deq64(packed[e], absmax[e], quant_type).T + _lora_delta(rows, lora, e)
        if swiglu:
            g = silu(g[:, : N // 2]) * g[:, N // 2 :]
        out[lo:hi] = g
    if row_scale is not None:
        out *= np.asarray(row_scale, dtype=np.float64)[:P, None]
    return out


def moe_forward(x, logits, k, gu_packed, gu_absmax, dn_packed, dn_absmax,
                lora_gu=None, lora_dn=None, renormalize=True, quant_type="nf4"):
    """Full routed-expert layer, the plain per-expert loop, in fp64.

    ``x`` [T, H] holds the activation values (bf16 values widened exactly);
    ``logits`` [T, E] fp32.  Returns ``(y [T, H] fp64, info)`` where ``info``
    holds the routing (ids, weights, permutation, offsets).
    """
    x = np.asarray(x, dtype=np.float64)
    T, H = x.shape
    E = gu_packed.shape[0]
    ids, w = route_topk(logits, k, renormalize)
    sorted_pair, pair_pos, offsets = permute_pairs(ids, E)
    y = np.zeros((T, H), dtype=np.float64)
    w_flat = w.reshape(-1)
    for e in range(E):
        lo, hi = int(offsets[e]), int(offsets[e + 1])
        if hi == lo:
            continue
        pairs = sorted_pair[lo:hi].astype(np.int64)
        toks = pairs // k  # each token appears at most once per expert
        o, _, _ = expert_mlp(x[toks], _deq64(gu_packed[e], gu_absmax[e], quant_type),
                             _deq64(dn_packed[e], dn_absmax[e], quant_type),
                             lora_gu, lora_dn, e)
        y[toks] += w_flat[pairs][:, None] * o
    info = dict(ids=ids, w=w, sorted_pair=sorted_pair, pair_pos=pair_pos,
                offsets=offsets)
    return y, info


def moe_forward_tokens(tokens, x, logits, k, gu_packed, gu_absmax, dn_packed,
                       dn_absmax, lora_gu=None, lora_dn=None,
                       renormalize=True, quant_type="nf4"):
    """Outputs y[t] for the listed tokens only (fp64 [len(tokens), H]).

    Used to check full-size runs on a sample of tokens: each token is routed
    on its own logits row and sent through its k experts.
    """
    x = np.asarray(x, dtype=np.float64)
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
            o, _, _ = expert_mlp(x[t : t + 1], w_gu, w_dn, lora_gu, lora_dn, e)
            out[n] += w[0, j] * o[0]
    return out
