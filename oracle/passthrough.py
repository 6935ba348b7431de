"""bf16 / fp16 passthrough storage of the expert stack (oracle).

TEST INFRASTRUCTURE ONLY -- see ``oracle/__init__.py``.

What the pages fix (experts4bit-qlora README "Training + expert offload":
QUANT_TYPE selects the frozen base's storage precision, bf16 and fp16 among
the choices; the narrative page, "What it does": the same fused stack at
selectable precision): the stack kept as plain 16-bit weights, with no
blocks, codes or scales.

Readings taken where the pages are silent:

* The stored weight is the input rounded once to the storage type, round to
  nearest with ties to even: for fp16 the IEEE binary16 rounding (overflow
  to +-inf, gradual underflow); for bf16 the nearest value on the bf16 grid
  (the upper 16 bits of an fp32 pattern), ties to the even last bit.
* The stack is ``[E, N, K]`` of those 16-bit patterns (uint16 here).
* The grouped GEMM and the layer are the NF4 ones with the weight replaced
  by the stored value, exactly (fp64).

Parity of every function: pinned in ``tests/test_oracle_passthrough.py``.
"""

from __future__ import annotations

import numpy as np

PASSTHROUGH = ("bf16", "fp16")


def bf16_store(w: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit patterns (uint16), nearest value, ties to even.

    The fp32 pattern's upper 16 bits are the candidate; the lower 16 bits
    decide: above half a bf16 step rounds up, below rounds down, exactly
    half rounds to the candidate whose last bit is 0.
    """
    w = np.asarray(w, dtype=np.float32)
    assert np.all(np.isfinite(w))
    bits = w.view(np.uint32).astype(np.int64)
    hi = bits >> 16
    lo = bits & 0xFFFF
    up = (lo > 0x8000) | ((lo == 0x8000) & ((hi & 1) == 1))
    return (hi + up).astype(np.uint16)


def bf16_value(bits: np.ndarray) -> np.ndarray:
    """fp64 values of bf16 bit patterns."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


def fp16_store(w: np.ndarray) -> np.ndarray:
    """fp32 -> fp16 bit patterns (uint16): IEEE binary16 round to nearest
    even (NumPy's float16 cast, a library primitive)."""
    w = np.asarray(w, dtype=np.float32)
    assert np.all(np.isfinite(w))
    return w.astype(np.float16).view(np.uint16)


def fp16_value(bits: np.ndarray) -> np.ndarray:
    """fp64 values of fp16 bit patterns."""
    return np.asarray(bits, dtype=np.uint16).view(np.float16).astype(np.float64)


def store16(w: np.ndarray, quant_type: str) -> np.ndarray:
    """The stored stack: uint16 patterns of w [..., K] in bf16 or fp16."""
    assert quant_type in PASSTHROUGH
    return bf16_store(w) if quant_type == "bf16" else fp16_store(w)


def value16(bits: np.ndarray, quant_type: str) -> np.ndarray:
    """fp64 weights of a stored stack."""
    assert quant_type in PASSTHROUGH
    return bf16_value(bits) if quant_type == "bf16" else fp16_value(bits)


def grouped_gemm16(a, bits, offsets, quant_type, gather=None, gather_div=1, swiglu=False,
                   row_scale=None):
    """The grouped GEMM of ``oracle.moe.grouped_gemm`` on a stored 16-bit
    stack ``bits`` [E, N, K]."""
    a = np.asarray(a, dtype=np.float64)
    offsets = np.asarray(offsets, dtype=np.int64)
    E, N = bits.shape[0], bits.shape[1]
    P = int(offsets[E])
    out = np.zeros((P, N // 2 if swiglu else N), dtype=np.float64)
    for e in range(E):
        lo, hi = int(offsets[e]), int(offsets[e + 1])
        if hi == lo:
            continue
        idx = np.arange(lo, hi)
        src = idx if gather is None else np.asarray(gather)[idx] // gather_div
        g = a[src] @ value16(bits[e], quant_type).T
        if swiglu:
            z = g[:, : N // 2]
            g = z / (1.0 + np.exp(-z)) * g[:, N // 2:]
        out[lo:hi] = g
    if row_scale is not None:
        out *= np.asarray(row_scale, dtype=np.float64)[:P, None]
    return out


def moe_forward16(x, logits, k, gu_bits, dn_bits, quant_type, renormalize=True):
    """The routed-expert layer of ``oracle.moe.moe_forward`` on stored 16-bit
    stacks (same routing, SwiGLU and combine readings)."""
    from .moe import expert_mlp
    from .routing import permute_pairs, route_topk

    x = np.asarray(x, dtype=np.float64)
    T, H = x.shape
    E = gu_bits.shape[0]
    ids, w = route_topk(logits, k, renormalize)
    sorted_pair, _, offsets = permute_pairs(ids, E)
    y = np.zeros((T, H), dtype=np.float64)
    w_flat = w.reshape(-1)
    for e in range(E):
        lo, hi = int(offsets[e]), int(offsets[e + 1])
        if hi == lo:
            continue
        pairs = sorted_pair[lo:hi].astype(np.int64)
        toks = pairs // k
        o, _, _ = expert_mlp(x[toks], value16(gu_bits[e], quant_type),
                             value16(dn_bits[e], quant_type))
        y[toks] += w_flat[pairs][:, None] * o
    return y
