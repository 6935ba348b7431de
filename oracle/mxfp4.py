"""MXFP4 expert weights (e2m1 elements + e8m0 block scales) -- oracle.

TEST INFRASTRUCTURE ONLY -- see ``oracle/__init__.py``.

What the pages fix (grouped-nf4-gemm solutions entry "How do I run MoE
expert inference natively on MXFP4 (e2m1 + e8m0) weights, straight from the
released checkpoint bytes?"; experts4bit-qlora README "Scope", the gpt-oss
family): expert stacks released as MXFP4 are multiplied on their own e2m1
blocks and e8m0 scales, with no requantisation to NF4 and no bf16 copy.

Readings taken where the pages are silent (the OCP Microscaling format, the
plainest reading of "e2m1 + e8m0"):

* Blocks of 32 consecutive elements along the contraction axis K share one
  scale byte s: scale = 2**(s - 127); s = 255 is NaN.
* An element is a 4-bit e2m1 code: sign bit 3, exponent bits 2..1 (bias 1),
  mantissa bit 0; exponent 0 is subnormal (0 or 0.5), otherwise
  2**(e-1) * (1 + m/2): magnitudes {0, 0.5, 1, 1.5, 2, 3, 4, 6}.
* Two elements per byte, element 2i in the LOW nibble (bits 0..3) and
  element 2i+1 in the high nibble -- the packing of the released checkpoint
  blocks, opposite to this package's NF4/fp4 nibble order.
* A stack is ``blocks [E, N, K/2]`` uint8 and ``scales [E, N, K/32]`` uint8;
  the weight is element * scale, exactly (every product is a dyadic number).

Parity of every function: pinned in ``tests/test_oracle_mxfp4.py``.
"""

from __future__ import annotations

import numpy as np

MX_BLOCK = 32


def e2m1_value(code) -> np.ndarray:
    """Value of e2m1 codes (0..15) from their bit fields, fp64."""
    c = np.asarray(code, dtype=np.int64)
    sign = np.where((c >> 3) & 1, -1.0, 1.0)
    e = (c >> 1) & 3
    m = c & 1
    mag = np.where(e == 0, 0.5 * m, np.ldexp(1.0 + 0.5 * m, e - 1))
    return sign * mag


def e8m0_value(s) -> np.ndarray:
    """Scale of e8m0 bytes: 2**(s - 127), NaN for 255, fp64."""
    s = np.asarray(s, dtype=np.int64)
    return np.where(s == 255, np.nan, np.ldexp(1.0, s - 127))


def unpack_mx(blocks: np.ndarray) -> np.ndarray:
    """[..., K/2] bytes -> [..., K] codes, element 2i from the low nibble."""
    b = np.asarray(blocks, dtype=np.uint8)
    out = np.empty(b.shape[:-1] + (b.shape[-1] * 2,), dtype=np.uint8)
    out[..., 0::2] = b & 15
    out[..., 1::2] = b >> 4
    return out


def pack_mx(codes: np.ndarray) -> np.ndarray:
    """[..., K] codes -> [..., K/2] bytes (element 2i in the low nibble)."""
    c = np.asarray(codes, dtype=np.uint8)
    return (c[..., 0::2] | (c[..., 1::2] << 4)).astype(np.uint8)


def dequantize_mxfp4(blocks: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """[E, N, K/2] + [E, N, K/32] -> fp64 weights [E, N, K]."""
    codes = unpack_mx(blocks)
    vals = e2m1_value(codes)
    sc = np.repeat(e8m0_value(scales), MX_BLOCK, axis=-1)
    return vals * sc


def grouped_gemm_mxfp4(a, blocks, scales, offsets, gather=None, gather_div=1,
                       swiglu=False, row_scale=None):
    """The grouped GEMM of ``oracle.moe.grouped_gemm`` on MXFP4 weights."""
    a = np.asarray(a, dtype=np.float64)
    offsets = np.asarray(offsets, dtype=np.int64)
    E, N = blocks.shape[0], blocks.shape[1]
    P = int(offsets[E])
    n_out = N // 2 if swiglu else N
    out = np.zeros((P, n_out), dtype=np.float64)
    for e in range(E):
        lo, hi = int(offsets[e]), int(offsets[e + 1])
        if hi == lo:
            continue
        idx = np.arange(lo, hi)
        src = idx if gather is None else np.asarray(gather)[idx] // gather_div
        g = a[src] @ dequantize_mxfp4(blocks[e:e + 1], scales[e:e + 1])[0].T
        if swiglu:
            z = g[:, : N // 2]
            g = z / (1.0 + np.exp(-z)) * g[:, N // 2:]
        out[lo:hi] = g
    if row_scale is not None:
        out *= np.asarray(row_scale, dtype=np.float64)[:P, None]
    return out


def moe_forward_mxfp4(x, logits, k, gu_blocks, gu_scales, dn_blocks, dn_scales,
                      renormalize=True):
    """The routed-expert layer of ``oracle.moe.moe_forward`` on MXFP4 stacks.

    The stacks are dequantised exactly and handed to the NF4 layer's
    per-expert loop (same routing, SwiGLU and combine readings).
    """
    from .moe import expert_mlp
    from .routing import permute_pairs, route_topk

    x = np.asarray(x, dtype=np.float64)
    T, H = x.shape
    E = gu_blocks.shape[0]
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
        o, _, _ = expert_mlp(x[toks], dequantize_mxfp4(gu_blocks[e:e + 1], gu_scales[e:e + 1])[0],
                             dequantize_mxfp4(dn_blocks[e:e + 1], dn_scales[e:e + 1])[0])
        y[toks] += w_flat[pairs][:, None] * o
    return y
