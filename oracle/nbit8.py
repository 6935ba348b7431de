"""8-bit blockwise storage modes, int8 and fp8 (oracle).

TEST INFRASTRUCTURE ONLY -- see ``oracle/__init__.py``.

What the pages fix (experts4bit-qlora README "Training + expert offload":
QUANT_TYPE=nf4|fp4|int8|fp8|bf16|fp16 selects the frozen base's storage
precision; the narrative page, "What it does": the same fused stack at
selectable precision with a test-pinned fidelity ordering): int8 and fp8 are
blockwise storage modes of the same fused stack.  They do not give the maps.

Readings (the plain absmax-scaled forms, blocks of 64 along K as for NF4):

* int8: xn = x / absmax (fp32 division); code = round-half-even(fp32(xn *
  127)) as a two's-complement byte; value = code / 127 * absmax.
* fp8: the OCP e4m3 format (1 sign, 4 exponent bits with bias 7, 3 mantissa
  bits, subnormals, no infinities; S.1111.111 is NaN, largest finite 448);
  code = the e4m3 value nearest to y = fp32(xn * 448), an exact tie going to
  the even mantissa (the even code); a zero of either sign is code 0;
  value = e4m3(code) / 448 * absmax.
* One byte per element: codes [..., K] uint8.  An all-zero block stores
  absmax 0 and code 0.

Parity: pinned in ``tests/test_oracle_nbit8.py``.
"""

from __future__ import annotations

import numpy as np

BLOCK = 64


def e4m3_value(code) -> np.ndarray:
    """fp64 value of e4m3 codes (0..255) from their bit fields."""
    c = np.asarray(code, dtype=np.int64)
    sign = np.where((c >> 7) & 1, -1.0, 1.0)
    e = (c >> 3) & 15
    m = c & 7
    mag = np.where(e == 0, m * 2.0 ** -9, np.ldexp(1.0 + m / 8.0, e - 7))
    mag = np.where((e == 15) & (m == 7), np.nan, mag)
    return sign * mag


def int8_code(xn: np.ndarray) -> np.ndarray:
    """Codes (uint8 bytes of int8) of normalised fp32 values."""
    y = (np.asarray(xn, dtype=np.float32) * np.float32(127)).astype(np.float32)
    return np.rint(y).astype(np.int64).astype(np.int8).view(np.uint8)


def fp8_code(xn: np.ndarray) -> np.ndarray:
    """Nearest e4m3 codes of fp32(xn * 448), by enumeration of the 127
    non-negative finite values; exact ties to the even code."""
    y = (np.asarray(xn, dtype=np.float32) * np.float32(448)).astype(np.float64)
    vals = e4m3_value(np.arange(127))          # codes 0..126, ascending
    a = np.abs(y)[..., None]
    d = np.abs(vals - a)
    best = d.min(axis=-1, keepdims=True)
    cand = d == best
    # the lowest even candidate when two tie, else the single one
    even = cand & (np.arange(127) % 2 == 0)
    pick = np.where(even.any(axis=-1, keepdims=True), even, cand)
    code = np.argmax(pick, axis=-1).astype(np.int64)
    code = np.where((y < 0) & (code != 0), code | 0x80, code)
    return code.astype(np.uint8)


def quantize_blockwise8(w: np.ndarray, quant_type: str, blocksize: int = BLOCK):
    """``w`` [..., K] fp32 -> (codes uint8 [..., K], absmax fp32 [..., K/64])."""
    w = np.asarray(w)
    assert w.dtype == np.float32 and w.shape[-1] % blocksize == 0
    assert np.all(np.isfinite(w))
    assert quant_type in ("int8", "fp8")
    blocks = w.reshape(w.shape[:-1] + (w.shape[-1] // blocksize, blocksize))
    absmax = np.max(np.abs(blocks), axis=-1)
    safe = np.where(absmax == 0, np.float32(1), absmax).astype(np.float32)
    xn = (blocks / safe[..., None]).astype(np.float32)
    codes = int8_code(xn) if quant_type == "int8" else fp8_code(xn)
    codes[absmax == 0] = 0
    return codes.reshape(w.shape), absmax.astype(np.float32)


def dequantize_blockwise8(codes: np.ndarray, absmax: np.ndarray, quant_type: str,
                          blocksize: int = BLOCK) -> np.ndarray:
    """fp64 weights [..., K] of 8-bit codes."""
    c = np.asarray(codes, dtype=np.uint8)
    if quant_type == "int8":
        v = c.view(np.int8).astype(np.float64) / 127.0
    else:
        v = e4m3_value(c) / 448.0
    return v * np.repeat(np.asarray(absmax, dtype=np.float64), blocksize, axis=-1)
