"""NF4 codebook, blockwise quantisation and dequantisation (oracle).

TEST INFRASTRUCTURE ONLY -- see ``oracle/__init__.py``.

What the pages fix:

* experts4bit-qlora 0.22.0 README, "The problem": nf4 is one of the 4-bit
  packed storage modes of the fused expert stack.
* experts4bit-qlora 0.22.0 README, "Which door?": storage is "nf4/64", i.e.
  one scale per 64 consecutive elements.
* "Why does load_in_4bit still OOM...", "Which project solves it":
  quantisation blocks never cross an expert boundary.
* experts4bit-qlora 0.22.0 README, "Training + expert offload" and the 2026
  narrative, "What it does": a 48-layer Qwen3-30B-A3B 4-bit stack hashes to
  16.31 GB; the narrative's "What these numbers do not say" hashes
  12,846,366,720 bytes per cell for the second model.  Both totals factor as
  0.5 byte per weight plus a 4-byte fp32 absmax per 64 weights with no second
  level of quantisation, which fixes the byte format (pinned in the tests).

Readings taken where the pages are silent (each listed in the design notes):

* Codebook: the 4-bit NormalFloat construction (QLoRA, Dettmers et al. 2023):
  8 positive levels at the normal quantiles of a 9-point grid from delta down
  to 1/2 (1/2 dropped), 7 negative levels from an 8-point grid, plus an exact
  zero, normalised by the largest magnitude.  delta = ((1 - 1/32) +
  (1 - 1/30)) / 2.  Built in fp64, rounded once to fp32.
* Code of an element: xn = fl32(x / absmax) (IEEE fp32 division), then the
  index of the nearest fp32 level in exact arithmetic; an exact tie goes to
  the lower index.  An all-zero block stores absmax 0 and code 7 (level 0).
* Packing: two codes per byte, the even element in the high nibble.
* Dequantise: fl32(level[code] * absmax), in fp32.

The other 4-bit packed mode, fp4 (README, "The problem": nf4 / fp4 are the
4-bit packed storage modes, with a test-pinned fidelity ordering in which
nf4 reconstructs better than fp4).  The pages give no fp4 codebook; the
plainest reading, taken here, is the OCP e2m1 element format scaled so that
the block's absmax maps to its largest magnitude (6):
* code = s << 3 | m: sign bit s, magnitude index m, magnitudes
  {0, 0.5, 1, 1.5, 2, 3, 4, 6} / 6 (m = 0..7); code 8 is -0.
* Code of an element: xn = fl32(x / absmax) as for nf4; s = (xn < 0); m =
  the nearest fp32 magnitude level to |xn| in exact arithmetic, an exact tie
  going to the even m (round half to even, as e2m1 conversion does).  An
  all-zero block stores absmax 0 and code 0.
* Same packing, absmax and dequantisation as nf4.
"""

from __future__ import annotations

import numpy as np

BLOCKSIZE = 64

_DELTA = 0.5 * ((1.0 - 1.0 / 32.0) + (1.0 - 1.0 / 30.0))


def _norm_ppf(p: float) -> float:
    """Standard normal quantile, via scipy (library primitive)."""
    from scipy.stats import norm

    return float(norm.ppf(p))


def nf4_levels_unnormalised(ppf=_norm_ppf) -> np.ndarray:
    """The 16 NormalFloat-4 points before normalisation, ascending, fp64.

    ``ppf`` is the standard-normal quantile function to use (injectable so a
    test can build the table with a second, independent implementation).
    """
    pos_grid = np.linspace(_DELTA, 0.5, 9)[:-1]  # 8 probabilities > 1/2
    neg_grid = np.linspace(_DELTA, 0.5, 8)[:-1]  # 7 probabilities > 1/2
    pos = [ppf(float(p)) for p in pos_grid]
    neg = [-ppf(float(p)) for p in neg_grid]
    return np.array(sorted(pos + [0.0] + neg), dtype=np.float64)


def nf4_codebook_f64(ppf=_norm_ppf) -> np.ndarray:
    """NF4 levels in fp64, normalised to [-1, 1] (index 7 is exactly 0)."""
    v = nf4_levels_unnormalised(ppf)
    return v / np.max(np.abs(v))


def nf4_codebook() -> np.ndarray:
    """NF4 levels rounded once to fp32 (the stored codebook)."""
    return nf4_codebook_f64().astype(np.float32)


QUANT_TYPES = ("nf4", "fp4")

_E2M1_MAGNITUDES = (0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0)


def fp4_codebook_f64() -> np.ndarray:
    """fp4 levels by code (not sorted): codes 0..7 = +magnitude/6, 8..15 the
    negatives (code 8 is -0)."""
    mags = np.array(_E2M1_MAGNITUDES, dtype=np.float64) / 6.0
    return np.concatenate([mags, -mags])


def fp4_codebook() -> np.ndarray:
    """fp4 levels rounded once to fp32, by code."""
    return fp4_codebook_f64().astype(np.float32)


def codebook(quant_type: str = "nf4") -> np.ndarray:
    """The 16 fp32 levels of a storage mode, indexed by code."""
    if quant_type == "nf4":
        return nf4_codebook()
    if quant_type == "fp4":
        return fp4_codebook()
    raise ValueError(f"unknown quant_type {quant_type!r}")


def fp4_code(xn: np.ndarray) -> np.ndarray:
    """fp4 code of each fp32 value in ``xn``: sign bit (xn < 0) and the
    nearest magnitude level (fp64 distances), exact ties to the even index."""
    x = np.asarray(xn, dtype=np.float32)
    mags = fp4_codebook()[:8].astype(np.float64)
    ax = np.abs(x.astype(np.float64)).reshape(-1)
    m = np.empty(ax.shape, dtype=np.uint8)
    step = 1 << 20
    for s0 in range(0, ax.size, step):
        d = np.abs(ax[s0:s0 + step, None] - mags[None, :])
        best = np.min(d, axis=1, keepdims=True)
        hit = d == best  # one or (at an exact tie) two adjacent indices
        even = hit & ((np.arange(8) % 2) == 0)[None, :]
        idx = np.where(even.any(axis=1), np.argmax(even, axis=1), np.argmax(hit, axis=1))
        m[s0:s0 + step] = idx.astype(np.uint8)
    sign = (x.reshape(-1) < 0).astype(np.uint8)
    return ((sign << 3) | m).reshape(x.shape).astype(np.uint8)


def packed_bytes(E: int, N: int, K: int, blocksize: int = BLOCKSIZE) -> int:
    """Bytes of one quantised stack: E*N*K/2 codes + E*N*K/blocksize fp32."""
    assert K % blocksize == 0
    return E * N * K // 2 + (E * N * K // blocksize) * 4


def nearest_code(xn: np.ndarray, levels: np.ndarray) -> np.ndarray:
    """Index of the nearest level to each fp32 value in ``xn``; ties -> lower.

    Distances are taken in fp64.  For |xn| <= 1 and fp32 levels in [-1, 1] the
    difference of two fp32 numbers near a midpoint is exact in fp64, so the
    tie test is exact; ``np.argmin`` returns the first minimum, which is the
    lower index.
    """
    x64 = np.asarray(xn, dtype=np.float32).astype(np.float64)
    q64 = np.asarray(levels, dtype=np.float32).astype(np.float64)
    out = np.empty(x64.shape, dtype=np.uint8)
    flat_x = x64.reshape(-1)
    flat_o = out.reshape(-1)
    step = 1 << 20
    for s in range(0, flat_x.size, step):
        d = np.abs(flat_x[s : s + step, None] - q64[None, :])
        flat_o[s : s + step] = np.argmin(d, axis=1).astype(np.uint8)
    return out


def pack_codes(codes: np.ndarray) -> np.ndarray:
    """[..., K] codes (0..15) -> [..., K/2] bytes, even element high nibble."""
    c = np.asarray(codes, dtype=np.uint8)
    assert c.shape[-1] % 2 == 0
    return ((c[..., 0::2] << 4) | c[..., 1::2]).astype(np.uint8)


def unpack_codes(packed: np.ndarray) -> np.ndarray:
    """Inverse of :func:`pack_codes`."""
    p = np.asarray(packed, dtype=np.uint8)
    out = np.empty(p.shape[:-1] + (p.shape[-1] * 2,), dtype=np.uint8)
    out[..., 0::2] = p >> 4
    out[..., 1::2] = p & 0x0F
    return out


def quantize_blockwise(w: np.ndarray, blocksize: int = BLOCKSIZE, quant_type: str = "nf4"):
    """Quantise ``w`` [..., K] (fp32) blockwise along the last axis.

    Returns ``(packed uint8 [..., K/2], absmax fp32 [..., K/blocksize])``.
    The leading axes are (expert, row): a block is ``blocksize`` consecutive
    elements of one row of one expert, so it never crosses either.
    ``quant_type`` is "nf4" or "fp4".
    """
    w = np.asarray(w)
    assert w.dtype == np.float32, "the oracle quantises fp32 values"
    assert w.shape[-1] % blocksize == 0
    assert np.all(np.isfinite(w)), "non-finite input is outside the definition"
    assert quant_type in QUANT_TYPES
    blocks = w.reshape(w.shape[:-1] + (w.shape[-1] // blocksize, blocksize))
    absmax = np.max(np.abs(blocks), axis=-1)  # exact in fp32
    safe = np.where(absmax == 0, np.float32(1), absmax).astype(np.float32)
    # IEEE fp32 division, round to nearest even (numpy float32 '/').
    xn = (blocks / safe[..., None]).astype(np.float32)
    if quant_type == "nf4":
        codes = nearest_code(xn, nf4_codebook())
        codes[absmax == 0] = 7  # all-zero block -> the exact-zero level
    else:
        codes = fp4_code(xn)
        codes[absmax == 0] = 0  # all-zero block -> +0
    codes = codes.reshape(w.shape)
    return pack_codes(codes), absmax.astype(np.float32)


def dequantize_blockwise(packed: np.ndarray, absmax: np.ndarray,
                         blocksize: int = BLOCKSIZE, quant_type: str = "nf4") -> np.ndarray:
    """fp32 weights: level[code] * absmax, one fp32 multiply per element.

    The 8-bit modes ("int8", "fp8"; one code byte per element) are the
    exact fp64 values of ``oracle.nbit8``."""
    if quant_type in ("int8", "fp8"):
        from .nbit8 import dequantize_blockwise8

        return dequantize_blockwise8(packed, absmax, quant_type, blocksize)
    levels = codebook(quant_type)
    codes = unpack_codes(packed)
    vals = levels[codes]
    K = vals.shape[-1]
    scale = np.repeat(np.asarray(absmax, dtype=np.float32), blocksize, axis=-1)
    assert scale.shape[-1] == K
    return (vals * scale).astype(np.float32)


def block_error_bound(absmax: np.ndarray, quant_type: str = "nf4") -> np.ndarray:
    """Largest round-trip error a block can see: half the widest level gap."""
    q = np.unique(codebook(quant_type).astype(np.float64))
    return np.asarray(absmax, np.float64) * float(np.max(np.diff(q))) / 2.0

