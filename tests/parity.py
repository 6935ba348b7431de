"""Parity helpers shared by the GPU tests (comparison rules, no method code).

Output tolerance (bf16 outputs versus the fp64 oracle):
    relative Frobenius error  <= 5e-3
    max |y_gpu - y_ref|       <= 2e-2 * RMS(y_ref)
Both sides of every integer decision (codes, ids, permutation) must agree
bit for bit.  Alongside the max-abs figure the report gives the floor that
rounding the exact result to bf16 alone costs, max|bf16(y_ref) - y_ref|/RMS.
"""

from __future__ import annotations

import numpy as np

from grouped_nf4_gemm_quantize_amd import synth

FRO_TOL = 5e-3
MAXABS_TOL = 2e-2


def metrics(y_gpu: np.ndarray, y_ref: np.ndarray) -> dict:
    y_gpu = np.asarray(y_gpu, dtype=np.float64)
    y_ref = np.asarray(y_ref, dtype=np.float64)
    rms = float(np.sqrt(np.mean(y_ref ** 2)))
    diff = y_gpu - y_ref
    fro = float(np.linalg.norm(diff) / max(np.linalg.norm(y_ref), 1e-300))
    mx = float(np.max(np.abs(diff)) / max(rms, 1e-300)) if diff.size else 0.0
    yb = synth.round_to_bf16(y_ref.astype(np.float32)).astype(np.float64)
    floor = float(np.max(np.abs(yb - y_ref)) / max(rms, 1e-300)) if diff.size else 0.0
    return dict(fro=fro, maxabs=mx, floor=floor, rms=rms)


def assert_parity(y_gpu, y_ref, fro_tol: float = FRO_TOL, maxabs_tol: float = MAXABS_TOL,
                  what: str = "") -> dict:
    m = metrics(y_gpu, y_ref)
    assert m["fro"] <= fro_tol and m["maxabs"] <= maxabs_tol, (
        f"{what}: rel-Frobenius {m['fro']:.3e} (tol {fro_tol:g}), max-abs/RMS "
        f"{m['maxabs']:.3e} (tol {maxabs_tol:g}; bf16 floor {m['floor']:.3e})")
    return m
