"""Seeded synthetic inputs for the routed-expert layer.

This module only draws random inputs; it holds none of the method's
arithmetic (no quantisation, routing or GEMM), so both the CPU oracle and the
HIP path can consume its output without sharing any method code.

The workloads stand in for the real checkpoints the pages measure on
(OLMoE-1B-7B and Qwen3-30B-A3B, experts4bit-qlora 0.22.0 README "What it buys
you" and the 2026 narrative "Measured"): the layer shapes are those models',
the values are random.

Recipe (seed s):
    streams = SeedSequence(s).spawn(8) for
        w_gu, w_dn, x, logits, lora A_gu, lora B_gu, lora A_dn, lora B_dn;
    the weight streams are split once more per expert, so one expert's
    weights can be drawn alone.
    weights  fp32, standard normal * 0.02
    x        fp32 standard normal, rounded to bf16 (round to nearest even)
    logits   fp32 standard normal, or for the Zipf workload
             ln(r^-1.1 / Z) + Gumbel(0, 1) over a seeded permutation of the
             expert ids (top-k of Gumbel-perturbed log-weights draws k experts
             without replacement in proportion to the Zipf weights)
    LoRA A,B fp32 standard normal * 0.01, rounded to bf16
"""

from __future__ import annotations

from dataclasses import dataclass
from typing import Optional

import numpy as np

_STREAMS = ("w_gu", "w_dn", "x", "logits", "a_gu", "b_gu", "a_dn", "b_dn", "dy", "mx")


@dataclass(frozen=True)
class LayerConfig:
    name: str
    E: int
    H: int
    I: int
    k: int
    T: int
    logits: str = "normal"  # "normal" or "zipf"
    zipf_s: float = 1.1
    lora_r: int = 0
    lora_alpha: float = 0.0
    renormalize: bool = True

    @property
    def P(self) -> int:
        return self.T * self.k

    @property
    def lora_scale(self) -> float:
        return self.lora_alpha / self.lora_r if self.lora_r else 0.0

    def flops(self) -> float:
        """Algorithmic FLOPs of one layer forward (both projections + LoRA)."""
        f = 6.0 * self.P * self.H * self.I
        if self.lora_r:
            r = self.lora_r
            # gate_up: x A^T (2 P H r) + u B^T (2 P 2I r); down: h A^T + u B^T
            f += 2.0 * self.P * r * (self.H + 2 * self.I)
            f += 2.0 * self.P * r * (self.I + self.H)
        return f


CONFIGS = {
    "tiny": LayerConfig("tiny", E=8, H=256, I=128, k=2, T=64),
    "olmoe": LayerConfig("olmoe", E=64, H=2048, I=1024, k=8, T=4096),
    "qwen3_zipf": LayerConfig("qwen3_zipf", E=128, H=2048, I=768, k=8, T=4096,
                              logits="zipf"),
    "decode": LayerConfig("decode", E=128, H=2048, I=768, k=8, T=1),
    "qlora": LayerConfig("qlora", E=128, H=2048, I=768, k=8, T=4096,
                         lora_r=8, lora_alpha=16.0),
}


def config(name: str, **overrides) -> LayerConfig:
    base = CONFIGS[name]
    if not overrides:
        return base
    fields = dict(base.__dict__)
    fields.update(overrides)
    return LayerConfig(**fields)


def round_to_bf16(x: np.ndarray) -> np.ndarray:
    """fp32 -> nearest bf16 value (ties to even), returned as fp32."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    r = ((u.astype(np.uint64) + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint32)
    return (r << 16).view(np.float32)


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """Upper 16 bits of fp32 values that are already bf16 values."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    assert np.all((u & 0xFFFF) == 0), "values are not bf16"
    return (u >> 16).astype(np.uint16)


def _streams(seed: int):
    ss = np.random.SeedSequence(seed).spawn(len(_STREAMS))
    return dict(zip(_STREAMS, ss))


def expert_weights(cfg: LayerConfig, which: str, e: int, seed: int = 0):
    """fp32 weights of one expert: which='gu' -> [2I, H], 'dn' -> [H, I]."""
    key = "w_gu" if which == "gu" else "w_dn"
    child = _streams(seed)[key].spawn(cfg.E)[e]
    rng = np.random.default_rng(child)
    shape = (2 * cfg.I, cfg.H) if which == "gu" else (cfg.H, cfg.I)
    return rng.standard_normal(shape, dtype=np.float32) * np.float32(0.02)


def stack_weights(cfg: LayerConfig, which: str, seed: int = 0,
                  experts: Optional[range] = None) -> np.ndarray:
    """All (or a range of) experts' fp32 weights, stacked on axis 0."""
    experts = range(cfg.E) if experts is None else experts
    return np.stack([expert_weights(cfg, which, e, seed) for e in experts])


def activations(cfg: LayerConfig, seed: int = 0) -> np.ndarray:
    """x [T, H]: bf16 values held in fp32."""
    rng = np.random.default_rng(_streams(seed)["x"])
    return round_to_bf16(rng.standard_normal((cfg.T, cfg.H), dtype=np.float32))


def output_grad(cfg: LayerConfig, seed: int = 0) -> np.ndarray:
    """dL/dy [T, H] for the backward: bf16 values (N(0,1)) held in fp32."""
    rng = np.random.default_rng(_streams(seed)["dy"])
    return round_to_bf16(rng.standard_normal((cfg.T, cfg.H), dtype=np.float32))


def router_logits(cfg: LayerConfig, seed: int = 0) -> np.ndarray:
    """logits [T, E] fp32."""
    rng = np.random.default_rng(_streams(seed)["logits"])
    if cfg.logits == "normal":
        return rng.standard_normal((cfg.T, cfg.E), dtype=np.float32)
    if cfg.logits == "zipf":
        perm = rng.permutation(cfg.E)
        ranks = np.arange(1, cfg.E + 1, dtype=np.float64)
        logp = -cfg.zipf_s * np.log(ranks)
        logp -= np.log(np.sum(np.exp(logp)))
        base = np.empty(cfg.E, dtype=np.float64)
        base[perm] = logp  # expert perm[r] has rank r+1
        g = rng.gumbel(size=(cfg.T, cfg.E))
        return (base[None, :] + g).astype(np.float32)
    raise ValueError(cfg.logits)


def lora_weights(cfg: LayerConfig, seed: int = 0):
    """Per-expert LoRA factors as bf16 values held in fp32, or None.

    Returns dict(a_gu [E, r, H], b_gu [E, 2I, r], a_dn [E, r, I],
    b_dn [E, H, r]).
    """
    if not cfg.lora_r:
        return None
    st = _streams(seed)
    r, E, H, I = cfg.lora_r, cfg.E, cfg.H, cfg.I
    shapes = dict(a_gu=(E, r, H), b_gu=(E, 2 * I, r), a_dn=(E, r, I),
                  b_dn=(E, H, r))
    out = {}
    for name, shape in shapes.items():
        rng = np.random.default_rng(st[name])
        out[name] = round_to_bf16(
            rng.standard_normal(shape, dtype=np.float32) * np.float32(0.01))
    return out


# magnitude index frequencies (0, 0.5, 1, 1.5, 2, 3, 4, 6) of the synthetic
# MXFP4 elements, shaped like a block-quantised bell curve
_MX_MAG_P = (0.10, 0.20, 0.19, 0.15, 0.14, 0.11, 0.07, 0.04)


def mxfp4_stack(cfg: LayerConfig, which: str, seed: int = 0):
    """Synthetic released-MXFP4 stack bytes: (blocks [E, N, K/2] uint8,
    scales [E, N, K/32] uint8).  Element codes are sign | magnitude index
    drawn from _MX_MAG_P; scale bytes 127 + {-8, -7, -6} (2^-8 .. 2^-6, the
    range a 0.02-scale weight's blocks take).  Random bytes only."""
    child = _streams(seed)["mx"].spawn(2)[0 if which == "gu" else 1]
    rng = np.random.default_rng(child)
    N, K = (2 * cfg.I, cfg.H) if which == "gu" else (cfg.H, cfg.I)
    # a random byte per element: bit 7 is the sign, the low 7 bits pick the
    # magnitude index through a 128-entry table of the frequencies
    bounds = np.cumsum(_MX_MAG_P) * 128
    table = np.searchsorted(bounds, np.arange(128) + 0.5).astype(np.uint8)
    r = rng.integers(0, 256, size=(cfg.E, N, K), dtype=np.uint8)
    codes = table[r & 127] | ((r >> 7) << 3)
    del r
    blocks = (codes[..., 0::2] | (codes[..., 1::2] << 4)).astype(np.uint8)
    scales = (127 + rng.integers(-8, -5, size=(cfg.E, N, K // 32))).astype(np.uint8)
    return blocks, scales
