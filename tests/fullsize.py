"""Full-size quantised stacks for the GPU parity tests (test infrastructure).

Every expert of both projections is quantised twice from the same seeded fp32
weights: on the GPU through the C ABI, and by the oracle on the host.  The
two must agree bit for bit on all four arrays (codes and absmax of gate_up
and of down) for every expert; the agreed bytes are then cached for the
session, so the Qwen3-shaped workloads (Zipf prefill, decode, QLoRA), which
share one stack shape and seed, quantise it once.

The oracle runs expert by expert in a thread pool (NumPy releases the GIL in
its array loops); the pool is sized to the process's CPU affinity, at most 16.
"""

from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

import oracle
from grouped_nf4_gemm_quantize_amd import synth

_CACHE: dict = {}
_GROUP = 16


def host_threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover - non-Linux
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def full_stacks(gpu_lib, cfg, seed: int = 0):
    """``(gpu, ref)``: the GPU-quantised stacks (gp, ga, dp, da) as device
    tensors and the oracle's bytes as NumPy arrays, after checking that they
    are identical for every expert."""
    import torch

    key = (cfg.E, cfg.H, cfg.I, seed)
    if key in _CACHE:
        return _CACHE[key]
    E, H, I = cfg.E, cfg.H, cfg.I
    dev = "cuda"
    shapes = {"gu": (2 * I, H), "dn": (H, I)}
    gpu = {}
    ref = {}
    for which, (N, K) in shapes.items():
        gpu[which] = (torch.empty((E, N, K // 2), dtype=torch.uint8, device=dev),
                      torch.empty((E, N, K // 64), dtype=torch.float32, device=dev))
        ref[which] = (np.empty((E, N, K // 2), dtype=np.uint8),
                      np.empty((E, N, K // 64), dtype=np.float32))
    bad = []
    with ThreadPoolExecutor(host_threads()) as pool:
        for which in shapes:
            for e0 in range(0, E, _GROUP):
                ex = list(range(e0, min(e0 + _GROUP, E)))
                ws = list(pool.map(lambda e: synth.expert_weights(cfg, which, e, seed), ex))
                p, a = gpu_lib.quantize(torch.from_numpy(np.stack(ws)).to(dev))
                gpu[which][0][e0:e0 + len(ex)] = p
                gpu[which][1][e0:e0 + len(ex)] = a
                for e, (pr, ar) in zip(ex, pool.map(oracle.quantize_blockwise, ws)):
                    ref[which][0][e] = pr
                    ref[which][1][e] = ar
                del ws
                ph = p.cpu().numpy()
                ah = a.cpu().numpy().view(np.uint32)
                for n, e in enumerate(ex):
                    if not (np.array_equal(ph[n], ref[which][0][e])
                            and np.array_equal(ah[n], ref[which][1][e].view(np.uint32))):
                        bad.append((which, e))
    assert not bad, f"GPU quantiser differs from the oracle on (stack, expert) {bad[:8]}"
    out = ((gpu["gu"][0], gpu["gu"][1], gpu["dn"][0], gpu["dn"][1]),
           (ref["gu"][0], ref["gu"][1], ref["dn"][0], ref["dn"][1]))
    _CACHE[key] = out
    return out
