"""Router top-k and the token/expert pair permutation (oracle).

TEST INFRASTRUCTURE ONLY -- see ``oracle/__init__.py``.

What the pages fix:

* experts4bit-qlora 0.22.0 README, "Which door?" (hot_rows paragraph): a
  forward routes each token to a subset of the experts.
* experts4bit-qlora 0.22.0 README, "Which training path?": the token/expert
  pairs are sorted and run as groups, and experts are summed in group-sorted
  order.

Readings taken where the pages are silent:

* Top-k: the k largest fp32 logits of a token, in descending order; equal
  logits go to the lower expert id.
* Weights: softmax over the k selected logits (renormalize=1), which is the
  full softmax renormalised over the selection and sums to 1.  With
  renormalize=0 the weights are the full softmax probabilities of the
  selected experts (they then sum to at most 1).
* Pair id p = t*k + j for token t and slot j.  The permutation lists the pair
  ids grouped by expert id ascending, and by p ascending inside an expert
  (a stable sort by expert).  Offsets are the exclusive prefix sum of the
  per-expert counts, with offsets[E] = T*k.
"""

from __future__ import annotations

import numpy as np


def route_topk(logits: np.ndarray, k: int, renormalize: bool = True):
    """Return ``(ids int32 [T,k], weights fp64 [T,k])``.

    Selection is a stable sort of the negated fp32 logits (negation is exact),
    so equal logits keep ascending expert order.  Weights are computed in fp64
    from the fp32 logits.
    """
    lg = np.asarray(logits, dtype=np.float32)
    assert lg.ndim == 2
    T, E = lg.shape
    assert 1 <= k <= E
    assert np.all(np.isfinite(lg))
    order = np.argsort(-lg, axis=1, kind="stable")
    ids = order[:, :k].astype(np.int32)
    l64 = lg.astype(np.float64)
    sel = np.take_along_axis(l64, ids.astype(np.int64), axis=1)
    m = np.max(l64, axis=1, keepdims=True)  # the top-1 logit
    if renormalize:
        e = np.exp(sel - m)
        w = e / np.sum(e, axis=1, keepdims=True)
    else:
        e_all = np.exp(l64 - m)
        w = np.exp(sel - m) / np.sum(e_all, axis=1, keepdims=True)
    return ids, w


def permute_pairs(ids: np.ndarray, E: int):
    """Group pair ids by expert.

    Returns ``(sorted_pair int32 [P], pair_pos int32 [P], offsets int32 [E+1])``
    where ``sorted_pair[i]`` is the pair id at sorted position i,
    ``pair_pos[p]`` is the sorted position of pair p, and rows
    ``offsets[e]:offsets[e+1]`` belong to expert e.
    """
    flat = np.asarray(ids, dtype=np.int64).reshape(-1)
    P = flat.size
    assert np.all((flat >= 0) & (flat < E))
    sorted_pair = np.argsort(flat, kind="stable").astype(np.int32)
    pair_pos = np.empty(P, dtype=np.int32)
    pair_pos[sorted_pair] = np.arange(P, dtype=np.int32)
    counts = np.bincount(flat, minlength=E)
    offsets = np.zeros(E + 1, dtype=np.int32)
    offsets[1:] = np.cumsum(counts)
    return sorted_pair, pair_pos, offsets
