"""Oracle: UV-Prune visual-token score (test infrastructure only).

Source: ParallelVLM notes (CVPR 2026), method section 1, "UV-Prune": over a
set of early target layers l = 1..L, the cosine similarity between video
token i and text token j at layer l is
    S^l_ij = <V^l_i, X^l_j> / (|V^l_i| |X^l_j|),
the score of video token i is the change of that alignment across the layers
summed over all text tokens,
    dS_i = sum_j sum_l (S^l_ij - S^(l-1)_ij),
and the kept set is the top-K of dS for the pruning ratio alpha.

Readings taken where the pages are silent:
  * "layer l" means the hidden state after l target layers; l - 1 = 0 is the
    layer input (the embeddings entering the first layer);
  * a zero hidden vector has no direction: its similarities are 0;
  * the top-K keeps ceil((1 - alpha) * m) tokens, ordered by score
    descending, index ascending on ties (the same order as svlm_select).

The oracle takes every layer's hidden states and evaluates the double sum as
printed; the library kernel uses the fact that the inner sum over l
telescopes to S^L_ij - S^0_ij, so it only reads layers 0 and L.  Both are
pinned against each other and against closed forms in
tests/test_oracle_uvprune.py.
"""
from __future__ import annotations

import math

import numpy as np


def _f64(x) -> np.ndarray:
    return np.asarray(x, dtype=np.float32).astype(np.float64)


def cosine_matrix(v, x) -> np.ndarray:
    """S_ij = <v_i, x_j> / (|v_i| |x_j|) for v [m][d], x [n][d]; 0 where a norm is 0."""
    v, x = _f64(v), _f64(x)
    nv = np.sqrt((v * v).sum(axis=1))
    nx = np.sqrt((x * x).sum(axis=1))
    dots = v @ x.T
    denom = nv[:, None] * nx[None, :]
    out = np.zeros_like(dots)
    ok = denom > 0
    out[ok] = dots[ok] / denom[ok]
    return out


def uvprune_scores(v_layers, x_layers) -> np.ndarray:
    """v_layers: [L+1][m][d] video hidden states of layers 0..L; x_layers:
    [L+1][n][d] text hidden states.  Returns dS [m] (fp64)."""
    L1 = len(v_layers)
    if L1 < 2 or len(x_layers) != L1:
        raise ValueError("need hidden states of at least two layers, the same for video and text")
    m = np.asarray(v_layers[0]).shape[0]
    ds = np.zeros(m)
    prev = cosine_matrix(v_layers[0], x_layers[0])
    for l in range(1, L1):
        cur = cosine_matrix(v_layers[l], x_layers[l])
        ds += (cur - prev).sum(axis=1)
        prev = cur
    return ds


def uvprune_keep(scores, alpha: float) -> np.ndarray:
    """Top-K of the scores for pruning ratio alpha: K = ceil((1 - alpha) * m)
    tokens, score descending then index ascending; returned ascending."""
    s = np.asarray(scores, dtype=np.float64)
    m = s.shape[0]
    k = min(m, max(0, math.ceil((1.0 - alpha) * m)))
    order = np.lexsort((np.arange(m), -s))
    return np.sort(order[:k]).astype(np.int64)
