"""Oracle: compaction of the kept KV rows (test infrastructure only).

Source: Sparse-to-Dense explainer, technical summary ("dual-module
architecture"): the sparse draft attends only to the selected KV entries,
which cuts the draft stage's I/O.  The draft cache holds the kept visual
rows followed by rows that are always kept (the text prompt).
"""
from __future__ import annotations

import numpy as np


def gather_kv(src, idx, tail_start: int = 0, n_tail: int = 0):
    """src: [Hkv][N][D]; idx: [n_idx] (one list for all heads) or [Hkv][n_idx].

    dst[g] = concat(src[g, idx[g]], src[g, tail_start : tail_start + n_tail])."""
    src = np.asarray(src)
    idx = np.asarray(idx, dtype=np.int64)
    Hkv = src.shape[0]
    parts = []
    for g in range(Hkv):
        ig = idx if idx.ndim == 1 else idx[g]
        parts.append(np.concatenate([src[g, ig], src[g, tail_start:tail_start + n_tail]], axis=0))
    return np.stack(parts)
