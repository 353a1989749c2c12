"""Oracle: two-stage visual token selection (test infrastructure only).

Source: SpecVLM technology-transfer listing, section 5 ("solution"): by
their score the visual tokens split into high-information tokens and
low-attention tokens; (i) the high-information ones are kept by a Top-P rule
on the share of attention score, (ii) among the low-attention ones a subset
is kept spread evenly in space, to keep some spatial structure.  SpecVLM
abstract: stage I is verifier-guided, stage II is spatially uniform, up to
90% of video tokens are pruned.  Sparse-to-Dense explainer ("KV cache
selection"): plain top-K of the mean text-to-visual attention, per layer and
head (top_p >= 1 here).

Readings (the pages give no formulas):
  * order: score descending, ties by lower token index first;
  * "share of attention score" is measured in exact fixed point: each score
    s (fp32 in [0, 1]) has mass floor(s * 2**40), an exact integer; the row
    total is Q and the stage-I target is ceil(double(Q) * P) with IEEE
    round-to-nearest double arithmetic;
  * stage I keeps the shortest top prefix whose mass reaches the target,
    truncated to the budget B when it needs more than B tokens (the budget
    is hard); top_p >= 1 keeps the top B, top_p <= 0 keeps none;
  * stage II walks the remaining tokens in frame-major raster order (token
    n = f*H*W + y*W + x, so frames come one after another and each frame's
    H x W grid row by row) and takes m = B - k1 of the n_rem of them at one
    constant stride with centred phase: ranks floor((2j + 1) * n_rem / (2m)),
    j = 0..m-1.  Each frame then receives its proportional share of picks,
    spaced evenly over its grid;
  * only visual tokens take part; text tokens are always kept by the caller.
"""
from __future__ import annotations

import math

import numpy as np

FIXED_POINT_SHIFT = 40


def _masses(s32: np.ndarray) -> np.ndarray:
    """floor(s * 2**40) for fp32 s in [0, 1]: exact (a power-of-two scale of an fp32)."""
    s = s32.astype(np.float64)
    return np.floor(np.ldexp(s, FIXED_POINT_SHIFT)).astype(np.uint64)


def select_row(scores, F: int, H: int, W: int, top_p: float, budget: int):
    """Returns (kept [B] int64 ascending, k1, tag [N] uint8: 0 drop, 1 stage I, 2 stage II)."""
    s32 = np.asarray(scores, dtype=np.float32)
    N = s32.shape[0]
    if F * H * W != N:
        raise ValueError("F*H*W must equal the number of visual tokens")
    if not (0 <= budget <= N):
        raise ValueError("budget out of range")
    if not np.all(np.isfinite(s32)) or np.any(s32 < 0) or np.any(s32 > 1):
        raise ValueError("scores must be finite and in [0, 1]")
    idx = np.arange(N)
    # order: score descending, index ascending
    order = np.lexsort((idx, -s32.astype(np.float64)))

    # ---- stage I: Top-P on the fixed-point score mass, capped at the budget
    if budget == 0 or top_p <= 0.0:
        k1 = 0
    elif top_p >= 1.0:
        k1 = budget
    else:
        m = _masses(s32)
        total = int(m.sum(dtype=np.uint64))
        target = math.ceil(float(total) * float(top_p))
        if target <= 0:
            k1 = 0
        else:
            csum = np.cumsum(m[order], dtype=np.uint64)
            # shortest prefix length k with mass(prefix) >= target
            k_p = int(np.searchsorted(csum, np.uint64(target), side="left")) + 1
            k1 = min(budget, k_p)
    stage1 = order[:k1]

    tag = np.zeros(N, dtype=np.uint8)
    tag[stage1] = 1

    # ---- stage II: constant-stride, centred picks through the raster-order remainder
    rest = idx[tag == 0]
    n_rem = rest.shape[0]
    m_fill = budget - k1
    if m_fill > 0:
        j = np.arange(m_fill, dtype=np.int64)
        ranks = ((2 * j + 1) * n_rem) // (2 * m_fill)
        tag[rest[ranks]] = 2
    kept = idx[tag != 0]
    assert kept.shape[0] == budget
    return kept.astype(np.int64), int(k1), tag


def select_rows(rows, F: int, H: int, W: int, top_p: float, budget: int):
    """Row-wise select_row: (kept [R][B], k1 [R], tag [R][N])."""
    rows = np.asarray(rows, dtype=np.float32)
    out = [select_row(r, F, H, W, top_p, budget) for r in rows]
    kept = np.stack([o[0] for o in out]) if out else np.zeros((0, budget), np.int64)
    k1 = np.array([o[1] for o in out], dtype=np.int64)
    tag = np.stack([o[2] for o in out]) if out else np.zeros((0, F * H * W), np.uint8)
    return kept, k1, tag
