"""Oracle: mean text-to-visual attention score (test infrastructure only).

Source: SpecVLM technology-transfer listing, section 5 ("solution"): the
pruning module first computes, from the target model's attention matrix, the
average attention that the text tokens pay to each visual token.  The
Sparse-to-Dense explainer ("KV cache selection") computes the same mean
text-to-visual attention at prefill, separately for every layer and head.

Readings taken where the pages are silent:
  * every text token of the prompt is a query; text query t sits at absolute
    position q_pos0 + t and, being causal, sees keys 0..q_pos0 + t;
  * the softmax runs over that whole visible range (sink and text keys
    included); the visual columns are then read out of the normalised row;
  * inputs are post-rotary q and k; scale = 1/sqrt(D) unless given;
  * grouped-query attention: q head h reads KV head h // (Hq / Hkv);
  * aggregation: a KV-head row is the mean over its q heads, a layer row is
    the mean over all q heads; several layers are averaged by the caller.
"""
from __future__ import annotations

import numpy as np


def _f64(x) -> np.ndarray:
    return np.asarray(x, dtype=np.float32).astype(np.float64)


def attention_probs(q_text, k, q_pos0: int, h: int, hkv: int, scale: float | None = None) -> np.ndarray:
    """Full causal softmax rows of q head h: [T][n_ctx], masked entries 0.

    q_text: [T][Hq][D]; k: [Hkv][n_ctx][D]."""
    q = _f64(q_text)
    kk = _f64(k)
    T, Hq, D = q.shape
    n_ctx = kk.shape[1]
    G = Hq // hkv
    if scale is None:
        scale = 1.0 / np.sqrt(D)
    g = h // G
    s = scale * (q[:, h, :] @ kk[g].T)                        # [T][n_ctx]
    pos = q_pos0 + np.arange(T)[:, None]
    visible = np.arange(n_ctx)[None, :] <= pos
    s = np.where(visible, s, -np.inf)
    m = s.max(axis=1, keepdims=True)
    e = np.where(visible, np.exp(s - m), 0.0)
    return e / e.sum(axis=1, keepdims=True)


def score_layer(q_text, k, q_pos0: int, vis_start: int, n_vis: int, hkv: int,
                scale: float | None = None) -> np.ndarray:
    """Per q head h and visual token i: mean over text queries of P[t, h, vis_start + i].

    Returns [Hq][n_vis] fp64."""
    Hq = np.asarray(q_text).shape[1]
    T = np.asarray(q_text).shape[0]
    out = np.empty((Hq, n_vis), dtype=np.float64)
    for h in range(Hq):
        p = attention_probs(q_text, k, q_pos0, h, hkv, scale)
        out[h] = p[:, vis_start:vis_start + n_vis].sum(axis=0) / T
    return out


def aggregate_heads(score_qh: np.ndarray, hkv: int, agg: str) -> np.ndarray:
    """agg = "qhead" -> [Hq][n]; "kvhead" -> mean over each group, [Hkv][n]; "all" -> [1][n]."""
    Hq, n = score_qh.shape
    G = Hq // hkv
    if agg == "qhead":
        return score_qh.copy()
    if agg == "kvhead":
        return score_qh.reshape(hkv, G, n).mean(axis=1)
    if agg == "all":
        return score_qh.mean(axis=0, keepdims=True)
    raise ValueError(agg)


def score_rows_for_config(layers_q_k, q_pos0: int, n_vis: int, hkv: int, rows: str) -> np.ndarray:
    """Selection rows from several layers.

    rows = "all": one row, mean over layers and heads (the single SpecVLM
    signal); "layer": one row per layer (mean over its heads);
    "layer_kvhead": one row per (layer, KV head), the per-layer, per-head
    selection of the Sparse-to-Dense method."""
    per_layer = []
    for q_text, k in layers_q_k:
        sq = score_layer(q_text, k, q_pos0, 0, n_vis, hkv)
        if rows == "all" or rows == "layer":
            per_layer.append(aggregate_heads(sq, hkv, "all"))
        elif rows == "layer_kvhead":
            per_layer.append(aggregate_heads(sq, hkv, "kvhead"))
        else:
            raise ValueError(rows)
    stacked = np.concatenate(per_layer, axis=0)
    if rows == "all":
        return stacked.mean(axis=0, keepdims=True)
    return stacked
