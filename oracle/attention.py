"""Oracle: draft and verify decode attention (test infrastructure only).

Sources: Sparse-to-Dense explainer, technical summary ("decoding process"):
the sparse model drafts gamma tokens one at a time over the selected KV; the
dense model checks all gamma of them with a single I/O pass over the full KV
cache.  SpecVLM listing, section 4 ("pain points"): at every decode step the
whole, growing KV cache must be loaded, so decoding is bound by memory
bandwidth.

Definition (a causal decoder): for batch b, new query i < nq and q head h,
the visible keys are n < kv_len[b] - nq + i + 1 when causal_tail is set (the
nq new tokens' own keys are already appended and query i sees up to itself),
otherwise all n < kv_len[b];
    o[b,i,h] = sum_n softmax_n(scale * <q[b,i,h], k[b,g,n]>) * v[b,g,n],
    lse[b,i,h] = log sum_n exp(scale * <q, k_n>),   g = h // (Hq / Hkv).
"""
from __future__ import annotations

import numpy as np


def decode_attn(q, k, v, kv_len, causal_tail: bool, scale: float | None = None):
    """q: [B][nq][Hq][D]; k, v: [B][Hkv][N][D] (or [Hkv][N][D] for B = 1).

    Returns (o [B][nq][Hq][D] fp64, lse [B][nq][Hq] fp64)."""
    q = np.asarray(q, dtype=np.float32).astype(np.float64)
    k = np.asarray(k, dtype=np.float32).astype(np.float64)
    v = np.asarray(v, dtype=np.float32).astype(np.float64)
    if k.ndim == 3:
        k = k[None]
        v = v[None]
    B, nq, Hq, D = q.shape
    Hkv = k.shape[1]
    G = Hq // Hkv
    if scale is None:
        scale = 1.0 / np.sqrt(D)
    kv_len = np.asarray(kv_len, dtype=np.int64).reshape(B)
    o = np.zeros((B, nq, Hq, D))
    lse = np.zeros((B, nq, Hq))
    for b in range(B):
        n_kv = int(kv_len[b])
        for i in range(nq):
            limit = n_kv - nq + i + 1 if causal_tail else n_kv
            for h in range(Hq):
                g = h // G
                if limit <= 0:
                    o[b, i, h] = 0.0
                    lse[b, i, h] = -np.inf
                    continue
                s = scale * (k[b, g, :limit] @ q[b, i, h])
                m = s.max()
                e = np.exp(s - m)
                z = e.sum()
                o[b, i, h] = (e @ v[b, g, :limit]) / z
                lse[b, i, h] = m + np.log(z)
    return o, lse
