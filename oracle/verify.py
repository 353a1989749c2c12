"""Oracle: acceptance of drafted tokens (test infrastructure only).

Greedy rule - Sparse-to-Dense explainer, technical summary ("decoding
process"): the dense model finds the longest prefix of the gamma drafted
tokens that matches its own predictions (n tokens) and additionally accepts
one "bonus" token, its own prediction after that prefix.

Rejection rule - ParallelVLM notes, background and "parallel decoding":
drafted candidates are accepted by rejection sampling, which keeps the output
distribution identical to the target's; a rejected token is resampled from
the target's distribution.  The pages print no formula; the rule taken is the
standard speculative-sampling one (Leviathan et al. 2023; Chen et al. 2023):
accept draft token d_i with probability min(1, p_i(d_i) / q_i(d_i)); at the
first rejection draw from max(0, p_i - q_i) renormalised; if all gamma are
accepted draw the bonus token from p_gamma.

Readings fixed so that results are exactly reproducible:
  * the acceptance test is u_i * q_i(d_i) <= p_i(d_i) in fp64 (the product of
    two fp32 numbers is exact there); q_i(d_i) = 0 accepts;
  * exactly one categorical draw happens per call and it uses u_gamma;
  * the draw is an inverse CDF in fixed point: weights w (fp32 in [0, 1])
    become m_v = floor(w_v * 2**40), W = sum m_v,
    t = min(floor(double(u) * double(W)), W - 1), and the token is the least
    v whose running sum of m exceeds t;
  * the residual max(0, p - q) is formed in fp32; if its fixed-point mass is
    0 the draw falls back to p_i, and if that is 0 too, to argmax p_i;
  * argmax takes the lowest index among equal maxima.
"""
from __future__ import annotations

import math

import numpy as np

SHIFT = 40


def _argmax_lowest(x) -> int:
    x = np.asarray(x)
    return int(np.flatnonzero(x == x.max())[0])


def sample_fixed_point(w, u) -> int:
    """Inverse-CDF draw from non-negative fp32 weights w with fp32 uniform u; -1 if mass is 0."""
    w = np.asarray(w, dtype=np.float32)
    m = np.floor(np.ldexp(w.astype(np.float64), SHIFT)).astype(np.uint64)
    total = int(m.sum(dtype=np.uint64))
    if total == 0:
        return -1
    t = math.floor(float(np.float32(u)) * float(total))
    t = min(t, total - 1)
    csum = np.cumsum(m, dtype=np.uint64)
    return int(np.searchsorted(csum, np.uint64(t), side="right"))


def verify_greedy(draft_tok, logits):
    """draft_tok: [B][gamma]; logits: [B][gamma+1][V] fp32 -> (n_accept [B], next_tok [B])."""
    draft_tok = np.asarray(draft_tok, dtype=np.int64)
    logits = np.asarray(logits, dtype=np.float32)
    B, gamma = draft_tok.shape
    n_acc = np.zeros(B, np.int64)
    nxt = np.zeros(B, np.int64)
    for b in range(B):
        a = [_argmax_lowest(logits[b, i]) for i in range(gamma + 1)]
        n = 0
        while n < gamma and draft_tok[b, n] == a[n]:
            n += 1
        n_acc[b] = n
        nxt[b] = a[n]
    return n_acc, nxt


def verify_reject(draft_tok, p, q, u):
    """draft_tok: [B][gamma]; p: [B][gamma+1][V]; q: [B][gamma][V]; u: [B][gamma+1] (all fp32).

    Returns (n_accept [B], next_tok [B])."""
    draft_tok = np.asarray(draft_tok, dtype=np.int64)
    p = np.asarray(p, dtype=np.float32)
    q = np.asarray(q, dtype=np.float32)
    u = np.asarray(u, dtype=np.float32)
    B, gamma = draft_tok.shape
    n_acc = np.zeros(B, np.int64)
    nxt = np.zeros(B, np.int64)
    for b in range(B):
        n = gamma
        for i in range(gamma):
            d = int(draft_tok[b, i])
            pd = float(p[b, i, d])
            qd = float(q[b, i, d])
            if not (float(u[b, i]) * qd <= pd):
                n = i
                break
        if n < gamma:
            resid = np.maximum(p[b, n] - q[b, n], np.float32(0.0))   # fp32 arithmetic
            tok = sample_fixed_point(resid, u[b, gamma])
        else:
            tok = sample_fixed_point(p[b, gamma], u[b, gamma])
        if tok < 0:
            tok = sample_fixed_point(p[b, n], u[b, gamma])
        if tok < 0:
            tok = _argmax_lowest(p[b, n])
        n_acc[b] = n
        nxt[b] = tok
    return n_acc, nxt
