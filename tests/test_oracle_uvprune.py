"""Pins of the UV-Prune oracle (ParallelVLM notes, method section 1) against
closed forms, brute force in plain Python, invariants and the telescoping
identity of the printed double sum."""
import math

import numpy as np
import pytest

from oracle.uvprune import cosine_matrix, uvprune_keep, uvprune_scores


def _layers(seed, L1, m, n, d):
    rng = np.random.default_rng(seed)
    v = [rng.standard_normal((m, d)).astype(np.float32) for _ in range(L1)]
    x = [rng.standard_normal((n, d)).astype(np.float32) for _ in range(L1)]
    return v, x


def _brute(v_layers, x_layers):
    """the printed double sum, one term at a time, in plain Python with fsum"""
    L1, m, n = len(v_layers), len(v_layers[0]), len(x_layers[0])

    def cos(a, b):
        na = math.sqrt(math.fsum(float(t) * float(t) for t in a))
        nb = math.sqrt(math.fsum(float(t) * float(t) for t in b))
        if na == 0.0 or nb == 0.0:
            return 0.0
        return math.fsum(float(s) * float(t) for s, t in zip(a, b)) / (na * nb)

    out = []
    for i in range(m):
        terms = []
        for j in range(n):
            for l in range(1, L1):
                terms.append(cos(v_layers[l][i], x_layers[l][j]) - cos(v_layers[l - 1][i], x_layers[l - 1][j]))
        out.append(math.fsum(terms))
    return np.array(out)


def test_matches_plain_python_brute_force():
    v, x = _layers(1, 4, 6, 5, 7)
    np.testing.assert_allclose(uvprune_scores(v, x), _brute(v, x), rtol=0, atol=1e-12)


def test_telescoping_to_first_and_last_layer():
    """sum over l of (S^l - S^(l-1)) equals S^L - S^0 for any intermediate layers"""
    v, x = _layers(2, 6, 40, 9, 32)
    full = uvprune_scores(v, x)
    two = uvprune_scores([v[0], v[-1]], [x[0], x[-1]])
    np.testing.assert_allclose(full, two, rtol=0, atol=1e-12)
    # and a wrong-sign or dropped-layer variant would differ
    assert not np.allclose(full, uvprune_scores([v[1], v[-1]], [x[1], x[-1]]), atol=1e-6)


def test_closed_form_aligned_at_L_orthogonal_at_0():
    """video token aligned with every text token at layer L and orthogonal to
    all of them at layer 0 scores exactly n; the reverse scores -n"""
    d, n = 8, 5
    e0, e1 = np.eye(d, dtype=np.float32)[0], np.eye(d, dtype=np.float32)[1]
    x0 = np.tile(e0, (n, 1)) * np.arange(1, n + 1, dtype=np.float32)[:, None]   # norms differ, direction e0
    xL = np.tile(e1, (n, 1)) * 3.0
    v0 = np.stack([e1, e0])
    vL = np.stack([2.5 * e1, e1 + e0 * 0])
    vL[1] = e0            # token 1: aligned at 0, orthogonal at L
    s = uvprune_scores([v0, vL], [x0, xL])
    assert s[0] == pytest.approx(n, abs=1e-12)
    assert s[1] == pytest.approx(-n, abs=1e-12)


def test_zero_vectors_score_zero_and_scale_invariance():
    v, x = _layers(3, 2, 10, 4, 16)
    v[0][3] = 0.0
    v[1][3] = 0.0
    s = uvprune_scores(v, x)
    assert s[3] == 0.0
    # positive rescaling of any hidden vector changes nothing
    v2 = [a.copy() for a in v]
    x2 = [a.copy() for a in x]
    v2[1][5] *= 8.0   # powers of two keep the fp32 inputs exact
    x2[0][2] *= 0.25
    np.testing.assert_allclose(uvprune_scores(v2, x2), s, rtol=0, atol=1e-12)
    # negating a layer-L video vector flips the sign of its layer-L similarities
    v3 = [a.copy() for a in v]
    v3[1][6] *= -1.0
    c0 = cosine_matrix(v[0], x[0]).sum(axis=1)
    cL = cosine_matrix(v[1], x[1]).sum(axis=1)
    assert uvprune_scores(v3, x)[6] == pytest.approx(-cL[6] - c0[6], abs=1e-12)


def test_permutations():
    v, x = _layers(4, 3, 12, 6, 8)
    s = uvprune_scores(v, x)
    pt = np.random.default_rng(0).permutation(6)
    np.testing.assert_allclose(uvprune_scores(v, [a[pt] for a in x]), s, rtol=0, atol=1e-12)
    pv = np.random.default_rng(1).permutation(12)
    np.testing.assert_allclose(uvprune_scores([a[pv] for a in v], x), s[pv], rtol=0, atol=1e-12)


def test_cosine_matrix_against_numpy_normalisation():
    rng = np.random.default_rng(5)
    a, b = rng.standard_normal((7, 11)), rng.standard_normal((4, 11))
    ref = (a / np.linalg.norm(a, axis=1, keepdims=True)) @ (b / np.linalg.norm(b, axis=1, keepdims=True)).T
    np.testing.assert_allclose(cosine_matrix(a, b), ref.astype(np.float64), rtol=1e-6, atol=1e-7)


@pytest.mark.parametrize("alpha", [0.0, 0.5, 0.9, 1.0])
def test_keep_is_top_k_by_score_then_index(alpha):
    rng = np.random.default_rng(6)
    s = rng.integers(0, 20, size=101).astype(np.float64)   # many exact ties
    k = uvprune_keep(s, alpha)
    K = min(101, max(0, math.ceil((1.0 - alpha) * 101)))
    assert k.size == K
    brute = sorted(range(101), key=lambda i: (-s[i], i))[:K]
    assert list(k) == sorted(brute)
