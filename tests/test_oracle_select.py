"""Pins for the selection oracle: hand-worked fixture, exact brute force,
exhaustive subsets, library top-K, closed forms and invariants."""
import itertools
import math
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle
import workloads as W

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "select_worked.txt")


def _load_golden():
    cases = []
    scores = grid = None
    for line in open(GOLDEN):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        if line.startswith("scores_k64:"):
            scores = np.array([int(t) for t in line.split(":")[1].split()], np.float32) / np.float32(64)
        elif line.startswith("grid:"):
            grid = tuple(int(t) for t in line.split(":")[1].split())
        else:
            a, b, c = line.split("|")
            p, budget = a.split()
            cases.append((float(p), int(budget), int(b), [int(t) for t in c.split()]))
    return scores, grid, cases


def test_golden_worked_examples():
    scores, (F, H, Wd), cases = _load_golden()
    assert len(cases) == 5
    for p, budget, k1, kept in cases:
        got, gk1, tag = oracle.select_row(scores, F, H, Wd, p, budget)
        assert gk1 == k1, (p, budget)
        assert got.tolist() == kept, (p, budget)
        assert set(np.flatnonzero(tag == 1)) <= set(kept)


# ---------------------------------------------------------------------------
# exact brute force of stage I (pure Python, rational arithmetic)
# ---------------------------------------------------------------------------

def _mass_exact(s: float) -> int:
    return math.floor(Fraction(s) * (1 << 40))


def _stage1_brute(s, top_p, budget):
    N = len(s)
    order = sorted(range(N), key=lambda i: (-float(s[i]), i))
    if budget == 0 or top_p <= 0:
        return []
    if top_p >= 1:
        return order[:budget]
    masses = [_mass_exact(float(x)) for x in s]
    total = sum(masses)
    target = math.ceil(float(total) * top_p)
    if target <= 0:
        return []
    acc = 0
    taken = []
    for i in order:
        if len(taken) == budget or acc >= target:
            break
        taken.append(i)
        acc += masses[i]
    return taken


@pytest.mark.parametrize("kind", W.SCORE_KINDS)
@pytest.mark.parametrize("top_p", [0.0, 0.1, 0.5, 0.6, 0.9, 1.0])
def test_stage1_matches_brute_force(kind, top_p):
    F, H, Wd = 3, 5, 7
    N = F * H * Wd
    rows = W.score_rows(kind, 3, N, seed=11)
    for r, budget in zip(rows, (1, 10, 60)):
        kept, k1, tag = oracle.select_row(r, F, H, Wd, top_p, budget)
        s1 = _stage1_brute(r, top_p, budget)
        assert k1 == len(s1)
        assert sorted(np.flatnonzero(tag == 1).tolist()) == sorted(s1)


def test_exhaustive_subsets_minimum_cardinality():
    """For tiny rows the Top-P count equals the least size of ANY subset reaching the target."""
    rng = np.random.default_rng(5)
    for trial in range(60):
        N = int(rng.integers(2, 11))
        s = rng.random(N).astype(np.float32)
        if trial % 3 == 0:
            s[rng.integers(0, N)] = s[0]       # ties
        s = (s / np.float32(s.sum() * 1.0001)).astype(np.float32)
        P = float(rng.choice([0.2, 0.5, 0.75, 0.95]))
        masses = [_mass_exact(float(x)) for x in s]
        target = math.ceil(float(sum(masses)) * P)
        best = None
        for k in range(N + 1):
            if any(sum(masses[i] for i in c) >= target for c in itertools.combinations(range(N), k)):
                best = k
                break
        _, k1, _ = oracle.select_row(s, 1, 1, N, P, N)
        assert k1 == best, (s, P)


def test_topk_matches_numpy_lexsort():
    N = 4 * 6 * 6
    for kind in ("uniform", "ties", "zeros", "lognormal2"):
        r = W.score_rows(kind, 1, N, seed=3)[0]
        for B in (1, 7, 50, N):
            kept, k1, _ = oracle.select_row(r, 4, 6, 6, 1.0, B)
            ref = np.sort(np.lexsort((np.arange(N), -r.astype(np.float64)))[:B])
            assert k1 == B
            assert kept.tolist() == ref.tolist()


@pytest.mark.parametrize("N,B", [(196, 20), (196, 49), (120, 12), (8192, 820), (1000, 1000), (10, 3)])
def test_uniform_only_closed_form(N, B):
    r = W.score_rows("uniform", 1, N, seed=1)[0]
    kept, k1, tag = oracle.select_row(r, 1, 1, N, 0.0, B)
    assert k1 == 0 and np.all(tag != 1)
    if N % B == 0:
        s = N // B
        assert kept.tolist() == [j * s + s // 2 for j in range(B)]     # centres of B equal blocks
    gaps = np.diff(kept)
    assert set(gaps.tolist()) <= {N // B, -(-N // B)}
    assert kept[0] == N // (2 * B)


@pytest.mark.parametrize("kind", W.SCORE_KINDS)
@pytest.mark.parametrize("top_p", [0.1, 0.5, 0.6])
def test_selection_invariants(kind, top_p):
    F, H, Wd = 8, 7, 7
    N = F * H * Wd
    budget = int(math.ceil(0.1 * N))
    r = W.score_rows(kind, 1, N, seed=2)[0]
    kept, k1, tag = oracle.select_row(r, F, H, Wd, top_p, budget)
    assert kept.shape == (budget,)
    assert np.all(np.diff(kept) > 0)
    s1 = np.flatnonzero(tag == 1)
    assert len(s1) == k1 and set(s1) <= set(kept.tolist())
    # every token outside S1 ranks below every token in S1
    key = lambda i: (-float(r[i]), i)
    if k1 and k1 < N:
        worst_in = max(key(i) for i in s1)
        best_out = min(key(i) for i in np.flatnonzero(tag != 1))
        assert worst_in < best_out
    masses = [_mass_exact(float(x)) for x in r]
    target = math.ceil(float(sum(masses)) * top_p)
    m1 = sum(masses[i] for i in s1)
    if k1 < budget:
        assert m1 >= target                      # Top-P kept mass reaches P (fixed point)
        assert m1 >= top_p * sum(masses) * (1 - 1e-15)
    if k1 > 0 and k1 < budget:
        last = max(s1, key=key)
        assert m1 - masses[last] < target        # and it is the shortest such prefix
    # stage II is grid-strided through the remainder
    rest = np.flatnonzero(tag != 1)
    u = np.flatnonzero(tag == 2)
    m = budget - k1
    assert len(u) == m
    if m > 1:
        ranks = np.searchsorted(rest, u)
        n = len(rest)
        assert set(np.diff(ranks).tolist()) <= {n // m, -(-n // m)}
        # per-frame share differs from the proportional share by at most one
        per_frame = np.bincount(u // (H * Wd), minlength=F)
        rest_frame = np.bincount(rest // (H * Wd), minlength=F)
        assert np.all(np.abs(per_frame - m * rest_frame / n) <= 1 + 1e-9)


def test_budget_edges():
    r = W.score_rows("uniform", 1, 30, seed=4)[0]
    kept, k1, tag = oracle.select_row(r, 1, 5, 6, 0.5, 0)
    assert kept.size == 0 and k1 == 0
    kept, k1, tag = oracle.select_row(r, 1, 5, 6, 0.5, 30)
    assert kept.tolist() == list(range(30))
    with pytest.raises(ValueError):
        oracle.select_row(r, 1, 5, 6, 0.5, 31)
    with pytest.raises(ValueError):
        oracle.select_row(r, 2, 5, 6, 0.5, 3)


def test_flat_attention_truncates_at_budget():
    """Nearly flat rows (the configs' value model) need more than the budget: stage I caps at B."""
    N = 196
    r = np.full(N, 1.0 / N, np.float32)
    kept, k1, tag = oracle.select_row(r, 4, 7, 7, 0.5, 20)
    assert k1 == 20 and kept.tolist() == list(range(20))
