"""Pins for the acceptance oracle: greedy brute force, greedy speculative
decoding == plain greedy decoding on a toy model, acceptance frequency ->
sum_v min(p, q), emitted token ~ p, fixed-point sampler = inverse CDF."""
import math

import numpy as np
import pytest

import oracle
import workloads as W


def test_greedy_examples_by_hand():
    V = 5
    logits = np.full((1, 4, V), -1.0, np.float32)
    # argmaxes of the 4 rows: 2, 0, 4, 1 (row 1 has a tie at 0 and 3 -> lowest index)
    logits[0, 0, 2] = 5
    logits[0, 1, 0] = 3
    logits[0, 1, 3] = 3
    logits[0, 2, 4] = 1
    logits[0, 3, 1] = 2
    cases = [([2, 0, 4], 3, 1), ([2, 0, 1], 2, 4), ([1, 0, 4], 0, 2), ([2, 3, 4], 1, 0)]
    for d, n, nxt in cases:
        na, nt = oracle.verify_greedy(np.array([d]), logits)
        assert (na[0], nt[0]) == (n, nxt)


def _toy_logits(prefix, V, seed, noise=0.0):
    """A deterministic toy 'model': next-token logits as a hash of the prefix."""
    h = hash((tuple(prefix), seed)) & 0xFFFFFFFF
    rng = np.random.default_rng(h)
    base = rng.standard_normal(V)
    if noise:
        nrng = np.random.default_rng(h ^ 0x5A5A5A5A)
        base = base + noise * nrng.standard_normal(V)
    return base.astype(np.float32)


@pytest.mark.parametrize("gamma", [1, 4, 9])
def test_greedy_speculative_output_equals_dense_greedy(gamma):
    V, steps = 16, 40
    prompt = [1, 2, 3]
    # plain greedy decoding with the target
    ref = list(prompt)
    while len(ref) < len(prompt) + steps:
        ref.append(int(np.argmax(_toy_logits(ref, V, 0))))
    # speculative decoding: a noisy draft proposes gamma tokens, the oracle verifies
    out = list(prompt)
    cycles = 0
    while len(out) < len(prompt) + steps:
        draft = []
        for _ in range(gamma):
            draft.append(int(np.argmax(_toy_logits(out + draft, V, 0, noise=0.8))))
        tl = np.stack([_toy_logits(out + draft[:i], V, 0) for i in range(gamma + 1)])
        n, nxt = oracle.verify_greedy(np.array([draft]), tl[None])
        out += draft[:n[0]] + [int(nxt[0])]
        cycles += 1
    assert out[:len(ref)] == ref
    assert cycles < steps   # some drafts were accepted


def test_fixed_point_sampler_is_inverse_cdf():
    w = np.array([0.25, 0.0, 0.5, 0.25], np.float32)
    # cumulative fixed-point mass: 1/4, 1/4, 3/4, 1 of 2^40
    assert oracle.sample_fixed_point(w, 0.0) == 0
    assert oracle.sample_fixed_point(w, 0.2499) == 0
    assert oracle.sample_fixed_point(w, 0.25) == 2
    assert oracle.sample_fixed_point(w, 0.7499) == 2
    assert oracle.sample_fixed_point(w, 0.75) == 3
    assert oracle.sample_fixed_point(w, np.nextafter(np.float32(1), np.float32(0))) == 3
    assert oracle.sample_fixed_point(np.zeros(4, np.float32), 0.5) == -1
    # unnormalised weights are fine
    assert oracle.sample_fixed_point(np.array([1e-3, 1e-3], np.float32), 0.6) == 1


def test_sampler_distribution_chi2():
    rng = np.random.default_rng(0)
    w = np.array([0.1, 0.4, 0.05, 0.3, 0.15], np.float32)
    n = 40000
    counts = np.zeros(5)
    for u in rng.random(n, dtype=np.float32):
        counts[oracle.sample_fixed_point(w, u)] += 1
    exp = n * w / w.sum()
    chi2 = ((counts - exp) ** 2 / exp).sum()
    assert chi2 < 20.5   # 4 dof, p ~ 4e-4


def _mc_reject(p, q, trials, seed):
    """Monte Carlo of one-position verify: d ~ q, u ~ U[0,1); returns (accept rate, emitted counts)."""
    rng = np.random.default_rng(seed)
    V = p.shape[-1]
    acc = 0
    emitted = np.zeros(V)
    qs = q.astype(np.float64) / q.astype(np.float64).sum()
    ds = rng.choice(V, size=trials, p=qs)
    us = rng.random((trials, 2), dtype=np.float32)
    P = np.stack([p, p])[None]
    Q = q[None, None]
    for d, u in zip(ds, us):
        n, nxt = oracle.verify_reject(np.array([[d]]), P, Q, u[None])
        acc += int(n[0])
        emitted[d if n[0] == 1 else nxt[0]] += 1
    return acc / trials, emitted


def test_acceptance_rate_matches_sum_min_and_output_is_target_distribution():
    V = 8
    rng = np.random.default_rng(3)
    lp = 1.5 * rng.standard_normal(V)
    lq = lp + rng.standard_normal(V)
    p = (np.exp(lp) / np.exp(lp).sum()).astype(np.float32)
    q = (np.exp(lq) / np.exp(lq).sum()).astype(np.float32)
    trials = 100_000
    rate, emitted = _mc_reject(p, q, trials, seed=9)
    beta = float(np.minimum(p.astype(np.float64), q.astype(np.float64)).sum())
    sigma = math.sqrt(beta * (1 - beta) / trials)
    assert abs(rate - beta) < 4 * sigma, (rate, beta)
    # the first emitted token (accepted draft or resample) is distributed as p
    exp = trials * p.astype(np.float64) / p.astype(np.float64).sum()
    chi2 = ((emitted - exp) ** 2 / exp).sum()
    assert chi2 < 29.9   # 7 dof, p ~ 1e-4


def test_expected_emitted_per_cycle_closed_form():
    """E[tokens per cycle] = sum_{k=0}^{gamma} prod_{i<k} beta_i with independent positions."""
    V, gamma, trials = 6, 3, 20_000
    rng = np.random.default_rng(4)
    ps, qs = [], []
    for i in range(gamma + 1):
        lp = rng.standard_normal(V)
        lq = lp + 0.7 * rng.standard_normal(V)
        ps.append((np.exp(lp) / np.exp(lp).sum()).astype(np.float32))
        qs.append((np.exp(lq) / np.exp(lq).sum()).astype(np.float32))
    P = np.stack(ps)[None]
    Q = np.stack(qs[:gamma])[None]
    betas = [float(np.minimum(ps[i].astype(np.float64), qs[i].astype(np.float64)).sum()) for i in range(gamma)]
    expect = sum(np.prod(betas[:k]) for k in range(gamma + 1))
    tot = 0
    for t in range(trials):
        d = np.array([[rng.choice(V, p=qs[i].astype(np.float64) / qs[i].astype(np.float64).sum())
                       for i in range(gamma)]])
        u = rng.random((1, gamma + 1), dtype=np.float32)
        n, _ = oracle.verify_reject(d, P, Q, u)
        tot += int(n[0]) + 1
    mean = tot / trials
    assert abs(mean - expect) < 0.03, (mean, expect)


def test_reject_special_cases():
    V = 4
    p = np.array([[[0.0, 1.0, 0.0, 0.0], [0.25, 0.25, 0.25, 0.25]]], np.float32)
    # draft equal to the target -> always accepted, bonus drawn from p_gamma with u_gamma
    q = np.array([[[0.0, 1.0, 0.0, 0.0]]], np.float32)
    n, t = oracle.verify_reject(np.array([[1]]), p, q, np.array([[0.999, 0.6]], np.float32))
    assert (n[0], t[0]) == (1, 2)
    # the draft puts all mass on a token the target never emits -> reject, residual is the target row
    q2 = np.array([[[0.0, 0.0, 1.0, 0.0]]], np.float32)
    n, t = oracle.verify_reject(np.array([[2]]), p, q2, np.array([[0.0001, 0.3]], np.float32))
    assert (n[0], t[0]) == (0, 1)


def test_acceptance_inputs_from_generator_are_probabilities():
    vi = W.verify_inputs(1, 2, 4, 1024)
    assert np.allclose(vi.p.astype(np.float64).sum(-1), 1.0, atol=1e-5)
    assert np.allclose(vi.q.astype(np.float64).sum(-1), 1.0, atol=1e-5)
    n, t = oracle.verify_reject(vi.draft_tok_sampled, vi.p, vi.q, vi.u)
    assert np.all((0 <= n) & (n <= 4)) and np.all((0 <= t) & (t < 1024))
