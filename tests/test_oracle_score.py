"""Pins for the text-to-visual score oracle: rows sum to 1, scipy softmax,
closed forms (equal keys), exact brute force, permutation and GQA invariants."""
import math

import numpy as np
import pytest
from scipy.special import softmax as sp_softmax

import oracle
import workloads as W


def _tiny():
    return W.prefill_layer(W.C1, 0)


def test_softmax_rows_sum_to_one():
    p = _tiny()
    for h in range(W.C1.hq):
        P = oracle.attention_probs(p.q_text, p.k, p.q_pos0, h, W.C1.hkv)
        assert np.allclose(P.sum(axis=1), 1.0, atol=1e-13)
        # causal: text query t sees keys up to q_pos0 + t only
        for t in range(P.shape[0]):
            assert np.all(P[t, p.q_pos0 + t + 1:] == 0.0)


def test_single_query_reduces_to_scipy_softmax():
    """T = 1 with the query after every key: score = softmax(q K^T / sqrt(D)) on the visual columns."""
    rng = np.random.default_rng(0)
    D, n_vis, n_txt = 32, 50, 3
    q = rng.standard_normal((1, 1, D)).astype(np.float32)
    k = rng.standard_normal((1, n_vis + n_txt, D)).astype(np.float32)
    sc = oracle.score_layer(q, k, q_pos0=n_vis + n_txt - 1, vis_start=0, n_vis=n_vis, hkv=1)
    ref = sp_softmax(k[0].astype(np.float64) @ q[0, 0].astype(np.float64) / math.sqrt(D))[:n_vis]
    assert np.allclose(sc[0], ref, atol=1e-15, rtol=1e-12)


def test_equal_keys_closed_form():
    """Equal keys -> query t spreads 1/(q_pos0+t+1) over each visible key."""
    rng = np.random.default_rng(1)
    T, Hq, Hkv, D, n_vis = 5, 4, 2, 8, 30
    n_ctx = n_vis + T
    q = rng.standard_normal((T, Hq, D)).astype(np.float32)
    k = np.tile(rng.standard_normal((1, 1, D)).astype(np.float32), (Hkv, n_ctx, 1))
    sc = oracle.score_layer(q, k, q_pos0=n_vis, vis_start=0, n_vis=n_vis, hkv=Hkv)
    ref = sum(1.0 / (n_vis + t + 1) for t in range(T)) / T
    assert np.allclose(sc, ref, atol=1e-15)
    # and with an offset visual window
    sc2 = oracle.score_layer(q, k, q_pos0=n_vis, vis_start=3, n_vis=10, hkv=Hkv)
    assert np.allclose(sc2, ref, atol=1e-15)


def test_fsum_brute_force_tiny_config():
    """Triple loop with math.fsum over the tiny configuration (4 heads x 16 text x 212 keys)."""
    cfg = W.C1
    p = _tiny()
    sc = oracle.score_layer(p.q_text, p.k, p.q_pos0, 0, cfg.n_vis, cfg.hkv)
    G = cfg.group
    s_ = 1.0 / math.sqrt(cfg.d)
    for h in range(cfg.hq):
        g = h // G
        acc = [[] for _ in range(cfg.n_vis)]
        for t in range(cfg.n_text):
            lim = p.q_pos0 + t + 1
            logits = [s_ * math.fsum(float(p.q_text[t, h, d]) * float(p.k[g, n, d]) for d in range(cfg.d))
                      for n in range(lim)]
            m = max(logits)
            w = [math.exp(x - m) for x in logits]
            z = math.fsum(w)
            for i in range(cfg.n_vis):
                acc[i].append(w[i] / z)
        ref = [math.fsum(a) / cfg.n_text for a in acc]
        assert np.allclose(sc[h], ref, atol=1e-15, rtol=1e-12)


def test_permuting_text_queries_leaves_scores_unchanged():
    """When every text query sees the whole context, the mean over queries is order-free."""
    rng = np.random.default_rng(2)
    T, Hq, Hkv, D, n_vis = 6, 4, 2, 16, 40
    q = rng.standard_normal((T, Hq, D)).astype(np.float32)
    k = rng.standard_normal((Hkv, n_vis + T, D)).astype(np.float32)
    pos0 = n_vis + T - 1
    a = oracle.score_layer(q, k, pos0, 0, n_vis, Hkv)
    b = oracle.score_layer(q[rng.permutation(T)], k, pos0, 0, n_vis, Hkv)
    assert np.allclose(a, b, atol=1e-15)


def test_gqa_equals_mha_with_repeated_keys():
    p = _tiny()
    cfg = W.C1
    a = oracle.score_layer(p.q_text, p.k, p.q_pos0, 0, cfg.n_vis, cfg.hkv)
    b = oracle.score_layer(p.q_text, np.repeat(p.k, cfg.group, axis=0), p.q_pos0, 0, cfg.n_vis, cfg.hq)
    assert np.allclose(a, b, atol=0)


def test_aggregation_invariants():
    p = _tiny()
    cfg = W.C1
    # identical q heads inside each group -> the KV-head row equals each q-head row
    q = p.q_text.copy()
    for g in range(cfg.hkv):
        q[:, g * cfg.group:(g + 1) * cfg.group] = q[:, g * cfg.group:g * cfg.group + 1]
    sq = oracle.score_layer(q, p.k, p.q_pos0, 0, cfg.n_vis, cfg.hkv)
    kv = oracle.aggregate_heads(sq, cfg.hkv, "kvhead")
    for h in range(cfg.hq):
        assert np.allclose(kv[h // cfg.group], sq[h], atol=1e-15)
    # the all-heads row of a layer sums to the mean visual attention mass (<= 1)
    al = oracle.aggregate_heads(sq, cfg.hkv, "all")
    assert al.shape == (1, cfg.n_vis) and 0 < al.sum() <= 1.0


def test_sink_and_salient_tokens_stand_out():
    """The value model's sink and query-aligned keys get more attention than the median token."""
    cfg = W.C1
    p = _tiny()
    sc = oracle.aggregate_heads(oracle.score_layer(p.q_text, p.k, p.q_pos0, 0, cfg.n_vis, cfg.hkv), cfg.hkv, "all")[0]
    med = np.median(sc)
    assert np.all(sc[p.salient] > med)


def test_aggregate_heads_hand_case():
    """Hand-computed group and overall means of a 4-head, 3-token score table
    (two KV heads of two q heads each)."""
    sq = np.array([[1.0, 2.0, 3.0],
                   [3.0, 6.0, 1.0],
                   [0.0, 4.0, 8.0],
                   [4.0, 0.0, 4.0]])
    assert np.array_equal(oracle.aggregate_heads(sq, 2, "qhead"), sq)
    assert np.array_equal(oracle.aggregate_heads(sq, 2, "kvhead"), [[2.0, 4.0, 2.0], [2.0, 2.0, 6.0]])
    assert np.array_equal(oracle.aggregate_heads(sq, 2, "all"), [[2.0, 3.0, 4.0]])
    assert np.array_equal(oracle.aggregate_heads(sq, 1, "kvhead"), [[2.0, 3.0, 4.0]])
    assert np.array_equal(oracle.aggregate_heads(sq, 4, "kvhead"), sq)


def _one_hot_layers(targets, T, D, hkv, n_vis, n_text):
    """Layers whose q head h sends every text query's whole softmax to one
    visual token targets[l][h]: that token's key is the unit vector e_h of its
    KV head (all other keys are zero), and every query of head h is 400 e_h,
    so its logit is 400/sqrt(D) = 100 above every other key's (exp(-100) is
    far below fp64 resolution of 1)."""
    layers = []
    Hq = len(targets[0])
    G = Hq // hkv
    for tl in targets:
        q = np.zeros((T, Hq, D), np.float32)
        k = np.zeros((hkv, n_vis + n_text, D), np.float32)
        for h, tok in enumerate(tl):
            q[:, h, h] = 400.0
            k[h // G, tok, h] = 1.0
        layers.append((q, k))
    return layers


def test_score_rows_for_config_one_hot_closed_form():
    """Each (layer, q head) puts all its attention on one known visual token,
    so its score row is exactly an indicator.  The rows then follow by hand:
    a (layer, KV head) row holds 1/G at its group's targets, a layer row 1/Hq
    at the layer's targets, and the single row 1/(L Hq) at every target
    (a token named twice collects twice)."""
    T, D, hkv, n_vis, n_text = 3, 16, 2, 12, 3
    targets = [[0, 5, 7, 11], [5, 2, 9, 9], [1, 1, 4, 6]]      # [layer][q head], G = 2
    L, Hq, G = len(targets), len(targets[0]), 2
    layers = _one_hot_layers(targets, T, D, hkv, n_vis, n_text)
    kvh = oracle.score_rows_for_config(layers, n_vis, n_vis, hkv, "layer_kvhead")
    lay = oracle.score_rows_for_config(layers, n_vis, n_vis, hkv, "layer")
    one = oracle.score_rows_for_config(layers, n_vis, n_vis, hkv, "all")
    want_kvh = np.zeros((L * hkv, n_vis))
    want_lay = np.zeros((L, n_vis))
    want_one = np.zeros((1, n_vis))
    for l, tl in enumerate(targets):
        for h, tok in enumerate(tl):
            want_kvh[l * hkv + h // G, tok] += 1.0 / G
            want_lay[l, tok] += 1.0 / Hq
            want_one[0, tok] += 1.0 / (L * Hq)
    assert kvh.shape == want_kvh.shape and np.allclose(kvh, want_kvh, atol=1e-15)
    assert lay.shape == want_lay.shape and np.allclose(lay, want_lay, atol=1e-15)
    assert one.shape == want_one.shape and np.allclose(one, want_one, atol=1e-15)
    # spot values, written out: layer 1, KV head 1 holds token 9 twice
    assert kvh[1 * hkv + 1, 9] == pytest.approx(1.0, abs=1e-15)
    assert one[0, 5] == pytest.approx(2.0 / 12.0, abs=1e-15)
    with pytest.raises(ValueError):
        oracle.score_rows_for_config(layers, n_vis, n_vis, hkv, "rows")
