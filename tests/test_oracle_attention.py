"""Pins for the decode-attention oracle: a hand-worked case, scipy softmax,
closed forms, exact brute force, verify == sequential single-query decode,
GQA == MHA with repeated KV."""
import math

import numpy as np
import pytest
from scipy.special import softmax as sp_softmax

import oracle
import workloads as W


def test_hand_worked_two_keys():
    # scale 1: logits 0 and ln 3 -> weights 1/4, 3/4; o = (1/4)(4,0) + (3/4)(0,4) = (1, 3); lse = ln 4
    q = np.array([[[[1.0, 0.0]]]], np.float32)
    k = np.array([[[0.0, 1.0], [math.log(3.0), 0.0]]], np.float32)
    v = np.array([[[4.0, 0.0], [0.0, 4.0]]], np.float32)
    o, lse = oracle.decode_attn(q, k, v, [2], causal_tail=False, scale=1.0)
    assert np.allclose(o[0, 0, 0], [1.0, 3.0], atol=1e-6)
    assert abs(lse[0, 0, 0] - math.log(4.0)) < 1e-6


def test_single_query_equals_scipy_softmax():
    rng = np.random.default_rng(0)
    D, N = 64, 300
    q = W.bf16_round(rng.standard_normal((1, 1, 1, D)).astype(np.float32))
    k = W.bf16_round(rng.standard_normal((1, N, D)).astype(np.float32))
    v = W.bf16_round(rng.standard_normal((1, N, D)).astype(np.float32))
    o, lse = oracle.decode_attn(q, k, v, [N], causal_tail=False)
    s = (k[0].astype(np.float64) @ q[0, 0, 0].astype(np.float64)) / math.sqrt(D)
    ref = sp_softmax(s) @ v[0].astype(np.float64)
    assert np.allclose(o[0, 0, 0], ref, rtol=1e-12, atol=1e-12)
    from scipy.special import logsumexp
    assert abs(lse[0, 0, 0] - logsumexp(s)) < 1e-12


def test_one_key_returns_its_value():
    rng = np.random.default_rng(1)
    q = rng.standard_normal((1, 1, 4, 32)).astype(np.float32)
    k = rng.standard_normal((2, 1, 32)).astype(np.float32)
    v = rng.standard_normal((2, 1, 32)).astype(np.float32)
    o, _ = oracle.decode_attn(q, k, v, [1], causal_tail=False)
    for h in range(4):
        assert np.allclose(o[0, 0, h], v[h // 2, 0], atol=0)


def test_equal_keys_give_mean_of_visible_values():
    """All keys equal -> uniform weights over the visible prefix (pins the causal limit)."""
    rng = np.random.default_rng(2)
    B, nq, Hq, Hkv, D, N = 2, 5, 6, 2, 16, 40
    q = rng.standard_normal((B, nq, Hq, D)).astype(np.float32)
    k = np.tile(rng.standard_normal((1, 1, 1, D)).astype(np.float32), (B, Hkv, N, 1))
    v = rng.standard_normal((B, Hkv, N, D)).astype(np.float32)
    kv_len = [N, N - 7]
    o, lse = oracle.decode_attn(q, k, v, kv_len, causal_tail=True)
    for b in range(B):
        for i in range(nq):
            lim = kv_len[b] - nq + i + 1
            for h in range(Hq):
                g = h // (Hq // Hkv)
                assert np.allclose(o[b, i, h], v[b, g, :lim].astype(np.float64).mean(axis=0), atol=1e-12)
                s0 = float(k[b, g, 0].astype(np.float64) @ q[b, i, h].astype(np.float64)) / math.sqrt(D)
                assert abs(lse[b, i, h] - (s0 + math.log(lim))) < 1e-9


def test_verify_equals_sequential_single_query_decodes():
    """One dense pass over gamma+1 queries == gamma+1 single-query decodes on the prefixes."""
    rng = np.random.default_rng(3)
    Hq, Hkv, D, N, nq = 8, 2, 32, 90, 6
    q = W.bf16_round(rng.standard_normal((1, nq, Hq, D)).astype(np.float32))
    k = W.bf16_round(rng.standard_normal((Hkv, N, D)).astype(np.float32))
    v = W.bf16_round(rng.standard_normal((Hkv, N, D)).astype(np.float32))
    o, lse = oracle.decode_attn(q, k, v, [N], causal_tail=True)
    for i in range(nq):
        n_i = N - nq + i + 1
        oi, li = oracle.decode_attn(q[:, i:i + 1], k[:, :n_i], v[:, :n_i], [n_i], causal_tail=False)
        assert np.allclose(o[0, i], oi[0, 0], atol=1e-13)
        assert np.allclose(lse[0, i], li[0, 0], atol=1e-13)


def test_gqa_equals_mha_with_repeated_kv():
    rng = np.random.default_rng(4)
    Hq, Hkv, D, N = 12, 3, 16, 50
    q = rng.standard_normal((1, 3, Hq, D)).astype(np.float32)
    k = rng.standard_normal((Hkv, N, D)).astype(np.float32)
    v = rng.standard_normal((Hkv, N, D)).astype(np.float32)
    o1, l1 = oracle.decode_attn(q, k, v, [N], causal_tail=True)
    G = Hq // Hkv
    o2, l2 = oracle.decode_attn(q, np.repeat(k, G, axis=0), np.repeat(v, G, axis=0), [N], causal_tail=True)
    assert np.allclose(o1, o2, atol=0) and np.allclose(l1, l2, atol=0)


def test_fsum_brute_force_tiny_config():
    """Pure-Python loops with math.fsum at the tiny configuration's head shape."""
    cfg = W.C1
    rng = np.random.default_rng(6)
    nq, N = cfg.gamma_verify + 1, 40
    q = W.bf16_round(rng.standard_normal((1, nq, cfg.hq, cfg.d)).astype(np.float32))
    k = W.bf16_round(rng.standard_normal((cfg.hkv, N, cfg.d)).astype(np.float32))
    v = W.bf16_round(rng.standard_normal((cfg.hkv, N, cfg.d)).astype(np.float32))
    o, lse = oracle.decode_attn(q, k, v, [N], causal_tail=True)
    G = cfg.group
    sc = 1.0 / math.sqrt(cfg.d)
    for i in range(nq):
        lim = N - nq + i + 1
        for h in range(cfg.hq):
            g = h // G
            s = [sc * math.fsum(float(q[0, i, h, d]) * float(k[g, n, d]) for d in range(cfg.d)) for n in range(lim)]
            m = max(s)
            w = [math.exp(x - m) for x in s]
            z = math.fsum(w)
            for d in range(0, cfg.d, 7):
                ref = math.fsum(w[n] * float(v[g, n, d]) for n in range(lim)) / z
                assert abs(o[0, i, h, d] - ref) < 1e-12
            assert abs(lse[0, i, h] - (m + math.log(z))) < 1e-12


def test_split_invariance_of_online_softmax():
    """Merging the (max, sum, weighted values) of two halves gives the full result."""
    rng = np.random.default_rng(7)
    D, N = 16, 64
    q = rng.standard_normal((1, 1, 1, D)).astype(np.float32)
    k = rng.standard_normal((1, N, D)).astype(np.float32)
    v = rng.standard_normal((1, N, D)).astype(np.float32)
    o, lse = oracle.decode_attn(q, k, v, [N], causal_tail=False)
    oa, la = oracle.decode_attn(q, k[:, :23], v[:, :23], [23], causal_tail=False)
    ob, lb = oracle.decode_attn(q, k[:, 23:], v[:, 23:], [N - 23], causal_tail=False)
    L = np.logaddexp(la, lb)
    merged = oa * np.exp(la - L)[..., None] + ob * np.exp(lb - L)[..., None]
    assert np.allclose(merged, o, atol=1e-12) and np.allclose(L, lse, atol=1e-12)
