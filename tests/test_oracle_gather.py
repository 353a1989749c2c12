"""Pins for the KV compaction oracle: NumPy fancy indexing and a hand case."""
import numpy as np

import oracle


def test_gather_shared_and_per_head_lists():
    rng = np.random.default_rng(0)
    src = rng.standard_normal((3, 20, 4)).astype(np.float32)
    idx = np.array([1, 5, 7])
    out = oracle.gather_kv(src, idx, tail_start=17, n_tail=3)
    assert out.shape == (3, 6, 4)
    assert np.array_equal(out[:, :3], src[:, idx]) and np.array_equal(out[:, 3:], src[:, 17:20])
    ph = np.array([[0, 1], [2, 3], [19, 4]])
    out2 = oracle.gather_kv(src, ph)
    for g in range(3):
        assert np.array_equal(out2[g], src[g][ph[g]])


def test_gather_hand_case():
    src = np.arange(2 * 5 * 1, dtype=np.float32).reshape(2, 5, 1)   # head g, token n -> 5g + n
    out = oracle.gather_kv(src, [4, 0], tail_start=2, n_tail=1)
    assert out[:, :, 0].tolist() == [[4, 0, 2], [9, 5, 7]]
