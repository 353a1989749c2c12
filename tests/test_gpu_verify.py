"""Acceptance on the GPU vs the oracle: bit-exact n_accept and next token."""
import numpy as np
import pytest

import oracle
import workloads as W
from tests._util import log

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")


def _t(x, dt=None):
    return torch.from_numpy(np.ascontiguousarray(x if dt is None else x.astype(dt))).to("cuda:0")


def _gpu(mode, d, target, q=None, u=None):
    from visual_kv_pruning_amd import ops
    n, t = ops.verify(mode, _t(d, np.int32), _t(target, np.float32), None if q is None else _t(q, np.float32),
                      None if u is None else _t(u, np.float32))
    torch.cuda.synchronize()
    return n.cpu().numpy(), t.cpu().numpy()


@pytest.mark.parametrize("vocab,gamma,batch", [(1024, 4, 3), (152064, 9, 2), (152064, 5, 1), (5000, 1, 4), (1, 3, 1)])
@pytest.mark.parametrize("seed", range(4))
def test_greedy_bit_exact(vocab, gamma, batch, seed):
    vi = W.verify_inputs(10 + seed, batch, gamma, vocab, extra=vocab)
    d = vi.draft_tok_greedy.copy()
    if seed % 2 == 0:   # force long accepted prefixes
        d[:, : gamma - 1] = np.argmax(vi.target_logits[:, : gamma - 1], axis=-1)
    log(f"verify greedy V={vocab} gamma={gamma} B={batch} seed={seed}")
    n, t = _gpu("greedy", d, vi.target_logits)
    rn, rt = oracle.verify_greedy(d, vi.target_logits)
    assert np.array_equal(n, rn) and np.array_equal(t, rt)


def test_greedy_ties_take_lowest_index():
    V = 9000
    logits = np.zeros((1, 3, V), np.float32)
    logits[0, 0, [4097, 8191, 12]] = 5.0        # tie across chunks -> 12
    logits[0, 1, [4096, 4095]] = 1.0            # tie at a chunk boundary -> 4095
    logits[0, 2, :] = -1.0
    logits[0, 2, [8999, 100]] = 0.0
    d = np.array([[12, 4095]], np.int32)
    n, t = _gpu("greedy", d, logits)
    assert (n[0], t[0]) == (2, 100)


@pytest.mark.parametrize("vocab,gamma,batch", [(1024, 4, 4), (152064, 9, 2), (152064, 5, 1), (777, 2, 3)])
@pytest.mark.parametrize("seed", range(6))
def test_reject_bit_exact(vocab, gamma, batch, seed):
    vi = W.verify_inputs(20 + seed, batch, gamma, vocab, extra=vocab)
    u = vi.u.copy()
    if seed >= 3:      # small uniforms -> long accepted runs, exercising the bonus draw
        u[:, :gamma] *= np.float32(0.05)
    log(f"verify reject V={vocab} gamma={gamma} B={batch} seed={seed}")
    n, t = _gpu("reject", vi.draft_tok_sampled, vi.p, vi.q, u)
    rn, rt = oracle.verify_reject(vi.draft_tok_sampled, vi.p, vi.q, u)
    assert np.array_equal(n, rn) and np.array_equal(t, rt)


def test_reject_special_cases():
    V = 4
    p = np.array([[[0.0, 1.0, 0.0, 0.0], [0.25, 0.25, 0.25, 0.25]]], np.float32)
    q = np.array([[[0.0, 1.0, 0.0, 0.0]]], np.float32)
    n, t = _gpu("reject", np.array([[1]]), p, q, np.array([[0.999, 0.6]], np.float32))
    assert (n[0], t[0]) == (1, 2)
    q2 = np.array([[[0.0, 0.0, 1.0, 0.0]]], np.float32)
    n, t = _gpu("reject", np.array([[2]]), p, q2, np.array([[0.0001, 0.3]], np.float32))
    assert (n[0], t[0]) == (0, 1)
    # residual with zero fixed-point mass falls back to p, then argmax
    pz = np.zeros((1, 2, V), np.float32)
    pz[0, :, 3] = 1e-30
    qz = np.zeros((1, 1, V), np.float32)
    qz[0, 0, 0] = 1.0
    n, t = _gpu("reject", np.array([[0]]), pz, qz, np.array([[0.5, 0.5]], np.float32))
    rn, rt = oracle.verify_reject(np.array([[0]]), pz, qz, np.array([[0.5, 0.5]], np.float32))
    assert (n[0], t[0]) == (rn[0], rt[0]) == (0, 3)


@pytest.mark.parametrize("first_miss", [None, 0, 63, 64, 66, 69])
def test_long_windows_cross_the_64_position_rounds(first_miss):
    """gamma = 70 drafted tokens: the first mismatch (or rejection) is searched
    64 positions at a time; drafts agree with the target up to `first_miss`
    (None: all accepted, the bonus token comes from the last row)."""
    gamma, V, B = 70, 300, 2
    rng = np.random.default_rng(99 if first_miss is None else first_miss)
    logits = rng.standard_normal((B, gamma + 1, V)).astype(np.float32)
    d = logits[:, :gamma].argmax(-1).astype(np.int32)
    if first_miss is not None:
        d[:, first_miss] = (d[:, first_miss] + 1) % V
    log(f"verify case long window greedy first_miss={first_miss}")
    n, t = _gpu("greedy", d, logits)
    rn, rt = oracle.verify_greedy(d, logits)
    assert np.array_equal(n, rn) and np.array_equal(t, rt)
    assert n[0] == (gamma if first_miss is None else first_miss)
    # rejection: u = 0 accepts every drafted token with p(d) > 0 ... unless forced
    p = np.exp(logits - logits.max(-1, keepdims=True))
    p = (p / p.sum(-1, keepdims=True)).astype(np.float32)
    q = np.roll(p[:, :gamma], 1, axis=-1).astype(np.float32)
    u = np.zeros((B, gamma + 1), np.float32)
    u[:, gamma] = 0.37
    if first_miss is not None:
        p[:, first_miss, d[:, first_miss]] = 0.0   # p(d) = 0 < u q(d) for u > 0
        u[:, first_miss] = 0.5
    log(f"verify case long window reject first_miss={first_miss}")
    n, t = _gpu("reject", d, p, q, u)
    rn, rt = oracle.verify_reject(d, p, q, u)
    assert np.array_equal(n, rn) and np.array_equal(t, rt)
