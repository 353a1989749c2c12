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


# gamma <= 9 takes the form that loads every candidate row up front; 10 and
# 16 the form that reads row n after finding it
@pytest.mark.parametrize("vocab,gamma,batch", [(1024, 4, 4), (152064, 9, 2), (152064, 5, 1), (777, 2, 3),
                                               (152064, 10, 2), (5000, 16, 3)])
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


def test_workspace_reused_across_calls_and_modes():
    """One zero-filled workspace serves a run of calls: each launch's last
    workgroup per sequence resets its arrival counter, so later calls (either
    mode, fewer sequences, a longer window) still reduce every chunk."""
    from visual_kv_pruning_amd import ops
    V = 152064
    ws = torch.zeros(ops.verify_workspace_bytes(4, 9, V), dtype=torch.uint8, device="cuda:0")
    cases = [("reject", 4, 5, 30), ("greedy", 4, 9, 31), ("reject", 1, 9, 32), ("greedy", 2, 3, 33),
             ("reject", 3, 2, 34), ("reject", 3, 2, 35), ("greedy", 1, 1, 36)]
    for rep in range(2):
        for mode, batch, gamma, seed in cases:
            vi = W.verify_inputs(seed, batch, gamma, V, extra=V)
            log(f"verify workspace reuse rep={rep} mode={mode} B={batch} gamma={gamma} seed={seed}")
            if mode == "greedy":
                d = vi.draft_tok_greedy.copy()
                d[:, : gamma // 2] = np.argmax(vi.target_logits[:, : gamma // 2], axis=-1)
                n, t = ops.verify("greedy", _t(d, np.int32), _t(vi.target_logits, np.float32), ws=ws)
                rn, rt = oracle.verify_greedy(d, vi.target_logits)
            else:
                n, t = ops.verify("reject", _t(vi.draft_tok_sampled, np.int32), _t(vi.p, np.float32),
                                  _t(vi.q, np.float32), _t(vi.u, np.float32), ws=ws)
                rn, rt = oracle.verify_reject(vi.draft_tok_sampled, vi.p, vi.q, vi.u)
            torch.cuda.synchronize()
            assert np.array_equal(n.cpu().numpy(), rn) and np.array_equal(t.cpu().numpy(), rt)
    # every call left the counters zero
    tail = ws[: 4 * 4].cpu().numpy()
    assert not tail.any()


def test_greedy_vocab_past_64_chunks():
    """A vocabulary of more than 64 greedy chunks (16384 entries each): the
    final pass takes the chunk results of a row in several rounds."""
    V, gamma = 1_100_000, 2
    rng = np.random.default_rng(41)
    logits = rng.standard_normal((1, gamma + 1, V)).astype(np.float32)
    logits[0, 1, V - 3] = 9.0      # row maxima in the last round of chunks
    logits[0, 2, 70 * 16384 // 2] = 9.0
    d = np.array([[int(np.argmax(logits[0, 0])), V - 3]], np.int32)
    log(f"verify greedy V={V} gamma={gamma}")
    n, t = _gpu("greedy", d, logits)
    rn, rt = oracle.verify_greedy(d, logits)
    assert np.array_equal(n, rn) and np.array_equal(t, rt) and n[0] == 2


@pytest.mark.parametrize("mode", ["reject", "greedy"])
def test_graph_replays_reset_the_counters(mode):
    """The call captured once in a HIP graph and replayed on new inputs (copied
    in eagerly between replays): every replay's arrival counters start at zero
    because the previous replay's last workgroups reset them."""
    from visual_kv_pruning_amd import ops
    V, gamma, B = 152064, (5 if mode == "reject" else 9), 2
    ws = torch.zeros(ops.verify_workspace_bytes(B, gamma, V), dtype=torch.uint8, device="cuda:0")
    vi0 = W.verify_inputs(60, B, gamma, V, extra=V)
    d_t = _t(vi0.draft_tok_sampled if mode == "reject" else vi0.draft_tok_greedy, np.int32)
    t_t = _t(vi0.p if mode == "reject" else vi0.target_logits, np.float32)
    q_t = _t(vi0.q, np.float32) if mode == "reject" else None
    u_t = _t(vi0.u, np.float32) if mode == "reject" else None
    ops.verify(mode, d_t, t_t, q_t, u_t, ws=ws)  # warm-up outside the capture
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        n_out, t_out = ops.verify(mode, d_t, t_t, q_t, u_t, ws=ws)
    for rep in range(4):
        vi = W.verify_inputs(61 + rep, B, gamma, V, extra=V)
        if mode == "reject":
            d = vi.draft_tok_sampled
            d_t.copy_(_t(d, np.int32)); t_t.copy_(_t(vi.p, np.float32))
            q_t.copy_(_t(vi.q, np.float32)); u_t.copy_(_t(vi.u, np.float32))
            rn, rt = oracle.verify_reject(d, vi.p, vi.q, vi.u)
        else:
            d = vi.draft_tok_greedy.copy()
            d[:, : rep + 1] = np.argmax(vi.target_logits[:, : rep + 1], axis=-1)
            d_t.copy_(_t(d, np.int32)); t_t.copy_(_t(vi.target_logits, np.float32))
            rn, rt = oracle.verify_greedy(d, vi.target_logits)
        log(f"verify graph replay mode={mode} rep={rep}")
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(n_out.cpu().numpy(), rn) and np.array_equal(t_out.cpu().numpy(), rt)
    assert not ws[: 4 * B].cpu().numpy().any()


def test_seeded_random_shapes_both_modes():
    """40 seeded random calls of either mode: batch 1-5, window 1-20 (both
    rejection forms), vocabularies from 1 to 200000 (chunk counts of 1 to
    over 100, ragged last chunks), uniforms scaled so that accepted runs are
    short or long; each bit-exact against the oracle."""
    rng = np.random.default_rng(2024)
    for case in range(40):
        mode = "reject" if case % 2 == 0 else "greedy"
        batch = int(rng.integers(1, 6))
        gamma = int(rng.integers(1, 21))
        V = int(rng.choice([1, 3, 1000, 1024, 1025, 4097, 16383, 16385, 65536, 152064, 200000]))
        vi = W.verify_inputs(100 + case, batch, gamma, V, extra=V)
        log(f"verify random case {case}: mode={mode} B={batch} gamma={gamma} V={V}")
        if mode == "reject":
            u = vi.u.copy()
            u[:, :gamma] *= np.float32(rng.choice([1.0, 0.2, 0.01]))
            n, t = _gpu("reject", vi.draft_tok_sampled, vi.p, vi.q, u)
            rn, rt = oracle.verify_reject(vi.draft_tok_sampled, vi.p, vi.q, u)
        else:
            d = vi.draft_tok_greedy.copy()
            k = int(rng.integers(0, gamma + 1))
            d[:, :k] = np.argmax(vi.target_logits[:, :k], axis=-1)
            n, t = _gpu("greedy", d, vi.target_logits)
            rn, rt = oracle.verify_greedy(d, vi.target_logits)
        assert np.array_equal(n, rn) and np.array_equal(t, rt), f"case {case}"
