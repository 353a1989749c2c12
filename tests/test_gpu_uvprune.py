"""UV-Prune score on the GPU (layers 0 and L only) vs the fp64 oracle's
printed double sum over every layer; top-K selection from the GPU scores.

Tolerance: dS lies in [-2 n_text, 2 n_text]; the kernel accumulates in fp32
(row norms and dots over d, the normalised text sum over n_text), so it is
held to 4e-6 of that range: |dS - dS_ref| <= 8e-6 * n_text."""
import math

import numpy as np
import pytest

import oracle
import workloads as W
from tests._util import dev_bf16, log

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")


def _gpu(vs, xs, scale=1.0, offset=0.0, pad=0):
    from visual_kv_pruning_amd import ops
    def dev(a):
        t = dev_bf16(np.pad(a, ((0, 0), (0, pad))) if pad else a)
        return t[:, :a.shape[1]] if pad else t
    out = ops.uvprune_score(dev(vs[0]), dev(vs[-1]), dev(xs[0]), dev(xs[-1]), scale, offset)
    torch.cuda.synchronize()
    return out.cpu().numpy().astype(np.float64)


@pytest.mark.parametrize("cfg,layers", [(W.C1, 1), (W.C1, 4), (W.C2, 3)], ids=lambda x: getattr(x, "name", str(x)))
def test_matches_oracle_double_sum(cfg, layers):
    vs, xs = W.uv_hidden(cfg, layers)
    log(f"uvprune case {cfg.name} layers={layers} d={vs[0].shape[1]}")
    got = _gpu(vs, xs)
    ref = oracle.uvprune_scores(vs, xs)
    err = float(np.abs(got - ref).max())
    log(f"  max |dS err| {err:.2e} (n_text {cfg.n_text})")
    assert err <= 8e-6 * cfg.n_text


def test_strided_rows_and_zero_vectors():
    cfg = W.C1
    vs, xs = W.uv_hidden(cfg, 1, extra=1)
    vs = [v.copy() for v in vs]
    xs = [x.copy() for x in xs]
    vs[0][5] = 0.0
    vs[1][5] = 0.0
    xs[1][3] = 0.0
    log("uvprune case strided rows, zero vectors")
    got = _gpu(vs, xs, pad=24)
    ref = oracle.uvprune_scores(vs, xs)
    assert got[5] == 0.0
    assert float(np.abs(got - ref).max()) <= 8e-6 * cfg.n_text


def test_llava72b_shape_sampled_rows_and_top_k_selection():
    """full 72B shape (25088 video tokens, 128 text, hidden 8192): the oracle
    checks 1500 sampled rows; the kept top 10% (mapped into [0, 1]) equals the
    oracle selection on the same scores and holds every drifting token"""
    from visual_kv_pruning_amd import ops
    cfg = W.C3
    vs, xs = W.uv_hidden(cfg, 1)
    n = cfg.n_text
    log(f"uvprune case 72B shape d={vs[0].shape[1]}")
    got = _gpu(vs, xs)
    rows = np.sort(np.random.default_rng(0).choice(cfg.n_vis, 1500, replace=False))
    ref = oracle.uvprune_scores([vs[0][rows], vs[1][rows]], xs)
    err = float(np.abs(got[rows] - ref).max())
    log(f"  max |dS err| on sampled rows {err:.2e}")
    assert err <= 8e-6 * n
    # top-K through svlm_select (pure top-K) on the unit-interval map of the scores
    unit = torch.tensor(((got + 2 * n) / (4 * n))[None].astype(np.float32), device="cuda:0")
    K = math.ceil(0.1 * cfg.n_vis)
    kept, _, _ = ops.select(unit, cfg.frames, cfg.gh, cfg.gw, 1.0, K)
    kept = kept[0].cpu().numpy()
    ref_kept, _, _ = oracle.select_row(unit[0].cpu().numpy(), cfg.frames, cfg.gh, cfg.gw, 1.0, K)
    assert np.array_equal(kept, ref_kept)
    assert np.isin(W.salient_positions(cfg), kept).all()


def test_deterministic():
    vs, xs = W.uv_hidden(W.C2, 1)
    assert np.array_equal(_gpu(vs, xs), _gpu(vs, xs))


@pytest.mark.parametrize("n_vis,n_text,d", [(1, 1, 8), (37, 3, 72), (300, 5, 1000), (100, 4, 16384)])
def test_edge_sizes(n_vis, n_text, d):
    """One video and one text token at the smallest hidden size; hidden sizes
    that are not multiples of 64 (the text sums work in 64-dim slices); the
    largest hidden size, whose two text vectors take 128 KB of LDS."""
    rng = np.random.default_rng(n_vis * 31 + d)
    vs = [W.bf16_round(rng.standard_normal((n_vis, d)).astype(np.float32)) for _ in range(2)]
    xs = [W.bf16_round(rng.standard_normal((n_text, d)).astype(np.float32)) for _ in range(2)]
    log(f"uvprune case edge n_vis={n_vis} n_text={n_text} d={d}")
    got = _gpu(vs, xs)
    ref = oracle.uvprune_scores(vs, xs)
    assert float(np.abs(got - ref).max()) <= 8e-6 * n_text
