"""Selection on the GPU vs the oracle: bit-exact kept lists, stage-I counts and tags
when both sides see the same fp32 scores."""
import math

import numpy as np
import pytest

import oracle
import workloads as W
from tests._util import log

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")


def _gpu_select(rows, F, H, Wd, top_p, budget):
    from visual_kv_pruning_amd import ops
    s = torch.from_numpy(np.ascontiguousarray(rows, np.float32)).to("cuda:0")
    kept, n1, tag = ops.select(s, F, H, Wd, top_p, budget, with_tag=True)
    torch.cuda.synchronize()
    return kept.cpu().numpy(), n1.cpu().numpy(), tag.cpu().numpy()


def _check(rows, F, H, Wd, top_p, budget, name):
    log(f"select case {name}: R={rows.shape[0]} N={rows.shape[1]} P={top_p} B={budget}")
    kept, n1, tag = _gpu_select(rows, F, H, Wd, top_p, budget)
    rk, r1, rt = oracle.select_rows(rows, F, H, Wd, top_p, budget)
    assert np.array_equal(n1, r1), name
    assert np.array_equal(kept, rk.astype(np.int32)), name
    assert np.array_equal(tag, rt), name


@pytest.mark.parametrize("kind", W.SCORE_KINDS)
@pytest.mark.parametrize("top_p", [0.0, 0.1, 0.5, 0.6, 1.0])
def test_heavy_tailed_rows(kind, top_p):
    F, H, Wd = 8, 14, 14
    N = F * H * Wd
    rows = W.score_rows(kind, 3, N, seed=5)
    _check(rows, F, H, Wd, top_p, int(math.ceil(0.1 * N)), f"{kind}")


@pytest.mark.parametrize("budget", [0, 1, 7, 196, 700, 1567, 1568])
def test_budget_edges(budget):
    F, H, Wd = 8, 14, 14
    rows = W.score_rows("lognormal2", 2, F * H * Wd, seed=6)
    _check(rows, F, H, Wd, 0.5, budget, f"budget={budget}")


@pytest.mark.parametrize("kind", W.SCORE_KINDS)
@pytest.mark.parametrize("top_p", [0.0, 0.5, 1.0])
def test_long_rows_chunked(kind, top_p):
    """Rows past the register-resident limit (32768 tokens) are taken in chunks
    of 16384 tokens with the ordered scans carried across them; 50 frames of
    28 x 28 = 39200 tokens end in a partial chunk."""
    F, H, Wd = 50, 28, 28
    N = F * H * Wd
    rows = W.score_rows(kind, 2, N, seed=11)
    _check(rows, F, H, Wd, top_p, int(math.ceil(0.1 * N)), f"long {kind}")


@pytest.mark.parametrize("budget", [0, 1, 16383, 16384, 16385, 39199, 39200])
def test_long_rows_budget_edges(budget):
    """Budgets at the chunk boundary and at the row length on the chunked path."""
    F, H, Wd = 50, 28, 28
    rows = W.score_rows("lognormal2", 1, F * H * Wd, seed=12)
    _check(rows, F, H, Wd, 0.5, budget, f"long budget={budget}")


def _check_split(rows, F, H, Wd, top_p, budget, name, pad=0):
    """Pure top-K without tags: rows past 32768 tokens take the split form
    (segment top-K, then a top-K over the candidates).  Kept lists and stage-I
    counts must equal the oracle's, and the tagged one-workgroup form's."""
    from visual_kv_pruning_amd import ops
    R, N = rows.shape
    log(f"select split case {name}: R={R} N={N} P={top_p} B={budget} pad={pad} "
        f"ws={ops.select_workspace_bytes(R, N, budget, top_p)}")
    wide = np.ones((R, N + pad), np.float32)   # padding past each row is never read
    wide[:, :N] = rows
    s = torch.from_numpy(wide).to("cuda:0")[:, :N]
    kept, n1, _ = ops.select(s, F, H, Wd, top_p, budget)
    kept_t, n1_t, _ = ops.select(s, F, H, Wd, top_p, budget, with_tag=True)
    torch.cuda.synchronize()
    rk, r1, _ = oracle.select_rows(rows, F, H, Wd, top_p, budget)
    assert np.array_equal(n1.cpu().numpy(), r1), name
    assert np.array_equal(kept.cpu().numpy(), rk.astype(np.int32)), name
    assert np.array_equal(kept_t.cpu().numpy(), rk.astype(np.int32)), name
    assert np.array_equal(n1_t.cpu().numpy(), r1), name


@pytest.mark.parametrize("kind", W.SCORE_KINDS)
def test_split_topk_long_rows(kind):
    """50 frames of 28 x 28 = 39200 tokens: two segments of 19600; budget 10%."""
    F, H, Wd = 50, 28, 28
    rows = W.score_rows(kind, 3, F * H * Wd, seed=21)
    _check_split(rows, F, H, Wd, 1.0, 3920, f"split {kind}")


@pytest.mark.parametrize("budget", [1, 2, 1024, 16383, 16384, 16385, 19600, 39199, 39200])
def test_split_topk_budget_edges(budget):
    """Budgets around the split form's limits (two segments of 19600 tokens):
    2 x 16384 candidates fill one register-resident row (16385 does not, and
    falls back to the one-workgroup form), the segment length, and the whole
    row."""
    F, H, Wd = 50, 28, 28
    rows = W.score_rows("lognormal2", 2, F * H * Wd, seed=22)
    _check_split(rows, F, H, Wd, 1.0, budget, f"split budget={budget}")


def test_split_topk_ties_across_segments():
    """Scores quantised to 1/64: long runs of equal scores cross every
    segment boundary, so the index tie-break decides which tokens are kept."""
    F, H, Wd = 50, 28, 28
    rows = W.score_rows("lognormal2", 2, F * H * Wd, seed=23)
    rows = (np.floor(rows / rows.max(axis=1, keepdims=True) * 64) / 64).astype(np.float32)
    for budget in (1, 500, 3920, 9000):
        _check_split(rows, F, H, Wd, 2.0, budget, f"split ties budget={budget}")


def test_split_topk_long_segments():
    """120 rows of 350 x 10 x 20 = 70000 tokens: three segments would take a
    second round of workgroups on a 256-CU chip, so the plan keeps two
    segments of 35000 tokens (36 per thread)."""
    F, H, Wd = 350, 10, 20
    rows = W.score_rows("lognormal3", 120, F * H * Wd, seed=25)
    _check_split(rows, F, H, Wd, 1.0, 700, "split long segments")


def test_split_topk_hour_shape():
    """The hour-long shape: 720 frames x 14 x 14 = 141120 tokens, top-K 1024
    (6 segments of 23520), four rows, a strided view."""
    F, H, Wd = 720, 14, 14
    rows = W.score_rows("pareto1.1", 4, F * H * Wd, seed=24)
    _check_split(rows, F, H, Wd, 1.0, 1024, "split hour", pad=40)


@pytest.mark.parametrize("F,H,Wd", [(1, 1, 1), (1, 1, 2), (3, 1, 1), (1, 2, 2)])
def test_tiny_rows_every_budget(F, H, Wd):
    """Rows of one to four tokens, every budget from 0 to N, three Top-P values."""
    N = F * H * Wd
    rows = W.score_rows("lognormal2", 3, N, seed=14)
    for top_p in (0.0, 0.5, 1.0):
        for budget in range(N + 1):
            _check(rows, F, H, Wd, top_p, budget, f"tiny N={N} P={top_p} B={budget}")


def test_strided_rows():
    """Rows taken from a wider matrix (row stride > F*H*W), as from a slice."""
    from visual_kv_pruning_amd import ops
    F, H, Wd = 4, 7, 9
    N = F * H * Wd
    rows = W.score_rows("lognormal2", 5, N, seed=13)
    wide = np.zeros((5, N + 37), np.float32)
    wide[:, :N] = rows
    wide[:, N:] = 1.0                      # never read: past each row
    log("select case strided rows")
    s = torch.from_numpy(wide).to("cuda:0")[:, :N]
    kept, n1, tag = ops.select(s, F, H, Wd, 0.5, 25, with_tag=True)
    torch.cuda.synchronize()
    rk, r1, rt = oracle.select_rows(rows, F, H, Wd, 0.5, 25)
    assert np.array_equal(n1.cpu().numpy(), r1)
    assert np.array_equal(kept.cpu().numpy(), rk.astype(np.int32))
    assert np.array_equal(tag.cpu().numpy(), rt)


def test_golden_worked_example():
    s = np.array([4, 0, 1, 8, 2, 2, 0, 3, 16, 1, 2, 1], np.float32) / np.float32(64)
    for p, b in ((0.5, 5), (0.9, 5), (0.0, 4), (1.0, 4), (0.3, 5)):
        _check(s[None], 2, 2, 3, p, b, f"golden P={p}")


@pytest.mark.parametrize("cfg", [W.C1, W.C2, W.C3, W.C4, W.C5], ids=lambda c: c.name)
def test_config_shapes(cfg):
    """Each configuration's row length, budget and Top-P, on heavy-tailed and flat rows."""
    R = {"all": 1, "layer": 4, "layer_kvhead": 6}[cfg.rows]
    for kind in ("lognormal3", "flat", "pareto1.1"):
        rows = W.score_rows(kind, R, cfg.n_vis, seed=cfg.index)
        _check(rows, cfg.frames, cfg.gh, cfg.gw, cfg.top_p, cfg.budget, f"{cfg.name}/{kind}")


def test_scores_from_the_value_model():
    """Rows from the oracle's own score of the tiny configuration (nearly flat attention)."""
    cfg = W.C1
    p = W.prefill_layer(cfg, 0)
    row = oracle.aggregate_heads(oracle.score_layer(p.q_text, p.k, p.q_pos0, 0, cfg.n_vis, cfg.hkv), cfg.hkv, "all")
    _check(row.astype(np.float32), cfg.frames, cfg.gh, cfg.gw, cfg.top_p, cfg.budget, "tiny value model")


def test_split_topk_workspace_errors():
    """The split form names its workspace: a short one is an error, a
    caller-supplied one of the queried size gives the oracle's result."""
    from visual_kv_pruning_amd import ops
    from visual_kv_pruning_amd._lib import SvlmError, SVLM_E_WORKSPACE
    F, H, Wd = 50, 28, 28
    N = F * H * Wd
    rows = W.score_rows("lognormal1", 2, N, seed=26)
    log("select split case workspace errors")
    s = torch.from_numpy(rows).to("cuda:0")
    need = ops.select_workspace_bytes(2, N, 500, 1.0)
    assert need > 0
    short = torch.empty(need - 256, dtype=torch.uint8, device="cuda:0")
    with pytest.raises(SvlmError) as e:
        ops.select(s, F, H, Wd, 1.0, 500, ws=short)
    assert e.value.status == SVLM_E_WORKSPACE
    ws = torch.empty(need, dtype=torch.uint8, device="cuda:0")
    kept, n1, _ = ops.select(s, F, H, Wd, 1.0, 500, ws=ws)
    torch.cuda.synchronize()
    rk, r1, _ = oracle.select_rows(rows, F, H, Wd, 1.0, 500)
    assert np.array_equal(kept.cpu().numpy(), rk.astype(np.int32))
    assert np.array_equal(n1.cpu().numpy(), r1)
