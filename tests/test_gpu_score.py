"""Mean text->visual attention on the GPU vs the fp64 oracle: within 1e-5 absolute
(and the relative error on scores >= 1e-6 reported)."""
import dataclasses

import numpy as np
import pytest

import oracle
import workloads as W
from tests._util import dev_bf16, log

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")
ABS_TOL = 1e-5


def _gpu_score(p, cfg, agg, n_vis=None, vis_start=0):
    from visual_kv_pruning_amd import ops
    n_vis = cfg.n_vis if n_vis is None else n_vis
    out = ops.score(dev_bf16(p.q_text), dev_bf16(p.k), p.q_pos0, n_vis, vis_start=vis_start, agg=agg)
    torch.cuda.synchronize()
    return out.cpu().numpy()


def _ref(p, cfg, agg, n_vis=None, vis_start=0):
    n_vis = cfg.n_vis if n_vis is None else n_vis
    sq = oracle.score_layer(p.q_text, p.k, p.q_pos0, vis_start, n_vis, cfg.hkv)
    return oracle.aggregate_heads(sq, cfg.hkv, {"qhead": "qhead", "kvhead": "kvhead", "all": "all"}[agg])


def _compare(got, ref, name):
    err = float(np.abs(got - ref).max())
    big = ref >= 1e-6
    rel = float((np.abs(got - ref)[big] / ref[big]).max()) if big.any() else 0.0
    log(f"score {name}: max abs err {err:.2e}, max rel err (scores >= 1e-6) {rel:.2e}")
    assert err <= ABS_TOL, name
    return rel


@pytest.mark.parametrize("agg", ["qhead", "kvhead", "all"])
def test_tiny_config_all_aggregations(agg):
    cfg = W.C1
    p = W.prefill_layer(cfg, 0)
    log(f"score case tiny agg={agg}")
    _compare(_gpu_score(p, cfg, agg), _ref(p, cfg, agg), f"tiny/{agg}")


def test_tiny_config_offset_visual_window():
    cfg = W.C1
    p = W.prefill_layer(cfg, 0)
    log("score case tiny offset window")
    _compare(_gpu_score(p, cfg, "qhead", n_vis=77, vis_start=50), _ref(p, cfg, "qhead", 77, 50), "tiny/window")


def test_rows_sum_property_and_alpha_beta_accumulation():
    """Two layers averaged with alpha/beta equal the mean of the per-layer rows."""
    from visual_kv_pruning_amd import ops
    cfg = W.C1
    p0, p1 = W.prefill_layer(cfg, 0), W.prefill_layer(cfg, 1)
    log("score case alpha/beta")
    out = ops.score(dev_bf16(p0.q_text), dev_bf16(p0.k), p0.q_pos0, cfg.n_vis, agg="all", alpha=0.5, beta=0.0)
    ops.score(dev_bf16(p1.q_text), dev_bf16(p1.k), p1.q_pos0, cfg.n_vis, agg="all", alpha=0.5, beta=1.0, out=out)
    torch.cuda.synchronize()
    ref = 0.5 * (_ref(p0, cfg, "all") + _ref(p1, cfg, "all"))
    _compare(out.cpu().numpy(), ref, "tiny/two layers")


@pytest.mark.parametrize("cfg", [W.C2, W.C4], ids=lambda c: c.name)
def test_full_size_layer(cfg):
    p = W.prefill_layer(cfg, 0)
    log(f"score case {cfg.name} full layer")
    _compare(_gpu_score(p, cfg, "kvhead"), _ref(p, cfg, "kvhead"), cfg.name)


def test_llava72b_layer_sampled_heads():
    """Full 72B-shape layer on the GPU; the oracle checks every q head of KV head 0 and 7."""
    cfg = W.C3
    p = W.prefill_layer(cfg, 0)
    log("score case 72B layer")
    got = _gpu_score(p, cfg, "qhead")
    G = cfg.group
    for g in (0, cfg.hkv - 1):
        heads = list(range(g * G, (g + 1) * G))
        ref = oracle.score_layer(p.q_text[:, heads], p.k[g:g + 1], p.q_pos0, 0, cfg.n_vis, 1)
        _compare(got[heads], ref, f"72B kv head {g}")


def test_deterministic():
    cfg = W.C1
    p = W.prefill_layer(cfg, 0)
    a = _gpu_score(p, cfg, "qhead")
    b = _gpu_score(p, cfg, "qhead")
    assert np.array_equal(a, b)


def test_deterministic_full_layer():
    """Repeated calls on a full 72B-shape layer give bit-identical rows (every
    pass-1 reference maximum and every merge is order-fixed)."""
    cfg = W.C3
    p = W.prefill_layer(cfg, 0)
    log("score case 72B layer, repeated calls")
    first = _gpu_score(p, cfg, "all")
    for _ in range(3):
        assert np.array_equal(first, _gpu_score(p, cfg, "all"))


def test_wide_score_range():
    """Queries scaled by 4 (exactly, in bf16) spread the scores over ~25 log2
    units, so the per-lane reference maximum of pass 1 is raised many times."""
    cfg = W.C2
    p = W.prefill_layer(cfg, 0)
    p = dataclasses.replace(p, q_text=p.q_text * 4.0)
    log("score case wide score range")
    _compare(_gpu_score(p, cfg, "kvhead"), _ref(p, cfg, "kvhead"), "C2 q x4")


@dataclasses.dataclass
class _Layer:
    q_text: np.ndarray
    k: np.ndarray
    q_pos0: int


@dataclasses.dataclass
class _Shape:
    n_vis: int
    hkv: int


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("T,n_vis,pre,post,Hq,Hkv", [
    (1, 1, 0, 0, 2, 2),        # one text query, one visual token
    (1, 300, 5, 3, 4, 1),      # one query; keys before and after the visual window
    (17, 63, 0, 0, 6, 2),      # ragged text rows and keys (not multiples of 16 or 64)
    (33, 1000, 12, 40, 8, 8),  # MHA (one head per group), visual window inside the context
    (128, 129, 1, 0, 16, 2),   # a full 128-row block of text queries
    (20, 500, 0, 8, 32, 2),    # 16 q heads per KV head (two head groups in both passes)
])
def test_edge_shapes(D, T, n_vis, pre, post, Hq, Hkv):
    """Edge shapes vs the oracle: single query and single visual token, ragged
    text rows and key counts, keys before the visual window (vis_start > 0)
    and text tokens between it and the queries."""
    rng = np.random.default_rng(D * 1000 + T * 7 + n_vis)
    q_pos0 = pre + n_vis + post
    n_ctx = q_pos0 + T
    q = W.bf16_round(rng.standard_normal((T, Hq, D)).astype(np.float32))
    k = W.bf16_round(rng.standard_normal((Hkv, n_ctx, D)).astype(np.float32))
    p = _Layer(q, k, q_pos0)
    shape = _Shape(n_vis, Hkv)
    log(f"score case edge D{D} T{T} n_vis{n_vis} pre{pre} post{post} Hq{Hq} Hkv{Hkv}")
    for agg in ("qhead", "kvhead", "all"):
        _compare(_gpu_score(p, shape, agg, n_vis=n_vis, vis_start=pre), _ref(p, shape, agg, n_vis, pre),
                 f"edge {agg}")
