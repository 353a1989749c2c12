"""Mean text->visual attention on the GPU vs the fp64 oracle: within 1e-5
absolute (the contract).  Scores are ~1e-5 to 4e-5 at the full shapes, so the
absolute bound alone is loose; a regression bound is asserted beside it:
relative error <= 1e-4 on every score >= 1e-6 (the kernels reach ~3e-6)."""
import dataclasses

import numpy as np
import pytest

import oracle
import workloads as W
from tests._util import dev_bf16, log

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")
ABS_TOL = 1e-5
REL_TOL = 1e-4       # regression bound on scores >= 1e-6
F32_REL_TOL = 1e-5   # fp32 operands


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


def _compare(got, ref, name, rel_tol=REL_TOL):
    err = float(np.abs(got - ref).max())
    big = ref >= 1e-6
    rel = float((np.abs(got - ref)[big] / ref[big]).max()) if big.any() else 0.0
    log(f"score {name}: max abs err {err:.2e}, max rel err (scores >= 1e-6) {rel:.2e}")
    assert err <= ABS_TOL, name
    assert rel <= rel_tol, f"{name}: relative error {rel:.2e} above the regression bound"
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


def test_late_logit_spikes():
    """Keys set to 8, 16 and 32 times one text query (exact in bf16), placed
    past the first tile of their key splits: that query's scores with them
    lie ~130 to ~520 log2 units above everything before them, so pass 1's
    per-lane reference must be raised long after the first keys set it (the
    unchecked tile form overflows its limit there and the tile is redone with
    rescaling).  Other rows of the group see spikes of either sign."""
    cfg = W.C2
    p = W.prefill_layer(cfg, 0)
    k = p.k.copy()
    for pos, beta, t0, h0 in ((192 * 10 + 100, 8.0, 3, 0), (192 * 25 + 130, 16.0, 3, 0),
                              (192 * 40 + 170, 32.0, 17, 2), (cfg.n_vis - 40, 8.0, 40, 5)):
        k[h0 // cfg.group, pos, :] = beta * p.q_text[t0, h0, :]
    p = dataclasses.replace(p, k=k)
    log("score case late logit spikes")
    for agg in ("qhead", "kvhead"):
        _compare(_gpu_score(p, cfg, agg), _ref(p, cfg, agg), f"C2 late spikes {agg}")


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


@pytest.mark.parametrize("T,n_vis,Hq,Hkv", [
    (96, 16500, 5, 1),   # 5 heads x 6 row blocks over 8 waves: 4 or 3 units each, both passes
    (64, 3000, 7, 1),    # 7 x 4 units; pass 2 on 4 waves in two workgroups (4 and 3 units per wave)
    (40, 2000, 6, 2),    # 3 x 3 units over 4 waves: 3, 2, 2, 2
    (128, 16500, 6, 1),  # 6 x 8 units: pass 1 at 6 per wave; pass 2 keeps a wave per head
    (20, 2500, 12, 1),   # 12 x 2 units over two workgroups of 8 waves (2 or 1 per wave)
    (16, 16400, 10, 2),  # 5 units over 8 waves: waves 5-7 hold none
])
def test_unit_form_shapes(T, n_vis, Hq, Hkv):
    """Group sizes that are not a multiple of the waves run the passes over
    (q head, row block) units spread round-robin over the waves; every
    aggregation against the oracle (per-head rows keep a wave per head in
    pass 2, after a unit-form pass 1)."""
    D, pre, post = 128, 7, 5
    rng = np.random.default_rng(T * 100 + Hq)
    q_pos0 = pre + n_vis + post
    q = W.bf16_round(rng.standard_normal((T, Hq, D)).astype(np.float32))
    k = W.bf16_round(rng.standard_normal((Hkv, q_pos0 + T, D)).astype(np.float32))
    p, shape = _Layer(q, k, q_pos0), _Shape(n_vis, Hkv)
    log(f"score case units T{T} n_vis{n_vis} Hq{Hq} Hkv{Hkv}")
    for agg in ("qhead", "kvhead", "all"):
        _compare(_gpu_score(p, shape, agg, n_vis=n_vis, vis_start=pre), _ref(p, shape, agg, n_vis, pre),
                 f"units {agg}")


def test_hour_long_layer_sampled_kv_heads():
    """The hour-long shape (141120 visual + 64 text tokens, 28 q / 4 KV heads)
    at full size with one row per KV head, the signal its per-(layer, KV head)
    top-K consumes; the oracle checks KV heads 0 and 3 (their 7 q heads each)."""
    cfg = W.C5
    p = W.prefill_layer(cfg, 0)
    log("score case hour-long layer, per KV head")
    got = _gpu_score(p, cfg, "kvhead")
    G = cfg.group
    for g in (0, cfg.hkv - 1):
        heads = list(range(g * G, (g + 1) * G))
        sq = oracle.score_layer(p.q_text[:, heads], p.k[g:g + 1], p.q_pos0, 0, cfg.n_vis, 1)
        ref = oracle.aggregate_heads(sq, 1, "kvhead")
        _compare(got[g:g + 1], ref, f"hour-long kv head {g}")


def test_two_layers_per_layer_rows_match_oracle_rows():
    """Several layers into the per-layer rows of the 32B-shape selection and the
    per-(layer, KV head) rows of the hour-long selection, against the oracle's
    multi-layer row builder (reduced context so the oracle stays quick)."""
    from visual_kv_pruning_amd import ops
    cfg = W.C1
    layers = [W.prefill_layer(cfg, l) for l in range(3)]
    log("score case multi-layer rows")
    per_layer = torch.empty(3, cfg.n_vis, device="cuda:0")
    per_kv = torch.empty(3 * cfg.hkv, cfg.n_vis, device="cuda:0")
    one = torch.empty(1, cfg.n_vis, device="cuda:0")
    for l, p in enumerate(layers):
        ops.score(dev_bf16(p.q_text), dev_bf16(p.k), p.q_pos0, cfg.n_vis, agg="all", out=per_layer[l:l + 1])
        ops.score(dev_bf16(p.q_text), dev_bf16(p.k), p.q_pos0, cfg.n_vis, agg="kvhead",
                  out=per_kv[l * cfg.hkv:(l + 1) * cfg.hkv])
        ops.score(dev_bf16(p.q_text), dev_bf16(p.k), p.q_pos0, cfg.n_vis, agg="all", alpha=1.0 / 3,
                  beta=0.0 if l == 0 else 1.0, out=one)
    torch.cuda.synchronize()
    qk = [(p.q_text, p.k) for p in layers]
    _compare(per_layer.cpu().numpy(), oracle.score_rows_for_config(qk, cfg.n_vis, cfg.n_vis, cfg.hkv, "layer"),
             "rows per layer")
    _compare(per_kv.cpu().numpy(),
             oracle.score_rows_for_config(qk, cfg.n_vis, cfg.n_vis, cfg.hkv, "layer_kvhead"), "rows per kv head")
    _compare(one.cpu().numpy(), oracle.score_rows_for_config(qk, cfg.n_vis, cfg.n_vis, cfg.hkv, "all"),
             "one row over layers")


@pytest.mark.parametrize("agg", ["qhead", "kvhead", "all"])
def test_tiny_config_fp32_operands(agg):
    """The tiny reference configuration in fp32: unrounded q and k through the
    plain fp32 kernels against the oracle on the same values."""
    from visual_kv_pruning_amd import ops
    cfg = W.C1
    p = W.prefill_layer(cfg, 0, round_bf16=False)
    assert np.any(W.bf16_round(p.q_text) != p.q_text)
    log(f"score case tiny fp32 agg={agg}")
    f32 = lambda x: torch.from_numpy(np.ascontiguousarray(x, np.float32)).to("cuda:0")
    out = ops.score(f32(p.q_text), f32(p.k), p.q_pos0, cfg.n_vis, agg=agg)
    out2 = ops.score(f32(p.q_text), f32(p.k), p.q_pos0, cfg.n_vis, agg=agg, alpha=0.5, beta=0.25,
                     out=out.clone())
    torch.cuda.synchronize()
    ref = _ref(p, cfg, agg)
    _compare(out.cpu().numpy(), ref, f"tiny fp32/{agg}", rel_tol=F32_REL_TOL)
    _compare(out2.cpu().numpy(), 0.75 * ref, f"tiny fp32/{agg} alpha beta", rel_tol=F32_REL_TOL)


# ---------------------------------------------------------------------------
# svlm_score_layers: every layer in one call


def _stack_layers(cfg, n):
    ps = [W.prefill_layer(cfg, l) for l in range(n)]
    return ps, np.stack([p.q_text for p in ps]), np.stack([p.k for p in ps])


@pytest.mark.parametrize("cfg,n", [(W.C1, 5), (W.C2, 3)], ids=["tiny5", "qwen2vl7b3"])
@pytest.mark.parametrize("rows", ["all", "layer", "layer_kvhead", "kvhead_mean"])
def test_layers_in_one_call_match_oracle_rows(cfg, n, rows):
    """One call over n layers against the oracle's multi-layer rows: the
    single row averaged over layers and heads, one row per layer, one row
    per (layer, KV head), and the per-KV-head rows averaged over layers."""
    from visual_kv_pruning_amd import ops
    ps, q, k = _stack_layers(cfg, n)
    agg = "kvhead" if rows in ("layer_kvhead", "kvhead_mean") else "all"
    mean = rows in ("all", "kvhead_mean")
    log(f"score_layers case {cfg.name} x{n} {rows}")
    out = ops.score_layers(dev_bf16(q), dev_bf16(k), ps[0].q_pos0, cfg.n_vis, agg=agg, layer_mean=mean)
    torch.cuda.synchronize()
    got = out.cpu().numpy().reshape(-1, cfg.n_vis)
    if rows == "kvhead_mean":
        ref = np.mean([_ref(p, cfg, "kvhead") for p in ps], axis=0)
    else:
        ref = oracle.score_rows_for_config([(p.q_text, p.k) for p in ps], ps[0].q_pos0, cfg.n_vis, cfg.hkv, rows)
    _compare(got, ref, f"{cfg.name} x{n} {rows}")


def test_layers_alpha_beta():
    """out = alpha * (layer mean) + beta * out."""
    from visual_kv_pruning_amd import ops
    cfg = W.C1
    ps, q, k = _stack_layers(cfg, 3)
    prev = np.random.default_rng(2).random((1, cfg.n_vis)).astype(np.float32) * 1e-3
    out = torch.from_numpy(prev).cuda()
    log("score_layers case alpha/beta")
    ops.score_layers(dev_bf16(q), dev_bf16(k), ps[0].q_pos0, cfg.n_vis, agg="all", layer_mean=True,
                     alpha=0.25, beta=2.0, out=out)
    torch.cuda.synchronize()
    ref = 0.25 * oracle.score_rows_for_config([(p.q_text, p.k) for p in ps], ps[0].q_pos0, cfg.n_vis, cfg.hkv,
                                              "all") + 2.0 * prev
    _compare(out.cpu().numpy(), ref, "tiny x3 alpha/beta")


@pytest.mark.parametrize("agg", ["qhead", "kvhead", "all"])
def test_one_layer_call_is_svlm_score(agg):
    """layers = 1 runs svlm_score's launches: bit-identical rows, with or
    without the layer mean."""
    from visual_kv_pruning_amd import ops
    cfg = W.C2
    p = W.prefill_layer(cfg, 0)
    qd, kd = dev_bf16(p.q_text), dev_bf16(p.k)
    log(f"score_layers case one layer {agg}")
    a = ops.score(qd, kd, p.q_pos0, cfg.n_vis, agg=agg)
    b = ops.score_layers(qd[None], kd[None], p.q_pos0, cfg.n_vis, agg=agg, layer_mean=False)
    c = ops.score_layers(qd[None], kd[None], p.q_pos0, cfg.n_vis, agg=agg, layer_mean=agg != "qhead")
    torch.cuda.synchronize()
    assert torch.equal(a, b[0]) and torch.equal(a, c.reshape(a.shape))


def test_llava72b_four_layers_sampled_kv_head():
    """Four full 72B-shape layers in one call, rows per KV head averaged over
    the layers; the oracle checks KV head 0 (its 8 q heads, every layer)."""
    from visual_kv_pruning_amd import ops
    cfg = W.C3
    ps, q, k = _stack_layers(cfg, 4)
    log("score_layers case 72B x4, KV head 0")
    out = ops.score_layers(dev_bf16(q), dev_bf16(k), ps[0].q_pos0, cfg.n_vis, agg="kvhead", layer_mean=True)
    torch.cuda.synchronize()
    G = cfg.group
    ref = np.mean([oracle.aggregate_heads(oracle.score_layer(p.q_text[:, :G], p.k[:1], p.q_pos0, 0, cfg.n_vis, 1),
                                          1, "kvhead") for p in ps], axis=0)
    _compare(out.cpu().numpy()[:1], ref, "72B x4 kv head 0")


def test_llava72b_eighty_layers_equal_per_layer_calls():
    """The launch bench.py times: all 80 layers of the 72B shape in one call,
    against the mean of 80 svlm_score calls (each pinned to the oracle above);
    the two differ by fp32 summation order only.  Repeated calls are
    bit-identical."""
    from visual_kv_pruning_amd import ops
    cfg = W.C3
    L, T, Hq, Hkv, D, NV = cfg.layers, cfg.n_text, cfg.hq, cfg.hkv, cfg.d, cfg.n_vis
    g = torch.Generator(device="cuda:0").manual_seed(9)
    k = torch.empty(L, Hkv, cfg.n_ctx, D, dtype=torch.bfloat16, device="cuda:0")
    for l in range(L):
        k[l].copy_(torch.randn(Hkv, cfg.n_ctx, D, generator=g, device="cuda:0"))
    q = torch.randn(L, T, Hq, D, generator=g, device="cuda:0").to(torch.bfloat16)
    log("score_layers case 72B x80 vs per-layer calls")
    per = torch.empty(1, NV, device="cuda:0")
    for l in range(L):
        ops.score(q[l], k[l], NV, NV, agg="all", alpha=1.0 / L, beta=0.0 if l == 0 else 1.0, out=per)
    one = ops.score_layers(q, k, NV, NV, agg="all", layer_mean=True)
    again = ops.score_layers(q, k, NV, NV, agg="all", layer_mean=True)
    torch.cuda.synchronize()
    assert torch.equal(one, again)
    a, b = one.cpu().numpy().astype(np.float64), per.cpu().numpy().astype(np.float64)
    rel = float((np.abs(a - b) / np.abs(b)).max())
    log(f"  max relative difference {rel:.2e}")
    assert rel <= 1e-5


def test_hour_long_two_layers_in_one_call_sampled_kv_heads():
    """Two hour-long layers (141120 visual + 64 text tokens, 28 q / 4 KV heads)
    in one call with one row per (layer, KV head), the rows the hour-long
    top-K consumes; the oracle checks KV heads 0 and 3 of both layers."""
    from visual_kv_pruning_amd import ops
    cfg = W.C5
    ps, q, k = _stack_layers(cfg, 2)
    log("score_layers case hour-long x2, per (layer, KV head)")
    out = ops.score_layers(dev_bf16(q), dev_bf16(k), ps[0].q_pos0, cfg.n_vis, agg="kvhead", layer_mean=False)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    G = cfg.group
    for l, p in enumerate(ps):
        for g in (0, cfg.hkv - 1):
            heads = list(range(g * G, (g + 1) * G))
            sq = oracle.score_layer(p.q_text[:, heads], p.k[g:g + 1], p.q_pos0, 0, cfg.n_vis, 1)
            _compare(got[l, g:g + 1], oracle.aggregate_heads(sq, 1, "kvhead"), f"hour-long layer {l} kv head {g}")


@pytest.mark.parametrize("rows", ["all", "layer_kvhead"])
def test_layers_fp32_operands(rows):
    """svlm_score_layers on fp32 operands (the plain fp32 kernels, one layer
    after another): three unrounded tiny-shape layers against the oracle."""
    from visual_kv_pruning_amd import ops
    cfg = W.C1
    ps = [W.prefill_layer(cfg, l, round_bf16=False) for l in range(3)]
    q = np.stack([p.q_text for p in ps])
    k = np.stack([p.k for p in ps])
    f32 = lambda x: torch.from_numpy(np.ascontiguousarray(x, np.float32)).to("cuda:0")
    agg, mean = ("all", True) if rows == "all" else ("kvhead", False)
    log(f"score_layers case tiny fp32 x3 {rows}")
    out = ops.score_layers(f32(q), f32(k), ps[0].q_pos0, cfg.n_vis, agg=agg, layer_mean=mean)
    torch.cuda.synchronize()
    ref = oracle.score_rows_for_config([(p.q_text, p.k) for p in ps], ps[0].q_pos0, cfg.n_vis, cfg.hkv, rows)
    _compare(out.cpu().numpy().reshape(-1, cfg.n_vis), ref, f"tiny fp32 x3 {rows}", rel_tol=F32_REL_TOL)


def _random_case(seed):
    rng = np.random.default_rng(1000 + seed)
    D = int(rng.choice([64, 128]))
    Hkv = int(rng.choice([1, 2, 4]))
    G = int(rng.choice([1, 2, 3, 5, 7, 8, 12]))
    T = int(rng.integers(1, 129))
    wide = seed % 3 == 0  # visual ranges past 16384 keys take eight pass-2 waves
    n_vis = int(rng.integers(16384, 17500)) if wide else int(rng.integers(1, 3000))
    pre, post = int(rng.integers(0, 40)), int(rng.integers(0, 40))
    layers = int(rng.integers(1, 3 if wide else 5))
    agg = str(rng.choice(["qhead", "kvhead", "all"]))
    mean = bool(rng.integers(0, 2)) and agg != "qhead"
    return D, Hkv, G, T, n_vis, pre, post, layers, agg, mean


@pytest.mark.parametrize("seed", range(12))
def test_layers_random_shapes(seed):
    """Seeded random shapes through svlm_score_layers against the oracle:
    head dims, group sizes that are not powers of two (idle waves), ragged
    text rows, keys before and after the visual window, one to four layers,
    every aggregation, with and without the layer mean, and visual ranges on
    both sides of the eight-wave threshold."""
    from visual_kv_pruning_amd import ops
    D, Hkv, G, T, n_vis, pre, post, layers, agg, mean = _random_case(seed)
    Hq = G * Hkv
    q_pos0 = pre + n_vis + post
    n_ctx = q_pos0 + T
    rng = np.random.default_rng(seed)
    q = W.bf16_round(rng.standard_normal((layers, T, Hq, D)).astype(np.float32))
    k = W.bf16_round(rng.standard_normal((layers, Hkv, n_ctx, D)).astype(np.float32))
    log(f"score_layers case random {seed}: D{D} Hkv{Hkv} G{G} T{T} n_vis{n_vis} pre{pre} post{post} "
        f"layers{layers} {agg} mean={mean}")
    out = ops.score_layers(dev_bf16(q), dev_bf16(k), q_pos0, n_vis, vis_start=pre, agg=agg, layer_mean=mean)
    torch.cuda.synchronize()
    refs = [_ref(_Layer(q[l], k[l], q_pos0), _Shape(n_vis, Hkv), agg, n_vis, pre) for l in range(layers)]
    ref = np.mean(refs, axis=0) if mean else np.concatenate(refs, axis=0)
    _compare(out.cpu().numpy().reshape(ref.shape), ref, f"random {seed}")
