"""Decode attention (draft and dense verify) on the GPU vs the fp64 oracle.

Tolerance (the contract): per (query, head) row,
max_d |o - o_ref| / max_d |o_ref| <= 2e-3 (bf16 inputs, fp32 accumulation);
lse within 1e-3 absolute.  Regression bounds, asserted beside it at about ten
times the error the kernels reach (~1e-5): row-relative <= 1e-4 and lse
within 1e-4 relative, so a kernel that rounded the softmax weights or the
output to bf16 (~2e-3) fails even though it would meet the contract."""
import math

import numpy as np
import pytest

import oracle
import workloads as W
from tests._util import dev_bf16, log, row_rel_err

pytestmark = pytest.mark.gpu
TOL = 2e-3
REG_TOL = 1e-4       # regression bound: ~10x the achieved row-relative error
F32_REG_TOL = 1e-5   # fp32 operands: no bf16 rounding of the weights at all

torch = pytest.importorskip("torch")


def _run(q, k, v, kv_len, causal, num_splits=0):
    from visual_kv_pruning_amd import ops
    qd = dev_bf16(q)
    kd = dev_bf16(k)
    vd = dev_bf16(v)
    kl = torch.tensor(np.asarray(kv_len, np.int32), device="cuda:0")
    o, lse = ops.decode_attn(qd, kd, vd, kl, causal, num_splits=num_splits)
    torch.cuda.synchronize()
    return o.cpu().numpy(), lse.cpu().numpy()


def _check(q, k, v, kv_len, causal, num_splits=0, name=""):
    log(f"decode_attn case {name}: q{q.shape} k{k.shape} kv_len={list(kv_len)} causal={causal} splits={num_splits}")
    o, lse = _run(q, k, v, kv_len, causal, num_splits)
    ro, rl = oracle.decode_attn(q, k, v, kv_len, causal)
    err = row_rel_err(o, ro)
    lerr = float(np.abs(lse - rl).max())
    lrel = float((np.abs(lse - rl) / np.maximum(1.0, np.abs(rl))).max())
    log(f"  row-rel err {err:.2e}  lse err {lerr:.2e}")
    assert err <= TOL, name
    assert lerr <= 1e-3, name
    assert err <= REG_TOL, f"{name}: row-relative error {err:.2e} above the regression bound"
    assert lrel <= REG_TOL, f"{name}: lse error {lrel:.2e} above the regression bound"
    return o, lse


def _rand(seed, *shape):
    rng = np.random.default_rng(seed)
    return W.bf16_round(rng.standard_normal(shape).astype(np.float32))


def test_tiny_config_verify_and_draft():
    cfg = W.C1
    p = W.prefill_layer(cfg, 0)
    nq = cfg.gamma_verify + 1
    kn, vn = W.new_kv(cfg, 0, nq)
    k = np.concatenate([p.k, kn], axis=1)
    v = np.concatenate([p.v, vn], axis=1)
    q = W.decode_queries(cfg, 0, nq)
    _check(q, k, v, [k.shape[1]], True, name="tiny verify")
    # draft over the kept visual rows + text + the newest token
    kept = np.sort(np.random.default_rng(0).choice(cfg.n_vis, cfg.budget, replace=False))
    rows = np.concatenate([kept, np.arange(cfg.n_vis, k.shape[1] - nq + 1)])
    _check(q[:, :1], k[:, rows], v[:, rows], [len(rows)], False, name="tiny draft")


# every (G, nq) with every key count that holds the nq new tokens
_SHAPES = [(G, nq, N) for G, nq in [(1, 1), (2, 5), (5, 10), (7, 1), (7, 10), (8, 6), (8, 1), (16, 6)]
           for N in [1, 31, 33, 65, 1000, 4099] if N >= nq]


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("G,nq,N", _SHAPES)
def test_shapes_and_ragged_tails(D, G, nq, N):
    Hkv = 2
    Hq = G * Hkv
    seed = D * 100000 + G * 1000 + nq * 100 + N
    q = _rand(seed, 1, nq, Hq, D)
    k = _rand(seed + 1, Hkv, N, D)
    v = _rand(seed + 2, Hkv, N, D)
    _check(q, k, v, [N], nq > 1, name=f"D{D} G{G} nq{nq} N{N}")


@pytest.mark.parametrize("splits", [1, 2, 3, 7, 40])
def test_forced_split_counts_agree(splits):
    q = _rand(7, 1, 6, 16, 128)
    k = _rand(8, 2, 3000, 128)
    v = _rand(9, 2, 3000, 128)
    _check(q, k, v, [3000], True, num_splits=splits, name=f"splits={splits}")


@pytest.mark.parametrize("nq,splits", [(1, 14), (6, 3), (6, 40)])
def test_workspace_reused_across_calls(nq, splits):
    """One workspace serves repeated calls; results are identical each time."""
    from visual_kv_pruning_amd import ops
    q = _rand(41, 1, nq, 16, 128)
    k = _rand(42, 2, 3000, 128)
    v = _rand(43, 2, 3000, 128)
    ro, rl = oracle.decode_attn(q, k, v, [3000], nq > 1)
    qd, kd, vd = dev_bf16(q), dev_bf16(k), dev_bf16(v)
    kl = torch.tensor([3000], dtype=torch.int32, device="cuda:0")
    need = ops.decode_attn_workspace_bytes(1, nq, 16, 2, 128, 3000, splits)
    ws = torch.full((need,), 0xFF, dtype=torch.uint8, device="cuda:0")
    log(f"decode_attn case workspace reuse nq={nq} splits={splits} ws={need}")
    first = None
    for rep in range(3):
        out = torch.full((1, nq, 16, 128), float("nan"), device="cuda:0")
        lse = torch.full((1, nq, 16), float("nan"), device="cuda:0")
        ops.decode_attn(qd, kd, vd, kl, nq > 1, num_splits=splits, out=out, lse=lse, ws=ws)
        torch.cuda.synchronize()
        o, l = out.cpu().numpy(), lse.cpu().numpy()
        assert row_rel_err(o, ro) <= REG_TOL and np.abs(l - rl).max() <= 1e-3, rep
        if first is None:
            first = (o, l)
        else:
            assert np.array_equal(first[0], o) and np.array_equal(first[1], l), rep


def test_batch_with_ragged_lengths_and_strided_cache():
    B, nq, Hq, Hkv, D, Ncap = 3, 4, 8, 2, 128, 700
    q = _rand(11, B, nq, Hq, D)
    k = _rand(12, B, Hkv, Ncap, D)
    v = _rand(13, B, Hkv, Ncap, D)
    kv_len = [700, 333, 4]
    log("decode_attn case batch ragged")
    o, lse = _run(q, k, v, kv_len, True)
    for b in range(B):
        ro, rl = oracle.decode_attn(q[b:b + 1], k[b], v[b], [kv_len[b]], True)
        assert row_rel_err(o[b:b + 1], ro) <= REG_TOL
        assert np.abs(lse[b:b + 1] - rl).max() <= 1e-3


@pytest.mark.parametrize("D,kv_len,splits", [(128, [9000, 300], 64), (128, [9000, 9000], 100), (64, [20000, 77], 100)])
def test_many_splits_batched_merge(D, kv_len, splits):
    """More partials per merge thread than one load round holds: the merge
    takes them in batches and carries its reference maximum between them.
    The short sequence leaves whole batches and whole split ranges empty."""
    B, nq, Hq, Hkv = len(kv_len), 3, 8, 2
    Ncap = max(kv_len)
    q = _rand(71 + D, B, nq, Hq, D)
    k = _rand(72 + D, B, Hkv, Ncap, D)
    v = _rand(73 + D, B, Hkv, Ncap, D)
    log(f"decode_attn case batched merge D={D} kv_len={kv_len} splits={splits}")
    o, lse = _run(q, k, v, kv_len, True, num_splits=splits)
    for b in range(B):
        ro, rl = oracle.decode_attn(q[b:b + 1], k[b], v[b], [kv_len[b]], True)
        err = row_rel_err(o[b:b + 1], ro)
        log(f"  batch {b}: row-rel err {err:.2e}")
        assert err <= REG_TOL
        assert np.abs(lse[b:b + 1] - rl).max() <= 1e-3


def test_verify_equals_sequential_draft_calls_on_gpu():
    """One dense pass over nq queries == nq single-query calls on the prefixes (same kernel family)."""
    nq, Hq, Hkv, D, N = 6, 16, 2, 128, 2500
    q = _rand(21, 1, nq, Hq, D)
    k = _rand(22, Hkv, N, D)
    v = _rand(23, Hkv, N, D)
    o, _ = _run(q, k, v, [N], True)
    for i in range(nq):
        n_i = N - nq + i + 1
        oi, _ = _run(q[:, i:i + 1], k[:, :n_i], v[:, :n_i], [n_i], False)
        assert row_rel_err(o[:, i:i + 1], oi) <= 1e-4


def test_deterministic_across_runs():
    q = _rand(31, 1, 6, 64, 128)
    k = _rand(32, 8, 5000, 128)
    v = _rand(33, 8, 5000, 128)
    a, la = _run(q, k, v, [5000], True)
    b, lb = _run(q, k, v, [5000], True)
    assert np.array_equal(a, b) and np.array_equal(la, lb)


def test_llava72b_shape_verify_and_draft_full_size():
    """72B shape at full size: 64 q / 8 KV heads, 25088 visual + 128 text + 6 verify tokens."""
    cfg = W.C3
    nq = cfg.gamma_verify + 1
    N = cfg.n_ctx + nq
    k, v = W.random_kv(cfg.index, cfg.hkv, N, cfg.d, layer=0)
    q = W.decode_queries(cfg, 0, nq)
    _check(q, k, v, [N], True, name="72B verify (launch used by the bench)")
    # 10% draft: kept visual + text + newest
    nk = cfg.budget + cfg.n_text + 1
    _check(q[:, :1], k[:, :nk], v[:, :nk], [nk], False, name="72B draft")


@pytest.mark.parametrize("cfg", [W.C2, W.C4], ids=lambda c: c.name)
def test_qwen_shapes_verify_and_draft_full_size(cfg):
    """The Qwen2-VL-7B (28 q / 4 KV heads, 8266 verify keys, two row chunks)
    and Qwen2.5-VL-32B (40 q / 8 KV heads, 20842 verify keys, one chunk of
    four row blocks) shapes at full size, every head, as the bench times them:
    dense verify of gamma + 1 = 10 queries and the 10% draft."""
    nq = cfg.gamma_verify + 1
    N = cfg.n_ctx + nq
    k, v = W.random_kv(cfg.index, cfg.hkv, N, cfg.d, layer=0)
    q = W.decode_queries(cfg, 0, nq)
    _check(q, k, v, [N], True, name=f"{cfg.name} verify")
    nk = cfg.budget + cfg.n_text + 1
    _check(q[:, :1], k[:, :nk], v[:, :nk], [nk], False, name=f"{cfg.name} draft")


def test_hour_long_shape_verify_sampled_heads():
    """141,194-key dense verify at the hour-long shape; oracle on the first KV head's rows."""
    cfg = W.C5
    nq = cfg.gamma_verify + 1
    N = cfg.n_ctx + nq
    k, v = W.random_kv(cfg.index, cfg.hkv, N, cfg.d, layer=0)
    q = W.decode_queries(cfg, 0, nq)
    log("decode_attn case hour-long verify")
    o, lse = _run(q, k, v, [N], True)
    G = cfg.group
    ro, rl = oracle.decode_attn(q[:, :, :G], k[:1], v[:1], [N], True)
    err = row_rel_err(o[:, :, :G], ro)
    log(f"  row-rel err {err:.2e}")
    assert err <= REG_TOL
    assert np.abs(lse[:, :, :G] - rl).max() <= 1e-3


@pytest.mark.parametrize("G,nq,N", [(5, 10, 20842), (7, 10, 16384), (8, 10, 17001), (16, 6, 16500)])
def test_long_context_row_chunks(G, nq, N):
    """At D = 128 and long contexts, 49-80 query rows run as one chunk of four
    or five row blocks (merged in two groups); the 32B shape is the first case.
    96 rows need two chunks even there."""
    Hkv = 2
    q = _rand(61 + G, 1, nq, G * Hkv, 128)
    k = _rand(62 + G, Hkv, N, 128)
    v = _rand(63 + G, Hkv, N, 128)
    _check(q, k, v, [N], True, name=f"long context G{G} nq{nq} N{N}")


@pytest.mark.parametrize("scale_q", [8.0, 32.0])
def test_wide_score_range(scale_q):
    """Queries scaled by a power of two (exact in bf16) spread the scores over
    tens to hundreds of log2 units, so every row's reference maximum is raised
    many times along the key loop, in split kernels and across splits."""
    q = _rand(61, 1, 6, 16, 128) * scale_q
    k = _rand(62, 2, 3000, 128)
    v = _rand(63, 2, 3000, 128)
    for splits in (1, 7):
        _check(q, k, v, [3000], True, num_splits=splits, name=f"wide range q x{scale_q:g} splits {splits}")


def test_binding_rejects_misshaped_outputs():
    """The library sees only pointers, so the binding refuses caller-supplied
    outputs that are not exactly what the kernels write."""
    from visual_kv_pruning_amd import ops
    log("decode_attn case binding output checks")
    qd = dev_bf16(_rand(51, 1, 2, 8, 64))
    kd = dev_bf16(_rand(52, 2, 100, 64))
    kl = torch.tensor([100], dtype=torch.int32, device="cuda:0")
    with pytest.raises(ValueError):
        ops.decode_attn(qd, kd, kd, kl, True, out=torch.empty(1, 2, 8, 32, device="cuda:0"))
    with pytest.raises(ValueError):
        ops.decode_attn(qd, kd, kd, kl, True, lse=torch.empty(1, 2, 4, device="cuda:0"))
    with pytest.raises(ValueError):
        ops.gather_kv(kd, kd, torch.arange(10, dtype=torch.int32, device="cuda:0"), 90, 10,
                      k_dst=torch.empty(2, 19, 64, dtype=torch.bfloat16, device="cuda:0"),
                      v_dst=torch.empty(2, 19, 64, dtype=torch.bfloat16, device="cuda:0"))
    with pytest.raises(ValueError):
        ops.gather_kv(kd, kd, torch.arange(10, dtype=torch.int32, device="cuda:0"),
                      k_dst=torch.empty(2, 10, 64, dtype=torch.bfloat16, device="cuda:0"))


def _f32_dev(x):
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to("cuda:0")


def test_tiny_config_fp32_operands():
    """The tiny reference configuration names fp32 values: q, k and v go to the
    plain fp32 kernels unrounded, and the oracle sees the same fp32 values.
    Verify (5 queries, causal tail) and the 10% draft, compact and in place."""
    from visual_kv_pruning_amd import ops
    cfg = W.C1
    p = W.prefill_layer(cfg, 0, round_bf16=False)
    nq = cfg.gamma_verify + 1
    kn, vn = W.new_kv(cfg, 0, nq, round_bf16=False)
    k = np.concatenate([p.k, kn], axis=1)
    v = np.concatenate([p.v, vn], axis=1)
    q = W.decode_queries(cfg, 0, nq, round_bf16=False)
    assert np.any(W.bf16_round(q) != q), "inputs should not be bf16 values"
    log("decode_attn case tiny fp32 verify")
    kl = torch.tensor([k.shape[1]], dtype=torch.int32, device="cuda:0")
    o, lse = ops.decode_attn(_f32_dev(q), _f32_dev(k), _f32_dev(v), kl, True)
    torch.cuda.synchronize()
    ro, rl = oracle.decode_attn(q, k, v, [k.shape[1]], True)
    err = row_rel_err(o.cpu().numpy(), ro)
    log(f"  row-rel err {err:.2e}")
    assert err <= F32_REG_TOL and np.abs(lse.cpu().numpy() - rl).max() <= 1e-5
    # draft over kept visual rows + text + newest, gathered in fp32 (bit-exact copy) and read in place
    kept = np.sort(np.random.default_rng(0).choice(cfg.n_vis, cfg.budget, replace=False)).astype(np.int32)
    n_tail = k.shape[1] - nq + 1 - cfg.n_vis
    kd, vd = ops.gather_kv(_f32_dev(k), _f32_dev(v), torch.from_numpy(kept).to("cuda:0"), cfg.n_vis, n_tail)
    rows = np.concatenate([kept, np.arange(cfg.n_vis, cfg.n_vis + n_tail)])
    torch.cuda.synchronize()
    assert np.array_equal(kd.cpu().numpy(), k[:, rows]) and np.array_equal(vd.cpu().numpy(), v[:, rows])
    rd, rdl = oracle.decode_attn(q[:, :1], k[:, rows], v[:, rows], [len(rows)], False)
    nk = torch.tensor([len(rows)], dtype=torch.int32, device="cuda:0")
    od, _ = ops.decode_attn(_f32_dev(q[:, :1]), kd, vd, nk, False)
    oi, li = ops.decode_attn_indexed(_f32_dev(q[:, :1]), _f32_dev(k), _f32_dev(v),
                                     torch.from_numpy(rows.astype(np.int32)).to("cuda:0"), nk, False)
    torch.cuda.synchronize()
    for got in (od, oi):
        err = row_rel_err(got.cpu().numpy(), rd)
        log(f"  draft row-rel err {err:.2e}")
        assert err <= F32_REG_TOL
    assert np.abs(li.cpu().numpy() - rdl).max() <= 1e-5


@pytest.mark.parametrize("D,G,nq,N", [(64, 2, 5, 217), (128, 8, 6, 3000), (64, 1, 1, 1), (128, 7, 10, 70)])
def test_fp32_operands_shapes(D, G, nq, N):
    """fp32 operands beyond the tiny shape: both head dims, MHA, one key, a
    ragged key count and a batch of two with different lengths."""
    from visual_kv_pruning_amd import ops
    rng = np.random.default_rng(D + G * 10 + nq * 100 + N)
    Hkv, B = 2, 2
    q = rng.standard_normal((B, nq, G * Hkv, D)).astype(np.float32)
    k = rng.standard_normal((B, Hkv, N, D)).astype(np.float32)
    v = rng.standard_normal((B, Hkv, N, D)).astype(np.float32)
    lens = [N, max(nq, N // 2)]
    log(f"decode_attn case fp32 D{D} G{G} nq{nq} N{N}")
    o, lse = ops.decode_attn(_f32_dev(q), _f32_dev(k), _f32_dev(v),
                             torch.tensor(lens, dtype=torch.int32, device="cuda:0"), nq > 1)
    torch.cuda.synchronize()
    for b in range(B):
        ro, rl = oracle.decode_attn(q[b:b + 1], k[b], v[b], [lens[b]], nq > 1)
        assert row_rel_err(o.cpu().numpy()[b:b + 1], ro) <= F32_REG_TOL
        assert np.abs(lse.cpu().numpy()[b:b + 1] - rl).max() <= 1e-5


def test_binding_rejects_batch_mismatch_and_bad_grid():
    """A 4-D cache whose batch axis is neither B nor 1 would be read past its
    end; the binding refuses it before any launch.  A batch axis of 1 is shared
    by every batch entry.  select refuses a frame grid that does not tile the row."""
    from visual_kv_pruning_amd import ops
    log("decode_attn case binding batch checks")
    q = _rand(71, 3, 1, 8, 64)
    k = _rand(72, 1, 2, 100, 64)
    v = _rand(73, 1, 2, 100, 64)
    kl = torch.tensor([100, 50, 7], dtype=torch.int32, device="cuda:0")
    with pytest.raises(ValueError):
        ops.decode_attn(dev_bf16(q), dev_bf16(np.concatenate([k, k])), dev_bf16(np.concatenate([v, v])), kl, False)
    with pytest.raises(ValueError):
        ops.decode_attn_indexed(dev_bf16(q), dev_bf16(np.concatenate([k, k])), dev_bf16(np.concatenate([v, v])),
                                torch.arange(10, dtype=torch.int32, device="cuda:0"),
                                torch.tensor([10, 10, 10], dtype=torch.int32, device="cuda:0"), False)
    o, _ = ops.decode_attn(dev_bf16(q), dev_bf16(k), dev_bf16(v), kl, False)     # shared cache
    torch.cuda.synchronize()
    for b, n in enumerate([100, 50, 7]):
        ro, _ = oracle.decode_attn(q[b:b + 1], k[0], v[0], [n], False)
        assert row_rel_err(o.cpu().numpy()[b:b + 1], ro) <= REG_TOL
    with pytest.raises(ValueError):
        ops.select(torch.rand(1, 100, device="cuda:0"), 2, 7, 7, 0.5, 10)


def test_seeded_random_shapes():
    """30 seeded random calls: batch 1-3 with ragged lengths, D 64 or 128,
    1-16 q heads per KV head over 1-4 KV heads, 1-10 queries, causal tail or
    not, the planner's split count or a forced one; each sequence against the
    oracle at the regression bound."""
    rng = np.random.default_rng(77)
    for case in range(30):
        B = int(rng.integers(1, 4))
        D = int(rng.choice([64, 128]))
        Hkv = int(rng.choice([1, 2, 4]))
        G = int(rng.integers(1, 17))
        nq = int(rng.integers(1, 11))
        Ncap = int(rng.integers(nq, 5001))
        kv_len = [int(rng.integers(nq, Ncap + 1)) for _ in range(B)]
        causal = bool(rng.integers(0, 2))
        splits = int(rng.choice([0, 0, int(rng.integers(1, 41))]))
        q = _rand(500 + case, B, nq, G * Hkv, D)
        k = _rand(600 + case, B, Hkv, Ncap, D)
        v = _rand(700 + case, B, Hkv, Ncap, D)
        log(f"decode_attn random case {case}: B={B} D={D} Hkv={Hkv} G={G} nq={nq} kv_len={kv_len} "
            f"causal={causal} splits={splits}")
        o, lse = _run(q, k, v, kv_len, causal, splits)
        for b in range(B):
            ro, rl = oracle.decode_attn(q[b:b + 1], k[b], v[b], [kv_len[b]], causal)
            err = row_rel_err(o[b:b + 1], ro)
            assert err <= REG_TOL, f"case {case} b {b}: {err:.2e}"
            assert np.abs(lse[b:b + 1] - rl).max() <= 1e-3, f"case {case} b {b}"
