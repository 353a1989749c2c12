"""Decode attention over an index list read in place (gather fused into the
draft) vs the fp64 oracle on the gathered rows; and bit-equality with the
compact path (gather, then svlm_decode_attn) when both use the same split plan.

Tolerance as for svlm_decode_attn: per (query, head) row
max_d |o - o_ref| / max_d |o_ref| <= 2e-3; lse within 1e-3 absolute; and the
same regression bound of 1e-4 row-relative (about ten times the achieved
error), which a bf16 rounding of the weights or the output would break."""
import numpy as np
import pytest

import oracle
import workloads as W
from tests._util import dev_bf16, log, row_rel_err

pytestmark = pytest.mark.gpu
TOL = 2e-3
REG_TOL = 1e-4
torch = pytest.importorskip("torch")


def _rand(seed, *shape):
    rng = np.random.default_rng(seed)
    return W.bf16_round(rng.standard_normal(shape).astype(np.float32))


def _list(seed, n_rows, n_keep, tail):
    """kept rows (sorted, from the first n_rows - tail) then the last `tail` rows"""
    rng = np.random.default_rng(seed)
    kept = np.sort(rng.choice(n_rows - tail, n_keep, replace=False))
    return np.concatenate([kept, np.arange(n_rows - tail, n_rows)]).astype(np.int32)


def _ref_rows(q, k, v, lists, n_idx, causal):
    """oracle on the gathered rows; lists [B][Hkv][n] (numpy)"""
    B, Hkv = k.shape[0], k.shape[1]
    n = lists.shape[-1]
    kg = np.stack([np.stack([k[b, h, lists[b, h]] for h in range(Hkv)]) for b in range(B)])
    vg = np.stack([np.stack([v[b, h, lists[b, h]] for h in range(Hkv)]) for b in range(B)])
    return oracle.decode_attn(q, kg, vg, list(n_idx), causal)


def _check(q, k, v, lists_dev, lists_np, n_idx, causal, name, num_splits=0):
    """k, v: [B][Hkv][rows][D] numpy (batch 1 goes to the device as [Hkv][rows][D])"""
    from visual_kv_pruning_amd import ops
    log(f"decode_attn_indexed case {name}: q{q.shape} k{k.shape} n_idx={list(n_idx)} causal={causal}")
    ni = torch.tensor(np.asarray(n_idx, np.int32), device="cuda:0")
    kd, vd = (dev_bf16(k[0]), dev_bf16(v[0])) if k.shape[0] == 1 else (dev_bf16(k), dev_bf16(v))
    o, lse = ops.decode_attn_indexed(dev_bf16(q), kd, vd, lists_dev, ni, causal, num_splits=num_splits)
    torch.cuda.synchronize()
    ro, rl = _ref_rows(q, k, v, lists_np, n_idx, causal)
    err = row_rel_err(o.cpu().numpy(), ro)
    lerr = float(np.abs(lse.cpu().numpy() - rl).max())
    log(f"  row-rel err {err:.2e}  lse err {lerr:.2e}")
    assert err <= TOL and lerr <= 1e-3, name
    assert err <= REG_TOL, f"{name}: row-relative error {err:.2e} above the regression bound"


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("n_keep,tail", [(20, 17), (300, 129), (2509, 129)])
def test_shared_list_draft(D, n_keep, tail):
    Hq, Hkv, rows = 16, 2, 3200
    q = _rand(1 + n_keep, 1, 1, Hq, D)
    k = _rand(2 + n_keep, 1, Hkv, rows, D)
    v = _rand(3 + n_keep, 1, Hkv, rows, D)
    lst = _list(4 + n_keep, rows, n_keep, tail)
    lists_np = np.broadcast_to(lst, (1, Hkv, lst.size))
    _check(q, k, v, torch.tensor(lst, device="cuda:0"), lists_np, [lst.size], False,
           f"shared list D{D} keep {n_keep} + {tail}")


def test_per_head_lists_and_verify_tail():
    """different lists per KV head; 6 queries with the causal tail over the list"""
    Hq, Hkv, rows, D, nq = 16, 2, 2000, 128, 6
    q = _rand(11, 1, nq, Hq, D)
    k = _rand(12, 1, Hkv, rows, D)
    v = _rand(13, 1, Hkv, rows, D)
    lists = np.stack([_list(14 + h, rows, 700, 64) for h in range(Hkv)])
    _check(q, k, v, torch.tensor(lists, device="cuda:0"), lists[None], [lists.shape[1]], True,
           "per-head lists, verify")


def test_batch_ragged_lists_strided_cache():
    """three batch entries, [B][Hkv][n] lists of different valid lengths, cache rows with padding"""
    B, Hq, Hkv, rows, D, nq = 3, 8, 2, 900, 128, 2
    q = _rand(21, B, nq, Hq, D)
    kp = _rand(22, B, Hkv, rows, D + 64)          # padded rows: kv_sn = D + 64
    vp = _rand(23, B, Hkv, rows, D + 64)
    n = 400
    lists = np.stack([np.stack([_list(24 + 10 * b + h, rows, n - 16, 16) for h in range(Hkv)]) for b in range(B)])
    n_idx = [400, 257, 3]
    from visual_kv_pruning_amd import ops
    log("decode_attn_indexed case batch ragged strided")
    kd = dev_bf16(kp)[..., :D]
    vd = dev_bf16(vp)[..., :D]
    ni = torch.tensor(np.asarray(n_idx, np.int32), device="cuda:0")
    o, lse = ops.decode_attn_indexed(dev_bf16(q), kd, vd, torch.tensor(lists, device="cuda:0"), ni, True)
    torch.cuda.synchronize()
    ro, rl = _ref_rows(q, kp[..., :D], vp[..., :D], lists, n_idx, True)
    assert row_rel_err(o.cpu().numpy(), ro) <= REG_TOL
    assert float(np.abs(lse.cpu().numpy() - rl).max()) <= 1e-3


def test_long_list_forces_capped_splits():
    """a 9000-key list with one split asked for runs in several (the split's
    list is staged on chip); results unchanged"""
    Hq, Hkv, rows, D = 8, 2, 12000, 128
    q = _rand(31, 1, 1, Hq, D)
    k = _rand(32, 1, Hkv, rows, D)
    v = _rand(33, 1, Hkv, rows, D)
    lst = _list(34, rows, 8900, 100)
    lists_np = np.broadcast_to(lst, (1, Hkv, lst.size))
    _check(q, k, v, torch.tensor(lst, device="cuda:0"), lists_np, [lst.size], False, "long list", num_splits=1)


@pytest.mark.parametrize("nq", [1, 6])
def test_bit_equal_to_gather_then_attend(nq):
    """same keys, same split plan: the in-place read and the compact copy give identical bits"""
    from visual_kv_pruning_amd import ops
    Hq, Hkv, rows, D = 64, 8, 4000, 128
    q = dev_bf16(_rand(41, 1, nq, Hq, D))
    k = dev_bf16(_rand(42, Hkv, rows, D))
    v = dev_bf16(_rand(43, Hkv, rows, D))
    lst = _list(44, rows, 1200, 129)
    idx = torch.tensor(lst, device="cuda:0")
    n = lst.size
    kc, vc = ops.gather_kv(k, v, idx, 0, 0)
    ni = torch.tensor([n], dtype=torch.int32, device="cuda:0")
    log(f"decode_attn_indexed case bit-equality nq={nq}")
    o1, l1 = ops.decode_attn(q, kc, vc, ni, nq > 1)
    o2, l2 = ops.decode_attn_indexed(q, k, v, idx, ni, nq > 1)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_hour_long_per_head_lists_full_size():
    """The hour-long shape's in-place draft at full size: per-head lists of
    1024 kept visual rows + the 64 text rows + the newest row, read from a
    141194-row cache (28 q / 4 KV heads); the launch the bench times."""
    cfg = W.C5
    rows = cfg.n_ctx + 1
    n_keep, tail = cfg.budget, cfg.n_text + 1
    k, v = W.random_kv(cfg.index, cfg.hkv, rows, cfg.d, layer=3)
    q = W.decode_queries(cfg, 3, 1)
    lists = np.stack([_list(70 + h, rows, n_keep, tail) for h in range(cfg.hkv)])
    _check(q, k[None], v[None], torch.tensor(lists, device="cuda:0"), lists[None], [lists.shape[1]], False,
           "hour-long per-head lists, full size")


@pytest.mark.parametrize("G,nq,n_list", [(7, 10, 17000), (5, 10, 16500)])
def test_long_list_five_and_four_row_blocks(G, nq, n_list):
    """Lists of at least 16384 keys with 50-80 query rows run as one chunk of
    four or five row blocks through the index list (the long-context path)."""
    Hkv, D, rows = 2, 128, 20000
    q = _rand(81 + G, 1, nq, G * Hkv, D)
    k = _rand(82 + G, 1, Hkv, rows, D)
    v = _rand(83 + G, 1, Hkv, rows, D)
    lists = np.stack([_list(84 + G + h, rows, n_list - 64, 64) for h in range(Hkv)])
    _check(q, k, v, torch.tensor(lists, device="cuda:0"), lists[None], [lists.shape[1]], True,
           f"long list G{G} nq{nq} n{n_list}")


@pytest.mark.parametrize("nq", [1, 4])
def test_ragged_per_head_lengths(nq):
    """Per-(batch, KV head) list lengths (the per-layer, per-head selection of
    the Sparse-to-Dense explainer, "KV cache selection", keeps a different
    number of rows per head): n_idx [B][Hkv].  Each (b, KV head) is checked
    against the oracle on its own list prefix; the causal tail applies to the
    last nq positions of each list."""
    from visual_kv_pruning_amd import ops
    B, G, Hkv, rows, D = 2, 4, 4, 3000, 128
    Hq = G * Hkv
    q = _rand(91 + nq, B, nq, Hq, D)
    k = _rand(92, B, Hkv, rows, D)
    v = _rand(93, B, Hkv, rows, D)
    n_max = 1100
    lists = np.stack([np.stack([_list(94 + 10 * b + h, rows, n_max - 40, 40) for h in range(Hkv)])
                      for b in range(B)])
    n_idx = np.array([[1100, 517, 64, nq], [3 + nq, 1024, 1099, 700]], np.int32)
    log(f"decode_attn_indexed case ragged per-head lengths nq={nq}")
    o, lse = ops.decode_attn_indexed(dev_bf16(q), dev_bf16(k), dev_bf16(v), torch.tensor(lists, device="cuda:0"),
                                     torch.tensor(n_idx, device="cuda:0"), nq > 1)
    torch.cuda.synchronize()
    o, lse = o.cpu().numpy(), lse.cpu().numpy()
    worst = 0.0
    for b in range(B):
        for g in range(Hkv):
            n = int(n_idx[b, g])
            rsel = lists[b, g, :n]
            heads = slice(g * G, (g + 1) * G)
            ro, rl = oracle.decode_attn(q[b:b + 1, :, heads], k[b, g][None, rsel], v[b, g][None, rsel], [n],
                                        nq > 1)
            err = row_rel_err(o[b:b + 1, :, heads], ro)
            worst = max(worst, err)
            assert err <= REG_TOL, (b, g, n)
            assert float(np.abs(lse[b:b + 1, :, heads] - rl).max()) <= 1e-3, (b, g, n)
    log(f"  worst row-rel err {worst:.2e}")
    # the same lists with one length per batch entry give the per-batch result
    o1, _ = ops.decode_attn_indexed(dev_bf16(q), dev_bf16(k), dev_bf16(v), torch.tensor(lists, device="cuda:0"),
                                    torch.tensor([n_max, n_max], dtype=torch.int32, device="cuda:0"), nq > 1)
    o2, _ = ops.decode_attn_indexed(dev_bf16(q), dev_bf16(k), dev_bf16(v), torch.tensor(lists, device="cuda:0"),
                                    torch.full((B, Hkv), n_max, dtype=torch.int32, device="cuda:0"), nq > 1)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2)


def test_fp32_operands_ragged_per_head_lists():
    """fp32 operands through the index lists with ragged per-(batch, KV head)
    lengths and the causal tail, against the oracle on each list prefix; and
    the fp32 gather of per-head lists is a bit-exact copy."""
    from visual_kv_pruning_amd import ops
    B, G, Hkv, rows, D, nq = 2, 3, 2, 700, 64, 3
    rng = np.random.default_rng(123)
    q = rng.standard_normal((B, nq, G * Hkv, D)).astype(np.float32)
    k = rng.standard_normal((B, Hkv, rows, D)).astype(np.float32)
    v = rng.standard_normal((B, Hkv, rows, D)).astype(np.float32)
    lists = np.stack([np.stack([_list(200 + 10 * b + h, rows, 290, 10) for h in range(Hkv)]) for b in range(B)])
    n_idx = np.array([[300, 57], [nq, 211]], np.int32)
    f32 = lambda x: torch.from_numpy(np.ascontiguousarray(x)).to("cuda:0")
    log("decode_attn_indexed case fp32 ragged per-head lists")
    o, lse = ops.decode_attn_indexed(f32(q), f32(k), f32(v), f32(lists), f32(n_idx), True)
    torch.cuda.synchronize()
    o, lse = o.cpu().numpy(), lse.cpu().numpy()
    for b in range(B):
        for g in range(Hkv):
            n = int(n_idx[b, g])
            sel = lists[b, g, :n]
            heads = slice(g * G, (g + 1) * G)
            ro, rl = oracle.decode_attn(q[b:b + 1, :, heads], k[b, g][None, sel], v[b, g][None, sel], [n], True)
            assert row_rel_err(o[b:b + 1, :, heads], ro) <= 1e-5, (b, g)
            assert float(np.abs(lse[b:b + 1, :, heads] - rl).max()) <= 1e-5, (b, g)
    # fp32 gather of per-head lists (+ a text tail): a bit-exact copy
    kd, vd = ops.gather_kv(f32(k[0]), f32(v[0]), f32(lists[0, :, :100]), 690, 10)
    torch.cuda.synchronize()
    for g in range(Hkv):
        want = np.concatenate([k[0, g, lists[0, g, :100]], k[0, g, 690:700]])
        assert np.array_equal(kd.cpu().numpy()[g], want)
        want = np.concatenate([v[0, g, lists[0, g, :100]], v[0, g, 690:700]])
        assert np.array_equal(vd.cpu().numpy()[g], want)
