"""KV compaction on the GPU vs NumPy indexing: bit-exact."""
import numpy as np
import pytest

import oracle
import workloads as W
from tests._util import dev_bf16, log

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("per_head", [False, True])
def test_gather_matches_indexing(D, per_head):
    from visual_kv_pruning_amd import ops
    Hkv, N, n_idx, T = 4, 3000, 301, 17
    k, v = W.random_kv(3, Hkv, N, D)
    rng = np.random.default_rng(D + per_head)
    if per_head:
        idx = np.stack([np.sort(rng.choice(N - T, n_idx, replace=False)) for _ in range(Hkv)]).astype(np.int32)
    else:
        idx = np.sort(rng.choice(N - T, n_idx, replace=False)).astype(np.int32)
    log(f"gather case D={D} per_head={per_head}")
    kd, vd = ops.gather_kv(dev_bf16(k), dev_bf16(v), torch.from_numpy(idx).cuda(), N - T, T)
    torch.cuda.synchronize()
    rk = oracle.gather_kv(k, idx, N - T, T)
    rv = oracle.gather_kv(v, idx, N - T, T)
    assert np.array_equal(kd.float().cpu().numpy(), rk)
    assert np.array_equal(vd.float().cpu().numpy(), rv)


def test_all_layers_in_one_call():
    """Layers folded into the head axis ([L][Hkv] -> L*Hkv heads, uniform
    strides) gather every layer's kept rows in one call, into a destination
    with room for more rows per head (the draft cache), as bench.py does."""
    from visual_kv_pruning_amd import ops
    L, Hkv, N, D, T, n_idx, n_cap = 5, 4, 2000, 128, 16, 203, 240
    rng = np.random.default_rng(17)
    kv = W.bf16_round(rng.standard_normal((2, L, Hkv, N, D)).astype(np.float32))
    idx = np.sort(rng.choice(N - T, n_idx, replace=False)).astype(np.int32)
    kvd = dev_bf16(kv)
    dst = torch.zeros(2, L, Hkv, n_cap, D, dtype=torch.bfloat16, device="cuda:0")
    log(f"gather case all layers in one call L={L}")
    n = n_idx + T
    dk, dv = dst[0, :, :, :n].reshape(L * Hkv, n, D), dst[1, :, :, :n].reshape(L * Hkv, n, D)
    assert dk.data_ptr() == dst[0].data_ptr() and dk.stride(0) == n_cap * D  # views, not copies
    ops.gather_kv(kvd[0].reshape(L * Hkv, N, D), kvd[1].reshape(L * Hkv, N, D), torch.from_numpy(idx).cuda(),
                  N - T, T, dk, dv)
    torch.cuda.synchronize()
    got = dst.float().cpu().numpy()
    for l in range(L):
        for t in range(2):
            assert np.array_equal(got[t, l, :, :n], oracle.gather_kv(kv[t, l], idx, N - T, T)), (l, t)
    assert not got[:, :, :, n:].any()  # rows past the gathered ones untouched


def test_gather_into_strided_destination_and_empty():
    from visual_kv_pruning_amd import ops
    k, v = W.random_kv(4, 2, 500, 128)
    idx = torch.tensor([5, 7, 499, 0], dtype=torch.int32, device="cuda:0")
    big_k = torch.zeros(2, 64, 128, dtype=torch.bfloat16, device="cuda:0")
    big_v = torch.zeros(2, 64, 128, dtype=torch.bfloat16, device="cuda:0")
    log("gather case strided destination")
    ops.gather_kv(dev_bf16(k), dev_bf16(v), idx, 100, 3, big_k[:, 10:], big_v[:, 10:])
    torch.cuda.synchronize()
    ref = oracle.gather_kv(k, [5, 7, 499, 0], 100, 3)
    assert np.array_equal(big_k[:, 10:17].float().cpu().numpy(), ref)
    assert torch.count_nonzero(big_k[:, :10]) == 0 and torch.count_nonzero(big_k[:, 17:]) == 0
    # nothing to copy
    ops.gather_kv(dev_bf16(k), dev_bf16(v), idx[:0], 0, 0, big_k[:, :0], big_v[:, :0])


def test_out_of_range_index_writes_zeros():
    from visual_kv_pruning_amd import ops
    k, v = W.random_kv(5, 1, 100, 128)
    idx = torch.tensor([3, 100, -1, 99], dtype=torch.int32, device="cuda:0")
    log("gather case out-of-range indices")
    kd, vd = ops.gather_kv(dev_bf16(k), dev_bf16(v), idx)
    torch.cuda.synchronize()
    out = kd.float().cpu().numpy()
    assert np.array_equal(out[0, 0], k[0, 3]) and np.array_equal(out[0, 3], k[0, 99])
    assert not out[0, 1].any() and not out[0, 2].any()
