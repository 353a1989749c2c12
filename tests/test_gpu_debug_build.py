"""The SVLM_DEBUG build (libsvlm_debug.so): kernels record the device
preconditions that calls violate, beside the clamping every build does.
Each check is driven through the C ABI with one out-of-range value of the
kind it watches, which the kernels provably keep inside the buffers (an
index outside the cache reads a zero row, a length is clamped into
[0, max], a draft token into [0, V), a score above 1 only changes
arithmetic), and must raise exactly its bit; valid inputs raise none."""
import ctypes as C
import math

import pytest

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")

from tests._util import log  # noqa: E402
from visual_kv_pruning_amd import _lib as L  # noqa: E402

DEV = "cuda:0"


@pytest.fixture(scope="module")
def dbg():
    lib = L.load_debug()
    torch.cuda.synchronize()
    L.debug_flags(lib)  # start clean
    return lib


def _p(t):
    return C.c_void_p(t.data_ptr())


def _stream():
    return C.c_void_p(torch.cuda.current_stream().cuda_stream)


def _flags(lib):
    torch.cuda.synchronize()
    return L.debug_flags(lib)


def _gather(lib, k, v, idx, n_idx, tail_start, n_tail):
    Hkv, n_src, D = k.shape
    n = n_idx + n_tail
    kd = torch.full((Hkv, n, D), 7.0, device=DEV).to(torch.bfloat16)
    vd = kd.clone()
    st = lib.svlm_gather_kv(_p(k), _p(v), n_src * D, D, n_src, _p(idx), idx.shape[1], n_idx, tail_start, n_tail,
                            _p(kd), _p(vd), n * D, D, Hkv, D, L.SVLM_BF16, _stream())
    assert st == L.SVLM_OK, lib.svlm_last_error()
    return kd, vd


def test_gather_index_outside_the_source(dbg):
    log("debug build case gather index")
    g = torch.Generator(device=DEV).manual_seed(1)
    k = torch.randn(2, 100, 128, generator=g, device=DEV).to(torch.bfloat16)
    v = torch.randn(2, 100, 128, generator=g, device=DEV).to(torch.bfloat16)
    good = torch.tensor([[0, 5, 99, 3, 4], [1, 2, 3, 4, 5]], dtype=torch.int32, device=DEV)
    _gather(dbg, k, v, good, 5, 98, 2)
    assert _flags(dbg) == 0
    bad = good.clone()
    bad[0, 3], bad[1, 4] = 100, -1
    kd, vd = _gather(dbg, k, v, bad, 5, 98, 2)
    assert _flags(dbg) == L.SVLM_DBG_GATHER_INDEX
    assert torch.equal(kd[0, 3], torch.zeros_like(kd[0, 3])) and torch.equal(vd[1, 4], torch.zeros_like(vd[1, 4]))
    assert torch.equal(kd[0, 2], k[0, 99]) and torch.equal(kd[1, 5], k[1, 98])
    assert _flags(dbg) == 0  # reading cleared them


def _attn_inputs(dtype, B, nq, Hq, Hkv, D, N, seed):
    g = torch.Generator(device=DEV).manual_seed(seed)
    q = torch.randn(B, nq, Hq, D, generator=g, device=DEV).to(dtype)
    k = torch.randn(B, Hkv, N, D, generator=g, device=DEV).to(dtype)
    v = torch.randn(B, Hkv, N, D, generator=g, device=DEV).to(dtype)
    return q, k, v


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_attention_length_above_its_bound(dbg, dtype):
    log(f"debug build case attention length {dtype}")
    B, nq, Hq, Hkv, D, N = 2, 6, 8, 2, 128, 1500
    q, k, v = _attn_inputs(dtype, B, nq, Hq, Hkv, D, N, 2)
    dt = L.SVLM_BF16 if dtype == torch.bfloat16 else L.SVLM_F32
    out = torch.empty(B, nq, Hq, D, device=DEV)
    lse = torch.empty(B, nq, Hq, device=DEV)
    wsb = max(256, dbg.svlm_decode_attn_workspace(B, nq, Hq, Hkv, D, N, 0))
    ws = torch.empty(wsb, dtype=torch.uint8, device=DEV)

    def run(lengths):
        kl = torch.tensor(lengths, dtype=torch.int32, device=DEV)
        st = dbg.svlm_decode_attn(_p(q), nq * Hq * D, _p(k), _p(v), Hkv * N * D, N * D, D, _p(kl), N, dt, B, nq, Hq,
                                  Hkv, D, 1.0 / math.sqrt(D), 1, _p(out), _p(lse), 0, _p(ws), wsb, _stream())
        assert st == L.SVLM_OK, dbg.svlm_last_error()
        return out.clone()

    ref = run([N, 900])
    assert _flags(dbg) == 0
    got = run([N + 40, 900])   # clamped to N: the same result
    assert _flags(dbg) == L.SVLM_DBG_KV_LEN
    assert torch.equal(got, ref)


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_attention_index_outside_the_cache(dbg, dtype):
    log(f"debug build case attention index {dtype}")
    B, nq, Hq, Hkv, D, rows = 1, 1, 8, 2, 128, 3000
    q, k, v = _attn_inputs(dtype, B, nq, Hq, Hkv, D, rows, 3)
    dt = L.SVLM_BF16 if dtype == torch.bfloat16 else L.SVLM_F32
    n = 300
    g = torch.Generator(device=DEV).manual_seed(4)
    idx = torch.randperm(rows, generator=g, device=DEV)[:n].sort().values.to(torch.int32).reshape(1, n)
    n_idx = torch.full((1,), n, dtype=torch.int32, device=DEV)
    out = torch.empty(B, nq, Hq, D, device=DEV)
    lse = torch.empty(B, nq, Hq, device=DEV)
    wsb = max(256, dbg.svlm_decode_attn_indexed_workspace(B, nq, Hq, Hkv, D, n, 0))
    ws = torch.empty(wsb, dtype=torch.uint8, device=DEV)

    def run(lst):
        st = dbg.svlm_decode_attn_indexed(_p(q), nq * Hq * D, _p(k), _p(v), Hkv * rows * D, rows * D, D, rows,
                                          _p(lst), n, 0, _p(n_idx), 1, 0, n, dt, B, nq, Hq, Hkv, D,
                                          1.0 / math.sqrt(D), 0, _p(out), _p(lse), 0, _p(ws), wsb, _stream())
        assert st == L.SVLM_OK, dbg.svlm_last_error()

    run(idx)
    assert _flags(dbg) == 0
    bad = idx.clone()
    bad[0, 17] = rows       # one past the cache: read as a zero row
    run(bad)
    assert _flags(dbg) == L.SVLM_DBG_KV_INDEX
    assert torch.isfinite(out).all()


@pytest.mark.parametrize("mode", [L.SVLM_VERIFY_GREEDY, L.SVLM_VERIFY_REJECT])
def test_verify_draft_token_outside_the_vocabulary(dbg, mode):
    log(f"debug build case verify draft token mode {mode}")
    B, gamma, V = 2, 4, 5000
    g = torch.Generator(device=DEV).manual_seed(5)
    if mode == L.SVLM_VERIFY_GREEDY:
        target = torch.randn(B, gamma + 1, V, generator=g, device=DEV)
        q = u = None
    else:
        target = torch.softmax(torch.randn(B, gamma + 1, V, generator=g, device=DEV), -1)
        q = torch.softmax(torch.randn(B, gamma, V, generator=g, device=DEV), -1)
        u = torch.rand(B, gamma + 1, generator=g, device=DEV)
    n_acc = torch.empty(B, dtype=torch.int32, device=DEV)
    nxt = torch.empty(B, dtype=torch.int32, device=DEV)
    wsb = dbg.svlm_verify_workspace(B, gamma, V)
    ws = torch.zeros(wsb, dtype=torch.uint8, device=DEV)  # arrival counters start at zero

    def run(draft):
        st = dbg.svlm_verify(mode, B, gamma, V, _p(draft), _p(target), _p(q) if q is not None else None,
                             _p(u) if u is not None else None, _p(n_acc), _p(nxt), _p(ws), wsb, _stream())
        assert st == L.SVLM_OK, dbg.svlm_last_error()

    draft = torch.randint(0, V, (B, gamma), generator=g, device=DEV, dtype=torch.int32)
    run(draft)
    assert _flags(dbg) == 0
    bad = draft.clone()
    bad[0, 0] = V + 2 if mode == L.SVLM_VERIFY_GREEDY else -1
    run(bad)
    assert _flags(dbg) == L.SVLM_DBG_DRAFT_TOKEN


def test_select_score_above_one(dbg):
    log("debug build case select score range")
    F, H, W = 4, 7, 7
    n = F * H * W
    g = torch.Generator(device=DEV).manual_seed(6)
    row = torch.rand(1, n, generator=g, device=DEV) * 1e-2
    kept = torch.empty(1, 20, dtype=torch.int32, device=DEV)
    n1 = torch.empty(1, dtype=torch.int32, device=DEV)

    def run(r):
        st = dbg.svlm_select(_p(r), n, 1, F, H, W, 0.5, 20, _p(kept), _p(n1), None, None, 0, _stream())
        assert st == L.SVLM_OK, dbg.svlm_last_error()

    run(row)
    assert _flags(dbg) == 0
    bad = row.clone()
    bad[0, 11] = 1.5
    run(bad)
    assert _flags(dbg) == L.SVLM_DBG_SCORE_RANGE
