"""svlm_decode_attn_noalloc (the entry point for callers that cannot
allocate: its split-K state lives in the library's static device scratch)
against svlm_decode_attn with a caller workspace, through the C ABI: the same
kernels and split plan, so the outputs must be bit-identical.  Two calls in a
row, the second with a smaller input, then the first again; and the size
limit is refused before anything is enqueued."""
import ctypes as C

import numpy as np
import pytest

import workloads as W
from tests._util import dev_bf16, log

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")


def _rand(seed, *shape):
    rng = np.random.default_rng(seed)
    return W.bf16_round(rng.standard_normal(shape).astype(np.float32))


def _call(name, q, k, v, kv_len, nq, Hq, Hkv, D, causal, out, lse, ws=None):
    from visual_kv_pruning_amd import _lib as L
    lib = L.load()
    stream = torch.cuda.current_stream().cuda_stream
    args = [q.data_ptr(), nq * Hq * D, k.data_ptr(), v.data_ptr(), 0, k.stride(0), k.stride(1), kv_len.data_ptr(),
            k.shape[1], L.SVLM_BF16, 1, nq, Hq, Hkv, D, C.c_float(1.0 / np.sqrt(D)), int(causal), out.data_ptr(),
            lse.data_ptr(), 0]
    if name == "svlm_decode_attn":
        args += [ws.data_ptr() if ws is not None else None, ws.numel() if ws is not None else 0]
    st = getattr(lib, name)(*args, stream)
    return st


def _both(seed, nq, Hq, Hkv, D, N):
    from visual_kv_pruning_amd import _lib as L, ops
    q = dev_bf16(_rand(seed, 1, nq, Hq, D))
    k = dev_bf16(_rand(seed + 1, Hkv, N, D))
    v = dev_bf16(_rand(seed + 2, Hkv, N, D))
    kl = torch.tensor([N], dtype=torch.int32, device="cuda:0")
    need = ops.decode_attn_workspace_bytes(1, nq, Hq, Hkv, D, N)
    ws = torch.empty(max(need, 16), dtype=torch.uint8, device="cuda:0")
    o_ref = torch.full((1, nq, Hq, D), float("nan"), device="cuda:0")
    l_ref = torch.full((1, nq, Hq), float("nan"), device="cuda:0")
    o = torch.full_like(o_ref, float("nan"))
    l = torch.full_like(l_ref, float("nan"))
    assert _call("svlm_decode_attn", q, k, v, kl, nq, Hq, Hkv, D, nq > 1, o_ref, l_ref, ws) == L.SVLM_OK
    assert _call("svlm_decode_attn_noalloc", q, k, v, kl, nq, Hq, Hkv, D, nq > 1, o, l) == L.SVLM_OK
    torch.cuda.synchronize()
    log(f"noalloc case nq={nq} Hq={Hq} Hkv={Hkv} D={D} N={N}: split state {need} bytes")
    assert not torch.isnan(o).any() and not torch.isnan(l).any()
    assert torch.equal(o, o_ref) and torch.equal(l, l_ref)


def test_noalloc_matches_workspace_entry_point_twice():
    """72B-shape dense verify (the largest state here, ~5.4 MB), then a smaller
    draft call on the same scratch, then a verify of another size again."""
    _both(1, 6, 64, 8, 128, 25222)
    _both(11, 1, 64, 8, 128, 2638)
    _both(21, 6, 16, 2, 64, 3001)


def test_noalloc_refuses_state_beyond_the_scratch():
    from visual_kv_pruning_amd import _lib as L, ops
    lib = L.load()
    # 64 queries x 64 heads over 10^6 keys with 256 splits needs far more than 16 MiB
    assert ops.decode_attn_workspace_bytes(1, 64, 64, 8, 128, 1 << 20, 256) > L.SVLM_NOALLOC_SCRATCH_BYTES
    fake = C.c_void_p(4096)
    st = lib.svlm_decode_attn_noalloc(fake, 64 * 64 * 128, fake, fake, 0, 128 << 20, 128, fake, 1 << 20,
                                      L.SVLM_BF16, 1, 64, 64, 8, 128, C.c_float(0.1), 1, fake, fake, 256, None)
    assert st == L.SVLM_E_UNSUPPORTED
    assert b"scratch" in lib.svlm_last_error()


def test_noalloc_fp32_operands_need_no_scratch():
    """fp32 operands use no split state: the no-allocation call gives the
    workspace call's bits without touching the scratch."""
    from visual_kv_pruning_amd import _lib as L
    lib = L.load()
    rng = np.random.default_rng(9)
    nq, Hq, Hkv, D, N = 3, 8, 2, 64, 500
    f32 = lambda x: torch.from_numpy(np.ascontiguousarray(x, np.float32)).to("cuda:0")
    q, k, v = f32(rng.standard_normal((1, nq, Hq, D))), f32(rng.standard_normal((Hkv, N, D))), \
        f32(rng.standard_normal((Hkv, N, D)))
    kl = torch.tensor([N], dtype=torch.int32, device="cuda:0")
    outs = []
    for name in ("svlm_decode_attn", "svlm_decode_attn_noalloc"):
        o = torch.full((1, nq, Hq, D), float("nan"), device="cuda:0")
        l = torch.full((1, nq, Hq), float("nan"), device="cuda:0")
        args = [q.data_ptr(), nq * Hq * D, k.data_ptr(), v.data_ptr(), 0, k.stride(0), k.stride(1), kl.data_ptr(), N,
                L.SVLM_F32, 1, nq, Hq, Hkv, D, C.c_float(0.125), 1, o.data_ptr(), l.data_ptr(), 0]
        if name == "svlm_decode_attn":
            args += [None, 0]
        assert getattr(lib, name)(*args, torch.cuda.current_stream().cuda_stream) == L.SVLM_OK
        outs.append((o, l))
    torch.cuda.synchronize()
    log("noalloc case fp32 operands")
    assert torch.equal(outs[0][0], outs[1][0]) and torch.equal(outs[0][1], outs[1][1])
    assert not torch.isnan(outs[0][0]).any()
