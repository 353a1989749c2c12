"""Thin PyTorch-facing wrappers over the libsvlm C ABI.

Each function checks devices, dtypes and shapes, allocates outputs and
workspaces with torch (device memory only), and calls the matching svlm_*
entry point on torch's current stream.  Every step of the computation runs
in the HIP kernels; nothing here computes on tensors.
"""
from __future__ import annotations

import math

import torch

from . import _lib as L

_AGG = {"qhead": L.SVLM_AGG_QHEAD, "kvhead": L.SVLM_AGG_KVHEAD, "all": L.SVLM_AGG_ALL}


def _stream() -> int:
    return torch.cuda.current_stream().cuda_stream


def _dev(*ts):
    for t in ts:
        if t is not None and not t.is_cuda:
            raise ValueError("svlm tensors must live on the GPU")


def _bf16(*ts):
    for t in ts:
        if t.dtype != torch.bfloat16:
            raise TypeError(f"expected bfloat16, got {t.dtype}")
        if t.stride(-1) != 1:
            raise ValueError("the last (head-dim) axis must be contiguous")


_DTYPES = {torch.bfloat16: L.SVLM_BF16, torch.float32: L.SVLM_F32}


def _operands(*ts) -> int:
    """Attention operands: all bf16 (the matrix-core kernels) or all fp32 (the
    plain fp32 kernels), head-dim axis contiguous.  Returns the svlm dtype code."""
    dt = ts[0].dtype
    if dt not in _DTYPES:
        raise TypeError(f"expected bfloat16 or float32 operands, got {dt}")
    for t in ts:
        if t.dtype != dt:
            raise TypeError(f"operands must share one dtype ({dt} and {t.dtype})")
        if t.stride(-1) != 1:
            raise ValueError("the last (head-dim) axis must be contiguous")
    return _DTYPES[dt]


def _ws(nbytes: int, device) -> torch.Tensor:
    return torch.empty(max(int(nbytes), 16), dtype=torch.uint8, device=device)


def _nbytes(t: torch.Tensor | None) -> int:
    return 0 if t is None else t.numel() * t.element_size()


def _check_out(t: torch.Tensor, shape: tuple, dtype, name: str) -> None:
    """A caller-supplied output must be exactly what the kernel writes: the
    library sees only its pointer."""
    if t.dtype != dtype or not t.is_contiguous() or tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must be a contiguous {dtype} tensor of shape {tuple(shape)}")



# ---------------------------------------------------------------------------
def score_workspace_bytes(T: int, Hq: int, Hkv: int, q_pos0: int, n_vis: int) -> int:
    return int(L.load().svlm_score_workspace(T, Hq, Hkv, q_pos0, n_vis))


def score(q_text: torch.Tensor, k: torch.Tensor, q_pos0: int, n_vis: int, vis_start: int = 0,
          agg: str = "all", alpha: float = 1.0, beta: float = 0.0, out: torch.Tensor | None = None,
          scale: float | None = None, ws: torch.Tensor | None = None) -> torch.Tensor:
    """Mean text->visual attention of one layer.  q_text [T][Hq][D], k [Hkv][n_ctx][D]
    (both bf16, or both fp32 for the plain fp32 kernels)."""
    _dev(q_text, k, out, ws)
    dtype = _operands(q_text, k)
    T, Hq, D = q_text.shape
    Hkv, n_ctx, Dk = k.shape
    if Dk != D:
        raise ValueError("head dims differ")
    rows = {"qhead": Hq, "kvhead": Hkv, "all": 1}[agg]
    if out is None:
        if beta != 0.0:
            raise ValueError("beta != 0 needs an existing out")
        out = torch.empty(rows, n_vis, dtype=torch.float32, device=q_text.device)
    if out.dtype != torch.float32 or not out.is_contiguous() or tuple(out.shape) != (rows, n_vis):
        raise ValueError("out must be contiguous fp32 [rows][n_vis]")
    need = score_workspace_bytes(T, Hq, Hkv, q_pos0, n_vis)
    if ws is None:
        ws = _ws(need, q_text.device)
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    L.call("svlm_score", q_text.data_ptr(), q_text.stride(0), q_text.stride(1), k.data_ptr(), k.stride(0),
           k.stride(1), dtype, T, n_ctx, q_pos0, vis_start, n_vis, Hq, Hkv, D, float(scale), _AGG[agg],
           float(alpha), float(beta), out.data_ptr(), ws.data_ptr(), _nbytes(ws), _stream())
    return out


def score_layers_workspace_bytes(layers: int, T: int, Hq: int, Hkv: int, q_pos0: int, n_vis: int) -> int:
    return int(L.load().svlm_score_layers_workspace(layers, T, Hq, Hkv, q_pos0, n_vis))


def score_layers(q_text: torch.Tensor, k: torch.Tensor, q_pos0: int, n_vis: int, vis_start: int = 0,
                 agg: str = "all", layer_mean: bool = True, alpha: float = 1.0, beta: float = 0.0,
                 out: torch.Tensor | None = None, scale: float | None = None,
                 ws: torch.Tensor | None = None) -> torch.Tensor:
    """score() over every layer in one call.  q_text [L][T][Hq][D], k [L][Hkv][n_ctx][D].
    layer_mean: out [rows][n_vis] = the mean over layers of each layer's rows;
    otherwise out [L][rows][n_vis], one row set per layer."""
    _dev(q_text, k, out, ws)
    dtype = _operands(q_text, k)
    if q_text.dim() != 4 or k.dim() != 4 or q_text.shape[0] != k.shape[0]:
        raise ValueError("q_text must be [L][T][Hq][D] and k [L][Hkv][n_ctx][D] with the same L")
    layers, T, Hq, D = q_text.shape
    _, Hkv, n_ctx, Dk = k.shape
    if Dk != D:
        raise ValueError("head dims differ")
    rows = {"qhead": Hq, "kvhead": Hkv, "all": 1}[agg]
    shape = (rows, n_vis) if layer_mean else (layers, rows, n_vis)
    if out is None:
        if beta != 0.0:
            raise ValueError("beta != 0 needs an existing out")
        out = torch.empty(shape, dtype=torch.float32, device=q_text.device)
    if out.dtype != torch.float32 or not out.is_contiguous() or tuple(out.shape) != shape:
        raise ValueError(f"out must be contiguous fp32 {list(shape)}")
    need = score_layers_workspace_bytes(layers, T, Hq, Hkv, q_pos0, n_vis)
    if ws is None:
        ws = _ws(need, q_text.device)
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    L.call("svlm_score_layers", q_text.data_ptr(), q_text.stride(1), q_text.stride(2), q_text.stride(0),
           k.data_ptr(), k.stride(1), k.stride(2), k.stride(0), layers, dtype, T, n_ctx, q_pos0, vis_start, n_vis,
           Hq, Hkv, D, float(scale), _AGG[agg], int(bool(layer_mean)), float(alpha), float(beta), out.data_ptr(),
           ws.data_ptr(), _nbytes(ws), _stream())
    return out


# ---------------------------------------------------------------------------
def select_workspace_bytes(R: int, n_vis: int, budget: int, top_p: float) -> int:
    return int(L.load().svlm_select_workspace(R, n_vis, budget, float(top_p)))


def select(scores: torch.Tensor, F: int, H: int, W: int, top_p: float, budget: int, with_tag: bool = False,
           ws: torch.Tensor | None = None):
    """Two-stage selection per row.  scores [R][F*H*W] fp32 -> (kept [R][budget] int32, n_stage1 [R], tag).

    Pure top-K (top_p >= 1) on rows past 32768 tokens without tags runs split
    over row segments and needs select_workspace_bytes(R, n_vis, budget, top_p)
    bytes of device workspace: `ws` if given, else allocated here."""
    _dev(scores, ws)
    if scores.dtype != torch.float32 or scores.dim() != 2 or scores.stride(1) != 1:
        raise ValueError("scores must be fp32 [R][n_vis] with contiguous rows")
    R, n = scores.shape
    if F * H * W != n:
        raise ValueError(f"F*H*W = {F * H * W} must equal the row length {n}")
    dev = scores.device
    kept = torch.empty(R, budget, dtype=torch.int32, device=dev)
    n1 = torch.empty(R, dtype=torch.int32, device=dev)
    tag = torch.empty(R, n, dtype=torch.uint8, device=dev) if with_tag else None
    row_stride = scores.stride(0) if R > 1 else n
    need = 0 if with_tag else select_workspace_bytes(R, n, budget, top_p)
    if need and ws is None:
        ws = _ws(need, dev)
    L.call("svlm_select", scores.data_ptr(), row_stride, R, F, H, W, float(top_p), budget,
           kept.data_ptr(), n1.data_ptr(), tag.data_ptr() if tag is not None else None,
           ws.data_ptr() if need else None, _nbytes(ws) if need else 0, _stream())
    return kept, n1, tag


# ---------------------------------------------------------------------------
def gather_kv(k: torch.Tensor, v: torch.Tensor, idx: torch.Tensor, tail_start: int = 0, n_tail: int = 0,
              k_dst: torch.Tensor | None = None, v_dst: torch.Tensor | None = None):
    """k, v [Hkv][N][D] bf16 (or fp32); idx [n_idx] or [Hkv][n_idx] int32 -> compact [Hkv][n_idx+n_tail][D]."""
    _dev(k, v, idx, k_dst, v_dst)
    dtype = _operands(k, v)
    if k.shape != v.shape or k.stride() != v.stride():
        raise ValueError("k and v must have the same shape and strides")
    if idx.dtype != torch.int32 or idx.stride(-1) != 1:
        raise ValueError("idx must be int32 with a contiguous last axis")
    Hkv, N, D = k.shape
    n_idx = idx.shape[-1]
    idx_sh = 0 if idx.dim() == 1 else idx.stride(0)
    n_out = n_idx + n_tail
    if (k_dst is None) != (v_dst is None):
        raise ValueError("give both k_dst and v_dst, or neither")
    if k_dst is None:
        k_dst = torch.empty(Hkv, n_out, D, dtype=k.dtype, device=k.device)
        v_dst = torch.empty(Hkv, n_out, D, dtype=k.dtype, device=k.device)
    if _operands(k, v, k_dst, v_dst) != dtype:
        raise TypeError("destination dtype differs")
    if k_dst.shape != v_dst.shape or k_dst.stride() != v_dst.stride():
        raise ValueError("k_dst and v_dst must have the same shape and strides")
    if k_dst.dim() != 3 or k_dst.shape[0] != Hkv or k_dst.shape[1] < n_out or k_dst.shape[2] != D:
        raise ValueError(f"k_dst and v_dst must be [Hkv={Hkv}][>= {n_out}][D={D}]")
    if idx.dim() == 2 and idx.shape[0] != Hkv:
        raise ValueError("2-D idx must be [Hkv][n_idx]")
    L.call("svlm_gather_kv", k.data_ptr(), v.data_ptr(), k.stride(0), k.stride(1), N, idx.data_ptr(), idx_sh,
           n_idx, tail_start, n_tail, k_dst.data_ptr(), v_dst.data_ptr(), k_dst.stride(0), k_dst.stride(1), Hkv, D,
           dtype, _stream())
    return k_dst, v_dst


# ---------------------------------------------------------------------------
def decode_attn_workspace_bytes(batch, nq, Hq, Hkv, D, max_kv_len, num_splits=0) -> int:
    return int(L.load().svlm_decode_attn_workspace(batch, nq, Hq, Hkv, D, max_kv_len, num_splits))


def decode_attn(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, kv_len: torch.Tensor, causal_tail: bool,
                scale: float | None = None, num_splits: int = 0, out: torch.Tensor | None = None,
                lse: torch.Tensor | None = None, ws: torch.Tensor | None = None, want_lse: bool = True):
    """q [B][nq][Hq][D]; k, v [B][Hkv][N][D] or [Hkv][N][D]; kv_len int32 [B] -> (out fp32, lse fp32).

    q, k, v are all bf16 (matrix-core kernels) or all fp32 (plain fp32 kernels)."""
    _dev(q, k, v, kv_len, out, lse, ws)
    dtype = _operands(q, k, v)
    B, nq, Hq, D = q.shape
    if q[0].stride() != (Hq * D, D, 1):
        raise ValueError("q must be contiguous inside each batch entry")
    if k.dim() == 3:
        if B != 1:
            raise ValueError("3-D KV means batch 1")
        kv_sb = 0
        Hkv, N, _ = k.shape
        kv_sh, kv_sn = k.stride(0), k.stride(1)
    else:
        if k.dim() != 4 or k.shape[0] not in (1, B):
            raise ValueError(f"4-D k and v must be [B={B} or 1][Hkv][N][D]")
        Hkv, N = k.shape[1], k.shape[2]
        # a batch axis of 1 is shared by every batch entry (batch stride 0)
        kv_sb, kv_sh, kv_sn = k.stride(0) if k.shape[0] > 1 else 0, k.stride(1), k.stride(2)
    q_sb = q.stride(0) if B > 1 else nq * Hq * D
    if k.stride() != v.stride() or k.shape != v.shape:
        raise ValueError("k and v must have identical shapes and strides")
    if kv_len.dtype != torch.int32 or kv_len.numel() != B:
        raise ValueError("kv_len must be int32 [B]")
    if out is None:
        out = torch.empty(B, nq, Hq, D, dtype=torch.float32, device=q.device)
    _check_out(out, (B, nq, Hq, D), torch.float32, "out")
    if lse is None and want_lse:
        lse = torch.empty(B, nq, Hq, dtype=torch.float32, device=q.device)
    if lse is not None:
        _check_out(lse, (B, nq, Hq), torch.float32, "lse")
    need = decode_attn_workspace_bytes(B, nq, Hq, Hkv, D, N, num_splits) if dtype == L.SVLM_BF16 else 0
    if ws is None and need > 0:
        ws = _ws(need, q.device)
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    L.call("svlm_decode_attn", q.data_ptr(), q_sb, k.data_ptr(), v.data_ptr(), kv_sb, kv_sh, kv_sn,
           kv_len.data_ptr(), N, dtype, B, nq, Hq, Hkv, D, float(scale), 1 if causal_tail else 0,
           out.data_ptr(), lse.data_ptr() if lse is not None else None, num_splits,
           ws.data_ptr() if ws is not None else None, _nbytes(ws), _stream())
    return out, lse


def decode_attn_indexed_workspace_bytes(batch, nq, Hq, Hkv, D, max_n_idx, num_splits=0) -> int:
    return int(L.load().svlm_decode_attn_indexed_workspace(batch, nq, Hq, Hkv, D, max_n_idx, num_splits))


def decode_attn_indexed(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, kv_idx: torch.Tensor,
                        n_idx: torch.Tensor, causal_tail: bool, scale: float | None = None, num_splits: int = 0,
                        out: torch.Tensor | None = None, lse: torch.Tensor | None = None,
                        ws: torch.Tensor | None = None, want_lse: bool = True):
    """Decode attention over cache rows named by kv_idx, read in place.

    q [B][nq][Hq][D]; k, v [B][Hkv][rows][D] or [Hkv][rows][D]; kv_idx int32
    [n] (one list), [Hkv][n] (per head) or [B][Hkv][n]; n_idx int32 [B] (one
    length per batch entry) or [B][Hkv] (ragged per-head lengths) -> (out
    fp32, lse fp32).  q, k, v all bf16, or all fp32."""
    _dev(q, k, v, kv_idx, n_idx, out, lse, ws)
    dtype = _operands(q, k, v)
    B, nq, Hq, D = q.shape
    if q[0].stride() != (Hq * D, D, 1):
        raise ValueError("q must be contiguous inside each batch entry")
    if k.dim() == 3:
        if B != 1:
            raise ValueError("3-D KV means batch 1")
        kv_sb = 0
        Hkv, rows, _ = k.shape
        kv_sh, kv_sn = k.stride(0), k.stride(1)
    else:
        if k.dim() != 4 or k.shape[0] not in (1, B):
            raise ValueError(f"4-D k and v must be [B={B} or 1][Hkv][rows][D]")
        Hkv, rows = k.shape[1], k.shape[2]
        # a batch axis of 1 is shared by every batch entry (batch stride 0)
        kv_sb, kv_sh, kv_sn = k.stride(0) if k.shape[0] > 1 else 0, k.stride(1), k.stride(2)
    if k.stride() != v.stride() or k.shape != v.shape:
        raise ValueError("k and v must have identical shapes and strides")
    if kv_idx.dtype != torch.int32 or kv_idx.stride(-1) != 1:
        raise ValueError("kv_idx must be int32 with a contiguous last axis")
    if kv_idx.dim() == 1:
        idx_sb, idx_sh = 0, 0
    elif kv_idx.dim() == 2:
        if kv_idx.shape[0] != Hkv:
            raise ValueError("2-D kv_idx must be [Hkv][n]")
        idx_sb, idx_sh = 0, kv_idx.stride(0)
    else:
        if tuple(kv_idx.shape[:2]) != (B, Hkv):
            raise ValueError("3-D kv_idx must be [B][Hkv][n]")
        idx_sb, idx_sh = kv_idx.stride(0), kv_idx.stride(1)
    max_n = kv_idx.shape[-1]
    if n_idx.dtype != torch.int32 or not n_idx.is_contiguous():
        raise ValueError("n_idx must be contiguous int32")
    if tuple(n_idx.shape) == (B, Hkv) and Hkv > 1:
        n_sb, n_sh = Hkv, 1
    elif n_idx.numel() == B:
        n_sb, n_sh = 1, 0
    else:
        raise ValueError(f"n_idx must be int32 [B={B}] or [B][Hkv={Hkv}]")
    q_sb = q.stride(0) if B > 1 else nq * Hq * D
    if out is None:
        out = torch.empty(B, nq, Hq, D, dtype=torch.float32, device=q.device)
    _check_out(out, (B, nq, Hq, D), torch.float32, "out")
    if lse is None and want_lse:
        lse = torch.empty(B, nq, Hq, dtype=torch.float32, device=q.device)
    if lse is not None:
        _check_out(lse, (B, nq, Hq), torch.float32, "lse")
    need = decode_attn_indexed_workspace_bytes(B, nq, Hq, Hkv, D, max_n, num_splits) if dtype == L.SVLM_BF16 else 0
    if ws is None and need > 0:
        ws = _ws(need, q.device)
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    L.call("svlm_decode_attn_indexed", q.data_ptr(), q_sb, k.data_ptr(), v.data_ptr(), kv_sb, kv_sh, kv_sn, rows,
           kv_idx.data_ptr(), idx_sb, idx_sh, n_idx.data_ptr(), n_sb, n_sh, max_n, dtype, B, nq, Hq, Hkv, D,
           float(scale), 1 if causal_tail else 0, out.data_ptr(), lse.data_ptr() if lse is not None else None,
           num_splits, ws.data_ptr() if ws is not None else None, _nbytes(ws), _stream())
    return out, lse


# ---------------------------------------------------------------------------
def uvprune_workspace_bytes(n_text: int, d: int) -> int:
    return int(L.load().svlm_uvprune_workspace(n_text, d))


def uvprune_score(v0: torch.Tensor, vL: torch.Tensor, x0: torch.Tensor, xL: torch.Tensor,
                  out_scale: float = 1.0, out_offset: float = 0.0, out: torch.Tensor | None = None,
                  ws: torch.Tensor | None = None) -> torch.Tensor:
    """UV-Prune score.  v0, vL [n_vis][d], x0, xL [n_text][d] bf16 hidden states of
    layers 0 and L -> out [n_vis] fp32 = out_scale * dS + out_offset."""
    _dev(v0, vL, x0, xL, out, ws)
    _bf16(v0, vL, x0, xL)
    if v0.shape != vL.shape or x0.shape != xL.shape or v0.shape[1] != x0.shape[1]:
        raise ValueError("v0/vL and x0/xL must have matching shapes and the same hidden size")
    if v0.stride() != vL.stride() or x0.stride() != xL.stride() or v0.stride(1) != 1 or x0.stride(1) != 1:
        raise ValueError("rows must be contiguous, with the same strides for both layers")
    n_vis, d = v0.shape
    n_text = x0.shape[0]
    if out is None:
        out = torch.empty(n_vis, dtype=torch.float32, device=v0.device)
    _check_out(out, (n_vis,), torch.float32, "out")
    need = uvprune_workspace_bytes(n_text, d)
    if ws is None:
        ws = _ws(need, v0.device)
    L.call("svlm_uvprune_score", v0.data_ptr(), vL.data_ptr(), v0.stride(0), n_vis, x0.data_ptr(), xL.data_ptr(),
           x0.stride(0), n_text, d, L.SVLM_BF16, float(out_scale), float(out_offset), out.data_ptr(),
           ws.data_ptr(), _nbytes(ws), _stream())
    return out


# ---------------------------------------------------------------------------
def verify_workspace_bytes(batch, gamma, V) -> int:
    return int(L.load().svlm_verify_workspace(batch, gamma, V))


def verify(mode: str, draft_tok: torch.Tensor, target: torch.Tensor, draft_prob: torch.Tensor | None = None,
           u: torch.Tensor | None = None, ws: torch.Tensor | None = None):
    """mode "greedy": target = logits [B][gamma+1][V]; "reject": target = p, draft_prob = q, u [B][gamma+1].
    A caller-held `ws` (verify_workspace_bytes) must be zero-filled before its first use."""
    _dev(draft_tok, target, draft_prob, u, ws)
    B, gamma = draft_tok.shape
    V = target.shape[-1]
    if draft_tok.dtype != torch.int32 or not draft_tok.is_contiguous():
        raise ValueError("draft_tok must be contiguous int32 [B][gamma]")
    if target.dtype != torch.float32 or not target.is_contiguous() or tuple(target.shape) != (B, gamma + 1, V):
        raise ValueError("target must be contiguous fp32 [B][gamma+1][V]")
    m = {"greedy": L.SVLM_VERIFY_GREEDY, "reject": L.SVLM_VERIFY_REJECT}[mode]
    if m == L.SVLM_VERIFY_REJECT:
        if draft_prob is None or u is None:
            raise ValueError("rejection mode needs draft_prob and u")
        if tuple(draft_prob.shape) != (B, gamma, V) or not draft_prob.is_contiguous() or draft_prob.dtype != torch.float32:
            raise ValueError("draft_prob must be contiguous fp32 [B][gamma][V]")
        if tuple(u.shape) != (B, gamma + 1) or not u.is_contiguous() or u.dtype != torch.float32:
            raise ValueError("u must be contiguous fp32 [B][gamma+1]")
    n_acc = torch.empty(B, dtype=torch.int32, device=target.device)
    nxt = torch.empty(B, dtype=torch.int32, device=target.device)
    need = verify_workspace_bytes(B, gamma, V)
    if ws is None:
        # the workspace ends in arrival counters that must start at zero (every
        # call leaves them zero, so a caller-held workspace is cleared only once)
        ws = torch.zeros(max(need, 16), dtype=torch.uint8, device=target.device)
    L.call("svlm_verify", m, B, gamma, V, draft_tok.data_ptr(), target.data_ptr(),
           draft_prob.data_ptr() if draft_prob is not None else None, u.data_ptr() if u is not None else None,
           n_acc.data_ptr(), nxt.data_ptr(), ws.data_ptr(), _nbytes(ws), _stream())
    return n_acc, nxt


# ---------------------------------------------------------------------------
def stream_read(src: torch.Tensor | None, workgroups: int, sink: torch.Tensor) -> None:
    """Measurement helper: read src once in the attention kernels' access
    pattern over `workgroups` workgroups (src None: one empty workgroup)."""
    _dev(src, sink)
    if sink.dtype != torch.float32 or sink.numel() < workgroups:
        raise ValueError("sink must be fp32 with at least `workgroups` elements")
    nbytes = 0 if src is None else _nbytes(src)
    if src is not None and not src.is_contiguous():
        raise ValueError("src must be contiguous")
    L.call("svlm_stream_read", src.data_ptr() if src is not None else None, nbytes, workgroups, sink.data_ptr(),
           _stream())
