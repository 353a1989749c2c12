"""End-to-end speculative decoding with the svlm calls on a small random decoder.

A lossless-decoding check of the whole path, not a model: a decoder with
random weights (no RoPE; positions enter only through the causal limit) runs

  prefill (plain torch attention, once)
  -> svlm_score per layer, averaged into one row
  -> svlm_select (Top-P on score mass, then the spatially uniform fill)
  -> svlm_gather_kv per layer into the draft cache (kept visual rows + text),
     or, with draft_mode="indexed", no copy: the draft reads the full cache in
     place through the key list with svlm_decode_attn_indexed
  -> loop: gamma draft steps with svlm_decode_attn over the draft cache,
           one dense verify pass with svlm_decode_attn (gamma + 1 queries,
           causal tail) over the full cache, svlm_verify greedy acceptance,
           then the full cache is cut back to the accepted length and the
           draft cache takes the target's K/V rows of the accepted tokens.

Sparse-to-Dense explainer, "dual-module architecture" and "decoding process":
the draft is the same model reading only the selected KV; the dense module
verifies all drafted tokens in one pass over the full cache and keeps the
longest matching prefix plus one token, so greedy output equals plain greedy
decoding.  SpecVLM abstract and technology-transfer listing, section 5: the
selection of the visual KV from the target's text-to-visual attention.

Attention on the decode path runs in the library's kernels; the projections,
norms and MLP are plain torch on the GPU (they are the model, not the path).
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import torch

from . import ops


@dataclass
class TinyDecoder:
    layers: int
    d_model: int
    hq: int
    hkv: int
    d: int
    vocab: int
    w: dict = field(default_factory=dict)

    @staticmethod
    def random(seed: int, layers: int = 2, d_model: int = 256, hq: int = 4, hkv: int = 2, d: int = 64,
               vocab: int = 512, device: str = "cuda:0") -> "TinyDecoder":
        g = torch.Generator(device="cpu").manual_seed(seed)

        def mat(rows, cols, scale):
            return (torch.randn(rows, cols, generator=g) * scale).to(device)

        m = TinyDecoder(layers, d_model, hq, hkv, d, vocab)
        s = 1.0 / math.sqrt(d_model)
        m.w["emb"] = mat(vocab, d_model, 1.0)
        m.w["lm"] = mat(d_model, vocab, s)
        for l in range(layers):
            m.w[f"q{l}"] = mat(d_model, hq * d, s)
            m.w[f"k{l}"] = mat(d_model, hkv * d, s)
            m.w[f"v{l}"] = mat(d_model, hkv * d, s)
            m.w[f"o{l}"] = mat(hq * d, d_model, 1.0 / math.sqrt(hq * d))
            m.w[f"up{l}"] = mat(d_model, 2 * d_model, s)
            m.w[f"dn{l}"] = mat(2 * d_model, d_model, 1.0 / math.sqrt(2 * d_model))
        return m


def _rms(x: torch.Tensor) -> torch.Tensor:
    return x * torch.rsqrt((x * x).mean(-1, keepdim=True) + 1e-6)


@dataclass
class KVCache:
    """Per-layer K and V, [Hkv][capacity][D] bf16, and the filled length."""
    k: list
    v: list
    length: int = 0

    @staticmethod
    def empty(model: TinyDecoder, capacity: int, device) -> "KVCache":
        shape = (model.hkv, capacity, model.d)
        return KVCache([torch.zeros(shape, dtype=torch.bfloat16, device=device) for _ in range(model.layers)],
                       [torch.zeros(shape, dtype=torch.bfloat16, device=device) for _ in range(model.layers)])


def prefill(model: TinyDecoder, x: torch.Tensor, cache: KVCache):
    """Causal prefill of inputs x [N][d_model] (plain torch attention over the
    bf16-rounded K/V the cache keeps).  Fills cache rows [0, N); returns the
    last position's logits and, per layer, the queries [N][Hq][D]."""
    N = x.shape[0]
    G = model.hq // model.hkv
    h = x
    qs = []
    mask = torch.ones(N, N, dtype=torch.bool, device=x.device).tril()
    for l in range(model.layers):
        a = _rms(h)
        q = (a @ model.w[f"q{l}"]).view(N, model.hq, model.d)
        k = (a @ model.w[f"k{l}"]).view(N, model.hkv, model.d).to(torch.bfloat16)
        v = (a @ model.w[f"v{l}"]).view(N, model.hkv, model.d).to(torch.bfloat16)
        cache.k[l][:, :N] = k.transpose(0, 1)
        cache.v[l][:, :N] = v.transpose(0, 1)
        qs.append(q)
        kf = k.float().repeat_interleave(G, dim=1)          # [N][Hq][D]
        vf = v.float().repeat_interleave(G, dim=1)
        s = torch.einsum("nhd,mhd->hnm", q.to(torch.bfloat16).float(), kf) / math.sqrt(model.d)
        s = s.masked_fill(~mask, float("-inf"))
        o = torch.einsum("hnm,mhd->nhd", torch.softmax(s, dim=-1), vf).reshape(N, model.hq * model.d)
        h = h + o @ model.w[f"o{l}"]
        h = h + torch.relu(_rms(h) @ model.w[f"up{l}"]) @ model.w[f"dn{l}"]
    cache.length = N
    return _rms(h[-1:]) @ model.w["lm"], qs


def decode(model: TinyDecoder, tokens: torch.Tensor, cache: KVCache) -> torch.Tensor:
    """Runs n = len(tokens) new positions against `cache` (appending their K/V
    at cache.length) with svlm_decode_attn; n > 1 is a dense verify pass with
    the causal tail.  Returns logits [n][vocab]; cache.length grows by n."""
    n = tokens.shape[0]
    p0 = cache.length
    kv_len = torch.tensor([p0 + n], dtype=torch.int32, device=tokens.device)
    h = model.w["emb"][tokens]
    for l in range(model.layers):
        a = _rms(h)
        q = (a @ model.w[f"q{l}"]).view(1, n, model.hq, model.d).to(torch.bfloat16)
        cache.k[l][:, p0:p0 + n] = (a @ model.w[f"k{l}"]).view(n, model.hkv, model.d).to(torch.bfloat16).transpose(0, 1)
        cache.v[l][:, p0:p0 + n] = (a @ model.w[f"v{l}"]).view(n, model.hkv, model.d).to(torch.bfloat16).transpose(0, 1)
        o, _ = ops.decode_attn(q, cache.k[l][:, :p0 + n], cache.v[l][:, :p0 + n], kv_len, n > 1, want_lse=False)
        h = h + o.view(n, model.hq * model.d) @ model.w[f"o{l}"]
        h = h + torch.relu(_rms(h) @ model.w[f"up{l}"]) @ model.w[f"dn{l}"]
    cache.length = p0 + n
    return _rms(h) @ model.w["lm"]


def decode_draft_indexed(model: TinyDecoder, token: torch.Tensor, full: KVCache, lst: torch.Tensor,
                         n_idx: int) -> torch.Tensor:
    """One draft step that reads the full cache in place: the token's K/V go to
    row full.length (the verify pass rewrites that row), and attention runs
    with svlm_decode_attn_indexed over the first n_idx rows named by `lst`
    (kept visual rows, then every row from the text on, this one included).
    Returns logits [1][vocab]; full.length grows by one."""
    p0 = full.length
    nt = torch.tensor([n_idx], dtype=torch.int32, device=token.device)
    h = model.w["emb"][token]
    for l in range(model.layers):
        a = _rms(h)
        q = (a @ model.w[f"q{l}"]).view(1, 1, model.hq, model.d).to(torch.bfloat16)
        full.k[l][:, p0] = (a @ model.w[f"k{l}"]).view(model.hkv, model.d).to(torch.bfloat16)
        full.v[l][:, p0] = (a @ model.w[f"v{l}"]).view(model.hkv, model.d).to(torch.bfloat16)
        o, _ = ops.decode_attn_indexed(q, full.k[l], full.v[l], lst, nt, False, want_lse=False)
        h = h + o.view(1, model.hq * model.d) @ model.w[f"o{l}"]
        h = h + torch.relu(_rms(h) @ model.w[f"up{l}"]) @ model.w[f"dn{l}"]
    full.length = p0 + 1
    return _rms(h) @ model.w["lm"]


@dataclass
class Video:
    """A prompt of F x H x W visual embeddings followed by T text tokens."""
    frames: int
    gh: int
    gw: int
    visual: torch.Tensor      # [F*H*W][d_model]
    text: torch.Tensor        # [T] token ids

    @property
    def n_vis(self) -> int:
        return self.frames * self.gh * self.gw


def greedy_dense(model: TinyDecoder, video: Video, n_new: int) -> list:
    """Plain greedy decoding, one token per step over the full cache."""
    dev = video.text.device
    N = video.n_vis + video.text.shape[0]
    cache = KVCache.empty(model, N + n_new + 1, dev)
    x = torch.cat([video.visual, model.w["emb"][video.text]])
    logits, _ = prefill(model, x, cache)
    tok = int(logits[0].argmax())
    out = [tok]
    while len(out) < n_new:
        tok = int(decode(model, torch.tensor([tok], device=dev), cache)[0].argmax())
        out.append(tok)
    return out


def speculative(model: TinyDecoder, video: Video, n_new: int, gamma: int, keep: float, top_p: float,
                draft_mode: str = "compact"):
    """Greedy speculative decoding with a pruned-KV self-draft.  draft_mode
    "compact" gathers the kept KV into a draft cache; "indexed" reads it in
    place from the full cache through the key list.  Returns the tokens and
    per-cycle accepted-draft counts."""
    if draft_mode not in ("compact", "indexed"):
        raise ValueError(f"unknown draft_mode {draft_mode!r}")
    dev = video.text.device
    T = video.text.shape[0]
    n_vis = video.n_vis
    N = n_vis + T
    cap = N + n_new + gamma + 2
    full = KVCache.empty(model, cap, dev)
    x = torch.cat([video.visual, model.w["emb"][video.text]])
    logits, qs = prefill(model, x, full)

    # selection from the target's mean text-to-visual attention over all layers and heads
    row = torch.empty(1, n_vis, dtype=torch.float32, device=dev)
    for l in range(model.layers):
        ops.score(qs[l][n_vis:].to(torch.bfloat16).contiguous(), full.k[l][:, :N], n_vis, n_vis, agg="all",
                  alpha=1.0 / model.layers, beta=0.0 if l == 0 else 1.0, out=row)
    budget = math.ceil(keep * n_vis)
    kept, _, _ = ops.select(row, video.frames, video.gh, video.gw, top_p, budget)
    if draft_mode == "indexed":
        # list entry budget + j names row n_vis + j (text, then generated tokens)
        lst = torch.cat([kept[0], torch.arange(n_vis, cap, dtype=torch.int32, device=dev)])
    else:
        draft = KVCache.empty(model, budget + T + n_new + gamma + 2, dev)
        for l in range(model.layers):
            ops.gather_kv(full.k[l][:, :N], full.v[l][:, :N], kept[0], n_vis, T,
                          draft.k[l][:, :budget + T], draft.v[l][:, :budget + T])
        draft.length = budget + T

    tok = int(logits[0].argmax())
    out = [tok]
    accepted = []
    while len(out) < n_new:
        f0 = full.length
        d0 = draft.length if draft_mode == "compact" else 0
        drafts = []
        t = tok
        for _ in range(gamma):
            tt = torch.tensor([t], device=dev)
            if draft_mode == "indexed":
                lg = decode_draft_indexed(model, tt, full, lst, budget + full.length + 1 - n_vis)
            else:
                lg = decode(model, tt, draft)
            t = int(lg[0].argmax())
            drafts.append(t)
        full.length = f0          # the draft's rows are rewritten by the verify pass
        vt = torch.tensor([tok] + drafts, dtype=torch.int64, device=dev)
        lv = decode(model, vt, full)                                   # [gamma + 1][vocab]
        n_acc, nxt = ops.verify("greedy", torch.tensor([drafts], dtype=torch.int32, device=dev),
                                lv[None].contiguous())
        n = int(n_acc[0])
        # keep the verified rows (tok and the accepted drafts) in both caches
        full.length = f0 + 1 + n
        if draft_mode == "compact":
            for l in range(model.layers):
                draft.k[l][:, d0:d0 + 1 + n] = full.k[l][:, f0:f0 + 1 + n]
                draft.v[l][:, d0:d0 + 1 + n] = full.v[l][:, f0:f0 + 1 + n]
            draft.length = d0 + 1 + n
        accepted.append(n)
        tok = int(nxt[0])
        out.extend(drafts[:n] + [tok])
    return out[:n_new], accepted
