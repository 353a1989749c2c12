"""End-to-end speculative decoding with the svlm calls on a small random decoder.

A lossless-decoding check of the whole path, not a model: a decoder with
random weights (no RoPE; positions enter only through the causal limit) runs

  prefill (plain torch attention, once)
  -> svlm_score per layer, averaged into one row
  -> svlm_select (Top-P on score mass, then the spatially uniform fill)
  -> svlm_gather_kv per layer into the draft cache (kept visual rows + text),
     or, with draft_mode="indexed", no copy: the draft reads the full cache in
     place through the key list with svlm_decode_attn_indexed
  -> cycles: gamma draft steps with svlm_decode_attn over the draft cache,
           one dense verify pass with svlm_decode_attn (gamma + 1 queries,
           causal tail) over the full cache, svlm_verify acceptance (greedy,
           or rejection sampling on probabilities), then both caches are cut
           back to the verified rows (rollback).

Sparse-to-Dense explainer, "dual-module architecture" and "decoding process":
the draft is the same model reading only the selected KV; the dense module
verifies all drafted tokens in one pass over the full cache and keeps the
longest matching prefix plus one token, so greedy output equals plain greedy
decoding.  ParallelVLM notes, background and "parallel decoding": acceptance by
rejection sampling keeps the target's distribution, a rejected token is
resampled from the target; in parallel decoding the draft writes the next
window while the target verifies the current one, a rejection discards the
pre-drafted window ("pre-rollback"), and the window size is the speed ratio
c* = T_p / T_q of a target pass to a draft step.  SpecVLM abstract and
technology-transfer listing, section 5: the selection of the visual KV from
the target's text-to-visual attention.

Attention on the decode path runs in the library's kernels; the projections,
norms, MLP, softmax of the logits and the draft's own sampling are plain torch
on the GPU (they are the model, not the path).
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


def greedy_dense(model: TinyDecoder, video: Video, n_new: int, margins: list | None = None) -> list:
    """Plain greedy decoding, one token per step over the full cache.  With
    `margins`, the gap between the two largest logits of every step is
    appended to it (a near-tie is where two correct implementations may pick
    different tokens)."""
    dev = video.text.device
    N = video.n_vis + video.text.shape[0]
    cache = KVCache.empty(model, N + n_new + 1, dev)
    x = torch.cat([video.visual, model.w["emb"][video.text]])
    logits, _ = prefill(model, x, cache)

    def pick(lg):
        if margins is not None:
            top = torch.topk(lg.double(), 2).values
            margins.append(float(top[0] - top[1]))
        return int(lg.argmax())

    tok = pick(logits[0])
    out = [tok]
    while len(out) < n_new:
        tok = pick(decode(model, torch.tensor([tok], device=dev), cache)[0])
        out.append(tok)
    return out


def probs(logits: torch.Tensor) -> torch.Tensor:
    """Next-token probabilities at temperature 1: an fp64 softmax rounded once
    to fp32, so the acceptance sees exactly the p and q the sampler used."""
    return torch.softmax(logits.double(), dim=-1).float()


def _sample(prob: torch.Tensor, u: torch.Tensor) -> torch.Tensor:
    """The draft's own draw from one probability row with uniform u (device
    tensors; inverse CDF in fp64).  Any exact sampler keeps decoding lossless."""
    c = torch.cumsum(prob.double(), 0)
    t = torch.searchsorted(c, (u.double() * c[-1]).reshape(1), right=True)
    return t.clamp_(max=prob.shape[0] - 1)


class SpecDecoder:
    """One request's speculative-decoding state: the full (target) cache, the
    draft's view of the KV (a compact cache or a key list into the full cache)
    and the token whose K/V is not yet in the caches.

    cycle() runs one draft-then-verify round; run() decodes n_new tokens with
    cycles one after the other, run_parallel() with the draft of the next
    window overlapped with the verify pass of the current one."""

    def __init__(self, model: TinyDecoder, video: Video, keep: float, top_p: float, draft_mode: str = "compact",
                 max_new: int = 256, gamma_max: int = 16):
        if draft_mode not in ("compact", "indexed"):
            raise ValueError(f"unknown draft_mode {draft_mode!r}")
        self.model, self.video, self.draft_mode = model, video, draft_mode
        self.dev = dev = video.text.device
        T = video.text.shape[0]
        n_vis = self.n_vis = video.n_vis
        N = n_vis + T
        self.cap = cap = N + max_new + 2 * gamma_max + 4
        self.full = KVCache.empty(model, cap, dev)
        x = torch.cat([video.visual, model.w["emb"][video.text]])
        logits, qs = prefill(model, x, self.full)
        self.first_logits = logits[0]

        # selection from the target's mean text-to-visual attention over all layers and heads
        row = torch.empty(1, n_vis, dtype=torch.float32, device=dev)
        for l in range(model.layers):
            ops.score(qs[l][n_vis:].to(torch.bfloat16).contiguous(), self.full.k[l][:, :N], n_vis, n_vis,
                      agg="all", alpha=1.0 / model.layers, beta=0.0 if l == 0 else 1.0, out=row)
        self.budget = budget = math.ceil(keep * n_vis)
        kept, _, _ = ops.select(row, video.frames, video.gh, video.gw, top_p, budget)
        self.kept = kept[0]
        self.draft = None
        if draft_mode == "indexed":
            # list entry budget + j names row n_vis + j (text, then generated tokens)
            self.lst = torch.cat([kept[0], torch.arange(n_vis, cap, dtype=torch.int32, device=dev)])
        else:
            self.draft = KVCache.empty(model, budget + T + max_new + 2 * gamma_max + 4, dev)
            for l in range(model.layers):
                ops.gather_kv(self.full.k[l][:, :N], self.full.v[l][:, :N], kept[0], n_vis, T,
                              self.draft.k[l][:, :budget + T], self.draft.v[l][:, :budget + T])
            self.draft.length = budget + T

    # -- state --------------------------------------------------------------
    def snapshot(self):
        """Cache lengths: rows past them are rewritten before they are read, so
        restoring the lengths restores the state."""
        return self.full.length, (self.draft.length if self.draft is not None else 0)

    def restore(self, snap) -> None:
        self.full.length = snap[0]
        if self.draft is not None:
            self.draft.length = snap[1]

    # -- the two modules ------------------------------------------------------
    def _draft_step(self, tok: torch.Tensor) -> torch.Tensor:
        """One draft token position: appends tok's draft K/V, returns logits [vocab]."""
        if self.draft_mode == "indexed":
            n_idx = self.budget + self.full.length + 1 - self.n_vis
            return decode_draft_indexed(self.model, tok, self.full, self.lst, n_idx)[0]
        return decode(self.model, tok, self.draft)[0]

    def draft_window(self, x_last: torch.Tensor, gamma: int, mode: str, u: torch.Tensor | None = None):
        """gamma draft tokens after x_last (device [1] int64): argmax (greedy) or
        drawn from q with uniforms u [gamma] (reject).  Appends the draft K/V of
        x_last and the first gamma - 1 tokens.  Returns (tokens [gamma] int64,
        q [gamma][vocab] fp32 or None), both on the device, with no host sync."""
        toks, qs = [], []
        t = x_last
        for j in range(gamma):
            lg = self._draft_step(t)
            if mode == "greedy":
                t = lg.argmax().reshape(1)
            else:
                q = probs(lg)
                qs.append(q)
                t = _sample(q, u[j])
            toks.append(t)
        return torch.cat(toks), (torch.stack(qs) if qs else None)

    def verify(self, x_last: torch.Tensor, window: torch.Tensor, mode: str, q: torch.Tensor | None = None,
               u: torch.Tensor | None = None):
        """The dense pass over [x_last] + window on the full cache (appending
        their K/V) and the acceptance.  Returns device (n_accept [1], next [1])."""
        lv = decode(self.model, torch.cat([x_last, window]), self.full)      # [gamma + 1][vocab]
        d = window.to(torch.int32)[None]
        if mode == "greedy":
            return ops.verify("greedy", d, lv[None].contiguous())
        return ops.verify("reject", d, probs(lv)[None].contiguous(), q[None].contiguous(), u.reshape(1, -1))

    def commit(self, f0: int, d0: int, n: int) -> None:
        """Keep x_last and the n accepted tokens: the full cache is cut back to
        them (rollback), and the draft cache takes the target's K/V rows of them."""
        self.full.length = f0 + 1 + n
        if self.draft is not None:
            for l in range(self.model.layers):
                self.draft.k[l][:, d0:d0 + 1 + n] = self.full.k[l][:, f0:f0 + 1 + n]
                self.draft.v[l][:, d0:d0 + 1 + n] = self.full.v[l][:, f0:f0 + 1 + n]
            self.draft.length = d0 + 1 + n

    def cycle(self, x_last: int, gamma: int, mode: str = "greedy", u_draft: torch.Tensor | None = None,
              u_accept: torch.Tensor | None = None):
        """One draft-then-verify round from x_last.  Returns (emitted tokens, n accepted)."""
        f0, d0 = self.snapshot()
        xt = torch.tensor([x_last], device=self.dev)
        win, q = self.draft_window(xt, gamma, mode, u_draft)
        self.full.length = f0          # the draft's rows (indexed mode) are rewritten by the verify pass
        n_acc, nxt = self.verify(xt, win, mode, q, u_accept)
        n, nx = int(n_acc[0]), int(nxt[0])
        self.commit(f0, d0, n)
        return win[:n].tolist() + [nx], n

    def first_token(self, mode: str, u: float | None = None) -> int:
        if mode == "greedy":
            return int(self.first_logits.argmax())
        return int(_sample(probs(self.first_logits), torch.tensor(u, device=self.dev)))

    # -- decoding loops ---------------------------------------------------------
    def run(self, n_new: int, gamma: int, mode: str = "greedy", gen: torch.Generator | None = None,
            start_tok: int | None = None):
        """Serial cycles, from the prefill's next token (or start_tok, whose K/V
        is not yet in the caches).  Returns (tokens, accepted per cycle)."""
        rand = lambda n: torch.rand(n, generator=gen, device=self.dev)
        tok = start_tok if start_tok is not None else \
            self.first_token(mode, None if mode == "greedy" else float(rand(1)))
        out, accepted = [tok], []
        while len(out) < n_new:
            ud, ua = (None, None) if mode == "greedy" else (rand(gamma), rand(gamma + 1))
            emitted, n = self.cycle(tok, gamma, mode, ud, ua)
            accepted.append(n)
            out.extend(emitted)
            tok = out[-1]
        return out[:n_new], accepted

    def run_parallel(self, n_new: int, gamma, mode: str = "greedy", gen: torch.Generator | None = None,
                     gamma_max: int = 16, start_tok: int | None = None):
        """Parallel decoding (ParallelVLM notes, "parallel decoding"), compact
        draft cache only: while the target verifies the window W after x_last
        (on the current stream), the draft already writes the next window after
        W's last token (on a second stream).  If every token of W is accepted
        and the target's next token equals the pre-drafted one, the rest of the
        pre-drafted window is the next window; otherwise it is discarded
        (pre-rollback) and the draft restarts from the target's token.
        gamma: an int, or "adaptive": every round's next window takes
        c* = T_p / T_q, the measured verify time over the measured time per
        draft step (at least 2, at most gamma_max).  Starts from the prefill's
        next token, or from start_tok.
        Returns (tokens, accepted per round, window sizes used)."""
        if self.draft is None:
            raise ValueError("parallel decoding needs the compact draft cache (draft_mode='compact')")
        adaptive = gamma == "adaptive"
        g = 4 if adaptive else int(gamma)
        if g < 2:
            raise ValueError("parallel decoding drafts ahead at least 2 tokens per window")
        dev = self.dev
        rand = lambda n: torch.rand(n, generator=gen, device=dev)
        main = torch.cuda.current_stream(dev)
        side = torch.cuda.Stream(device=dev)
        tok = start_tok if start_tok is not None else \
            self.first_token(mode, None if mode == "greedy" else float(rand(1)))
        out, accepted, windows = [tok], [], []
        xt = torch.tensor([tok], device=dev)
        win, q = self.draft_window(xt, g, mode, None if mode == "greedy" else rand(g))
        while len(out) < n_new:
            f0 = self.full.length
            d0 = self.draft.length - win.numel()         # rows of x_last and win[:-1] follow the committed ones
            ua = None if mode == "greedy" else rand(win.numel() + 1)
            ud = None if mode == "greedy" else rand(g)
            ready = torch.cuda.Event()
            ready.record(main)
            t_v = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
            t_d = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
            t_v[0].record(main)
            n_acc, nxt = self.verify(xt, win, mode, q, ua)
            t_v[1].record(main)
            side.wait_event(ready)
            with torch.cuda.stream(side):
                t_d[0].record(side)
                nwin, nq = self.draft_window(win[-1:], g, mode, ud)
                t_d[1].record(side)
            main.wait_stream(side)
            # made on the side stream, used on this one from here on
            nwin.record_stream(main)
            if nq is not None:
                nq.record_stream(main)
            n, nx = int(n_acc[0]), int(nxt[0])
            windows.append(win.numel())
            accepted.append(n)
            out.extend(win[:n].tolist() + [nx])
            full_accept = n == win.numel()
            self.commit(f0, d0, n)
            if full_accept and int(nwin[0]) == nx:
                # the pre-drafted window continues the emitted text: its draft
                # rows for nx and nwin[1:-1] already follow the committed rows
                self.draft.length = d0 + 1 + n + (g - 1)
                xt, win, q = nwin[:1], nwin[1:], (nq[1:] if nq is not None else None)
            else:
                xt = torch.tensor([nx], device=dev)
                win, q = self.draft_window(xt, g, mode, None if mode == "greedy" else rand(g))
            if adaptive:
                t_p = t_v[0].elapsed_time(t_v[1])
                t_q = t_d[0].elapsed_time(t_d[1]) / g
                g = int(min(gamma_max, max(2, round(t_p / max(t_q, 1e-6)))))
        return out[:n_new], accepted, windows


def speculative(model: TinyDecoder, video: Video, n_new: int, gamma: int, keep: float, top_p: float,
                draft_mode: str = "compact", mode: str = "greedy", gen: torch.Generator | None = None):
    """Speculative decoding with a pruned-KV self-draft, cycles one after the
    other.  draft_mode "compact" gathers the kept KV into a draft cache;
    "indexed" reads it in place from the full cache through the key list.
    mode "greedy" or "reject" (rejection sampling at temperature 1, uniforms
    from `gen`).  Returns the tokens and per-cycle accepted-draft counts."""
    sd = SpecDecoder(model, video, keep, top_p, draft_mode, max_new=n_new, gamma_max=max(16, gamma))
    return sd.run(n_new, gamma, mode, gen)
