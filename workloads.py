"""Seeded synthetic inputs for the svlm calls, shared by tests, bench and smoke.

This module holds shapes, seeds and value models only.  It computes no step
of the method (no attention, no selection, no acceptance): both the HIP path
and the CPU oracle consume what it produces.

Shapes stand in for the video benchmarks the pages measure on (Video-MME,
MLVU, LVBench, LongVideoBench); none of those is used.  The token counts
follow the pages: 128 frames of 14x14 = 196 tokens each for 25,088 visual
tokens (ParallelVLM page, experimental setup), and more than 140k visual
tokens for an hour of video (Sparse-to-Dense page, problem statement).

Value model, per layer:
  * q, k, v ~ N(0, 1), then rounded to bf16 (round to nearest even);
  * the key at position 0 is scaled by 8 (an attention sink);
  * a set of "salient" visual positions gets 3 * qbar_g added to its key for
    every KV head g, where qbar_g is the mean of that group's text queries;
  * logits for acceptance are 3 * N(0, 1); draft logits add N(0, 1) noise;
    probabilities are an fp64 softmax rounded once to fp32.
Seeds: numpy PCG64 from SeedSequence(1000 * config_index, spawn_key=(tensor
id, layer)), so every tensor is reproducible on its own.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

# ---------------------------------------------------------------------------
# configurations
# ---------------------------------------------------------------------------


@dataclass(frozen=True)
class Config:
    name: str
    index: int              # seed base = 1000 * index
    layers: int
    hq: int
    hkv: int
    d: int
    frames: int
    gh: int                 # frame grid height
    gw: int                 # frame grid width
    n_text: int
    salient: str            # "c1" | "spans" | "frames"
    n_salient: int
    salient_frames: tuple = ()
    top_p: float = 0.5      # >= 1: pure top-K
    budget: int = 0
    rows: str = "all"       # score aggregation: "all" | "layer" | "layer_kvhead"
    gamma_verify: int = 4
    gamma_draft: int = 4
    vocab: int = 1024
    verify_mode: str = "greedy"  # "greedy" | "reject"
    dtype: str = "bf16"

    @property
    def n_vis(self) -> int:
        return self.frames * self.gh * self.gw

    @property
    def group(self) -> int:
        return self.hq // self.hkv

    @property
    def n_ctx(self) -> int:
        """Prefill context: visual tokens then text tokens."""
        return self.n_vis + self.n_text


def _ceil_frac(frac: float, n: int) -> int:
    return int(math.ceil(frac * n - 1e-9))


C1 = Config("tiny_ref", 1, layers=1, hq=4, hkv=2, d=64, frames=4, gh=7, gw=7, n_text=16,
            salient="c1", n_salient=4, top_p=0.5, budget=20, rows="all",
            gamma_verify=4, gamma_draft=4, vocab=1024, verify_mode="both", dtype="f32")
C2 = Config("qwen2vl7b_8k", 2, layers=28, hq=28, hkv=4, d=128, frames=32, gh=16, gw=16, n_text=64,
            salient="spans", n_salient=_ceil_frac(0.02, 8192), top_p=0.6,
            budget=_ceil_frac(0.10, 8192), rows="all", gamma_verify=9, gamma_draft=9,
            vocab=152064, verify_mode="greedy")
C3 = Config("llavaov72b_25k", 3, layers=80, hq=64, hkv=8, d=128, frames=128, gh=14, gw=14, n_text=128,
            salient="spans", n_salient=_ceil_frac(0.02, 25088), top_p=0.5,
            budget=_ceil_frac(0.10, 25088), rows="all", gamma_verify=5, gamma_draft=9,
            vocab=152064, verify_mode="reject")
C4 = Config("qwen25vl32b_20k", 4, layers=64, hq=40, hkv=8, d=128, frames=64, gh=18, gw=18, n_text=96,
            salient="frames", n_salient=_ceil_frac(0.02, 20736), salient_frames=(20, 40),
            top_p=0.5, budget=_ceil_frac(0.10, 20736), rows="layer", gamma_verify=9, gamma_draft=9,
            vocab=152064, verify_mode="reject")
C5 = Config("hour_std_141k", 5, layers=28, hq=28, hkv=4, d=128, frames=720, gh=14, gw=14, n_text=64,
            salient="spans", n_salient=_ceil_frac(0.02, 141120), top_p=1.0, budget=1024,
            rows="layer_kvhead", gamma_verify=9, gamma_draft=9, vocab=152064, verify_mode="greedy")

CONFIGS = {c.index: c for c in (C1, C2, C3, C4, C5)}

# tensor ids for the seed spawn keys
_IDS = {name: i for i, name in enumerate(
    ("q_text", "k", "v", "salient", "q_dec", "k_new", "v_new", "logits", "draft_noise",
     "draft_tok", "uniform", "scores", "misc", "span_starts", "hidden_v", "hidden_x"))}


def rng_for(cfg_index: int, name: str, layer: int = 0, extra: int = 0) -> np.random.Generator:
    ss = np.random.SeedSequence(1000 * cfg_index, spawn_key=(_IDS[name], layer, extra))
    return np.random.Generator(np.random.PCG64(ss))


# ---------------------------------------------------------------------------
# bf16 helpers (input preparation only)
# ---------------------------------------------------------------------------


def bf16_round(x: np.ndarray) -> np.ndarray:
    """Round fp32 values to the nearest bf16 (ties to even); returns fp32 holding bf16 values."""
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    rounded = (b + np.uint32(0x7FFF) + ((b >> np.uint32(16)) & np.uint32(1))) & np.uint32(0xFFFF0000)
    return rounded.view(np.float32)


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """uint16 bit patterns of an fp32 array whose values are already bf16."""
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    assert not np.any(b & np.uint32(0xFFFF)), "values are not bf16-representable"
    return (b >> np.uint32(16)).astype(np.uint16)


def _normal(rng: np.random.Generator, shape) -> np.ndarray:
    return rng.standard_normal(size=shape, dtype=np.float32)


# ---------------------------------------------------------------------------
# prefill tensors
# ---------------------------------------------------------------------------


def salient_positions(cfg: Config) -> np.ndarray:
    """Visual positions whose keys get the query-aligned shift (sorted, never 0)."""
    rng = rng_for(cfg.index, "salient")
    hw = cfg.gh * cfg.gw
    if cfg.salient == "c1":
        pool = np.arange(1, cfg.n_vis)
    elif cfg.salient == "spans":
        span = int(math.ceil(cfg.frames / 8))
        # three non-overlapping spans of `span` frames with seeded starts
        srng = rng_for(cfg.index, "span_starts")
        while True:
            starts = np.sort(srng.choice(cfg.frames - span + 1, size=3, replace=False))
            if np.all(np.diff(starts) >= span):
                break
        pool = np.concatenate([np.arange(s * hw, (s + span) * hw) for s in starts])
        pool = pool[pool != 0]
    elif cfg.salient == "frames":
        f0, f1 = cfg.salient_frames
        pool = np.arange(f0 * hw, (f1 + 1) * hw)
    else:
        raise ValueError(cfg.salient)
    return np.sort(rng.choice(pool, size=cfg.n_salient, replace=False)).astype(np.int64)


@dataclass
class Prefill:
    """One layer of prefill inputs.  q_text: [T][Hq][D]; k, v: [Hkv][n_ctx][D].

    Values are fp32 arrays holding bf16-representable numbers (except C1 kept
    in fp32 when requested)."""
    q_text: np.ndarray
    k: np.ndarray
    v: np.ndarray
    salient: np.ndarray
    q_pos0: int
    vis_start: int = 0


def prefill_layer(cfg: Config, layer: int, round_bf16: bool = True) -> Prefill:
    T, Hq, Hkv, D, G = cfg.n_text, cfg.hq, cfg.hkv, cfg.d, cfg.group
    n = cfg.n_ctx
    q = _normal(rng_for(cfg.index, "q_text", layer), (T, Hq, D))
    k = _normal(rng_for(cfg.index, "k", layer), (Hkv, n, D))
    v = _normal(rng_for(cfg.index, "v", layer), (Hkv, n, D))
    rnd = bf16_round if round_bf16 else (lambda a: a)
    q = rnd(q)
    # sink: key 0 scaled by 8, same direction
    k[:, 0, :] *= 8.0
    sal = salient_positions(cfg)
    # qbar_g: mean over the G heads of group g and the T text queries
    qbar = q.reshape(T, Hkv, G, D).astype(np.float64).mean(axis=(0, 2)).astype(np.float32)
    k[:, sal, :] += 3.0 * qbar[:, None, :]
    k = rnd(k)
    v = rnd(v)
    return Prefill(q_text=q, k=k, v=v, salient=sal, q_pos0=cfg.n_vis)


# ---------------------------------------------------------------------------
# decode tensors
# ---------------------------------------------------------------------------


def decode_queries(cfg: Config, layer: int, nq: int, batch: int = 1, extra: int = 0,
                   round_bf16: bool = True) -> np.ndarray:
    """[B][nq][Hq][D] bf16-valued fp32 queries (plain fp32 with round_bf16=False)."""
    q = _normal(rng_for(cfg.index, "q_dec", layer, extra), (batch, nq, cfg.hq, cfg.d))
    return bf16_round(q) if round_bf16 else q


def new_kv(cfg: Config, layer: int, n_new: int, extra: int = 0, round_bf16: bool = True):
    """[Hkv][n_new][D] keys and values of freshly decoded tokens."""
    rnd = bf16_round if round_bf16 else (lambda a: a)
    k = rnd(_normal(rng_for(cfg.index, "k_new", layer, extra), (cfg.hkv, n_new, cfg.d)))
    v = rnd(_normal(rng_for(cfg.index, "v_new", layer, extra), (cfg.hkv, n_new, cfg.d)))
    return k, v


def random_kv(cfg_index: int, hkv: int, n: int, d: int, layer: int = 0, extra: int = 0):
    k = bf16_round(_normal(rng_for(cfg_index, "k", layer, 1000 + extra), (hkv, n, d)))
    v = bf16_round(_normal(rng_for(cfg_index, "v", layer, 1000 + extra), (hkv, n, d)))
    return k, v


# ---------------------------------------------------------------------------
# acceptance tensors
# ---------------------------------------------------------------------------


def _softmax64(x: np.ndarray) -> np.ndarray:
    """Input preparation only: logits -> probabilities, rounded once to fp32."""
    x = x.astype(np.float64)
    x = x - x.max(axis=-1, keepdims=True)
    e = np.exp(x)
    return (e / e.sum(axis=-1, keepdims=True)).astype(np.float32)


@dataclass
class VerifyInputs:
    target_logits: np.ndarray     # [B][gamma+1][V] fp32
    draft_logits: np.ndarray      # [B][gamma][V] fp32
    p: np.ndarray                 # [B][gamma+1][V] fp32 probabilities
    q: np.ndarray                 # [B][gamma][V] fp32 probabilities
    draft_tok_greedy: np.ndarray  # [B][gamma] int32: argmax of draft logits
    draft_tok_sampled: np.ndarray  # [B][gamma] int32: sampled from q
    u: np.ndarray                 # [B][gamma+1] fp32 in [0, 1)


def verify_inputs(cfg_index: int, batch: int, gamma: int, vocab: int, extra: int = 0,
                  logit_scale: float = 3.0, noise: float = 1.0) -> VerifyInputs:
    rl = rng_for(cfg_index, "logits", 0, extra)
    tl = (logit_scale * rl.standard_normal((batch, gamma + 1, vocab))).astype(np.float32)
    rn = rng_for(cfg_index, "draft_noise", 0, extra)
    dl = (tl[:, :gamma].astype(np.float64)
          + noise * rn.standard_normal((batch, gamma, vocab))).astype(np.float32)
    p = _softmax64(tl)
    q = _softmax64(dl)
    greedy = np.argmax(dl, axis=-1).astype(np.int32)
    rd = rng_for(cfg_index, "draft_tok", 0, extra)
    sampled = np.empty((batch, gamma), np.int32)
    for b in range(batch):
        for i in range(gamma):
            w = q[b, i].astype(np.float64)
            sampled[b, i] = rd.choice(vocab, p=w / w.sum())
    u = rng_for(cfg_index, "uniform", 0, extra).random((batch, gamma + 1), dtype=np.float32)
    return VerifyInputs(tl, dl, p, q, greedy, sampled, u)


# ---------------------------------------------------------------------------
# score rows for selection tests (heavy-tailed, ties, zeros, spikes)
# ---------------------------------------------------------------------------

SCORE_KINDS = ("lognormal1", "lognormal2", "lognormal3", "pareto1.1", "ties", "zeros",
               "spike", "flat", "uniform")


def score_rows(kind: str, rows: int, n: int, seed: int = 0) -> np.ndarray:
    """[rows][n] fp32 non-negative rows, each summing to at most 1."""
    rng = rng_for(1, "scores", seed, SCORE_KINDS.index(kind))
    if kind.startswith("lognormal"):
        s = float(kind[len("lognormal"):])
        x = rng.lognormal(0.0, s, (rows, n))
    elif kind == "pareto1.1":
        x = rng.pareto(1.1, (rows, n)) + 1e-3
    elif kind == "ties":
        x = rng.integers(0, 6, (rows, n)).astype(np.float64)
    elif kind == "zeros":
        x = rng.random((rows, n))
        x[rng.random((rows, n)) < 0.7] = 0.0
    elif kind == "spike":
        x = rng.random((rows, n)) * 1e-3
        x[np.arange(rows), rng.integers(0, n, rows)] = 10.0 * n * 1e-3
    elif kind == "flat":
        x = np.ones((rows, n))
    elif kind == "uniform":
        x = rng.random((rows, n))
    else:
        raise ValueError(kind)
    x = x / np.maximum(x.sum(axis=1, keepdims=True), 1e-300)
    x = x.astype(np.float32)
    # float32 rounding can push a row sum just above 1; scale down so it stays <= 1
    over = x.astype(np.float64).sum(axis=1) > 1.0
    if np.any(over):
        x[over] = (x[over].astype(np.float64) * (1.0 - 1e-6)).astype(np.float32)
    return x


# ---------------------------------------------------------------------------
# hidden states for the UV-Prune score (layers 0 .. n_layers)
# ---------------------------------------------------------------------------

# hidden size of the model family each config is shaped like
HIDDEN = {"tiny_ref": 256, "qwen2vl7b_8k": 3584, "llavaov72b_25k": 8192, "qwen25vl32b_20k": 5120,
          "hour_std_141k": 3584}


def uv_hidden(cfg: Config, n_layers: int = 2, d_model: int | None = None, extra: int = 0):
    """Video [n_layers+1][n_vis][d] and text [n_layers+1][n_text][d] hidden states (bf16 values).

    Every vector is N(0,1) noise plus, for the text, a shared direction u; the
    salient video tokens (the same positions as the attention value model)
    drift towards u with depth (weight 3 l / n_layers at layer l), so they
    gain alignment with the text across the layers."""
    d = d_model or HIDDEN[cfg.name]
    rng_v = rng_for(cfg.index, "hidden_v", 0, extra)
    rng_x = rng_for(cfg.index, "hidden_x", 0, extra)
    u = _normal(rng_x, (d,))
    u = u / np.float32(np.sqrt(float((u.astype(np.float64) ** 2).sum()) / d))   # unit RMS direction
    sal = salient_positions(cfg)
    vs, xs = [], []
    for l in range(n_layers + 1):
        v = _normal(rng_v, (cfg.n_vis, d))
        v[sal] += np.float32(3.0 * l / n_layers) * u
        x = _normal(rng_x, (cfg.n_text, d)) + np.float32(2.0) * u
        vs.append(bf16_round(v))
        xs.append(bf16_round(x))
    return vs, xs

