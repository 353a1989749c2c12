"""End-to-end speculative decoding with the svlm calls on a small random
decoder, checked against the oracle.

* Greedy (Sparse-to-Dense explainer, "decoding process": longest matching
  prefix plus one token): the GPU speculative token stream equals plain greedy
  decoding driven by the fp64 oracle on the CPU (the same model and prompt,
  every library call replaced by the oracle), wherever the oracle's two
  largest logits differ by at least MARGIN.  Below that, two correct
  implementations may pick different tokens (bf16 rounding of K, V and q can
  flip on fp32 differences of the projections), so the comparison stops at
  the first such step; every case is chosen so that it covers at least
  MIN_PREFIX tokens.
* Parallel decoding (ParallelVLM notes, "parallel decoding"): the draft of the
  next window overlapped with the verify pass, fixed and adaptive windows
  (gamma = c* = T_p / T_q), gives the same tokens.
* Rejection sampling (ParallelVLM notes, background): over many seeded cycles
  from one state, the first emitted token is distributed as the target's p
  (chi-square), for serial and parallel decoding."""
import math

import numpy as np
import pytest

from tests._oracle_ops import substitute
from tests._util import log

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")

MARGIN = 5e-3       # logits; smaller gaps may legitimately resolve either way
MIN_PREFIX = 16
N_NEW = 40


def _video(model, seed, device, frames=4, gh=7, gw=7, n_text=16):
    from visual_kv_pruning_amd.spec_decode import Video
    g = torch.Generator(device="cpu").manual_seed(seed)
    vis = torch.randn(frames * gh * gw, model.d_model, generator=g)
    text = torch.randint(0, model.vocab, (n_text,), generator=g)
    return Video(frames, gh, gw, vis.to(device), text.to(device))


_REF = {}


def _oracle_greedy(seed):
    """Plain greedy decoding of the model on the CPU with the oracle in place
    of every library call: (tokens, top-2 logit margins)."""
    if seed not in _REF:
        from visual_kv_pruning_amd.spec_decode import TinyDecoder, greedy_dense
        mp = pytest.MonkeyPatch()
        try:
            substitute(mp)
            model = TinyDecoder.random(seed, device="cpu")
            margins = []
            toks = greedy_dense(model, _video(model, 100 + seed, "cpu"), N_NEW, margins)
        finally:
            mp.undo()
        _REF[seed] = (toks, margins)
    return _REF[seed]


def _compare(got, seed, name):
    ref, margins = _oracle_greedy(seed)
    n_cmp = next((i for i, m in enumerate(margins) if m < MARGIN), len(ref))
    assert n_cmp >= MIN_PREFIX, f"seed {seed}: near-tie at token {n_cmp}; pick another seed"
    log(f"  {name}: {n_cmp} tokens compared with the oracle (smallest margin there "
        f"{min(margins[:n_cmp]):.3g})")
    assert got[:n_cmp] == ref[:n_cmp], name


def _model(seed):
    from visual_kv_pruning_amd.spec_decode import TinyDecoder
    model = TinyDecoder.random(seed)
    return model, _video(model, 100 + seed, "cuda:0")


@pytest.mark.parametrize("draft_mode", ["compact", "indexed"])
@pytest.mark.parametrize("seed,gamma", [(1, 4), (2, 9)])
def test_speculative_equals_oracle_greedy(seed, gamma, draft_mode):
    """compact: gather + svlm_decode_attn over the draft cache; indexed:
    svlm_decode_attn_indexed over the full cache in place."""
    from visual_kv_pruning_amd.spec_decode import greedy_dense, speculative
    model, video = _model(seed)
    log(f"spec decode case seed={seed} gamma={gamma} draft={draft_mode}")
    got, acc = speculative(model, video, N_NEW, gamma=gamma, keep=0.1, top_p=0.5, draft_mode=draft_mode)
    log(f"  accepted drafts per cycle {acc}")
    _compare(got, seed, "speculative")
    _compare(greedy_dense(model, video, N_NEW), seed, "GPU dense greedy")
    assert len(acc) >= 1 and all(0 <= a <= gamma for a in acc)
    assert sum(acc) > 0


@pytest.mark.parametrize("gamma", [3, "adaptive"])
def test_parallel_decoding_equals_oracle_greedy(gamma):
    from visual_kv_pruning_amd.spec_decode import SpecDecoder
    seed = 1
    model, video = _model(seed)
    log(f"spec decode case parallel gamma={gamma}")
    sd = SpecDecoder(model, video, keep=0.1, top_p=0.5, max_new=N_NEW)
    got, acc, windows = sd.run_parallel(N_NEW, gamma)
    log(f"  windows {windows}, accepted {acc}")
    _compare(got, seed, f"parallel gamma={gamma}")
    assert all(0 <= a <= w for a, w in zip(acc, windows))
    if gamma == "adaptive":
        assert all(2 - 1 <= w <= 16 for w in windows)


def _chi2_first_token(draw, p, trials, name):
    """Chi-square of the first emitted token against p over `trials` draws:
    bins with an expected count >= 5, the rest pooled.  Returns the p-value."""
    from scipy.stats import chi2
    counts = np.zeros(p.size)
    for i in range(trials):
        counts[draw(i)] += 1
    exp = p * trials
    big = exp >= 5
    obs = np.append(counts[big], counts[~big].sum())
    ex = np.append(exp[big], exp[~big].sum())
    keep = ex > 0
    stat = float(((obs[keep] - ex[keep]) ** 2 / ex[keep]).sum())
    dof = int(keep.sum()) - 1
    pv = float(chi2.sf(stat, dof))
    log(f"  {name}: chi2 {stat:.1f} on {dof} dof, p-value {pv:.3f}")
    return pv


@pytest.mark.parametrize("parallel", [False, True])
def test_rejection_sampling_first_token_distributed_as_target(parallel):
    """One state, 1500 seeded cycles (gamma 4): the first token each cycle
    emits (the first draft if accepted, else the resample from max(0, p - q))
    follows the target's next-token distribution p."""
    from visual_kv_pruning_amd.spec_decode import SpecDecoder, decode, probs
    seed = 3
    model, video = _model(seed)
    log(f"spec decode case rejection chi2 parallel={parallel}")
    sd = SpecDecoder(model, video, keep=0.1, top_p=0.5, max_new=64)
    tok = sd.first_token("greedy")
    snap = sd.snapshot()
    p = probs(decode(model, torch.tensor([tok], device="cuda:0"), sd.full)[0]).double().cpu().numpy()
    sd.restore(snap)
    p = p / p.sum()
    gen = torch.Generator(device="cuda:0").manual_seed(1234)
    gamma = 4

    def draw(i):
        sd.restore(snap)
        if not parallel:
            emitted, _ = sd.cycle(tok, gamma, "reject", torch.rand(gamma, generator=gen, device="cuda:0"),
                                  torch.rand(gamma + 1, generator=gen, device="cuda:0"))
            return emitted[0]
        out, _, _ = sd.run_parallel(2, gamma, "reject", gen, start_tok=tok)
        return out[1]

    pv = _chi2_first_token(draw, p, 1500, "serial" if not parallel else "parallel")
    assert pv > 1e-3
