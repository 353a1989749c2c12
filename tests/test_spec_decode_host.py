"""Host-side checks of the speculative-decoding driver (`spec_decode.py`):
the library calls are replaced by the fp64 oracle on the CPU, so the loop's
bookkeeping (cache appends, rollback to the verified rows, draft-cache refill,
acceptance) is exercised without a GPU.

Sparse-to-Dense explainer, "decoding process": longest matching prefix plus
one token, hence greedy speculative output equals greedy decoding.
ParallelVLM notes, "parallel decoding": rejection sampling with a target
resample on rejection; both caches are rolled back to the verified rows."""
import pytest

from tests._oracle_ops import substitute

torch = pytest.importorskip("torch")


def _setup(monkeypatch, seed=3, n_frames=4):
    from visual_kv_pruning_amd.spec_decode import TinyDecoder, Video
    substitute(monkeypatch)
    model = TinyDecoder.random(seed, layers=2, d_model=128, hq=4, hkv=2, d=64, vocab=256, device="cpu")
    g = torch.Generator().manual_seed(7)
    video = Video(n_frames, 7, 7, torch.randn(n_frames * 49, model.d_model, generator=g),
                  torch.randint(0, model.vocab, (16,), generator=g))
    return model, video


@pytest.mark.parametrize("draft_mode", ["compact", "indexed"])
@pytest.mark.parametrize("gamma", [3, 6])
def test_speculative_loop_equals_greedy_on_host(monkeypatch, gamma, draft_mode):
    from visual_kv_pruning_amd.spec_decode import greedy_dense, speculative
    model, video = _setup(monkeypatch)
    ref = greedy_dense(model, video, 24)
    got, acc = speculative(model, video, 24, gamma=gamma, keep=0.1, top_p=0.5, draft_mode=draft_mode)
    assert got == ref
    assert all(0 <= a <= gamma for a in acc)


def _prefill_rows(model, video, tokens):
    """K/V of every position of (visual, text, tokens) from one causal prefill."""
    from visual_kv_pruning_amd.spec_decode import KVCache, prefill
    x = torch.cat([video.visual, model.w["emb"][video.text], model.w["emb"][torch.tensor(tokens, dtype=torch.long)]])
    cache = KVCache.empty(model, x.shape[0], "cpu")
    prefill(model, x, cache)
    return cache


@pytest.mark.parametrize("mode", ["greedy", "reject"])
@pytest.mark.parametrize("draft_mode", ["compact", "indexed"])
def test_rollback_leaves_the_caches_of_the_emitted_text(monkeypatch, mode, draft_mode):
    """After many cycles with rejections, the full cache holds exactly the K/V
    of the prompt and the emitted tokens (all but the last, whose K/V the next
    cycle appends), as one prefill over that text gives them; the compact draft
    cache holds the kept visual rows, the text, and the same generated rows."""
    from visual_kv_pruning_amd.spec_decode import SpecDecoder
    model, video = _setup(monkeypatch)
    sd = SpecDecoder(model, video, keep=0.1, top_p=0.5, draft_mode=draft_mode, max_new=40)
    gen = torch.Generator().manual_seed(11)
    out, acc = sd.run(30, 4, mode, gen)
    assert len(out) == 30 and min(acc) < 4        # at least one rejection happened
    # run() stops after the cycle that passes 30 tokens; the caches hold its verified rows
    n_prompt = video.n_vis + video.text.shape[0]
    emitted_rows = sd.full.length - n_prompt
    assert 0 < emitted_rows
    n_cmp = n_prompt + min(emitted_rows, len(out))     # rows whose tokens run() returned
    ref = _prefill_rows(model, video, out[:n_cmp - n_prompt])
    for l in range(model.layers):
        got_k = sd.full.k[l][:, :n_cmp].float()
        want_k = ref.k[l][:, :n_cmp].float()
        # decode and prefill attention differ in rounding only: allow a bf16 ulp
        assert torch.allclose(got_k, want_k, rtol=2e-2, atol=2e-2), l
        if sd.draft is not None:
            B = sd.budget + video.text.shape[0]
            assert sd.draft.length == B + emitted_rows
            assert torch.equal(sd.draft.k[l][:, B:sd.draft.length], sd.full.k[l][:, n_prompt:sd.full.length])
            assert torch.equal(sd.draft.v[l][:, B:sd.draft.length], sd.full.v[l][:, n_prompt:sd.full.length])


def test_reject_cycle_emits_drafts_then_one_target_token(monkeypatch):
    """Every rejection-mode cycle emits its accepted drafts plus exactly one
    token, and the accepted drafts are the drafted ones."""
    from visual_kv_pruning_amd.spec_decode import SpecDecoder
    model, video = _setup(monkeypatch)
    sd = SpecDecoder(model, video, keep=0.2, top_p=0.5, max_new=64)
    gen = torch.Generator().manual_seed(5)
    tok = sd.first_token("reject", float(torch.rand(1, generator=gen)))
    seen = set()
    for _ in range(12):
        snap = sd.snapshot()
        emitted, n = sd.cycle(tok, 5, "reject", torch.rand(5, generator=gen), torch.rand(6, generator=gen))
        assert len(emitted) == n + 1 and 0 <= n <= 5
        assert sd.full.length == snap[0] + 1 + n and sd.draft.length == snap[1] + 1 + n
        seen.add(n)
        tok = emitted[-1]
    assert len(seen) >= 2
