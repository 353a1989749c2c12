"""End-to-end greedy speculative decoding with the svlm calls on a small
random decoder: the emitted tokens equal plain greedy decoding (lossless), the
draft reads only the selected visual KV, and some drafts are accepted.

Sparse-to-Dense explainer, "decoding process": the dense pass keeps the
longest matching prefix plus one token, so greedy speculative output equals
greedy decoding of the dense model."""
import pytest

from tests._util import log

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")


def _video(model, seed, frames=4, gh=7, gw=7, n_text=16):
    from visual_kv_pruning_amd.spec_decode import Video
    g = torch.Generator(device="cpu").manual_seed(seed)
    vis = torch.randn(frames * gh * gw, model.d_model, generator=g)
    text = torch.randint(0, model.vocab, (n_text,), generator=g)
    return Video(frames, gh, gw, vis.to("cuda:0"), text.to("cuda:0"))


@pytest.mark.parametrize("draft_mode", ["compact", "indexed"])
@pytest.mark.parametrize("seed,gamma", [(1, 4), (2, 9)])
def test_speculative_equals_dense_greedy(seed, gamma, draft_mode):
    """compact: gather + svlm_decode_attn over the draft cache; indexed:
    svlm_decode_attn_indexed over the full cache in place."""
    from visual_kv_pruning_amd.spec_decode import TinyDecoder, greedy_dense, speculative
    model = TinyDecoder.random(seed)
    video = _video(model, 100 + seed)
    n_new = 40
    log(f"spec decode case seed={seed} gamma={gamma} draft={draft_mode}")
    ref = greedy_dense(model, video, n_new)
    got, acc = speculative(model, video, n_new, gamma=gamma, keep=0.1, top_p=0.5, draft_mode=draft_mode)
    log(f"  accepted drafts per cycle {acc}")
    assert got == ref
    assert len(acc) >= 1 and all(0 <= a <= gamma for a in acc)
