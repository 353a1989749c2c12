"""Host-side check of the speculative-decoding driver (`spec_decode.py`): the
library calls are replaced by the fp64 oracle on the CPU, so the loop's
bookkeeping (cache appends, rollback to the verified rows, draft-cache
refill, acceptance) is exercised without a GPU.  The emitted tokens must
equal plain greedy decoding with the same substitutes.

Sparse-to-Dense explainer, "decoding process": longest matching prefix plus
one token, hence greedy speculative output equals greedy decoding."""
import numpy as np
import pytest

import oracle

torch = pytest.importorskip("torch")


def _substitutes(monkeypatch):
    from visual_kv_pruning_amd import ops

    def decode_attn(q, k, v, kv_len, causal, want_lse=True, **kw):
        assert k.shape[1] == int(kv_len[0])
        o, _ = oracle.decode_attn(q.float().numpy(), k.float().numpy()[None], v.float().numpy()[None],
                                  [k.shape[1]], causal)
        return torch.from_numpy(o).float(), None

    def score(q_text, k, q_pos0, n_vis, vis_start=0, agg="all", alpha=1.0, beta=0.0, out=None, **kw):
        s = oracle.score_layer(q_text.float().numpy(), k.float().numpy(), q_pos0, vis_start, n_vis, k.shape[0])
        out[:] = alpha * torch.from_numpy(oracle.aggregate_heads(s, k.shape[0], agg)).float() + beta * out
        return out

    def select(row, F, H, W, top_p, budget, with_tag=False):
        kept, _, _ = oracle.select_row(row[0].numpy(), F, H, W, top_p, budget)
        return torch.from_numpy(kept.astype(np.int32))[None], None, None

    def gather_kv(k, v, idx, tail_start, n_tail, k_dst, v_dst):
        rows = torch.cat([idx.long(), torch.arange(tail_start, tail_start + n_tail)])
        k_dst[:] = k[:, rows]
        v_dst[:] = v[:, rows]
        return k_dst, v_dst

    def decode_attn_indexed(q, k, v, kv_idx, n_idx, causal, want_lse=True, **kw):
        rows = kv_idx[:int(n_idx[0])].long()
        o, _ = oracle.decode_attn(q.float().numpy(), k[:, rows].float().numpy()[None],
                                  v[:, rows].float().numpy()[None], [len(rows)], causal)
        return torch.from_numpy(o).float(), None

    def verify(mode, draft_tok, target, **kw):
        n, tok = oracle.verify_greedy(draft_tok.numpy(), target.numpy())
        return torch.from_numpy(n), torch.from_numpy(tok)

    for name, fn in dict(decode_attn=decode_attn, decode_attn_indexed=decode_attn_indexed, score=score,
                         select=select, gather_kv=gather_kv, verify=verify).items():
        monkeypatch.setattr(ops, name, fn)


@pytest.mark.parametrize("draft_mode", ["compact", "indexed"])
@pytest.mark.parametrize("gamma", [3, 6])
def test_speculative_loop_equals_greedy_on_host(monkeypatch, gamma, draft_mode):
    from visual_kv_pruning_amd.spec_decode import TinyDecoder, Video, greedy_dense, speculative
    _substitutes(monkeypatch)
    model = TinyDecoder.random(3, layers=2, d_model=128, hq=4, hkv=2, d=64, vocab=256, device="cpu")
    g = torch.Generator().manual_seed(7)
    video = Video(4, 7, 7, torch.randn(196, model.d_model, generator=g),
                  torch.randint(0, model.vocab, (16,), generator=g))
    ref = greedy_dense(model, video, 24)
    got, acc = speculative(model, video, 24, gamma=gamma, keep=0.1, top_p=0.5, draft_mode=draft_mode)
    assert got == ref
    assert all(0 <= a <= gamma for a in acc)
