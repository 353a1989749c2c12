"""The fp64 oracle standing in for the library's calls, on CPU tensors, so the
speculative-decoding driver (`spec_decode.py`) can run on the host: with these
substitutes its bookkeeping is checked without a GPU, and its dense greedy
output is the oracle-driven reference for the GPU run.  (Test infrastructure:
the product path never calls the oracle.)"""
import numpy as np
import torch

import oracle


def substitute(mp) -> None:
    """Replace ops.score / select / gather_kv / decode_attn / decode_attn_indexed
    / verify with oracle-backed versions (mp: a pytest MonkeyPatch)."""
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
        k_dst[:] = torch.from_numpy(oracle.gather_kv(k.float().numpy(), idx.numpy(), tail_start, n_tail)).to(k_dst.dtype)
        v_dst[:] = torch.from_numpy(oracle.gather_kv(v.float().numpy(), idx.numpy(), tail_start, n_tail)).to(v_dst.dtype)
        return k_dst, v_dst

    def decode_attn_indexed(q, k, v, kv_idx, n_idx, causal, want_lse=True, **kw):
        rows = kv_idx[:int(n_idx[0])].long()
        o, _ = oracle.decode_attn(q.float().numpy(), k[:, rows].float().numpy()[None],
                                  v[:, rows].float().numpy()[None], [len(rows)], causal)
        return torch.from_numpy(o).float(), None

    def verify(mode, draft_tok, target, draft_prob=None, u=None, **kw):
        if mode == "greedy":
            n, tok = oracle.verify_greedy(draft_tok.numpy(), target.numpy())
        else:
            n, tok = oracle.verify_reject(draft_tok.numpy(), target.numpy(), draft_prob.numpy(), u.numpy())
        return torch.from_numpy(n), torch.from_numpy(tok)

    for name, fn in dict(decode_attn=decode_attn, decode_attn_indexed=decode_attn_indexed, score=score,
                         select=select, gather_kv=gather_kv, verify=verify).items():
        mp.setattr(ops, name, fn)
