"""Plain, slow CPU oracle for the svlm hot path (test infrastructure only).

This package is NOT part of the product.  Only the test suite, the smoke
check and the bench's CPU-baseline leg may import it.  It shares no code with
the HIP path (no kernels, headers, helpers or tables) and imports nothing from
it; both sides consume the same seeded inputs from ``workloads``.

Everything is NumPy in fp64; bf16 inputs are upcast exactly (bf16 -> fp32 ->
fp64).  Integer work (selection masses, sampling) uses Python / NumPy
integers, which are exact.

Sources, cited by page title and section:
  * SpecVLM, Zhejiang University technology-transfer listing, section 5
    "solution": the pruning module averages text-to-visual attention from the
    target model, then keeps tokens in two stages (Top-P by attention share,
    then a spatially uniform pick of the low-attention rest).
  * SpecVLM abstract (arXiv 2508.16201): stage I is guided by the verifier's
    attention, stage II prunes the rest in a spatially uniform way; up to 90%
    of video tokens pruned.
  * Sparse-to-Dense explainer (arXiv 2505.19155), technical summary,
    "decoding process" and "KV cache selection": top-K visual KV chosen at
    prefill from the mean text-to-visual attention, per layer and head; the
    dense model verifies the gamma drafted tokens in one pass over the full
    KV cache, accepts the longest matching prefix plus one bonus token.
  * ParallelVLM notes (CVPR 2026), background and "parallel decoding":
    drafted tokens are accepted by rejection sampling, so the output
    distribution is the target's; a rejected token is resampled from the
    target.  Method section 1, "UV-Prune": video tokens scored by the change,
    across early target layers, of their cosine similarity to the text
    tokens, summed over the text; top-K by the pruning ratio.

Parity status: every function here is pinned by tests that do not reuse its
code (brute force, closed forms, invariants, library routines); see
``tests/test_oracle_*.py``.  No function is parity-unpinned.
"""
from .score import attention_probs, score_layer, aggregate_heads, score_rows_for_config
from .select import select_row, select_rows, FIXED_POINT_SHIFT
from .gather import gather_kv
from .attention import decode_attn
from .verify import verify_greedy, verify_reject, sample_fixed_point
from .uvprune import cosine_matrix, uvprune_scores, uvprune_keep

__all__ = [
    "attention_probs", "score_layer", "aggregate_heads", "score_rows_for_config",
    "select_row", "select_rows", "FIXED_POINT_SHIFT",
    "gather_kv", "decode_attn",
    "verify_greedy", "verify_reject", "sample_fixed_point",
    "cosine_matrix", "uvprune_scores", "uvprune_keep",
]
